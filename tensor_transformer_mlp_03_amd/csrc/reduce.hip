// Memory-bound helpers: ordered float32 sums of equally shaped buffers and a
// bf16 transpose.
//
//  * sum_kernel: out = p_0 + p_1 + ... + p_{t-1}, the local stand-in for the
//    tensor-parallel all-reduce (the ranks' partial outputs are added,
//    "大模型训练" notes §3.1).
//  * splitk_kernel: the sum of the split-K slices of one product, finished with
//    that product's epilogue (float32 store, GeLU or bf16 store), so that a
//    product split along K ends exactly like an unsplit one.
//  * splitk_dgelu_kernel: the same for the dGeLU epilogue, which also writes G
//    transposed; it works on 64 x 64 tiles and transposes through LDS.
//
//  * transpose_kernel: out[c][r] = in[r][c] for bf16 matrices, so that the
//    weight-gradient products read both operands K-contiguous.
//
// All are HBM-bound: each lane moves 16-byte vectors, and parts are added left
// to right so that a sum does not depend on the launch shape.

#include "../../include/tpmlp.h"
#include "common.h"
#include "epilogue.h"

namespace tpmlp {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));

struct SumArgs {
  const float* parts[TPMLP_MAX_SHARDS];
  int n_parts;
  int64_t n4;  // number of float4 vectors
  float* out;
};

__global__ void __launch_bounds__(256) sum_kernel(SumArgs a) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < a.n4; j += stride) {
    f32x4_t s = reinterpret_cast<const f32x4_t*>(a.parts[0])[j];
    for (int i = 1; i < a.n_parts; ++i) s += reinterpret_cast<const f32x4_t*>(a.parts[i])[j];
    __builtin_nontemporal_store(s, reinterpret_cast<f32x4_t*>(a.out) + j);
  }
}

struct SplitArgs {
  const float* part;  // splits x n float32, slice i at part + i * n ([rows][cols])
  int splits;
  int64_t n;          // elements per slice (multiple of 4)
  int cols;           // slice row length (multiple of 4)
  int64_t ldo;        // row stride of out and out2
  void* out;          // float* (EPI_F32) or uint16_t*
  uint16_t* out2;     // second bf16 output or null
  const uint16_t* aux;
  uint32_t* amax;     // EPI_BF16 of an FP8 product: amax slot of the output (or its GeLU), or null
  int amax_gelu;
};

template <int EPI>
__global__ void __launch_bounds__(256) splitk_kernel(SplitArgs a) {
  const int64_t n4 = a.n / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const bool dense = a.ldo == a.cols;
  const uint32_t c4n = (uint32_t)a.cols / 4;
  AmaxTrack am;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n4; j += stride) {
    f32x4_t s = reinterpret_cast<const f32x4_t*>(a.part)[j];
    for (int i = 1; i < a.splits; ++i) s += reinterpret_cast<const f32x4_t*>(a.part + i * a.n)[j];
    // Element offset of the 4 values in the outputs (rows of ldo).
    const int64_t o = dense ? 4 * j : (int64_t)((uint64_t)j / c4n) * a.ldo + 4 * ((uint64_t)j % c4n);
    if (EPI == EPI_F32) {
      *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(a.out) + o) = s;
    } else if (EPI == EPI_F32_ACC) {
      // The product (its slices summed first) is added to the running sum.
      f32x4_t* p = reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(a.out) + o);
      *p = *p + s;
    } else if (EPI == EPI_GELU) {
      u16x4_t g, p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        g[e] = epi_gelu(s[e]);
        p[e] = f32_to_bf16(s[e]);
      }
      *reinterpret_cast<u16x4_t*>(reinterpret_cast<uint16_t*>(a.out) + o) = g;
      if (a.out2) *reinterpret_cast<u16x4_t*>(a.out2 + o) = p;
    } else if (EPI == EPI_BF16) {
      u16x4_t p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = f32_to_bf16(s[e]);
        if (a.amax) am.add(bf16_to_f32(p[e]));
      }
      *reinterpret_cast<u16x4_t*>(reinterpret_cast<uint16_t*>(a.out) + o) = p;
    }
  }
  if (EPI == EPI_BF16 && a.amax) slot_max(a.amax, AMAX_SUB, am.result(a.amax_gelu != 0));
}

struct SplitDGeluArgs {
  const float* part;    // splits x M x N float32
  int splits;
  int M, N;
  int64_t ldo, ldt;     // row strides of dp and p, and of g_t
  uint16_t* dp;         // [M][ldo]
  uint16_t* g_t;        // [N][ldt], or null (an FP8 product: no G^T)
  const uint16_t* p;    // [M][ldo] pre-activation
  uint32_t* amax;       // FP8 product: amax slot of dP, or null
};

typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));

// One 64 x 64 tile per block of 256 threads.  Thread t finishes columns
// 8*(t%8) .. +7 of rows t/8 and t/8 + 32 (eight threads cover a row's 256 bytes
// of each float32 slice), issuing the pre-activation loads and the slices'
// loads before it adds, then, after a barrier, writes 16 consecutive rows of
// one column of the transposed output.
__global__ void __launch_bounds__(256) splitk_dgelu_kernel(SplitDGeluArgs a) {
  __shared__ uint16_t s_g[64][72];  // 8 elements of padding per row
  const int tiles_n = (a.N + 63) / 64;
  const int m0 = (blockIdx.x / tiles_n) * 64, n0 = (blockIdx.x % tiles_n) * 64;
  const int t = threadIdx.x;
  const int64_t plane = (int64_t)a.M * a.N;
  {
    const int rq = t >> 3, c = 8 * (t & 7), col = n0 + c;
    bool ok[2];
    int64_t o[2];
    u16x8_t pb[2];
    f32x4_t s0[2], s1[2];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int row = m0 + rq + 32 * v;
      ok[v] = row < a.M && col < a.N;  // N % 8 == 0: 8 columns in or out together
      o[v] = ok[v] ? (int64_t)row * a.N + col : 0;
      const int64_t oo = ok[v] ? (int64_t)row * a.ldo + col : 0;
      pb[v] = *reinterpret_cast<const u16x8_t*>(a.p + oo);
      s0[v] = *reinterpret_cast<const f32x4_t*>(a.part + o[v]);
      s1[v] = *reinterpret_cast<const f32x4_t*>(a.part + o[v] + 4);
    }
#pragma unroll 2
    for (int i = 1; i < a.splits; ++i) {
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        s0[v] += *reinterpret_cast<const f32x4_t*>(a.part + i * plane + o[v]);
        s1[v] += *reinterpret_cast<const f32x4_t*>(a.part + i * plane + o[v] + 4);
      }
    }
    AmaxTrack am;
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      if (!ok[v]) continue;
      const int r = rq + 32 * v;
      const float x[8] = {s0[v][0], s0[v][1], s0[v][2], s0[v][3], s1[v][0], s1[v][1], s1[v][2], s1[v][3]};
      u16x8_t dp;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const DGelu d = epi_dgelu(x[e], pb[v][e]);  // dP's bits equal bf16(dgelu_f32(x, p))
        dp[e] = d.dp;
        s_g[r][c + e] = d.g;
        if (a.amax) am.add(bf16_to_f32(d.dp));
      }
      *reinterpret_cast<u16x8_t*>(a.dp + (int64_t)(m0 + r) * a.ldo + col) = dp;
    }
    if (a.amax) slot_max(a.amax, AMAX_SUB, am.result(false));
  }
  if (!a.g_t) return;  // uniform: the whole block returns before the barrier
  __syncthreads();
  {
    const int c = t >> 2, col = n0 + c;   // a column of the tile = a row of the transposed output
    const int r0 = 16 * (t & 3), row = m0 + r0;
    if (col < a.N) {
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        if (row + 8 * v >= a.M) continue;  // M % 8 == 0
        u16x8_t gv;
#pragma unroll
        for (int e = 0; e < 8; ++e) gv[e] = s_g[r0 + 8 * v + e][c];
        const int64_t o = (int64_t)col * a.ldt + row + 8 * v;
        *reinterpret_cast<u16x8_t*>(a.g_t + o) = gv;
      }
    }
  }
}

int grid_for(int64_t n4) {
  const int64_t want = (n4 + 255) / 256;  // 2048 blocks of 256 measured best on 2.4 GB sums
  return (int)(want < 2048 ? (want > 0 ? want : 1) : 2048);
}

// bf16 transpose, one 64 x 64 tile per wave.  Lane (rb, cb) = (lane / 8,
// lane % 8) loads the 8 x 8 block at rows 8*rb .. +7, columns 8*cb .. +7 of the
// tile (8 loads of 16 bytes: one instruction reads 8 rows x 128 bytes), turns
// it around in registers with v_perm_b32 and writes rows 8*cb .. +7 of the
// output tile, columns 8*rb .. +7 (one instruction writes 8 rows x 128 bytes).
// R and C are multiples of 8, so a block is entirely inside or outside.
// The four waves of a workgroup take four consecutive row tiles of one column
// tile, and consecutive workgroups continue along the rows, so that the output
// rows (R * 2 bytes apart, often a power of two) are written in long runs
// rather than 64 rows at a time at one stride, which would load one memory
// channel.  One launch can transpose two matrices of the same shape (X and dZ
// before a backward): workgroups [0, blocks) take the first, [blocks, 2 blocks)
// the second.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct TransposeArgs {
  const uint16_t* in[2];
  uint16_t* out[2];
  int64_t R, C;  // in is [R][C] (rows of ld_in elements), out is [C][R] (rows of ld_out)
  int64_t ld_in, ld_out;
  int row_groups;  // groups of four 64-row tiles
  int blocks;      // workgroups per matrix
};

__global__ void __launch_bounds__(256) transpose_kernel(TransposeArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int lane = threadIdx.x & 63;
  const int job = (int)blockIdx.x >= a.blocks ? 1 : 0;  // uniform over the workgroup
  const int bid = (int)blockIdx.x - job * a.blocks;
  const uint16_t* in = job ? a.in[1] : a.in[0];
  uint16_t* out = job ? a.out[1] : a.out[0];
  const int rg = bid % a.row_groups, ct = bid / a.row_groups;
  // The wave's 64 x 64 tile starts at (tr, tc); the buffer descriptor is built
  // from that wave-uniform origin (a per-lane base would not fit the scalar
  // descriptor and would serialize the loads).
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t tr = ((int64_t)rg * 4 + wave) * 64, tc = (int64_t)ct * 64;
  if (tr >= a.R) return;
  const int lr = 8 * (lane >> 3), lc = 8 * (lane & 7);
  const int64_t r0 = tr + lr, c0 = tc + lc;
  if (r0 >= a.R || c0 >= a.C) return;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(in + tr * a.ld_in + tc), (short)0, 0x7FFFFFF0, 0x00020000);
  u32x4_t v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = __builtin_bit_cast(u32x4_t,
                              __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(((lr + i) * a.ld_in + lc) * 2), 0, 0));
  // Output row c0 + j takes element j of each of the 8 input rows: dword e
  // packs input rows 2e and 2e+1, i.e. the halves of v[2e] and v[2e+1] that
  // hold column j (low halves for even j, high halves for odd j).
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
    u32x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = __builtin_amdgcn_perm(v[2 * e + 1][j >> 1], v[2 * e][j >> 1], sel);
    *reinterpret_cast<u32x4_t*>(out + (c0 + j) * a.ld_out + r0) = o;
  }
#else
  (void)a;
#endif
}

}  // namespace

hipError_t launch_sum(const float* const* parts, int n_parts, float* out, int64_t n, hipStream_t stream) {
  if (!parts || n_parts < 1 || n_parts > TPMLP_MAX_SHARDS || (n & 3)) return hipErrorInvalidValue;
  SumArgs a;
  for (int i = 0; i < n_parts; ++i) a.parts[i] = parts[i];
  a.n_parts = n_parts;
  a.n4 = n / 4;
  a.out = out;
  return launch_kernel(sum_kernel, dim3(grid_for(a.n4)), dim3(256), stream, a);
}

hipError_t launch_splitk_epilogue(Epi epi, const float* part, int splits, int64_t M, int64_t N, void* out,
                                  uint16_t* out2, const uint16_t* aux, int64_t ldo, int64_t ldt,
                                  hipStream_t stream, uint32_t* amax, bool amax_gelu) {
  const int64_t n = M * N;
  if (!part || splits < 1 || (N & 3) || ldo < N) return hipErrorInvalidValue;
  if (epi == EPI_DGELU) {
    SplitDGeluArgs a{part, splits, (int)M, (int)N, ldo, ldt, static_cast<uint16_t*>(out), out2, aux, amax};
    const int64_t tiles = ((M + 63) / 64) * ((N + 63) / 64);
    return launch_kernel(splitk_dgelu_kernel, dim3((unsigned)tiles), dim3(256), stream, a);
  }
  SplitArgs a{part, splits, n, (int)N, ldo, out, out2, aux, amax, amax_gelu ? 1 : 0};
  const dim3 grid(grid_for(n / 4)), block(256);
  switch (epi) {
    case EPI_F32: return launch_kernel(splitk_kernel<EPI_F32>, grid, block, stream, a);
    case EPI_F32_ACC: return launch_kernel(splitk_kernel<EPI_F32_ACC>, grid, block, stream, a);
    case EPI_GELU: return launch_kernel(splitk_kernel<EPI_GELU>, grid, block, stream, a);
    case EPI_BF16: return launch_kernel(splitk_kernel<EPI_BF16>, grid, block, stream, a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_transpose2(const uint16_t* in0, uint16_t* out0, const uint16_t* in1, uint16_t* out1, int64_t R,
                             int64_t C, int64_t ld_in, hipStream_t stream, int64_t ld_out) {
  if (ld_out == 0) ld_out = R;
  if (ld_in < C || (ld_in & 7) || ld_out < R || (ld_out & 7)) return hipErrorInvalidValue;
  if (!in0 || !out0 || (in1 && !out1)) return hipErrorInvalidValue;
  TransposeArgs a;
  a.in[0] = in0;
  a.out[0] = out0;
  a.in[1] = in1;
  a.out[1] = out1;
  a.R = R;
  a.C = C;
  a.ld_in = ld_in;
  a.ld_out = ld_out;
  a.row_groups = (int)((R + 255) / 256);
  const int64_t blocks = (int64_t)a.row_groups * ((C + 63) / 64);
  const int jobs = in1 ? 2 : 1;
  if (blocks * jobs > INT32_MAX) return hipErrorInvalidValue;
  a.blocks = (int)blocks;
  return launch_kernel(transpose_kernel, dim3((unsigned)(blocks * jobs)), dim3(256), stream, a);
}

hipError_t launch_transpose(const uint16_t* in, int64_t R, int64_t C, int64_t ld_in, uint16_t* out,
                            hipStream_t stream, int64_t ld_out) {
  return launch_transpose2(in, out, nullptr, nullptr, R, C, ld_in, stream, ld_out);
}

}  // namespace tpmlp
