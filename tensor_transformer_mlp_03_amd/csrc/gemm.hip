// bf16 MFMA GEMM core for gfx950 with the MLP's fused epilogues.
//
// C[m,n] = sum_k A[m,k] B[k,n], bf16 operands, float32 accumulation on
// v_mfma_f32_32x32x16_bf16.  Every product of the tensor-parallel MLP's forward
// and backward is one launch of this kernel with a different operand layout and
// epilogue:
//
//   forward   P_i = X A_i          A: KC  B: MC  epilogue GeLU -> G_i (and P_i)
//             Z_i = G_i B_i        A: KC  B: MC  epilogue float32
//   backward  P_i = X A_i          A: KC  B: MC  epilogue bf16 (recompute)
//             dG_i = dZ B_i^T      A: KC  B: KC  epilogue dGeLU -> dP_i, G_i
//             dB_i = G_i^T dZ      A: MC  B: MC  epilogue float32 (split-K)
//             dA_i = X^T dP_i      A: MC  B: MC  epilogue float32 (split-K)
//             dX_i = dP_i A_i^T    A: KC  B: KC  epilogue float32
//
// (The split of A by columns and B by rows that makes rank i's work exactly
// these products: "大模型训练" notes §3.1; GeLU between the two GEMMs: QLM page
// §2.1.2.2 part 3; fusing the activation into the producing kernel so the
// float32 pre-activation never round-trips through memory: asorrir.com survey,
// part 三, 算子融合.)
//
// Design for CDNA4:
//  * A block computes a BM x BN output tile with 64-wide waves laid out
//    WAVES_M x WAVES_N; each wave owns a (BM/WAVES_M) x (BN/WAVES_N) sub-tile of
//    32 x 32 MFMA fragments held in accumulator registers.
//  * K advances in steps of 64.  Global tiles are loaded 16 bytes per lane into
//    registers one step ahead, then written to one of two LDS stages; one barrier
//    per K step separates the stage being read from the stage being written.
//  * LDS keeps each operand in its memory layout.  A K-contiguous tile is read
//    with ds_read_b128 (8 consecutive k of one row per lane, the MFMA operand
//    layout); an M/N-contiguous tile is read with two ds_read_b64_tr_b16, whose
//    16-lane transpose delivers 4 consecutive k of one column per lane.  No
//    operand is transposed in registers or in memory.
//  * 16-byte chunks are XOR-swizzled inside each LDS row so that the rows one
//    read instruction touches fall on distinct banks.
//  * Ragged edges (sizes that are multiples of 8 but not of the tile) are
//    handled by zero-filling out-of-range chunks and masking the stores.
//  * Workgroups are renumbered so that consecutive output tiles (which share
//    operand panels) run on the same XCD and its L2, then grouped 8 tiles tall.

#include "common.h"

namespace tpmlp {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int BK = TILE_BK;
constexpr int GROUP_M = 8;
constexpr int NUM_XCD = 8;

// Swizzle of the 16-byte chunk index inside a 128-byte row of a K-contiguous
// tile: rows r .. r+15 read at one chunk land on 16 distinct (half, chunk) bank
// groups, and rows r .. r+7 on 8 distinct chunks.
__device__ __forceinline__ int swz_kc(int row) { return (row ^ (row >> 3)) & 7; }

// Swizzle of the chunk index inside a row of an M/N-contiguous tile (one row per
// k).  A transpose read touches rows k..k+3 at 2-4 adjacent chunks; XOR-ing
// chunk bits 1..3 with (k0, k1, k0) sends them to distinct banks.
template <int CHUNKS>
__device__ __forceinline__ int swz_mc(int k) {
  int s = ((k & 1) << 1) | ((k & 2) << 1) | ((k & 1) << 3);
  return s & (CHUNKS - 1);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// GeLU(p) = p Phi(p), Phi(p) = (1 + erf(p / sqrt 2)) / 2.
__device__ __forceinline__ float gelu_f(float p) {
  return 0.5f * p * (1.0f + erff(p * 0.70710678118654752f));
}

// Staging of one operand's K step: global -> registers -> LDS.
//   KC: LDS tile [R][BK], element (r, k) at r*BK*2 + ((k/8) ^ swz_kc(r))*16 + (k%8)*2
//   MC: LDS tile [BK][R], element (k, r) at k*R*2 + ((r/8) ^ swz_mc(k))*16 + (r%8)*2
template <int R, int THREADS, int LAYOUT>
struct Stager {
  static constexpr int CHUNKS = R * BK / 8;            // 16-byte chunks per tile
  static constexpr int PER_THREAD = CHUNKS / THREADS;
  static_assert(CHUNKS % THREADS == 0, "tile must divide evenly over threads");
  u32x4_t v[PER_THREAD];

  // rows/cols of the operand: `outer` indexes the non-K dimension.
  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int64_t ld, int outer0,
                                       int outer_n, int k0, int k_end, int tid) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int q = i * THREADS + tid;
      int o, kk;
      if (LAYOUT == KC) {
        o = q / (BK / 8);
        kk = (q % (BK / 8)) * 8;
      } else {
        kk = q / (R / 8);
        o = (q % (R / 8)) * 8;
      }
      const int go = outer0 + o, gk = k0 + kk;
      const bool ok = (go < outer_n) && (gk < k_end);
      const int64_t off = (LAYOUT == KC) ? (int64_t)go * ld + gk : (int64_t)gk * ld + go;
      if (ok) {
        v[i] = *reinterpret_cast<const u32x4_t*>(base + off);
      } else {
        v[i] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }

  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int q = i * THREADS + tid;
      int byte;
      if (LAYOUT == KC) {
        const int r = q / (BK / 8), c = q % (BK / 8);
        byte = r * BK * 2 + ((c ^ swz_kc(r)) << 4);
      } else {
        const int k = q / (R / 8), c = q % (R / 8);
        byte = k * R * 2 + ((c ^ swz_mc<R / 8>(k)) << 4);
      }
      *reinterpret_cast<u32x4_t*>(lds + byte) = v[i];
    }
  }
};

// MFMA operand fragment of a 32-row (or 32-column) slice at K step kk (16 wide):
// lane l gets 8 consecutive k (8*(l/32) .. +7 within the step) of row/column l%32.
template <int R, int LAYOUT>
__device__ __forceinline__ bf16x8_t read_frag(const char* lds, int o0, int kk, int lane) {
  if (LAYOUT == KC) {
    const int r = o0 + (lane & 31);
    const int c = 2 * kk + (lane >> 5);
    return *reinterpret_cast<const bf16x8_t*>(lds + r * BK * 2 + ((c ^ swz_kc(r)) << 4));
  } else {
    // ds_read_b64_tr_b16: in each 16-lane group, result lane i element e comes
    // from source lane 4e + i/4, slot i%4.  Source lane j therefore reads the 4
    // elements (k0 + j/4, o .. o+3) with o = o0 + 4*(j%4): result lane i then
    // holds column o0 + i at k0 .. k0+3.
    const int g = lane >> 4, j = lane & 15;
    const int o = o0 + 16 * (g & 1) + 4 * (j & 3);
    const int kbase = 16 * kk + 8 * (g >> 1) + (j >> 2);
    const int c = o >> 3, half = (o & 7) * 2;
    const int k_lo = kbase, k_hi = kbase + 4;
    const char* p_lo = lds + k_lo * R * 2 + ((c ^ swz_mc<R / 8>(k_lo)) << 4) + half;
    const char* p_hi = lds + k_hi * R * 2 + ((c ^ swz_mc<R / 8>(k_hi)) << 4) + half;
    i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p_lo));
    i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p_hi));
    typedef short i16x8_t __attribute__((ext_vector_type(8)));
    i16x8_t both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, both);
  }
}

// Logical tile of workgroup `bid`: XCD-aware renumbering, then grouped order.
__device__ __forceinline__ void tile_of(int bid, int nblocks, int tiles_m, int tiles_n, int& tm,
                                        int& tn, int& split) {
  const int q = nblocks / NUM_XCD, rem = nblocks % NUM_XCD;
  const int xcd = bid % NUM_XCD, idx = bid / NUM_XCD;
  const int logical = xcd * q + min(xcd, rem) + idx;
  const int tiles = tiles_m * tiles_n;
  split = logical / tiles;
  const int t = logical % tiles;
  const int per_group = GROUP_M * tiles_n;
  const int group = t / per_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int in_group = t % per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int LA, int LB, int EPI>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N)
gemm_kernel(GemmArgs args) {
  constexpr int THREADS = 64 * WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  constexpr int STAGE = A_BYTES + B_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  int tm, tn, split;
  tile_of(blockIdx.x, gridDim.x, args.tiles_m, args.tiles_n, tm, tn, split);
  const int m0 = tm * BM, n0 = tn * BN;
  const int k_begin = split * args.k_split;
  const int k_end = min(args.K, k_begin + args.k_split);
  const int nk = (k_end - k_begin + BK - 1) / BK;

  Stager<BM, THREADS, LA> sa;
  Stager<BN, THREADS, LB> sb;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  if (nk > 0) {
    sa.load(args.a, args.lda, m0, args.M, k_begin, k_end, tid);
    sb.load(args.b, args.ldb, n0, args.N, k_begin, k_end, tid);
    sa.store(smem, tid);
    sb.store(smem + A_BYTES, tid);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const char* cur = smem + (kt & 1) * STAGE;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k0 = k_begin + (kt + 1) * BK;
      sa.load(args.a, args.lda, m0, args.M, k0, k_end, tid);
      sb.load(args.b, args.ldb, n0, args.N, k0, k_end, tid);
    }
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = read_frag<BM, LA>(cur, wm * WM + 32 * i, kk, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = read_frag<BN, LB>(cur + A_BYTES, wn * WN + 32 * j, kk, lane);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      char* nxt = smem + ((kt + 1) & 1) * STAGE;
      sa.store(nxt, tid);
      sb.store(nxt + A_BYTES, tid);
    }
    __syncthreads();
  }

  // Epilogue.  Accumulator register r of fragment (i, j) holds
  // C[32i + 8(r/4) + 4(lane/32) + r%4][32j + lane%32] of the wave's sub-tile.
  const int col_base = n0 + wn * WN + (lane & 31);
  const int row_base = m0 + wm * WM + 4 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = col_base + 32 * j;
      if (col >= args.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row_base + 32 * i + 8 * (r >> 2) + (r & 3);
        if (row >= args.M) continue;
        const int64_t o = (int64_t)row * args.ldo + col;
        const float x = acc[i][j][r];
        if (EPI == EPI_F32) {
          float* out = reinterpret_cast<float*>(args.out) + (int64_t)split * args.split_stride;
          out[o] = x;
        } else if (EPI == EPI_GELU) {
          reinterpret_cast<uint16_t*>(args.out)[o] = f32_to_bf16(gelu_f(x));
          if (args.out2) args.out2[o] = f32_to_bf16(x);
        } else if (EPI == EPI_BF16) {
          reinterpret_cast<uint16_t*>(args.out)[o] = f32_to_bf16(x);
        } else {  // EPI_DGELU
          const float p = bf16_to_f32(args.aux[o]);
          const float phi_cdf = 0.5f * (1.0f + erff(p * 0.70710678118654752f));
          const float pdf = 0.39894228040143268f * expf(-0.5f * p * p);
          reinterpret_cast<uint16_t*>(args.out)[o] = f32_to_bf16(x * (phi_cdf + p * pdf));
          args.out2[o] = f32_to_bf16(p * phi_cdf);
        }
      }
    }
  }
}

template <int BM, int BN, int WM_, int WN_, int LA, int LB, int EPI>
hipError_t launch_one(const GemmArgs& a, int splits, hipStream_t s) {
  const int blocks = a.tiles_m * a.tiles_n * splits;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM_, WN_, LA, LB, EPI>), dim3(blocks), dim3(64 * WM_ * WN_), 0, s, a);
  return hipGetLastError();
}

template <int BM, int BN, int WM_, int WN_>
hipError_t dispatch_layout(Layout la, Layout lb, Epi epi, const GemmArgs& a, int splits, hipStream_t s) {
  if (la == KC && lb == MC) {
    switch (epi) {
      case EPI_GELU: return launch_one<BM, BN, WM_, WN_, KC, MC, EPI_GELU>(a, splits, s);
      case EPI_F32: return launch_one<BM, BN, WM_, WN_, KC, MC, EPI_F32>(a, splits, s);
      case EPI_BF16: return launch_one<BM, BN, WM_, WN_, KC, MC, EPI_BF16>(a, splits, s);
      default: break;
    }
  } else if (la == KC && lb == KC) {
    switch (epi) {
      case EPI_DGELU: return launch_one<BM, BN, WM_, WN_, KC, KC, EPI_DGELU>(a, splits, s);
      case EPI_F32: return launch_one<BM, BN, WM_, WN_, KC, KC, EPI_F32>(a, splits, s);
      default: break;
    }
  } else if (la == MC && lb == MC) {
    if (epi == EPI_F32) return launch_one<BM, BN, WM_, WN_, MC, MC, EPI_F32>(a, splits, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int tile_bm(TileCfg t) { return t == TILE_256x256 ? 256 : 128; }
int tile_bn(TileCfg t) { return t == TILE_256x256 ? 256 : 128; }

hipError_t launch_gemm(TileCfg tile, Layout la, Layout lb, Epi epi, const GemmArgs& args, int splits,
                       hipStream_t stream) {
  switch (tile) {
    case TILE_256x256: return dispatch_layout<256, 256, 2, 4>(la, lb, epi, args, splits, stream);
    case TILE_128x128: return dispatch_layout<128, 128, 2, 2>(la, lb, epi, args, splits, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tpmlp
