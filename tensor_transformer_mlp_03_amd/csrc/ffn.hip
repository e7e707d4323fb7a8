// Fused forward of one rank's MLP shard for small hidden sizes: both products
// and the GeLU between them in one launch, with the GeLU output kept in LDS.
//
// Rank i computes Z_i = GeLU(X A_i) B_i ("大模型训练" notes §3.1; GeLU between
// the widening and the narrowing product: QLM page §2.1.2.2 part 3).  Tokens
// do not interact inside the MLP (sequence-parallel series, §2.4 FFN 切分), and
// the intermediate columns f of A_i and rows f of B_i enter Z_i as a plain sum
// over f, so the work splits into independent (row block, column chunk) pieces:
//
//   Z_i[m, :] = sum over chunks c of GeLU(X[m, :] A_i[:, c]) B_i[c, :]
//
// Workgroup (row block r, chunk c) loads its 64 rows of X, the 64 columns c of
// A_i and the 64 rows c of B_i with every load in flight at once, computes
// P = X A_i[:, c] (64 x 64) on the matrix cores, applies GeLU in registers and
// writes G to LDS as bf16 (the same rounding as the two-launch path, which
// stores it in memory), then multiplies G by B_i[c, :] and writes the float32
// partial [64, H] of chunk c.  The chunks' partials are added in chunk order by
// the split-K reduction, so the result does not depend on the launch shape.
// Only G's trip through memory and the second product's launch are saved:
// the path is meant for shapes whose time is latency, not bandwidth or matrix
// throughput (the blockwise feed-forward idea of computing the FFN block by
// block: sequence-parallel series, Blockwise Parallel Transformer).
//
// Limits (checked by the host): H a multiple of 64 and at most 256, so a row
// block's X, a chunk of A_i and a chunk of B_i are all loaded up front; any
// M and F_i that are multiples of 8 (rows and columns beyond them read as zero
// and are not written).

#include "common.h"
#include "epilogue.h"

namespace tpmlp {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));

constexpr int RB = FFN_ROWS;    // rows of X per workgroup
constexpr int FC = FFN_CHUNK;   // columns of A_i (rows of B_i) per workgroup
constexpr int HMAX = FFN_HMAX;
constexpr int XL = HMAX + 8;    // LDS row length (elements) of the X and A_i^T tiles
constexpr int CL = FC + 8;      // LDS row length of the B_i^T and G tiles
constexpr int VPT = RB * HMAX / 8 / 256;  // 16-byte loads per thread for X
constexpr uint32_t OOB = 0x7FFFFFF0u;      // an offset past every descriptor's range

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)OOB, 0x00020000);
}

// 16 bytes at byte offset `off` of the buffer; zeros when off is past its range.
__device__ __forceinline__ u16x8_t load16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(u16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
}

}  // namespace

namespace kern {

// 256 threads, four waves.  Stage 1: wave w computes the 32 x 32 block
// (rows 32 (w & 1), chunk columns 32 (w >> 1)) of P over K = H.  Stage 2: the
// [64, H] partial is H / 16 blocks of 32 x 32, wave w taking blocks w, w + 4, ...
// The MFMA takes the B fragment first, so a lane's accumulator holds one row m
// (lane % 32) and runs of 4 consecutive columns (8 (r / 4) + 4 (lane / 32) + r % 4).
__global__ void __launch_bounds__(256) ffn_fwd_kernel(FfnArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[RB][XL];    // X rows [m][k]
  __shared__ __attribute__((aligned(16))) uint16_t at[FC][XL];    // A_i chunk transposed [f][k]
  __shared__ __attribute__((aligned(16))) uint16_t bt[HMAX][CL];  // B_i chunk transposed [n][f]
  __shared__ __attribute__((aligned(16))) uint16_t gs[RB][CL];    // G chunk [m][f]

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m0 = blockIdx.x * RB, f0 = blockIdx.y * FC;
  const int H = g.H, hv = H >> 3;  // 16-byte vectors per row of X and of B_i

  // All loads first, so that one memory latency covers them.  X goes to LDS as
  // stored.  The chunks of A_i and B_i are needed K-contiguous (8 consecutive
  // k per MFMA operand), so thread t < H loads an 8 x 8 block of each (eight
  // 16-byte rows), transposes it in registers and writes eight 16-byte rows
  // of the transposed tile.
  // Loads go through buffer descriptors: a lane outside the operand passes an
  // offset past the descriptor's range and reads zeros, with no branch (a
  // branch per load would let the compiler wait on earlier loads inside it).
  u16x8_t xr[VPT], ar[8], br[8];
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(g.x + (int64_t)m0 * H);
  // A_i rows of this wave's threads (64 w .. 64 w + 63) from a wave-uniform base,
  // so that offsets stay within 64 rows of lda elements.
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(g.a + f0 + (int64_t)(64 * wave) * g.lda);
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(g.b + (int64_t)f0 * H);
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int q = i * 256 + tid, r = q / hv, v = q - r * hv;
    const bool ok = r < RB && m0 + r < g.M;
    xr[i] = load16(xrs, ok ? (uint32_t)(r * H + 8 * v) * 2 : OOB);
  }
  // A_i rows k = 8 (t / 8) + i, columns f0 + 8 (t % 8) .. +7.
  const int akb = tid >> 3, av = tid & 7;
  const bool a_ok = tid < H && f0 + 8 * av < g.F;  // F % 8 == 0: a vector is in or out whole
#pragma unroll
  for (int i = 0; i < 8; ++i)
    ar[i] = load16(ars, a_ok ? (uint32_t)(((8 * akb + i - 64 * wave) * g.lda + 8 * av) * 2) : OOB);
  // B_i rows f0 + 8 (t % 8) + i, columns 8 (t / 8) .. +7.
  const int bv = tid >> 3, bfb = tid & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool ok = tid < H && f0 + 8 * bfb + i < g.F;
    br[i] = load16(brs, ok ? (uint32_t)((8 * bfb + i) * H + 8 * bv) * 2 : OOB);
  }
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int q = i * 256 + tid, r = q / hv, v = q - r * hv;
    if (r < RB) *reinterpret_cast<u16x8_t*>(&xs[r][8 * v]) = xr[i];
  }
  if (tid < H) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u16x8_t ta, tb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ta[i] = ar[i][j];
        tb[i] = br[i][j];
      }
      *reinterpret_cast<u16x8_t*>(&at[8 * av + j][8 * akb]) = ta;  // A_i^T [f][k]
      *reinterpret_cast<u16x8_t*>(&bt[8 * bv + j][8 * bfb]) = tb;  // B_i^T [n][f]
    }
  }
  __syncthreads();

  const int l32 = lane & 31, lhi = lane >> 5;

  // Stage 1: P = X A_i[:, chunk], GeLU -> G in LDS (and P -> P_save).
  {
    const int mt = wave & 1, nt = wave >> 1;
    f32x16_t acc = {};
    for (int ks = 0; ks < H / 16; ++ks) {
      const int k = 16 * ks + 8 * lhi;
      const bf16x8_t fa = *reinterpret_cast<const bf16x8_t*>(&xs[32 * mt + l32][k]);
      const bf16x8_t fb = *reinterpret_cast<const bf16x8_t*>(&at[32 * nt + l32][k]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb, fa, acc, 0, 0, 0);
    }
    const int m = 32 * mt + l32;
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int n = 32 * nt + 8 * rq + 4 * lhi;
      u16x4_t gv, pv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gv[e] = epi_gelu(acc[4 * rq + e]);
        pv[e] = f32_to_bf16(acc[4 * rq + e]);
      }
      *reinterpret_cast<u16x4_t*>(&gs[m][n]) = gv;
      if (g.p_save && m0 + m < g.M && f0 + n < g.F)
        *reinterpret_cast<u16x4_t*>(g.p_save + (int64_t)(m0 + m) * g.ldp + f0 + n) = pv;
    }
  }
  __syncthreads();

  // Stage 2: partial[m, :] = G[m, chunk] B_i[chunk, :], float32 to slice c.
  float* out = g.part + (int64_t)blockIdx.y * g.M * H;
  const int blocks = H / 16;
#pragma unroll
  for (int i = 0; i < HMAX / 64; ++i) {
    const int id = wave + 4 * i;
    if (id >= blocks) break;
    const int mt = id & 1, nt = id >> 1;
    f32x16_t acc = {};
#pragma unroll
    for (int ks = 0; ks < FC / 16; ++ks) {
      const int k = 16 * ks + 8 * lhi;
      const bf16x8_t fa = *reinterpret_cast<const bf16x8_t*>(&gs[32 * mt + l32][k]);
      const bf16x8_t fb = *reinterpret_cast<const bf16x8_t*>(&bt[32 * nt + l32][k]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb, fa, acc, 0, 0, 0);
    }
    const int m = 32 * mt + l32;
    if (m0 + m < g.M) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int n = 32 * nt + 8 * rq + 4 * lhi;
        f32x4_t v = {acc[4 * rq], acc[4 * rq + 1], acc[4 * rq + 2], acc[4 * rq + 3]};
        *reinterpret_cast<f32x4_t*>(out + (int64_t)(m0 + m) * H + n) = v;
      }
    }
  }
}

}  // namespace kern

bool ffn_fused_fits(int64_t H) { return H % 64 == 0 && H <= FFN_HMAX; }

int ffn_chunks(int64_t F) { return (int)((F + FFN_CHUNK - 1) / FFN_CHUNK); }

hipError_t launch_ffn_fwd(const FfnArgs& a, hipStream_t s) {
  if (!ffn_fused_fits(a.H) || a.M <= 0 || a.F <= 0 || a.M % 8 || a.F % 8) return hipErrorInvalidValue;
  const dim3 grid((a.M + FFN_ROWS - 1) / FFN_ROWS, ffn_chunks(a.F));
  return launch_kernel(kern::ffn_fwd_kernel, grid, dim3(256), s, a);
}

}  // namespace tpmlp
