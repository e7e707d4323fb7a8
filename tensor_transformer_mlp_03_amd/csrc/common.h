// Internal declarations shared by the library's host and kernel sources.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

// Timing events that the calling thread's next kernel dispatches attach to: the
// first dispatch takes `start`, the `left`-th takes `stop`.  hipExtLaunchKernel
// binds them to the dispatch itself, so they hold the kernel's own start and end
// times and add no marker packets between kernels.  Set by the library's timing
// wrapper; all null outside a timing window.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  int left = 0;
};
extern thread_local LaunchEvents g_launch_events;

// Every kernel of the library takes one argument struct by value and is launched here.
template <typename T>
hipError_t launch_kernel(void (*kernel)(T), dim3 grid, dim3 block, hipStream_t s, T arg) {
  LaunchEvents& le = g_launch_events;
  hipEvent_t start = nullptr, stop = nullptr;
  if (le.left > 0) {
    start = le.start;
    le.start = nullptr;
    if (--le.left == 0) stop = le.stop;
  }
  void* args[] = {&arg};
  const hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, s, start,
                                          stop, 0);
  return e != hipSuccess ? e : hipGetLastError();
}

// How an operand sits in memory, seen from the GEMM C[m,n] = sum_k A[m,k] B[k,n].
//   KC: K is the contiguous dimension (A stored [M][ld], B stored [N][ld]).
//   MC: the other dimension is contiguous (A stored [K][ld] with M contiguous,
//       B stored [K][ld] with N contiguous).
enum Layout : int { KC = 0, MC = 1 };

// What the epilogue does with the float32 accumulator of C[m,n].
enum Epi : int {
  EPI_F32 = 0,      // out_f32[m,n] = acc (split-K: slice z writes its own partial)
  EPI_GELU = 1,     // out_bf16[m,n] = GeLU(acc); out2_bf16[m,n] = acc if out2 != null
  EPI_BF16 = 2,     // out_bf16[m,n] = acc
  EPI_DGELU = 3,    // p = aux_bf16[m,n]; out_bf16[m,n] = acc * GeLU'(p); transposed:
                    //   out2_bf16[n,m] = GeLU(p)
  EPI_F32_ACC = 4,  // out_f32[m,n] = out_f32[m,n] + acc: adds the product to a running
                    //   float32 sum (no split-K slices; the reduction applies it instead)
  // Two products of one shape in one launch (no split-K, 256 x 128 or 128 x 128
  // tiles): product p takes A from a_arr[p] and B from b_arr[p], a workgroup runs
  // both K loops for its tile into two accumulator sets, and the epilogue adds
  // them in order, as two launches of EPI_F32 / EPI_F32_ACC would:
  EPI_F32_PAIR = 5,      // out_f32[m,n] = acc0 + acc1
  EPI_F32_ACC_PAIR = 6,  // out_f32[m,n] = (out_f32[m,n] + acc0) + acc1
};

// Largest output row stride of an EPI_F32_ACC product (its loads of the running
// sum take 32-bit byte offsets within a 64-row band).
constexpr int64_t ACC_MAX_LDO = int64_t(1) << 22;

// Most products one batched launch holds (GemmArgs::batch).
constexpr int MAX_BATCH = 8;

struct GemmArgs {
  const uint16_t* a;  // A operand base (bf16 bits)
  const uint16_t* b;  // B operand base
  int64_t lda, ldb;   // leading dimensions in elements
  int M, N, K;        // problem size
  int k_split;        // K elements per split-K slice (multiple of the K tile); K if none
  void* out;          // float* (EPI_F32) or uint16_t* (bf16 epilogues)
  uint16_t* out2;     // second bf16 output or null
  const uint16_t* aux;  // EPI_DGELU's pre-activation input
  int64_t ldo;        // leading dimension of out, aux and (EPI_GELU) out2
  int64_t ldt;        // leading dimension of EPI_DGELU's transposed outputs
  int64_t split_stride;  // elements between split-K partial outputs
  int tiles_m, tiles_n;  // output tiles along M and N
  // FP8 products only (gemm kernels instantiated with operand formats): the
  // operands' amax slots (float bits; the scales follow from them), and an
  // optional slot that receives the amax of the bf16 output, of its GeLU when
  // amax_gelu is set (EPI_BF16), or of dP (EPI_DGELU, which then writes no G^T).
  const uint32_t* amax_a;
  const uint32_t* amax_b;
  uint32_t* amax_out;
  int amax_gelu;
  // Batched launch (batch > 1, no split-K): `batch` products of one shape and
  // leading dimensions; product j's operands and outputs are a_arr[j],
  // b_arr[j], out_arr[j], out2_arr[j] and aux_arr[j].  The workgroups cover
  // batch x tiles_m x tiles_n tiles.  batch 0 or 1: a, b, out, out2 and aux.
  int batch;
  const uint16_t* a_arr[MAX_BATCH];
  const uint16_t* b_arr[MAX_BATCH];
  void* out_arr[MAX_BATCH];
  uint16_t* out2_arr[MAX_BATCH];
  const uint16_t* aux_arr[MAX_BATCH];
};

// Tile shapes the library instantiates.
enum TileCfg : int {
  TILE_256x256 = 0,  // 4 waves, 2 x 2, wave tile 128 x 128
  TILE_128x128 = 1,  // 4 waves, 2 x 2, wave tile 64 x 64
  TILE_256x128 = 2,  // 4 waves, 2 x 2, wave tile 128 x 64 (the 256 x 256 kernel's ring)
  TILE_COUNT = 3,
};

// Launches C = A B with the given layouts and epilogue on `stream`.
// Returns the launch error (hipSuccess on success).  Shapes must already be valid.
hipError_t launch_gemm(TileCfg tile, Layout la, Layout lb, Epi epi, const GemmArgs& args,
                       int splits, hipStream_t stream);

// out[j] = sum over i < n_parts of parts[i][j], left to right, j < n (n % 4 == 0).
hipError_t launch_sum(const float* const* parts, int n_parts, float* out, int64_t n,
                      hipStream_t stream);

// Sum of `splits` float32 slices of an [M][N] product (slice i at part + i*M*N,
// rows of N) finished with the epilogue `epi` into out/out2 as the GEMM
// epilogue would.  out, out2 (GeLU's pre-activation) and aux (the dGeLU
// pre-activation) have rows of ldo elements; dGeLU's transposed out2 has rows
// of ldt (null: none written).  The outputs may be a column block of wider
// matrices.  FP8 products: `amax` (an AMAX_SUB-word slot, or null) collects the
// max |output| of EPI_BF16 (of its GeLU with amax_gelu) or of EPI_DGELU's dP.
hipError_t launch_splitk_epilogue(Epi epi, const float* part, int splits, int64_t M, int64_t N, void* out,
                                  uint16_t* out2, const uint16_t* aux, int64_t ldo, int64_t ldt,
                                  hipStream_t stream, uint32_t* amax = nullptr, bool amax_gelu = false);

// out[c][r] = in[r][c] for a bf16 matrix in[R][C] with rows of ld_in >= C
// elements, into out with rows of ld_out >= R elements (0: R), so that the
// transpose can be a column block of a wider matrix (R, C, ld_in, ld_out
// multiples of 8).
hipError_t launch_transpose(const uint16_t* in, int64_t R, int64_t C, int64_t ld_in, uint16_t* out,
                            hipStream_t stream, int64_t ld_out = 0);
// Two matrices of the same shape and strides in one launch (in1 null: one).
hipError_t launch_transpose2(const uint16_t* in0, uint16_t* out0, const uint16_t* in1, uint16_t* out1, int64_t R,
                             int64_t C, int64_t ld_in, hipStream_t stream, int64_t ld_out = 0);

// Fused forward for small hidden sizes (ffn.hip): workgroup (row block r,
// chunk c) computes GeLU(X[r] A_i[:, c]) B_i[c, :] with G kept in LDS and
// writes that float32 partial [rows][H] to slice c of `part` (slices of M x H,
// in chunk order); P_save (nullable) receives X A_i in bf16.
constexpr int FFN_ROWS = 64;    // rows of X per workgroup
constexpr int FFN_CHUNK = 64;   // intermediate columns per workgroup
constexpr int FFN_HMAX = 256;   // largest hidden size the fused kernel takes

struct FfnArgs {
  const uint16_t* x;   // X [M][H]
  const uint16_t* a;   // A_i [H][lda]
  const uint16_t* b;   // B_i [F][H]
  float* part;         // ffn_chunks(F) slices of [M][H] float32
  uint16_t* p_save;    // P_i [M][ldp] bf16, or null
  int64_t lda, ldp;
  int M, H, F;
};

// H a multiple of 64 and at most FFN_HMAX.
bool ffn_fused_fits(int64_t H);
// Number of partial slices (chunks of FFN_CHUNK intermediate columns).
int ffn_chunks(int64_t F);
hipError_t launch_ffn_fwd(const FfnArgs& a, hipStream_t stream);

int tile_bm(TileCfg t);
int tile_bn(TileCfg t);
constexpr int TILE_BK = 64;

// FP8 products: C = (A_codes B_codes) s_a s_b with A [M][lda] and B [N][ldb] FP8
// codes (both K-contiguous; K, lda, ldb and k_split counted in FP8 elements, all
// multiples of 16), fmt_a and fmt_b 0 for E4M3 and 1 for E5M2 (pairs (0,0), (1,0)
// and (0,1)), the scales from args.amax_a / amax_b.  `a` and `b` point at the codes.
hipError_t launch_gemm_fp8(TileCfg tile, int fmt_a, int fmt_b, Epi epi, const GemmArgs& args, int splits,
                           hipStream_t stream);

// An amax slot: AMAX_SUB 32-bit words, AMAX_SUB_STRIDE words apart so that each
// sits in its own 128-byte line.  Atomics on one address serialize (about 12 ns
// each here), so writers spread theirs over the words and readers take the max.
// The library's workspace slots have AMAX_SUB words; a caller's single float
// (tpmlp_fp8_quantize) is a slot of one word.
constexpr int AMAX_SUB = 16, AMAX_SUB_STRIDE = 32;
constexpr int AMAX_SLOT_WORDS = AMAX_SUB * AMAX_SUB_STRIDE;

// The FP8 element-wise kernels (fp8.hip).
struct Fp8ZeroArgs {
  uint32_t* p;
  int n;
};
struct Fp8AmaxArgs {
  const uint16_t* in;
  int64_t R, C, ld;
  uint32_t* slot;
  int nsub;  // words of the slot (epilogue.h)
};
struct Fp8QuantArgs {
  const uint16_t* in;
  uint8_t* out;
  int64_t R, C, ld_in, ld_out;
  int gelu, fmt;
  const uint32_t* slot;
  int nsub;       // words of the slot (epilogue.h)
  uint8_t* out2;  // transposed launches: also the row-major codes (nullable)
  int64_t ld_out2;
};
// p[0 .. n) = 0 (amax slots).
hipError_t launch_fp8_zero(uint32_t* p, int n, hipStream_t s);
// slot = max(slot, max |x|) over a bf16 [R][C] tensor (rows of ld; C % 8 == 0);
// the slot has nsub words (epilogue.h; 1 or AMAX_SUB).
hipError_t launch_fp8_amax(const uint16_t* in, int64_t R, int64_t C, int64_t ld, uint32_t* slot, int nsub,
                           hipStream_t s);
// FP8 codes of a bf16 [R][C] tensor (or of its GeLU) under the scale in `slot`:
// out [R][ld_out] bytes, or with transpose out [C][ld_out] (R, C multiples of 16)
// and, when out_rows is set, the row-major codes in out_rows [R][ld_rows] too.
hipError_t launch_fp8_quant(const uint16_t* in, int64_t R, int64_t C, int64_t ld_in, bool gelu, int fmt,
                            const uint32_t* slot, int nsub, uint8_t* out, int64_t ld_out, bool transpose, hipStream_t s,
                            uint8_t* out_rows = nullptr, int64_t ld_rows = 0);

}  // namespace tpmlp
