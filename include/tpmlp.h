/*
 * libtpmlp — one tensor-parallel rank's share of the transformer MLP on MI355X (gfx950).
 *
 * The MLP is Y = GeLU(X A) B.  Its first weight A[H, F] is cut into column blocks
 * A_i[H, F_i] and its second weight B[F, H] into row blocks B_i[F_i, H], so rank i
 * computes Z_i = GeLU(X A_i) B_i with no exchange between the two products, and
 * the layer output is the sum of the ranks' Z_i ("大模型训练" notes, §3.1 张量并行,
 * MLP-layer formula and its two-GPU split).  The first product widens H to 4H and
 * the second narrows it back, with GeLU between them (QLM page, "大模型训练技术：
 * 使用QLM提升Qwen2-7B 128k训练效率3.4倍", §2.1.2.2 part 3); GeLU is taken in its
 * exact form p * Phi(p) = 0.5 p (1 + erf(p / sqrt 2)).
 *
 * Conventions for every call below
 * --------------------------------
 *  - Tensors are DEVICE pointers, row-major and contiguous.  bf16 tensors are raw
 *    16-bit patterns (1 sign, 8 exponent, 7 mantissa bits; "大模型训练" notes §6.1).
 *    Gradients and the partial outputs that ranks sum are float32.
 *  - The caller owns every buffer.  The library allocates nothing on these paths;
 *    its scratch space is the caller's workspace `ws` of at least the size the
 *    matching *_workspace_bytes query returns (any contents; it is overwritten).
 *  - Outputs are fully overwritten.  No output may overlap an input or another
 *    output (TPMLP_ERR_ALIAS).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  A call
 *    validates its arguments, enqueues its kernels on `stream` and returns; it
 *    does not synchronise.  Argument errors are reported before any HIP call is
 *    made and nothing is enqueued then.
 *  - M (token rows), H (hidden size) and F_i (the rank's slice of the intermediate
 *    size) must be positive multiples of 8 and at most 2^23; pointers must be
 *    16-byte aligned.  Sizes need not be multiples of any tile size.
 *  - Only gfx950 devices are supported (TPMLP_ERR_UNSUPPORTED otherwise).
 *  - All entry points are thread-safe; calls that share a workspace must not
 *    overlap in time.
 */
#ifndef TPMLP_H_
#define TPMLP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TPMLP_ABI_VERSION 12
#define TPMLP_MAX_SHARDS 64

typedef uint16_t tpmlp_bf16; /* raw bf16 bits */

typedef enum {
  TPMLP_OK = 0,
  TPMLP_ERR_NULL = 1,        /* a required pointer is NULL */
  TPMLP_ERR_SHAPE = 2,       /* M, H or F_i not a positive multiple of 8, or above 2^23 */
  TPMLP_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
  TPMLP_ERR_WORKSPACE = 4,   /* ws_bytes is below the workspace query's result */
  TPMLP_ERR_SHARDS = 5,      /* t outside 1..TPMLP_MAX_SHARDS */
  TPMLP_ERR_HIP = 6,         /* a HIP runtime call or a kernel launch failed */
  TPMLP_ERR_UNSUPPORTED = 7, /* the current device is not gfx950 */
  TPMLP_ERR_ALIAS = 8,       /* an output overlaps an input or another output */
  TPMLP_ERR_NO_FORWARD = 9   /* tpmlp_fp8_tp_bwd: ws holds no forward of these inputs */
} tpmlp_status;

/* TPMLP_ABI_VERSION of the built library. */
int tpmlp_abi_version(void);

/* Static English name of a status code; never NULL. */
const char* tpmlp_status_str(int status);

/* Detail of the last error on the calling thread (which argument, which HIP
 * error); "" if the last call succeeded.  Valid until the thread's next call. */
const char* tpmlp_last_error(void);

/* ------------------------------------------------------------------------ */
/* One rank's shard                                                          */
/* ------------------------------------------------------------------------ */

/* Workspace bytes that tpmlp_fwd needs for (M, H, F_i); 0 if the shape is invalid. */
size_t tpmlp_fwd_workspace_bytes(int64_t M, int64_t H, int64_t F_i);

/* Rank i's forward (the column-parallel GEMM, GeLU, the row-parallel GEMM):
 *   P_i = X A_i            X[M,H] bf16, A_i[H,F_i] bf16, float32 accumulation
 *   G_i = GeLU(P_i)        kept in the workspace as bf16 (round to nearest even)
 *   Z_i = G_i B_i          B_i[F_i,H] bf16 -> Z_i[M,H] float32 (the rank's partial)
 * P_save (nullable): if given, receives P_i[M,F_i] in bf16 (round to nearest even),
 * for a backward that keeps the pre-activation instead of recomputing it.
 * For small hidden sizes (H a multiple of 64, at most 256) with small M, the
 * call runs both products and GeLU in one fused launch per chunk of 64
 * intermediate columns, G_i staying on chip, and adds the chunks' float32
 * partials in chunk order (blockwise computation of the FFN: sequence-parallel
 * series, Blockwise Parallel Transformer); G_i is rounded to bf16 either way.
 * Sources: "大模型训练" notes §3.1; QLM page §2.1.2.2 part 3. */
tpmlp_status tpmlp_fwd(const tpmlp_bf16* X, const tpmlp_bf16* A_i, const tpmlp_bf16* B_i,
                       float* Z_i, tpmlp_bf16* P_save,
                       int64_t M, int64_t H, int64_t F_i,
                       void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes that tpmlp_bwd needs; `recompute` is 1 when P_saved will be
 * NULL.  0 if the shape is invalid.  The workspace holds the bf16 intermediates
 * [M,F_i] (dP_i, G_i^T, and P_i when recomputed), the transposes X^T and dZ^T
 * [H,M] in bf16, A_i^T [F_i,H] in bf16 when the shape gains from it, and float32
 * split-K slices. */
size_t tpmlp_bwd_workspace_bytes(int64_t M, int64_t H, int64_t F_i, int recompute);

/* Rank i's backward, given the output gradient dZ[M,H] (bf16), which every rank
 * holds whole because the row-parallel layer's forward sum has an identity
 * backward (QLM page §2.1.2.2 parts 1-2, operators read as the f/g pair):
 *   P_i   = P_saved, or X A_i recomputed when P_saved is NULL (products need their
 *           inputs for their gradients: asorrir.com survey, part 二, Checkpoint 技术;
 *           recompute: "大模型训练" notes §7)
 *   dG_i  = dZ B_i^T
 *   dP_i  = dG_i * GeLU'(P_i), GeLU'(p) = Phi(p) + p phi(p)   (bf16 in the workspace)
 *   dB_i  = GeLU(P_i)^T dZ     -> dB_i[F_i,H] float32
 *   dA_i  = X^T dP_i           -> dA_i[H,F_i] float32
 *   dX_i  = dP_i A_i^T         -> dX_i[M,H] float32, this rank's partial of dX
 * P_saved is bf16 [M,F_i] as written by tpmlp_fwd's P_save. */
tpmlp_status tpmlp_bwd(const tpmlp_bf16* dZ, const tpmlp_bf16* X, const tpmlp_bf16* A_i,
                       const tpmlp_bf16* B_i, const tpmlp_bf16* P_saved,
                       float* dX_i, float* dA_i, float* dB_i,
                       int64_t M, int64_t H, int64_t F_i,
                       void* ws, size_t ws_bytes, void* stream);

/* Activation memory that one rank keeps from its forward to its backward, in
 * bytes: X[M,H] in bf16, which the backward reads either way (its weight
 * gradient dA_i = X^T dP_i needs it), plus the pre-activation P_i[M,F_i] in bf16
 * unless it is recomputed.  Recomputing saves those M F_i 2 bytes at the cost of
 * one more product of 2 M H F_i flops, a sixth of the shard's model FLOPs
 * (products need their inputs for their gradients, recomputation trades compute
 * for memory: asorrir.com survey, part 二, Checkpoint 技术; "大模型训练" notes §7).
 * 0 if the shape is invalid. */
size_t tpmlp_saved_activation_bytes(int64_t M, int64_t H, int64_t F_i, int recompute);

/* Store-or-recompute choice for one rank's shard under an activation budget of
 * `budget_bytes` per rank: 0 = keep P_i (no extra work) when that fits, 1 =
 * recompute P_i when only the smaller footprint fits, -1 when neither fits or the
 * shape is invalid.  Storing is preferred because it costs no FLOPs. */
int tpmlp_recompute_policy(int64_t M, int64_t H, int64_t F_i, size_t budget_bytes);

/* ------------------------------------------------------------------------ */
/* The t-shard driver: all t ranks' shards run one after another on one GPU and */
/* their partials are summed locally in rank order 0..t-1, in float32.  The sum */
/* stands in for the all-reduce of Z (forward) and of dX (backward).           */
/* ------------------------------------------------------------------------ */

/* Workspace bytes for tpmlp_tp_fwd and tpmlp_tp_bwd (either backward mode) with
 * t shards: the largest per-shard workspace plus room for t float32 partials
 * [M,H].  0 if the arguments are invalid. */
size_t tpmlp_tp_workspace_bytes(int t, int64_t M, int64_t H, int64_t F_i);

/* Z = sum_i GeLU(X A_sh[i]) B_sh[i].
 * A_sh, B_sh: host arrays of t device pointers (shard i's A_i[H,F_i], B_i[F_i,H]).
 * P_sh (nullable host array; entries nullable): per-shard P_save.
 * Z_sh (nullable host array; entries nullable): where shard i's partial Z_i[M,H]
 * goes; a NULL array or entry puts it in the workspace.
 * Z[M,H] float32: the summed output. */
tpmlp_status tpmlp_tp_fwd(const tpmlp_bf16* X, const tpmlp_bf16* const* A_sh,
                          const tpmlp_bf16* const* B_sh, tpmlp_bf16* const* P_sh,
                          float* const* Z_sh, float* Z,
                          int t, int64_t M, int64_t H, int64_t F_i,
                          void* ws, size_t ws_bytes, void* stream);

/* Backward of all t shards, dX = sum_i dX_i.
 * P_sh: NULL host array => every shard recomputes P_i; otherwise t device
 * pointers written by tpmlp_tp_fwd (no NULL entries).
 * dA_sh, dB_sh: host arrays of t device pointers (float32 weight gradients).
 * dX_sh (nullable host array; entries nullable): per-shard partial dX_i. */
tpmlp_status tpmlp_tp_bwd(const tpmlp_bf16* dZ, const tpmlp_bf16* X,
                          const tpmlp_bf16* const* A_sh, const tpmlp_bf16* const* B_sh,
                          const tpmlp_bf16* const* P_sh,
                          float* const* dA_sh, float* const* dB_sh, float* const* dX_sh,
                          float* dX, int t, int64_t M, int64_t H, int64_t F_i,
                          void* ws, size_t ws_bytes, void* stream);

/* The t-shard driver over unsharded weights, with no copy of the shards.  A is
 * the whole first weight [H, t F_i] and B the whole second weight [t F_i, H];
 * shard i reads A_i = columns [i F_i, (i+1) F_i) of A (a strided view, rows of
 * t F_i elements) and B_i = rows [i F_i, (i+1) F_i) of B, which is exactly the
 * column split of A and row split of B that makes the shards independent
 * ("大模型训练" notes §3.1, A = [A_1 | A_2], B = [B_1; B_2]).
 * P (nullable): t consecutive blocks [M, F_i] of bf16, block i receiving shard
 * i's pre-activation as tpmlp_fwd's P_save.  Z[M,H] float32: the rank-order sum
 * of the shards' partials (shards one after another, as tpmlp_tp_fwd).
 * Workspace: tpmlp_tp_workspace_bytes(t, M, H, F_i).  t * F_i must be at most
 * 2^23 (TPMLP_ERR_SHAPE). */
tpmlp_status tpmlp_tp_fwd_full(const tpmlp_bf16* X, const tpmlp_bf16* A, const tpmlp_bf16* B,
                               tpmlp_bf16* P, float* Z, int t, int64_t M, int64_t H, int64_t F_i,
                               void* ws, size_t ws_bytes, void* stream);

/* Backward over unsharded weights: dA[H, t F_i] and dB[t F_i, H] (float32) are
 * the whole weight gradients, shard i writing its column block of dA (rows of
 * t F_i elements) and its row block of dB; dX[M,H] is the rank-order sum of the
 * shards' partial input gradients.  P: NULL => every shard recomputes its
 * pre-activation; otherwise the t blocks written by tpmlp_tp_fwd_full. */
tpmlp_status tpmlp_tp_bwd_full(const tpmlp_bf16* dZ, const tpmlp_bf16* X, const tpmlp_bf16* A,
                               const tpmlp_bf16* B, const tpmlp_bf16* P,
                               float* dA, float* dB, float* dX, int t, int64_t M, int64_t H, int64_t F_i,
                               void* ws, size_t ws_bytes, void* stream);

/* out[j] = parts[0][j] + parts[1][j] + ... + parts[t-1][j] (float32, left to right)
 * for j < n: the local stand-in for a sum all-reduce across t ranks
 * ("大模型训练" notes §3.1, the AllReduce of the ranks' Y_i).  `parts` is a host
 * array of t device pointers; n must be a positive multiple of 4.  `out` may not
 * overlap any part. */
tpmlp_status tpmlp_shard_sum(const float* const* parts, int t, float* out, int64_t n, void* stream);

/* ------------------------------------------------------------------------ */
/* The t-shard driver at the sequence-parallel boundary                       */
/* ------------------------------------------------------------------------ */
/* With sequence parallelism the tokens outside the MLP are split by rank: rank
 * r holds the rows [r M/t, (r+1) M/t) of X.  Before the column-parallel product
 * an all-gather gives every rank all M rows, and after the row-parallel product
 * a reduce-scatter leaves rank r the sum over ranks of its own rows of Z; the
 * backward runs the reverse (all-gather of dZ, reduce-scatter of dX).  An
 * all-reduce is a reduce-scatter plus an all-gather, so this costs no extra
 * communication (QLM page §2.1.3 顺序并行; "大模型训练" notes §3.2 序列并行, the
 * all-reduce replaced by all-gather + reduce-scatter; sequence-parallel series
 * §3.2, Megatron's split of the token-wise operations across ranks).
 *
 * These calls take and return the ranks' row slices.  On one GPU the gather is
 * never materialised: each product whose rows are tokens runs once per rank row
 * block, reading that rank's slice directly, and each rank's output slice
 * receives the rank-order sum of the shards' rows in the products' epilogues
 * (shard 0 writes, shards 1 .. t-1 add), which is the reduce-scatter's result.
 * The weight-gradient products contract over all M tokens and read X^T and dZ^T,
 * which are assembled from the slices by the transposes.
 *
 * M must split into t slices of S = M / t rows, S a positive multiple of 8, and
 * H must be at most 2^22 when t > 1 (TPMLP_ERR_SHAPE). */

/* Workspace bytes for tpmlp_sp_fwd and tpmlp_sp_bwd (either backward mode); 0 if
 * the arguments are invalid. */
size_t tpmlp_sp_workspace_bytes(int t, int64_t M, int64_t H, int64_t F_i);

/* Z_sl[r] = rows [r S, (r+1) S) of sum_i GeLU(X A_sh[i]) B_sh[i], for each rank r.
 * X_sl: host array of t device pointers, rank r's tokens X_r[S, H] (bf16).
 * A_sh, B_sh: host arrays of t device pointers (shard i's A_i[H,F_i], B_i[F_i,H]).
 * P_sh (nullable host array; entries nullable): shard i's pre-activation over all
 * M tokens, [M, F_i] bf16 (row block r from rank r's tokens), for a backward that
 * keeps it.
 * Z_sl: host array of t device pointers, rank r's output rows [S, H] float32. */
tpmlp_status tpmlp_sp_fwd(const tpmlp_bf16* const* X_sl, const tpmlp_bf16* const* A_sh,
                          const tpmlp_bf16* const* B_sh, tpmlp_bf16* const* P_sh, float* const* Z_sl,
                          int t, int64_t M, int64_t H, int64_t F_i,
                          void* ws, size_t ws_bytes, void* stream);

/* Backward at the sequence-parallel boundary: dZ_sl[r] and X_sl[r] are rank r's
 * rows [S, H] (bf16); dX_sl[r] receives rank r's rows [S, H] of sum_i dX_i
 * (float32); dA_sh[i], dB_sh[i] are shard i's weight gradients over all M tokens
 * (float32).  P_sh: NULL host array => every shard recomputes P_i; otherwise t
 * device pointers written by tpmlp_sp_fwd (no NULL entries). */
tpmlp_status tpmlp_sp_bwd(const tpmlp_bf16* const* dZ_sl, const tpmlp_bf16* const* X_sl,
                          const tpmlp_bf16* const* A_sh, const tpmlp_bf16* const* B_sh,
                          const tpmlp_bf16* const* P_sh,
                          float* const* dA_sh, float* const* dB_sh, float* const* dX_sl,
                          int t, int64_t M, int64_t H, int64_t F_i,
                          void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* The t-shard driver with FP8 operands                                      */
/* ------------------------------------------------------------------------ */
/* The same products as tpmlp_tp_fwd / tpmlp_tp_bwd with every operand in one of
 * the two 8-bit float formats of the "大模型训练" notes (§6.1 数据类型对比): E4M3
 * (4 exponent, 3 mantissa bits, range +-448) for the activations and weights X,
 * A_i, B_i and G_i, E5M2 (5 and 2 bits, range +-57344) for the gradients dZ and
 * dP_i.  The encodings are the OCP ones those ranges imply (E4M3: bias 7, no
 * infinities; E5M2: bias 15, IEEE specials).  The pages give no scaling recipe;
 * the one used is per-tensor current scaling: a tensor T's scale is
 * s = amax|T| / FMAX (1 if T is all zero), its codes are fp8(T * (1/s)) with the
 * product rounded to float32, then to the nearest FP8 value (ties to even),
 * saturating at +-FMAX; a product of two tensors accumulates the codes'
 * products in float32 and multiplies the sum by the two scales.  G_i is
 * quantized from GeLU of the bf16 pre-activation P_i, dP_i from its bf16 value.
 * Inputs, outputs and the bf16 P_i are as in tpmlp_tp_fwd / tpmlp_tp_bwd (the
 * rank sums of Z and dX are always formed by the drivers, rank order 0..t-1).
 *
 * M, H and F_i must be positive multiples of 16, at most 2^23 (TPMLP_ERR_SHAPE).
 * The workspace (tpmlp_fp8_workspace_bytes, for either call) holds the FP8
 * copies of the operands, the amax slots and the split-K slices.  The forward
 * leaves there what the backward reuses: the codes of X and of every A_i and
 * B_i in both layouts, the codes of G_i^T for every shard whose P_i it stored,
 * and the scales of X, A_i, B_i and G_i; so a backward takes the workspace of
 * the matching forward, unchanged in between (one workspace per forward whose
 * backward is still to run, as for the stored P_i). */
size_t tpmlp_fp8_workspace_bytes(int t, int64_t M, int64_t H, int64_t F_i);

/* Z = sum_i Z_i with FP8 operands.  P_sh: NULL, or t entries (each nullable)
 * receiving P_i [M, F_i] bf16 for a backward that keeps it. */
tpmlp_status tpmlp_fp8_tp_fwd(const tpmlp_bf16* X, const tpmlp_bf16* const* A_sh, const tpmlp_bf16* const* B_sh,
                              tpmlp_bf16* const* P_sh, float* Z, int t, int64_t M, int64_t H, int64_t F_i,
                              void* ws, size_t ws_bytes, void* stream);

/* Backward with FP8 operands: dA_sh[i], dB_sh[i] (float32, shard i's weight
 * gradients) and dX = sum_i dX_i (float32).  P_sh: NULL => every shard
 * recomputes P_i with the FP8 forward product; otherwise t device pointers
 * written by tpmlp_fp8_tp_fwd.  ws: the workspace of the tpmlp_fp8_tp_fwd call
 * with the same X, A_sh, B_sh, t, M, H, F_i (and, with P_sh, the same P_sh),
 * not written since.  The library records each forward's arguments per
 * workspace address on the host (of the 256 latest forwards' workspaces) and
 * returns TPMLP_ERR_NO_FORWARD when they do not match or were not kept; it
 * cannot see a workspace or an input changed in between. */
tpmlp_status tpmlp_fp8_tp_bwd(const tpmlp_bf16* dZ, const tpmlp_bf16* X, const tpmlp_bf16* const* A_sh,
                              const tpmlp_bf16* const* B_sh, const tpmlp_bf16* const* P_sh,
                              float* const* dA_sh, float* const* dB_sh, float* dX, int t, int64_t M, int64_t H,
                              int64_t F_i, void* ws, size_t ws_bytes, void* stream);

/* FP8 codes of one bf16 tensor T[R, C] under the scaling above: *amax (device
 * float, overwritten) receives max|T|, and codes[R, C] (or codes[C, R] with
 * transpose != 0, row-major bytes) its codes in format fmt (0: E4M3, 1: E5M2).
 * R and C positive multiples of 16; T, codes and amax 16-byte aligned. */
tpmlp_status tpmlp_fp8_quantize(const tpmlp_bf16* T, int64_t R, int64_t C, int fmt, int transpose,
                                uint8_t* codes, float* amax, void* stream);

/* ------------------------------------------------------------------------ */
/* Forward without allocation or workspace                                  */
/* ------------------------------------------------------------------------ */

/* Bytes of the library's own device scratch array that tpmlp_fwd_noalloc
 * uses in place of a workspace: 64 MiB per GPU, reserved when the library's
 * code is loaded on that GPU and held until the process ends. */
#define TPMLP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* tpmlp_fwd with no workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same kernels, same launches and the same bits as
 * tpmlp_fwd; the intermediate G_i and any split-K slices live in a file-scope
 * device array of TPMLP_NOALLOC_SCRATCH_BYTES, one per GPU, whose address is
 * looked up once per device (hipGetSymbolAddress) on the first call there.
 * The call allocates nothing and frees nothing.  Nothing in the array has to
 * start at zero: every byte a launch reads was written earlier in the call.
 * Returns TPMLP_ERR_WORKSPACE when tpmlp_fwd_workspace_bytes(M, H, F_i)
 * exceeds TPMLP_NOALLOC_SCRATCH_BYTES.  All calls on one GPU share its array:
 * calls that overlap in time on one GPU (different streams, or different host
 * threads) race and must not be made. */
tpmlp_status tpmlp_fwd_noalloc(const tpmlp_bf16* X, const tpmlp_bf16* A_i, const tpmlp_bf16* B_i,
                               float* Z_i, tpmlp_bf16* P_save,
                               int64_t M, int64_t H, int64_t F_i, void* stream);

/* ------------------------------------------------------------------------ */
/* Kernel timing (measurement aid; not needed to compute anything)           */
/* ------------------------------------------------------------------------ */

/* Kernel kinds that timing distinguishes. */
typedef enum {
  TPMLP_K_FWD_GEMM1_GELU = 0, /* P_i = X A_i, G_i = GeLU(P_i) */
  TPMLP_K_FWD_GEMM2 = 1,      /* Z_i = G_i B_i */
  TPMLP_K_BWD_RECOMPUTE = 2,  /* P_i = X A_i recomputed */
  TPMLP_K_BWD_DGELU = 3,      /* dG_i = dZ B_i^T, dP_i, G_i */
  TPMLP_K_BWD_DB = 4,         /* dB_i = G_i^T dZ */
  TPMLP_K_BWD_DA = 5,         /* dA_i = X^T dP_i */
  TPMLP_K_BWD_DX = 6,         /* dX_i = dP_i A_i^T */
  TPMLP_K_SPLITK_REDUCE = 7,  /* sum of split-K float32 partials */
  TPMLP_K_SHARD_SUM = 8,      /* tpmlp_shard_sum and the drivers' partial sums */
  TPMLP_K_TRANSPOSE = 9,      /* X^T with dZ^T (one launch), dP_i^T, and the weights transposed */
  TPMLP_K_FWD_FUSED = 10,     /* Z_i chunk partials = GeLU(X A_i) B_i in one launch, G in LDS */
  TPMLP_K_FP8_QUANT = 11,     /* FP8 drivers: amax and quantization of operands */
  TPMLP_K_BWD_DB_DX = 12,     /* dB_i and dX_i in one launch (one shape: M = F_i, no running sum) */
  TPMLP_K_COUNT = 13
} tpmlp_kernel_kind;

/* Static name of a kernel kind ("?" if out of range). */
const char* tpmlp_kernel_name(int kind);

/* Start timing every kernel launch the library enqueues on the calling thread,
 * for up to `capacity` launches, with a HIP event pair per launch (events are
 * created here, outside any timed region).  The pair is bound to the launch's
 * kernel dispatches on their stream (hipExtLaunchKernel): it holds the start of
 * the first and the end of the last, and inserts nothing between kernels.
 * Restarting discards earlier records. */
tpmlp_status tpmlp_timing_begin(int capacity);

/* As tpmlp_timing_begin, but only launches of the kinds whose bit (1u << kind)
 * is set in `kinds` are timed and recorded; the others run as with timing off.
 * Each timed launch makes its dispatches report their start and end times,
 * which delays the next kernel by a few microseconds; timing one kind keeps
 * that cost off the rest.  TPMLP_ERR_SHAPE if capacity < 1 or `kinds` is zero
 * or has a bit at or above TPMLP_K_COUNT. */
tpmlp_status tpmlp_timing_begin_kinds(int capacity, unsigned kinds);

/* Stop recording, wait for the recorded events and add up, per kernel kind, the
 * launches (`counts[kind]`) and their total milliseconds (`total_ms[kind]`).
 * Both arrays have TPMLP_K_COUNT entries.  Records beyond `capacity` are dropped
 * and counted in *dropped (nullable). */
tpmlp_status tpmlp_timing_end(int* counts, double* total_ms, int* dropped);

/* The launches recorded by the last tpmlp_timing_begin/end pair, in launch
 * order: kinds[i] and ms[i] for i < min(capacity, count).  Returns the number
 * of records (or -1 if kinds or ms is NULL).  Valid until the next
 * tpmlp_timing_begin on the calling thread. */
int tpmlp_timing_records(int* kinds, double* ms, int capacity);

/* Kernel dispatches inside each of those records, in the same order: 1, or 2
 * for a product planned as whole-wave tiles plus a split tail (one record
 * spans both launches).  Returns the number of records (or -1 if dispatches is
 * NULL).  Lets a profiler's per-dispatch list be matched to the records. */
int tpmlp_timing_dispatches(int* dispatches, int capacity);

#ifdef __cplusplus
}
#endif
#endif /* TPMLP_H_ */
