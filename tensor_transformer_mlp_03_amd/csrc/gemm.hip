// bf16 MFMA GEMM core for gfx950 with the MLP's fused epilogues.
//
// C[m,n] = sum_k A[m,k] B[k,n], bf16 operands, float32 accumulation on the
// bf16 MFMA instructions.  Every product of the tensor-parallel MLP's forward
// and backward is one launch with an operand layout and an epilogue (KC: K
// contiguous; MC: the other dimension contiguous; X^T, dZ^T and, when the
// planner chooses, A_i^T and B_i^T are transposed copies):
//
//   forward   P_i = X A_i          A: KC  B: MC (A_i) or KC (A_i^T)  epilogue GeLU -> G_i (and P_i)
//             Z_i = G_i B_i        A: KC  B: MC (B_i) or KC (B_i^T)  epilogue float32
//   backward  P_i = X A_i          as in the forward, epilogue bf16 (recompute)
//             dG_i = dZ B_i^T      A: KC  B: KC          epilogue dGeLU -> dP_i, G_i^T
//             dB_i = G_i^T dZ      A: KC  B: KC (dZ^T)   epilogue float32 (split-K)
//             dA_i = X^T dP_i      A: KC (X^T)  B: MC    epilogue float32 (split-K)
//             dX_i = dP_i A_i^T    A: KC  B: KC          epilogue float32
//
// (The split of A by columns and B by rows that makes rank i's work exactly
// these products: "大模型训练" notes §3.1; GeLU between the two GEMMs: QLM page
// §2.1.2.2 part 3; fusing the activation into the producing kernel so the
// float32 pre-activation never round-trips through memory: asorrir.com survey,
// part 三, 算子融合.)
//
// One kernel, gemm_x16_kernel, in three tile shapes (256 x 256, 256 x 128, 128 x
// 128): four waves, one per SIMD, each accumulating its sub-tile as 16 x 16
// blocks on v_mfma_f32_16x16x32_bf16, with loads and LDS reads placed between
// its MFMAs (its comment has the schedule).  Design points:
//  * A K-contiguous operand sits in LDS as 128-row slots of [rows][64 k]
//    (128-byte rows), so an MFMA operand fragment is one ds_read_b128 per lane
//    (8 consecutive k of one row); an N-contiguous one as [64 k][128 n] slots,
//    read with two ds_read_b64_tr_b16 per fragment.
//  * Operands go from memory straight into LDS with buffer_load ... lds (16
//    bytes per lane, no staging registers, no LDS write instructions).  Buffer
//    descriptors return zeros for out-of-range chunks, which handles ragged
//    sizes without branches.
//  * 16-byte chunks are XOR-swizzled within LDS rows so that the lanes of one
//    read instruction fall on distinct banks; the DMA loads apply the inverse
//    permutation on the memory side, so each DMA still writes 1 KiB of
//    contiguous LDS.
//  * The MFMA takes the B fragment as its first operand, so each lane ends with
//    4 consecutive output columns of one row; the epilogue restages them
//    through LDS and stores whole 128-byte lines.
//  * Workgroups are renumbered so that consecutive output tiles (which share
//    operand panels) run on the same XCD and its L2, then grouped 4 tiles tall.

#include "common.h"
#include "epilogue.h"

namespace tpmlp {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// Rows of tiles per group of the grouped order: an XCD's 32 co-resident tiles span
// 4 rows x 8 columns of tiles (measured 1% faster than 8 x 4 and 2 x 16).
constexpr int GROUP_M = 4;
constexpr int NUM_XCD = 8;
constexpr uint32_t OOB = 0x7FFFFFF0u;  // voffset past num_records: the load returns 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)OOB, 0x00020000);
}

// ds_read_b64_tr_b16 from LDS address `p`.  Issued through inline assembly:
// the builtin makes the compiler wait for every vector-memory load in flight
// (vmcnt(0)) before it, in case an LDS-DMA load targets the same bytes, which
// would stall the load pipeline of this kernel on every memory phase (30 such
// waits in the main loop of the N-contiguous kernels with this compiler).
// Callers read only bytes whose loads and writes have already been waited for
// and made visible by a barrier, and wait for the results themselves
// (lgkmcnt(0)) before using them.  The compiler takes the output register as
// written when the statement issues, so no result may be left unused (its
// register could be handed out again while the read is in flight): every one
// is a fragment that the MFMAs after that wait consume.
typedef __attribute__((address_space(3))) char lds_char_t;
__device__ __forceinline__ i16x4_t ds_read_tr(const char* p) {
  i16x4_t v;
  const uint32_t a = (uint32_t)(uintptr_t)(const lds_char_t*)p;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(a));
  return v;
}
// The same through the builtin, for the epilogue: no LDS-DMA load is in flight
// there, so the compiler orders the read after the wave's own LDS stores and
// waits for its result by itself, without waiting for the global loads.
__device__ __forceinline__ i16x4_t ds_read_tr_lds(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(const lds_char_t*)p);
}

// ---------------------------------------------------------------------------
// Pieces of the 16 x 16 x 32 kernel (gemm_x16_kernel)
// ---------------------------------------------------------------------------

// N-contiguous slot of the 16 x 16 x 32 kernel: 64 k-rows of 128 n, 256-byte rows.
// The 16-byte chunk holding n .. n+7 of k-row k sits at (n / 8) ^ (4 (k % 4) + 2
// ((k / 8) % 2)).  A transposing fragment read takes, per 16-lane group, 4
// consecutive k-rows x 32 bytes, and the LDS serves two groups per cycle whose
// k-rows lie 8 apart: the first term puts a group's 4 rows on distinct banks
// (unswizzled, rows 256 bytes apart hit the same ones), the second moves the
// other group's to the remaining banks.
__device__ __forceinline__ int mc16_x(int k) { return 4 * (k & 3) + 2 * ((k >> 3) & 1); }
__device__ __forceinline__ int mc16_off(int k, int n) { return k * 256 + (((n >> 3) ^ mc16_x(k)) << 4) + (n & 7) * 2; }

// K-contiguous [128 rows][64 k] slot of the 16 x 16 x 32 kernel: the 16-byte chunk c
// of row r sits at position c ^ ((r / 2) % 8).  The XOR depends on r % 16 only, so
// the 16-row fragments of a slot differ by a constant 2048 bytes (one base register
// per lane serves all of them), and the 16 rows of a fragment read at one chunk
// land on distinct 16-byte bank groups (even rows on 8 positions in one half of
// the banks, odd rows on 8 in the other).
__device__ __forceinline__ int swz16(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int tile16_off(int r, int c) { return r * 128 + ((c ^ swz16(r)) << 4); }

// LDS-DMA loads of one 128-row K-contiguous quarter of a K step: 4 instructions per
// wave of 1 KiB, instruction i of wave w filling rows 8 (4i + w) .. +7 of the slot;
// lane q writes position q % 8 of row q / 8 and loads the chunk the swizzle places
// there, which depends on the lane and w % 2 only.  Each lane's byte offset from
// the quarter's (first row, first k of the step) is computed once per tile, with
// lanes whose row is outside the operand set to OOB, so the only per-step masking
// left is that of a K tail.
struct QuarterKC {
  uint32_t voff[4];  // instruction i
  int kc;            // first k of the lane's chunk inside the K step

  __device__ __forceinline__ void init(int64_t ld, int rows_left, int w, int lane) {
    kc = 8 * ((lane & 7) ^ swz16(8 * w + (lane >> 3)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * (4 * i + w) + (lane >> 3);
      voff[i] = r < rows_left ? (uint32_t)(((int64_t)r * ld + kc) * 2) : OOB;
    }
  }
  // rs: descriptor based at the quarter's (first row, first k of the step); k_left:
  // elements of K from the step's first k (64 or more: no tail).
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, char* slot, int k_left, int w, int i) const {
    const uint32_t off = kc < k_left ? voff[i] : OOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(slot + (4 * i + w) * 1024), 16, off, 0, 0, 0);
  }
};

// The same for an N-contiguous quarter (64 k-rows x 128 n, mc16_off layout):
// instruction i of wave w fills k-rows 4 (4i + w) .. +3; lane q writes position
// q % 16 of k-row q / 16 and loads the chunk placed there, which depends on the
// lane and on w / 2 only.
struct QuarterMC {
  uint32_t voff[4];
  int lane_k;  // k-row of the lane's chunk in instruction 0

  __device__ __forceinline__ void init(int64_t ld, int n_left, int w, int lane) {
    lane_k = 4 * w + (lane >> 4);
    const int n = 8 * ((lane & 15) ^ mc16_x(lane_k));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      voff[i] = n < n_left ? (uint32_t)(((int64_t)(lane_k + 16 * i) * ld + n) * 2) : OOB;
  }
  // rs: descriptor based at the quarter's (first k of the step, first n).
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, char* slot, int k_left, int w, int i) const {
    const uint32_t off = lane_k + 16 * i < k_left ? voff[i] : OOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(slot + (4 * i + w) * 1024), 16, off, 0, 0, 0);
  }
};

// Byte offset of lane `lane`'s first transposing read of the 16 x 16 x 32 B
// fragment at columns n0 .. n0+15 of an N-contiguous half, sub-step 0: in 16-lane
// group g, source lane s reads k-row 8g + s / 4, columns n0 + 4 (s % 4) .. +3, and
// ds_read_b64_tr_b16 hands lane i of the group the 4 k-values of column n0 + i.
// The second read (k-rows + 4) is 1024 bytes further, sub-step 1 (k + 32) 8192.
__device__ __forceinline__ uint32_t mc16_lane_off(int n0, int lane) {
  const int g = lane >> 4, sl = lane & 15;
  return mc16_off(8 * g + (sl >> 2), n0 + 4 * (sl & 3));
}

// Logical tile of workgroup `bid`: XCD-aware renumbering, then grouped order.
__device__ __forceinline__ void tile_of(int bid, int nblocks, int tiles_m, int tiles_n, int& tm, int& tn,
                                        int& split) {
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

// Epilogue.  With the B fragment as the MFMA's first operand, accumulator
// register r of fragment (i, j) holds C[32i + lane%32][32j + 8(r/4) + 4(lane/32) + r%4]
// of the wave's sub-tile.  Each wave stages 64 rows of its float32 sub-tile
// at a time in LDS (row stride 256 bytes, 16-byte chunks XOR-swizzled by the
// row), reads them back row-contiguous and finishes 8 (bf16 outputs) or 4
// (float32) consecutive columns per lane, so every store instruction writes
// whole 128-byte lines.
// `stage` is this wave's 16 KiB of LDS, free of operand data; row_w and col_w
// are the first output row and column of the wave's (32 FM) x 64 tile.
constexpr int ROW_B = 256;  // staged row stride in bytes (64 float32)

// The dGeLU epilogue keeps the bf16 G rows of a chunk in its staging bytes at a
// 128-byte pitch (rows 2i and 2i+1 share one 256-byte line, so a store of two
// rows covers all 64 banks), 16-byte chunks swizzled by the row.  A transposing
// read of a 16-lane group takes rows b + 8 q + r (q, r < 4; b a multiple of 32)
// at one column chunk: for each parity of r those are 8 rows, and the swizzle
// puts them on 8 distinct chunks (one bank half per parity); the two groups that
// share a 32-lane half read different 8-byte halves of their chunks, so every
// read and store is free of bank conflicts.
__device__ __forceinline__ int gt_swz(int r) { return ((r >> 3) + 4 * ((r >> 1) & 1)) & 7; }
constexpr int G_ROW_B = 128;  // staged G row pitch in bytes

// The epilogue proper, independent of the MFMA accumulator layout.  The wave's
// region is NC chunks of 64 x 64, laid out nh chunks tall: chunk c covers rows
// row_w + 64 (c % nh) and columns col_w + 64 (c / nh) onward.  stage_chunk(c, sc)
// writes the chunk's float32 values (times sc for FP8 products, scale_fn() the
// product of the operands' scales) into `stage` (row r in 0..63 at r * ROW_B,
// 16-byte chunk q in 0..15 at position q ^ (r & 15)), and the chunk is finished
// from there.
// FP8 (FP8 products): EPI_BF16 and EPI_DGELU also collect the amax of what they
// write into args.amax_out when set (of the GeLU of the written values with
// args.amax_gelu), and EPI_DGELU writes dP only (no G^T).
// Paired products (EPI_F32_PAIR, EPI_F32_ACC_PAIR): stage_chunk2(c) writes product
// 1's values of chunk c the same way into `stage2`, and each output element is
// (running sum + product 0) + product 1, in that order.
template <int EPI, int NC, bool FP8, class StageChunk, class ScaleFn, class StageChunk2>
__device__ __forceinline__ void store_staged(StageChunk&& stage_chunk, ScaleFn&& scale_fn, const GemmArgs& args,
                                             char* stage, int row_w, int col_w, int nh, int split, int lane,
                                             StageChunk2&& stage_chunk2, char* stage2) {
  constexpr bool PAIR = EPI == EPI_F32_PAIR || EPI == EPI_F32_ACC_PAIR;
  constexpr bool ACC = EPI == EPI_F32_ACC || EPI == EPI_F32_ACC_PAIR;
  // FP8: running extremes of the written values (AmaxTrack, epilogue.h; invalid
  // elements enter as 0), updated without branches.
  AmaxTrack am;
  // Each phase below issues all of its memory operations before it waits for
  // any, and the global loads an epilogue needs (the dGeLU pre-activations, the
  // EPI_F32_ACC running sum) are double-buffered: chunk c + 1's are in flight
  // while chunk c is finished, so only the first chunk's latency is exposed.
  // LDS reads are batched ahead of the stores that use them.  Both loads go
  // through a buffer descriptor on the chunk's (uniform) first row and column,
  // so rows and columns outside the output read as zero without a branch.
  u16x8_t pre[2][8];
  f32x4_t old[2][16];
  auto row0 = [&](int c) { return row_w + 64 * (c % nh); };
  auto col0 = [&](int c) { return col_w + 64 * (c / nh); };
  auto load_old = [&](int c) {
    const int r0 = row0(c), c0 = col0(c);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(reinterpret_cast<const float*>(args.out) + (int64_t)r0 * args.ldo + c0);
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int q = it * 64 + lane, r = q >> 4, cq = q & 15;
      const bool ok = r0 + r < args.M && c0 + 4 * cq < args.N;
      const uint32_t off = (uint32_t)(((int64_t)r * args.ldo + 4 * cq) * 4);
      old[c & 1][it] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? off : OOB, 0, 0));
    }
  };
  auto load_pre = [&](int c) {
    const int r0 = row0(c), c0 = col0(c);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(args.aux + (int64_t)r0 * args.ldo + c0);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int q = it * 64 + lane, r = q >> 3, cp = q & 7;
      const bool ok = r0 + r < args.M && c0 + 8 * cp < args.N;  // N % 8 == 0: 8 columns in or out together
      const uint32_t off = (uint32_t)(((int64_t)r * args.ldo + 8 * cp) * 2);
      pre[c & 1][it] = __builtin_bit_cast(u16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? off : OOB, 0, 0));
    }
  };
  // The loads stay where they are issued: a scheduling barrier after each batch
  // keeps the compiler from sinking them to their uses (one round trip each)
  // when registers run short.
  if (EPI == EPI_DGELU) load_pre(0);
  // (Paired launches hold two staged products: their running-sum loads are not
  // double-buffered, which leaves the registers that holds.)
  if (ACC && !PAIR) load_old(0);
  __builtin_amdgcn_sched_barrier(0);
  // FP8: the product of the operands' scales, which stage_chunk applies (taken
  // after the first loads are issued, so that the scales' load overlaps them).
  const float sc = FP8 ? scale_fn() : 1.0f;
#pragma unroll
  for (int ch = 0; ch < NC; ++ch) {
    const int h = ch % nh;  // used by the stores below through row_w + 64 * h
    const int col_c = col0(ch);
    if (ACC && PAIR) {
      load_old(ch);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (ACC && !PAIR && ch + 1 < NC) {
      load_old(ch + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    stage_chunk(ch, sc);
    if (PAIR) stage_chunk2(ch);
    if (EPI == EPI_DGELU && ch + 1 < NC) {
      load_pre(ch + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (EPI == EPI_F32 || ACC || PAIR) {
      const bool final_out = args.k_split >= args.K;  // not a split-K slice
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(reinterpret_cast<float*>(args.out) +
                                                  (int64_t)split * args.split_stride +
                                                  (int64_t)(row_w + 64 * h) * args.ldo + col_c);
      // Two batches of 8 vectors: with both running-sum buffers live, 16 would
      // not fit beside the accumulators.
#pragma unroll
      for (int b8 = 0; b8 < 16; b8 += 8) {
        f32x4_t xs[8], ys[PAIR ? 8 : 1];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int q = (b8 + u) * 64 + lane, r = q >> 4, c = q & 15;
          xs[u] = *reinterpret_cast<const f32x4_t*>(stage + r * ROW_B + ((c ^ (r & 15)) << 4));
          if constexpr (PAIR) ys[u] = *reinterpret_cast<const f32x4_t*>(stage2 + r * ROW_B + ((c ^ (r & 15)) << 4));
        }
        __builtin_amdgcn_sched_barrier(0);  // the reads stay one batch
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int it = b8 + u, q = it * 64 + lane, r = q >> 4, c = q & 15;
          const bool ok = row_w + 64 * h + r < args.M && col_c + 4 * c < args.N;
          if (ACC) xs[u] += old[ch & 1][it];
          if constexpr (PAIR) xs[u] += ys[u];
          const uint32_t off = (uint32_t)(((int64_t)r * args.ldo + 4 * c) * 4);
          if (final_out)  // non-temporal: a final output is not read again by this launch
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, xs[u]), rs, ok ? off : OOB, 0, 2);
          else
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, xs[u]), rs, ok ? off : OOB, 0, 0);
        }
      }
    } else {
      const int64_t base = (int64_t)(row_w + 64 * h) * args.ldo + col_c;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(reinterpret_cast<uint16_t*>(args.out) + base);
      f32x4_t x0s[8], x1s[8];
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int q = it * 64 + lane, r = q >> 3, cp = q & 7;
        x0s[it] = *reinterpret_cast<const f32x4_t*>(stage + r * ROW_B + (((2 * cp) ^ (r & 15)) << 4));
        x1s[it] = *reinterpret_cast<const f32x4_t*>(stage + r * ROW_B + (((2 * cp + 1) ^ (r & 15)) << 4));
      }
      __builtin_amdgcn_sched_barrier(0);  // the reads stay one batch
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int q = it * 64 + lane, r = q >> 3, cp = q & 7;
        const float x[8] = {x0s[it][0], x0s[it][1], x0s[it][2], x0s[it][3],
                            x1s[it][0], x1s[it][1], x1s[it][2], x1s[it][3]};
        const bool ok = row_w + 64 * h + r < args.M && col_c + 8 * cp < args.N;  // N % 8 == 0
        const uint32_t off = ok ? (uint32_t)(((int64_t)r * args.ldo + 8 * cp) * 2) : OOB;
        auto store = [&](const __amdgpu_buffer_rsrc_t& rd, const u16x8_t& v) {
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rd, off, 0, 0);
        };
        u16x8_t v1, v2;
        if (EPI == EPI_GELU) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            v1[e] = epi_gelu(x[e]);
            v2[e] = f32_to_bf16(x[e]);
          }
          store(rs, v1);
          if (args.out2) store(make_rsrc(args.out2 + base), v2);
        } else if (EPI == EPI_BF16) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v1[e] = f32_to_bf16(x[e]);
          store(rs, v1);
          if (FP8) {
#pragma unroll
            for (int e = 0; e < 8; ++e) am.add(ok ? bf16_to_f32(v1[e]) : 0.0f);
          }
        } else if (FP8) {  // EPI_DGELU of an FP8 product: dP and its amax
#pragma unroll
          for (int e = 0; e < 8; ++e) v1[e] = f32_to_bf16(dgelu_f32(x[e], pre[ch & 1][it][e]));
          store(rs, v1);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = ok ? bf16_to_f32(v1[e]) : 0.0f;
            am.v_max = fmaxf(am.v_max, v);
            am.v_min = fminf(am.v_min, v);
          }
        } else {  // EPI_DGELU
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const DGelu d = epi_dgelu(x[e], pre[ch & 1][it][e]);
            v1[e] = d.dp;
            v2[e] = d.g;
          }
          store(rs, v1);
          // Keep G of this row in LDS, over the chunk's float32 values (the
          // wave has read all of them above, and its LDS accesses complete in
          // order), at G_ROW_B pitch, 16-byte chunks swizzled by the row
          // (gt_swz).  Rows and columns outside the output hold values that no
          // transposed store below reads.
          *reinterpret_cast<u16x8_t*>(stage + r * G_ROW_B + ((cp ^ gt_swz(r)) << 4)) = v2;
        }
      }
      if (EPI == EPI_DGELU && !FP8) {
        // Transposed store of G in whole 128-byte lines.  ds_read_b64_tr_b16
        // takes, in each 16-lane group, 4 rows x 16 columns (source lane 4 r + q:
        // row r, columns 4 q .. +3) and hands lane i column i.  Source lane
        // 4 r + q reads the 4 columns 8 it + 4 (g % 2) .. +3 of G row
        // m0(q) + r, with m0(q) = 32 (g / 2) + 8 q, so lane 4 q + e receives
        // rows m0(q) .. +3 of column 8 it + 4 (g % 2) + e; a second read gives
        // rows +4 .. +7.  The 8 lanes (g / 2, q) of a column then hold its 64
        // rows: one store instruction writes 8 columns x 128 bytes of G^T.  All
        // eight steps are read first, then stored.
        const int g = lane >> 4, j = lane & 15, jq = j & 3, jr = j >> 2;
        const int half = (g & 1) ? 8 : 0;
        i16x4_t lo[8], hi[8];
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const int ka = 32 * (g >> 1) + 8 * jq + jr, kb = ka + 4;  // source role: q = jq, r = jr
          lo[it] = ds_read_tr_lds(stage + ka * G_ROW_B + ((it ^ gt_swz(ka)) << 4) + half);
          hi[it] = ds_read_tr_lds(stage + kb * G_ROW_B + ((it ^ gt_swz(kb)) << 4) + half);
        }
        const int m0 = row_w + 64 * h;
        const __amdgpu_buffer_rsrc_t rt = make_rsrc(args.out2 + (int64_t)col_c * args.ldt + m0);
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          // destination role: lane 4 q + e with q = jr, e = jq
          const int fo = 8 * it + 4 * (g & 1) + jq, mo = 32 * (g >> 1) + 8 * jr;
          const bool ok = col_c + fo < args.N && m0 + mo < args.M;
          const uint32_t off = (uint32_t)(((int64_t)fo * args.ldt + mo) * 2);
          const u16x8_t v = {(uint16_t)lo[it][0], (uint16_t)lo[it][1], (uint16_t)lo[it][2], (uint16_t)lo[it][3],
                             (uint16_t)hi[it][0], (uint16_t)hi[it][1], (uint16_t)hi[it][2], (uint16_t)hi[it][3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rt, ok ? off : OOB, 0, 0);
        }
      }
    }
  }
  if (FP8 && (EPI == EPI_BF16 || EPI == EPI_DGELU) && args.amax_out)
    slot_max(args.amax_out, AMAX_SUB, am.result(EPI == EPI_BF16 && args.amax_gelu));
}

}  // namespace

// The kernel has external linkage (a kernel template in an anonymous namespace
// does not get its host launch stubs emitted for every instantiation).
namespace kern {

// BM x BN tile (256 x 256, 256 x 128 or 128 x 128) on v_mfma_f32_16x16x32_bf16.
// The LDS is a ring of ten 16 KiB slots, each one 128-row (or 128-column)
// quarter of a K step (64): A's BM / 128 quarters, then B's BN / 128.  Wave (wm,
// wn) computes a (BM / 2) x (BN / 2) sub-tile as FI x FJ blocks of 16 x 16 (FI =
// BM / 32, FJ = BN / 32: 256, 128 or 64 accumulator registers).  A K step is two
// sub-steps of 32 k; in each a wave issues FI FJ MFMAs of 16 cycles and, between
// them, the LDS reads of the next sub-step's fragments and one batch of loads for
// step k+D (D = 2 for 256-row tiles, whose steps take four slots; D = 4 for 128 x
// 128, whose steps take two):
//   sub-step 0 of step k: the A quarters of step k+D (into slots of step k-1,
//         which no wave reads any more)
//   then: wait until the next sub-step's fragments are in registers and step k+1
//         has landed (vmcnt: only loads issued after step k+1's may be in
//         flight); barrier
//   sub-step 1 of step k: the B quarters of step k+D (256-row tiles: into step
//         k's first slots, which no wave reads after the barrier), and the reads
//         of step k+1's sub-step 0.
// The next sub-step's B fragments go to the other half of a double buffer; an A
// fragment is reloaded as soon as its row of MFMAs has been issued (MFMAs run
// row by row), so A needs no second buffer.  The deeper prefetch of the small
// tile covers memory latency over its shorter K steps (a quarter of the MFMAs).
template <int LB, int EPI, int BM, int BN, int F8>
__global__ void __launch_bounds__(256)
gemm_x16_kernel(GemmArgs args_in) {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert((BM == 256 && (BN == 256 || BN == 128)) || (BM == 128 && BN == 128), "tile shapes");
  static_assert(F8 == 0 || LB == KC, "FP8 operands are K-contiguous");
  // Paired products (EPI_F32_PAIR, EPI_F32_ACC_PAIR): two accumulator sets, which
  // only the 256 x 128 and 128 x 128 tiles have registers for.
  constexpr bool PAIR = EPI == EPI_F32_PAIR || EPI == EPI_F32_ACC_PAIR;
  static_assert(!PAIR || (F8 == 0 && BN == 128), "paired products: bf16, 256 x 128 or 128 x 128 tiles");
  static_assert(8 * 64 * ROW_B <= 160 * 1024, "two staging regions per wave fit the LDS");
  constexpr int BK = TILE_BK;
  constexpr int SLOT = 128 * BK * 2;
  constexpr int NA = BM / 128;              // A quarters (128 rows x BK) per K step
  constexpr int NQ = NA + BN / 128;         // quarters loaded per K step
  constexpr int NSLOT = 10;
  constexpr int SPS = BM == 128 ? 2 : 4;    // ring slots per K step
  constexpr int P = 5;                      // ring period in K steps (SPS P = 0 mod 10)
  // Prefetch distance in K steps: as far as the ring allows.  Step k+D takes
  // step k-1's last slots (free once every wave has passed step k-1's mid-step
  // barrier) and, for 256-row tiles, step k's first ones (free after step k's).
  // (Packing 256 x 128 steps into three slots for a distance of 3 needs a
  // period of 10 steps, and measured slower.)
  constexpr int D = BM == 128 ? 4 : 2;
  constexpr int QS0 = BM == 128 ? 1 : 2;    // quarters of step k+D loaded in sub-step 0
  constexpr int FI = BM / 32, FJ = BN / 32;  // 16 x 16 blocks per wave: FI x FJ
  static_assert(BK == 64 && NSLOT * SLOT == 160 * 1024, "ten 16 KiB slots fill the LDS");
  __shared__ __attribute__((aligned(1024))) char smem[NSLOT * SLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  int tm, tn, split;
  tile_of(blockIdx.x, gridDim.x, args_in.tiles_m, args_in.tiles_n, tm, tn, split);
  // A batched launch is unsplit: the "split" index names the workgroup's product.
  GemmArgs args = args_in;
  if (args_in.batch > 1) {
    const int j = split;
    split = 0;
    args.a = args_in.a_arr[j];
    args.b = args_in.b_arr[j];
    args.out = args_in.out_arr[j];
    args.out2 = args_in.out2_arr[j];
    args.aux = args_in.aux_arr[j];
  }
  if (PAIR) {  // product 0's operands; product 1's are a_arr[1] and b_arr[1]
    args.a = args_in.a_arr[0];
    args.b = args_in.b_arr[0];
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int k_begin = split * args.k_split;
  const int k_end = min(args.K, k_begin + args.k_split);
  const int nk = (k_end - k_begin + BK - 1) / BK;
  // K steps of the whole loop: product 1 (paired launches) follows product 0's nk.
  const int nk_all = PAIR ? 2 * nk : nk;

  QuarterKC qa[NA], qb[BN / 128];
  QuarterMC qm[BN / 128];
#pragma unroll
  for (int q = 0; q < NA; ++q) qa[q].init(args.lda, args.M - m0 - 128 * q, wave, lane);
#pragma unroll
  for (int q = 0; q < NQ - NA; ++q) {
    if (LB == KC) qb[q].init(args.ldb, args.N - n0 - 128 * q, wave, lane);
    else qm[q].init(args.ldb, args.N - n0 - 128 * q, wave, lane);
  }

  auto slot = [&](int r, int q) -> char* { return smem + ((SPS * r + q) % NSLOT) * SLOT; };
  // Instruction i of this wave's share of quarter q of K step `step` (r = step % P).
  // Paired launches: steps nk .. 2 nk - 1 are product 1's steps 0 .. nk - 1.
  auto load = [&](int step, int r, int q, int i) {
    if (q >= NQ) return;
    const bool second = PAIR && step >= nk;
    const int k = k_begin + (second ? step - nk : step) * BK;
    const uint16_t* pa = second ? args_in.a_arr[1] : args.a;
    const uint16_t* pb = second ? args_in.b_arr[1] : args.b;
    char* dst = slot(r, q);
    if (q < NA) {
      qa[q].issue(make_rsrc(pa + (int64_t)(m0 + 128 * q) * args.lda + k), dst, k_end - k, wave, i);
    } else if (LB == KC) {
      qb[q - NA].issue(make_rsrc(pb + (int64_t)(n0 + 128 * (q - NA)) * args.ldb + k), dst, k_end - k, wave, i);
    } else {
      qm[q - NA].issue(make_rsrc(pb + (int64_t)k * args.ldb + n0 + 128 * (q - NA)), dst, k_end - k, wave, i);
    }
  };

  f32x4_t acc[FI][FJ];
  f32x4_t acc2[PAIR ? FI : 1][PAIR ? FJ : 1];  // product 1's (paired launches)
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // (acc2 is cleared where product 1 starts, so that it holds no registers before.)

  if constexpr (F8 == 0) {
  bf16x8_t fa[FI], fb[2][FJ];
  // K-contiguous fragment f (rows 16f .. +15 of a 128-row quarter) in sub-step kk:
  // lane l reads row 16f + l % 16, 16-byte chunk 4kk + l / 16, at lane_kc[kk] + 2048 f.
  uint32_t lane_kc[2], lane_mc[FJ];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) lane_kc[kk] = tile16_off(lane & 15, 4 * kk + (lane >> 4));
  const int wcol = BN == 256 ? 0 : 64 * wn;  // the wave's first column inside its B quarter
#pragma unroll
  for (int j = 0; j < FJ; ++j) lane_mc[j] = mc16_lane_off(wcol + 16 * j, lane);
  // A fragment f of the wave: rows 16 f of its quarter (BM = 256: quarter wm),
  // or of its half of the one quarter (BM = 128: rows 64 wm + 16 f).
  auto read_a = [&](int r, int kk, int f) {
    const char* ta = BM == 256 ? slot(r, wm) + 2048 * f : slot(r, 0) + 2048 * (4 * wm + f);
    fa[f] = *reinterpret_cast<const bf16x8_t*>(ta + lane_kc[kk]);
  };
  auto read_b = [&](int buf, int r, int kk, int j) {
    const char* tb = slot(r, BN == 256 ? NA + wn : NA);
    if (LB == KC) {
      const int f = (BN == 256 ? 0 : 4 * wn) + j;  // 16-row block of the B quarter
      fb[buf][j] = *reinterpret_cast<const bf16x8_t*>(tb + lane_kc[kk] + 2048 * f);
    } else {
      const char* p = tb + lane_mc[j] + 8192 * kk;
      const i16x4_t lo = ds_read_tr(p), hi = ds_read_tr(p + 1024);
      const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      fb[buf][j] = __builtin_bit_cast(bf16x8_t, v);
    }
  };
  constexpr int NB = LB == KC ? FJ : 2 * FJ;  // LDS read instructions for the B fragments
  // acc += A B for one 16 x 16 block, the B fragment as the first operand.  Inline
  // assembly ties the accumulator to one AGPR quadruple for the whole K loop (the
  // builtin's results were moved between registers every iteration at this
  // register pressure).  The compiler still waits for the LDS reads that produce
  // the operands; the accumulators are next read by the epilogue, after explicit
  // wait states.
  auto mfma16 = [](f32x4_t& c, const bf16x8_t& b, const bf16x8_t& a) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a));
  };

  // One sub-step: the MFMAs on fa and fb[cur], row by row; with `reads`, the next
  // sub-step's fragments (ring position rn, sub-step kn): B into fb[1 - cur] during
  // row 0, A fragment f right after row f's MFMAs (its old value has then fed its
  // last MFMA).  Load n of the sub-step's NL goes after MFMA 1 (and FJ/2 + 1 for a
  // second) of row n * FI / NL.  Every MFMA with the reads and loads placed after it
  // is its own scheduling region, so the order is exactly this one.
  auto sub_step = [&](auto& C, int cur, bool reads, int rn, int kn, auto nl, auto&& issue_load) {
    constexpr int NL = decltype(nl)::value;
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      int n_row = 0, n_first = 0;  // loads of this row and the first one's index
#pragma unroll
      for (int n = NL - 1; n >= 0; --n)
        if (n * FI / NL == i) {
          ++n_row;
          n_first = n;
        }
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        mfma16(C[i][j], fb[cur][j], fa[i]);
        if (reads && i == 0) {
#pragma unroll
          for (int u = 0; u < NB / FJ; ++u) {
            const int jb = j * (NB / FJ) + u;  // B read jb: fragment jb / (NB / FJ), half jb % (NB / FJ)
            if (NB == FJ || u == NB / FJ - 1) read_b(1 - cur, rn, kn, jb / (NB / FJ));
          }
        }
        if (j == 1 && n_row >= 1) issue_load(n_first);
        if (j == FJ / 2 + 1 && n_row >= 2) issue_load(n_first + 1);
        if (j == FJ - 1 && reads) read_a(rn, kn, i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  auto vm_wait = [&](auto n) {
    constexpr int N = decltype(n)::value;
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  };
  using L0 = std::integral_constant<int, 0>;
  constexpr int HALF_LOADS = 4 * QS0;          // sub-step 0's quarters: 4 instructions each
  constexpr int TAIL_LOADS = 4 * (NQ - QS0);    // sub-step 1's
  constexpr int STEP_LOADS = HALF_LOADS + TAIL_LOADS;
  static_assert((D - 1) * STEP_LOADS < 64, "vmcnt");

  if (nk_all > 0) {
    // Prologue: steps 0 .. D-1 (as many as there are); wait for step 0.
#pragma unroll
    for (int st = 0; st < D; ++st)
      if (st < nk_all) {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) load(st, st, q, i);
      }
    if (D >= 4 && nk_all >= 4) vm_wait(std::integral_constant<int, (D >= 4 ? 3 : 0) * STEP_LOADS>{});
    else if (D >= 3 && nk_all >= 3) vm_wait(std::integral_constant<int, (D >= 3 ? 2 : 0) * STEP_LOADS>{});
    else if (nk_all >= 2) vm_wait(std::integral_constant<int, STEP_LOADS>{});
    else vm_wait(L0{});
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < FJ; ++j) read_b(0, 0, 0, j);
#pragma unroll
    for (int f = 0; f < FI; ++f) read_a(0, 0, f);

    // K step k with LEFT = min(D, steps after it) known at compile time; r = k % P;
    // C the accumulator set of the step's product.
    auto k_step = [&](int k, auto left, int r, auto& C) {
      constexpr int LEFT = decltype(left)::value;
      const int r1 = r == P - 1 ? 0 : r + 1, rd = (r + D) % P;
      // sub-step 0: reads sub-step 1 of this step; loads the quarters of step k+D
      // whose slots step k does not use
      sub_step(C, 0, true, r, 1, std::integral_constant<int, LEFT >= D ? HALF_LOADS : 0>{},
               [&](int n) { load(k + D, rd, n >> 2, n & 3); });
      if constexpr (LEFT >= 1) {
        // Step k+1 has landed once at most the loads issued after its own are
        // in flight: whole steps k+2 .. k+D-1 and the part of step k+D just issued.
        constexpr int WHOLE = LEFT - 1 < D - 2 ? LEFT - 1 : D - 2;
        constexpr int AFTER = STEP_LOADS * (WHOLE > 0 ? WHOLE : 0) + (LEFT >= D ? HALF_LOADS : 0);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): sub-step 1's fragments are in registers
        vm_wait(std::integral_constant<int, AFTER>{});
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
      // sub-step 1: reads sub-step 0 of step k+1; loads the rest of step k+D (for
      // 256-row tiles into step k's first slots)
      sub_step(C, 1, LEFT >= 1, r1, 0, std::integral_constant<int, LEFT >= D ? TAIL_LOADS : 0>{},
               [&](int n) { load(k + D, rd, QS0 + (n >> 2), n & 3); });
    };
    using Full = std::integral_constant<int, D>;
    int k = 0;
    if constexpr (PAIR) {
      // Product 0: steps 0 .. nk - 1 into acc, each with D or more steps after it
      // (the host pairs products of at least D K steps).
      for (; k + P <= nk; k += P) {
#pragma unroll
        for (int u = 0; u < P; ++u) k_step(k + u, Full{}, u, acc);
      }
      for (; k < nk; ++k) k_step(k, Full{}, k % P, acc);
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) acc2[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // The rest (product 1's steps into acc2 for paired launches), the last D
    // steps (or all of them, if fewer) each with its own LEFT.
    auto rest = [&](auto& C) {
      if constexpr (PAIR) {
        // Whole ring periods with the ring position known at compile time (both
        // accumulator sets are live here, and run-time positions cost registers);
        // the steps before nk and from the tail on are skipped.
        const int stop = nk_all - D;
        for (int k0 = nk - nk % P; k0 < stop; k0 += P) {
#pragma unroll
          for (int u = 0; u < P; ++u)
            if (k0 + u >= nk && k0 + u < stop) k_step(k0 + u, Full{}, u, C);
        }
      } else {
        for (; k + P + D <= nk_all; k += P) {  // steps k .. k+P-1, each with D more after it
#pragma unroll
          for (int u = 0; u < P; ++u) k_step(k + u, Full{}, u, C);
        }
        for (; k + D < nk_all; ++k) k_step(k, Full{}, k % P, C);
      }
      auto tail = [&](auto jc) {
        constexpr int J = decltype(jc)::value;
        if constexpr (J < D) {
          if (nk_all >= J + 1) k_step(nk_all - 1 - J, std::integral_constant<int, J>{}, (nk_all - 1 - J) % P, C);
        }
      };
      tail(std::integral_constant<int, 3>{});
      tail(std::integral_constant<int, 2>{});
      tail(std::integral_constant<int, 1>{});
      tail(std::integral_constant<int, 0>{});
    };
    if constexpr (PAIR) rest(acc2);
    else rest(acc);
    vm_wait(L0{});
  }
  } else {
    // FP8 operands (formats FA of A, FB of B: 0 E4M3, 1 E5M2).  A K step holds 128
    // FP8 values per row, the bytes of a bf16 step, so the ring, the loads and the
    // slot schedule are those above.  Each 16 x 16 block takes one
    // v_mfma_scale_f32_16x16x128_f8f6f4 per step (unit block scales; the tensors'
    // scales multiply the accumulators in the epilogue), on fragments of 32
    // bytes per lane: the two 16-byte fragments of a row that the bf16 sub-steps
    // read, in the same order for A and B (the instruction pairs the K positions
    // of its two operands lane by lane, so any common order is the same sum).
    // A step runs in two halves of FI/2 rows each, split by the mid-step wait and
    // barrier.  Half 0 reads A rows FI/2.. of this step after its rows; half 1
    // reads A rows 0..FI/2-1 of step k+1 after its rows, and B fragment j of step
    // k+1 right after the last MFMA that uses this step's fragment j.
    constexpr int FA = (F8 - 1) & 1, FB = (F8 - 1) >> 1, HR = FI / 2;
    typedef int i32x8_t __attribute__((ext_vector_type(8)));
    i32x8_t fa8[FI], fb8[FJ];
    uint32_t lane_kc[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) lane_kc[kk] = tile16_off(lane & 15, 4 * kk + (lane >> 4));
    auto frag8 = [&](const char* base) -> i32x8_t {
      const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(base + lane_kc[0]);
      const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(base + lane_kc[1]);
      return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    auto read_a8 = [&](int r, int f) {
      fa8[f] = frag8(BM == 256 ? slot(r, wm) + 2048 * f : slot(r, 0) + 2048 * (4 * wm + f));
    };
    auto read_b8 = [&](int r, int j) {
      fb8[j] = frag8(slot(r, BN == 256 ? NA + wn : NA) + 2048 * ((BN == 256 ? 0 : 4 * wn) + j));
    };
    const int unit_scale = 127;  // E8M0 block scale 2^0
    auto mfma8 = [&](f32x4_t& c, const i32x8_t& b, const i32x8_t& a) {
      if constexpr (FB == 0 && FA == 0)
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                     : "+a"(c) : "v"(b), "v"(a), "v"(unit_scale));
      else if constexpr (FB == 1 && FA == 0)
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0] cbsz:1"
                     : "+a"(c) : "v"(b), "v"(a), "v"(unit_scale));
      else
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0] blgp:1"
                     : "+a"(c) : "v"(b), "v"(a), "v"(unit_scale));
    };
    auto vm_wait = [&](auto n) {
      constexpr int N = decltype(n)::value;
      static_assert(N >= 0 && N < 64, "vmcnt");
      __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
    };
    using L0 = std::integral_constant<int, 0>;
    constexpr int HALF_LOADS = 4 * QS0, TAIL_LOADS = 4 * (NQ - QS0), STEP_LOADS = HALF_LOADS + TAIL_LOADS;
    static_assert((D - 1) * STEP_LOADS < 64, "vmcnt");

    // Half h of a step at ring position r: rows h HR .. h HR + HR - 1.  With
    // `reads` (half 1 only), the next step's fragments come from ring position rn.
    auto half8 = [&](int h, int r, bool reads, int rn, auto nl, auto&& issue_load) {
      constexpr int NL = decltype(nl)::value;
#pragma unroll
      for (int ii = 0; ii < HR; ++ii) {
        const int i = h * HR + ii;
        int n_row = 0, n_first = 0;
#pragma unroll
        for (int n = NL - 1; n >= 0; --n)
          if (n * HR / NL == ii) {
            ++n_row;
            n_first = n;
          }
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
          mfma8(acc[i][j], fb8[j], fa8[i]);
          if (h == 1 && reads && ii == HR - 1) read_b8(rn, j);
          if (j == 1 && n_row >= 1) issue_load(n_first);
          if (j == FJ / 2 + 1 && n_row >= 2) issue_load(n_first + 1);
          if (j == FJ - 1) {
            if (h == 0) read_a8(r, i + HR);
            else if (reads) read_a8(rn, i - HR);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };

    if (nk > 0) {
#pragma unroll
      for (int st = 0; st < D; ++st)
        if (st < nk) {
#pragma unroll
          for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) load(st, st, q, i);
        }
      if (D >= 4 && nk >= 4) vm_wait(std::integral_constant<int, (D >= 4 ? 3 : 0) * STEP_LOADS>{});
      else if (D >= 3 && nk >= 3) vm_wait(std::integral_constant<int, (D >= 3 ? 2 : 0) * STEP_LOADS>{});
      else if (nk >= 2) vm_wait(std::integral_constant<int, STEP_LOADS>{});
      else vm_wait(L0{});
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < FJ; ++j) read_b8(0, j);
#pragma unroll
      for (int f = 0; f < HR; ++f) read_a8(0, f);

      auto k_step8 = [&](int k, auto left, int r) {
        constexpr int LEFT = decltype(left)::value;
        const int r1 = r == P - 1 ? 0 : r + 1, rd = (r + D) % P;
        half8(0, r, false, r1, std::integral_constant<int, LEFT >= D ? HALF_LOADS : 0>{},
              [&](int n) { load(k + D, rd, n >> 2, n & 3); });
        if constexpr (LEFT >= 1) {
          constexpr int WHOLE = LEFT - 1 < D - 2 ? LEFT - 1 : D - 2;
          constexpr int AFTER = STEP_LOADS * (WHOLE > 0 ? WHOLE : 0) + (LEFT >= D ? HALF_LOADS : 0);
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): half 1's A fragments are in registers
          vm_wait(std::integral_constant<int, AFTER>{});
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
        half8(1, r, LEFT >= 1, r1, std::integral_constant<int, LEFT >= D ? TAIL_LOADS : 0>{},
              [&](int n) { load(k + D, rd, QS0 + (n >> 2), n & 3); });
      };
      using Full = std::integral_constant<int, D>;
      int k = 0;
      for (; k + P + D <= nk; k += P) {
#pragma unroll
        for (int u = 0; u < P; ++u) k_step8(k + u, Full{}, u);
      }
      for (; k + D < nk; ++k) k_step8(k, Full{}, k % P);
      auto tail = [&](auto jc) {
        constexpr int J = decltype(jc)::value;
        if constexpr (J < D) {
          if (nk >= J + 1) k_step8(nk - 1 - J, std::integral_constant<int, J>{}, (nk - 1 - J) % P);
        }
      };
      tail(std::integral_constant<int, 3>{});
      tail(std::integral_constant<int, 2>{});
      tail(std::integral_constant<int, 1>{});
      tail(std::integral_constant<int, 0>{});
      vm_wait(L0{});
    }
  }
  // The last MFMAs' results are read below; 32 wait states cover the longest
  // write-to-read distance of a 16 x 16 x 32 MFMA (issued as inline assembly, so
  // the compiler does not insert them).
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
  __syncthreads();  // every wave is done with the operand slots

  // Epilogue, one 64 x 64 chunk of the wave's sub-tile at a time (FI / 4 chunks
  // tall, FJ / 4 wide), staged in the wave's own 16 KiB of LDS.  Block (i, j)
  // register e holds C[16i + lane%16][16j + 4 (lane/16) + e] of the wave's
  // sub-tile.
  // FP8: the product of the two tensors' scales (unit for bf16 operands).
  // FP8: the two operands' amax slots in one load, one word per lane (lanes 0-15
  // the words of A's slot, 16-31 B's); the epilogue takes the max over each
  // 16-lane group (lane 0 then holds A's amax, lane 16 B's) once its first loads
  // are issued.
  static_assert(2 * AMAX_SUB <= 64 && (AMAX_SUB & (AMAX_SUB - 1)) == 0, "two slots' words fit one wave");
  uint32_t amax_word = 0;
  if (F8 != 0 && lane < 2 * AMAX_SUB)
    amax_word = (lane < AMAX_SUB ? args.amax_a : args.amax_b)[(lane & (AMAX_SUB - 1)) * AMAX_SUB_STRIDE];
  auto scales = [&]() {
#pragma unroll
    for (int off = AMAX_SUB / 2; off > 0; off >>= 1)
      amax_word = max(amax_word, (uint32_t)__shfl_xor((int)amax_word, off, 64));
    const float amax_a = __builtin_bit_cast(float, __builtin_amdgcn_readlane((int)amax_word, 0));
    const float amax_b = __builtin_bit_cast(float, __builtin_amdgcn_readlane((int)amax_word, AMAX_SUB));
    return fp8_scale_of(amax_a, fp8_fmax((F8 - 1) & 1)) * fp8_scale_of(amax_b, fp8_fmax((F8 - 1) >> 1));
  };
  store_staged<EPI, (FI / 4) * (FJ / 4), F8 != 0>(
      [&](int ch, float sc) {
        const int h = ch % (FI / 4), hc = ch / (FI / 4);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int r = 16 * ii + (lane & 15), c = 4 * jj + (lane >> 4);
            f32x4_t v = acc[4 * h + ii][4 * hc + jj];
            if constexpr (F8 != 0) v = v * sc;
            *reinterpret_cast<f32x4_t*>(smem + wave * (64 * ROW_B) + r * ROW_B + ((c ^ (r & 15)) << 4)) = v;
          }
      },
      scales, args, smem + wave * (64 * ROW_B), m0 + (BM / 2) * wm, n0 + (BN / 2) * wn, FI / 4, split, lane,
      // paired launches: product 1's chunk in the LDS above the four waves' first regions
      [&](int ch) {
        if constexpr (PAIR) {
          const int h = ch % (FI / 4), hc = ch / (FI / 4);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int r = 16 * ii + (lane & 15), c = 4 * jj + (lane >> 4);
              *reinterpret_cast<f32x4_t*>(smem + (4 + wave) * (64 * ROW_B) + r * ROW_B + ((c ^ (r & 15)) << 4)) =
                  acc2[4 * h + ii][4 * hc + jj];
            }
        }
      },
      smem + (4 + wave) * (64 * ROW_B));
#else
  (void)args_in;
#endif
}

}  // namespace kern

namespace {

template <int BM, int BN, int LB, int EPI, int F8 = 0>
hipError_t launch_one(const GemmArgs& a, int splits, hipStream_t s) {
  if (a.batch > 1 && (splits != 1 || a.batch > MAX_BATCH)) return hipErrorInvalidValue;
  const int blocks = a.tiles_m * a.tiles_n * splits * (a.batch > 1 ? a.batch : 1);
  return launch_kernel(kern::gemm_x16_kernel<LB, EPI, BM, BN, F8>, dim3(blocks), dim3(256), s, a);
}

// FP8 products: (fmt_a, fmt_b) in {(0, 0), (1, 0), (0, 1)} with the epilogues the
// FP8 path uses for each.
template <int BM, int BN>
hipError_t dispatch_fp8(int fa, int fb, Epi epi, const GemmArgs& a, int splits, hipStream_t s) {
  if (fa == 0 && fb == 0) {
    switch (epi) {
      case EPI_BF16: return launch_one<BM, BN, KC, EPI_BF16, 1>(a, splits, s);
      case EPI_F32: return launch_one<BM, BN, KC, EPI_F32, 1>(a, splits, s);
      case EPI_F32_ACC: return launch_one<BM, BN, KC, EPI_F32_ACC, 1>(a, splits, s);
      default: break;
    }
  } else if (fa == 1 && fb == 0) {
    switch (epi) {
      case EPI_DGELU: return launch_one<BM, BN, KC, EPI_DGELU, 2>(a, splits, s);
      case EPI_F32: return launch_one<BM, BN, KC, EPI_F32, 2>(a, splits, s);
      case EPI_F32_ACC: return launch_one<BM, BN, KC, EPI_F32_ACC, 2>(a, splits, s);
      default: break;
    }
  } else if (fa == 0 && fb == 1) {
    if (epi == EPI_F32) return launch_one<BM, BN, KC, EPI_F32, 3>(a, splits, s);
  }
  return hipErrorInvalidValue;
}

// Every product reads A K-contiguous; B is K- or N-contiguous.
template <int BM, int BN>
hipError_t dispatch_layout(Layout la, Layout lb, Epi epi, const GemmArgs& a, int splits, hipStream_t s) {
  if (la != KC) return hipErrorInvalidValue;
  if constexpr (BN == 128) {  // paired products: no split-K, no batch
    if (epi == EPI_F32_PAIR || epi == EPI_F32_ACC_PAIR) {
      if (splits != 1 || a.batch > 1) return hipErrorInvalidValue;
      if (lb == MC)
        return epi == EPI_F32_PAIR ? launch_one<BM, BN, MC, EPI_F32_PAIR>(a, 1, s)
                                   : launch_one<BM, BN, MC, EPI_F32_ACC_PAIR>(a, 1, s);
      return epi == EPI_F32_PAIR ? launch_one<BM, BN, KC, EPI_F32_PAIR>(a, 1, s)
                                 : launch_one<BM, BN, KC, EPI_F32_ACC_PAIR>(a, 1, s);
    }
  }
  if (lb == MC) {
    switch (epi) {
      case EPI_GELU: return launch_one<BM, BN, MC, EPI_GELU>(a, splits, s);
      case EPI_F32: return launch_one<BM, BN, MC, EPI_F32>(a, splits, s);
      case EPI_F32_ACC: return launch_one<BM, BN, MC, EPI_F32_ACC>(a, splits, s);
      case EPI_BF16: return launch_one<BM, BN, MC, EPI_BF16>(a, splits, s);
      default: break;
    }
  } else {
    switch (epi) {
      case EPI_DGELU: return launch_one<BM, BN, KC, EPI_DGELU>(a, splits, s);
      case EPI_F32: return launch_one<BM, BN, KC, EPI_F32>(a, splits, s);
      case EPI_F32_ACC: return launch_one<BM, BN, KC, EPI_F32_ACC>(a, splits, s);
      case EPI_GELU: return launch_one<BM, BN, KC, EPI_GELU>(a, splits, s);
      case EPI_BF16: return launch_one<BM, BN, KC, EPI_BF16>(a, splits, s);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

int tile_bm(TileCfg t) { return t == TILE_128x128 ? 128 : 256; }
int tile_bn(TileCfg t) { return t == TILE_256x256 ? 256 : 128; }

hipError_t launch_gemm_fp8(TileCfg tile, int fmt_a, int fmt_b, Epi epi, const GemmArgs& args, int splits,
                           hipStream_t stream) {
  // The kernel counts K, leading dimensions and K slices in 16-bit units: an FP8
  // row of K bytes is K/2 of them, and a K step of 64 units is 128 FP8 values.
  if ((args.K | args.lda | args.ldb | args.k_split) & 15) return hipErrorInvalidValue;
  GemmArgs g = args;
  g.K /= 2;
  g.lda /= 2;
  g.ldb /= 2;
  g.k_split /= 2;
  switch (tile) {
    case TILE_256x256: return dispatch_fp8<256, 256>(fmt_a, fmt_b, epi, g, splits, stream);
    case TILE_128x128: return dispatch_fp8<128, 128>(fmt_a, fmt_b, epi, g, splits, stream);
    case TILE_256x128: return dispatch_fp8<256, 128>(fmt_a, fmt_b, epi, g, splits, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(TileCfg tile, Layout la, Layout lb, Epi epi, const GemmArgs& args, int splits,
                       hipStream_t stream) {
  switch (tile) {
    case TILE_256x256: return dispatch_layout<256, 256>(la, lb, epi, args, splits, stream);
    case TILE_128x128: return dispatch_layout<128, 128>(la, lb, epi, args, splits, stream);
    case TILE_256x128: return dispatch_layout<256, 128>(la, lb, epi, args, splits, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tpmlp
