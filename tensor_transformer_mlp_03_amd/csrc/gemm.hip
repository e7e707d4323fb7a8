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
// Two kernels:
//  * gemm_x16_kernel: 256 x 256 or 256 x 128 tiles, A K-contiguous, B either;
//    four waves, one per SIMD, each accumulating a 128 x 128 (or 128 x 64)
//    sub-tile as 16 x 16 blocks on v_mfma_f32_16x16x32_bf16, with loads and LDS
//    reads placed between its MFMAs (its comment has the schedule).  The main
//    path.
//  * gemm_kernel: a synchronous two-stage pipeline with 128 x 128 tiles on
//    v_mfma_f32_32x32x16_bf16, an N-contiguous operand transposed in registers;
//    used for outputs too small for 256-row tiles.
// Shared design points:
//  * A K-contiguous operand tile sits in LDS as [rows][64] (128-byte rows), so
//    an MFMA operand fragment is one ds_read_b128 per lane (8 consecutive k of
//    one row); an N-contiguous one in gemm_x16_kernel as [64 k][128 n] slots,
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
//    4 consecutive output columns of one row: epilogues store 8- or 16-byte
//    vectors.
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

// Swizzle of the 16-byte chunk index inside a 128-byte row of a K-contiguous
// tile ([rows][64]): rows r .. r+15 read at one chunk land on 16 distinct
// (row parity, chunk) bank groups, and rows r .. r+7 on 8 distinct chunks.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Byte offset of 16-byte chunk c (k = 8c .. 8c+7) of row r in a [rows][64] tile.
__device__ __forceinline__ int tile_off(int r, int c) { return r * 128 + ((c ^ swz(r)) << 4); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)OOB, 0x00020000);
}

// A K-contiguous operand's [R][64] tile of one K step, loaded straight into LDS.
// DMA instruction i of wave w writes LDS chunks (i*NWAVES + w)*64 + lane of the
// tile; each lane loads the memory chunk that the swizzle places there.
template <int R, int NWAVES>
struct DmaLoader {
  static constexpr int CHUNKS = R * 8;
  static constexpr int PER_WAVE = CHUNKS / 64 / NWAVES;
  static_assert(CHUNKS % (64 * NWAVES) == 0, "tile must divide evenly over the waves");
  uint32_t off[PER_WAVE];  // byte offset of the lane's chunk from the K step's base
  int row[PER_WAVE];       // the chunk's row inside the tile
  int kc[PER_WAVE];        // the chunk's first k inside the K step

  __device__ __forceinline__ void init(int64_t ld, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int q = (i * NWAVES + wave) * 64 + lane;
      const int r = q >> 3, c = (q & 7) ^ swz(r);
      row[i] = r;
      kc[i] = 8 * c;
      off[i] = (uint32_t)(((int64_t)r * ld + 8 * c) * 2);
    }
  }

  // base: element (row0, k0) of the operand.
  __device__ __forceinline__ void issue(const uint16_t* base, char* tile, int rows_left, int k_left,
                                        int wave) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base);
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const bool ok = (row[i] < rows_left) && (kc[i] < k_left);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(tile + (i * NWAVES + wave) * 1024), 16,
                                               ok ? off[i] : OOB, 0, 0, 0);
    }
  }
};

// An M/N-contiguous operand's tile of one K step (64 k-rows of R contiguous
// elements in memory), loaded by R threads as 8x8 blocks into registers and
// written transposed into the [R][64] LDS tile.
template <int R>
struct RegLoader {
  u32x4_t v[8];  // v[i]: elements (k = 8*kb + i, r = 8*mb .. 8*mb+7)
  int mb, kb;
  uint32_t off0, step;

  __device__ __forceinline__ void init(int64_t ld, int t) {
    mb = t % (R / 8);
    kb = t / (R / 8);
    off0 = (uint32_t)(((int64_t)(8 * kb) * ld + 8 * mb) * 2);
    step = (uint32_t)(ld * 2);
  }

  // base: element (k0, r0) of the operand.
  __device__ __forceinline__ void load(const uint16_t* base, int r_left, int k_left) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base);
    const bool r_ok = 8 * mb < r_left;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = r_ok && (8 * kb + i < k_left);
      v[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? off0 + i * step : OOB, 0, 0));
    }
  }

  // Row r of the block gets the 8 k-values of element r: dword e packs
  // (k = 2e, k = 2e+1), i.e. the halves of v[2e] and v[2e+1] that hold r.
  __device__ __forceinline__ void store(char* tile) const {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint32_t sel = (r & 1) ? 0x07060302u : 0x05040100u;
      u32x4_t o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = __builtin_amdgcn_perm(v[2 * e + 1][r >> 1], v[2 * e][r >> 1], sel);
      *reinterpret_cast<u32x4_t*>(tile + tile_off(8 * mb + r, kb)) = o;
    }
  }
};

// MFMA operand fragment of a 32-row slice at sub-step kk (16 wide) of a
// [rows][64] tile: lane l gets the 8 k-values 16*kk + 8*(l/32) .. +7 of row l%32.
__device__ __forceinline__ bf16x8_t read_frag(const char* tile, int r0, int kk, int lane) {
  const int r = r0 + (lane & 31);
  return *reinterpret_cast<const bf16x8_t*>(tile + tile_off(r, 2 * kk + (lane >> 5)));
}

// ds_read_b64_tr_b16 from LDS address `p`.  Issued through inline assembly:
// the builtin makes the compiler wait for every vector-memory load in flight
// (vmcnt(0)) before it, in case an LDS-DMA load targets the same bytes, which
// would stall the load pipeline of this kernel on every memory phase.  Callers
// read only bytes whose loads and writes have already been waited for and made
// visible by a barrier, and wait for the results themselves (lgkmcnt(0))
// before using them.
typedef __attribute__((address_space(3))) char lds_char_t;
__device__ __forceinline__ i16x4_t ds_read_tr(const char* p) {
  i16x4_t v;
  const uint32_t a = (uint32_t)(uintptr_t)(const lds_char_t*)p;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(a));
  return v;
}
// The same, ordered after every earlier memory access of the calling code (for
// reads of bytes that the same wave has just written with ordinary stores).
__device__ __forceinline__ i16x4_t ds_read_tr_after_stores(const char* p) {
  i16x4_t v;
  const uint32_t a = (uint32_t)(uintptr_t)(const lds_char_t*)p;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(a) : "memory");
  return v;
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

// Chunk swizzle of the bf16 G rows that the dGeLU epilogue keeps in staging
// rows.  A transposing read of a 16-lane group takes rows b + 8 q + r (q, r < 4)
// at one column chunk; shifting the chunk by r + 4 q spreads them over 8
// positions, two lanes per bank pair (the same as the row-contiguous reads).
__device__ __forceinline__ int gt_swz(int r) { return (r + 4 * (r >> 3)) & 7; }

// The epilogue proper, independent of the MFMA accumulator layout: for each of
// NH 64-row halves of the wave's (64 NH) x 64 region, stage_half(h) writes the
// half's float32 values into `stage` (row r in 0..63 at r * ROW_B, 16-byte chunk c
// in 0..15 at position c ^ (r & 15)), and the half is finished from there.
template <int EPI, int NH, class StageHalf>
__device__ __forceinline__ void store_staged(StageHalf&& stage_half, const GemmArgs& args, char* stage, int row_w,
                                             int col_w, int split, int lane) {
  // Each phase below issues all of its memory operations before it waits for
  // any: the dGeLU pre-activations of a 64-row half are loaded together (one
  // memory latency instead of one per vector; the next half's are in flight
  // while this half is finished), and LDS reads are batched ahead of the
  // stores that use them.  The pre-activations come through a buffer
  // descriptor on the wave's (uniform) first row and column, so rows and
  // columns outside the output read as zero without a branch.
  u16x8_t pre[2][8];
  __amdgpu_buffer_rsrc_t pre_rs;
  // EPI_F32_ACC: the running sum under a 64-row half, loaded before the half is
  // staged so that the loads overlap the staging (descriptor on the half's first
  // row and column; rows and columns outside the output read as zero).
  f32x4_t old[16];
  auto load_old = [&](int h) {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(reinterpret_cast<const float*>(args.out) + (int64_t)(row_w + 64 * h) * args.ldo + col_w);
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int q = it * 64 + lane, r = q >> 4, c = q & 15;
      const bool ok = row_w + 64 * h + r < args.M && col_w + 4 * c < args.N;
      const uint32_t off = (uint32_t)(((int64_t)r * args.ldo + 4 * c) * 4);
      old[it] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? off : OOB, 0, 0));
    }
  };
  auto load_pre = [&](int h) {
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int q = it * 64 + lane, r = q >> 3, cp = q & 7;
      const int row = row_w + 64 * h + r, col = col_w + 8 * cp;
      const bool ok = row < args.M && col < args.N;  // N % 8 == 0: 8 columns in or out together
      const uint32_t off = (uint32_t)(((int64_t)(64 * h + r) * args.ldo + 8 * cp) * 2);
      pre[h & 1][it] = __builtin_bit_cast(u16x8_t, __builtin_amdgcn_raw_buffer_load_b128(pre_rs, ok ? off : OOB, 0, 0));
    }
  };
  if (EPI == EPI_DGELU) {
    pre_rs = make_rsrc(args.aux + (int64_t)row_w * args.ldo + col_w);
    load_pre(0);
  }
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    if (EPI == EPI_F32_ACC) load_old(h);
    stage_half(h);
    if (EPI == EPI_DGELU && h + 1 < NH) load_pre(h + 1);
    if (EPI == EPI_F32 || EPI == EPI_F32_ACC) {
      float* out = reinterpret_cast<float*>(args.out) + (int64_t)split * args.split_stride;
      f32x4_t xs[16];
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int q = it * 64 + lane, r = q >> 4, c = q & 15;
        xs[it] = *reinterpret_cast<const f32x4_t*>(stage + r * ROW_B + ((c ^ (r & 15)) << 4));
      }
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int q = it * 64 + lane, r = q >> 4, c = q & 15;
        const int row = row_w + 64 * h + r, col = col_w + 4 * c;
        if (EPI == EPI_F32_ACC) xs[it] += old[it];
        if (row < args.M && col < args.N) *reinterpret_cast<f32x4_t*>(out + (int64_t)row * args.ldo + col) = xs[it];
      }
    } else {
      f32x4_t x0s[8], x1s[8];
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int q = it * 64 + lane, r = q >> 3, cp = q & 7;
        x0s[it] = *reinterpret_cast<const f32x4_t*>(stage + r * ROW_B + (((2 * cp) ^ (r & 15)) << 4));
        x1s[it] = *reinterpret_cast<const f32x4_t*>(stage + r * ROW_B + (((2 * cp + 1) ^ (r & 15)) << 4));
      }
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int q = it * 64 + lane, r = q >> 3, cp = q & 7;
        const float x[8] = {x0s[it][0], x0s[it][1], x0s[it][2], x0s[it][3],
                            x1s[it][0], x1s[it][1], x1s[it][2], x1s[it][3]};
        const int row = row_w + 64 * h + r, col = col_w + 8 * cp;
        const bool ok = row < args.M && col < args.N;  // N % 8 == 0: 8 columns in or out together
        const int64_t o = (int64_t)row * args.ldo + col;
        u16x8_t v1, v2;
        if (EPI == EPI_GELU) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            v1[e] = epi_gelu(x[e]);
            v2[e] = f32_to_bf16(x[e]);
          }
          if (ok) {
            *reinterpret_cast<u16x8_t*>(reinterpret_cast<uint16_t*>(args.out) + o) = v1;
            if (args.out2) *reinterpret_cast<u16x8_t*>(args.out2 + o) = v2;
          }
        } else if (EPI == EPI_BF16) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v1[e] = f32_to_bf16(x[e]);
          if (ok) *reinterpret_cast<u16x8_t*>(reinterpret_cast<uint16_t*>(args.out) + o) = v1;
        } else {  // EPI_DGELU
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const DGelu d = epi_dgelu(x[e], pre[h & 1][it][e]);
            v1[e] = d.dp;
            v2[e] = d.g;
          }
          if (ok) *reinterpret_cast<u16x8_t*>(reinterpret_cast<uint16_t*>(args.out) + o) = v1;
          // Keep G of this row in LDS, in place of its float32 values (every
          // lane has read its float32 values above), in bytes [0, 128) of the
          // row, 16-byte chunks swizzled by the row (gt_swz).  Rows and columns
          // outside the output hold values that no transposed store below reads.
          *reinterpret_cast<u16x8_t*>(stage + r * ROW_B + ((cp ^ gt_swz(r)) << 4)) = v2;
        }
      }
      if (EPI == EPI_DGELU) {
        // Transposed store of G in whole 128-byte lines.  ds_read_b64_tr_b16
        // takes, in each 16-lane group, 4 rows x 16 columns (source lane 4 r + q:
        // row r, columns 4 q .. +3) and hands lane i column i.  Source lane
        // 4 r + q reads the 4 columns 8 it + 4 (g / 2) .. +3 of G row
        // m0(q) + r, with m0(q) = 32 (g % 2) + 8 q, so lane 4 q + e receives
        // rows m0(q) .. +3 of column 8 it + 4 (g / 2) + e; a second read gives
        // rows +4 .. +7.  The 8 lanes (g % 2, q) of a column then hold its 64
        // rows: one store instruction writes 8 columns x 128 bytes of G^T.  All
        // eight steps are read first, then stored.
        const int g = lane >> 4, j = lane & 15, jq = j & 3, jr = j >> 2;
        const int half = (g >> 1) ? 8 : 0;
        i16x4_t lo[8], hi[8];
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const int ka = 32 * (g & 1) + 8 * jq + jr, kb = ka + 4;  // source role: q = jq, r = jr
          lo[it] = ds_read_tr_after_stores(stage + ka * ROW_B + ((it ^ gt_swz(ka)) << 4) + half);
          hi[it] = ds_read_tr_after_stores(stage + kb * ROW_B + ((it ^ gt_swz(kb)) << 4) + half);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the transposed reads above are complete
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          // destination role: lane 4 q + e with q = jr, e = jq
          const int f = col_w + 8 * it + 4 * (g >> 1) + jq, m = row_w + 64 * h + 32 * (g & 1) + 8 * jr;
          if (f < args.N && m < args.M) {
            const u16x8_t v = {(uint16_t)lo[it][0], (uint16_t)lo[it][1], (uint16_t)lo[it][2], (uint16_t)lo[it][3],
                               (uint16_t)hi[it][0], (uint16_t)hi[it][1], (uint16_t)hi[it][2], (uint16_t)hi[it][3]};
            *reinterpret_cast<u16x8_t*>(args.out2 + (int64_t)f * args.ldt + m) = v;
          }
        }
      }
    }
  }
}

// Epilogue of a (32 FM) x 64 region held as 32 x 32 MFMA accumulators: register
// r of fragment (i, j) holds C[32i + lane%32][32j + 8(r/4) + 4(lane/32) + r%4].
template <int EPI, int FM, int FN>
__device__ __forceinline__ void store_tile(const f32x16_t (&acc)[FM][FN], const GemmArgs& args, char* stage,
                                           int row_w, int col_w, int split, int lane) {
  static_assert(FN == 2 && FM % 2 == 0, "staging layout: 64 columns, 64-row halves");
  store_staged<EPI, FM / 2>(
      [&](int h) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int r = 32 * ii + (lane & 31);
              const int c = 8 * j + 2 * g + (lane >> 5);  // 16-byte chunk (4 columns) of the row
              const f32x4_t x = {acc[2 * h + ii][j][4 * g], acc[2 * h + ii][j][4 * g + 1],
                                 acc[2 * h + ii][j][4 * g + 2], acc[2 * h + ii][j][4 * g + 3]};
              *reinterpret_cast<f32x4_t*>(stage + r * ROW_B + ((c ^ (r & 15)) << 4)) = x;
            }
      },
      args, stage, row_w, col_w, split, lane);
}

}  // namespace

// The kernel has external linkage (a kernel template in an anonymous namespace
// does not get its host launch stubs emitted for every instantiation).
namespace kern {

template <int BM, int BN, int WAVES_M, int WAVES_N, int LA, int LB, int EPI>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N)
gemm_kernel(GemmArgs args) {
  // The body is compiled for the device only: the host pass needs just the
  // launch stub, and device builtins (buffer descriptors, LDS DMA) have no host
  // form.
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BK = TILE_BK;
  constexpr int NWAVES = WAVES_M * WAVES_N;
  constexpr int THREADS = 64 * NWAVES;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  constexpr int STAGE = A_BYTES + B_BYTES;
  // Threads that load an M/N-contiguous operand: A's blocks first, then B's.
  constexpr int A_REG_T = (LA == MC) ? BM : 0;
  constexpr int B_REG_T = (LB == MC) ? BN : 0;
  static_assert(A_REG_T + B_REG_T <= THREADS, "one 8x8 block per loading thread");
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  int tm, tn, split;
  tile_of(blockIdx.x, gridDim.x, args.tiles_m, args.tiles_n, tm, tn, split);
  const int m0 = tm * BM, n0 = tn * BN;
  const int k_begin = split * args.k_split;
  const int k_end = min(args.K, k_begin + args.k_split);
  const int nk = (k_end - k_begin + BK - 1) / BK;

  DmaLoader<BM, NWAVES> da;
  DmaLoader<BN, NWAVES> db;
  if (LA == KC) da.init(args.lda, wave, lane);
  if (LB == KC) db.init(args.ldb, wave, lane);

  // One register loader per thread: threads [0, A_REG_T) take 8x8 blocks of
  // A (when A is M/N-contiguous), threads [A_REG_T, A_REG_T + B_REG_T) blocks
  // of B.  Both operands' tiles have R rows in LDS.
  static_assert(LA == KC || LB == KC || BM == BN, "one register loader shape");
  constexpr int R_REG = (LA == MC) ? BM : BN;
  RegLoader<R_REG> rl;
  const bool reg_a = (LA == MC) && tid < A_REG_T;
  const bool reg_b = (LB == MC) && tid >= A_REG_T && tid < A_REG_T + B_REG_T;
  const bool reg_any = reg_a || reg_b;
  const uint16_t* reg_src = reg_a ? args.a : args.b;
  const int64_t reg_ld = reg_a ? args.lda : args.ldb;
  const int reg_o0 = reg_a ? m0 : n0;
  const int reg_left = reg_a ? args.M - m0 : args.N - n0;
  const int reg_tile = reg_a ? 0 : A_BYTES;
  if (LA == MC || LB == MC) rl.init(reg_ld, reg_a ? tid : tid - A_REG_T);

  // Issue the memory loads of K step `step`: DMA into its stage for
  // K-contiguous operands, into registers for M/N-contiguous ones.
  auto issue = [&](int step) {
    const int k = k_begin + step * BK;
    char* st = smem + (step & 1) * STAGE;
    if (LA == KC) da.issue(args.a + (int64_t)m0 * args.lda + k, st, args.M - m0, k_end - k, wave);
    if (LB == KC) db.issue(args.b + (int64_t)n0 * args.ldb + k, st + A_BYTES, args.N - n0, k_end - k, wave);
    if ((LA == MC || LB == MC) && reg_any) rl.load(reg_src + (int64_t)k * reg_ld + reg_o0, reg_left, k_end - k);
  };
  // Write the register-held blocks of K step `step` into its stage.
  auto commit = [&](int step) {
    if ((LA == MC || LB == MC) && reg_any) rl.store(smem + (step & 1) * STAGE + reg_tile);
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Fragments of one 16-wide sub-step, double-buffered in registers: the reads
  // of sub-step kk+1 are in flight while the MFMAs of sub-step kk issue.
  bf16x8_t fa[2][FM], fb[2][FN];
  auto read_sub = [&](int buf, const char* st, int kk) {
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[buf][i] = read_frag(st, wm * WM + 32 * i, kk, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[buf][j] = read_frag(st + A_BYTES, wn * WN + 32 * j, kk, lane);
  };
  auto mfma_sub = [&](int buf) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
  };
  constexpr int SUB = BK / 16;
  static_assert(SUB % 2 == 0, "sub-steps alternate between the two fragment buffers");

  if (nk > 0) {
    issue(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    commit(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    if (nk > 1) issue(1);
    read_sub(0, smem, 0);
  }

  // One K step.  With a next step: after the reads of the last sub-step, wait
  // for this wave's loads of step kt+1, write its register-held blocks, and
  // wait until its LDS reads and writes are complete; after the barrier the
  // same holds for every wave, so step kt+1's stage can be read and the
  // current stage refilled, while the last sub-step's MFMAs run from
  // registers.  The last step is peeled so that the loop body has one path (no
  // conservative waits at a merge).
  auto k_step = [&](int kt, bool has_next) {
    const char* cur = smem + (kt & 1) * STAGE;
#pragma unroll
    for (int kk = 0; kk < SUB - 1; ++kk) {
      read_sub((kk + 1) & 1, cur, kk + 1);
      mfma_sub(kk & 1);
    }
    if (has_next) {
      // sched_barrier(0): the compiler may not move instructions across, so the
      // last sub-step's MFMAs stay behind the barrier and the next reads.
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      commit(kt + 1);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      if (kt + 2 < nk) issue(kt + 2);
      read_sub(0, smem + ((kt + 1) & 1) * STAGE, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_sub((SUB - 1) & 1);
  };
  for (int kt = 0; kt < nk - 1; ++kt) k_step(kt, true);
  if (nk > 0) k_step(nk - 1, false);

  // Epilogue: each wave stages its tile through its own 16 KiB of LDS.
  static_assert(NWAVES * 64 * ROW_B <= 2 * STAGE, "staging fits in the operand stages");
  __syncthreads();  // every wave is done with the operand stages
  store_tile<EPI>(acc, args, smem + wave * (64 * ROW_B), m0 + wm * WM, n0 + wn * WN, split, lane);
#else
  (void)args;
#endif
}


// 256 x BN tile (BN = 256 or 128) on v_mfma_f32_16x16x32_bf16: the four-wave
// kernel's ring of ten 16 KiB slots, LDS layouts and loads, with 16 x 16
// accumulator blocks.  Wave (wm, wn) computes a 128 x (BN / 2) sub-tile as 8 x FJ
// blocks (FJ = 8 or 4, 256 or 128 accumulator registers).  A K step (64) is two
// sub-steps of 32 k; in each a wave issues 8 FJ MFMAs of 16 cycles and, between
// them, the LDS reads of the next sub-step's fragments and one batch of loads:
//   sub-step 0 of step k: quarters 0 and 1 of step k+2 (into step k-1's slots 2, 3)
//   then: wait until the next sub-step's fragments are in registers and step k+1
//         has landed (vmcnt: only the batch just issued may be in flight); barrier
//   sub-step 1 of step k: quarters 2 and 3 of step k+2 (into step k's slots 0, 1,
//         which no wave reads any more), and the reads of step k+1's sub-step 0.
// The next sub-step's B fragments go to the other half of a double buffer; an A
// fragment is reloaded as soon as its row of MFMAs has been issued (MFMAs run
// row by row), so A needs no second buffer.
template <int LB, int EPI, int BN>
__global__ void __launch_bounds__(256)
gemm_x16_kernel(GemmArgs args) {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(BN == 256 || BN == 128, "tile widths");
  constexpr int BK = TILE_BK;
  constexpr int SLOT = 128 * BK * 2;
  constexpr int NSLOT = 10;
  constexpr int FI = 8, FJ = BN / 32;     // 16 x 16 blocks per wave: 8 x FJ
  constexpr int NQ = BN == 256 ? 4 : 3;   // quarters loaded per K step
  constexpr int NM = FI * FJ;             // MFMAs per sub-step
  static_assert(BK == 64 && NSLOT * SLOT == 160 * 1024, "ten 16 KiB slots fill the LDS");
  __shared__ __attribute__((aligned(1024))) char smem[NSLOT * SLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  int tm, tn, split;
  tile_of(blockIdx.x, gridDim.x, args.tiles_m, args.tiles_n, tm, tn, split);
  const int m0 = tm * 256, n0 = tn * BN;
  const int k_begin = split * args.k_split;
  const int k_end = min(args.K, k_begin + args.k_split);
  const int nk = (k_end - k_begin + BK - 1) / BK;

  QuarterKC qa[2], qb[2];
  QuarterMC qm[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) qa[q].init(args.lda, args.M - m0 - 128 * q, wave, lane);
#pragma unroll
  for (int q = 0; q < NQ - 2; ++q) {
    if (LB == KC) qb[q].init(args.ldb, args.N - n0 - 128 * q, wave, lane);
    else qm[q].init(args.ldb, args.N - n0 - 128 * q, wave, lane);
  }

  auto slot = [&](int r, int q) -> char* { return smem + ((4 * r + q) % NSLOT) * SLOT; };
  // Instruction i of this wave's share of quarter q of K step `step` (r = step % 5).
  auto load = [&](int step, int r, int q, int i) {
    if (q >= NQ) return;
    const int k = k_begin + step * BK;
    char* dst = slot(r, q);
    if (q < 2) {
      qa[q].issue(make_rsrc(args.a + (int64_t)(m0 + 128 * q) * args.lda + k), dst, k_end - k, wave, i);
    } else if (LB == KC) {
      qb[q - 2].issue(make_rsrc(args.b + (int64_t)(n0 + 128 * (q - 2)) * args.ldb + k), dst, k_end - k, wave, i);
    } else {
      qm[q - 2].issue(make_rsrc(args.b + (int64_t)k * args.ldb + n0 + 128 * (q - 2)), dst, k_end - k, wave, i);
    }
  };

  f32x4_t acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  bf16x8_t fa[FI], fb[2][FJ];
  // K-contiguous fragment f (rows 16f .. +15 of a 128-row quarter) in sub-step kk:
  // lane l reads row 16f + l % 16, 16-byte chunk 4kk + l / 16, at lane_kc[kk] + 2048 f.
  uint32_t lane_kc[2], lane_mc[FJ];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) lane_kc[kk] = tile16_off(lane & 15, 4 * kk + (lane >> 4));
  const int wcol = BN == 256 ? 0 : 64 * wn;  // the wave's first column inside its B quarter
#pragma unroll
  for (int j = 0; j < FJ; ++j) lane_mc[j] = mc16_lane_off(wcol + 16 * j, lane);
  auto read_a = [&](int r, int kk, int f) {
    fa[f] = *reinterpret_cast<const bf16x8_t*>(slot(r, wm) + lane_kc[kk] + 2048 * f);
  };
  auto read_b = [&](int buf, int r, int kk, int j) {
    const char* tb = slot(r, BN == 256 ? 2 + wn : 2);
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
  auto sub_step = [&](int cur, bool reads, int rn, int kn, auto nl, auto&& issue_load) {
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
        mfma16(acc[i][j], fb[cur][j], fa[i]);
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
  constexpr int HALF_LOADS = 8;                 // quarters 0 and 1: 4 instructions each
  constexpr int TAIL_LOADS = 4 * (NQ - 2);      // quarters 2 (and 3)

  if (nk > 0) {
    // Prologue: steps 0 and 1 (slots 0-7); wait for step 0.
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) load(0, 0, q, i);
    if (nk > 1) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) load(1, 1, q, i);
      vm_wait(std::integral_constant<int, HALF_LOADS + TAIL_LOADS>{});
    } else {
      vm_wait(L0{});
    }
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < FJ; ++j) read_b(0, 0, 0, j);
#pragma unroll
    for (int f = 0; f < FI; ++f) read_a(0, 0, f);

    // K step k with LEFT = min(2, steps after it) known at compile time; r = k % 5.
    auto k_step = [&](int k, auto left, int r) {
      constexpr int LEFT = decltype(left)::value;
      const int r1 = r == 4 ? 0 : r + 1, r2 = r >= 3 ? r - 3 : r + 2;
      // sub-step 0: reads sub-step 1 of this step; loads quarters 0, 1 of step k+2
      sub_step(0, true, r, 1, std::integral_constant<int, LEFT >= 2 ? HALF_LOADS : 0>{},
               [&](int n) { load(k + 2, r2, n >> 2, n & 3); });
      if constexpr (LEFT >= 1) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): sub-step 1's fragments are in registers
        if constexpr (LEFT >= 2) vm_wait(std::integral_constant<int, HALF_LOADS>{});  // step k+1 has landed
        else vm_wait(L0{});
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
      // sub-step 1: reads sub-step 0 of step k+1; loads quarters 2, 3 of step k+2
      sub_step(1, LEFT >= 1, r1, 0, std::integral_constant<int, LEFT >= 2 ? TAIL_LOADS : 0>{},
               [&](int n) { load(k + 2, r2, 2 + (n >> 2), n & 3); });
    };
    using Full = std::integral_constant<int, 2>;
    int k = 0;
    for (; k + 7 <= nk; k += 5) {  // steps k .. k+4, each with two more after it
#pragma unroll
      for (int u = 0; u < 5; ++u) k_step(k + u, Full{}, u);
    }
    for (; k + 2 < nk; ++k) k_step(k, Full{}, k % 5);
    if (nk >= 2) k_step(nk - 2, std::integral_constant<int, 1>{}, (nk - 2) % 5);
    k_step(nk - 1, std::integral_constant<int, 0>{}, (nk - 1) % 5);
    vm_wait(L0{});
  }
  // The last MFMAs' results are read below; 32 wait states cover the longest
  // write-to-read distance of a 16 x 16 x 32 MFMA (issued as inline assembly, so
  // the compiler does not insert them).
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
  __syncthreads();  // every wave is done with the operand slots

  // Epilogue, one 64-column half of the wave's sub-tile at a time, staged in the
  // wave's own 16 KiB of LDS.  Block (i, j) register e holds C[16i + lane%16][16j +
  // 4 (lane/16) + e] of the wave's sub-tile.
#pragma unroll
  for (int hc = 0; hc < FJ / 4; ++hc) {
    store_staged<EPI, 2>(
        [&](int h) {
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int r = 16 * ii + (lane & 15), c = 4 * jj + (lane >> 4);
              *reinterpret_cast<f32x4_t*>(smem + wave * (64 * ROW_B) + r * ROW_B + ((c ^ (r & 15)) << 4)) =
                  acc[4 * h + ii][4 * hc + jj];
            }
        },
        args, smem + wave * (64 * ROW_B), m0 + 128 * wm, n0 + (BN / 2) * wn + 64 * hc, split, lane);
  }
#else
  (void)args;
#endif
}

}  // namespace kern

namespace {

template <int BM, int BN, int WM_, int WN_, int LA, int LB, int EPI>
hipError_t launch_one(const GemmArgs& a, int splits, hipStream_t s) {
  const int blocks = a.tiles_m * a.tiles_n * splits;
  if constexpr (BM == 256 && LA == KC)
    return launch_kernel(kern::gemm_x16_kernel<LB, EPI, BN>, dim3(blocks), dim3(256), s, a);
  else
    return launch_kernel(kern::gemm_kernel<BM, BN, WM_, WN_, LA, LB, EPI>, dim3(blocks), dim3(64 * WM_ * WN_), s, a);
}

template <int BM, int BN, int WM_, int WN_>
hipError_t dispatch_layout(Layout la, Layout lb, Epi epi, const GemmArgs& a, int splits, hipStream_t s) {
  if (la == KC && lb == MC) {
    switch (epi) {
      case EPI_GELU: return launch_one<BM, BN, WM_, WN_, KC, MC, EPI_GELU>(a, splits, s);
      case EPI_F32: return launch_one<BM, BN, WM_, WN_, KC, MC, EPI_F32>(a, splits, s);
      case EPI_F32_ACC: return launch_one<BM, BN, WM_, WN_, KC, MC, EPI_F32_ACC>(a, splits, s);
      case EPI_BF16: return launch_one<BM, BN, WM_, WN_, KC, MC, EPI_BF16>(a, splits, s);
      default: break;
    }
  } else if (la == KC && lb == KC) {
    switch (epi) {
      case EPI_DGELU: return launch_one<BM, BN, WM_, WN_, KC, KC, EPI_DGELU>(a, splits, s);
      case EPI_F32: return launch_one<BM, BN, WM_, WN_, KC, KC, EPI_F32>(a, splits, s);
      case EPI_F32_ACC: return launch_one<BM, BN, WM_, WN_, KC, KC, EPI_F32_ACC>(a, splits, s);
      case EPI_GELU: return launch_one<BM, BN, WM_, WN_, KC, KC, EPI_GELU>(a, splits, s);
      case EPI_BF16: return launch_one<BM, BN, WM_, WN_, KC, KC, EPI_BF16>(a, splits, s);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

int tile_bm(TileCfg t) { return t == TILE_128x128 ? 128 : 256; }
int tile_bn(TileCfg t) { return t == TILE_256x256 ? 256 : 128; }

hipError_t launch_gemm(TileCfg tile, Layout la, Layout lb, Epi epi, const GemmArgs& args, int splits,
                       hipStream_t stream) {
  switch (tile) {
    case TILE_256x256: return dispatch_layout<256, 256, 2, 2>(la, lb, epi, args, splits, stream);
    case TILE_128x128: return dispatch_layout<128, 128, 2, 2>(la, lb, epi, args, splits, stream);
    case TILE_256x128: return dispatch_layout<256, 128, 2, 2>(la, lb, epi, args, splits, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tpmlp
