// bf16 MFMA GEMM core for gfx950 with the MLP's fused epilogues.
//
// C[m,n] = sum_k A[m,k] B[k,n], bf16 operands, float32 accumulation on
// v_mfma_f32_32x32x16_bf16.  Every product of the tensor-parallel MLP's forward
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
//  * gemm_w4_kernel: 256 x 256 tiles, A K-contiguous, B either; four waves,
//    one per SIMD, each accumulating a 128 x 128 quadrant, with loads and LDS
//    reads interleaved between its MFMAs (its comment has the schedule).  The
//    main path.
//  * gemm_kernel: a synchronous two-stage pipeline with 128 x 128 tiles, an
//    N-contiguous operand transposed in registers; used for outputs too small
//    for 256 x 256 tiles.
// Shared design points:
//  * A K-contiguous operand tile sits in LDS as [rows][64] (128-byte rows), so
//    an MFMA operand fragment is one ds_read_b128 per lane (8 consecutive k of
//    one row); an N-contiguous one in gemm_w4_kernel as [64 k][128 n] halves,
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
//    operand panels) run on the same XCD and its L2, then grouped 8 tiles tall.

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

// Four waves' LDS-DMA loads of 128 rows x 64 k of a K-contiguous operand into
// one 16 KiB [128][64] LDS slot: 16 instructions of 1 KiB, 4 per wave.
// Instruction i of wave w fills rows 8*(4i + w) .. +7 of the slot; lane q
// writes 16-byte position q & 7 of row q / 8 and loads the chunk that the
// swizzle places there.  A row's swizzle depends on the lane and on
// (4i + w) & 7, so even and odd i use two lane patterns.
struct HalfDma {
  uint32_t lane_off[2];  // byte offset of the lane's chunk for even / odd i
  int kc[2];             // its first k inside the K step

  __device__ __forceinline__ void init(int64_t ld, int w, int lane) {
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int c = (lane & 7) ^ (((lane >> 3) ^ (4 * par + w)) & 7);
      kc[par] = 8 * c;
      lane_off[par] = (uint32_t)(((int64_t)(lane >> 3) * ld + 8 * c) * 2);
    }
  }
  // Instruction i of the wave's share; base: element (first row of the half,
  // first k of the step).
  __device__ __forceinline__ void issue_one(const uint16_t* base, int64_t ld, char* half, int rows_left, int k_left,
                                            int w, int lane, int i) const {
    const int r0 = 8 * (4 * i + w);
    const bool ok = (kc[i & 1] < k_left) && (r0 + (lane >> 3) < rows_left);
    const uint32_t off = lane_off[i & 1] + (uint32_t)((int64_t)r0 * ld * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(base), (lds_void_t*)(half + (4 * i + w) * 1024), 16,
                                             ok ? off : OOB, 0, 0, 0);
  }
};

// The same for an N-contiguous operand (stored [K][ld], n contiguous): one half
// of a K step is 64 k-rows x 128 n, kept in LDS as [64][128] (256-byte rows),
// 16 KiB.  The 16-byte chunk holding n .. n+7 of k-row k sits at position
// (n / 8) ^ (4 * (k % 4)) of the row (mc_off): a transposing fragment read
// touches 4 consecutive k-rows of 32 columns per 32 lanes, which this spreads
// over all 64 banks (unswizzled, the 4 rows, 256 bytes apart, hit the same
// banks).  Instruction i of wave w fills k-rows 4*(4i + w) .. +3 (LDS bytes
// (4i + w) * 1024 ..); lane q writes position q % 16 of k-row q / 16 and loads
// the chunk placed there, which depends only on the lane since k % 4 = (q / 16)
// % 4.  One instruction reads 4 k-rows x 256 bytes.
__device__ __forceinline__ int mc_off(int k, int n) { return k * 256 + (((n >> 3) ^ (4 * (k & 3))) << 4) + (n & 7) * 2; }

struct HalfDmaMC {
  uint32_t lane_off;  // byte offset of the lane's chunk in instruction 0
  int lane_k, lane_n;  // the chunk's k-row in instruction 0 and first n

  __device__ __forceinline__ void init(int64_t ld, int w, int lane) {
    lane_k = 4 * w + (lane >> 4);
    lane_n = 8 * ((lane & 15) ^ (4 * ((lane >> 4) & 3)));
    lane_off = (uint32_t)(((int64_t)lane_k * ld + lane_n) * 2);
  }
  // Instruction i of the wave's share; base: element (first k of the step,
  // first n of the half).
  __device__ __forceinline__ void issue_one(const uint16_t* base, int64_t ld, char* half, int n_left, int k_left,
                                            int w, int lane, int i) const {
    const bool ok = lane_n < n_left && (lane_k + 16 * i < k_left);
    const uint32_t off = lane_off + (uint32_t)((int64_t)(16 * i) * ld * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(base), (lds_void_t*)(half + (4 * i + w) * 1024), 16,
                                             ok ? off : OOB, 0, 0, 0);
  }
};

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

// MFMA B fragment of 32 columns (n0 .. n0+31, inside one 128-wide half) at
// sub-step kk from an N-contiguous [64][128] half: lane l needs k = 16*kk +
// 8*(l/32) .. +7 of column n0 + l%32.  ds_read_b64_tr_b16 reads, in each
// 16-lane group, 4 k-rows x 16 columns (lane s: k-row s/4, columns 4*(s%4) ..
// +3) and hands lane i the 4 k-values of column i; two such reads give 8.
// This returns the lane's byte offset of the first read at kk = 0; the
// second is 4 k-rows (1024 bytes) further, and sub-step kk adds 4096 bytes
// (the swizzle depends on k only through k % 4).
__device__ __forceinline__ uint32_t mc_lane_off(int n0, int lane) {
  const int g = lane >> 4, sl = lane & 15;
  return mc_off(8 * (g >> 1) + (sl >> 2), n0 + 16 * (g & 1) + 4 * (sl & 3));
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

template <int EPI, int FM, int FN>
__device__ __forceinline__ void store_tile(const f32x16_t (&acc)[FM][FN], const GemmArgs& args, char* stage,
                                           int row_w, int col_w, int split, int lane) {
  static_assert(FN == 2 && FM % 2 == 0, "staging layout: 64 columns, 64-row halves");
  constexpr int NH = FM / 2;
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
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r = 32 * ii + (lane & 31);
          const int c = 8 * j + 2 * g + (lane >> 5);  // 16-byte chunk (4 columns) of the row
          const f32x4_t x = {acc[2 * h + ii][j][4 * g], acc[2 * h + ii][j][4 * g + 1], acc[2 * h + ii][j][4 * g + 2],
                             acc[2 * h + ii][j][4 * g + 3]};
          *reinterpret_cast<f32x4_t*>(stage + r * ROW_B + ((c ^ (r & 15)) << 4)) = x;
        }
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


// Orders of the four-wave kernel's fragment reads and MFMAs (see there).
__device__ constexpr int w4_read(int r) {
  constexpr int order[8] = {0, 4, 5, 1, 6, 2, 7, 3};  // A0 B0 B1 A1 B2 A2 B3 A3
  return order[r];
}
__device__ constexpr int w4_mi(int m) {
  constexpr int order[16] = {0, 0, 1, 1, 0, 1, 2, 2, 2, 0, 1, 2, 3, 3, 3, 3};
  return order[m];
}
__device__ constexpr int w4_mj(int m) {
  constexpr int order[16] = {0, 1, 0, 1, 2, 2, 0, 1, 2, 3, 3, 3, 0, 1, 2, 3};
  return order[m];
}
// The same for a 128 x 64 wave tile (256 x 128 workgroup tile): reads A0 B0 B1
// A1 A2 A3, MFMAs row by row.
__device__ constexpr int w4n_read(int r) {
  constexpr int order[6] = {0, 4, 5, 1, 2, 3};
  return order[r];
}

// 256 x 256 tile, A K-contiguous and B either, four waves (one per SIMD) that
// each compute a 128 x 128 quadrant: wave w owns rows 128 (w / 2) and columns
// 128 (w % 2) of the tile, its 256 accumulator registers in the AGPRs.  Against
// eight waves of 128 x 64, a K step reads a third less from LDS (each wave
// reads 128 rows of A and 128 of B) and needs one barrier instead of four.
//
// LDS is a ring of ten 16 KiB slots.  Quarter q of K step s (A rows 0-127,
// A rows 128-255, B's first 128 columns, B's last 128) lives in slot
// (4 s + q) mod 10, so steps s and s+1 and half of s+2 fit at once.  Every wave
// loads a quarter of every quarter-slot (4 LDS-DMA instructions of 1 KiB).
//
// A K step is four sub-steps of 16 k.  In each, a wave issues the LDS reads of
// the next sub-step's operand fragments and one quarter-slot's loads between
// the current sub-step's 16 MFMAs (sched_group_barrier keeps the MFMA pipe fed
// while the other instructions issue; with one wave per SIMD nothing else
// would).  In K step k:
//   sub-step 0: quarter 3 of step k+1 (into the slot of step k-1's quarter 1)
//   sub-step 1: quarter 0 of step k+2 (step k-1's quarter 2)
//   sub-step 2: quarter 1 of step k+2 (step k-1's quarter 3)
//   then: wait until step k+1 has landed (vmcnt: only the two batches just
//         issued may be in flight) and until sub-step 3's fragments are in
//         registers, and barrier: every wave is done with step k's slots and
//         step k+1 is visible to all
//   sub-step 3: quarter 2 of step k+2 (step k's quarter 0), and the LDS reads
//         of step k+1's first sub-step.
// The loads thus run at an even 16 KiB per sub-step per workgroup; each batch
// has at least two sub-steps before it is waited for.
//
// BN = 128 (256 x 128 tiles) keeps the ring and the schedule: a K step has no
// fourth quarter (B's 128 columns are quarter 2, read by both column waves,
// each a 128 x 64 sub-tile), so its loads are simply not issued and every
// vmcnt wait above still counts the loads that follow the ones it needs.
template <int LB, int EPI, int BN>
__global__ void __launch_bounds__(256)
gemm_w4_kernel(GemmArgs args) {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(BN == 256 || BN == 128, "tile widths");
  constexpr int BK = TILE_BK;
  constexpr int SLOT = 128 * BK * 2;
  constexpr int NSLOT = 10;
  constexpr int FM = 4, FN = BN / 64;  // 32 x 32 fragments per wave: 128 x BN/2
  constexpr int NQ = BN == 256 ? 4 : 3;  // quarters loaded per K step
  // A window's 16 loads, four per sub-step: even issue measured best (eight in
  // one sub-step stall the wave on the address unit).
  constexpr int LC3 = 4, LC0 = 4, LC1 = 4;
  static_assert(BK == 64 && NSLOT * SLOT == 160 * 1024, "ten 16 KiB slots fill the LDS");
  static_assert(4 * 64 * ROW_B <= NSLOT * SLOT, "epilogue staging fits");
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

  HalfDma dma_a, dma_b;
  HalfDmaMC dma_bm;
  dma_a.init(args.lda, wave, lane);
  if (LB == KC) dma_b.init(args.ldb, wave, lane);
  else dma_bm.init(args.ldb, wave, lane);

  // Slot of quarter q of a K step with step % 5 == r (4 * 5 = 20 slots is a
  // whole number of turns of the ring).  The main loop is unrolled five times so
  // that r, and every LDS address, is a compile-time constant there.
  auto slot = [&](int r, int q) -> char* { return smem + ((4 * r + q) % NSLOT) * SLOT; };
  // Instruction i of this wave's share of quarter q of K step `step` (r = step % 5).
  auto load = [&](int step, int r, int q, int i) {
    if (q >= NQ) return;
    const int k = k_begin + step * BK;
    char* dst = slot(r, q);
    if (q < 2) {
      dma_a.issue_one(args.a + (int64_t)(m0 + 128 * q) * args.lda + k, args.lda, dst, args.M - m0 - 128 * q,
                      k_end - k, wave, lane, i);
    } else if (LB == KC) {
      dma_b.issue_one(args.b + (int64_t)(n0 + 128 * (q - 2)) * args.ldb + k, args.ldb, dst,
                      args.N - n0 - 128 * (q - 2), k_end - k, wave, lane, i);
    } else {
      dma_bm.issue_one(args.b + (int64_t)k * args.ldb + n0 + 128 * (q - 2), args.ldb, dst,
                       args.N - n0 - 128 * (q - 2), k_end - k, wave, lane, i);
    }
  };

  // The 16 loads of window k, issued between barrier k-1 and barrier k: quarters
  // 2 and 3 of step k+1 (loads 0-7), then quarters 0 and 1 of step k+2 (8-15),
  // into the slots of step k-1.  r1, r2: (k+1) % 5, (k+2) % 5.  The first LC3
  // are issued in sub-step 3 of step k-1, LC0 and LC1 in sub-steps 0 and 1 of
  // step k, the rest in sub-step 2.
  auto window_load = [&](int k, int n, int r1, int r2) {
    const int b = n >> 2, i = n & 3;
    if (b < 2) load(k + 1, r1, 2 + b, i);
    else load(k + 2, r2, b - 2, i);
  };
  static_assert(LC3 <= 8 && LC0 <= 8 && LC1 <= 8 && 16 - LC3 - LC0 - LC1 <= 8 && LC3 + LC0 + LC1 <= 16,
                "at most eight loads per sub-step; window k+1's first LC3 exist whenever step k+2 does");

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  bf16x8_t fa[2][FM], fb[2][FN];
  // The fragments are read, and the MFMAs run, in an order in which the n-th
  // read is first needed as late as possible: read r fetches A fragment
  // w4_read(r) (B fragment w4_read(r) - 4 from 4 on); MFMA m updates block
  // (w4_mi(m), w4_mj(m)).  The first MFMA needs two reads, the last read is
  // first used by the 13th.
  // The lane's byte offsets of its fragment reads inside a slot, so that a
  // read is a register base plus an immediate.  K-contiguous (read_frag): the
  // fragment of row block f in sub-step kk is at lane_kc[kk][f % 2] + 8192 (f / 2),
  // because the swizzle of row r + 64 equals that of row r.  N-contiguous
  // (mc_lane_off): fragment f's low half is at lane_mc[f] + 4096 kk and its
  // high half 1024 further, because the swizzle depends on k only through k % 4.
  uint32_t lane_kc[4][2], lane_mc[FN];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int par = 0; par < 2; ++par) lane_kc[kk][par] = tile_off(32 * par + (lane & 31), 2 * kk + (lane >> 5));
  // BN = 128: the wave's columns are 64 wn .. +63 of the one B quarter.
  const int wcol = BN == 256 ? 0 : 64 * wn;
#pragma unroll
  for (int f = 0; f < FN; ++f) lane_mc[f] = mc_lane_off(wcol + 32 * f, lane);
  auto read_sub = [&](int buf, int r, int kk) {
    const char* ta = slot(r, wm);
    const char* tb = slot(r, BN == 256 ? 2 + wn : 2);
#pragma unroll
    for (int x = 0; x < FM + FN; ++x) {
      const int f = BN == 256 ? w4_read(x) : w4n_read(x);
      if (f < FM) {
        fa[buf][f] = *reinterpret_cast<const bf16x8_t*>(ta + lane_kc[kk][f & 1] + 8192 * (f >> 1));
      } else if (LB == KC) {
        const int rb = (BN == 256 ? 0 : 2 * wn) + (f - FM);  // 32-row block of the B quarter
        fb[buf][f - FM] = *reinterpret_cast<const bf16x8_t*>(tb + lane_kc[kk][rb & 1] + 8192 * (rb >> 1));
      } else {
        const char* p = tb + lane_mc[f - FM] + 4096 * kk;
        const i16x4_t lo = ds_read_tr(p), hi = ds_read_tr(p + 1024);
        const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        fb[buf][f - FM] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
  };
  auto mfma_sub = [&](int buf) {
#pragma unroll
    for (int m = 0; m < FM * FN; ++m) {
      const int i = BN == 256 ? w4_mi(m) : m >> 1, j = BN == 256 ? w4_mj(m) : m & 1;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
    }
  };
  // Scheduling of one sub-step: its 16 MFMAs, with the 8 LDS reads between the
  // first eight and NL (at most 8) loads spread over the last eight (a load
  // writes LDS, so the compiler keeps it behind the reads before it).
  auto interleave = [&](auto nl) {
    constexpr int NL = decltype(nl)::value;
    constexpr int NM = FM * FN, NR = FM + FN, S = NM - NR;  // MFMAs, reads, MFMAs after the reads
    static_assert(NL >= 0 && NL <= 8, "loads per sub-step");
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                            // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);                            // up to 3 VALU
      if (m < NR) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                          // LDS read
      } else {
#pragma unroll
        for (int u = (m - NR) * NL / S; u < (m - NR + 1) * NL / S; ++u)
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                        // global load
      }
    }
  };
  auto fence = [&]() { __builtin_amdgcn_sched_barrier(0); };
  using L0 = std::integral_constant<int, 0>;
  using L8 = std::integral_constant<int, 8>;

  // s_waitcnt immediate for vmcnt(n), n < 64, leaving the other counters free.
  auto vm_wait = [&](auto n) {
    constexpr int N = decltype(n)::value;
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  };

  if (nk > 0) {
    // Prologue: K step 0, quarters 0 and 1 of step 1 and the first LC3 loads of
    // window 0 (slots 0-5 and part of 6); wait for step 0.
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) load(0, 0, q, i);
    if (nk > 1) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) load(1, 1, q, i);
#pragma unroll
      for (int n = 0; n < LC3; ++n) window_load(0, n, 1, 2);
      vm_wait(std::integral_constant<int, 8 + LC3>{});
    } else {
      vm_wait(L0{});
    }
    __builtin_amdgcn_s_barrier();
    fence();
    read_sub(0, 0, 0);

    // One K step; LEFT = min(2, K steps after this one) is known at compile time
    // (2: every load is issued; 1: the last but one step; 0: the last); r = k % 5.
    auto k_step = [&](int k, auto left, int r) {
      const int r1 = r == 4 ? 0 : r + 1, r2 = r >= 3 ? r - 3 : r + 2;
      constexpr int LEFT = decltype(left)::value;
      constexpr bool more2 = LEFT >= 2;  // step k+2 exists: load it
      constexpr bool more1 = LEFT >= 1;  // step k+1 exists: wait for it, read it
      // Loads [lo, hi) of window k that exist (those from 8 on load step k+2).
      auto window_part = [&](auto lo, auto hi) {
        constexpr int LO = decltype(lo)::value, HI = decltype(hi)::value;
        constexpr int END = more2 ? HI : more1 ? (HI < 8 ? HI : 8) : LO;
#pragma unroll
        for (int n = LO; n < END; ++n) window_load(k, n, r1, r2);
        interleave(std::integral_constant<int, (END > LO ? END - LO : 0)>{});
      };
      // sub-step 0
      fence();
      read_sub(1, r, 1);
      mfma_sub(0);
      window_part(std::integral_constant<int, LC3>{}, std::integral_constant<int, LC3 + LC0>{});
      fence();
      // sub-step 1
      read_sub(0, r, 2);
      mfma_sub(1);
      window_part(std::integral_constant<int, LC3 + LC0>{}, std::integral_constant<int, LC3 + LC0 + LC1>{});
      fence();
      // sub-step 2
      read_sub(1, r, 3);
      mfma_sub(0);
      window_part(std::integral_constant<int, LC3 + LC0 + LC1>{}, std::integral_constant<int, 16>{});
      fence();
      if constexpr (more1) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): sub-step 3's fragments are in registers
        if constexpr (more2) vm_wait(L8{});  // step k+1 has landed; k+2's first half may be in flight
        else vm_wait(L0{});
        __builtin_amdgcn_s_barrier();
        fence();
        // sub-step 3: the first LC3 loads of window k+1, into step k's slots
        read_sub(0, r1, 0);
        const int r3 = r2 == 4 ? 0 : r2 + 1;
        if constexpr (more2) {
#pragma unroll
          for (int n = 0; n < LC3; ++n) window_load(k + 1, n, r2, r3);
        }
        mfma_sub(1);
        if constexpr (more2) interleave(std::integral_constant<int, LC3>{}); else interleave(L0{});
        fence();
      } else {
        mfma_sub(1);
        fence();
      }
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
  __syncthreads();  // every wave is done with the operand slots

  // Epilogue, one 64-column half of the wave's sub-tile at a time, staged in the
  // wave's own 16 KiB of LDS.
#pragma unroll
  for (int h = 0; h < FN / 2; ++h) {
    f32x16_t part[FM][2];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) part[i][j] = acc[i][2 * h + j];
    store_tile<EPI>(part, args, smem + wave * (64 * ROW_B), m0 + 128 * wm, n0 + (BN / 2) * wn + 64 * h, split,
                    lane);
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
    return launch_kernel(kern::gemm_w4_kernel<LB, EPI, BN>, dim3(blocks), dim3(256), s, a);
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
