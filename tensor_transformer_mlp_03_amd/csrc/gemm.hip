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
//  * Operand tiles go from memory straight into LDS with buffer_load ... lds
//    (16 bytes per lane, no staging registers, no LDS write instructions) into a
//    ring of STAGES buffers, STAGES-1 K steps ahead of the MFMAs.  A buffer
//    descriptor returns zeros for out-of-range chunks, which handles ragged
//    sizes without branches.  One s_waitcnt + s_barrier per K step.
//  * LDS keeps each operand in its memory layout.  A K-contiguous tile is read
//    with ds_read_b128 (8 consecutive k of one row per lane, the MFMA operand
//    layout); an M/N-contiguous tile is read with two ds_read_b64_tr_b16, whose
//    16-lane transpose delivers 4 consecutive k of one column per lane.  No
//    operand is transposed in registers or in memory.
//  * 16-byte chunks are XOR-swizzled inside each LDS row so that the rows one
//    read instruction touches fall on distinct banks; the loads apply the
//    inverse permutation on the memory side, so each DMA still writes 1 KiB of
//    contiguous LDS.
//  * The MFMA takes the B fragment as its first operand, so each lane ends with
//    4 consecutive output columns of one row: epilogues store 8- or 16-byte
//    vectors.
//  * Workgroups are renumbered so that consecutive output tiles (which share
//    operand panels) run on the same XCD and its L2, then grouped 8 tiles tall.

#include "common.h"

namespace tpmlp {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

#ifndef TPMLP_GEMM_BK
#define TPMLP_GEMM_BK 64
#endif
#ifndef TPMLP_GEMM_STAGES
#define TPMLP_GEMM_STAGES 2
#endif
#ifndef TPMLP_GEMM_WAVES_M
#define TPMLP_GEMM_WAVES_M 2
#endif
#ifndef TPMLP_GEMM_WAVES_N
#define TPMLP_GEMM_WAVES_N 4
#endif

constexpr int GROUP_M = 8;
constexpr int NUM_XCD = 8;
constexpr uint32_t OOB = 0x7FFFFFF0u;  // voffset past num_records: the load returns 0

// ds read offsets below are byte offsets inside one LDS stage.

// Swizzle of the 16-byte chunk index inside a row of a K-contiguous tile
// ([rows][BK]).  With 8 chunks per row: rows r .. r+15 read at one chunk land on
// 16 distinct (row parity, chunk) bank groups.  With 4 chunks per row (64-byte
// rows, four to a 256-byte bank window): rows r, r+4, r+8, r+12 get distinct chunks.
template <int CHUNKS>
__device__ __forceinline__ int swz_kc(int r) {
  if (CHUNKS == 8) return (r ^ (r >> 3)) & 7;
  return (r >> 2) & 3;
}

// Swizzle of the chunk index inside a row of an M/N-contiguous tile ([BK][cols],
// one row per k).  A transpose read touches rows k..k+3 at 2-4 adjacent chunks;
// XOR-ing chunk bits 1..3 with (k0, k1, k0) sends them to distinct banks.
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
__device__ __forceinline__ float phi_cdf(float p) { return 0.5f + 0.5f * erff(p * 0.70710678118654752f); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)OOB, 0x00020000);
}

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt at their maxima (waits on vmcnt only).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Wait until at most min(ahead, S) K steps' loads (LOADS each) are outstanding.
template <int S, int LOADS>
__device__ __forceinline__ void wait_steps(int ahead) {
  if constexpr (S == 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= S) wait_vmcnt<S * LOADS>();
    else wait_steps<S - 1, LOADS>(ahead);
  }
}

// One operand's tile of one K step, loaded straight into LDS.
//   KC: tile [R][BK],  element (r, k) at r*BK*2 + ((k/8) ^ swz_kc(r))*16 + (k%8)*2
//   MC: tile [BK][R],  element (k, r) at k*R*2 + ((r/8) ^ swz_mc(k))*16 + (r%8)*2
// DMA instruction i of wave w writes LDS chunks (i*NWAVES + w)*64 + lane; each
// lane loads the memory chunk that the swizzle places there.
template <int R, int BK, int NWAVES, int LAYOUT>
struct Loader {
  static constexpr int CHUNKS = R * BK / 8;
  static constexpr int PER_WAVE = CHUNKS / 64 / NWAVES;  // DMA instructions per wave and K step
  static_assert(CHUNKS % (64 * NWAVES) == 0, "tile must divide evenly over the waves");
  uint32_t off[PER_WAVE];   // byte offset of the lane's chunk from the K step's base
  int o_lim[PER_WAVE];      // the chunk's outer index (row for KC, column for MC)
  int k_rel[PER_WAVE];      // the chunk's k offset inside the K step

  __device__ __forceinline__ void init(int64_t ld, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int q = (i * NWAVES + wave) * 64 + lane;
      if (LAYOUT == KC) {
        constexpr int CPR = BK / 8;
        const int r = q / CPR, c = (q % CPR) ^ swz_kc<CPR>(r);
        o_lim[i] = r;
        k_rel[i] = 8 * c;
        off[i] = (uint32_t)(((int64_t)r * ld + 8 * c) * 2);
      } else {
        constexpr int CPR = R / 8;
        const int k = q / CPR, c = (q % CPR) ^ swz_mc<CPR>(k);
        o_lim[i] = 8 * c;
        k_rel[i] = k;
        off[i] = (uint32_t)(((int64_t)k * ld + 8 * c) * 2);
      }
    }
  }

  // base: the operand's element (outer0, k0) for KC, (k0, outer0) for MC.
  __device__ __forceinline__ void issue(const uint16_t* base, char* lds_stage, int outer_left, int k_left,
                                        int wave) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base);
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const bool ok = (o_lim[i] < outer_left) && (k_rel[i] < k_left);
      char* dst = lds_stage + (i * NWAVES + wave) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)dst, 16, ok ? off[i] : OOB, 0, 0, 0);
    }
  }
};

// MFMA operand fragment of a 32-row (or 32-column) slice at sub-step kk (16 wide):
// lane l gets 8 consecutive k (8*(l/32) .. +7 within the sub-step) of row/column l%32.
template <int R, int BK, int LAYOUT>
__device__ __forceinline__ bf16x8_t read_frag(const char* lds, int o0, int kk, int lane) {
  if (LAYOUT == KC) {
    constexpr int CPR = BK / 8;
    const int r = o0 + (lane & 31);
    const int c = 2 * kk + (lane >> 5);
    return *reinterpret_cast<const bf16x8_t*>(lds + r * BK * 2 + ((c ^ swz_kc<CPR>(r)) << 4));
  } else {
    // ds_read_b64_tr_b16: in each 16-lane group, result lane i element e comes
    // from source lane 4e + i/4, slot i%4.  Source lane j therefore reads the 4
    // elements (k0 + j/4, o .. o+3) with o = o0 + 4*(j%4): result lane i then
    // holds column o0 + i at k0 .. k0+3.
    constexpr int CPR = R / 8;
    const int g = lane >> 4, j = lane & 15;
    const int o = o0 + 16 * (g & 1) + 4 * (j & 3);
    const int kbase = 16 * kk + 8 * (g >> 1) + (j >> 2);
    const int c = o >> 3, half = (o & 7) * 2;
    const int k_lo = kbase, k_hi = kbase + 4;
    const char* p_lo = lds + k_lo * R * 2 + ((c ^ swz_mc<CPR>(k_lo)) << 4) + half;
    const char* p_hi = lds + k_hi * R * 2 + ((c ^ swz_mc<CPR>(k_hi)) << 4) + half;
    i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p_lo));
    i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p_hi));
    i16x8_t both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, both);
  }
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

}  // namespace

// The kernel has external linkage (a kernel template in an anonymous namespace
// does not get its host launch stubs emitted for every instantiation).
namespace kern {

template <int BM, int BN, int BK, int STAGES, int WAVES_M, int WAVES_N, int LA, int LB, int EPI>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N)
gemm_kernel(GemmArgs args) {
  // The body is compiled for the device only: the host pass needs just the
  // launch stub, and device builtins (buffer descriptors, LDS DMA) have no host
  // form.
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NWAVES = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  constexpr int STAGE = A_BYTES + B_BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];

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

  using LoaderA = Loader<BM, BK, NWAVES, LA>;
  using LoaderB = Loader<BN, BK, NWAVES, LB>;
  LoaderA la;
  LoaderB lb;
  la.init(args.lda, wave, lane);
  lb.init(args.ldb, wave, lane);
  constexpr int LOADS = LoaderA::PER_WAVE + LoaderB::PER_WAVE;

  // Element (outer0, k) of an operand for the K step starting at k.
  auto a_base = [&](int k) {
    return LA == KC ? args.a + (int64_t)m0 * args.lda + k : args.a + (int64_t)k * args.lda + m0;
  };
  auto b_base = [&](int k) {
    return LB == KC ? args.b + (int64_t)n0 * args.ldb + k : args.b + (int64_t)k * args.ldb + n0;
  };
  auto issue = [&](int step) {
    const int k = k_begin + step * BK;
    char* st = smem + (step % STAGES) * STAGE;
    la.issue(a_base(k), st, args.M - m0, k_end - k, wave);
    lb.issue(b_base(k), st + A_BYTES, args.N - n0, k_end - k, wave);
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue(s);

  for (int kt = 0; kt < nk; ++kt) {
    // This wave's loads for step kt are done once at most the loads of the
    // steps issued after it are outstanding.
    wait_steps<STAGES - 2, LOADS>(nk - 1 - kt);
    // Everyone's loads for step kt have landed, and everyone has finished
    // reading the stage that the next issue overwrites (step kt-1's).
    __builtin_amdgcn_s_barrier();
    if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1);
    const char* cur = smem + (kt % STAGES) * STAGE;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = read_frag<BM, BK, LA>(cur, wm * WM + 32 * i, kk, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = read_frag<BN, BK, LB>(cur + A_BYTES, wn * WN + 32 * j, kk, lane);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
  }

  // Epilogue.  With the B fragment as the MFMA's first operand, accumulator
  // register r of fragment (i, j) holds C[32i + lane%32][32j + 8(r/4) + 4(lane/32) + r%4]
  // of the wave's sub-tile: 4 consecutive columns per register group.
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row = m0 + wm * WM + 32 * i + (lane & 31);
    if (row >= args.M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = n0 + wn * WN + 32 * j + 8 * g + 4 * (lane >> 5);
        if (col >= args.N) continue;  // N % 8 == 0: the 4 columns are in or out together
        const int64_t o = (int64_t)row * args.ldo + col;
        const f32x4_t x = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        if (EPI == EPI_F32) {
          float* out = reinterpret_cast<float*>(args.out) + (int64_t)split * args.split_stride;
          *reinterpret_cast<f32x4_t*>(out + o) = x;
        } else if (EPI == EPI_GELU) {
          u16x4_t gv, pv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            gv[e] = f32_to_bf16(x[e] * phi_cdf(x[e]));
            pv[e] = f32_to_bf16(x[e]);
          }
          *reinterpret_cast<u16x4_t*>(reinterpret_cast<uint16_t*>(args.out) + o) = gv;
          if (args.out2) *reinterpret_cast<u16x4_t*>(args.out2 + o) = pv;
        } else if (EPI == EPI_BF16) {
          u16x4_t pv;
#pragma unroll
          for (int e = 0; e < 4; ++e) pv[e] = f32_to_bf16(x[e]);
          *reinterpret_cast<u16x4_t*>(reinterpret_cast<uint16_t*>(args.out) + o) = pv;
        } else {  // EPI_DGELU
          const u16x4_t pb = *reinterpret_cast<const u16x4_t*>(args.aux + o);
          u16x4_t dv, gv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = bf16_to_f32(pb[e]);
            const float cdf = phi_cdf(p);
            const float pdf = 0.39894228040143268f * __expf(-0.5f * p * p);
            dv[e] = f32_to_bf16(x[e] * (cdf + p * pdf));
            gv[e] = f32_to_bf16(p * cdf);
          }
          *reinterpret_cast<u16x4_t*>(reinterpret_cast<uint16_t*>(args.out) + o) = dv;
          *reinterpret_cast<u16x4_t*>(args.out2 + o) = gv;
        }
      }
    }
  }
#else
  (void)args;
#endif
}

}  // namespace kern

namespace {

template <int BM, int BN, int BK, int ST, int WM_, int WN_, int LA, int LB, int EPI>
hipError_t launch_one(const GemmArgs& a, int splits, hipStream_t s) {
  const int blocks = a.tiles_m * a.tiles_n * splits;
  hipLaunchKernelGGL((kern::gemm_kernel<BM, BN, BK, ST, WM_, WN_, LA, LB, EPI>), dim3(blocks), dim3(64 * WM_ * WN_), 0, s, a);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int ST, int WM_, int WN_>
hipError_t dispatch_layout(Layout la, Layout lb, Epi epi, const GemmArgs& a, int splits, hipStream_t s) {
  if (la == KC && lb == MC) {
    switch (epi) {
      case EPI_GELU: return launch_one<BM, BN, BK, ST, WM_, WN_, KC, MC, EPI_GELU>(a, splits, s);
      case EPI_F32: return launch_one<BM, BN, BK, ST, WM_, WN_, KC, MC, EPI_F32>(a, splits, s);
      case EPI_BF16: return launch_one<BM, BN, BK, ST, WM_, WN_, KC, MC, EPI_BF16>(a, splits, s);
      default: break;
    }
  } else if (la == KC && lb == KC) {
    switch (epi) {
      case EPI_DGELU: return launch_one<BM, BN, BK, ST, WM_, WN_, KC, KC, EPI_DGELU>(a, splits, s);
      case EPI_F32: return launch_one<BM, BN, BK, ST, WM_, WN_, KC, KC, EPI_F32>(a, splits, s);
      default: break;
    }
  } else if (la == MC && lb == MC) {
    if (epi == EPI_F32) return launch_one<BM, BN, BK, ST, WM_, WN_, MC, MC, EPI_F32>(a, splits, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int tile_bm(TileCfg t) { return t == TILE_256x256 ? 256 : 128; }
int tile_bn(TileCfg t) { return t == TILE_256x256 ? 256 : 128; }

hipError_t launch_gemm(TileCfg tile, Layout la, Layout lb, Epi epi, const GemmArgs& args, int splits,
                       hipStream_t stream) {
  switch (tile) {
    case TILE_256x256: return dispatch_layout<256, 256, TPMLP_GEMM_BK, TPMLP_GEMM_STAGES, TPMLP_GEMM_WAVES_M, TPMLP_GEMM_WAVES_N>(la, lb, epi, args, splits, stream);
    case TILE_128x128: return dispatch_layout<128, 128, 64, 2, 2, 2>(la, lb, epi, args, splits, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tpmlp
