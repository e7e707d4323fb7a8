// libtpmlp host side: the C ABI of include/tpmlp.h.
//
// Argument checking (pointers, shapes, alignment, workspace size, overlaps)
// happens before any HIP call, so that every error path can be exercised on a
// machine without a GPU.  Then the device is checked to be gfx950 and the
// kernels are enqueued on the caller's stream.
//
// Rank i's forward is two launches (the column-parallel GEMM with the GeLU
// epilogue, the row-parallel GEMM writing the float32 partial), or, for small
// hidden sizes, one fused launch and its chunk sum; its backward is four or five
// (optional recompute of the pre-activation, the dGeLU GEMM, the two
// weight-gradient GEMMs, the input-gradient GEMM), plus split-K reductions where
// an output has too few tiles to fill the chip.  The weight-gradient GEMMs read
// X and dZ transposed (and dP for large H), so that their operands are
// K-contiguous; the transposes of X and dZ are made once per backward call (once
// for all shards in the t-shard driver).  The t-shard drivers run the shards one
// after another and add the partials in rank order, standing in for the
// all-reduces of the row-parallel output (forward) and of the column-parallel
// input gradient (backward) ("大模型训练" notes §3.1; QLM page §2.1.2.2 parts
// 1-3); without per-shard outputs the additions happen in the epilogues of the
// products that make the partials.

#include "../../include/tpmlp.h"
#include "common.h"

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

namespace tpmlp {

thread_local LaunchEvents g_launch_events;

namespace {

// The no-allocation forward's workspace: one array per GPU, reserved with the
// library's code object.  In host code its name is only a stand-in for the
// symbol; the device address comes from hipGetSymbolAddress (noalloc_scratch).
__device__ __align__(256) unsigned char scratch[TPMLP_NOALLOC_SCRATCH_BYTES];

// Largest M, H, F_i (and t * F_i for the whole-weight drivers).  The kernels
// address operands through buffer descriptors with 32-bit byte offsets from a
// wave-uniform base, spanning at most 128 rows of a row-major operand:
// 127 * 2^23 * 2 bytes stays below the descriptors' 2^31-byte range.
constexpr int64_t MAX_DIM = int64_t(1) << 23;
constexpr int NUM_CU = 256;  // MI355X compute units, used to size split-K
constexpr size_t WS_ALIGN = 256;

thread_local std::string g_last_error;

tpmlp_status fail(tpmlp_status s, const std::string& what) {
  g_last_error = what;
  return s;
}

size_t align_up(size_t x) { return (x + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN; }

bool shape_ok(int64_t v) { return v > 0 && v <= MAX_DIM && (v % 8) == 0; }

// ---------------------------------------------------------------------------
// Launch plan: tile shape and split-K count of each GEMM, workspace layout.
// Depends on shapes only, so workspace queries need no device.
// ---------------------------------------------------------------------------
struct GemmPlan {
  TileCfg tile;
  int splits;
  int k_split;
  // Hybrid plan (n_full > 0): output columns [0, n_full) are whole waves of
  // unsplit 256 x 256 tiles with the product's own epilogue; only the tail
  // columns [n_full, N) are split along K (splits, k_split) and reduced.
  int n_full = 0;
};

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Time model used to pick a tile and a split-K count: workgroups run in waves
// over the chip's CUs (one block per CU: every tile takes the whole LDS); a
// block's time is proportional to its MACs at the measured per-CU rate of its
// tile; split-K adds a float32 round trip of the slices through memory and one
// reduction launch.  Splits keep at least 512 of K each.
constexpr double CU_RATE_256 = 4.3e12;      // flop/s per CU, 256x256 tile
constexpr double CU_RATE_256x128 = 3.8e12;  // flop/s per CU, 256x128 tile (half the MFMAs per load)
constexpr double CU_RATE_128 = 3.3e12;      // flop/s per CU, 128x128 tile (a quarter)
constexpr double SPLIT_BW = 4.0e12;         // bytes/s for the slices' write and re-read
constexpr double LAUNCH_S = 5e-6;

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K) {
  GemmPlan best{TILE_256x256, 1, (int)((K + TILE_BK - 1) / TILE_BK * TILE_BK)};
  double best_t = 1e30;
  for (TileCfg tile : {TILE_256x256, TILE_256x128, TILE_128x128}) {
    const int64_t bm = tile_bm(tile), bn = tile_bn(tile);
    const int64_t tiles = (int64_t)ceil_div(M, bm) * ceil_div(N, bn);
    for (int s = 1; s <= 16; ++s) {
      const int64_t kslice = ((K + s - 1) / s + TILE_BK - 1) / TILE_BK * TILE_BK;
      const int splits = ceil_div(K, kslice);
      if (splits != s) continue;
      if (s > 1 && kslice < 512) break;
      const double flops = double(bm * bn * 2 * kslice);
      const int64_t blocks = tiles * s;
      const double rate = tile == TILE_256x256 ? CU_RATE_256 : tile == TILE_256x128 ? CU_RATE_256x128 : CU_RATE_128;
      double t = double((blocks + NUM_CU - 1) / NUM_CU) * flops / rate;
      if (s > 1) t += double(s) * M * N * 4 * 2 / SPLIT_BW + LAUNCH_S;
      if (t < best_t * (1 - 1e-9)) {
        best_t = t;
        best = GemmPlan{tile, s, (int)kslice};
      }
    }
  }
  // Hybrid: when the 256 x 256 tiles are not a whole number of waves, run the
  // largest block of columns that is as whole waves unsplit, and split only the
  // tail.  The split-K round trip then covers the tail alone.
  {
    const int64_t tm = ceil_div(M, 256), tn = ceil_div(N, 256);
    int64_t c = tn - 1;
    while (c > 0 && (tm * c) % NUM_CU != 0) --c;
    if (tm * tn > NUM_CU && c > 0) {
      const int64_t kfull = (K + TILE_BK - 1) / TILE_BK * TILE_BK, nt = N - c * 256;
      const double t_full = double(tm * c / NUM_CU) * double(256 * 256 * 2 * kfull) / CU_RATE_256;
      for (int s = 2; s <= 16; ++s) {
        const int64_t kslice = ((K + s - 1) / s + TILE_BK - 1) / TILE_BK * TILE_BK;
        if (ceil_div(K, kslice) != s) continue;
        if (kslice < 512) break;
        const int64_t waves = (tm * (tn - c) * s + NUM_CU - 1) / NUM_CU;
        const double t = t_full + double(waves) * double(256 * 256 * 2 * kslice) / CU_RATE_256 +
                         double(s) * M * nt * 4 * 2 / SPLIT_BW + 2 * LAUNCH_S;
        if (t < best_t * (1 - 1e-9)) {
          best_t = t;
          best = GemmPlan{TILE_256x256, s, (int)kslice, (int)(c * 256)};
        }
      }
    }
  }
  return best;
}

size_t part_bytes(const GemmPlan& p, int64_t M, int64_t N) {
  return p.splits > 1 ? size_t(p.splits) * M * (N - p.n_full) * 4 : 0;
}

// Batches of the t-shard drivers' first products.  F1, the recompute and dGeLU
// of different shards share their A operand (X or dZ) and differ only in the
// weight and the outputs, so several shards' can run as one launch.  Where one
// shard's product is a single unsplit wave of small tiles (short K, few
// tiles: the 7B-class shard), a batch of g shards on 256 x 256 tiles fills the
// chip with the faster tile and pays the launch, the ramp and the last tiles'
// epilogue once per g.  Taken when the model above gives at least 10% less
// time per shard.  Unsplit either way, so every output element is summed in
// the same order and the results have the same bits as unbatched launches.
struct BatchPlan {
  int g = 1;     // shards per launch (1: no batching)
  GemmPlan plan;
};

double unsplit_time(TileCfg tile, int64_t M, int64_t N, int64_t K, int copies) {
  const int64_t tiles = (int64_t)ceil_div(M, tile_bm(tile)) * ceil_div(N, tile_bn(tile)) * copies;
  const double rate = tile == TILE_256x256 ? CU_RATE_256 : tile == TILE_256x128 ? CU_RATE_256x128 : CU_RATE_128;
  const int64_t kfull = (K + TILE_BK - 1) / TILE_BK * TILE_BK;
  return double((tiles + NUM_CU - 1) / NUM_CU) * double(tile_bm(tile) * tile_bn(tile) * 2 * kfull) / rate;
}

BatchPlan plan_batch(int64_t M, int64_t N, int64_t K, int t) {
  BatchPlan b;
  b.plan = plan_gemm(M, N, K);
  if (t < 2 || b.plan.splits != 1) return b;
  double best = unsplit_time(b.plan.tile, M, N, K, 1);
  for (int g = 2; g <= std::min(t, MAX_BATCH); ++g)
    for (TileCfg tile : {TILE_256x256, TILE_256x128, TILE_128x128}) {
      const double per_shard = unsplit_time(tile, M, N, K, g) / g;
      if (per_shard < 0.9 * best) {
        best = per_shard;
        b.g = g;
        b.plan = GemmPlan{tile, 1, (int)((K + TILE_BK - 1) / TILE_BK * TILE_BK)};
      }
    }
  return b;
}

// The forward products read A_i and B_i N-contiguous.  Transposing them first
// (4*H*F bytes of memory traffic at about 5.5 TB/s) lets the products run with
// both operands K-contiguous, measured at about 1.2 PFLOP/s against about 1.14
// with B read through transposing LDS loads.  On two products of 2*M*H*F flops
// that saves about M*H*F*1.75e-16 s against H*F*7.3e-13 s for the transposes;
// they are made only when the saving is 1.5 times the cost, which covers the
// rates' spread over shapes (M above about 6000: the long-context chunk,
// M = 32768, qualifies; M = 2048 and 4096 do not).
constexpr double RATE_KC = 1.2e15, RATE_MC = 1.14e15, TRANSPOSE_BW = 5.5e12, TRANSPOSE_MARGIN = 1.5;

bool transpose_weights(int64_t M, int64_t H, int64_t F) {
  const double saved = 2.0 * 2.0 * double(M) * H * F * (1.0 / RATE_MC - 1.0 / RATE_KC);
  const double cost = 4.0 * double(H) * F / TRANSPOSE_BW;
  return saved > TRANSPOSE_MARGIN * cost;
}

// The fused forward (both products and GeLU in one launch, G kept in LDS) is
// taken for hidden sizes it holds (H a multiple of 64, at most 256) when its
// float32 chunk partials, F/64 slices of M x H, stay small: it trades G's trip
// through memory (4 M F bytes) and a launch for partials of M H F / 16 bytes,
// which pays only where the shard's time is launch and memory latency.
constexpr size_t FUSED_PART_MAX = size_t(8) << 20;

bool fused_fwd(int64_t M, int64_t H, int64_t F) {
  return ffn_fused_fits(H) && size_t(ffn_chunks(F)) * M * H * 4 <= FUSED_PART_MAX;
}

struct FwdPlan {
  GemmPlan g1, g2;
  bool wt;     // products read A_i^T and B_i^T from the workspace
  bool fused;  // one fused launch (chunk partials at off_part) and their sum
  size_t off_G, off_At, off_Bt, off_part, total;
};

FwdPlan plan_fwd(int64_t M, int64_t H, int64_t F) {
  FwdPlan p;
  p.fused = fused_fwd(M, H, F);
  if (p.fused) {
    p.g1 = p.g2 = GemmPlan{TILE_128x128, 1, 0};
    p.wt = false;
    p.off_G = p.off_At = p.off_Bt = p.off_part = 0;
    p.total = ffn_chunks(F) > 1 ? align_up(size_t(ffn_chunks(F)) * M * H * 4) : WS_ALIGN;
    return p;
  }
  p.g1 = plan_gemm(M, F, H);
  p.g2 = plan_gemm(M, H, F);
  p.wt = transpose_weights(M, H, F);
  const size_t hf = p.wt ? align_up(size_t(H) * F * 2) : 0;
  p.off_G = 0;
  p.off_At = align_up(size_t(M) * F * 2);
  p.off_Bt = p.off_At + hf;
  p.off_part = p.off_Bt + hf;
  p.total = p.off_part + align_up(std::max(part_bytes(p.g1, M, F), part_bytes(p.g2, M, H)));
  return p;
}

// dA_i = X^T dP_i reads dP_i N-contiguous unless dP_i is transposed first; the
// transpose (4 M F bytes) pays when the one product's saving, at the rates above,
// is 1.5 times its cost, i.e. for H above about 12400 (the 530B-class shard).
bool transpose_dp(int64_t M, int64_t H, int64_t F) {
  const double saved = 2.0 * double(M) * H * F * (1.0 / RATE_MC - 1.0 / RATE_KC);
  const double cost = 4.0 * double(M) * F / TRANSPOSE_BW;
  return saved > TRANSPOSE_MARGIN * cost;
}

struct BwdPlan {
  GemmPlan g0, g1, gdb, gda, gdx;
  bool wt;   // the recompute product reads A_i^T from the workspace
  bool tdp;  // dA reads dP_i^T from the workspace
  size_t off_Xt, off_dZt, off_At, off_P, off_Gt, off_dP, off_dPt, off_part, total;
};

BwdPlan plan_bwd(int64_t M, int64_t H, int64_t F, bool recompute) {
  BwdPlan p;
  p.g0 = plan_gemm(M, F, H);
  p.g1 = plan_gemm(M, F, H);
  p.gdb = plan_gemm(F, H, M);
  p.gda = plan_gemm(H, F, M);
  p.gdx = plan_gemm(M, H, F);
  const size_t mf = align_up(size_t(M) * F * 2);
  const size_t mh = align_up(size_t(M) * H * 2);
  p.wt = recompute && transpose_weights(M, H, F);
  p.off_Xt = 0;
  p.off_dZt = mh;
  p.off_At = 2 * mh;
  p.off_P = p.off_At + (p.wt ? align_up(size_t(H) * F * 2) : 0);
  p.off_Gt = p.off_P + (recompute ? mf : 0);
  p.tdp = transpose_dp(M, H, F);
  p.off_dP = p.off_Gt + mf;
  p.off_dPt = p.off_dP + mf;
  p.off_part = p.off_dPt + (p.tdp ? mf : 0);
  size_t part = recompute ? part_bytes(p.g0, M, F) : 0;
  part = std::max({part, part_bytes(p.g1, M, F), part_bytes(p.gdb, F, H), part_bytes(p.gda, H, F),
                   part_bytes(p.gdx, M, H)});
  p.total = p.off_part + align_up(part);
  return p;
}

// Workspace of one shard inside the t-shard drivers: fits the forward and both
// backward modes; the drivers' partial buffers follow it.
size_t shard_ws_bytes(int64_t M, int64_t H, int64_t F) {
  return align_up(std::max(plan_fwd(M, H, F).total, plan_bwd(M, H, F, true).total));
}

// The t-shard drivers batch the shards' first products (F1; the recompute and
// dGeLU) when the forward runs unfused on weights read in place.
BatchPlan plan_shard_batch(int t, int64_t M, int64_t H, int64_t F) {
  if (fused_fwd(M, H, F) || transpose_weights(M, H, F)) return BatchPlan{1, plan_gemm(M, F, H)};
  return plan_batch(M, F, H, t);
}

// Per batched shard: G_i (forward) or P_i, G_i^T and dP_i (backward), bf16 [M][F].
size_t batch_slot_bytes(int64_t M, int64_t F) { return 3 * align_up(size_t(M) * F * 2); }

size_t batch_area_bytes(int t, int64_t M, int64_t H, int64_t F) {
  const BatchPlan b = plan_shard_batch(t, M, H, F);
  return b.g > 1 ? size_t(b.g) * batch_slot_bytes(M, F) : 0;
}

// ---------------------------------------------------------------------------
// Device check (gfx950 only), cached per device.
// ---------------------------------------------------------------------------
std::mutex g_dev_mu;
std::vector<int> g_dev_ok;  // -1 unknown, 0 no, 1 yes

tpmlp_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TPMLP_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if ((int)g_dev_ok.size() <= dev) g_dev_ok.resize(dev + 1, -1);
  if (g_dev_ok[dev] < 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(TPMLP_ERR_HIP, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
    g_dev_ok[dev] = std::string(prop.gcnArchName).rfind("gfx950", 0) == 0 ? 1 : 0;
    if (!g_dev_ok[dev]) {
      g_last_error = std::string("device is ") + prop.gcnArchName + ", not gfx950";
    }
  }
  if (!g_dev_ok[dev]) return fail(TPMLP_ERR_UNSUPPORTED, "current device is not gfx950");
  return TPMLP_OK;
}

// ---------------------------------------------------------------------------
// Kernel timing: while enabled, an event pair bound to each timed call's first
// and last kernel dispatch (launch_kernel; g_launch_events is defined at the
// top of this file).
// ---------------------------------------------------------------------------

struct Timing {
  bool on = false;
  unsigned kinds = 0;  // bit k set: launches of kind k are timed
  int cap = 0, n = 0, dropped = 0;
  std::vector<hipEvent_t> ev;
  std::vector<int> kind, disp;   // per record: kernel kind, kernel dispatches inside it
  std::vector<int> last_kind;     // records of the last finished timing window
  std::vector<int> last_disp;
  std::vector<double> last_ms;
  ~Timing() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  }
};
thread_local Timing g_timing;

// One timing record of kind `kind` around `launch`, which enqueues `dispatches`
// kernels (a hybrid split product is two).
template <class F>
hipError_t timed(int kind, hipStream_t s, F&& launch, int dispatches = 1) {
  Timing& t = g_timing;
  if (!t.on || !((t.kinds >> kind) & 1u)) return launch();
  if (t.n >= t.cap) {
    ++t.dropped;
    return launch();
  }
  LaunchEvents& le = g_launch_events;
  le = LaunchEvents{t.ev[2 * t.n], t.ev[2 * t.n + 1], dispatches};
  hipError_t e = launch();
  const LaunchEvents rest = le;
  le = LaunchEvents{};
  if (e != hipSuccess) return e;
  // A call that dispatched fewer kernels than it declared leaves an event
  // unbound: record it on the stream instead.
  if (rest.start) e = hipEventRecord(rest.start, s);
  if (e == hipSuccess && rest.left > 0) e = hipEventRecord(rest.stop, s);
  if (e != hipSuccess) return e;
  t.disp[t.n] = dispatches;
  t.kind[t.n++] = kind;
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Argument checks
// ---------------------------------------------------------------------------
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

struct Range {
  const void* p;
  size_t bytes;
  const char* name;
};

bool overlap(const Range& a, const Range& b) {
  if (!a.p || !b.p || !a.bytes || !b.bytes) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Each output must be disjoint from every other range.
tpmlp_status check_alias(const std::vector<Range>& outs, const std::vector<Range>& ins) {
  for (size_t i = 0; i < outs.size(); ++i) {
    for (size_t j = i + 1; j < outs.size(); ++j)
      if (overlap(outs[i], outs[j]))
        return fail(TPMLP_ERR_ALIAS, std::string(outs[i].name) + " overlaps " + outs[j].name);
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return fail(TPMLP_ERR_ALIAS, std::string(outs[i].name) + " overlaps " + r.name);
  }
  return TPMLP_OK;
}

tpmlp_status check_shape(int64_t M, int64_t H, int64_t F) {
  if (!shape_ok(M) || !shape_ok(H) || !shape_ok(F))
    return fail(TPMLP_ERR_SHAPE, "M, H and F_i must be positive multiples of 8, at most 2^23");
  return TPMLP_OK;
}

tpmlp_status check_ptrs(std::initializer_list<std::pair<const void*, const char*>> ptrs) {
  for (auto& p : ptrs)
    if (!p.first) return fail(TPMLP_ERR_NULL, std::string(p.second) + " is NULL");
  for (auto& p : ptrs)
    if (!aligned16(p.first)) return fail(TPMLP_ERR_ALIGN, std::string(p.second) + " is not 16-byte aligned");
  return TPMLP_OK;
}

tpmlp_status hip_fail(hipError_t e, const char* what) {
  return fail(TPMLP_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// GEMM launch helpers
// ---------------------------------------------------------------------------
GemmArgs gemm_args(const void* a, int64_t lda, const void* b, int64_t ldb, int64_t M, int64_t N,
                   int64_t K, const GemmPlan& p, void* out, int64_t ldo) {
  GemmArgs g{};
  g.a = static_cast<const uint16_t*>(a);
  g.b = static_cast<const uint16_t*>(b);
  g.lda = lda;
  g.ldb = ldb;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.k_split = p.k_split;
  g.out = out;
  g.ldo = ldo;
  g.split_stride = M * N;
  g.tiles_m = ceil_div(M, tile_bm(p.tile));
  g.tiles_n = ceil_div(N, tile_bn(p.tile));
  return g;
}

// One product with its epilogue.  Split along K, the slices go to `part` as
// float32 and the reduction applies the epilogue.
hipError_t run_gemm(int kind, Layout la, Layout lb, Epi epi, const void* a, int64_t lda, const void* b,
                    int64_t ldb, int64_t M, int64_t N, int64_t K, const GemmPlan& p, void* out, uint16_t* out2,
                    const uint16_t* aux, float* part, hipStream_t s, int64_t ldo = 0, int64_t ldt = 0) {
  // ldo: row stride of out (and of out2 and aux for the GeLU and dGeLU
  // epilogues); 0 means N.  ldt: row stride of the dGeLU epilogue's transposed
  // out2; 0 means M (the product's rows can be a row block of a taller one).
  if (ldo == 0) ldo = N;
  if (ldt == 0) ldt = M;
  if (p.splits == 1) {
    GemmArgs g = gemm_args(a, lda, b, ldb, M, N, K, p, out, ldo);
    g.out2 = out2;
    g.aux = aux;
    g.ldt = ldt;
    return timed(kind, s, [&] { return launch_gemm(p.tile, la, lb, epi, g, 1, s); });
  }
  if (p.n_full > 0) {
    // Hybrid: the whole-wave column block with the epilogue, then the tail
    // columns split into `part` (one timing record for both launches).
    const int64_t nf = p.n_full, nt = N - nf;
    const GemmPlan pf{p.tile, 1, (int)((K + TILE_BK - 1) / TILE_BK * TILE_BK)};
    GemmArgs gf = gemm_args(a, lda, b, ldb, M, nf, K, pf, out, ldo);
    gf.out2 = out2;
    gf.aux = aux;
    gf.ldt = ldt;
    const void* b_tail = static_cast<const uint16_t*>(b) + (lb == KC ? nf * ldb : nf);
    GemmArgs gt = gemm_args(a, lda, b_tail, ldb, M, nt, K, p, part, nt);
    hipError_t e = timed(
        kind, s,
        [&] {
          hipError_t r = launch_gemm(p.tile, la, lb, epi, gf, 1, s);
          return r != hipSuccess ? r : launch_gemm(p.tile, la, lb, EPI_F32, gt, p.splits, s);
        },
        2);
    if (e != hipSuccess) return e;
    const size_t esz = (epi == EPI_F32 || epi == EPI_F32_ACC) ? 4 : 2;
    void* out_tail = static_cast<char*>(out) + nf * esz;
    uint16_t* out2_tail = out2 ? out2 + (epi == EPI_DGELU ? nf * ldt : nf) : nullptr;
    const uint16_t* aux_tail = aux ? aux + nf : nullptr;
    return timed(TPMLP_K_SPLITK_REDUCE, s, [&] {
      return launch_splitk_epilogue(epi, part, p.splits, M, nt, out_tail, out2_tail, aux_tail, ldo, ldt, s);
    });
  }
  GemmArgs g = gemm_args(a, lda, b, ldb, M, N, K, p, part, N);
  hipError_t e = timed(kind, s, [&] { return launch_gemm(p.tile, la, lb, EPI_F32, g, p.splits, s); });
  if (e != hipSuccess) return e;
  return timed(TPMLP_K_SPLITK_REDUCE, s,
               [&] { return launch_splitk_epilogue(epi, part, p.splits, M, N, out, out2, aux, ldo, ldt, s); });
}

// g products of one plan (unsplit) in one launch: product j's A operand a[j],
// B operand b[j] and outputs out[j], out2[j] (nullable array), aux[j]
// (nullable); ldo is the outputs' row stride (0: N).
hipError_t run_gemm_batch(int kind, Layout lb, Epi epi, const void* const* a, int64_t lda, const void* const* b,
                          int64_t ldb, int64_t M, int64_t N, int64_t K, const GemmPlan& p, int g, void* const* out,
                          uint16_t* const* out2, const uint16_t* const* aux, hipStream_t s, int64_t ldo = 0) {
  if (g < 1 || g > MAX_BATCH || p.splits != 1) return hipErrorInvalidValue;
  GemmArgs ga = gemm_args(a[0], lda, b[0], ldb, M, N, K, p, out[0], ldo ? ldo : N);
  ga.ldt = M;
  ga.batch = g;
  for (int j = 0; j < g; ++j) {
    ga.a_arr[j] = static_cast<const uint16_t*>(a[j]);
    ga.b_arr[j] = static_cast<const uint16_t*>(b[j]);
    ga.out_arr[j] = out[j];
    ga.out2_arr[j] = out2 ? out2[j] : nullptr;
    ga.aux_arr[j] = aux ? aux[j] : nullptr;
  }
  ga.out2 = ga.out2_arr[0];
  ga.aux = ga.aux_arr[0];
  return timed(kind, s, [&] { return launch_gemm(p.tile, KC, lb, epi, ga, 1, s); });
}

// Whether two products of this plan and K can share a paired launch: unsplit
// whole tiles, a tile with registers for two accumulator sets (256 x 128 or
// 128 x 128), and at least the prefetch distance in K steps in each product.
bool pair_ok(const GemmPlan& p, int64_t K) {
  return p.splits == 1 && p.n_full == 0 && p.tile != TILE_256x256 &&
         K >= (p.tile == TILE_128x128 ? 4 : 2) * TILE_BK;
}

// Two products of one shape added into the float32 [M][N] `out` in one launch:
// out = (out + a0 b0) + a1 b1 with acc, else a0 b0 + a1 b1, rounded as two
// launches of EPI_F32_ACC (or EPI_F32) and EPI_F32_ACC in that order would.
hipError_t run_gemm_pair(int kind, Layout lb, bool acc, const void* a0, const void* a1, int64_t lda, const void* b0,
                         const void* b1, int64_t ldb, int64_t M, int64_t N, int64_t K, const GemmPlan& p, float* out,
                         hipStream_t s) {
  if (!pair_ok(p, K)) return hipErrorInvalidValue;
  GemmArgs ga = gemm_args(a0, lda, b0, ldb, M, N, K, p, out, N);
  ga.a_arr[0] = static_cast<const uint16_t*>(a0);
  ga.a_arr[1] = static_cast<const uint16_t*>(a1);
  ga.b_arr[0] = static_cast<const uint16_t*>(b0);
  ga.b_arr[1] = static_cast<const uint16_t*>(b1);
  return timed(kind, s,
               [&] { return launch_gemm(p.tile, KC, lb, acc ? EPI_F32_ACC_PAIR : EPI_F32_PAIR, ga, 1, s); });
}

char* ws_at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// Enqueue rank i's forward (arguments already checked).
// A (A_i) has rows of lda >= F elements: a column block of a wider weight.
// acc: Z already holds the sum of earlier shards' partials and this shard's is
// added to it (Z = Z + Z_i, in float32) instead of overwriting it.
// weights_ready: A_i^T and B_i^T are already in the workspace (an earlier call
// for the same shard and plan made them).
hipError_t enqueue_fwd(const tpmlp_bf16* X, const tpmlp_bf16* A, int64_t lda, const tpmlp_bf16* B, float* Z,
                       tpmlp_bf16* P_save, int64_t M, int64_t H, int64_t F, void* ws, hipStream_t s,
                       bool acc = false, bool weights_ready = false) {
  const FwdPlan p = plan_fwd(M, H, F);
  const Epi out_epi = acc ? EPI_F32_ACC : EPI_F32;
  uint16_t* G = reinterpret_cast<uint16_t*>(ws_at(ws, p.off_G));
  float* part = reinterpret_cast<float*>(ws_at(ws, p.off_part));
  hipError_t e;
  if (p.fused) {
    // Z_i = GeLU(X A_i) B_i per chunk of 64 intermediate columns, G in LDS;
    // a single chunk writes Z_i itself, more are added in chunk order.
    const int chunks = ffn_chunks(F);
    FfnArgs fa{};
    fa.x = X;
    fa.a = A;
    fa.b = B;
    const bool direct = chunks == 1 && !acc;
    fa.part = direct ? Z : part;
    fa.p_save = P_save;
    fa.lda = lda;
    fa.ldp = F;
    fa.M = (int)M;
    fa.H = (int)H;
    fa.F = (int)F;
    e = timed(TPMLP_K_FWD_FUSED, s, [&] { return launch_ffn_fwd(fa, s); });
    if (e != hipSuccess || direct) return e;
    return timed(TPMLP_K_SPLITK_REDUCE, s, [&] {
      return launch_splitk_epilogue(out_epi, part, chunks, M, H, Z, nullptr, nullptr, H, M, s);
    });
  }
  if (p.wt) {
    uint16_t* At = reinterpret_cast<uint16_t*>(ws_at(ws, p.off_At));
    uint16_t* Bt = reinterpret_cast<uint16_t*>(ws_at(ws, p.off_Bt));
    if (!weights_ready && H == F && lda == H) {  // A_i and B_i of one shape: one launch
      e = timed(TPMLP_K_TRANSPOSE, s, [&] { return launch_transpose2(A, At, B, Bt, H, F, H, s); });
      if (e != hipSuccess) return e;
    } else if (!weights_ready) {
      e = timed(TPMLP_K_TRANSPOSE, s, [&] { return launch_transpose(A, H, F, lda, At, s); });
      if (e != hipSuccess) return e;
      e = timed(TPMLP_K_TRANSPOSE, s, [&] { return launch_transpose(B, F, H, H, Bt, s); });
      if (e != hipSuccess) return e;
    }
    // P_i = X A_i; G_i = GeLU(P_i)      X: [M][H], A_i^T: [F][H] (both K-contig)
    e = run_gemm(TPMLP_K_FWD_GEMM1_GELU, KC, KC, EPI_GELU, X, H, At, H, M, F, H, p.g1, G, P_save,
                 nullptr, part, s);
    if (e != hipSuccess) return e;
    // Z_i = G_i B_i                    G_i: [M][F], B_i^T: [H][F] (both K-contig)
    return run_gemm(TPMLP_K_FWD_GEMM2, KC, KC, out_epi, G, F, Bt, F, M, H, F, p.g2, Z, nullptr, nullptr,
                    part, s);
  }
  // P_i = X A_i; G_i = GeLU(P_i)        X: [M][H] (K-contig), A_i: [H][F] (N-contig)
  e = run_gemm(TPMLP_K_FWD_GEMM1_GELU, KC, MC, EPI_GELU, X, H, A, lda, M, F, H, p.g1, G, P_save, nullptr,
               part, s);
  if (e != hipSuccess) return e;
  // Z_i = G_i B_i                      G_i: [M][F] (K-contig), B_i: [F][H] (N-contig)
  return run_gemm(TPMLP_K_FWD_GEMM2, KC, MC, out_epi, G, F, B, H, M, H, F, p.g2, Z, nullptr, nullptr,
                  part, s);
}

// Enqueue rank i's backward (arguments already checked).
// X^T and dZ^T [H][M] into the backward workspace (shared by all shards), in
// one launch.
// The drivers fold the rank-order sum of the shards' partials into the
// products that make them when no per-shard partial is asked for: shard 0's
// row-parallel product (forward) or input-gradient product (backward) writes
// the output, and shard i > 0's adds its partial to it in its epilogue.  The
// additions are the float32 ones of the separate sum, in the same order
// (((p_0 + p_1) + p_2) + ...), so the result has the same bits, and the t
// partial buffers are neither written nor read back.
bool fold_sum(float* const* per_shard, int t, int64_t H) {
  if (t < 2 || H > ACC_MAX_LDO) return false;
  for (int i = 0; per_shard && i < t; ++i)
    if (per_shard[i]) return false;
  return true;
}

hipError_t enqueue_transposes(const tpmlp_bf16* dZ, const tpmlp_bf16* X, int64_t M, int64_t H, void* ws,
                              hipStream_t s) {
  const BwdPlan p = plan_bwd(M, H, 8, false);  // the transposes' offsets do not depend on F or recompute
  uint16_t* Xt = reinterpret_cast<uint16_t*>(ws_at(ws, p.off_Xt));
  uint16_t* dZt = reinterpret_cast<uint16_t*>(ws_at(ws, p.off_dZt));
  return timed(TPMLP_K_TRANSPOSE, s, [&] { return launch_transpose2(X, Xt, dZ, dZt, M, H, H, s); });
}

hipError_t enqueue_bwd_weights_dx(const BwdPlan& p, const uint16_t* dP, const uint16_t* Gt, const uint16_t* Xt,
                                  const uint16_t* dZt, const tpmlp_bf16* A, int64_t lda, float* dX, float* dA,
                                  int64_t ldda, float* dB, int64_t M, int64_t H, int64_t F, void* ws, hipStream_t s,
                                  bool acc, bool do_db = true, bool do_da = true, bool do_dx = true);

// Enqueue rank i's backward (arguments already checked; X^T and dZ^T already
// in the workspace).
// A (A_i) has rows of lda >= F elements and dA (dA_i) rows of ldda >= F.
// acc: this shard's partial input gradient is added to dX (dX = dX + dX_i).
hipError_t enqueue_bwd(const tpmlp_bf16* dZ, const tpmlp_bf16* X, const tpmlp_bf16* A, int64_t lda,
                       const tpmlp_bf16* B, const tpmlp_bf16* P_saved, float* dX, float* dA, int64_t ldda,
                       float* dB, int64_t M, int64_t H, int64_t F, void* ws, hipStream_t s, bool acc = false) {
  const bool recompute = P_saved == nullptr;
  const BwdPlan p = plan_bwd(M, H, F, recompute);
  const uint16_t* Xt = reinterpret_cast<const uint16_t*>(ws_at(ws, p.off_Xt));
  const uint16_t* dZt = reinterpret_cast<const uint16_t*>(ws_at(ws, p.off_dZt));
  uint16_t* Gt = reinterpret_cast<uint16_t*>(ws_at(ws, p.off_Gt));
  uint16_t* dP = reinterpret_cast<uint16_t*>(ws_at(ws, p.off_dP));
  float* part = reinterpret_cast<float*>(ws_at(ws, p.off_part));
  const uint16_t* P = P_saved;
  hipError_t e;
  if (recompute) {
    // P_i = X A_i again, kept as bf16 like a saved pre-activation
    uint16_t* Pw = reinterpret_cast<uint16_t*>(ws_at(ws, p.off_P));
    if (p.wt) {
      uint16_t* At = reinterpret_cast<uint16_t*>(ws_at(ws, p.off_At));
      e = timed(TPMLP_K_TRANSPOSE, s, [&] { return launch_transpose(A, H, F, lda, At, s); });
      if (e != hipSuccess) return e;
      e = run_gemm(TPMLP_K_BWD_RECOMPUTE, KC, KC, EPI_BF16, X, H, At, H, M, F, H, p.g0, Pw, nullptr, nullptr,
                   part, s);
    } else {
      e = run_gemm(TPMLP_K_BWD_RECOMPUTE, KC, MC, EPI_BF16, X, H, A, lda, M, F, H, p.g0, Pw, nullptr, nullptr,
                   part, s);
    }
    if (e != hipSuccess) return e;
    P = Pw;
  }
  // dG_i = dZ B_i^T; dP_i = dG_i GeLU'(P_i) -> dP_i [M][F]; G_i^T = GeLU(P_i)^T [F][M]
  //   dZ: [M][H] (K-contig), B_i: [F][H] = [N][K] (K-contig)
  e = run_gemm(TPMLP_K_BWD_DGELU, KC, KC, EPI_DGELU, dZ, H, B, H, M, F, H, p.g1, dP, Gt, P, part, s);
  if (e != hipSuccess) return e;
  return enqueue_bwd_weights_dx(p, dP, Gt, Xt, dZt, A, lda, dX, dA, ldda, dB, M, H, F, ws, s, acc);
}

// The rest of rank i's backward once dP_i and G_i^T exist: dB_i, dA_i (unless
// a batched launch made them) and dX_i.
hipError_t enqueue_bwd_weights_dx(const BwdPlan& p, const uint16_t* dP, const uint16_t* Gt, const uint16_t* Xt,
                                  const uint16_t* dZt, const tpmlp_bf16* A, int64_t lda, float* dX, float* dA,
                                  int64_t ldda, float* dB, int64_t M, int64_t H, int64_t F, void* ws, hipStream_t s,
                                  bool acc, bool do_db, bool do_da, bool do_dx) {
  float* part = reinterpret_cast<float*>(ws_at(ws, p.off_part));
  hipError_t e = hipSuccess;
  // With M = F_i (and A_i's rows F_i long), dB_i and dX_i are one shape: [F_i or M] x H
  // over K = M = F_i, both operands K-contiguous with row stride M.  Without a
  // running sum to add, they run as one batched launch when the planner's model
  // gives the pair at least 10% less time (short-K shapes: the launch, the ramp and
  // the last tiles' epilogue are paid once).
  if (do_db && do_dx && !acc && M == F && lda == F) {
    const BatchPlan bp = plan_batch(F, H, M, 2);
    if (bp.g == 2) {
      const void* a2[2] = {Gt, dP};
      const void* b2[2] = {dZt, A};
      void* o2[2] = {dB, dX};
      e = run_gemm_batch(TPMLP_K_BWD_DB_DX, KC, EPI_F32, a2, M, b2, M, F, H, M, bp.plan, 2, o2, nullptr, nullptr, s);
      if (e != hipSuccess) return e;
      do_db = do_dx = false;
    }
  }
  // dB_i = G_i^T dZ    G_i^T: [F][M] = [M'][K], dZ^T: [H][M] = [N'][K] (both K-contig)
  if (do_db)
    e = run_gemm(TPMLP_K_BWD_DB, KC, KC, EPI_F32, Gt, M, dZt, M, F, H, M, p.gdb, dB, nullptr, nullptr, part, s);
  if (e != hipSuccess) return e;
  if (!do_da) {
  } else if (p.tdp) {
    uint16_t* dPt = reinterpret_cast<uint16_t*>(ws_at(ws, p.off_dPt));
    e = timed(TPMLP_K_TRANSPOSE, s, [&] { return launch_transpose(dP, M, F, F, dPt, s); });
    if (e != hipSuccess) return e;
    // dA_i = X^T dP_i  X^T: [H][M] = [M'][K], dP_i^T: [F][M] = [N'][K] (both K-contig)
    e = run_gemm(TPMLP_K_BWD_DA, KC, KC, EPI_F32, Xt, M, dPt, M, H, F, M, p.gda, dA, nullptr, nullptr, part, s,
                 ldda);
  } else {
    // dA_i = X^T dP_i  X^T: [H][M] = [M'][K] (K-contig), dP_i: [M][F] = [K][N'] (N'-contig)
    e = run_gemm(TPMLP_K_BWD_DA, KC, MC, EPI_F32, Xt, M, dP, F, H, F, M, p.gda, dA, nullptr, nullptr, part, s,
                 ldda);
  }
  if (e != hipSuccess || !do_dx) return e;
  // dX_i = dP_i A_i^T  dP_i: [M][F] (K-contig), A_i: [H][F] = [N][K] (K-contig)
  return run_gemm(TPMLP_K_BWD_DX, KC, KC, acc ? EPI_F32_ACC : EPI_F32, dP, F, A, lda, M, H, F, p.gdx, dX,
                  nullptr, nullptr, part, s);
}

// Device address of `scratch` on the current device, looked up once per device.
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;

tpmlp_status noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TPMLP_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(TPMLP_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TPMLP_OK;
}

// ---------------------------------------------------------------------------
// Sequence-parallel boundary (one GPU): every rank's tokens arrive as its own
// row slice [M/t, H], and every rank's output and input gradient leave as its
// own row slice.  The products whose rows are tokens run once per rank row
// block, reading that rank's X or dZ slice and writing that rank's Z or dX slice
// (the rank-order sum folded into the epilogues), so the gathered X and dZ and
// the t per-shard partials are never materialised; the weight-gradient products
// contract over all tokens and read X^T and dZ^T, which the transpose assembles
// column block by column block from the slices.
// ---------------------------------------------------------------------------
struct SpBwdLayout {
  int64_t S;               // rows per rank
  GemmPlan g0, g1, gdx;    // recompute, dGeLU and dX products, per row block (S rows)
  GemmPlan gdb, gda;       // weight-gradient products over all M tokens
  bool wt;                 // the recompute reads A_i^T
  bool tdp;                // dA reads dP_i^T
  size_t off_Xt, off_dZt, off_At, off_P, off_Gt, off_dP, off_dPt, off_part, total;
};

SpBwdLayout sp_bwd_layout(int t, int64_t M, int64_t H, int64_t F, bool recompute) {
  SpBwdLayout L;
  L.S = M / t;
  L.g0 = plan_gemm(L.S, F, H);
  L.g1 = plan_gemm(L.S, F, H);
  L.gdx = plan_gemm(L.S, H, F);
  L.gdb = plan_gemm(F, H, M);
  L.gda = plan_gemm(H, F, M);
  const size_t mf = align_up(size_t(M) * F * 2), mh = align_up(size_t(M) * H * 2);
  L.wt = recompute && transpose_weights(L.S, H, F);
  L.tdp = transpose_dp(M, H, F);
  L.off_Xt = 0;
  L.off_dZt = mh;
  L.off_At = 2 * mh;
  L.off_P = L.off_At + (L.wt ? align_up(size_t(H) * F * 2) : 0);
  L.off_Gt = L.off_P + (recompute ? mf : 0);
  L.off_dP = L.off_Gt + mf;
  L.off_dPt = L.off_dP + mf;
  L.off_part = L.off_dPt + (L.tdp ? mf : 0);
  size_t part = recompute ? part_bytes(L.g0, L.S, F) : 0;
  part = std::max({part, part_bytes(L.g1, L.S, F), part_bytes(L.gdb, F, H), part_bytes(L.gda, H, F),
                   part_bytes(L.gdx, L.S, H)});
  L.total = L.off_part + align_up(part);
  return L;
}

size_t sp_ws_bytes(int t, int64_t M, int64_t H, int64_t F) {
  return align_up(std::max({plan_fwd(M / t, H, F).total, sp_bwd_layout(t, M, H, F, true).total,
                            sp_bwd_layout(t, M, H, F, false).total}));
}

// X^T and dZ^T [H][M] from the ranks' slices: slice r fills columns [r S, (r+1) S);
// one launch per rank takes both.
hipError_t enqueue_sp_transposes(const tpmlp_bf16* const* dZ_sl, const tpmlp_bf16* const* X_sl, int t, int64_t M,
                                 int64_t H, void* ws, hipStream_t s) {
  const SpBwdLayout L = sp_bwd_layout(t, M, H, 8, false);  // the transposes' offsets depend on M and H only
  uint16_t* Xt = reinterpret_cast<uint16_t*>(ws_at(ws, L.off_Xt));
  uint16_t* dZt = reinterpret_cast<uint16_t*>(ws_at(ws, L.off_dZt));
  for (int r = 0; r < t; ++r) {
    const hipError_t e = timed(TPMLP_K_TRANSPOSE, s, [&] {
      return launch_transpose2(X_sl[r], Xt + r * L.S, dZ_sl[r], dZt + r * L.S, L.S, H, H, s, M);
    });
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Shard i's backward over the ranks' slices (arguments checked, transposes made).
// acc: add this shard's partial input gradient to the dX slices.
hipError_t enqueue_bwd_sp(const tpmlp_bf16* const* dZ_sl, const tpmlp_bf16* const* X_sl, const tpmlp_bf16* A,
                          const tpmlp_bf16* B, const tpmlp_bf16* P_saved, float* const* dX_sl, float* dA, float* dB,
                          int t, int64_t M, int64_t H, int64_t F, void* ws, hipStream_t s, bool acc) {
  const bool recompute = P_saved == nullptr;
  const SpBwdLayout L = sp_bwd_layout(t, M, H, F, recompute);
  const int64_t S = L.S;
  const uint16_t* Xt = reinterpret_cast<const uint16_t*>(ws_at(ws, L.off_Xt));
  const uint16_t* dZt = reinterpret_cast<const uint16_t*>(ws_at(ws, L.off_dZt));
  uint16_t* Gt = reinterpret_cast<uint16_t*>(ws_at(ws, L.off_Gt));
  uint16_t* dP = reinterpret_cast<uint16_t*>(ws_at(ws, L.off_dP));
  float* part = reinterpret_cast<float*>(ws_at(ws, L.off_part));
  const uint16_t* P = P_saved;
  hipError_t e;
  if (recompute) {
    // P_i = X A_i again, one rank row block at a time
    uint16_t* Pw = reinterpret_cast<uint16_t*>(ws_at(ws, L.off_P));
    uint16_t* At = reinterpret_cast<uint16_t*>(ws_at(ws, L.off_At));
    if (L.wt) {
      e = timed(TPMLP_K_TRANSPOSE, s, [&] { return launch_transpose(A, H, F, F, At, s); });
      if (e != hipSuccess) return e;
    }
    for (int r = 0; r < t; ++r) {
      e = L.wt ? run_gemm(TPMLP_K_BWD_RECOMPUTE, KC, KC, EPI_BF16, X_sl[r], H, At, H, S, F, H, L.g0, Pw + r * S * F,
                          nullptr, nullptr, part, s)
               : run_gemm(TPMLP_K_BWD_RECOMPUTE, KC, MC, EPI_BF16, X_sl[r], H, A, F, S, F, H, L.g0, Pw + r * S * F,
                          nullptr, nullptr, part, s);
      if (e != hipSuccess) return e;
    }
    P = Pw;
  }
  // dG_i = dZ B_i^T and the dGeLU epilogue, per rank row block: dP_i rows and
  // G_i^T columns of that block (G_i^T rows of M elements)
  for (int r = 0; r < t; ++r) {
    e = run_gemm(TPMLP_K_BWD_DGELU, KC, KC, EPI_DGELU, dZ_sl[r], H, B, H, S, F, H, L.g1, dP + r * S * F, Gt + r * S,
                 P + r * S * F, part, s, 0, M);
    if (e != hipSuccess) return e;
  }
  // dB_i = G_i^T dZ and dA_i = X^T dP_i over all tokens
  e = run_gemm(TPMLP_K_BWD_DB, KC, KC, EPI_F32, Gt, M, dZt, M, F, H, M, L.gdb, dB, nullptr, nullptr, part, s);
  if (e != hipSuccess) return e;
  if (L.tdp) {
    uint16_t* dPt = reinterpret_cast<uint16_t*>(ws_at(ws, L.off_dPt));
    e = timed(TPMLP_K_TRANSPOSE, s, [&] { return launch_transpose(dP, M, F, F, dPt, s); });
    if (e != hipSuccess) return e;
    e = run_gemm(TPMLP_K_BWD_DA, KC, KC, EPI_F32, Xt, M, dPt, M, H, F, M, L.gda, dA, nullptr, nullptr, part, s);
  } else {
    e = run_gemm(TPMLP_K_BWD_DA, KC, MC, EPI_F32, Xt, M, dP, F, H, F, M, L.gda, dA, nullptr, nullptr, part, s);
  }
  if (e != hipSuccess) return e;
  // dX_i = dP_i A_i^T, per rank row block, into (or added to) that rank's slice
  for (int r = 0; r < t; ++r) {
    e = run_gemm(TPMLP_K_BWD_DX, KC, KC, acc ? EPI_F32_ACC : EPI_F32, dP + r * S * F, F, A, F, S, H, F, L.gdx,
                 dX_sl[r], nullptr, nullptr, part, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Shape checks shared by the sequence-parallel entry points.
tpmlp_status check_sp_shape(int t, int64_t M, int64_t H, int64_t F) {
  tpmlp_status st = check_shape(M, H, F);
  if (st) return st;
  if (M % t || !shape_ok(M / t))
    return fail(TPMLP_ERR_SHAPE, "M must split into t row slices of a positive multiple of 8 rows");
  if (t > 1 && H > ACC_MAX_LDO) return fail(TPMLP_ERR_SHAPE, "H is above 2^22 (the folded rank sums' limit)");
  return TPMLP_OK;
}


// ---------------------------------------------------------------------------
// FP8 drivers: per-tensor scaled E4M3 / E5M2 operands (see the header).
// ---------------------------------------------------------------------------
constexpr int F8_E4M3 = 0, F8_E5M2 = 1;

bool shape16_ok(int64_t v) { return v > 0 && v <= MAX_DIM && (v % 16) == 0; }

tpmlp_status check_shape_fp8(int64_t M, int64_t H, int64_t F) {
  if (!shape16_ok(M) || !shape16_ok(H) || !shape16_ok(F))
    return fail(TPMLP_ERR_SHAPE, "M, H and F_i must be positive multiples of 16, at most 2^23");
  return TPMLP_OK;
}

// Amax slots: the forward's (X, then A_i, B_i, G_i per shard), then the
// backward's (dZ, then dP_i per shard), so that each call clears one range.
// Each slot is AMAX_SLOT_WORDS words (epilogue.h).
constexpr int SLOT_X = 0;
inline int slot_fwd(int i, int which) { return 1 + 3 * i + which; }  // which: 0 A, 1 B, 2 G
inline int slot_bwd0(int t) { return 1 + 3 * t; }                     // dZ; dP_i at slot_bwd0(t) + 1 + i
inline int n_slots(int t) { return 2 + 4 * t; }
inline uint32_t* slot_at(uint32_t* slots, int k) { return slots + size_t(k) * AMAX_SLOT_WORDS; }

// Workspace of the FP8 path.  What the forward writes and the backward reads
// stays put between the two calls: qX, qXt, the per-shard weight codes and
// qGt (shards whose P_i the forward stored).  The rest is per-call scratch.
struct Fp8Layout {
  GemmPlan g1, g2, gdg, gdb, gda, gdx;
  size_t slots, qX, qXt, qdZ, qdZt, qAt, qBt, qA, qB, P, qG, qGt, dP, qdP, qdPt, part, total;
  size_t hf, mf;  // bytes of one shard's weight codes, of one shard's G codes
  size_t qAt_i(int i) const { return qAt + size_t(i) * hf; }
  size_t qBt_i(int i) const { return qBt + size_t(i) * hf; }
  size_t qA_i(int i) const { return qA + size_t(i) * hf; }
  size_t qB_i(int i) const { return qB + size_t(i) * hf; }
  size_t qGt_i(int i) const { return qGt + size_t(i) * mf; }
};

Fp8Layout fp8_layout(int t, int64_t M, int64_t H, int64_t F) {
  Fp8Layout L;
  L.g1 = plan_gemm(M, F, H);   // P_i = X A_i (epilogue collects amax|GeLU(P_i)|)
  L.g2 = plan_gemm(M, H, F);   // Z_i = G_i B_i
  L.gdg = plan_gemm(M, F, H);  // dG_i = dZ B_i^T (epilogue collects amax|dP_i|)
  L.gdb = plan_gemm(F, H, M);
  L.gda = plan_gemm(H, F, M);
  L.gdx = plan_gemm(M, H, F);
  const size_t mh = size_t(M) * H, hf = size_t(H) * F, mf = size_t(M) * F;
  L.hf = align_up(hf);
  L.mf = align_up(mf);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  L.slots = take(size_t(n_slots(t)) * AMAX_SLOT_WORDS * 4);
  L.qX = take(mh);
  L.qXt = take(mh);
  L.qdZ = take(mh);
  L.qdZt = take(mh);
  L.qAt = take(size_t(t) * L.hf);
  L.qBt = take(size_t(t) * L.hf);
  L.qA = take(size_t(t) * L.hf);
  L.qB = take(size_t(t) * L.hf);
  L.P = take(mf * 2);
  L.qG = take(mf);
  L.qGt = take(size_t(t) * L.mf);
  L.dP = take(mf * 2);
  L.qdP = take(mf);
  L.qdPt = take(mf);
  L.part = take(std::max({part_bytes(L.g1, M, F), part_bytes(L.g2, M, H), part_bytes(L.gdg, M, F),
                          part_bytes(L.gdb, F, H), part_bytes(L.gda, H, F), part_bytes(L.gdx, M, H), size_t(1)}));
  L.total = o;
  return L;
}

hipError_t run_gemm_fp8(int kind, int fa, int fb, Epi epi, const uint8_t* a, int64_t lda, const uint8_t* b,
                        int64_t ldb, int64_t M, int64_t N, int64_t K, const GemmPlan& p, void* out,
                        const uint16_t* aux, const uint32_t* amax_a, const uint32_t* amax_b, uint32_t* amax_out,
                        bool amax_gelu, float* part, hipStream_t s) {
  auto args = [&](const uint8_t* bb, int64_t n, const GemmPlan& pl, void* o, int64_t ldo) {
    GemmArgs g = gemm_args(a, lda, bb, ldb, M, n, K, pl, o, ldo);
    // K slices of whole FP8 K steps (128 values); a slice past K adds zeros.
    g.k_split = (int)(((K + pl.splits - 1) / pl.splits + 127) / 128 * 128);
    g.aux = aux;
    g.amax_a = amax_a;
    g.amax_b = amax_b;
    g.amax_out = amax_out;
    g.amax_gelu = amax_gelu ? 1 : 0;
    return g;
  };
  if (p.splits == 1) {
    const GemmArgs g = args(b, N, p, out, N);
    return timed(kind, s, [&] { return launch_gemm_fp8(p.tile, fa, fb, epi, g, 1, s); });
  }
  // Split products: the float32 slices go to `part`; the reduction applies the
  // epilogue, collects the amax (bf16 and dGeLU outputs) and writes no G^T.
  const size_t out_elem = (epi == EPI_F32 || epi == EPI_F32_ACC) ? 4 : 2;
  if (p.n_full > 0) {  // whole-wave tiles on the first n_full columns, split tiles on the rest
    const int64_t nf = p.n_full, nt = N - nf;
    const GemmPlan pf{p.tile, 1, (int)((K + TILE_BK - 1) / TILE_BK * TILE_BK)};
    GemmArgs gf = args(b, nf, pf, out, N);
    GemmArgs gt = args(b + nf * ldb, nt, p, part, nt);
    gt.amax_out = nullptr;
    gt.aux = nullptr;
    hipError_t e = timed(
        kind, s,
        [&] {
          hipError_t r = launch_gemm_fp8(p.tile, fa, fb, epi, gf, 1, s);
          return r != hipSuccess ? r : launch_gemm_fp8(p.tile, fa, fb, EPI_F32, gt, p.splits, s);
        },
        2);
    if (e != hipSuccess) return e;
    void* out_tail = static_cast<char*>(out) + nf * out_elem;
    const uint16_t* aux_tail = aux ? aux + nf : nullptr;
    return timed(TPMLP_K_SPLITK_REDUCE, s, [&] {
      return launch_splitk_epilogue(epi, part, p.splits, M, nt, out_tail, nullptr, aux_tail, N, M, s, amax_out,
                                    amax_gelu);
    });
  }
  GemmArgs g = args(b, N, p, part, N);
  g.amax_out = nullptr;
  g.aux = nullptr;
  hipError_t e = timed(kind, s, [&] { return launch_gemm_fp8(p.tile, fa, fb, EPI_F32, g, p.splits, s); });
  if (e != hipSuccess) return e;
  return timed(TPMLP_K_SPLITK_REDUCE, s, [&] {
    return launch_splitk_epilogue(epi, part, p.splits, M, N, out, nullptr, aux, N, M, s, amax_out, amax_gelu);
  });
}

hipError_t fp8_amax(const tpmlp_bf16* in, int64_t R, int64_t C, uint32_t* slot, hipStream_t s) {
  return timed(TPMLP_K_FP8_QUANT, s, [&] { return launch_fp8_amax(in, R, C, C, slot, AMAX_SUB, s); });
}

hipError_t fp8_quant(const tpmlp_bf16* in, int64_t R, int64_t C, bool gelu, int fmt, const uint32_t* slot,
                     uint8_t* out, bool transpose, hipStream_t s) {
  return timed(TPMLP_K_FP8_QUANT, s, [&] {
    return launch_fp8_quant(in, R, C, C, gelu, fmt, slot, AMAX_SUB, out, transpose ? R : C, transpose, s);
  });
}

// Both layouts from one read: rows [R][C] into `rows`, the transpose [C][R] into `cols`.
hipError_t fp8_quant2(const tpmlp_bf16* in, int64_t R, int64_t C, bool gelu, int fmt, const uint32_t* slot,
                      uint8_t* rows, uint8_t* cols, hipStream_t s) {
  return timed(TPMLP_K_FP8_QUANT, s,
               [&] { return launch_fp8_quant(in, R, C, C, gelu, fmt, slot, AMAX_SUB, cols, R, true, s, rows, C); });
}

#define F8_TRY(x)                         \
  do {                                    \
    const hipError_t e_ = (x);            \
    if (e_ != hipSuccess) return e_;      \
  } while (0)

hipError_t enqueue_fp8_fwd(const tpmlp_bf16* X, const tpmlp_bf16* const* A_sh, const tpmlp_bf16* const* B_sh,
                           tpmlp_bf16* const* P_sh, float* Z, int t, int64_t M, int64_t H, int64_t F, void* ws,
                           hipStream_t s) {
  const Fp8Layout L = fp8_layout(t, M, H, F);
  auto q = [&](size_t off) { return reinterpret_cast<uint8_t*>(ws_at(ws, off)); };
  uint32_t* slots = reinterpret_cast<uint32_t*>(ws_at(ws, L.slots));
  float* part = reinterpret_cast<float*>(ws_at(ws, L.part));
  F8_TRY(timed(TPMLP_K_FP8_QUANT, s, [&] { return launch_fp8_zero(slots, n_slots(t) * AMAX_SLOT_WORDS, s); }));
  F8_TRY(fp8_amax(X, M, H, slot_at(slots, SLOT_X), s));
  F8_TRY(fp8_quant2(X, M, H, false, F8_E4M3, slot_at(slots, SLOT_X), q(L.qX), q(L.qXt), s));  // X, X^T
  for (int i = 0; i < t; ++i) {
    uint32_t* sA = slot_at(slots, slot_fwd(i, 0));
    uint32_t* sB = slot_at(slots, slot_fwd(i, 1));
    uint32_t* sG = slot_at(slots, slot_fwd(i, 2));
    const bool keep = P_sh && P_sh[i];
    tpmlp_bf16* P = keep ? P_sh[i] : reinterpret_cast<tpmlp_bf16*>(ws_at(ws, L.P));
    F8_TRY(fp8_amax(A_sh[i], H, F, sA, s));
    F8_TRY(fp8_quant2(A_sh[i], H, F, false, F8_E4M3, sA, q(L.qA_i(i)), q(L.qAt_i(i)), s));  // A_i, A_i^T
    F8_TRY(fp8_amax(B_sh[i], F, H, sB, s));
    F8_TRY(fp8_quant2(B_sh[i], F, H, false, F8_E4M3, sB, q(L.qB_i(i)), q(L.qBt_i(i)), s));  // B_i, B_i^T
    F8_TRY(run_gemm_fp8(TPMLP_K_FWD_GEMM1_GELU, F8_E4M3, F8_E4M3, EPI_BF16, q(L.qX), H, q(L.qAt_i(i)), H, M, F, H,
                        L.g1, P, nullptr, slot_at(slots, SLOT_X), sA, sG, true, part, s));
    if (keep)  // G_i for the second product and G_i^T for the backward's dB_i
      F8_TRY(fp8_quant2(P, M, F, true, F8_E4M3, sG, q(L.qG), q(L.qGt_i(i)), s));
    else
      F8_TRY(fp8_quant(P, M, F, true, F8_E4M3, sG, q(L.qG), false, s));
    F8_TRY(run_gemm_fp8(TPMLP_K_FWD_GEMM2, F8_E4M3, F8_E4M3, i == 0 ? EPI_F32 : EPI_F32_ACC, q(L.qG), F,
                        q(L.qBt_i(i)), F, M, H, F, L.g2, Z, nullptr, sG, sB, nullptr, false, part, s));
  }
  return hipSuccess;
}

hipError_t enqueue_fp8_bwd(const tpmlp_bf16* dZ, const tpmlp_bf16* const* P_sh, float* const* dA_sh,
                           float* const* dB_sh, float* dX, int t, int64_t M, int64_t H, int64_t F, void* ws,
                           hipStream_t s) {
  const Fp8Layout L = fp8_layout(t, M, H, F);
  auto q = [&](size_t off) { return reinterpret_cast<uint8_t*>(ws_at(ws, off)); };
  uint32_t* slots = reinterpret_cast<uint32_t*>(ws_at(ws, L.slots));
  tpmlp_bf16* dP = reinterpret_cast<tpmlp_bf16*>(ws_at(ws, L.dP));
  float* part = reinterpret_cast<float*>(ws_at(ws, L.part));
  const bool recompute = P_sh == nullptr;
  uint32_t* sdZ = slot_at(slots, slot_bwd0(t));
  F8_TRY(timed(TPMLP_K_FP8_QUANT, s, [&] { return launch_fp8_zero(sdZ, (1 + t) * AMAX_SLOT_WORDS, s); }));
  F8_TRY(fp8_amax(dZ, M, H, sdZ, s));
  F8_TRY(fp8_quant2(dZ, M, H, false, F8_E5M2, sdZ, q(L.qdZ), q(L.qdZt), s));  // dZ, dZ^T
  for (int i = 0; i < t; ++i) {
    uint32_t* sA = slot_at(slots, slot_fwd(i, 0));
    uint32_t* sB = slot_at(slots, slot_fwd(i, 1));
    uint32_t* sG = slot_at(slots, slot_fwd(i, 2));
    uint32_t* sdP = slot_at(slots, slot_bwd0(t) + 1 + i);
    const tpmlp_bf16* P;
    if (recompute) {  // the forward's product again (its codes and scales are in ws); same P_i, same amax
      tpmlp_bf16* Pw = reinterpret_cast<tpmlp_bf16*>(ws_at(ws, L.P));
      F8_TRY(run_gemm_fp8(TPMLP_K_BWD_RECOMPUTE, F8_E4M3, F8_E4M3, EPI_BF16, q(L.qX), H, q(L.qAt_i(i)), H, M, F, H,
                          L.g1, Pw, nullptr, slot_at(slots, SLOT_X), sA, sG, true, part, s));
      F8_TRY(fp8_quant(Pw, M, F, true, F8_E4M3, sG, q(L.qGt_i(i)), true, s));  // G_i^T [F][M]
      P = Pw;
    } else {
      P = P_sh[i];  // G_i^T's codes came with the forward
    }
    F8_TRY(run_gemm_fp8(TPMLP_K_BWD_DGELU, F8_E5M2, F8_E4M3, EPI_DGELU, q(L.qdZ), H, q(L.qB_i(i)), H, M, F, H, L.gdg,
                        dP, P, sdZ, sB, sdP, false, part, s));
    F8_TRY(fp8_quant2(dP, M, F, false, F8_E5M2, sdP, q(L.qdP), q(L.qdPt), s));  // dP_i, dP_i^T
    F8_TRY(run_gemm_fp8(TPMLP_K_BWD_DB, F8_E4M3, F8_E5M2, EPI_F32, q(L.qGt_i(i)), M, q(L.qdZt), M, F, H, M, L.gdb,
                        dB_sh[i], nullptr, sG, sdZ, nullptr, false, part, s));
    F8_TRY(run_gemm_fp8(TPMLP_K_BWD_DA, F8_E4M3, F8_E5M2, EPI_F32, q(L.qXt), M, q(L.qdPt), M, H, F, M, L.gda,
                        dA_sh[i], nullptr, slot_at(slots, SLOT_X), sdP, nullptr, false, part, s));
    F8_TRY(run_gemm_fp8(TPMLP_K_BWD_DX, F8_E5M2, F8_E4M3, i == 0 ? EPI_F32 : EPI_F32_ACC, q(L.qdP), F, q(L.qA_i(i)),
                        F, M, H, F, L.gdx, dX, nullptr, sdP, sA, nullptr, false, part, s));
  }
  return hipSuccess;
}

// The arguments of the last forward per workspace address, for the backward's
// check that the workspace holds the forward of its inputs.
struct Fp8Stamp {
  int t;
  int64_t M, H, F;
  int device;
  const void* X;
  std::vector<const void*> A, B, P;  // P: nullptr where the forward did not store P_i
};
std::mutex g_fp8_mu;
std::vector<std::pair<const void*, Fp8Stamp>> g_fp8_stamps;

Fp8Stamp make_stamp(const void* X, const tpmlp_bf16* const* A_sh, const tpmlp_bf16* const* B_sh,
                    const tpmlp_bf16* const* P_sh, int t, int64_t M, int64_t H, int64_t F) {
  Fp8Stamp st{t, M, H, F, -1, X, {}, {}, {}};
  (void)hipGetDevice(&st.device);
  for (int i = 0; i < t; ++i) {
    st.A.push_back(A_sh[i]);
    st.B.push_back(B_sh[i]);
    st.P.push_back(P_sh ? static_cast<const void*>(P_sh[i]) : nullptr);
  }
  return st;
}

// A forward overwrites what an earlier forward left in ws, so its stamp goes
// first, and the new one is recorded only once every launch was enqueued.
void forget_fp8_forward(const void* ws) {
  std::lock_guard<std::mutex> lk(g_fp8_mu);
  g_fp8_stamps.erase(std::remove_if(g_fp8_stamps.begin(), g_fp8_stamps.end(),
                                    [&](const std::pair<const void*, Fp8Stamp>& e) { return e.first == ws; }),
                     g_fp8_stamps.end());
}

// At most this many workspaces' forwards are remembered; the least recently
// recorded goes first (its backward then returns TPMLP_ERR_NO_FORWARD).
constexpr size_t MAX_FP8_STAMPS = 256;

void record_fp8_forward(const void* ws, Fp8Stamp st) {
  std::lock_guard<std::mutex> lk(g_fp8_mu);  // the newest record is at the back
  g_fp8_stamps.erase(std::remove_if(g_fp8_stamps.begin(), g_fp8_stamps.end(),
                                    [&](const std::pair<const void*, Fp8Stamp>& e) { return e.first == ws; }),
                     g_fp8_stamps.end());
  if (g_fp8_stamps.size() >= MAX_FP8_STAMPS) g_fp8_stamps.erase(g_fp8_stamps.begin());
  g_fp8_stamps.emplace_back(ws, std::move(st));
}

// "" when ws holds the forward of these arguments, else what differs.
std::string check_fp8_forward(const void* ws, const Fp8Stamp& want, bool store) {
  std::lock_guard<std::mutex> lk(g_fp8_mu);
  for (const auto& e : g_fp8_stamps) {
    if (e.first != ws) continue;
    const Fp8Stamp& got = e.second;
    if (got.t != want.t || got.M != want.M || got.H != want.H || got.F != want.F) return "other shapes or t";
    if (got.device != want.device) return "another device";
    if (got.X != want.X || got.A != want.A || got.B != want.B) return "other X, A_sh or B_sh";
    if (store)
      for (int i = 0; i < want.t; ++i)
        if (!got.P[i] || got.P[i] != want.P[i]) return "P_sh[" + std::to_string(i) + "] was not stored there by it";
    return "";
  }
  return "no forward on this workspace";
}
#undef F8_TRY

}  // namespace
}  // namespace tpmlp

using namespace tpmlp;

extern "C" {

int tpmlp_abi_version(void) { return TPMLP_ABI_VERSION; }

const char* tpmlp_status_str(int status) {
  switch (status) {
    case TPMLP_OK: return "ok";
    case TPMLP_ERR_NULL: return "null pointer";
    case TPMLP_ERR_SHAPE: return "invalid shape";
    case TPMLP_ERR_ALIGN: return "misaligned pointer";
    case TPMLP_ERR_WORKSPACE: return "workspace too small";
    case TPMLP_ERR_SHARDS: return "invalid shard count";
    case TPMLP_ERR_HIP: return "HIP error";
    case TPMLP_ERR_UNSUPPORTED: return "unsupported device";
    case TPMLP_ERR_ALIAS: return "output overlaps another buffer";
    case TPMLP_ERR_NO_FORWARD: return "workspace holds no forward of these inputs";
    default: return "unknown status";
  }
}

const char* tpmlp_last_error(void) { return g_last_error.c_str(); }

const char* tpmlp_kernel_name(int kind) {
  static const char* names[TPMLP_K_COUNT] = {"fwd_gemm1_gelu", "fwd_gemm2", "bwd_recompute", "bwd_dgelu",
                                             "bwd_dB", "bwd_dA", "bwd_dX", "splitk_reduce", "shard_sum", "transpose", "fwd_fused",
                                             "fp8_quant", "bwd_dB_dX"};
  return (kind >= 0 && kind < TPMLP_K_COUNT) ? names[kind] : "?";
}

size_t tpmlp_fwd_workspace_bytes(int64_t M, int64_t H, int64_t F_i) {
  if (!shape_ok(M) || !shape_ok(H) || !shape_ok(F_i)) return 0;
  return plan_fwd(M, H, F_i).total;
}

size_t tpmlp_bwd_workspace_bytes(int64_t M, int64_t H, int64_t F_i, int recompute) {
  if (!shape_ok(M) || !shape_ok(H) || !shape_ok(F_i)) return 0;
  return plan_bwd(M, H, F_i, recompute != 0).total;
}

tpmlp_status tpmlp_fwd(const tpmlp_bf16* X, const tpmlp_bf16* A_i, const tpmlp_bf16* B_i, float* Z_i,
                       tpmlp_bf16* P_save, int64_t M, int64_t H, int64_t F_i, void* ws, size_t ws_bytes,
                       void* stream) {
  g_last_error.clear();
  tpmlp_status st = check_ptrs({{X, "X"}, {A_i, "A_i"}, {B_i, "B_i"}, {Z_i, "Z_i"}, {ws, "ws"}});
  if (st) return st;
  if (P_save && !aligned16(P_save)) return fail(TPMLP_ERR_ALIGN, "P_save is not 16-byte aligned");
  if ((st = check_shape(M, H, F_i))) return st;
  const size_t need = tpmlp_fwd_workspace_bytes(M, H, F_i);
  if (ws_bytes < need) return fail(TPMLP_ERR_WORKSPACE, "ws_bytes below tpmlp_fwd_workspace_bytes");
  const size_t mh = size_t(M) * H, hf = size_t(H) * F_i, mf = size_t(M) * F_i;
  std::vector<Range> ins = {{X, mh * 2, "X"}, {A_i, hf * 2, "A_i"}, {B_i, hf * 2, "B_i"}};
  std::vector<Range> outs = {{Z_i, mh * 4, "Z_i"}, {P_save, P_save ? mf * 2 : 0, "P_save"}, {ws, need, "ws"}};
  if ((st = check_alias(outs, ins))) return st;
  if ((st = check_device())) return st;
  hipError_t e = enqueue_fwd(X, A_i, F_i, B_i, Z_i, P_save, M, H, F_i, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TPMLP_OK : hip_fail(e, "tpmlp_fwd launch");
}


tpmlp_status tpmlp_fwd_noalloc(const tpmlp_bf16* X, const tpmlp_bf16* A_i, const tpmlp_bf16* B_i,
                               float* Z_i, tpmlp_bf16* P_save, int64_t M, int64_t H, int64_t F_i,
                               void* stream) {
  g_last_error.clear();
  tpmlp_status st = check_ptrs({{X, "X"}, {A_i, "A_i"}, {B_i, "B_i"}, {Z_i, "Z_i"}});
  if (st) return st;
  if (P_save && !aligned16(P_save)) return fail(TPMLP_ERR_ALIGN, "P_save is not 16-byte aligned");
  if ((st = check_shape(M, H, F_i))) return st;
  const size_t need = tpmlp_fwd_workspace_bytes(M, H, F_i);
  if (need > TPMLP_NOALLOC_SCRATCH_BYTES)
    return fail(TPMLP_ERR_WORKSPACE, "the shape needs " + std::to_string(need) +
                                         " bytes of workspace, above TPMLP_NOALLOC_SCRATCH_BYTES");
  const size_t mh = size_t(M) * H, hf = size_t(H) * F_i, mf = size_t(M) * F_i;
  std::vector<Range> ins = {{X, mh * 2, "X"}, {A_i, hf * 2, "A_i"}, {B_i, hf * 2, "B_i"}};
  std::vector<Range> outs = {{Z_i, mh * 4, "Z_i"}, {P_save, P_save ? mf * 2 : 0, "P_save"}};
  if ((st = check_alias(outs, ins))) return st;
  if ((st = check_device())) return st;
  void* ws = nullptr;
  if ((st = noalloc_scratch(&ws))) return st;
  hipError_t e = enqueue_fwd(X, A_i, F_i, B_i, Z_i, P_save, M, H, F_i, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TPMLP_OK : hip_fail(e, "tpmlp_fwd_noalloc launch");
}

tpmlp_status tpmlp_bwd(const tpmlp_bf16* dZ, const tpmlp_bf16* X, const tpmlp_bf16* A_i, const tpmlp_bf16* B_i,
                       const tpmlp_bf16* P_saved, float* dX_i, float* dA_i, float* dB_i, int64_t M, int64_t H,
                       int64_t F_i, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  tpmlp_status st = check_ptrs({{dZ, "dZ"}, {X, "X"}, {A_i, "A_i"}, {B_i, "B_i"}, {dX_i, "dX_i"},
                                {dA_i, "dA_i"}, {dB_i, "dB_i"}, {ws, "ws"}});
  if (st) return st;
  if (P_saved && !aligned16(P_saved)) return fail(TPMLP_ERR_ALIGN, "P_saved is not 16-byte aligned");
  if ((st = check_shape(M, H, F_i))) return st;
  const size_t need = tpmlp_bwd_workspace_bytes(M, H, F_i, P_saved == nullptr);
  if (ws_bytes < need) return fail(TPMLP_ERR_WORKSPACE, "ws_bytes below tpmlp_bwd_workspace_bytes");
  const size_t mh = size_t(M) * H, hf = size_t(H) * F_i, mf = size_t(M) * F_i;
  std::vector<Range> ins = {{dZ, mh * 2, "dZ"}, {X, mh * 2, "X"}, {A_i, hf * 2, "A_i"}, {B_i, hf * 2, "B_i"},
                            {P_saved, P_saved ? mf * 2 : 0, "P_saved"}};
  std::vector<Range> outs = {{dX_i, mh * 4, "dX_i"}, {dA_i, hf * 4, "dA_i"}, {dB_i, hf * 4, "dB_i"}, {ws, need, "ws"}};
  if ((st = check_alias(outs, ins))) return st;
  if ((st = check_device())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = enqueue_transposes(dZ, X, M, H, ws, s);
  if (e == hipSuccess) e = enqueue_bwd(dZ, X, A_i, F_i, B_i, P_saved, dX_i, dA_i, F_i, dB_i, M, H, F_i, ws, s);
  return e == hipSuccess ? TPMLP_OK : hip_fail(e, "tpmlp_bwd launch");
}

size_t tpmlp_saved_activation_bytes(int64_t M, int64_t H, int64_t F_i, int recompute) {
  if (!shape_ok(M) || !shape_ok(H) || !shape_ok(F_i)) return 0;
  return size_t(M) * H * 2 + (recompute ? 0 : size_t(M) * F_i * 2);
}

int tpmlp_recompute_policy(int64_t M, int64_t H, int64_t F_i, size_t budget_bytes) {
  if (!shape_ok(M) || !shape_ok(H) || !shape_ok(F_i)) return -1;
  if (tpmlp_saved_activation_bytes(M, H, F_i, 0) <= budget_bytes) return 0;
  if (tpmlp_saved_activation_bytes(M, H, F_i, 1) <= budget_bytes) return 1;
  return -1;
}

size_t tpmlp_tp_workspace_bytes(int t, int64_t M, int64_t H, int64_t F_i) {
  if (t < 1 || t > TPMLP_MAX_SHARDS || !shape_ok(M) || !shape_ok(H) || !shape_ok(F_i)) return 0;
  return shard_ws_bytes(M, H, F_i) + align_up(size_t(t) * M * H * 4) + batch_area_bytes(t, M, H, F_i);
}

tpmlp_status tpmlp_shard_sum(const float* const* parts, int t, float* out, int64_t n, void* stream) {
  g_last_error.clear();
  if (!parts || !out) return fail(TPMLP_ERR_NULL, "parts or out is NULL");
  if (t < 1 || t > TPMLP_MAX_SHARDS) return fail(TPMLP_ERR_SHARDS, "t outside 1..TPMLP_MAX_SHARDS");
  if (n <= 0 || (n % 4)) return fail(TPMLP_ERR_SHAPE, "n must be a positive multiple of 4");
  if (!aligned16(out)) return fail(TPMLP_ERR_ALIGN, "out is not 16-byte aligned");
  std::vector<Range> ins;
  for (int i = 0; i < t; ++i) {
    if (!parts[i]) return fail(TPMLP_ERR_NULL, "parts[" + std::to_string(i) + "] is NULL");
    if (!aligned16(parts[i])) return fail(TPMLP_ERR_ALIGN, "parts[" + std::to_string(i) + "] is not 16-byte aligned");
    ins.push_back({parts[i], size_t(n) * 4, "a part"});
  }
  tpmlp_status st = check_alias({{out, size_t(n) * 4, "out"}}, ins);
  if (st) return st;
  if ((st = check_device())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed(TPMLP_K_SHARD_SUM, s, [&] { return launch_sum(parts, t, out, n, s); });
  return e == hipSuccess ? TPMLP_OK : hip_fail(e, "tpmlp_shard_sum launch");
}

tpmlp_status tpmlp_tp_fwd(const tpmlp_bf16* X, const tpmlp_bf16* const* A_sh, const tpmlp_bf16* const* B_sh,
                          tpmlp_bf16* const* P_sh, float* const* Z_sh, float* Z, int t, int64_t M, int64_t H,
                          int64_t F_i, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (!A_sh || !B_sh) return fail(TPMLP_ERR_NULL, "A_sh or B_sh is NULL");
  if (t < 1 || t > TPMLP_MAX_SHARDS) return fail(TPMLP_ERR_SHARDS, "t outside 1..TPMLP_MAX_SHARDS");
  tpmlp_status st = check_ptrs({{X, "X"}, {Z, "Z"}, {ws, "ws"}});
  if (st) return st;
  if ((st = check_shape(M, H, F_i))) return st;
  const size_t need = tpmlp_tp_workspace_bytes(t, M, H, F_i);
  if (ws_bytes < need) return fail(TPMLP_ERR_WORKSPACE, "ws_bytes below tpmlp_tp_workspace_bytes");
  const size_t mh = size_t(M) * H, hf = size_t(H) * F_i, mf = size_t(M) * F_i;
  std::vector<Range> ins = {{X, mh * 2, "X"}};
  std::vector<Range> outs = {{Z, mh * 4, "Z"}, {ws, need, "ws"}};
  for (int i = 0; i < t; ++i) {
    if (!A_sh[i] || !B_sh[i]) return fail(TPMLP_ERR_NULL, "A_sh[" + std::to_string(i) + "] or B_sh[i] is NULL");
    if (!aligned16(A_sh[i]) || !aligned16(B_sh[i])) return fail(TPMLP_ERR_ALIGN, "a weight shard is not 16-byte aligned");
    ins.push_back({A_sh[i], hf * 2, "A_sh[i]"});
    ins.push_back({B_sh[i], hf * 2, "B_sh[i]"});
    if (P_sh && P_sh[i]) {
      if (!aligned16(P_sh[i])) return fail(TPMLP_ERR_ALIGN, "P_sh[i] is not 16-byte aligned");
      outs.push_back({P_sh[i], mf * 2, "P_sh[i]"});
    }
    if (Z_sh && Z_sh[i]) {
      if (!aligned16(Z_sh[i])) return fail(TPMLP_ERR_ALIGN, "Z_sh[i] is not 16-byte aligned");
      outs.push_back({Z_sh[i], mh * 4, "Z_sh[i]"});
    }
  }
  if ((st = check_alias(outs, ins))) return st;
  if ((st = check_device())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* partials = reinterpret_cast<float*>(ws_at(ws, shard_ws_bytes(M, H, F_i)));
  const bool direct = (t == 1) && !(Z_sh && Z_sh[0]);
  const bool fold = fold_sum(Z_sh, t, H);
  const float* parts[TPMLP_MAX_SHARDS];
  float* Zs[TPMLP_MAX_SHARDS];
  for (int i = 0; i < t; ++i) {
    Zs[i] = (direct || fold) ? Z : (Z_sh && Z_sh[i]) ? Z_sh[i] : partials + size_t(i) * mh;
    parts[i] = Zs[i];
  }
  const BatchPlan bp = plan_shard_batch(t, M, H, F_i);
  if (bp.g > 1) {
    // F1 of bp.g shards per launch (G_i in the batch area), then each shard's F3.
    const FwdPlan fp = plan_fwd(M, H, F_i);
    char* area = ws_at(ws, shard_ws_bytes(M, H, F_i) + align_up(size_t(t) * mh * 4));
    float* part = reinterpret_cast<float*>(ws_at(ws, fp.off_part));
    for (int i0 = 0; i0 < t; i0 += bp.g) {
      const int g = std::min(bp.g, t - i0);
      const void* a[MAX_BATCH];
      const void* b[MAX_BATCH];
      void* G[MAX_BATCH];
      uint16_t* P[MAX_BATCH];
      for (int j = 0; j < g; ++j) {
        a[j] = X;
        b[j] = A_sh[i0 + j];
        G[j] = area + size_t(j) * batch_slot_bytes(M, F_i);
        P[j] = P_sh ? P_sh[i0 + j] : nullptr;
      }
      // P_i = X A_i; G_i = GeLU(P_i)      X: [M][H] (K-contig), A_i: [H][F] (N-contig)
      hipError_t e = run_gemm_batch(TPMLP_K_FWD_GEMM1_GELU, MC, EPI_GELU, a, H, b, F_i, M, F_i, H, bp.plan, g, G, P,
                                    nullptr, s);
      // Z_i = G_i B_i                    G_i: [M][F] (K-contig), B_i: [F][H] (N-contig)
      // Folded into one Z, two consecutive shards' products share a launch when
      // their plan allows it (rank order kept: Z + Z_i, then + Z_{i+1}).
      const bool pairs = fold && pair_ok(fp.g2, F_i);
      for (int j = 0; j < g && e == hipSuccess;) {
        const int i = i0 + j;
        if (pairs && j + 1 < g) {
          e = run_gemm_pair(TPMLP_K_FWD_GEMM2, MC, i > 0, G[j], G[j + 1], F_i, B_sh[i], B_sh[i + 1], H, M, H, F_i,
                            fp.g2, Z, s);
          j += 2;
        } else {
          e = run_gemm(TPMLP_K_FWD_GEMM2, KC, MC, fold && i > 0 ? EPI_F32_ACC : EPI_F32, G[j], F_i, B_sh[i], H, M,
                       H, F_i, fp.g2, Zs[i], nullptr, nullptr, part, s);
          j += 1;
        }
      }
      if (e != hipSuccess) return hip_fail(e, "tpmlp_tp_fwd launch");
    }
  } else {
    for (int i = 0; i < t; ++i) {
      hipError_t e =
          enqueue_fwd(X, A_sh[i], F_i, B_sh[i], Zs[i], P_sh ? P_sh[i] : nullptr, M, H, F_i, ws, s, fold && i > 0);
      if (e != hipSuccess) return hip_fail(e, "tpmlp_tp_fwd launch");
    }
  }
  if (!direct && !fold) {
    hipError_t e = timed(TPMLP_K_SHARD_SUM, s, [&] { return launch_sum(parts, t, Z, int64_t(mh), s); });
    if (e != hipSuccess) return hip_fail(e, "tpmlp_tp_fwd sum");
  }
  return TPMLP_OK;
}

tpmlp_status tpmlp_tp_bwd(const tpmlp_bf16* dZ, const tpmlp_bf16* X, const tpmlp_bf16* const* A_sh,
                          const tpmlp_bf16* const* B_sh, const tpmlp_bf16* const* P_sh, float* const* dA_sh,
                          float* const* dB_sh, float* const* dX_sh, float* dX, int t, int64_t M, int64_t H,
                          int64_t F_i, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (!A_sh || !B_sh || !dA_sh || !dB_sh) return fail(TPMLP_ERR_NULL, "a shard array is NULL");
  if (t < 1 || t > TPMLP_MAX_SHARDS) return fail(TPMLP_ERR_SHARDS, "t outside 1..TPMLP_MAX_SHARDS");
  tpmlp_status st = check_ptrs({{dZ, "dZ"}, {X, "X"}, {dX, "dX"}, {ws, "ws"}});
  if (st) return st;
  if ((st = check_shape(M, H, F_i))) return st;
  const size_t need = tpmlp_tp_workspace_bytes(t, M, H, F_i);
  if (ws_bytes < need) return fail(TPMLP_ERR_WORKSPACE, "ws_bytes below tpmlp_tp_workspace_bytes");
  const size_t mh = size_t(M) * H, hf = size_t(H) * F_i, mf = size_t(M) * F_i;
  std::vector<Range> ins = {{dZ, mh * 2, "dZ"}, {X, mh * 2, "X"}};
  std::vector<Range> outs = {{dX, mh * 4, "dX"}, {ws, need, "ws"}};
  for (int i = 0; i < t; ++i) {
    const std::string idx = "[" + std::to_string(i) + "]";
    if (!A_sh[i] || !B_sh[i] || !dA_sh[i] || !dB_sh[i]) return fail(TPMLP_ERR_NULL, "a shard pointer" + idx + " is NULL");
    if (P_sh && !P_sh[i]) return fail(TPMLP_ERR_NULL, "P_sh" + idx + " is NULL");
    for (const void* p : {(const void*)A_sh[i], (const void*)B_sh[i], (const void*)dA_sh[i], (const void*)dB_sh[i]})
      if (!aligned16(p)) return fail(TPMLP_ERR_ALIGN, "a shard pointer" + idx + " is not 16-byte aligned");
    if (P_sh && !aligned16(P_sh[i])) return fail(TPMLP_ERR_ALIGN, "P_sh" + idx + " is not 16-byte aligned");
    ins.push_back({A_sh[i], hf * 2, "A_sh[i]"});
    ins.push_back({B_sh[i], hf * 2, "B_sh[i]"});
    if (P_sh) ins.push_back({P_sh[i], mf * 2, "P_sh[i]"});
    outs.push_back({dA_sh[i], hf * 4, "dA_sh[i]"});
    outs.push_back({dB_sh[i], hf * 4, "dB_sh[i]"});
    if (dX_sh && dX_sh[i]) {
      if (!aligned16(dX_sh[i])) return fail(TPMLP_ERR_ALIGN, "dX_sh" + idx + " is not 16-byte aligned");
      outs.push_back({dX_sh[i], mh * 4, "dX_sh[i]"});
    }
  }
  if ((st = check_alias(outs, ins))) return st;
  if ((st = check_device())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* partials = reinterpret_cast<float*>(ws_at(ws, shard_ws_bytes(M, H, F_i)));
  const bool direct = (t == 1) && !(dX_sh && dX_sh[0]);
  const bool fold = fold_sum(dX_sh, t, H);
  const float* parts[TPMLP_MAX_SHARDS];
  hipError_t et = enqueue_transposes(dZ, X, M, H, ws, s);
  if (et != hipSuccess) return hip_fail(et, "tpmlp_tp_bwd transpose");
  float* dXs[TPMLP_MAX_SHARDS];
  for (int i = 0; i < t; ++i) {
    dXs[i] = (direct || fold) ? dX : (dX_sh && dX_sh[i]) ? dX_sh[i] : partials + size_t(i) * mh;
    parts[i] = dXs[i];
  }
  const BatchPlan bp = plan_shard_batch(t, M, H, F_i);
  if (bp.g > 1) {
    // The recompute and dGeLU of bp.g shards per launch (P_i, G_i^T and dP_i in
    // the batch area), then each shard's dB_i, dA_i and dX_i.
    const bool recompute = P_sh == nullptr;
    const BwdPlan p = plan_bwd(M, H, F_i, recompute);
    const uint16_t* Xt = reinterpret_cast<const uint16_t*>(ws_at(ws, p.off_Xt));
    const uint16_t* dZt = reinterpret_cast<const uint16_t*>(ws_at(ws, p.off_dZt));
    char* area = ws_at(ws, shard_ws_bytes(M, H, F_i) + align_up(size_t(t) * mh * 4));
    const size_t mfa = align_up(mf * 2);
    for (int i0 = 0; i0 < t; i0 += bp.g) {
      const int g = std::min(bp.g, t - i0);
      const void* xs[MAX_BATCH];
      const void* dzs[MAX_BATCH];
      const void* a_w[MAX_BATCH];
      const void* b_w[MAX_BATCH];
      void* Pw[MAX_BATCH];
      const uint16_t* P[MAX_BATCH];
      void* dPs[MAX_BATCH];
      uint16_t* Gts[MAX_BATCH];
      for (int j = 0; j < g; ++j) {
        char* slot = area + size_t(j) * batch_slot_bytes(M, F_i);
        xs[j] = X;
        dzs[j] = dZ;
        a_w[j] = A_sh[i0 + j];
        b_w[j] = B_sh[i0 + j];
        Pw[j] = slot;
        P[j] = recompute ? reinterpret_cast<const uint16_t*>(slot) : P_sh[i0 + j];
        Gts[j] = reinterpret_cast<uint16_t*>(slot + mfa);
        dPs[j] = slot + 2 * mfa;
      }
      hipError_t e = hipSuccess;
      if (recompute)  // P_i = X A_i again   X: [M][H] (K-contig), A_i: [H][F] (N-contig)
        e = run_gemm_batch(TPMLP_K_BWD_RECOMPUTE, MC, EPI_BF16, xs, H, a_w, F_i, M, F_i, H, bp.plan, g, Pw, nullptr,
                           nullptr, s);
      // dG_i = dZ B_i^T; dP_i = dG_i GeLU'(P_i); G_i^T    dZ: [M][H], B_i: [F][H] (both K-contig)
      if (e == hipSuccess)
        e = run_gemm_batch(TPMLP_K_BWD_DGELU, KC, EPI_DGELU, dzs, H, b_w, H, M, F_i, H, bp.plan, g, dPs, Gts, P, s);
      // dB_i and dA_i (no cross-shard sum) in batches of their own size where that
      // pays, else one launch per shard; then each shard's dX_i.
      const BatchPlan bdb = plan_batch(F_i, H, M, g), bda = plan_batch(H, F_i, M, g);
      const void* dzt[MAX_BATCH];
      const void* xt[MAX_BATCH];
      for (int j = 0; j < g; ++j) {
        dzt[j] = dZt;
        xt[j] = Xt;
      }
      float* const* dBs = dB_sh + i0;
      float* const* dAs = dA_sh + i0;
      for (int j0 = 0; bdb.g > 1 && j0 < g && e == hipSuccess; j0 += bdb.g) {
        // dB_i = G_i^T dZ    G_i^T: [F][M], dZ^T: [H][M] (both K-contig)
        const int gb = std::min(bdb.g, g - j0);
        e = run_gemm_batch(TPMLP_K_BWD_DB, KC, EPI_F32, reinterpret_cast<const void* const*>(Gts + j0), M,
                           dzt + j0, M, F_i, H, M, bdb.plan, gb, reinterpret_cast<void* const*>(dBs + j0), nullptr,
                           nullptr, s);
      }
      const bool batch_da = bda.g > 1 && !p.tdp;
      for (int j0 = 0; batch_da && j0 < g && e == hipSuccess; j0 += bda.g) {
        // dA_i = X^T dP_i    X^T: [H][M] (K-contig), dP_i: [M][F] (N-contig)
        const int ga = std::min(bda.g, g - j0);
        e = run_gemm_batch(TPMLP_K_BWD_DA, MC, EPI_F32, xt + j0, M, const_cast<const void* const*>(dPs + j0), F_i,
                           H, F_i, M, bda.plan, ga, reinterpret_cast<void* const*>(dAs + j0), nullptr, nullptr, s);
      }
      // Folded into one dX, two consecutive shards' dX products share a launch when
      // their plan allows it (rank order kept), after both shards' dB and dA.
      const bool pairs = fold && pair_ok(p.gdx, F_i);
      for (int j = 0; j < g && e == hipSuccess;) {
        const int i = i0 + j;
        const bool pair = pairs && j + 1 < g;
        for (int u = 0; u < (pair ? 2 : 1) && e == hipSuccess; ++u)
          e = enqueue_bwd_weights_dx(p, static_cast<const uint16_t*>(dPs[j + u]), Gts[j + u], Xt, dZt, A_sh[i + u],
                                     F_i, dXs[i + u], dA_sh[i + u], F_i, dB_sh[i + u], M, H, F_i, ws, s,
                                     fold && i + u > 0, bdb.g == 1, !batch_da, !pair);
        // dX_i = dP_i A_i^T  dP_i: [M][F] (K-contig), A_i: [H][F] = [N][K] (K-contig)
        if (pair && e == hipSuccess)
          e = run_gemm_pair(TPMLP_K_BWD_DX, KC, i > 0, dPs[j], dPs[j + 1], F_i, A_sh[i], A_sh[i + 1], F_i, M, H, F_i,
                            p.gdx, dX, s);
        j += pair ? 2 : 1;
      }
      if (e != hipSuccess) return hip_fail(e, "tpmlp_tp_bwd launch");
    }
  } else {
    for (int i = 0; i < t; ++i) {
      hipError_t e = enqueue_bwd(dZ, X, A_sh[i], F_i, B_sh[i], P_sh ? P_sh[i] : nullptr, dXs[i], dA_sh[i], F_i,
                                 dB_sh[i], M, H, F_i, ws, s, fold && i > 0);
      if (e != hipSuccess) return hip_fail(e, "tpmlp_tp_bwd launch");
    }
  }
  if (!direct && !fold) {
    hipError_t e = timed(TPMLP_K_SHARD_SUM, s, [&] { return launch_sum(parts, t, dX, int64_t(mh), s); });
    if (e != hipSuccess) return hip_fail(e, "tpmlp_tp_bwd sum");
  }
  return TPMLP_OK;
}

tpmlp_status tpmlp_tp_fwd_full(const tpmlp_bf16* X, const tpmlp_bf16* A, const tpmlp_bf16* B, tpmlp_bf16* P,
                               float* Z, int t, int64_t M, int64_t H, int64_t F_i, void* ws, size_t ws_bytes,
                               void* stream) {
  g_last_error.clear();
  if (t < 1 || t > TPMLP_MAX_SHARDS) return fail(TPMLP_ERR_SHARDS, "t outside 1..TPMLP_MAX_SHARDS");
  tpmlp_status st = check_ptrs({{X, "X"}, {A, "A"}, {B, "B"}, {Z, "Z"}, {ws, "ws"}});
  if (st) return st;
  if (P && !aligned16(P)) return fail(TPMLP_ERR_ALIGN, "P is not 16-byte aligned");
  if ((st = check_shape(M, H, F_i))) return st;
  if (int64_t(t) * F_i > MAX_DIM) return fail(TPMLP_ERR_SHAPE, "t * F_i is above 2^23");
  const size_t need = tpmlp_tp_workspace_bytes(t, M, H, F_i);
  if (ws_bytes < need) return fail(TPMLP_ERR_WORKSPACE, "ws_bytes below tpmlp_tp_workspace_bytes");
  const int64_t F = int64_t(t) * F_i;
  const size_t mh = size_t(M) * H, hf = size_t(H) * F, mf = size_t(M) * F_i;
  std::vector<Range> ins = {{X, mh * 2, "X"}, {A, hf * 2, "A"}, {B, hf * 2, "B"}};
  std::vector<Range> outs = {{Z, mh * 4, "Z"}, {P, P ? mf * t * 2 : 0, "P"}, {ws, need, "ws"}};
  if ((st = check_alias(outs, ins))) return st;
  if ((st = check_device())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* partials = reinterpret_cast<float*>(ws_at(ws, shard_ws_bytes(M, H, F_i)));
  const float* parts[TPMLP_MAX_SHARDS];
  const bool fold = fold_sum(nullptr, t, H);
  for (int i = 0; i < t; ++i) {
    float* Zi = (t == 1 || fold) ? Z : partials + size_t(i) * mh;
    parts[i] = Zi;
    // Shard i: columns [i F_i, (i+1) F_i) of A (rows of F elements), rows of B.
    hipError_t e = enqueue_fwd(X, A + int64_t(i) * F_i, F, B + int64_t(i) * F_i * H, Zi,
                               P ? P + size_t(i) * mf : nullptr, M, H, F_i, ws, s, fold && i > 0);
    if (e != hipSuccess) return hip_fail(e, "tpmlp_tp_fwd_full launch");
  }
  if (t > 1 && !fold) {
    hipError_t e = timed(TPMLP_K_SHARD_SUM, s, [&] { return launch_sum(parts, t, Z, int64_t(mh), s); });
    if (e != hipSuccess) return hip_fail(e, "tpmlp_tp_fwd_full sum");
  }
  return TPMLP_OK;
}

tpmlp_status tpmlp_tp_bwd_full(const tpmlp_bf16* dZ, const tpmlp_bf16* X, const tpmlp_bf16* A,
                               const tpmlp_bf16* B, const tpmlp_bf16* P, float* dA, float* dB, float* dX, int t,
                               int64_t M, int64_t H, int64_t F_i, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (t < 1 || t > TPMLP_MAX_SHARDS) return fail(TPMLP_ERR_SHARDS, "t outside 1..TPMLP_MAX_SHARDS");
  tpmlp_status st =
      check_ptrs({{dZ, "dZ"}, {X, "X"}, {A, "A"}, {B, "B"}, {dA, "dA"}, {dB, "dB"}, {dX, "dX"}, {ws, "ws"}});
  if (st) return st;
  if (P && !aligned16(P)) return fail(TPMLP_ERR_ALIGN, "P is not 16-byte aligned");
  if ((st = check_shape(M, H, F_i))) return st;
  if (int64_t(t) * F_i > MAX_DIM) return fail(TPMLP_ERR_SHAPE, "t * F_i is above 2^23");
  const size_t need = tpmlp_tp_workspace_bytes(t, M, H, F_i);
  if (ws_bytes < need) return fail(TPMLP_ERR_WORKSPACE, "ws_bytes below tpmlp_tp_workspace_bytes");
  const int64_t F = int64_t(t) * F_i;
  const size_t mh = size_t(M) * H, hf = size_t(H) * F, mf = size_t(M) * F_i;
  std::vector<Range> ins = {{dZ, mh * 2, "dZ"}, {X, mh * 2, "X"}, {A, hf * 2, "A"}, {B, hf * 2, "B"},
                            {P, P ? mf * t * 2 : 0, "P"}};
  std::vector<Range> outs = {{dX, mh * 4, "dX"}, {dA, hf * 4, "dA"}, {dB, hf * 4, "dB"}, {ws, need, "ws"}};
  if ((st = check_alias(outs, ins))) return st;
  if ((st = check_device())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* partials = reinterpret_cast<float*>(ws_at(ws, shard_ws_bytes(M, H, F_i)));
  const float* parts[TPMLP_MAX_SHARDS];
  hipError_t et = enqueue_transposes(dZ, X, M, H, ws, s);
  if (et != hipSuccess) return hip_fail(et, "tpmlp_tp_bwd_full transpose");
  const bool fold = fold_sum(nullptr, t, H);
  for (int i = 0; i < t; ++i) {
    float* dXi = (t == 1 || fold) ? dX : partials + size_t(i) * mh;
    parts[i] = dXi;
    // Shard i: columns [i F_i, (i+1) F_i) of A and dA (rows of F elements), rows of B and dB.
    const int64_t c = int64_t(i) * F_i;
    hipError_t e = enqueue_bwd(dZ, X, A + c, F, B + c * H, P ? P + size_t(i) * mf : nullptr, dXi, dA + c, F,
                               dB + c * H, M, H, F_i, ws, s, fold && i > 0);
    if (e != hipSuccess) return hip_fail(e, "tpmlp_tp_bwd_full launch");
  }
  if (t > 1 && !fold) {
    hipError_t e = timed(TPMLP_K_SHARD_SUM, s, [&] { return launch_sum(parts, t, dX, int64_t(mh), s); });
    if (e != hipSuccess) return hip_fail(e, "tpmlp_tp_bwd_full sum");
  }
  return TPMLP_OK;
}

size_t tpmlp_sp_workspace_bytes(int t, int64_t M, int64_t H, int64_t F_i) {
  if (t < 1 || t > TPMLP_MAX_SHARDS || !shape_ok(M) || !shape_ok(H) || !shape_ok(F_i) || M % t || !shape_ok(M / t))
    return 0;
  return sp_ws_bytes(t, M, H, F_i);
}

tpmlp_status tpmlp_sp_fwd(const tpmlp_bf16* const* X_sl, const tpmlp_bf16* const* A_sh, const tpmlp_bf16* const* B_sh,
                          tpmlp_bf16* const* P_sh, float* const* Z_sl, int t, int64_t M, int64_t H, int64_t F_i,
                          void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (!X_sl || !A_sh || !B_sh || !Z_sl) return fail(TPMLP_ERR_NULL, "a slice or shard array is NULL");
  if (t < 1 || t > TPMLP_MAX_SHARDS) return fail(TPMLP_ERR_SHARDS, "t outside 1..TPMLP_MAX_SHARDS");
  tpmlp_status st = check_ptrs({{ws, "ws"}});
  if (st) return st;
  if ((st = check_sp_shape(t, M, H, F_i))) return st;
  const size_t need = tpmlp_sp_workspace_bytes(t, M, H, F_i);
  if (ws_bytes < need) return fail(TPMLP_ERR_WORKSPACE, "ws_bytes below tpmlp_sp_workspace_bytes");
  const int64_t S = M / t;
  const size_t sh = size_t(S) * H, hf = size_t(H) * F_i, mf = size_t(M) * F_i;
  std::vector<Range> ins, outs = {{ws, need, "ws"}};
  for (int i = 0; i < t; ++i) {
    const std::string idx = "[" + std::to_string(i) + "]";
    if (!X_sl[i] || !Z_sl[i] || !A_sh[i] || !B_sh[i]) return fail(TPMLP_ERR_NULL, "a slice or shard pointer" + idx + " is NULL");
    for (const void* p : {(const void*)X_sl[i], (const void*)Z_sl[i], (const void*)A_sh[i], (const void*)B_sh[i]})
      if (!aligned16(p)) return fail(TPMLP_ERR_ALIGN, "a slice or shard pointer" + idx + " is not 16-byte aligned");
    ins.push_back({X_sl[i], sh * 2, "X_sl[i]"});
    ins.push_back({A_sh[i], hf * 2, "A_sh[i]"});
    ins.push_back({B_sh[i], hf * 2, "B_sh[i]"});
    outs.push_back({Z_sl[i], sh * 4, "Z_sl[i]"});
    if (P_sh && P_sh[i]) {
      if (!aligned16(P_sh[i])) return fail(TPMLP_ERR_ALIGN, "P_sh" + idx + " is not 16-byte aligned");
      outs.push_back({P_sh[i], mf * 2, "P_sh[i]"});
    }
  }
  if ((st = check_alias(outs, ins))) return st;
  if ((st = check_device())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Shard i over the ranks' row blocks: block r reads rank r's tokens and writes
  // (shard 0) or adds to (shards 1 ..) rank r's output slice, so each slice ends
  // as the rank-order sum of the shards' rows: the reduce-scatter's result.
  for (int i = 0; i < t; ++i) {
    for (int r = 0; r < t; ++r) {
      tpmlp_bf16* Pi = (P_sh && P_sh[i]) ? P_sh[i] + size_t(r) * S * F_i : nullptr;
      hipError_t e = enqueue_fwd(X_sl[r], A_sh[i], F_i, B_sh[i], Z_sl[r], Pi, S, H, F_i, ws, s, i > 0, r > 0);
      if (e != hipSuccess) return hip_fail(e, "tpmlp_sp_fwd launch");
    }
  }
  return TPMLP_OK;
}

tpmlp_status tpmlp_sp_bwd(const tpmlp_bf16* const* dZ_sl, const tpmlp_bf16* const* X_sl,
                          const tpmlp_bf16* const* A_sh, const tpmlp_bf16* const* B_sh, const tpmlp_bf16* const* P_sh,
                          float* const* dA_sh, float* const* dB_sh, float* const* dX_sl, int t, int64_t M, int64_t H,
                          int64_t F_i, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (!dZ_sl || !X_sl || !A_sh || !B_sh || !dA_sh || !dB_sh || !dX_sl)
    return fail(TPMLP_ERR_NULL, "a slice or shard array is NULL");
  if (t < 1 || t > TPMLP_MAX_SHARDS) return fail(TPMLP_ERR_SHARDS, "t outside 1..TPMLP_MAX_SHARDS");
  tpmlp_status st = check_ptrs({{ws, "ws"}});
  if (st) return st;
  if ((st = check_sp_shape(t, M, H, F_i))) return st;
  const size_t need = tpmlp_sp_workspace_bytes(t, M, H, F_i);
  if (ws_bytes < need) return fail(TPMLP_ERR_WORKSPACE, "ws_bytes below tpmlp_sp_workspace_bytes");
  const int64_t S = M / t;
  const size_t sh = size_t(S) * H, hf = size_t(H) * F_i, mf = size_t(M) * F_i;
  std::vector<Range> ins, outs = {{ws, need, "ws"}};
  for (int i = 0; i < t; ++i) {
    const std::string idx = "[" + std::to_string(i) + "]";
    const void* ptrs[] = {dZ_sl[i], X_sl[i], A_sh[i], B_sh[i], dA_sh[i], dB_sh[i], dX_sl[i]};
    for (const void* p : ptrs) {
      if (!p) return fail(TPMLP_ERR_NULL, "a slice or shard pointer" + idx + " is NULL");
      if (!aligned16(p)) return fail(TPMLP_ERR_ALIGN, "a slice or shard pointer" + idx + " is not 16-byte aligned");
    }
    if (P_sh && !P_sh[i]) return fail(TPMLP_ERR_NULL, "P_sh" + idx + " is NULL");
    if (P_sh && !aligned16(P_sh[i])) return fail(TPMLP_ERR_ALIGN, "P_sh" + idx + " is not 16-byte aligned");
    ins.push_back({dZ_sl[i], sh * 2, "dZ_sl[i]"});
    ins.push_back({X_sl[i], sh * 2, "X_sl[i]"});
    ins.push_back({A_sh[i], hf * 2, "A_sh[i]"});
    ins.push_back({B_sh[i], hf * 2, "B_sh[i]"});
    if (P_sh) ins.push_back({P_sh[i], mf * 2, "P_sh[i]"});
    outs.push_back({dA_sh[i], hf * 4, "dA_sh[i]"});
    outs.push_back({dB_sh[i], hf * 4, "dB_sh[i]"});
    outs.push_back({dX_sl[i], sh * 4, "dX_sl[i]"});
  }
  if ((st = check_alias(outs, ins))) return st;
  if ((st = check_device())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = enqueue_sp_transposes(dZ_sl, X_sl, t, M, H, ws, s);
  if (e != hipSuccess) return hip_fail(e, "tpmlp_sp_bwd transpose");
  for (int i = 0; i < t; ++i) {
    e = enqueue_bwd_sp(dZ_sl, X_sl, A_sh[i], B_sh[i], P_sh ? P_sh[i] : nullptr, dX_sl, dA_sh[i], dB_sh[i], t, M, H,
                       F_i, ws, s, i > 0);
    if (e != hipSuccess) return hip_fail(e, "tpmlp_sp_bwd launch");
  }
  return TPMLP_OK;
}

size_t tpmlp_fp8_workspace_bytes(int t, int64_t M, int64_t H, int64_t F_i) {
  if (t < 1 || t > TPMLP_MAX_SHARDS || !shape16_ok(M) || !shape16_ok(H) || !shape16_ok(F_i)) return 0;
  return fp8_layout(t, M, H, F_i).total;
}

tpmlp_status tpmlp_fp8_tp_fwd(const tpmlp_bf16* X, const tpmlp_bf16* const* A_sh, const tpmlp_bf16* const* B_sh,
                              tpmlp_bf16* const* P_sh, float* Z, int t, int64_t M, int64_t H, int64_t F_i,
                              void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (!A_sh || !B_sh) return fail(TPMLP_ERR_NULL, "A_sh or B_sh is NULL");
  if (t < 1 || t > TPMLP_MAX_SHARDS) return fail(TPMLP_ERR_SHARDS, "t outside 1..TPMLP_MAX_SHARDS");
  tpmlp_status st = check_ptrs({{X, "X"}, {Z, "Z"}, {ws, "ws"}});
  if (st) return st;
  if ((st = check_shape_fp8(M, H, F_i))) return st;
  const size_t need = tpmlp_fp8_workspace_bytes(t, M, H, F_i);
  if (ws_bytes < need) return fail(TPMLP_ERR_WORKSPACE, "ws_bytes below tpmlp_fp8_workspace_bytes");
  const size_t mh = size_t(M) * H, hf = size_t(H) * F_i, mf = size_t(M) * F_i;
  std::vector<Range> ins = {{X, mh * 2, "X"}};
  std::vector<Range> outs = {{Z, mh * 4, "Z"}, {ws, need, "ws"}};
  for (int i = 0; i < t; ++i) {
    if (!A_sh[i] || !B_sh[i]) return fail(TPMLP_ERR_NULL, "A_sh[" + std::to_string(i) + "] or B_sh[i] is NULL");
    if (!aligned16(A_sh[i]) || !aligned16(B_sh[i])) return fail(TPMLP_ERR_ALIGN, "a weight shard is not 16-byte aligned");
    ins.push_back({A_sh[i], hf * 2, "A_sh[i]"});
    ins.push_back({B_sh[i], hf * 2, "B_sh[i]"});
    if (P_sh && P_sh[i]) {
      if (!aligned16(P_sh[i])) return fail(TPMLP_ERR_ALIGN, "P_sh[i] is not 16-byte aligned");
      outs.push_back({P_sh[i], mf * 2, "P_sh[i]"});
    }
  }
  if ((st = check_alias(outs, ins))) return st;
  if ((st = check_device())) return st;
  forget_fp8_forward(ws);
  hipError_t e = enqueue_fp8_fwd(X, A_sh, B_sh, P_sh, Z, t, M, H, F_i, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tpmlp_fp8_tp_fwd launch");
  record_fp8_forward(ws, make_stamp(X, A_sh, B_sh, P_sh, t, M, H, F_i));
  return TPMLP_OK;
}

tpmlp_status tpmlp_fp8_tp_bwd(const tpmlp_bf16* dZ, const tpmlp_bf16* X, const tpmlp_bf16* const* A_sh,
                              const tpmlp_bf16* const* B_sh, const tpmlp_bf16* const* P_sh,
                              float* const* dA_sh, float* const* dB_sh, float* dX, int t, int64_t M, int64_t H,
                              int64_t F_i, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (!A_sh || !B_sh || !dA_sh || !dB_sh) return fail(TPMLP_ERR_NULL, "a shard array is NULL");
  if (t < 1 || t > TPMLP_MAX_SHARDS) return fail(TPMLP_ERR_SHARDS, "t outside 1..TPMLP_MAX_SHARDS");
  tpmlp_status st = check_ptrs({{dZ, "dZ"}, {X, "X"}, {dX, "dX"}, {ws, "ws"}});
  if (st) return st;
  if ((st = check_shape_fp8(M, H, F_i))) return st;
  const size_t need = tpmlp_fp8_workspace_bytes(t, M, H, F_i);
  if (ws_bytes < need) return fail(TPMLP_ERR_WORKSPACE, "ws_bytes below tpmlp_fp8_workspace_bytes");
  const size_t mh = size_t(M) * H, hf = size_t(H) * F_i, mf = size_t(M) * F_i;
  std::vector<Range> ins = {{dZ, mh * 2, "dZ"}, {X, mh * 2, "X"}};
  std::vector<Range> outs = {{dX, mh * 4, "dX"}, {ws, need, "ws"}};
  for (int i = 0; i < t; ++i) {
    const std::string idx = "[" + std::to_string(i) + "]";
    if (!A_sh[i] || !B_sh[i] || !dA_sh[i] || !dB_sh[i]) return fail(TPMLP_ERR_NULL, "a shard pointer" + idx + " is NULL");
    if (P_sh && !P_sh[i]) return fail(TPMLP_ERR_NULL, "P_sh" + idx + " is NULL");
    for (const void* p : {(const void*)A_sh[i], (const void*)B_sh[i], (const void*)dA_sh[i], (const void*)dB_sh[i]})
      if (!aligned16(p)) return fail(TPMLP_ERR_ALIGN, "a shard pointer" + idx + " is not 16-byte aligned");
    if (P_sh && !aligned16(P_sh[i])) return fail(TPMLP_ERR_ALIGN, "P_sh" + idx + " is not 16-byte aligned");
    ins.push_back({A_sh[i], hf * 2, "A_sh[i]"});
    ins.push_back({B_sh[i], hf * 2, "B_sh[i]"});
    if (P_sh) ins.push_back({P_sh[i], mf * 2, "P_sh[i]"});
    outs.push_back({dA_sh[i], hf * 4, "dA_sh[i]"});
    outs.push_back({dB_sh[i], hf * 4, "dB_sh[i]"});
  }
  if ((st = check_alias(outs, ins))) return st;
  const std::string why = check_fp8_forward(ws, make_stamp(X, A_sh, B_sh, P_sh, t, M, H, F_i), P_sh != nullptr);
  if (!why.empty()) return fail(TPMLP_ERR_NO_FORWARD, "ws does not hold the forward of these inputs: " + why);
  if ((st = check_device())) return st;
  hipError_t e = enqueue_fp8_bwd(dZ, P_sh, dA_sh, dB_sh, dX, t, M, H, F_i, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TPMLP_OK : hip_fail(e, "tpmlp_fp8_tp_bwd launch");
}

tpmlp_status tpmlp_fp8_quantize(const tpmlp_bf16* T, int64_t R, int64_t C, int fmt, int transpose, uint8_t* codes,
                                float* amax, void* stream) {
  g_last_error.clear();
  tpmlp_status st = check_ptrs({{T, "T"}, {codes, "codes"}, {amax, "amax"}});
  if (st) return st;
  if (!shape16_ok(R) || !shape16_ok(C)) return fail(TPMLP_ERR_SHAPE, "R and C must be positive multiples of 16, at most 2^23");
  if (fmt != 0 && fmt != 1) return fail(TPMLP_ERR_SHAPE, "fmt must be 0 (E4M3) or 1 (E5M2)");
  if ((st = check_alias({{codes, size_t(R) * C, "codes"}, {amax, 4, "amax"}}, {{T, size_t(R) * C * 2, "T"}}))) return st;
  if ((st = check_device())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* slot = reinterpret_cast<uint32_t*>(amax);
  hipError_t e = launch_fp8_zero(slot, 1, s);  // the caller's float is a one-word slot
  if (e == hipSuccess) e = launch_fp8_amax(T, R, C, C, slot, 1, s);
  if (e == hipSuccess)
    e = launch_fp8_quant(T, R, C, C, false, fmt, slot, 1, codes, transpose ? R : C, transpose != 0, s);
  return e == hipSuccess ? TPMLP_OK : hip_fail(e, "tpmlp_fp8_quantize launch");
}

tpmlp_status tpmlp_timing_begin(int capacity) { return tpmlp_timing_begin_kinds(capacity, (1u << TPMLP_K_COUNT) - 1); }

tpmlp_status tpmlp_timing_begin_kinds(int capacity, unsigned kinds) {
  g_last_error.clear();
  if (capacity < 1) return fail(TPMLP_ERR_SHAPE, "capacity must be positive");
  if (kinds == 0 || (kinds >> TPMLP_K_COUNT) != 0)
    return fail(TPMLP_ERR_SHAPE, "kinds must be a nonzero mask of bits below TPMLP_K_COUNT");
  Timing& t = g_timing;
  for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
  t.ev.assign(2 * size_t(capacity), nullptr);
  t.kind.assign(capacity, 0);
  t.disp.assign(capacity, 1);
  for (auto& e : t.ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      t.on = false;
      return hip_fail(r, "hipEventCreate");
    }
  }
  t.cap = capacity;
  t.n = 0;
  t.dropped = 0;
  t.kinds = kinds;
  t.on = true;
  return TPMLP_OK;
}

tpmlp_status tpmlp_timing_end(int* counts, double* total_ms, int* dropped) {
  g_last_error.clear();
  if (!counts || !total_ms) return fail(TPMLP_ERR_NULL, "counts or total_ms is NULL");
  Timing& t = g_timing;
  for (int k = 0; k < TPMLP_K_COUNT; ++k) {
    counts[k] = 0;
    total_ms[k] = 0.0;
  }
  if (dropped) *dropped = t.dropped;
  t.on = false;
  t.last_kind.clear();
  t.last_disp.clear();
  t.last_ms.clear();
  for (int i = 0; i < t.n; ++i) {
    hipError_t e = hipEventSynchronize(t.ev[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, t.ev[2 * i], t.ev[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    counts[t.kind[i]] += 1;
    total_ms[t.kind[i]] += ms;
    t.last_kind.push_back(t.kind[i]);
    t.last_disp.push_back(t.disp[i]);
    t.last_ms.push_back(ms);
  }
  t.n = 0;
  return TPMLP_OK;
}

int tpmlp_timing_records(int* kinds, double* ms, int capacity) {
  if (!kinds || !ms) return -1;
  const Timing& t = g_timing;
  const int n = (int)t.last_kind.size();
  for (int i = 0; i < n && i < capacity; ++i) {
    kinds[i] = t.last_kind[i];
    ms[i] = t.last_ms[i];
  }
  return n;
}

int tpmlp_timing_dispatches(int* dispatches, int capacity) {
  if (!dispatches) return -1;
  const Timing& t = g_timing;
  const int n = (int)t.last_disp.size();
  for (int i = 0; i < n && i < capacity; ++i) dispatches[i] = t.last_disp[i];
  return n;
}

}  // extern "C"
