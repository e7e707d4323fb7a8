"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Acceptance per output tensor: max|gpu - oracle| <= 1e-2 * max|oracle| + 1e-3.
Small shapes are compared in full, with ragged tails on every dimension; the
benchmark configurations are run in the launch configuration the benchmark
times and compared in full where the oracle is quick, on sampled rows/columns
(each computed from the definition) where it is not.
"""
import sys

import numpy as np
import pytest

import margins
from oracle import oracle as O
from tensor_transformer_mlp_03_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tensor_transformer_mlp_03_amd import _lib as L
    L.lib()  # fails loudly if the library is not built


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dec(bits):
    return O.decode_bf16(bits)


def check(name, got, ref, ratios):
    err = O.max_abs_err(got, ref)
    tol = O.tolerance(ref)
    ratios[name] = err / tol
    margins.record(name, err / tol)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert err <= tol, f"{name}: max err {err:.3e} > tol {tol:.3e} (err/tol {err / tol:.3f})"


def check_dev(name, got, ref, ratios):
    """check() on two device tensors of the same shape, reduced on the GPU (for
    outputs too large to copy back whole); ref is the reference side."""
    err = (got.double() - ref.double()).abs().max().item()
    tol = 1e-2 * ref.double().abs().max().item() + 1e-3
    ratios[name] = err / tol
    margins.record(name, err / tol)
    assert bool(torch.isfinite(got).all()), f"{name}: non-finite values"
    assert err <= tol, f"{name}: max err {err:.3e} > tol {tol:.3e} (err/tol {err / tol:.3f})"


def run_device(inp, store_p=True, keep_partials=True):
    from tensor_transformer_mlp_03_amd.device import DeviceMLP
    d = DeviceMLP(inp, store_p=store_p, driver=True, keep_partials=keep_partials)
    d.step()
    torch.cuda.synchronize()
    return d


SMALL = [
    # (M, H, F_i, t, store_p): ragged in every dimension vs the 128/256 tiles and the 64-wide K step
    (64, 256, 512, 2, True),
    (200, 264, 392, 2, True),
    (328, 136, 776, 3, False),
    (8, 8, 8, 1, True),
    (520, 520, 264, 2, False),
    (1032, 1040, 1048, 1, True),
    # M large enough that the forward (and the recompute) transpose the weights
    # first and run every product K-contiguous
    (8200, 264, 392, 2, False),
    (8200, 136, 520, 2, True),
    # enough output tiles for 256 x 256 tiles, with the weights read N-contiguous
    (4104, 1032, 2056, 2, False),
    # 256 x 128 tiles, unsplit for [M, F_i] and split 7 ways for [M, H] (and the
    # other way round)
    (1024, 1032, 16640, 1, True),
    (1024, 16640, 1032, 1, False),
    # 4 x 65 output tiles of 256 x 256 (one wave and 4 more): the products with an
    # [M, F_i] output run 256 tiles whole and split only the last column block
    # along K (GeLU epilogue in the forward, dGeLU in the backward) ...
    (1024, 2056, 16640, 1, True),
    # ... and with an [M, H] output (float32 epilogue, forward and dX)
    (1024, 16640, 2056, 1, False),
    # fused forward (H a multiple of 64, at most 256): ragged rows and a ragged last
    # chunk of intermediate columns, with the pre-activation kept from it ...
    (200, 192, 392, 2, True),
    # ... one chunk (the kernel writes Z_i itself), the smallest hidden size ...
    (8, 64, 8, 1, True),
    # ... many chunks and row blocks, backward recomputing
    (520, 128, 1032, 2, False),
    (72, 256, 2056, 2, True),
    # M = F_i, ragged: with one shard its dB_i and dX_i run as one launch; with two the
    # driver batches the shards' dB instead
    (1048, 264, 1048, 1, True),
    (520, 1040, 520, 2, False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "x".join(map(str, c[:4])) + ("_store" if c[4] else "_recompute"))
def test_small_full(case):
    M, H, F, t, store = case
    say(f"[parity small] M={M} H={H} F_i={F} t={t} store_p={store}")
    w = I.custom_workload(200 + M % 97, M=M, H=H, F_i=F, t=t, w_std=0.05)
    inp = I.make_inputs(w)
    d = run_device(inp, store_p=store)
    X, dZ = dec(inp.X), dec(inp.dZ)
    A = [dec(a) for a in inp.A]
    B = [dec(b) for b in inp.B]
    Z, Zp = O.tp_forward(X, A, B)
    dX, dXp, dAp, dBp = O.tp_backward(dZ, X, A, B)
    r = {}
    check("Z", d.Z.cpu().numpy(), Z, r)
    check("dX", d.dX.cpu().numpy(), dX, r)
    for i in range(t):
        check(f"Z_{i}", d.Z_sh[i].cpu().numpy(), Zp[i], r)
        check(f"dX_{i}", d.dX_sh[i].cpu().numpy(), dXp[i], r)
        check(f"dA_{i}", d.dA[i].cpu().numpy(), dAp[i], r)
        check(f"dB_{i}", d.dB[i].cpu().numpy(), dBp[i], r)
    say("  err/tol:", {k: round(v, 3) for k, v in r.items()})


def _random_cases(n, seed):
    """Seeded shapes off every tile and chunk boundary: M, H, F_i multiples of 8 up
    to ~700 (some below 64, the epilogue chunk), t of 1-3, P kept or recomputed."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M, H, F = (int(8 * rng.integers(1, 88)) for _ in range(3))
        out.append((M, H, F, int(rng.integers(1, 4)), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("case", _random_cases(24, 2026),
                         ids=lambda c: "x".join(map(str, c[:4])) + ("_store" if c[4] else "_recompute"))
def test_random_shapes(case):
    """The t-shard forward and backward on random ragged shapes, every output
    element against the oracle (the planner's choices of tile, split, fused or
    batched launch vary with the shape)."""
    test_small_full(case)


def test_config0_forward():
    w = I.CONFIGS[0]
    say(f"[parity config0] {w}")
    inp = I.make_inputs(w)
    d = run_device(inp)
    X = dec(inp.X)
    A = [dec(a) for a in inp.A]
    B = [dec(b) for b in inp.B]
    Z, Zp = O.tp_forward(X, A, B)
    r = {}
    check("Z", d.Z.cpu().numpy(), Z, r)
    for i in range(w.t):
        check(f"Z_{i}", d.Z_sh[i].cpu().numpy(), Zp[i], r)
    # shard-sum identity against the unsharded MLP
    Zfull = O.mlp_forward(X, np.concatenate(A, 1), np.concatenate(B, 0))["Z"]
    check("Z_vs_unsharded", d.Z.cpu().numpy(), Zfull, r)
    say("  err/tol:", {k: round(v, 3) for k, v in r.items()})


@pytest.mark.parametrize("cfg", [1, 2])
def test_config_full(cfg):
    w = I.CONFIGS[cfg]
    say(f"[parity config{cfg}] {w}")
    inp = I.make_inputs(w)
    d = run_device(inp, store_p=not w.recompute, keep_partials=False)
    X, dZ = dec(inp.X), dec(inp.dZ)
    A = [dec(a) for a in inp.A]
    B = [dec(b) for b in inp.B]
    r = {}
    Zsum, dXsum = None, None
    for i in range(w.t):
        f = O.mlp_forward(X, A[i], B[i])
        g = O.mlp_backward(dZ, X, A[i], B[i])
        Zsum = f["Z"] if Zsum is None else Zsum + f["Z"]
        dXsum = g["dX"] if dXsum is None else dXsum + g["dX"]
        check(f"dA_{i}", d.dA[i].cpu().numpy(), g["dA"], r)
        check(f"dB_{i}", d.dB[i].cpu().numpy(), g["dB"], r)
    check("Z", d.Z.cpu().numpy(), Zsum, r)
    check("dX", d.dX.cpu().numpy(), dXsum, r)
    say("  err/tol:", {k: round(v, 3) for k, v in r.items()})


def _sample(n, k, rng, must=()):
    idx = set(int(v) for v in must)
    while len(idx) < min(k + len(must), n):
        idx.add(int(rng.integers(0, n)))
    return np.array(sorted(idx))


def _per_block(n, block, per_block, rng, exclude=()):
    """per_block distinct seeded indices from every block of `block` consecutive
    indices of range(n) (the last block may be short), none of them in `exclude`:
    every output tile row (or column) block is touched."""
    ex = np.zeros(n, dtype=bool)
    ex[np.asarray(exclude, dtype=np.int64)] = True
    out = []
    for b0 in range(0, n, block):
        cand = np.nonzero(~ex[b0:b0 + block])[0] + b0
        out.extend(rng.choice(cand, size=min(per_block, cand.size), replace=False).tolist())
    return np.array(sorted(out), dtype=np.int64)


def test_config3_sampled():
    """Long-context chunk at full size, all four shards, per-shard partials kept.

    Rows of Z_i, dX_i, Z and dX are compared in two classes, each against a
    tolerance from its own max|oracle|: two seeded rows from every 256-row tile of
    rows that are not outliers, and 32 of the 328 outlier rows (X scaled x8).  The
    outliers dominate max|oracle| of a mixed sample, so a mixed check would judge
    the normal rows at about 8x the stated tolerance.  Columns of dA_i and rows of
    dB_i: two from every 256-wide block of F_i (the split-K products' tiles)."""
    w = I.CONFIGS[3]
    say(f"[parity config3 sampled] {w}")
    inp = I.make_inputs(w)
    from tensor_transformer_mlp_03_amd.device import DeviceMLP
    d = DeviceMLP(inp, store_p=True, driver=True, keep_partials=True)
    d.step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(1234 + 3)
    normal = _per_block(w.M, 256, 2, rng, exclude=inp.outliers)
    outl = np.sort(rng.choice(inp.outliers, size=32, replace=False))
    cols = _per_block(w.F_i, 256, 2, rng)
    say(f"  {normal.size} normal rows, {outl.size} outlier rows, {cols.size} dA columns / dB rows")
    X, dZ = dec(inp.X), dec(inp.dZ)
    r = {}
    sums = {}
    for i in range(w.t):
        A, B = dec(inp.A[i]), dec(inp.B[i])
        for cls, rows in (("normal", normal), ("outlier", outl)):
            z = O.forward_rows(X, A, B, rows)
            dx = O.backward_dX_rows(dZ, X, A, B, rows)
            check(f"Z_{i}[{cls}]", d.Z_sh[i][rows].cpu().numpy(), z, r)
            check(f"dX_{i}[{cls}]", d.dX_sh[i][rows].cpu().numpy(), dx, r)
            zs, dxs = sums.get(cls, (0.0, 0.0))
            sums[cls] = (zs + z, dxs + dx)
        check(f"dA_{i}[:,cols]", d.dA[i][:, cols].cpu().numpy(), O.backward_dA_cols(dZ, X, A, B, cols), r)
        check(f"dB_{i}[cols,:]", d.dB[i][cols, :].cpu().numpy(), O.backward_dB_rows(dZ, X, A, B, cols), r)
        del A, B
    for cls, rows in (("normal", normal), ("outlier", outl)):
        check(f"Z[{cls}]", d.Z[rows].cpu().numpy(), sums[cls][0], r)
        check(f"dX[{cls}]", d.dX[rows].cpu().numpy(), sums[cls][1], r)
    # The launch configuration the benchmark times: no per-shard partials, the
    # sums folded into the products.  Same bits as the run checked above.
    b = DeviceMLP(inp, store_p=True, driver=True, keep_partials=False)
    b.step()
    torch.cuda.synchronize()
    assert torch.equal(b.Z, d.Z) and torch.equal(b.dX, d.dX)
    for x, y in list(zip(b.dA, d.dA)) + list(zip(b.dB, d.dB)):
        assert torch.equal(x, y)
    del b
    say("  err/tol:", {k: round(v, 3) for k, v in r.items()})


def test_config4_shard0_sampled():
    """530B-class shard 0 at full size in the launch configuration the benchmark
    times (one rank's tpmlp_fwd and tpmlp_bwd, pre-activation recomputed): two
    seeded rows from every 256-row tile plus the first and last rows, and two
    dA_0 columns / dB_0 rows from every 256-wide block of F_i (the hybrid
    products' whole-wave columns and their split tail, columns 8192 on)."""
    w = I.CONFIGS[4]
    say(f"[parity config4 shard 0 sampled] {w}")
    inp = I.make_inputs(w, shards=[0])
    from tensor_transformer_mlp_03_amd.device import DeviceMLP
    d = DeviceMLP(inp, store_p=False, driver=False, shards=[0])
    d.step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(1234 + 4)
    rows = np.union1d(_per_block(w.M, 256, 2, rng), [0, w.M - 1])
    cols = _per_block(w.F_i, 256, 2, rng)
    X, dZ = dec(inp.X), dec(inp.dZ)
    A, B = dec(inp.A[0]), dec(inp.B[0])
    r = {}
    check("Z_0[rows]", d.Z_sh[0][rows].cpu().numpy(), O.forward_rows(X, A, B, rows), r)
    check("dX_0[rows]", d.dX_sh[0][rows].cpu().numpy(), O.backward_dX_rows(dZ, X, A, B, rows), r)
    check("dA_0[:,cols]", d.dA[0][:, cols].cpu().numpy(), O.backward_dA_cols(dZ, X, A, B, cols), r)
    check("dB_0[cols,:]", d.dB[0][cols, :].cpu().numpy(), O.backward_dB_rows(dZ, X, A, B, cols), r)
    say("  err/tol:", {k: round(v, 3) for k, v in r.items()})


def test_config4_shard_sum_identity():
    """530B-class workload with all eight shards: the t-shard driver (sums folded
    into the products, pre-activation recomputed) against the unsharded MLP.

    * Z and dX on 64 seeded rows against the oracle of the unsharded weights
      A = [A_0 | ... | A_7], B = [B_0; ...; B_7] (each decoded whole, 13.4 GB of
      float64), so the identity sum_i GeLU(X A_i) B_i = GeLU(X A) B is checked at
      H = 20480, F = 81920;
    * Z, dX and the weight-gradient blocks against one GPU run with t = 1 on the
      whole weights (F_i = 81920);
    * the whole-weight driver (shards as strided views of A and B) gives the bits
      of the per-shard driver."""
    from tensor_transformer_mlp_03_amd.device import DeviceMLP
    w = I.CONFIGS[4]
    say(f"[identity config4] {w}: generating all {w.t} shards")
    inp = I.make_inputs(w)
    say("  t = 8 driver")
    d = DeviceMLP(inp, store_p=False, driver=True, keep_partials=False)
    d.step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(4321)
    rows = np.union1d(rng.choice(w.M, size=62, replace=False), [0, w.M - 1])
    say("  oracle of the unsharded MLP on 64 rows")
    Xr, dZr = dec(inp.X[rows]), dec(inp.dZ[rows])
    Af = dec(np.concatenate(inp.A, axis=1))          # [H, F] float64
    P = Xr @ Af
    Bf = dec(np.concatenate(inp.B, axis=0))          # [F, H]
    Z = O.gelu(P) @ Bf
    dP = (dZr @ Bf.T) * O.gelu_grad(P)
    del Bf
    dX = dP @ Af.T
    del Af, P, dP
    r = {}
    check("Z[rows]_vs_unsharded", d.Z[rows].cpu().numpy(), Z, r)
    check("dX[rows]_vs_unsharded", d.dX[rows].cpu().numpy(), dX, r)
    say("  t = 1 run on the whole weights")
    one = I.Inputs(I.custom_workload(340, M=w.M, H=w.H, F_i=w.F, t=1, w_std=w.w_std, recompute=True), inp.X,
                   [np.concatenate(inp.A, axis=1)], [np.concatenate(inp.B, axis=0)], inp.dZ)
    d1 = DeviceMLP(one, store_p=False, driver=True)
    del one
    d1.step()
    torch.cuda.synchronize()
    check_dev("Z_t8_vs_t1", d.Z, d1.Z, r)
    check_dev("dX_t8_vs_t1", d.dX, d1.dX, r)
    F = w.F_i
    for i in range(w.t):
        check_dev(f"dA_{i}_vs_t1_block", d.dA[i], d1.dA[0][:, i * F:(i + 1) * F], r)
        check_dev(f"dB_{i}_vs_t1_block", d.dB[i], d1.dB[0][i * F:(i + 1) * F], r)
    del d1
    torch.cuda.empty_cache()
    say("  whole-weight driver")
    f = DeviceMLP(inp, store_p=False, driver=True, full_weights=True)
    f.step()
    torch.cuda.synchronize()
    assert torch.equal(f.Z, d.Z) and torch.equal(f.dX, d.dX)
    for x, y in list(zip(f.dA, d.dA)) + list(zip(f.dB, d.dB)):
        assert torch.equal(x, y)
    say("  err/tol:", {k: round(v, 3) for k, v in r.items()})


def test_largest_hidden_size():
    """H at the library's limit, 2^23: a 256-row tile's operand rows are 2^24 bytes
    apart, so the loaders' 32-bit offsets within 128-row bands reach 2.1e9 bytes (X,
    dZ and B_i read with row stride H, the transposes of X and dZ).  M = 136 gives
    tiles with rows past 128.  Sampled rows of Z and dX and rows of dB are checked
    against the oracle (tokens are independent: a row needs only its own X and dZ)."""
    from tensor_transformer_mlp_03_amd.device import DeviceMLP
    M, H, F = 136, 1 << 23, 64
    say(f"[largest H] M={M} H={H} F_i={F}: generating inputs")
    w = I.custom_workload(322, M=M, H=H, F_i=F, t=1, w_std=0.02)
    inp = I.make_inputs(w)
    say("  running")
    d = DeviceMLP(inp, store_p=True, driver=False)
    d.step()
    torch.cuda.synchronize()
    say("  checking")
    rng = np.random.default_rng(322)
    rows = _sample(M, 6, rng, must=[0, 127, 128, M - 1])
    A, B = dec(inp.A[0]), dec(inp.B[0])
    Xr, dZr = dec(inp.X[rows]), dec(inp.dZ[rows])
    sub = np.arange(len(rows))
    r = {}
    check("Z[rows]", d.Z_sh[0][rows].cpu().numpy(), O.forward_rows(Xr, A, B, sub), r)
    check("dX[rows]", d.dX_sh[0][rows].cpu().numpy(), O.backward_dX_rows(dZr, Xr, A, B, sub), r)
    del Xr, dZr
    frows = np.array([0, F - 1])
    X, dZ = dec(inp.X), dec(inp.dZ)
    check("dB[frows]", d.dB[0][frows].cpu().numpy(), O.backward_dB_rows(dZ, X, A, B, frows), r)
    say("  err/tol:", {k: round(v, 3) for k, v in r.items()})


@pytest.mark.parametrize("t", [2, 4, 8])
def test_gpu_shard_sum_identity(t):
    """The t-shard driver's sum equals one unsharded run (t = 1) of the same A, B."""
    M, H, F = 512, 512, 2048
    say(f"[identity gpu] t={t} M={M} H={H} F={F}")
    w8 = I.custom_workload(300, M=M, H=H, F_i=F // 8, t=8)
    inp = I.make_inputs(w8)
    A = np.concatenate(inp.A, axis=1)
    B = np.concatenate(inp.B, axis=0)
    wt = I.custom_workload(301, M=M, H=H, F_i=F // t, t=t)
    sh = I.Inputs(wt, inp.X, [np.ascontiguousarray(a) for a in np.split(A, t, axis=1)],
                  [np.ascontiguousarray(b) for b in np.split(B, t, axis=0)], inp.dZ)
    w1 = I.custom_workload(302, M=M, H=H, F_i=F, t=1)
    one = I.Inputs(w1, inp.X, [A], [B], inp.dZ)
    ds, d1 = run_device(sh), run_device(one)
    ref = O.mlp_forward(dec(inp.X), dec(A), dec(B))["Z"]
    r = {}
    check("Z_t_vs_t1", ds.Z.cpu().numpy(), d1.Z.cpu().numpy().astype(np.float64), r)
    check("Z_t_vs_oracle", ds.Z.cpu().numpy(), ref, r)
    check("dX_t_vs_t1", ds.dX.cpu().numpy(), d1.dX.cpu().numpy().astype(np.float64), r)
    # the weight gradients of the shards are the column/row blocks of the unsharded ones
    check("dA_blocks", np.concatenate([a.cpu().numpy() for a in ds.dA], 1), d1.dA[0].cpu().numpy().astype(np.float64), r)
    check("dB_blocks", np.concatenate([b.cpu().numpy() for b in ds.dB], 0), d1.dB[0].cpu().numpy().astype(np.float64), r)
    say("  err/tol:", {k: round(v, 3) for k, v in r.items()})


@pytest.mark.parametrize("shape", [(1000, 520, 776), (200, 192, 392)], ids=["two_products", "fused_forward"])
def test_store_equals_recompute_bitwise(shape):
    """Keeping the bf16 pre-activation or recomputing it gives identical bits: both
    come from a chain of MFMAs over k in the same order (the fused forward's P_i
    included, H = 192)."""
    M, H, F = shape
    w = I.custom_workload(310, M=M, H=H, F_i=F, t=2)
    say(f"[store vs recompute] {w}")
    inp = I.make_inputs(w)
    a, b = run_device(inp, store_p=True), run_device(inp, store_p=False)
    for x, y in [(a.dX, b.dX)] + list(zip(a.dA, b.dA)) + list(zip(a.dB, b.dB)):
        assert torch.equal(x, y)


@pytest.mark.parametrize("case", [(200, 264, 392, 3, True), (520, 128, 1032, 2, False), (8200, 136, 520, 2, True),
                                  (1024, 1032, 16640, 1, False)],
                         ids=lambda c: "x".join(map(str, c[:4])) + ("_store" if c[4] else "_recompute"))
def test_full_weights_equal_shards_bitwise(case):
    """The whole-weight drivers (A_i a strided column view of A, dA_i of dA) give the
    bits of the per-shard drivers on contiguous copies of the same shards: the
    plans and kernels are the same, only the row strides differ.  Covers the
    fused forward, the weight transposes (M = 8200) and split products."""
    from tensor_transformer_mlp_03_amd.device import DeviceMLP
    M, H, F, t, store = case
    say(f"[full weights] M={M} H={H} F_i={F} t={t} store_p={store}")
    w = I.custom_workload(318, M=M, H=H, F_i=F, t=t, w_std=0.05)
    inp = I.make_inputs(w)
    a = DeviceMLP(inp, store_p=store, driver=True)
    b = DeviceMLP(inp, store_p=store, driver=True, full_weights=True)
    a.step()
    b.step()
    torch.cuda.synchronize()
    assert torch.equal(a.Z, b.Z) and torch.equal(a.dX, b.dX)
    for x, y in list(zip(a.dA, b.dA)) + list(zip(a.dB, b.dB)):
        assert torch.equal(x, y)
    if store:
        for x, y in zip(a.P, b.P):
            assert torch.equal(x, y)


def test_full_weights_oracle():
    """Whole-weight drivers against the oracle on the unsharded MLP: Z = GeLU(X A) B
    and its gradients, with dA and dB compared whole."""
    from tensor_transformer_mlp_03_amd.device import DeviceMLP
    M, H, F, t = 136, 520, 264, 4
    say(f"[full weights oracle] M={M} H={H} F_i={F} t={t}")
    w = I.custom_workload(319, M=M, H=H, F_i=F, t=t, w_std=0.05)
    inp = I.make_inputs(w)
    d = DeviceMLP(inp, store_p=False, driver=True, full_weights=True)
    d.step()
    torch.cuda.synchronize()
    X, dZ = dec(inp.X), dec(inp.dZ)
    A = np.concatenate([dec(a) for a in inp.A], 1)
    B = np.concatenate([dec(b) for b in inp.B], 0)
    fwd = O.mlp_forward(X, A, B)
    bwd = O.mlp_backward(dZ, X, A, B)
    r = {}
    check("Z", d.Z.cpu().numpy(), fwd["Z"], r)
    for name in ("dX", "dA", "dB"):
        got = {"dX": d.dX, "dA": d.dAf, "dB": d.dBf}[name]
        check(name, got.cpu().numpy(), bwd[name], r)
    say("  err/tol:", {k: round(v, 3) for k, v in r.items()})


@pytest.mark.parametrize("case", [(200, 264, 392, 3, True), (200, 192, 392, 2, False), (8, 64, 8, 2, True),
                                  (64, 256, 512, 2, True), (1024, 16640, 2056, 2, False),
                                  (1024, 16640, 1032, 2, True), (2048, 4096, 2048, 4, True)],
                         ids=lambda c: "x".join(map(str, c[:4])) + ("_store" if c[4] else "_recompute"))
def test_folded_sum_equals_separate_sum_bitwise(case):
    """Without per-shard partials the drivers add each shard's partial to Z and dX in
    its product's epilogue (or its split reduction); the float32 additions are those
    of the separate rank-order sum, so the bits are the same.  Covers the fused
    forward (one and several chunks), hybrid split products ([M, H] outputs with a
    split tail: H = 16640, F_i = 2056), split 256 x 128 products (F_i = 1032) and
    256 x 128 tiles at 7B-class shard shapes."""
    from tensor_transformer_mlp_03_amd.device import DeviceMLP
    M, H, F, t, store = case
    say(f"[folded sum] M={M} H={H} F_i={F} t={t} store_p={store}")
    w = I.custom_workload(320, M=M, H=H, F_i=F, t=t, w_std=0.05)
    inp = I.make_inputs(w)
    a = DeviceMLP(inp, store_p=store, driver=True, keep_partials=True)   # partials + separate sum
    b = DeviceMLP(inp, store_p=store, driver=True, keep_partials=False)  # folded
    c = DeviceMLP(inp, store_p=store, driver=True, full_weights=True)    # folded, whole weights
    for d in (a, b, c):
        d.step()
    torch.cuda.synchronize()
    for d in (b, c):
        assert torch.equal(a.Z, d.Z) and torch.equal(a.dX, d.dX)
    # and the sum is the sum of the partials, to float32 rounding of t - 1 additions
    Z = sum(z.double() for z in a.Z_sh)
    assert (a.Z.double() - Z).abs().max() <= t * 2.0 ** -23 * Z.abs().max()


@pytest.mark.parametrize("case", [(2048, 4096, 2048, 4, True), (2048, 4096, 2048, 3, False),
                                  (2048, 1024, 1024, 8, True)],
                         ids=lambda c: "x".join(map(str, c[:4])) + ("_store" if c[4] else "_recompute"))
def test_paired_products_equal_separate_sum_bitwise(case):
    """7B-class shard shapes: after a batched F1 (and dGeLU), two consecutive
    shards' F3 (and dX) run as one launch with two accumulator sets, adding into Z
    (dX) in rank order; the bits are those of the separate rank-order sum of the
    per-shard partials, and an odd shard count leaves one product unpaired."""
    from tensor_transformer_mlp_03_amd import _lib as L
    from tensor_transformer_mlp_03_amd.device import DeviceMLP
    M, H, F, t, store = case
    say(f"[paired products] M={M} H={H} F_i={F} t={t} store_p={store}")
    w = I.custom_workload(340 + t, M=M, H=H, F_i=F, t=t, w_std=0.05)
    inp = I.make_inputs(w)
    a = DeviceMLP(inp, store_p=store, driver=True, keep_partials=True)   # partials + separate sum
    b = DeviceMLP(inp, store_p=store, driver=True, keep_partials=False)  # folded, paired
    a.step()
    L.tpmlp_timing_begin(256)
    b.step()
    stats, dropped = L.tpmlp_timing_end()
    torch.cuda.synchronize()
    assert dropped == 0
    assert stats["fwd_gemm1_gelu"][0] < t, "the shapes batch F1"
    assert stats["fwd_gemm2"][0] == (t + 1) // 2 and stats["bwd_dX"][0] == (t + 1) // 2, stats
    assert torch.equal(a.Z, b.Z) and torch.equal(a.dX, b.dX)
    for i in range(t):
        assert torch.equal(a.dA[i], b.dA[i]) and torch.equal(a.dB[i], b.dB[i]), f"shard {i}"


@pytest.mark.parametrize("shape", [(200, 192, 392, 2), (1000, 520, 776, 2)], ids=["fused_forward", "two_products"])
def test_graph_replay_matches_eager(shape):
    """A step captured into a HIP graph gives, on every replay, the bits of the eager
    step; between replays the outputs are overwritten by eager work and the
    program synchronises, so each replay recomputes them."""
    from tensor_transformer_mlp_03_amd.device import DeviceMLP
    M, H, F, t = shape
    say(f"[graph replay] M={M} H={H} F_i={F} t={t}")
    w = I.custom_workload(321, M=M, H=H, F_i=F, t=t, w_std=0.05)
    d = DeviceMLP(I.make_inputs(w), store_p=True, driver=True)
    d.step()
    torch.cuda.synchronize()
    outs = lambda: [d.Z, d.dX] + list(d.dA) + list(d.dB) + list(d.P)
    ref = [x.clone() for x in outs()]
    g = d.capture()
    for rep in range(3):
        for x in outs():
            x.fill_(float("nan") if x.dtype == torch.float32 else -1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(outs(), ref):
            assert torch.equal(x, y), f"replay {rep} differs"


SP_CASES = [
    # (M, H, F_i, t, store_p): rows per rank slice a multiple of 8, ragged tiles
    (528, 264, 392, 2, True),
    (1056, 520, 264, 4, False),
    (208, 192, 392, 2, True),      # fused small-H forward per slice
    (16400, 136, 520, 2, False),   # 8200-row slices: the forward transposes the weights
    (2048, 1032, 2056, 8, True),   # 256-row slices, split and hybrid products
]


@pytest.mark.parametrize("case", SP_CASES, ids=lambda c: "x".join(map(str, c[:4])) + ("_store" if c[4] else "_recompute"))
def test_sequence_parallel_boundary(case):
    """tpmlp_sp_fwd / tpmlp_sp_bwd take every rank's token rows as a separate
    slice and return every rank's rows of Z and dX: rank r's output slice must be
    rows [r S, (r+1) S) of sum_i GeLU(X A_i) B_i (the reduce-scatter of the
    shards' partials), its dX slice the same rows of sum_i dX_i, and dA_i, dB_i the
    shard gradients over all tokens.  Each slice is its own allocation with a
    canary band on both sides.  The results also match the t-shard driver's on
    the gathered X within the tolerance."""
    from tensor_transformer_mlp_03_amd import _lib as L
    from tensor_transformer_mlp_03_amd.device import DeviceMLP, to_device
    M, H, F, t, store = case
    S = M // t
    say(f"[sp boundary] M={M} H={H} F_i={F} t={t} ({S} rows per rank) store_p={store}")
    w = I.custom_workload(350 + t, M=M, H=H, F_i=F, t=t, w_std=0.05)
    inp = I.make_inputs(w)
    bufs = []

    def slice_buf(n, dtype, src=None):
        fill = float("nan") if dtype == torch.float32 else -12345
        buf = torch.full((n + 2 * PAD,), fill, dtype=dtype, device="cuda")
        v = buf[PAD:PAD + n]
        if src is not None:
            v.copy_(src.reshape(-1))
        bufs.append((buf, n))
        return v

    Xd, dZd = to_device(inp.X), to_device(inp.dZ)
    X_sl = [slice_buf(S * H, torch.int16, Xd[r * S:(r + 1) * S]).view(S, H) for r in range(t)]
    dZ_sl = [slice_buf(S * H, torch.int16, dZd[r * S:(r + 1) * S]).view(S, H) for r in range(t)]
    Z_sl = [slice_buf(S * H, torch.float32).view(S, H) for _ in range(t)]
    dX_sl = [slice_buf(S * H, torch.float32).view(S, H) for _ in range(t)]
    A = [to_device(a) for a in inp.A]
    B = [to_device(b) for b in inp.B]
    P = [torch.empty((M, F), dtype=torch.int16, device="cuda") for _ in range(t)] if store else None
    dA = [torch.empty((H, F), dtype=torch.float32, device="cuda") for _ in range(t)]
    dB = [torch.empty((F, H), dtype=torch.float32, device="cuda") for _ in range(t)]
    ws = torch.empty(L.tpmlp_sp_workspace_bytes(t, M, H, F), dtype=torch.uint8, device="cuda")
    L.tpmlp_sp_fwd(X_sl, A, B, P, Z_sl, ws)
    L.tpmlp_sp_bwd(dZ_sl, X_sl, A, B, P, dA, dB, dX_sl, ws)
    torch.cuda.synchronize()
    for buf, n in bufs:
        _canary_intact(buf, n, "slice") if buf.dtype == torch.float32 else None
        if buf.dtype == torch.int16:
            assert bool((buf[:PAD] == -12345).all()) and bool((buf[PAD + n:] == -12345).all())
    Xo, dZo = dec(inp.X), dec(inp.dZ)
    Ao, Bo = [dec(a) for a in inp.A], [dec(b) for b in inp.B]
    Z, _ = O.tp_forward(Xo, Ao, Bo)
    dX, _, dAo, dBo = O.tp_backward(dZo, Xo, Ao, Bo)
    r_ = {}
    for r in range(t):
        check(f"Z_sl[{r}]", Z_sl[r].cpu().numpy(), Z[r * S:(r + 1) * S], r_)
        check(f"dX_sl[{r}]", dX_sl[r].cpu().numpy(), dX[r * S:(r + 1) * S], r_)
    for i in range(t):
        check(f"dA_{i}", dA[i].cpu().numpy(), dAo[i], r_)
        check(f"dB_{i}", dB[i].cpu().numpy(), dBo[i], r_)
    # the t-shard driver on the gathered tokens gives the same outputs within tolerance
    d = DeviceMLP(inp, store_p=store, driver=True)
    d.step()
    torch.cuda.synchronize()
    check_dev("Z_sl_vs_driver", torch.cat(Z_sl, 0), d.Z, r_)
    check_dev("dX_sl_vs_driver", torch.cat(dX_sl, 0), d.dX, r_)
    say("  err/tol:", {k: round(v, 3) for k, v in r_.items()})


def test_deterministic():
    w = I.custom_workload(311, M=768, H=1024, F_i=1536, t=2)
    say(f"[determinism] {w}")
    inp = I.make_inputs(w)
    a, b = run_device(inp), run_device(inp)
    assert torch.equal(a.Z, b.Z) and torch.equal(a.dX, b.dX)
    for x, y in list(zip(a.dA, b.dA)) + list(zip(a.dB, b.dB)):
        assert torch.equal(x, y)


def test_zero_input_gives_exact_zeros():
    """X = 0: P = 0 and GeLU(0) = 0, so Z, dA and dB are exactly zero."""
    w = I.custom_workload(312, M=264, H=256, F_i=384, t=2)
    inp = I.make_inputs(w)
    inp.X[:] = 0
    d = run_device(inp)
    assert torch.count_nonzero(d.Z) == 0
    for x in d.dA + d.dB:
        assert torch.count_nonzero(x) == 0
    # dX = 1/2 dZ B^T A^T per shard, summed
    X, dZ = dec(inp.X), dec(inp.dZ)
    ref = sum(0.5 * (dZ @ dec(b).T) @ dec(a).T for a, b in zip(inp.A, inp.B))
    r = {}
    check("dX", d.dX.cpu().numpy(), ref, r)


CANARY_F32 = float("nan")
CANARY_I16 = -12345
CANARY_U8 = 77
PAD = 4096  # canary elements on each side of every output


def _padded(n, dtype):
    """A buffer of n + 2 PAD elements filled with the canary, and its middle n."""
    fill = CANARY_F32 if dtype == torch.float32 else CANARY_I16 if dtype == torch.int16 else CANARY_U8
    buf = torch.full((n + 2 * PAD,), fill, dtype=dtype, device="cuda")
    return buf, buf[PAD:PAD + n]


def _canary_intact(buf, n, name):
    lo, hi = buf[:PAD], buf[PAD + n:]
    if buf.dtype == torch.float32:
        ok = bool(torch.isnan(lo).all()) and bool(torch.isnan(hi).all())
        assert bool(torch.isfinite(buf[PAD:PAD + n]).all()), f"{name}: unwritten or non-finite values inside"
    else:
        fill = CANARY_I16 if buf.dtype == torch.int16 else CANARY_U8
        ok = bool((lo == fill).all()) and bool((hi == fill).all())
    assert ok, f"{name}: a write landed outside the buffer"


CANARY_CASES = [
    # (M, H, F_i, t, store_p, mode): mode "rank" = tpmlp_fwd/tpmlp_bwd per shard,
    # "driver" = t-shard driver with the sums folded into the products, "whole" =
    # the whole-weight driver (A_i, dA_i strided column views)
    (136, 264, 200, 1, True, "rank"),        # plain ragged products, unsplit
    (1024, 2056, 16640, 1, True, "rank"),    # [M, F_i] products as whole waves + split tail (GeLU, dGeLU)
    (1024, 16640, 2056, 1, False, "rank"),   # [M, H] products as whole waves + split tail (float32, dX)
    (200, 192, 392, 1, True, "rank"),        # fused small-H forward: chunk partials, P_save from the fused kernel
    (200, 264, 392, 3, True, "driver"),      # folded sums: shards 1, 2 add into Z and dX in their epilogues
    (1024, 16640, 1032, 2, False, "driver"), # folded sums in split reductions
    (200, 264, 392, 3, True, "whole"),       # strided column blocks of A, P, dA
    (1024, 1032, 2056, 2, True, "whole"),    # the same with 256 x 128 tiles and splits
]


@pytest.mark.parametrize("case", CANARY_CASES, ids=lambda c: "x".join(map(str, c[:4])) + "_" + c[5])
def test_no_writes_outside_outputs(case):
    """Every output and the workspace sit inside larger buffers filled with a
    canary; after a forward and backward the canary bands are untouched and the
    outputs are finite.  For the whole-weight driver, shard i's column blocks of
    P, dA and dB sit between other shards' blocks: the results must also equal,
    bit for bit, those of the per-shard driver on separate buffers, so a shard
    that wrote into an earlier shard's block would show there (a write into a
    later block is overwritten by that shard, but every shard runs the same code
    with a different base, and the last shard's overrun would hit the canary or
    the next row's first block)."""
    from tensor_transformer_mlp_03_amd import _lib as L
    from tensor_transformer_mlp_03_amd.device import DeviceMLP, to_device
    M, H, F, t, store, mode = case
    say(f"[canary] M={M} H={H} F_i={F} t={t} store_p={store} {mode}")
    w = I.custom_workload(313, M=M, H=H, F_i=F, t=t, w_std=0.05)
    inp = I.make_inputs(w)
    X, dZ = to_device(inp.X), to_device(inp.dZ)
    A = [to_device(a) for a in inp.A]
    B = [to_device(b) for b in inp.B]
    bufs = []

    def out(n, dtype, name, shape):
        buf, v = _padded(n, dtype)
        bufs.append((buf, n, name))
        return v.view(*shape)

    f32, i16 = torch.float32, torch.int16
    if mode == "rank":
        wsn = max(L.tpmlp_fwd_workspace_bytes(M, H, F), L.tpmlp_bwd_workspace_bytes(M, H, F, not store))
        ws = out(wsn, torch.uint8, "ws", (wsn,))
        for i in range(t):
            Z = out(M * H, f32, f"Z_{i}", (M, H))
            P = out(M * F, i16, f"P_{i}", (M, F)) if store else None
            dX = out(M * H, f32, f"dX_{i}", (M, H))
            dA = out(H * F, f32, f"dA_{i}", (H, F))
            dB = out(F * H, f32, f"dB_{i}", (F, H))
            L.tpmlp_fwd(X, A[i], B[i], Z, P, ws)
            L.tpmlp_bwd(dZ, X, A[i], B[i], P, dX, dA, dB, ws)
    elif mode == "driver":
        wsn = L.tpmlp_tp_workspace_bytes(t, M, H, F)
        ws = out(wsn, torch.uint8, "ws", (wsn,))
        Z, dX = out(M * H, f32, "Z", (M, H)), out(M * H, f32, "dX", (M, H))
        P = [out(M * F, i16, f"P_{i}", (M, F)) for i in range(t)] if store else None
        dA = [out(H * F, f32, f"dA_{i}", (H, F)) for i in range(t)]
        dB = [out(F * H, f32, f"dB_{i}", (F, H)) for i in range(t)]
        L.tpmlp_tp_fwd(X, A, B, P, None, Z, ws)
        L.tpmlp_tp_bwd(dZ, X, A, B, P, dA, dB, None, dX, ws)
    else:
        wsn = L.tpmlp_tp_workspace_bytes(t, M, H, F)
        ws = out(wsn, torch.uint8, "ws", (wsn,))
        Af, Bf = torch.cat(A, 1).contiguous(), torch.cat(B, 0).contiguous()
        Z, dX = out(M * H, f32, "Z", (M, H)), out(M * H, f32, "dX", (M, H))
        P = out(t * M * F, i16, "P", (t, M, F)) if store else None
        dA = out(H * t * F, f32, "dA", (H, t * F))
        dB = out(t * F * H, f32, "dB", (t * F, H))
        L.tpmlp_tp_fwd_full(X, Af, Bf, P, Z, t, ws)
        L.tpmlp_tp_bwd_full(dZ, X, Af, Bf, P, dA, dB, dX, t, ws)
        ref = DeviceMLP(inp, store_p=store, driver=True)
        ref.step()
        torch.cuda.synchronize()
        assert torch.equal(Z, ref.Z) and torch.equal(dX, ref.dX)
        for i in range(t):
            assert torch.equal(dA[:, i * F:(i + 1) * F], ref.dA[i]), f"dA block {i}"
            assert torch.equal(dB[i * F:(i + 1) * F], ref.dB[i]), f"dB block {i}"
            if store:
                assert torch.equal(P[i], ref.P[i]), f"P block {i}"
    torch.cuda.synchronize()
    for buf, n, name in bufs:
        if name == "ws":
            fill_ok = bool((buf[:PAD] == CANARY_U8).all()) and bool((buf[PAD + n:] == CANARY_U8).all())
            assert fill_ok, "workspace: a write landed outside it"
        else:
            _canary_intact(buf, n, name)


def test_shard_sum_kernel_exact():
    from tensor_transformer_mlp_03_amd import _lib as L
    rng = np.random.default_rng(5)
    n, t = 3 * 1024 * 1024 + 12, 5
    parts = [rng.standard_normal(n).astype(np.float32) for _ in range(t)]
    want = parts[0].copy()
    for p in parts[1:]:
        want = want + p  # float32, left to right
    dev = [torch.from_numpy(p).cuda() for p in parts]
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    L.tpmlp_shard_sum(dev, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), want)


def test_timing_counts_launches():
    from tensor_transformer_mlp_03_amd import _lib as L
    w = I.custom_workload(314, M=256, H=264, F_i=256, t=2)
    inp = I.make_inputs(w)
    from tensor_transformer_mlp_03_amd.device import DeviceMLP
    d = DeviceMLP(inp, store_p=True, driver=True)
    L.tpmlp_timing_begin(64)
    d.step()
    stats, dropped = L.tpmlp_timing_end()
    assert dropped == 0
    # F1 and dGeLU of the two shards: one launch each, or one batched launch for both;
    # F3 and dX: one launch each, or (after a batched F1 or dGeLU) one paired launch
    n1 = stats["fwd_gemm1_gelu"][0]
    assert n1 in (1, 2) and stats["bwd_dgelu"][0] == n1
    n3 = stats["fwd_gemm2"][0]
    assert n3 in ((1, 2) if n1 == 1 else (2,))
    # no per-shard partials asked for: the sums are folded into the products' epilogues
    assert stats["bwd_dX"][0] == n3 and stats["shard_sum"][0] == 0
    assert stats["bwd_recompute"][0] == 0
    assert stats["transpose"][0] == 1  # X^T and dZ^T in one launch, once for both shards
    assert all(ms >= 0 for _, ms in stats.values())
    recs = L.tpmlp_timing_records()
    assert len(recs) == sum(n for n, _ in stats.values()) and all(ms > 0 for _, ms in recs)
    # Only the chosen kind is timed; every other launch runs as with timing off.
    L.tpmlp_timing_begin_kinds(64, ["fwd_gemm2"])
    d.step()
    stats, dropped = L.tpmlp_timing_end()
    assert dropped == 0
    assert {k: n for k, (n, _) in stats.items() if n} == {"fwd_gemm2": n3}
    assert [k for k, _ in L.tpmlp_timing_records()] == ["fwd_gemm2"] * n3
    assert L.tpmlp_timing_dispatches() == [1] * n3


@pytest.mark.parametrize("case", [(512, 1024, 512, 4, True), (640, 1032, 520, 3, False)],
                         ids=lambda c: "x".join(map(str, c[:4])) + ("_store" if c[4] else "_recompute"))
def test_batched_shards_equal_rank_calls_bitwise(case):
    """Short-K shapes: the t-shard driver runs several shards' F1 (and the
    recompute and dGeLU) as one batched launch.  Each product stays unsplit, so
    every shard's P_i, Z_i, dX_i, dA_i and dB_i have the bits of that rank's own
    tpmlp_fwd / tpmlp_bwd calls.  With M = F_i a rank's call runs its dB_i and dX_i
    as one launch, while the driver batches the shards' dB instead: the two ways
    give the same bits too."""
    from tensor_transformer_mlp_03_amd import _lib as L
    from tensor_transformer_mlp_03_amd.device import DeviceMLP
    M, H, F_, t, store = case
    say(f"[batched shards] M={M} H={H} F_i={F_} t={t} store_p={store}")
    w = I.custom_workload(330 + t, M=M, H=H, F_i=F_, t=t)
    inp = I.make_inputs(w)
    drv = DeviceMLP(inp, store_p=store, driver=True, keep_partials=True)
    L.tpmlp_timing_begin(256)
    drv.step()
    stats, _ = L.tpmlp_timing_end()
    assert stats["fwd_gemm1_gelu"][0] < t and stats["bwd_dgelu"][0] < t, stats  # batched
    rank = DeviceMLP(inp, store_p=store, driver=False)
    L.tpmlp_timing_begin(256)
    rank.step()
    stats, _ = L.tpmlp_timing_end()
    torch.cuda.synchronize()
    if M == F_:  # each rank's dB_i and dX_i share one launch; the driver batched dB instead
        assert stats["bwd_dB_dX"][0] == t and stats["bwd_dB"][0] == 0 and stats["bwd_dX"][0] == 0, stats
    for i in range(t):
        assert torch.equal(drv.Z_sh[i], rank.Z_sh[i]), f"Z_{i}"
        assert torch.equal(drv.dX_sh[i], rank.dX_sh[i]), f"dX_{i}"
        assert torch.equal(drv.dA[i], rank.dA[i]) and torch.equal(drv.dB[i], rank.dB[i]), f"dA_{i} / dB_{i}"
        if store:
            assert torch.equal(drv.P[i], rank.P[i]), f"P_{i}"


@pytest.mark.parametrize("shape", [(64, 256, 512), (200, 192, 392), (8, 64, 8)])
def test_fused_forward_is_taken(shape):
    """Small hidden sizes run the forward as one fused launch per shard (plus the
    chunk sum when F_i spans more than one chunk of 64), never the two products."""
    from tensor_transformer_mlp_03_amd import _lib as L
    from tensor_transformer_mlp_03_amd.device import DeviceMLP
    M, H, F = shape
    say(f"[fused taken] M={M} H={H} F_i={F}")
    w = I.custom_workload(316, M=M, H=H, F_i=F, t=2)
    d = DeviceMLP(I.make_inputs(w), store_p=True, driver=True)
    L.tpmlp_timing_begin(64)
    d.forward()
    stats, dropped = L.tpmlp_timing_end()
    assert dropped == 0
    counts = {k: n for k, (n, _) in stats.items() if n}
    # Shard 1's chunk sum also adds its partial to Z (no separate shard sum); with
    # a single chunk, shard 0 writes Z from the fused kernel itself.
    want = {"fwd_fused": 2, "splitk_reduce": 2 if F > 64 else 1}
    assert counts == want


def test_fused_forward_pre_activation():
    """P_save written by the fused kernel is X A_i rounded once to bf16: within half
    a bf16 ulp of the float64 product, plus float32 accumulation error."""
    M, H, F = 136, 256, 520
    say(f"[fused P_save] M={M} H={H} F_i={F}")
    w = I.custom_workload(317, M=M, H=H, F_i=F, t=1)
    inp = I.make_inputs(w)
    d = run_device(inp, store_p=True)
    P = O.decode_bf16(d.P[0].cpu().numpy().view(np.uint16))
    ref = dec(inp.X) @ dec(inp.A[0])
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * np.abs(ref).max()
    assert np.all(np.abs(P - ref) <= bound)


def test_timing_spans_hybrid_dispatches():
    """A product planned as whole-wave tiles plus a split tail is one timing record
    of two kernel dispatches, with a positive duration."""
    from tensor_transformer_mlp_03_amd import _lib as L
    from tensor_transformer_mlp_03_amd.device import DeviceMLP
    w = I.custom_workload(315, M=1024, H=2056, F_i=16640, t=1)
    say(f"[timing hybrid] M={w.M} H={w.H} F_i={w.F_i}")
    d = DeviceMLP(I.make_inputs(w), store_p=True, driver=True)
    L.tpmlp_timing_begin(64)
    d.step()
    L.tpmlp_timing_end()
    recs, disp = L.tpmlp_timing_records(), L.tpmlp_timing_dispatches()
    assert len(recs) == len(disp) and set(disp) <= {1, 2} and 2 in disp
    assert all(ms > 0 for _, ms in recs)


@pytest.mark.parametrize("M", [4096, 65536])
def test_gelu_epilogue_values(M):
    """With A = B = I the forward's Z is exactly bf16(GeLU(X)) and, for dZ = 1, the
    backward's dX is exactly bf16(GeLU'(X)): every finite bf16 value in [-12, 12]
    is compared with float64 GeLU within one bf16 unit in the last place.  M picks
    the 128x128 (4096) and the 256x256 (65536) tile."""
    from tensor_transformer_mlp_03_amd.device import DeviceMLP
    HF = 256
    say(f"[gelu epilogue] M={M} H=F={HF}")
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = O.decode_bf16(allb)
    keep = np.isfinite(vals) & (np.abs(vals) <= 12.0)
    xs = allb[keep]
    X = np.resize(xs, M * HF).reshape(M, HF)
    eye = I.f32_to_bf16_bits(np.eye(HF, dtype=np.float32))
    w = I.custom_workload(320, M=M, H=HF, F_i=HF, t=1)
    ones = I.f32_to_bf16_bits(np.ones((M, HF), dtype=np.float32))
    inp = I.Inputs(w, X, [eye], [eye], ones)
    d = run_device(inp, store_p=True, keep_partials=False)
    x = dec(X)

    def ulps(got_f32, want_f64):
        want = I.f32_to_bf16_bits(want_f64.astype(np.float32)).astype(np.int32)
        got = I.f32_to_bf16_bits(got_f32.astype(np.float32)).astype(np.int32)
        # order-preserving integer map of bf16 bit patterns
        key = lambda b: np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
        return np.abs(key(got) - key(want))

    z = d.Z.cpu().numpy()
    dx = d.dX.cpu().numpy()
    assert np.all(z == I.bf16_bits_to_f32(I.f32_to_bf16_bits(z))), "Z must be bf16 values"
    for name, got, want in (("GeLU", z, O.gelu(x)), ("GeLU'", dx, O.gelu_grad(x))):
        u = ulps(got, want)
        # within one bf16 ulp, or (far tail) within the erf approximation's
        # absolute bound 1.5e-7 carried through p * Phi(p) and phi(p)
        ok = (u <= 1) | (np.abs(got - want) <= 2e-7 * (1 + np.abs(x)))
        say(f"  {name}: max {u.max()} ulp, exact {np.mean(u == 0):.5f}, outside bound {np.sum(~ok)}")
        assert ok.all() and np.mean(u == 0) > 0.99
