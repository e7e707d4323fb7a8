"""The FP8 path on the GPU (through the C ABI) against the FP8 oracle (oracle/fp8.py).

* Quantization: the codes and the amax of tpmlp_fp8_quantize equal the oracle's,
  byte for byte, for both formats, row-major and transposed (the codes are integer
  decisions taken in float32 on both sides).
* The t-shard FP8 forward and backward: Z, dX, dA_i, dB_i against the oracle's
  FP8 path, element by element, within the bound of tests/fp8_bound.py (the bf16
  path's rule plus the moves of the FP8 codes that float32 accumulation can
  legitimately decide otherwise), and each stored bf16 P_i inside the interval of
  admissible roundings that bound assumes.
"""
import sys

import numpy as np
import pytest

import fp8_bound as FB
import margins
from oracle import fp8 as F
from oracle import oracle as O
from tensor_transformer_mlp_03_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tensor_transformer_mlp_03_amd import _lib as L
    L.lib()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check(name, got, ref, tol, ratios):
    """Element-wise: |got - ref| <= tol (an array of ref's shape)."""
    ratio, where = FB.worst_ratio(got, ref, tol)
    ratios[name] = ratio
    margins.record(name, ratio)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert ratio <= 1.0, (f"{name}: |err| / tol = {ratio:.3f} at {where}: got {float(got[where]):.6g}, "
                          f"oracle {float(ref[where]):.6g}, tol {float(tol[where]):.3g}")


def _bf16_bits(x):
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    return (((b + 0x7FFF + ((b >> 16) & 1)) >> 16) & 0xFFFF).astype(np.uint16)


@pytest.mark.parametrize("shape", [(272, 400), (16, 16), (1040, 64)], ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("fmt", [0, 1], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("transpose", [False, True], ids=["rows", "transposed"])
def test_fp8_quantize_matches_oracle_bytes(shape, fmt, transpose):
    from tensor_transformer_mlp_03_amd import _lib as L
    R, C = shape
    say(f"[fp8 quantize] {R}x{C} fmt={fmt} transpose={transpose}")
    rng = np.random.default_rng(1000 + R + 7 * fmt)
    # a wide spread of magnitudes (codes deep in the subnormals), exact and signed zeros
    x = rng.standard_normal((R, C)) * np.exp2(rng.integers(-14, 3, (R, C)))
    x[rng.random((R, C)) < 0.02] = 0.0
    x[rng.random((R, C)) < 0.02] = -0.0
    bits = _bf16_bits(x)
    T32 = O.decode_bf16(bits).astype(np.float32)
    ref_codes, ref_s = F.quantize(T32, F.E4M3 if fmt == 0 else F.E5M2)
    Td = torch.from_numpy(bits.view(np.int16)).cuda()
    codes = torch.empty((C, R) if transpose else (R, C), dtype=torch.uint8, device="cuda")
    amax = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    L.tpmlp_fp8_quantize(Td, fmt, transpose, codes, amax)
    torch.cuda.synchronize()
    got = codes.cpu().numpy()
    if transpose:
        got = got.T
    assert amax.item() == float(np.max(np.abs(T32)))
    diff = int((got != ref_codes).sum())
    assert diff == 0, f"{diff} codes differ, e.g. {np.argwhere(got != ref_codes)[:3].tolist()}"


FP8_CASES = [
    # (M, H, F_i, t, store_p): multiples of 16, ragged against the 128 / 256 tiles
    (96, 64, 48, 1, True),
    (256, 192, 320, 2, True),
    (528, 272, 400, 2, False),
    (1040, 1056, 1072, 1, True),
    (2048, 1024, 2048, 2, False),  # 256-row tiles, long K for dB / dA
    (8192, 256, 512, 1, True),     # K = 8192 for dB / dA: split-K slices
    (272, 144, 176, 8, False),     # eight shards: eight sets of codes and scales, sums in rank order
]


@pytest.mark.parametrize("case", FP8_CASES,
                         ids=lambda c: "x".join(map(str, c[:4])) + ("_store" if c[4] else "_recompute"))
def test_fp8_path_matches_oracle(case):
    from tensor_transformer_mlp_03_amd import _lib as L
    from tensor_transformer_mlp_03_amd.device import to_device
    M, H, F_, t, store = case
    say(f"[fp8 path] M={M} H={H} F_i={F_} t={t} store_p={store}")
    w = I.custom_workload(400 + t, M=M, H=H, F_i=F_, t=t, w_std=0.05)
    inp = I.make_inputs(w)
    X, dZ = to_device(inp.X), to_device(inp.dZ)
    A = [to_device(a) for a in inp.A]
    B = [to_device(b) for b in inp.B]
    P = [torch.empty((M, F_), dtype=torch.int16, device="cuda") for _ in range(t)] if store else None
    Z = torch.empty((M, H), dtype=torch.float32, device="cuda")
    dX = torch.empty((M, H), dtype=torch.float32, device="cuda")
    dA = [torch.empty((H, F_), dtype=torch.float32, device="cuda") for _ in range(t)]
    dB = [torch.empty((F_, H), dtype=torch.float32, device="cuda") for _ in range(t)]
    ws = torch.empty(L.tpmlp_fp8_workspace_bytes(t, M, H, F_), dtype=torch.uint8, device="cuda")
    L.tpmlp_fp8_tp_fwd(X, A, B, P, Z, ws)
    L.tpmlp_fp8_tp_bwd(dZ, X, A, B, P, dA, dB, dX, ws)
    torch.cuda.synchronize()
    Xo, dZo = O.decode_bf16(inp.X), O.decode_bf16(inp.dZ)
    Ao, Bo = [O.decode_bf16(a) for a in inp.A], [O.decode_bf16(b) for b in inp.B]
    bd = FB.path_bounds(Xo, Ao, Bo, dZo)
    r = {}
    check("Z", Z.cpu().numpy(), bd.Z, bd.tol_Z, r)
    check("dX", dX.cpu().numpy(), bd.dX, bd.tol_dX, r)
    for i in range(t):
        check(f"dA_{i}", dA[i].cpu().numpy(), bd.dA[i], bd.tol_dA[i], r)
        check(f"dB_{i}", dB[i].cpu().numpy(), bd.dB[i], bd.tol_dB[i], r)
        if store:
            Pg = O.decode_bf16(P[i].cpu().numpy().view(np.uint16))
            sh = bd.shards[i]
            outside = int(np.count_nonzero((Pg < sh.p_lo) | (Pg > sh.p_hi)))
            assert outside == 0, f"P_{i}: {outside} values outside the admissible roundings"
            r[f"P_{i} != oracle"] = int(np.count_nonzero(Pg != sh.fwd["P"]))
    say("  err/tol:", {k: round(v, 3) for k, v in r.items()},
        f"ambiguous codes G {bd.ambiguous_g} dP {bd.ambiguous_dp}")


def _random_fp8_cases(n, seed):
    """Seeded FP8 shapes: M, H, F_i multiples of 16 up to ~700 (some below one
    epilogue chunk), t of 1-3, P kept or recomputed."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M, H, F_ = (int(16 * rng.integers(1, 44)) for _ in range(3))
        out.append((M, H, F_, int(rng.integers(1, 4)), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("case", _random_fp8_cases(12, 2027),
                         ids=lambda c: "x".join(map(str, c[:4])) + ("_store" if c[4] else "_recompute"))
def test_fp8_random_shapes(case):
    """The FP8 forward and backward on random ragged shapes against the oracle's
    FP8 path, element by element within the acceptance bound."""
    test_fp8_path_matches_oracle(case)


def test_fp8_backward_needs_its_forward():
    """The backward reuses what the forward left in the workspace, and refuses a
    workspace that holds no forward of its inputs (before any launch); a
    backward that recomputes P_i after a forward that stored it is allowed and
    matches the oracle."""
    from tensor_transformer_mlp_03_amd import _lib as L
    from tensor_transformer_mlp_03_amd.device import to_device
    M, H, F_, t = 96, 64, 48, 2
    say(f"[fp8 forward state] M={M} H={H} F_i={F_} t={t}")
    w = I.custom_workload(450, M=M, H=H, F_i=F_, t=t, w_std=0.05)
    inp = I.make_inputs(w)
    X, dZ = to_device(inp.X), to_device(inp.dZ)
    A = [to_device(a) for a in inp.A]
    B = [to_device(b) for b in inp.B]
    P = [torch.empty((M, F_), dtype=torch.int16, device="cuda") for _ in range(t)]
    Z = torch.empty((M, H), dtype=torch.float32, device="cuda")
    dX = torch.empty((M, H), dtype=torch.float32, device="cuda")
    dA = [torch.empty((H, F_), dtype=torch.float32, device="cuda") for _ in range(t)]
    dB = [torch.empty((F_, H), dtype=torch.float32, device="cuda") for _ in range(t)]
    nbytes = L.tpmlp_fp8_workspace_bytes(t, M, H, F_)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def refused(fn):
        with pytest.raises(L.TpmlpError) as e:
            fn()
        assert e.value.status == 9, str(e.value)

    refused(lambda: L.tpmlp_fp8_tp_bwd(dZ, X, A, B, P, dA, dB, dX, ws2))  # nothing ran on ws2
    L.tpmlp_fp8_tp_fwd(X, A, B, P, Z, ws)
    X2 = X.clone()
    refused(lambda: L.tpmlp_fp8_tp_bwd(dZ, X2, A, B, P, dA, dB, dX, ws))          # another X
    refused(lambda: L.tpmlp_fp8_tp_bwd(dZ, X, A, B, P[::-1], dA, dB, dX, ws))     # P_sh not the forward's
    refused(lambda: L.tpmlp_fp8_tp_bwd(dZ, X, A, B, P, dA, dB, dX, ws2))          # another workspace
    # recompute after a storing forward: the check passes and the result is the oracle's
    L.tpmlp_fp8_tp_bwd(dZ, X, A, B, None, dA, dB, dX, ws)
    torch.cuda.synchronize()
    Xo, dZo = O.decode_bf16(inp.X), O.decode_bf16(inp.dZ)
    Ao, Bo = [O.decode_bf16(a) for a in inp.A], [O.decode_bf16(b) for b in inp.B]
    bd = FB.path_bounds(Xo, Ao, Bo, dZo)
    r = {}
    check("dX", dX.cpu().numpy(), bd.dX, bd.tol_dX, r)
    for i in range(t):
        check(f"dA_{i}", dA[i].cpu().numpy(), bd.dA[i], bd.tol_dA[i], r)
        check(f"dB_{i}", dB[i].cpu().numpy(), bd.dB[i], bd.tol_dB[i], r)
    # a second forward with other inputs on the same workspace replaces the first
    L.tpmlp_fp8_tp_fwd(X2, A, B, None, Z, ws)
    refused(lambda: L.tpmlp_fp8_tp_bwd(dZ, X, A, B, None, dA, dB, dX, ws))
    refused(lambda: L.tpmlp_fp8_tp_bwd(dZ, X2, A, B, P, dA, dB, dX, ws))         # it stored no P_i
    L.tpmlp_fp8_tp_bwd(dZ, X2, A, B, None, dA, dB, dX, ws)
    torch.cuda.synchronize()
    say("  err/tol:", {k: round(v, 3) for k, v in r.items()})


FP8_CANARY_CASES = [
    (528, 272, 400, 2, True),   # ragged against every tile shape
    (8192, 256, 512, 1, True),  # split-K weight gradients
    (272, 144, 176, 2, False),  # recomputed P_i
]


@pytest.mark.parametrize("case", FP8_CANARY_CASES,
                         ids=lambda c: "x".join(map(str, c[:4])) + ("_store" if c[4] else "_recompute"))
def test_fp8_no_writes_outside_outputs(case):
    """Every output and the workspace sit inside a larger allocation whose bands
    before and after hold a byte pattern; a forward and backward leave the bands
    unchanged."""
    from tensor_transformer_mlp_03_amd import _lib as L
    from tensor_transformer_mlp_03_amd.device import to_device
    M, H, F_, t, store = case
    say(f"[fp8 canary] M={M} H={H} F_i={F_} t={t} store_p={store}")
    w = I.custom_workload(470 + t, M=M, H=H, F_i=F_, t=t, w_std=0.05)
    inp = I.make_inputs(w)
    X, dZ = to_device(inp.X), to_device(inp.dZ)
    A = [to_device(a) for a in inp.A]
    B = [to_device(b) for b in inp.B]
    BAND = 4096  # bytes on each side, a multiple of 256
    bufs = []

    def banded(shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        raw = torch.full((n + 2 * BAND,), 0xA5, dtype=torch.uint8, device="cuda")
        bufs.append((raw, n))
        return raw[BAND:BAND + n].view(dtype).view(*shape)

    P = [banded((M, F_), torch.int16) for _ in range(t)] if store else None
    Z, dX = banded((M, H), torch.float32), banded((M, H), torch.float32)
    dA = [banded((H, F_), torch.float32) for _ in range(t)]
    dB = [banded((F_, H), torch.float32) for _ in range(t)]
    ws = banded((L.tpmlp_fp8_workspace_bytes(t, M, H, F_),), torch.uint8)
    L.tpmlp_fp8_tp_fwd(X, A, B, P, Z, ws)
    L.tpmlp_fp8_tp_bwd(dZ, X, A, B, P, dA, dB, dX, ws)
    torch.cuda.synchronize()
    for k, (raw, n) in enumerate(bufs):
        head, tail = raw[:BAND], raw[BAND + n:]
        assert bool((head == 0xA5).all()) and bool((tail == 0xA5).all()), f"buffer {k}: a band was written"
    assert torch.isfinite(Z).all() and torch.isfinite(dX).all()


FP8_SPLIT_CASES = [
    # (M, H, F_i, t, store_p, the first product's plan): F1 and dGeLU split along K
    (512, 4096, 2560, 1, True, "split"),      # 128 x 128 tiles, 3 K slices
    (256, 1536, 65552, 1, False, "hybrid"),   # 256 whole tiles + a 16-column split tail
]


@pytest.mark.parametrize("case", FP8_SPLIT_CASES, ids=lambda c: "x".join(map(str, c[:4])) + "_" + c[5])
def test_fp8_split_products_collect_amax(case):
    """F1 and dGeLU split along K (or as whole-wave tiles plus a split tail): the
    split-K reduction finishes the bf16 output and collects its amax (of GeLU(P_i)
    for F1, of dP_i for dGeLU), and the path matches the oracle.  The launch order
    shows that the split path ran."""
    from tensor_transformer_mlp_03_amd import _lib as L
    from tensor_transformer_mlp_03_amd.device import to_device
    M, H, F_, t, store, kind = case
    say(f"[fp8 split] M={M} H={H} F_i={F_} t={t} store_p={store} plan={kind}")
    w = I.custom_workload(480 + t, M=M, H=H, F_i=F_, t=t, w_std=0.05)
    inp = I.make_inputs(w)
    X, dZ = to_device(inp.X), to_device(inp.dZ)
    A = [to_device(a) for a in inp.A]
    B = [to_device(b) for b in inp.B]
    P = [torch.empty((M, F_), dtype=torch.int16, device="cuda") for _ in range(t)] if store else None
    Z = torch.empty((M, H), dtype=torch.float32, device="cuda")
    dX = torch.empty((M, H), dtype=torch.float32, device="cuda")
    dA = [torch.empty((H, F_), dtype=torch.float32, device="cuda") for _ in range(t)]
    dB = [torch.empty((F_, H), dtype=torch.float32, device="cuda") for _ in range(t)]
    ws = torch.empty(L.tpmlp_fp8_workspace_bytes(t, M, H, F_), dtype=torch.uint8, device="cuda")
    L.tpmlp_timing_begin(256)
    L.tpmlp_fp8_tp_fwd(X, A, B, P, Z, ws)
    L.tpmlp_fp8_tp_bwd(dZ, X, A, B, P, dA, dB, dX, ws)
    torch.cuda.synchronize()
    L.tpmlp_timing_end()
    recs = [k for k, _ in L.tpmlp_timing_records()]
    disp = L.tpmlp_timing_dispatches()
    for prod in ("fwd_gemm1_gelu", "bwd_dgelu"):
        at = [i for i, k in enumerate(recs) if k == prod]
        assert at and all(i + 1 < len(recs) and recs[i + 1] == "splitk_reduce" for i in at), (prod, recs)
        assert all(disp[i] == (2 if kind == "hybrid" else 1) for i in at), (prod, disp)
    Xo, dZo = O.decode_bf16(inp.X), O.decode_bf16(inp.dZ)
    Ao, Bo = [O.decode_bf16(a) for a in inp.A], [O.decode_bf16(b) for b in inp.B]
    bd = FB.path_bounds(Xo, Ao, Bo, dZo)
    r = {}
    check("Z", Z.cpu().numpy(), bd.Z, bd.tol_Z, r)
    check("dX", dX.cpu().numpy(), bd.dX, bd.tol_dX, r)
    for i in range(t):
        check(f"dA_{i}", dA[i].cpu().numpy(), bd.dA[i], bd.tol_dA[i], r)
        check(f"dB_{i}", dB[i].cpu().numpy(), bd.dB[i], bd.tol_dB[i], r)
        if store:
            Pg = O.decode_bf16(P[i].cpu().numpy().view(np.uint16))
            sh = bd.shards[i]
            assert int(np.count_nonzero((Pg < sh.p_lo) | (Pg > sh.p_hi))) == 0, f"P_{i} outside the admissible roundings"
    say("  err/tol:", {k: round(v, 3) for k, v in r.items()})


def test_fp8_long_context_chunk_sampled():
    """The FP8 path at the long-context chunk's full size (M=32768, H=3584,
    F_i=3584, t=4, P_i kept) in the launch configuration the benchmark times
    (DeviceFp8MLP: the t-shard driver over all four shards).  Rows of Z and dX
    in two classes, each with the R10 part of its tolerance from its own
    max|oracle|: two seeded rows from every 256-row tile of the rows that are
    not outliers, and 32 of the outlier rows (X scaled x8); columns of every
    dA_i and rows of every dB_i, two from every 256-wide block; the stored P_i on
    the sampled rows inside their admissible roundings.  The oracle's scales
    come from its full products (tests/fp8_bound.py, sampled_path_bounds)."""
    from tensor_transformer_mlp_03_amd.device import DeviceFp8MLP
    w = I.CONFIGS[3]
    say(f"[fp8 config3 sampled] {w}")
    inp = I.make_inputs(w)
    d = DeviceFp8MLP(inp, store_p=True)
    d.step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(1234 + 8)
    normal = []
    ex = np.zeros(w.M, dtype=bool)
    ex[np.asarray(inp.outliers)] = True
    for b0 in range(0, w.M, 256):
        cand = np.nonzero(~ex[b0:b0 + 256])[0] + b0
        normal.extend(rng.choice(cand, size=2, replace=False).tolist())
    normal = np.array(sorted(normal))
    outl = np.sort(rng.choice(inp.outliers, size=32, replace=False))
    rows = np.concatenate([normal, outl])
    cols = np.array(sorted(c for b0 in range(0, w.F_i, 256)
                           for c in rng.choice(np.arange(b0, min(b0 + 256, w.F_i)), 2, replace=False)))
    got = {"Z": d.Z[rows].cpu().numpy(), "dX": d.dX[rows].cpu().numpy(),
           "dA": [a[:, cols].cpu().numpy() for a in d.dA], "dB": [b[cols, :].cpu().numpy() for b in d.dB],
           "P": [O.decode_bf16(p[rows].cpu().numpy().view(np.uint16)) for p in d.P]}
    del d
    torch.cuda.empty_cache()
    X, dZ = O.decode_bf16(inp.X), O.decode_bf16(inp.dZ)
    A, B = [O.decode_bf16(a) for a in inp.A], [O.decode_bf16(b) for b in inp.B]
    del inp
    say(f"  {normal.size} normal rows, {outl.size} outlier rows, {cols.size} dA columns / dB rows; oracle ...")
    sb = FB.sampled_path_bounds(X, A, B, dZ, rows, cols)
    r = {}
    n = normal.size
    for cls, sl in (("normal", slice(0, n)), ("outlier", slice(n, None))):
        for name in ("Z", "dX"):
            ref = getattr(sb, name)[sl]
            moves = (getattr(sb, "tol_" + name) - O.tolerance(getattr(sb, name)))[sl]
            check(f"{name}[{cls}]", got[name][sl], ref, O.tolerance(ref) + moves, r)
    for i in range(w.t):
        check(f"dA_{i}[:,cols]", got["dA"][i], sb.dA[i], sb.tol_dA[i], r)
        check(f"dB_{i}[cols,:]", got["dB"][i], sb.dB[i], sb.tol_dB[i], r)
        outside = int(np.count_nonzero((got["P"][i] < sb.p_lo[i]) | (got["P"][i] > sb.p_hi[i])))
        assert outside == 0, f"P_{i}: {outside} sampled values outside the admissible roundings"
    say("  err/tol:", {k: round(v, 3) for k, v in r.items()})


@pytest.mark.parametrize("case", [(528, 272, 400, 2), (512, 4096, 2560, 1)], ids=lambda c: "x".join(map(str, c)))
def test_fp8_store_equals_recompute_bitwise(case):
    """The FP8 backward gives the same bits whether it takes the stored P_i or
    recomputes it: the recompute is the forward's product on the forward's codes
    and plan, its amax is the same, and G_i^T's codes come out the same."""
    from tensor_transformer_mlp_03_amd.device import DeviceFp8MLP
    M, H, F_, t = case
    say(f"[fp8 store vs recompute] M={M} H={H} F_i={F_} t={t}")
    inp = I.make_inputs(I.custom_workload(490 + t, M=M, H=H, F_i=F_, t=t, w_std=0.05))
    st, rc = DeviceFp8MLP(inp, store_p=True), DeviceFp8MLP(inp, store_p=False)
    st.step()
    rc.step()
    torch.cuda.synchronize()
    assert torch.equal(st.Z, rc.Z) and torch.equal(st.dX, rc.dX)
    for i in range(t):
        assert torch.equal(st.dA[i], rc.dA[i]) and torch.equal(st.dB[i], rc.dB[i]), f"shard {i}"
