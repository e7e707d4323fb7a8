"""Pins of the FP8 oracle (oracle/fp8.py) against what the pages and independent
implementations fix, CPU only.

* The formats' bit counts and ranges come from the "大模型训练" notes §6.1 table
  (E4M3: 4/3 bits, +-448; E5M2: 5/2 bits, +-57344).
* Decoding and encoding are checked against torch's float8_e4m3fn / float8_e5m2
  conversions (an independent implementation of the same OCP formats), on every code
  and on random float32 values, and against constructed ties and saturation cases.
* The scaling recipe: the largest element maps to +-FMAX, and scaling a tensor by a
  power of two changes its scale and not its codes.
* The FP8 path: its outputs stay within a first-order error bound, derived from the
  formats' rounding bounds, the bf16 rounding of P and dP, and the products'
  structure, of the exact (float64, unquantized) oracle, and do differ from it.
* bf16 rounding: round_bf16 against torch's float32 -> bfloat16 conversion.
"""
import numpy as np
import pytest

from oracle import fp8 as F
from oracle import oracle as O

torch = pytest.importorskip("torch")

FORMATS = [(F.E4M3, torch.float8_e4m3fn), (F.E5M2, torch.float8_e5m2)]


@pytest.mark.parametrize("fmt,tdt", FORMATS, ids=["e4m3", "e5m2"])
def test_decode_every_code_matches_torch(fmt, tdt):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(tdt).float().numpy().astype(np.float64)
    got = F.decode(codes, fmt)
    assert np.all((ref == got) | (np.isnan(ref) & np.isnan(got)))


def test_ranges_and_bits_from_the_pages():
    # +-448 and +-57344 are the largest finite values; the bit counts are the table's
    for fmt, top in ((F.E4M3, 448.0), (F.E5M2, 57344.0)):
        v = F.decode(np.arange(256, dtype=np.uint8), fmt)
        assert np.nanmax(v[np.isfinite(v)]) == top and np.nanmin(v[np.isfinite(v)]) == -top
        assert 1 + fmt.ebits + fmt.mbits == 8
    assert (F.E4M3.ebits, F.E4M3.mbits, F.E5M2.ebits, F.E5M2.mbits) == (4, 3, 5, 2)
    # E4M3 has no infinities (only S.1111.111 is NaN); E5M2 has +-inf
    v4 = F.decode(np.arange(256, dtype=np.uint8), F.E4M3)
    assert not np.any(np.isinf(v4)) and int(np.isnan(v4).sum()) == 2
    v5 = F.decode(np.arange(256, dtype=np.uint8), F.E5M2)
    assert int(np.isinf(v5).sum()) == 2 and int(np.isnan(v5).sum()) == 6


@pytest.mark.parametrize("fmt,tdt", FORMATS, ids=["e4m3", "e5m2"])
def test_encode_matches_torch_on_random_values(fmt, tdt):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(300000) * np.exp2(rng.integers(-24, 16, 300000))).astype(np.float32)
    x = x[np.abs(x) <= fmt.fmax]
    ref = torch.from_numpy(x).to(tdt).view(torch.uint8).numpy()
    assert np.array_equal(F.encode(x, fmt), ref)


def test_encode_ties_to_even_subnormals_signed_zero_and_saturation():
    # E4M3 near 1: grid step 1/8; 1 + 1/16 ties to 1 (even), 1 + 3/16 to 1.25
    x = np.array([1.0625, 1.1875, -1.0625, 0.0, -0.0], dtype=np.float32)
    assert list(F.decode(F.encode(x, F.E4M3), F.E4M3)) == [1.0, 1.25, -1.0, 0.0, 0.0]
    assert list(F.encode(x[3:], F.E4M3)) == [0x00, 0x80]
    # E4M3 subnormals are multiples of 2^-9; half of 2^-9 ties to 0, 1.5 * 2^-9 to 2^-8
    s = np.array([2.0 ** -10, 1.5 * 2.0 ** -9, 2.0 ** -9], dtype=np.float32)
    assert list(F.decode(F.encode(s, F.E4M3), F.E4M3)) == [0.0, 2.0 ** -8, 2.0 ** -9]
    # E5M2: smallest subnormal 2^-16
    assert F.decode(F.encode(np.float32([2.0 ** -16]), F.E5M2), F.E5M2)[0] == 2.0 ** -16
    # beyond the range: saturate to +-FMAX (no NaN, no inf)
    big = np.array([449.0, 1e6, -1e6, 470.0], dtype=np.float32)
    assert list(F.decode(F.encode(big, F.E4M3), F.E4M3)) == [448.0, 448.0, -448.0, 448.0]
    big5 = np.array([60000.0, -1e30], dtype=np.float32)
    assert list(F.decode(F.encode(big5, F.E5M2), F.E5M2)) == [57344.0, -57344.0]


@pytest.mark.parametrize("fmt", [F.E4M3, F.E5M2], ids=["e4m3", "e5m2"])
def test_scaling_recipe(fmt):
    rng = np.random.default_rng(5)
    T = (rng.standard_normal((64, 96)) * 0.02).astype(np.float32)
    codes, s = F.quantize(T, fmt)
    i = np.unravel_index(np.argmax(np.abs(T)), T.shape)
    assert abs(F.decode(codes[i], fmt)) == fmt.fmax  # the largest element takes the largest code
    assert s == np.float32(np.float32(np.max(np.abs(T))) / np.float32(fmt.fmax))
    # a power-of-two change of the tensor moves only its scale
    for k in (-6, 3):
        c2, s2 = F.quantize(T * np.float32(2.0 ** k), fmt)
        assert np.array_equal(c2, codes) and s2 == np.float32(s * 2.0 ** k)
    # all-zero tensor: scale 1, zero codes
    cz, sz = F.quantize(np.zeros((3, 4), np.float32), fmt)
    assert sz == 1.0 and not cz.any()
    # dequantized values are within the format's rounding bound of the tensor
    u, d = 2.0 ** -(fmt.mbits + 1), 2.0 ** (1 - fmt.bias - fmt.mbits - 1)
    err = np.abs(F.dequant(codes, s, fmt) - T)
    assert np.all(err <= (u + 4 * 2.0 ** -24) * np.abs(T) + float(s) * d)


# ---------------------------------------------------------------------------
# The FP8 path against the exact one, within a first-order error bound
# ---------------------------------------------------------------------------
def _qbound(T, fmt):
    """Elementwise bound of |qdq(T) - T| for a float32 tensor T (rounding of the
    float32 scaling, half an FP8 ulp in the normal range, half the subnormal step
    times the scale)."""
    codes, s = F.quantize(T, fmt)
    u, d = 2.0 ** -(fmt.mbits + 1), 2.0 ** (1 - fmt.bias - fmt.mbits - 1)
    return (u + 4 * 2.0 ** -24) * np.abs(T) + float(s) * d


def _inputs(seed, M=48, H=64, Fi=80):
    rng = np.random.default_rng(seed)
    f32 = lambda a: a.astype(np.float32).astype(np.float64)
    X = f32(rng.standard_normal((M, H)))
    A = f32(rng.standard_normal((H, Fi)) * 0.1)
    B = f32(rng.standard_normal((Fi, H)) * 0.1)
    dZ = f32(rng.standard_normal((M, H)))
    return X, A, B, dZ


L_GELU, L_DGELU = 1.1290, 0.7980  # max |GeLU'| and max |GeLU''| (= 2 phi(0))
U16 = 2.0 ** -8  # bound of the relative rounding of float64 -> float32 -> bf16 (half a bf16 ulp, plus slack)


def test_fp8_path_within_error_bound_of_exact():
    X, A, B, dZ = _inputs(21)
    ex_f = O.mlp_forward(X, A, B)
    ex_b = O.mlp_backward(dZ, X, A, B)
    f = F.mlp_forward_fp8(X, A, B)
    b = F.mlp_backward_fp8(dZ, X, A, B)
    ab = np.abs
    EX, EA, EB = _qbound(X, F.E4M3), _qbound(A, F.E4M3), _qbound(B, F.E4M3)
    Xq, Aq, Bq = ab(X) + EX, ab(A) + EA, ab(B) + EB          # bounds of |qdq(.)|
    EP = EX @ Aq + ab(X) @ EA + U16 * ab(f["P"]) * (1 + U16)  # |bf16(P_fp8) - P|
    G8 = O.gelu(f["P"])
    EGq = _qbound(G8, F.E4M3) + L_GELU * EP                 # |qdq(G(P_fp8)) - G(P)|
    EZ = EGq @ Bq + ab(ex_f["G"]) @ EB
    tol = lambda E: E * (1 + 1e-9) + 1e-12
    assert np.all(ab(f["Z"] - ex_f["Z"]) <= tol(EZ))
    EdZ = _qbound(dZ, F.E5M2)
    dZq = ab(dZ) + EdZ
    EdG = EdZ @ Bq.T + ab(dZ) @ EB.T
    dG8 = (F.qdq(dZ, F.E5M2)) @ F.qdq(B, F.E4M3).T
    EdPpre = (EdG * np.abs(O.gelu_grad(f["P"])) + ab(ex_b["dG"]) * L_DGELU * EP) + U16 * ab(b["dP"]) * (1 + U16)
    EdP = _qbound(b["dP"], F.E5M2) + EdPpre
    assert np.all(ab(b["dP"] - ex_b["dP"]) <= tol(EdPpre))
    dPq = ab(ex_b["dP"]) + EdP
    EdB = EGq.T @ dZq + ab(ex_f["G"]).T @ EdZ
    EdA = EX.T @ dPq + ab(X).T @ EdP
    EdX = EdP @ Aq.T + ab(ex_b["dP"]) @ EA.T
    for k, E in (("dB", EdB), ("dA", EdA), ("dX", EdX)):
        assert np.all(ab(b[k] - ex_b[k]) <= tol(E)), k
    # quantization does change every output
    for got, ref in ((f["Z"], ex_f["Z"]), (b["dB"], ex_b["dB"]), (b["dA"], ex_b["dA"]), (b["dX"], ex_b["dX"])):
        assert np.max(ab(got - ref)) > 1e-6 * np.max(ab(ref))
    assert np.all(np.isfinite(dG8))


def test_fp8_tp_sums_shards_in_rank_order():
    X, A, B, dZ = _inputs(22, Fi=96)
    As, Bs = O.split_columns(A, 3), O.split_rows(B, 3)
    Z, parts = F.tp_forward_fp8(X, As, Bs)
    assert np.array_equal(Z, (parts[0] + parts[1]) + parts[2])
    dX, dXp, dA, dB = F.tp_backward_fp8(dZ, X, As, Bs)
    assert np.array_equal(dX, (dXp[0] + dXp[1]) + dXp[2])
    # each shard quantizes its own weights: shard 1 alone gives shard 1's partial
    assert np.array_equal(F.mlp_forward_fp8(X, As[1], Bs[1])["Z"], parts[1])


def test_fp8_forward_closed_form_two_tokens():
    """X = [1, 0.5]^T (H = 1), A = B = [[1]]: every operand is on the grid (X's
    scale is 1/448 and 0.5 * 448 = 224 = 1.75 * 2^7; one-element A and B are
    exact), so P = [1, 0.5] and G = [GeLU(1), GeLU(0.5)] = [Phi(1), Phi(0.5)/2] =
    [0.8413447, 0.3457312] (normal CDF table values).  G's scale is GeLU(1)/448;
    GeLU(0.5) * 448 / GeLU(1) = 184.10, past the midpoint 184 of the E4M3 grid
    points 176 and 192 (step 16 in [128, 256)), so it becomes 192: Z = [GeLU(1),
    192/448 GeLU(1)]."""
    X = np.array([[1.0], [0.5]])
    A = np.array([[1.0]])
    B = np.array([[1.0]])
    Z = F.mlp_forward_fp8(X, A, B)["Z"][:, 0]
    phi1, phi05 = 0.8413447460685429, 0.6914624612740131
    # (float32 scales are within 1e-7 relative of the exact ratios)
    assert abs(Z[0] - phi1) < 1e-6
    assert abs(Z[1] - 192.0 / 448.0 * phi1) < 1e-6
    assert abs(Z[1] - 0.5 * phi05) > 1e-2  # not the unquantized GeLU(0.5)
    assert abs(0.5 * phi05 * 448 / phi1 - 184.0953) < 1e-3


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(200000) * np.exp2(rng.integers(-30, 30, 200000))
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(F.round_bf16(x), ref)
