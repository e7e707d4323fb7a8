"""The seeded input generator: determinism, bf16 rounding, workload structure."""
import numpy as np
import pytest

from tensor_transformer_mlp_03_amd import inputs as I


def test_configs_shapes():
    shapes = [(w.M, w.H, w.F, w.t, w.F_i) for w in I.CONFIGS]
    assert shapes == [
        (64, 256, 1024, 2, 512),
        (4096, 1024, 4096, 1, 4096),
        (2048, 4096, 16384, 8, 2048),
        (32768, 3584, 14336, 4, 3584),
        (2048, 20480, 81920, 8, 10240),
    ]
    # the MLP widens H to 4H (QLM page §2.1.2.2 part 3)
    assert all(w.F == 4 * w.H for w in I.CONFIGS)
    assert not I.CONFIGS[0].backward and all(w.backward for w in I.CONFIGS[1:])
    assert I.CONFIGS[4].recompute and I.CONFIGS[4].shards_timed == (0,)
    assert I.CONFIGS[3].n_outliers == 328


def test_rne_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    u = rng.integers(0, 1 << 32, size=500000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(I.f32_to_bf16_bits(x), want)


def test_rne_ties_to_even():
    # 1 + 2^-8 is exactly halfway between bf16 1.0 and 1.0078125: ties to even (1.0)
    # 1 + 3*2^-8 is halfway between 1.0078125 and 1.015625: ties to even (1.015625)
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, -0.0, 3.3895313892515355e38], dtype=np.float32)
    assert list(I.f32_to_bf16_bits(x)) == [0x3F80, 0x3F82, 0xBF80, 0x0000, 0x8000, 0x7F7F]
    assert I.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))[0] == 0x7FC0
    assert I.f32_to_bf16_bits(np.array([np.inf], dtype=np.float32))[0] == 0x7F80


def test_roundtrip_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    np.testing.assert_array_equal(I.f32_to_bf16_bits(I.bf16_bits_to_f32(bits[finite])), bits[finite])


def test_deterministic_and_independent_streams():
    w = I.custom_workload(901, M=64, H=32, F_i=48, t=3)
    a, b = I.make_inputs(w), I.make_inputs(w)
    np.testing.assert_array_equal(a.X, b.X)
    for i in range(3):
        np.testing.assert_array_equal(a.A[i], b.A[i])
        np.testing.assert_array_equal(a.B[i], b.B[i])
    assert not np.array_equal(a.A[0], a.A[1])
    assert not np.array_equal(a.X, a.dZ)
    # one shard alone equals the same shard of the full set
    only = I.make_inputs(w, shards=[2])
    assert only.A[0] is None and only.B[1] is None
    np.testing.assert_array_equal(only.A[2], a.A[2])
    # another seed gives other values
    assert not np.array_equal(I.make_inputs(w, seed=1).X, a.X)


def test_distributions():
    w = I.custom_workload(902, M=512, H=256, F_i=256, t=1, w_std=0.02)
    inp = I.make_inputs(w)
    X, A = I.bf16_bits_to_f32(inp.X), I.bf16_bits_to_f32(inp.A[0])
    assert abs(X.mean()) < 0.01 and abs(X.std() - 1.0) < 0.01
    assert abs(A.mean()) < 0.001 and abs(A.std() - 0.02) < 0.0005


def test_outlier_rows():
    w = I.custom_workload(903, M=1000, H=64, F_i=32, t=1, outlier_frac=0.01)
    rows = I.outlier_rows(w)
    assert rows.size == 10 and np.unique(rows).size == 10 and rows.max() < 1000
    X = I.make_X(w)
    base = I.normal_bf16(0, w.key, I.TID_X, 0, (w.M, w.H), 1.0)
    mask = np.zeros(w.M, bool)
    mask[rows] = True
    np.testing.assert_array_equal(X[~mask], base[~mask])
    np.testing.assert_array_equal(I.bf16_bits_to_f32(X[mask]), I.bf16_bits_to_f32(base[mask]) * 8)
