"""CPU oracle for the FP8 variant of one tensor-parallel rank's share of the MLP.

TEST INFRASTRUCTURE ONLY (like ``oracle.oracle``): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it, and it
shares no code with the HIP path.

The formats are the two 8-bit floats of the "大模型训练" notes (§6.1 数据类型对比):
E4M3, 4 exponent and 3 mantissa bits, range +-448, and E5M2, 5 exponent and 2
mantissa bits, range +-57344.  Those ranges fix the encodings: exponent bias 7 with
the all-ones exponent still finite (only S.1111.111 is NaN, no infinities) for E4M3,
and bias 15 with IEEE specials for E5M2; a zero exponent field holds subnormals.

The pages give no scaling recipe.  The one taken here (per-tensor current scaling):

* a tensor T of float32 values gets the scale s = fl32(amax / FMAX), amax = max |T|
  (s = 1 when T is all zero), and inv = fl32(1 / s);
* its codes are q = fp8(fl32(T * inv)): the product rounded to float32, then to the
  FP8 grid, nearest with ties to even, saturating at +-FMAX, the sign of zero kept;
* its value in a product is decode(q) * s.

E4M3 carries the activations and weights (X, A_i, B_i, G_i), E5M2 the gradients (dZ,
dP_i).  Products accumulate exactly here (float64) from the dequantized operands.
The pre-activation P_i and the gradient dP_i are held in bf16 between the products,
as in the bf16 path (its reading of the intermediate precision): G_i = GeLU(bf16(P_i))
is what gets quantized, dP_i = bf16(dG_i GeLU'(bf16(P_i))) likewise, each value
rounded to float32 first and then to bf16 (nearest, ties to even).  Where the
rounding of a float32 product decides a code, the oracle rounds in float32 exactly
as stated above, so quantizing the same float32 tensor gives the same bytes on both
sides.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Sequence, Tuple

import numpy as np

from .oracle import gelu, gelu_grad


@dataclass(frozen=True)
class Fp8Format:
    name: str
    ebits: int
    mbits: int
    bias: int
    fmax: float
    ieee_specials: bool  # True: the all-ones exponent is inf/NaN (E5M2)


# "大模型训练" notes §6.1: E4M3 4/3 bits, +-448; E5M2 5/2 bits, +-57344.
E4M3 = Fp8Format("e4m3", 4, 3, 7, 448.0, False)
E5M2 = Fp8Format("e5m2", 5, 2, 15, 57344.0, True)


def decode(codes: np.ndarray, fmt: Fp8Format) -> np.ndarray:
    """Exact float64 value of FP8 codes (NaN codes give NaN, E5M2 infinities inf)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> fmt.mbits) & ((1 << fmt.ebits) - 1)
    m = c & ((1 << fmt.mbits) - 1)
    emax_field = (1 << fmt.ebits) - 1
    normal = sign * (1.0 + m / float(1 << fmt.mbits)) * np.exp2(e.astype(np.float64) - fmt.bias)
    sub = sign * (m / float(1 << fmt.mbits)) * np.exp2(1.0 - fmt.bias)
    v = np.where(e == 0, sub, normal)
    if fmt.ieee_specials:
        v = np.where(e == emax_field, np.where(m == 0, sign * np.inf, np.nan), v)
    else:
        v = np.where((e == emax_field) & (m == (1 << fmt.mbits) - 1), np.nan, v)
    return v


def encode(x32: np.ndarray, fmt: Fp8Format) -> np.ndarray:
    """FP8 codes of float32 values: nearest grid value, ties to even, saturating at
    +-FMAX, sign of zero kept.  The inputs must be finite."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("finite inputs only")
    neg = np.signbit(x)
    a = np.abs(x)
    emin = 1 - fmt.bias  # exponent of the smallest normal
    # binade of a (floor(log2 a)), clamped to the subnormal binade's spacing
    _, k = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(k.astype(np.int64) - 1, emin)
    quantum = np.exp2((e - fmt.mbits).astype(np.float64))
    q = np.rint(a / quantum) * quantum  # exact: quantum is a power of two
    q = np.minimum(q, fmt.fmax)
    # the code of q
    _, kq = np.frexp(np.where(q > 0, q, 1.0))
    eq = kq.astype(np.int64) - 1
    is_sub = eq < emin
    mant_sub = np.rint(q / np.exp2(float(emin - fmt.mbits))).astype(np.int64)
    exp_field = np.where(is_sub, 0, eq + fmt.bias)
    mant_norm = np.rint((q / np.exp2(eq.astype(np.float64)) - 1.0) * (1 << fmt.mbits)).astype(np.int64)
    mant = np.where(is_sub, mant_sub, mant_norm)
    code = np.where(q == 0, 0, (exp_field << fmt.mbits) | mant)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


def scale_of(amax32, fmt: Fp8Format) -> np.float32:
    """s = fl32(amax / FMAX), or 1 for an all-zero tensor."""
    amax32 = np.float32(amax32)
    if amax32 == 0:
        return np.float32(1.0)
    return np.float32(amax32 / np.float32(fmt.fmax))


def quantize(T: np.ndarray, fmt: Fp8Format) -> Tuple[np.ndarray, np.float32]:
    """(codes, scale) of a tensor under per-tensor current scaling; T is rounded to
    float32 first (its values as the GPU holds them, for bf16 inputs exactly)."""
    t32 = np.asarray(T, dtype=np.float32)
    amax = np.float32(np.max(np.abs(t32))) if t32.size else np.float32(0)
    s = scale_of(amax, fmt)
    inv = np.float32(np.float32(1.0) / s)
    return encode(t32 * inv, fmt), s


def round_bf16(x: np.ndarray) -> np.ndarray:
    """x rounded to float32, then to bf16 (nearest, ties to even), as float64."""
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = ((b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)) << np.uint64(16)
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def dequant(codes: np.ndarray, s, fmt: Fp8Format) -> np.ndarray:
    return decode(codes, fmt) * np.float64(s)


def qdq(T: np.ndarray, fmt: Fp8Format) -> np.ndarray:
    """The value a tensor takes in a product after quantization."""
    c, s = quantize(T, fmt)
    return dequant(c, s, fmt)


# ---------------------------------------------------------------------------
# One rank's share with FP8 operands (the products of the bf16 path, each taking
# its operands through qdq)
# ---------------------------------------------------------------------------
def mlp_forward_fp8(X: np.ndarray, A_i: np.ndarray, B_i: np.ndarray) -> Dict[str, np.ndarray]:
    """P_i = bf16(qdq(X) qdq(A_i)); G_i = GeLU(P_i); Z_i = qdq(G_i) qdq(B_i)."""
    Xq, Aq, Bq = qdq(X, E4M3), qdq(A_i, E4M3), qdq(B_i, E4M3)
    P = round_bf16(Xq @ Aq)
    G = gelu(P)
    Gq = qdq(G, E4M3)
    return {"P": P, "G": G, "Gq": Gq, "Z": Gq @ Bq}


def mlp_backward_fp8(dZ: np.ndarray, X: np.ndarray, A_i: np.ndarray, B_i: np.ndarray) -> Dict[str, np.ndarray]:
    """dG_i = qdq5(dZ) qdq(B_i)^T; dP_i = bf16(dG_i GeLU'(P_i)); with dPq = qdq5(dP_i):
    dB_i = qdq(G_i)^T qdq5(dZ), dA_i = qdq(X)^T dPq, dX_i = dPq qdq(A_i)^T."""
    f = mlp_forward_fp8(X, A_i, B_i)
    Xq, Aq, Bq = qdq(X, E4M3), qdq(A_i, E4M3), qdq(B_i, E4M3)
    dZq = qdq(dZ, E5M2)
    dG = dZq @ Bq.T
    dP = round_bf16(dG * gelu_grad(f["P"]))
    dPq = qdq(dP, E5M2)
    return {"P": f["P"], "dG": dG, "dP": dP, "dB": f["Gq"].T @ dZq, "dA": Xq.T @ dPq, "dX": dPq @ Aq.T}


def _rank_order_sum(parts: Sequence[np.ndarray]) -> np.ndarray:
    total = np.array(parts[0], dtype=np.float64, copy=True)
    for p in parts[1:]:
        total = total + p
    return total


def tp_forward_fp8(X, A_sh, B_sh) -> Tuple[np.ndarray, List[np.ndarray]]:
    parts = [mlp_forward_fp8(X, a, b)["Z"] for a, b in zip(A_sh, B_sh)]
    return _rank_order_sum(parts), parts


def tp_backward_fp8(dZ, X, A_sh, B_sh):
    """Returns (dX, [dX_i], [dA_i], [dB_i])."""
    outs = [mlp_backward_fp8(dZ, X, a, b) for a, b in zip(A_sh, B_sh)]
    dXp = [o["dX"] for o in outs]
    return _rank_order_sum(dXp), dXp, [o["dA"] for o in outs], [o["dB"] for o in outs]
