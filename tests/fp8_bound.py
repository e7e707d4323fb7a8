"""How far a correct FP8 path may land from the FP8 oracle, element by element.

Test infrastructure (it calls the oracle, never the HIP path).

The oracle (oracle/fp8.py) forms each product exactly.  A correct implementation
accumulates in float32 and evaluates GeLU and GeLU' to a few float32 ulps, and then
takes integer decisions on what it got: the bf16 rounding of P_i and of dP_i, and
the FP8 codes of G_i = GeLU(P_i) and of dP_i, whose scales come from maxima of the
same values.  Where the exact value lies closer to a rounding boundary than that
float32 error, either side of the boundary is a correct decision, and every product
that consumes the code moves with it by one FP8 spacing of that element (1/8 of it
for E4M3, 1/4 for E5M2): far more than the float32 accumulation error, so a tolerance
on the whole tensor would have to allow that move everywhere.

Instead, this module carries intervals through the decisions, in the oracle's order:

* P = X A in [P - eP, P + eP], with eP = (K + 4) u (|X| |A|) + n c m, u = 2^-24,
  K = H.  The first term is the classic bound on a K-term float32 sum in any
  order, plus the roundings of the scale product and of the scaled result.  The
  second is the matrix cores' own: their FP8 dot product over a 128-deep K block
  is not a float32 sum rounded to nearest (hand-made operands show the bits of
  small products dropped against large ones, 2^17.6 + 2^-18 - 2^17.6 coming out
  0; on random E4M3 operands one instruction lands up to 2^-12 of its largest
  product away from the exact sum), so n = ceil(K / 128) instructions may each
  add c = 2^-10 (four times the largest seen) of m = max_k |X_mk| max_k |A_kf|,
  a bound on each product.  This is measured, not proved: the GPU test checks it
  where it would fail first, every stored bf16 P_i lying in the interval below;
* its bf16 rounding lies between the roundings of the two ends (rounding is
  monotone); so does GeLU over that range (its minimum at p0 = -0.7518 included),
  widened by the float32 GeLU's own error dG(p) = 6e-7 |p| (the erfc fit is good to
  7.5e-8 in Phi, the float32 steps add a few ulps of Phi(-|p|) <= 1/2);
* the amax of G_i lies between the maxima of the ends, so the scale s = amax / 448
  and 1 / s lie in intervals, and so do the float32 products G / s, and (encoding is
  monotone) the codes;
* dG = dZ B^T in [dG - edG, dG + edG], edG formed as eP; GeLU'(P) over P's range (its extrema
  at p = +-sqrt 2 included) widened by 1e-6; dP = bf16(dG GeLU'(P)) between the
  roundings of the extreme products; then amax, scale and E5M2 codes as for G.

For each element the largest distance between a value the interval admits and the
oracle's own dequantized value is dGq (for G_i) or ddPq (for dP_i); it is zero where
the decision is unique.  The admissible deviation of an output is then the bf16
path's tensor-wide rule, 1e-2 max|oracle| + 1e-3, plus, element by element, what the
admissible moves add to it:

    Z:    sum_i dGq_i |B_i|         dB_i: dGq_i^T |dZ|
    dX:   sum_i ddPq_i |A_i|^T      dA_i: |X|^T ddPq_i

(|.| of the dequantized FP8 operands).  A wrong tile, scale, index or operand moves
elements whose decisions were unique and fails the check; the CPU tests plant such
mistakes in a float32 emulation of the path to show that.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Sequence

import numpy as np

from oracle import fp8 as F
from oracle import oracle as O

U32 = 2.0 ** -24
MFMA_K = 128            # K depth of one FP8 matrix-core instruction
MFMA_REL_ERR = 2.0 ** -10  # its error, as a fraction of its largest product
GELU_MIN_AT = -0.7517916243
GELU_ABS_ERR_PER_P = 6e-7
GRAD_ABS_ERR = 1e-6
SQRT2 = float(np.sqrt(2.0))


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def _range_of(fn, lo, hi, critical: Sequence[float]):
    """[min, max] of fn over [lo, hi] (elementwise), fn smooth with the given
    stationary points."""
    a, b = fn(lo), fn(hi)
    mn, mx = np.minimum(a, b), np.maximum(a, b)
    for c in critical:
        inside = (lo < c) & (c < hi)
        if np.any(inside):
            fc = float(fn(np.float64(c)))
            mn = np.where(inside, np.minimum(mn, fc), mn)
            mx = np.where(inside, np.maximum(mx, fc), mx)
    return mn, mx


def _abs_range(lo, hi):
    """[min |x|, max |x|] for x in [lo, hi]."""
    amin = np.where((lo <= 0) & (hi >= 0), 0.0, np.minimum(np.abs(lo), np.abs(hi)))
    return amin, np.maximum(np.abs(lo), np.abs(hi))


def _code_moves(lo, hi, ref_q, fmt: F.Fp8Format):
    """For float values known to lie in [lo, hi] (already as float32 numbers, e.g.
    bf16), with the tensor's amax somewhere in [max min|x|, max max|x|]: the largest
    distance from ref_q (the oracle's dequantized value) of any value a correct
    quantization can produce, and how many elements have more than one admissible
    code."""
    alo, ahi = _abs_range(lo, hi)
    s_lo = F.scale_of(np.float32(np.max(alo)) if alo.size else 0.0, fmt)
    s_hi = F.scale_of(np.float32(np.max(ahi)) if ahi.size else 0.0, fmt)
    inv_hi = np.float32(np.float32(1.0) / s_lo)
    inv_lo = np.float32(np.float32(1.0) / s_hi)
    ends = [_f32(lo) * inv_lo, _f32(lo) * inv_hi, _f32(hi) * inv_lo, _f32(hi) * inv_hi]
    y_lo = np.minimum.reduce(ends)
    y_hi = np.maximum.reduce(ends)
    v_lo = F.decode(F.encode(y_lo, fmt), fmt)
    v_hi = F.decode(F.encode(y_hi, fmt), fmt)
    move = np.zeros(ref_q.shape, dtype=np.float64)
    for v in (v_lo, v_hi):
        for s in (np.float64(s_lo), np.float64(s_hi)):
            move = np.maximum(move, np.abs(v * s - ref_q))
    return move, int(np.count_nonzero(v_lo != v_hi))


@dataclass
class ShardMoves:
    """Admissible moves of one shard's FP8 operands G_i and dP_i, with the oracle's
    quantities they were derived from."""
    fwd: Dict[str, np.ndarray]
    bwd: Dict[str, np.ndarray]
    dGq: np.ndarray          # [M, F_i]
    ddPq: np.ndarray         # [M, F_i]
    ambiguous_g: int         # elements of G_i with more than one admissible code
    ambiguous_dp: int        # likewise for dP_i
    p_lo: np.ndarray         # the admissible bf16 P_i lie in [p_lo, p_hi]
    p_hi: np.ndarray


def shard_moves(X: np.ndarray, A_i: np.ndarray, B_i: np.ndarray, dZ: np.ndarray,
                n_round=None) -> ShardMoves:
    """n_round: how many float32 roundings the error bound of P and dG counts (by
    default K + 4, which holds for any summation order)."""
    fwd = F.mlp_forward_fp8(X, A_i, B_i)
    bwd = F.mlp_backward_fp8(dZ, X, A_i, B_i)
    Xq, Aq, Bq = F.qdq(X, F.E4M3), F.qdq(A_i, F.E4M3), F.qdq(B_i, F.E4M3)
    dZq = F.qdq(dZ, F.E5M2)
    H = X.shape[1]
    nr = H + 4 if n_round is None else n_round
    n_mfma = -(-H // MFMA_K)

    def accumulation_error(a, b):
        """Bound on |fl(a b) - a b| for the GPU's products (a [m, K], b [K, n])."""
        aa, ab = np.abs(a), np.abs(b)
        per_product = np.max(aa, axis=1)[:, None] * np.max(ab, axis=0)[None, :] if aa.size and ab.size \
            else np.zeros((a.shape[0], b.shape[1]))
        return nr * U32 * (aa @ ab) + n_mfma * MFMA_REL_ERR * per_product

    # P: float32 accumulation, then bf16
    exact_P = Xq @ Aq
    eP = accumulation_error(Xq, Aq)
    p_lo, p_hi = F.round_bf16(exact_P - eP), F.round_bf16(exact_P + eP)
    # G = GeLU(P) in float32, then E4M3 codes
    g_lo, g_hi = _range_of(O.gelu, p_lo, p_hi, [GELU_MIN_AT])
    g_err = GELU_ABS_ERR_PER_P * np.maximum(np.abs(p_lo), np.abs(p_hi))
    dGq, amb_g = _code_moves(g_lo - g_err, g_hi + g_err, fwd["Gq"], F.E4M3)
    # dP = bf16(dG GeLU'(P)), then E5M2 codes
    dG = bwd["dG"]
    edG = accumulation_error(dZq, Bq.T)
    d_lo, d_hi = _range_of(O.gelu_grad, p_lo, p_hi, [-SQRT2, SQRT2])
    d_lo, d_hi = d_lo - GRAD_ABS_ERR, d_hi + GRAD_ABS_ERR
    corners = [(dG - edG) * d_lo, (dG - edG) * d_hi, (dG + edG) * d_lo, (dG + edG) * d_hi]
    dp_lo = F.round_bf16(np.minimum.reduce(corners))
    dp_hi = F.round_bf16(np.maximum.reduce(corners))
    ddPq, amb_dp = _code_moves(dp_lo, dp_hi, F.qdq(bwd["dP"], F.E5M2), F.E5M2)
    return ShardMoves(fwd, bwd, dGq, ddPq, amb_g, amb_dp, p_lo, p_hi)


@dataclass
class PathBounds:
    """The oracle's outputs of the t-shard FP8 forward and backward and, per output,
    the element-wise admissible deviation."""
    Z: np.ndarray
    dX: np.ndarray
    dA: List[np.ndarray]
    dB: List[np.ndarray]
    P: List[np.ndarray]
    tol_Z: np.ndarray
    tol_dX: np.ndarray
    tol_dA: List[np.ndarray]
    tol_dB: List[np.ndarray]
    ambiguous_g: int
    ambiguous_dp: int
    shards: List[ShardMoves]


def path_bounds(X: np.ndarray, A_sh: Sequence[np.ndarray], B_sh: Sequence[np.ndarray],
                dZ: np.ndarray, n_round=None) -> PathBounds:
    moves = [shard_moves(X, a, b, dZ, n_round) for a, b in zip(A_sh, B_sh)]
    Xq, dZq = F.qdq(X, F.E4M3), F.qdq(dZ, F.E5M2)
    Aq = [F.qdq(a, F.E4M3) for a in A_sh]
    Bq = [F.qdq(b, F.E4M3) for b in B_sh]
    # the oracle's sums in rank order, as tp_forward_fp8 / tp_backward_fp8 form them
    Z = moves[0].fwd["Z"].copy()
    dX = moves[0].bwd["dX"].copy()
    for m in moves[1:]:
        Z = Z + m.fwd["Z"]
        dX = dX + m.bwd["dX"]
    dA = [m.bwd["dA"] for m in moves]
    dB = [m.bwd["dB"] for m in moves]
    move_Z = sum(m.dGq @ np.abs(b) for m, b in zip(moves, Bq))
    move_dX = sum(m.ddPq @ np.abs(a).T for m, a in zip(moves, Aq))
    return PathBounds(
        Z=Z, dX=dX, dA=dA, dB=dB, P=[m.fwd["P"] for m in moves],
        tol_Z=O.tolerance(Z) + move_Z,
        tol_dX=O.tolerance(dX) + move_dX,
        tol_dA=[O.tolerance(r) + np.abs(Xq).T @ m.ddPq for r, m in zip(dA, moves)],
        tol_dB=[O.tolerance(r) + m.dGq.T @ np.abs(dZq) for r, m in zip(dB, moves)],
        ambiguous_g=sum(m.ambiguous_g for m in moves),
        ambiguous_dp=sum(m.ambiguous_dp for m in moves),
        shards=moves)


def worst_ratio(got: np.ndarray, ref: np.ndarray, tol: np.ndarray):
    """(max over elements of |got - ref| / tol, the index where it is reached)."""
    r = np.abs(np.asarray(got, dtype=np.float64) - ref) / tol
    if r.size == 0:
        return 0.0, ()
    k = np.unravel_index(int(np.argmax(r)), r.shape)
    return float(r[k]), tuple(int(i) for i in k)
