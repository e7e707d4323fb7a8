"""CPU oracle for one tensor-parallel rank's share of the transformer MLP.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP path; the two meet only
in the seeded inputs, which arrive here as raw bf16 bit patterns.

What it computes is the plain definition, in float64, from the bf16-rounded inputs:

* The MLP is Y = GeLU(X A) B, with A cut into column blocks A_i and B into row
  blocks B_i; rank i computes Z_i = GeLU(X A_i) B_i and the ranks' partials are
  summed ("大模型训练" notes, §3.1 张量并行, MLP-layer formula and its two-GPU split;
  efficient-training survey on asorrir.com, part 一, 张量并行, the Megatron MLP
  figure; sequence-parallel series "大规模分布式 AI 模型训练系列——序列并行", §2.4).
* The first GEMM widens H to 4H, the second narrows 4H back to H, with GeLU in
  between (QLM page "大模型训练技术：使用QLM提升Qwen2-7B 128k训练效率3.4倍",
  §2.1.2.2 part 3).  The pages never write GeLU out; the reading taken is the exact
  form GeLU(p) = p * Phi(p) = 0.5 p (1 + erf(p / sqrt 2)), with Phi evaluated
  as erfc(-p / sqrt 2) / 2 (no cancellation in the negative tail).
* Splitting A by rows instead would need a sum before the non-linear GeLU, which is
  why A is split by columns (QLM page §2.1.2.2 part 3).
* Backward: the column-parallel input gradient is the sum of the per-rank
  gradients, the row-parallel layer's output gradient arrives replicated on every
  rank (QLM page §2.1.2.2 parts 1-2, with the operator names read as the f/g pair);
  the weight gradients of a product need that product's inputs (asorrir.com survey,
  part 二, Checkpoint 技术), so P_i = X A_i is either kept or recomputed.

Matrix products are numpy float64 ``@`` (a BLAS dgemm); erfc is ``scipy.special.erfc``.
There is no blocking, fusion or reordering beyond the definition.

Pins (tests/test_oracle.py): textbook GeLU values (tests/golden/gelu_values.txt),
brute-force scalar loops on tiny shapes, central finite differences of <dZ, Z>,
torch float64 autograd, the shard-sum identity for t in {1, 2, 4, 8}, linearity,
the A = 0 closed form of the backward, and the negative row-split test.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np
from scipy.special import erfc

_INV_SQRT2 = 1.0 / math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


# ---------------------------------------------------------------------------
# bf16 inputs ("大模型训练" notes §6.1: 1 sign bit, 8 exponent bits, 7 mantissa bits)
# ---------------------------------------------------------------------------
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns: the 16 bits are the top half of a
    float32 whose low half is zero."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# The activation
# ---------------------------------------------------------------------------
def normal_cdf(p: np.ndarray) -> np.ndarray:
    """Phi(p) = (1 + erf(p / sqrt 2)) / 2, evaluated as erfc(-p / sqrt 2) / 2, which
    is the same function without the cancellation of 1 + erf for p << 0."""
    return 0.5 * erfc(-p * _INV_SQRT2)


def gelu(p: np.ndarray) -> np.ndarray:
    """GeLU(p) = p * Phi(p), Phi the standard normal CDF."""
    return p * normal_cdf(p)


def gelu_grad(p: np.ndarray) -> np.ndarray:
    """d/dp [p Phi(p)] = Phi(p) + p phi(p), phi the standard normal density."""
    return normal_cdf(p) + p * np.exp(-0.5 * p * p) * _INV_SQRT_2PI


# ---------------------------------------------------------------------------
# The tensor-parallel split ("大模型训练" notes §3.1: A = [A_1 | A_2], B = [B_1 ; B_2])
# ---------------------------------------------------------------------------
def split_columns(A: np.ndarray, t: int) -> List[np.ndarray]:
    """A[H, F] -> t column blocks A_i[H, F/t]."""
    H, F = A.shape
    if F % t:
        raise ValueError("F must be divisible by t")
    f = F // t
    return [A[:, i * f:(i + 1) * f] for i in range(t)]


def split_rows(B: np.ndarray, t: int) -> List[np.ndarray]:
    """B[F, H] -> t row blocks B_i[F/t, H]."""
    F, H = B.shape
    if F % t:
        raise ValueError("F must be divisible by t")
    f = F // t
    return [B[i * f:(i + 1) * f, :] for i in range(t)]


# ---------------------------------------------------------------------------
# One rank's share: forward and backward
# ---------------------------------------------------------------------------
def mlp_forward(X: np.ndarray, A_i: np.ndarray, B_i: np.ndarray) -> Dict[str, np.ndarray]:
    """Rank i's forward: P_i = X A_i, G_i = GeLU(P_i), Z_i = G_i B_i (all float64)."""
    P = X @ A_i
    G = gelu(P)
    Z = G @ B_i
    return {"P": P, "G": G, "Z": Z}


def mlp_backward(dZ: np.ndarray, X: np.ndarray, A_i: np.ndarray, B_i: np.ndarray) -> Dict[str, np.ndarray]:
    """Rank i's backward given the replicated output gradient dZ.

    dG_i = dZ B_i^T, dP_i = dG_i * GeLU'(P_i), dB_i = G_i^T dZ, dA_i = X^T dP_i and
    the rank's partial input gradient dX_i = dP_i A_i^T.  P_i is recomputed from
    X and A_i here; keeping it from the forward gives the same float64 values.
    """
    P = X @ A_i
    G = gelu(P)
    dG = dZ @ B_i.T
    dP = dG * gelu_grad(P)
    return {
        "P": P,
        "G": G,
        "dG": dG,
        "dP": dP,
        "dB": G.T @ dZ,
        "dA": X.T @ dP,
        "dX": dP @ A_i.T,
    }


# ---------------------------------------------------------------------------
# All t ranks, partials summed in rank order (the all-reduce of the row-parallel
# output in the forward, of the column-parallel input gradient in the backward)
# ---------------------------------------------------------------------------
def _rank_order_sum(parts: Sequence[np.ndarray]) -> np.ndarray:
    total = np.array(parts[0], dtype=np.float64, copy=True)
    for p in parts[1:]:
        total = total + p
    return total


def tp_forward(X: np.ndarray, A_sh: Sequence[np.ndarray], B_sh: Sequence[np.ndarray]) -> Tuple[np.ndarray, List[np.ndarray]]:
    """Z = sum_i GeLU(X A_i) B_i over ranks 0..t-1; returns (Z, [Z_i])."""
    parts = [mlp_forward(X, a, b)["Z"] for a, b in zip(A_sh, B_sh)]
    return _rank_order_sum(parts), parts


def tp_backward(dZ: np.ndarray, X: np.ndarray, A_sh: Sequence[np.ndarray], B_sh: Sequence[np.ndarray]):
    """Returns (dX, [dX_i], [dA_i], [dB_i]); dX = sum_i dX_i in rank order."""
    outs = [mlp_backward(dZ, X, a, b) for a, b in zip(A_sh, B_sh)]
    dX_parts = [o["dX"] for o in outs]
    return _rank_order_sum(dX_parts), dX_parts, [o["dA"] for o in outs], [o["dB"] for o in outs]


# ---------------------------------------------------------------------------
# Single outputs, computed from the definition restricted to what they depend on.
# Tokens do not interact inside the MLP (sequence-parallel series §2.4), so a row
# of Z or dX needs only that row of X and dZ; a column of dA_i or a row of dB_i
# needs one column of P_i over all tokens.
# ---------------------------------------------------------------------------
def forward_rows(X: np.ndarray, A_i: np.ndarray, B_i: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Z_i[rows, :]."""
    return mlp_forward(X[rows], A_i, B_i)["Z"]


def backward_dX_rows(dZ, X, A_i, B_i, rows) -> np.ndarray:
    """dX_i[rows, :]."""
    return mlp_backward(dZ[rows], X[rows], A_i, B_i)["dX"]


def backward_dA_cols(dZ, X, A_i, B_i, cols) -> np.ndarray:
    """dA_i[:, cols] = X^T (dZ B_i[cols]^T * GeLU'(X A_i[:, cols]))."""
    P = X @ A_i[:, cols]
    dP = (dZ @ B_i[cols, :].T) * gelu_grad(P)
    return X.T @ dP


def backward_dB_rows(dZ, X, A_i, B_i, frows) -> np.ndarray:
    """dB_i[frows, :] = GeLU(X A_i[:, frows])^T dZ."""
    G = gelu(X @ A_i[:, frows])
    return G.T @ dZ


# ---------------------------------------------------------------------------
# Acceptance rule used against the GPU
# ---------------------------------------------------------------------------
def tolerance(ref: np.ndarray, rel: float = 1e-2, abs_: float = 1e-3) -> float:
    """max|gpu - oracle| must not exceed rel * max|oracle| + abs_ (per output tensor)."""
    return rel * float(np.max(np.abs(ref))) + abs_ if ref.size else abs_


def max_abs_err(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref))) if ref.size else 0.0
