"""Seeded synthetic inputs for one tensor-parallel rank's share of the transformer MLP.

This module is the only code that both the HIP path and the CPU oracle consume.  It
holds no arithmetic of the method itself: it draws normal samples, rounds them to
bf16 bit patterns and cuts them into the per-rank weight shards that the method
operates on.  Everything it returns is raw ``uint16`` bf16 bits, so both sides see
identical inputs.

Workloads follow the shapes the pages talk about:

* the MLP widens H to 4H and back (QLM page, "大模型训练技术：使用QLM提升Qwen2-7B 128k
  训练效率3.4倍", §2.1.2.2, part 3 on the transformer's MLP);
* the first weight is split by columns, the second by rows, one shard per rank
  ("大模型训练" notes, §3.1 张量并行);
* activations are [s, b, h], flattened to M = s*b token rows (sequence-parallel
  series "大规模分布式 AI 模型训练系列——序列并行", §3.2).

Seeding: every tensor (and every shard of a sharded weight) has its own PCG64
stream, keyed by ``SeedSequence(seed, spawn_key=(workload_key, tensor_id, shard))``.
The unsharded weights are *defined* as the concatenation of the shards, so any one
rank's shard can be generated on its own.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

TID_X, TID_A, TID_B, TID_DZ, TID_OUTLIER = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic MLP workload.

    ``M`` token rows, hidden size ``H``, intermediate size ``F`` split over ``t``
    ranks (``F_i = F // t``).  ``w_std`` is the standard deviation of both weights;
    X and dZ are standard normal.  ``outlier_frac`` of the rows of X are scaled by
    ``outlier_scale`` after bf16 rounding (a power of two, so the scaling is exact).
    """

    key: int
    name: str
    M: int
    H: int
    F: int
    t: int
    w_std: float = 0.02
    backward: bool = True
    recompute: bool = False
    outlier_frac: float = 0.0
    outlier_scale: float = 8.0
    timed_shards: Optional[tuple] = None  # None: all shards
    description: str = ""

    @property
    def F_i(self) -> int:
        return self.F // self.t

    @property
    def n_outliers(self) -> int:
        return int(round(self.outlier_frac * self.M))

    @property
    def shards_timed(self) -> tuple:
        return tuple(range(self.t)) if self.timed_shards is None else tuple(self.timed_shards)

    def model_flops_per_shard(self) -> float:
        """Model FLOPs of one shard: 4*M*H*F_i forward, 12*M*H*F_i forward+backward."""
        mult = 12 if self.backward else 4
        return float(mult) * self.M * self.H * self.F_i


# The five workloads.  Sizes, distributions, split counts and the recompute choice
# are those of the benchmark configurations; the key doubles as the seed stream key.
CONFIGS: List[Workload] = [
    Workload(0, "tiny_fwd_t2", M=64, H=256, F=1024, t=2, w_std=0.02, backward=False,
             description="Tiny TP MLP, forward only, t=2"),
    Workload(1, "gpt2_medium_t1", M=4096, H=1024, F=4096, t=1, w_std=0.02,
             description="GPT-2-medium-like MLP, s=1024 b=4, unsharded"),
    Workload(2, "7b_t8", M=2048, H=4096, F=16384, t=8, w_std=0.02,
             description="7B-class MLP, s=2048 b=1, t=8 shards run in sequence"),
    Workload(3, "longctx_chunk_t4", M=32768, H=3584, F=14336, t=4, w_std=0.02,
             outlier_frac=0.01, outlier_scale=8.0,
             description="One context-parallel slice of a 128k sequence, t=4, 1% outlier rows x8"),
    Workload(4, "530b_shard_t8", M=2048, H=20480, F=81920, t=8, w_std=0.006,
             recompute=True, timed_shards=(0,),
             description="530B-class rank shard, t=8, GeLU pre-activation recomputed"),
]


def custom_workload(key: int, M: int, H: int, F_i: int, t: int, w_std: float = 0.02,
                    outlier_frac: float = 0.0, backward: bool = True,
                    recompute: bool = False, name: str = "") -> Workload:
    """A workload for tests at shapes other than the five configurations."""
    return Workload(key, name or f"custom_{key}", M=M, H=H, F=F_i * t, t=t, w_std=w_std,
                    outlier_frac=outlier_frac, backward=backward, recompute=recompute)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (1 sign, 8 exponent, 7 mantissa bits) with
    round-to-nearest-even; returns the uint16 bit patterns.  NaN maps to a quiet NaN.

    The bf16 format is the one in the mixed-precision table of the "大模型训练" notes
    (§6.1); the rounding mode is not given there and is taken as IEEE's default.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if nan.any():
        rounded[nan] = np.uint16(0x7FC0)
    return rounded


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, key: int, tid: int, shard: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(key, tid, shard))))


def normal_bf16(seed: int, key: int, tid: int, shard: int, shape, std: float) -> np.ndarray:
    """bf16 bits of N(0, std^2) samples drawn as float32 and scaled in float32."""
    x = _rng(seed, key, tid, shard).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def outlier_rows(w: Workload, seed: int = 0) -> np.ndarray:
    """Sorted indices of the rows of X that are scaled as outliers."""
    n = w.n_outliers
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    rows = _rng(seed, w.key, TID_OUTLIER, 0).choice(w.M, size=n, replace=False)
    return np.sort(rows.astype(np.int64))


@dataclass
class Inputs:
    """bf16 bit arrays of one workload: X[M,H], A_i[H,F_i], B_i[F_i,H], dZ[M,H]."""

    workload: Workload
    X: np.ndarray
    A: List[Optional[np.ndarray]]
    B: List[Optional[np.ndarray]]
    dZ: Optional[np.ndarray]
    outliers: np.ndarray = field(default_factory=lambda: np.zeros(0, dtype=np.int64))


def make_X(w: Workload, seed: int = 0) -> np.ndarray:
    X = normal_bf16(seed, w.key, TID_X, 0, (w.M, w.H), 1.0)
    rows = outlier_rows(w, seed)
    if rows.size:
        scaled = bf16_bits_to_f32(X[rows]) * np.float32(w.outlier_scale)
        X[rows] = f32_to_bf16_bits(scaled)
    return X


def make_A_shard(w: Workload, i: int, seed: int = 0) -> np.ndarray:
    return normal_bf16(seed, w.key, TID_A, i, (w.H, w.F_i), w.w_std)


def make_B_shard(w: Workload, i: int, seed: int = 0) -> np.ndarray:
    return normal_bf16(seed, w.key, TID_B, i, (w.F_i, w.H), w.w_std)


def make_dZ(w: Workload, seed: int = 0) -> np.ndarray:
    return normal_bf16(seed, w.key, TID_DZ, 0, (w.M, w.H), 1.0)


def make_inputs(w: Workload, seed: int = 0, shards=None, workers: int = 8) -> Inputs:
    """Generate the workload's tensors.  ``shards`` limits which weight shards are
    generated (others are None); default: all ``t``.  Shards are drawn on up to
    ``workers`` threads (each has its own stream, so the values do not depend on
    the number of threads)."""
    from concurrent.futures import ThreadPoolExecutor
    shards = list(range(w.t) if shards is None else shards)
    A: List[Optional[np.ndarray]] = [None] * w.t
    B: List[Optional[np.ndarray]] = [None] * w.t
    jobs = [(A, make_A_shard, i) for i in shards] + [(B, make_B_shard, i) for i in shards]
    with ThreadPoolExecutor(max_workers=max(1, min(workers, len(jobs)))) as ex:
        for (dst, _, i), arr in zip(jobs, ex.map(lambda j: j[1](w, j[2], seed), jobs)):
            dst[i] = arr
    dZ = make_dZ(w, seed) if w.backward else None
    return Inputs(w, make_X(w, seed), A, B, dZ, outlier_rows(w, seed))
