#!/usr/bin/env python3
"""Benchmark of one tensor-parallel rank's share of the transformer MLP on MI355X.

A step is one pass of the whole path over one batch of synthetic input: the
forward of every shard (GEMM1 + GeLU, GEMM2), the rank-order sum of the partial
outputs, the backward of every shard (dGeLU GEMM, dB, dA, dX GEMMs, split-K
reductions) and the sum of the partial input gradients.  Inputs are resident in
HBM before the timed region starts.

Prints ONE JSON line.  ``value`` is model TFLOP/s of the whole job
(12*M*H*F_i per shard and step; recompute FLOPs are not counted), ``roofline``
describes the kernel that takes the most time (algorithmic FLOPs per launch over
its average launch time from HIP events recorded on its stream inside the timed
region), ``cpu_baseline`` is the CPU oracle timed on a bounded row sample of the
same workload.

``fp8`` times the FP8 path (E4M3 activations and weights, E5M2 gradients) on the
first workload, against the dense fp8 MFMA peak.

    python bench.py [--config 3] [--steps 20] [--warmup 5] [--no-cpu-baseline] [--no-fp8]
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

METRIC = "TP-MLP fwd+bwd TFLOP/s per rank shard (bf16) and % of MFMA dense peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, published
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "tensor_transformer_mlp_03_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def source_hash() -> str:
    """sha256 over the library's sources: counters taken from another build are stale."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()


def traffic_path(workload_name: str, fp8: bool = False) -> str:
    return os.path.join(PROFILES, f"{workload_name}{'_fp8' if fp8 else ''}_traffic.md")


def read_traffic(workload_name: str, fp8: bool = False):
    """{kernel kind: HBM bytes per launch} from the committed counter summary, or None
    if there is none or it was taken from other sources than the current ones."""
    path = traffic_path(workload_name, fp8)
    if not os.path.exists(path):
        return None
    sha, table = None, {}
    for line in open(path):
        parts = line.split()
        if len(parts) == 2 and parts[0] == "source_sha256:":
            sha = parts[1]
        if len(parts) == 4 and parts[0] == "traffic_bytes":
            table[parts[1]] = (float(parts[2]), float(parts[3]))
    return table if sha == source_hash() else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_flops(w):
    """Algorithmic FLOPs of one launch of each GEMM kind for one shard."""
    M, H, F = w.M, w.H, w.F_i
    f = 2.0 * M * H * F
    return {"fwd_gemm1_gelu": f, "fwd_gemm2": f, "bwd_recompute": f, "bwd_dgelu": f, "bwd_dB": f, "bwd_dA": f,
            "bwd_dX": f, "fwd_fused": 2 * f, "bwd_dB_dX": 2 * f}


def batch_factor(w, kind, launches, steps):
    """Shards one launch of a product kind covers: the t-shard driver may run
    several shards' F1, recompute, dGeLU, dB or dA as one batched launch, and two
    shards' F3 or dX as one paired launch, so a kind launched fewer times per step
    than there are shards covers several."""
    shards = len(w.shards_timed)
    per_step = launches / steps if steps else 0
    if kind not in ("fwd_gemm1_gelu", "bwd_recompute", "bwd_dgelu", "bwd_dB", "bwd_dA", "fwd_gemm2",
                    "bwd_dX") or per_step <= 0:
        return 1.0
    return max(1.0, shards / per_step)


def gemm_alg_bytes(w, recompute, fold=False):
    """Algorithmic HBM bytes of one launch of each GEMM kind (operands read once,
    outputs written once; bf16 = 2 bytes, float32 = 4).  fold: the t-shard driver adds
    the partials of Z and dX in the products' epilogues, so t - 1 of every t launches
    of those kinds also read the running sum (counted as its average per launch)."""
    M, H, F = w.M, w.H, w.F_i
    acc = 4 * M * H * (w.t - 1) / w.t if fold else 0
    return {
        "fwd_gemm1_gelu": 2 * (M * H + H * F) + 2 * M * F * (1 if recompute else 2),  # X, A_i -> G (+P)
        "fwd_gemm2": 2 * (M * F + F * H) + 4 * M * H + acc,                          # G, B_i (+Z) -> Z
        "bwd_recompute": 2 * (M * H + H * F) + 2 * M * F,                             # X, A_i -> P
        "bwd_dgelu": 2 * (M * H + F * H + M * F) + 4 * M * F,                         # dZ, B_i, P -> dP, G^T
        "bwd_dB": 2 * (M * F + M * H) + 4 * F * H,                                    # G^T, dZ^T -> dB_i
        "bwd_dA": 2 * (M * H + M * F) + 4 * H * F,                                    # X^T, dP -> dA_i
        "bwd_dX": 2 * (M * F + H * F) + 4 * M * H + acc,                              # dP, A_i (+dX) -> dX
        # dB_i and dX_i as one launch (M = F_i, no running sum)
        "bwd_dB_dX": 2 * (M * F + M * H) + 4 * F * H + 2 * (M * F + H * F) + 4 * M * H,
        "transpose": 8 * M * H,                                                       # X, dZ -> X^T, dZ^T (one launch)
        # X, A_i, B_i -> float32 partials of Z_i, one per chunk of 64 intermediate columns (+P)
        "fwd_fused": 2 * (M * H + 2 * H * F) + 4 * M * H * (-(-F // 64)) + (0 if recompute else 2 * M * F),
    }


def transpose_alg_bytes(w, launches):
    """Average algorithmic bytes of one of a step's `launches` transpose launches.
    The step transposes X and dZ (4 M H bytes each) before a backward, dP_i
    (4 M F_i) per shard when dA reads it transposed, and A_i and B_i (4 H F_i each)
    per shard in the forward, A_i again for the recompute, when the planner
    transposes the weights.  How many launches carry them (X with dZ, A_i with B_i
    when they share a shape) changes only the divisor."""
    n = len(w.shards_timed)
    total = 8 * w.M * w.H if w.backward else 0
    if w.backward and dp_transposed(w):
        total += n * 4 * w.M * w.F_i
    if weights_transposed(w):
        total += n * (2 + (1 if (w.backward and w.recompute) else 0)) * 4 * w.H * w.F_i
    return total / launches


def launch_alg_bytes(w, kind, factor, shards):
    """Algorithmic bytes of one launch of `kind` covering `factor` shards: batched
    launches move each shard's operands and outputs; a paired F3 or dX launch
    reads its two shards' operands but writes the output, and reads the running
    sum (all pairs but the first), once."""
    base = gemm_alg_bytes(w, w.recompute, fold=folds(w))
    if kind not in ("fwd_gemm2", "bwd_dX") or factor <= 1:
        return base[kind] * factor
    M, H, F = w.M, w.H, w.F_i
    per_step = shards / factor
    return factor * 2 * (M * F + F * H) + 4 * M * H + 4 * M * H * (per_step - 1) / per_step


def fp8_alg_bytes(w, fold=False):
    """Algorithmic HBM bytes of one launch of each product kind of the FP8 path:
    FP8 codes 1 byte, bf16 2, float32 4; operands read once, outputs written once
    (fold: as in gemm_alg_bytes, the accumulating launches' running-sum reads)."""
    M, H, F = w.M, w.H, w.F_i
    acc = 4 * M * H * (w.t - 1) / w.t if fold else 0
    return {
        "fwd_gemm1_gelu": (M * H + H * F) + 2 * M * F,              # X, A_i codes -> P (bf16)
        "bwd_recompute": (M * H + H * F) + 2 * M * F,
        "fwd_gemm2": (M * F + F * H) + 4 * M * H + acc,             # G, B_i codes -> Z
        "bwd_dgelu": (M * H + F * H) + 2 * M * F + 2 * M * F,       # dZ, B_i codes, P -> dP (bf16)
        "bwd_dB": (M * F + M * H) + 4 * F * H,                      # G^T, dZ^T codes -> dB_i
        "bwd_dA": (M * H + M * F) + 4 * H * F,                      # X^T, dP^T codes -> dA_i
        "bwd_dX": (M * F + H * F) + 4 * M * H + acc,                # dP, A_i codes -> dX
    }


def dp_transposed(w):
    """Whether the library transposes dP_i before dA_i = X^T dP_i for this shape: the
    saving on one product, 2 M H F_i (1/1.14e15 - 1/1.2e15) s, is 1.5 times the
    transpose, 4 M F_i / 5.5e12 s (the planner's rates), i.e. for H above ~12400."""
    saved = 2.0 * w.M * w.H * w.F_i * (1.0 / 1.14e15 - 1.0 / 1.2e15)
    return saved > 1.5 * 4.0 * w.M * w.F_i / 5.5e12


def weights_transposed(w):
    """Whether the library transposes A_i and B_i for the forward products (the
    planner's rule restated): the saving on two products, 4 M H F_i (1/1.14e15 -
    1/1.2e15) s, is 1.5 times the transposes' 4 H F_i / 5.5e12 s, i.e. M above ~6200."""
    saved = 4.0 * w.M * w.H * w.F_i * (1.0 / 1.14e15 - 1.0 / 1.2e15)
    return saved > 1.5 * 4.0 * w.H * w.F_i / 5.5e12


def folds(w):
    """Whether bench's step folds the partial sums into the products: it runs the
    t-shard driver (every shard) without per-shard partials."""
    return len(w.shards_timed) == w.t and w.t > 1


def cpu_baseline(w, target_s=12.0):
    """The oracle's forward+backward on a bounded sample of the workload: token rows
    of the first timed shard (tokens are independent, so the work per row is the
    full per-row work), and whole further shards while the total stays short."""
    import numpy as np
    from oracle import oracle as O
    from tensor_transformer_mlp_03_amd import inputs as I
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    X_all, dZ_all = I.make_X(w), I.make_dZ(w)

    def run(i, rows):
        A = O.decode_bf16(I.make_A_shard(w, i))
        B = O.decode_bf16(I.make_B_shard(w, i))
        X, dZ = O.decode_bf16(X_all[:rows]), O.decode_bf16(dZ_all[:rows])
        t0 = time.perf_counter()
        O.mlp_forward(X, A, B)
        O.mlp_backward(dZ, X, A, B)
        return time.perf_counter() - t0

    shards = list(w.shards_timed)
    rows = min(w.M, 256)
    dt = run(shards[0], rows)
    if dt < target_s / 4 and rows < w.M:
        rows = int(min(w.M, max(rows, rows * target_s / max(dt, 1e-3))) // 8 * 8)
        dt = run(shards[0], rows)
    done = [shards[0]]
    if rows == w.M:
        for i in shards[1:]:
            if dt >= target_s:
                break
            dt += run(i, rows)
            done.append(i)
    flops = 12.0 * rows * w.H * w.F_i * len(done)
    what = f"shards {done}" if len(done) > 1 else f"shard {done[0]}"
    cpu, blas = "unknown CPU", "unknown BLAS"
    try:
        cpu = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = ", ".join(sorted({p.get("internal_api", "?") for p in threadpool_info() if p.get("user_api") == "blas"}))
    except Exception:
        pass
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"float64 oracle forward+backward of {what} on the first {rows} of {w.M} token rows "
                      f"(H={w.H}, F_i={w.F_i}); {dt:.2f} s on {cpu}, numpy BLAS {blas}"}


def cpu_baseline_fp8(w, target_s=8.0):
    """The FP8 oracle's forward+backward of shard 0 on a bounded sample of token
    rows (the sample is the tensor the oracle quantizes), as cpu_baseline does
    for the bf16 oracle."""
    import numpy as np
    from oracle import fp8 as F8
    from oracle import oracle as O
    from tensor_transformer_mlp_03_amd import inputs as I
    i = w.shards_timed[0]
    A = O.decode_bf16(I.make_A_shard(w, i))
    B = O.decode_bf16(I.make_B_shard(w, i))
    X_all, dZ_all = I.make_X(w), I.make_dZ(w)

    def run(rows):
        X, dZ = O.decode_bf16(X_all[:rows]), O.decode_bf16(dZ_all[:rows])
        t0 = time.perf_counter()
        F8.mlp_forward_fp8(X, A, B)
        F8.mlp_backward_fp8(dZ, X, A, B)
        return time.perf_counter() - t0

    rows = min(w.M, 128)
    dt = run(rows)
    if dt < target_s / 4 and rows < w.M:
        rows = int(min(w.M, max(rows, rows * target_s / max(dt, 1e-3))) // 16 * 16)
        dt = run(rows)
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    return {"value": round(12.0 * rows * w.H * w.F_i / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"float64 FP8 oracle (oracle/fp8.py) forward+backward of shard {i} on the first {rows} of "
                      f"{w.M} token rows (H={w.H}, F_i={w.F_i}); {dt:.2f} s"}


def _order_entries(order):
    """Recorded launch order as [(kind, kernel dispatches)]: a timing record covers one
    dispatch, or two where a product runs as whole-wave tiles plus a split tail."""
    return [(e, 1) if isinstance(e, str) else (e[0], int(e[1])) for e in order]


def _kernel_kinds_of(csv_path, order):
    """Dispatches of libtpmlp kernels in a rocprofv3 counter CSV, in dispatch order,
    grouped into the timing records that bench recorded for the same run: one
    (kind, {"name", "counters"}) per record, counters summed over its dispatches."""
    rows = {}
    for r in csv.DictReader(open(csv_path)):
        if "tpmlp" not in r["Kernel_Name"]:
            continue
        d = int(r["Dispatch_Id"])
        rows.setdefault(d, {"name": r["Kernel_Name"], "counters": {}})
        rows[d]["counters"][r["Counter_Name"]] = rows[d]["counters"].get(r["Counter_Name"], 0.0) + float(
            r["Counter_Value"])
    disp = [rows[d] for d in sorted(rows)]
    entries = _order_entries(order)
    n_disp = sum(n for _, n in entries)
    if len(disp) != n_disp:
        raise SystemExit(f"{csv_path}: {len(disp)} libtpmlp dispatches, {n_disp} recorded "
                         f"({len(entries)} timing records)")
    out, i = [], 0
    for kind, n in entries:
        rec = {"name": disp[i]["name"], "counters": {}}
        for d in disp[i:i + n]:
            for c, v in d["counters"].items():
                rec["counters"][c] = rec["counters"].get(c, 0.0) + v
        out.append((kind, rec))
        i += n
    return out


def _copy_scale(csv_path, counter, mib):
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if "tpmlp" in r["Kernel_Name"] and r["Counter_Name"] == counter]
    return (mib * 1024.0) / (sum(vals) / len(vals))  # expected KiB / counted KiB


def summarize(d, config, fp8=False):
    """Write profiles/<workload>[_fp8]_kernels.md and ..._traffic.md (and _counters.md)
    from the rocprofv3 outputs in directory d (layout of the commands quoted in
    them); fp8: the runs timed the FP8 path only (--fp8-only)."""
    from tensor_transformer_mlp_03_amd import inputs as I
    w = I.CONFIGS[config]
    tag = "_fp8" if fp8 else ""
    path_name = "FP8 path, " if fp8 else ""
    cmd = json.load(open(os.path.join(d, "commands.json")))
    stats = list(csv.DictReader(open(glob.glob(os.path.join(d, "trace", "*_kernel_stats.csv"))[0])))
    order = json.load(open(os.path.join(d, "order.json")))
    fetch = _kernel_kinds_of(glob.glob(os.path.join(d, "fetch", "*_counter_collection.csv"))[0], order)
    write = _kernel_kinds_of(glob.glob(os.path.join(d, "write", "*_counter_collection.csv"))[0], order)
    mib = cmd["copy_mib"]
    f_scale = _copy_scale(glob.glob(os.path.join(d, "copy_fetch", "*_counter_collection.csv"))[0], "FETCH_SIZE", mib)
    w_scale = _copy_scale(glob.glob(os.path.join(d, "copy_write", "*_counter_collection.csv"))[0], "WRITE_SIZE", mib)
    agg = {}
    for (kind, f), (kind2, wr) in zip(fetch, write):
        assert kind == kind2
        a = agg.setdefault(kind, {"n": 0, "fetch": 0.0, "write": 0.0, "name": f["name"]})
        a["n"] += 1
        a["fetch"] += f["counters"]["FETCH_SIZE"] * 1024 * f_scale
        a["write"] += wr["counters"]["WRITE_SIZE"] * 1024 * w_scale
    alg = fp8_alg_bytes(w, fold=folds(w)) if fp8 else gemm_alg_bytes(w, w.recompute, fold=folds(w))
    if "transpose" in agg and not fp8:
        # A backward step transposes X and dZ ([M,H]) in one launch, and dP ([M,F_i]) once
        # per shard when the planner transposes it for dA (large H: the library's rule is
        # restated in dp_transposed); every further launch is a weight transpose
        # ([H,F_i] or [F_i,H]).  Per launch: the step's average.
        alg["transpose"] = transpose_alg_bytes(w, agg["transpose"]["n"])
    alg["shard_sum"] = (w.t + 1) * w.M * w.H * 4  # t float32 partials in, their sum out
    for kind, a in agg.items():  # a batched launch covers several shards (the counter passes run one step)
        if kind in alg and kind not in ("transpose", "shard_sum"):  # those two are per launch already
            f = batch_factor(w, kind, a["n"], 1)
            alg[kind] = alg[kind] * f if fp8 else launch_alg_bytes(w, kind, f, len(w.shards_timed))
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"{w.name}{tag}_kernels.md"), "w") as f:
        f.write(f"# Kernel times, {path_name}{w.name} (M={w.M}, H={w.H}, F_i={w.F_i}, t={w.t})\n\n")
        f.write("Command (rocprofv3 kernel trace and stats):\n\n```\n" + cmd["trace"] + "\n```\n\n")
        f.write("| kernel | calls | average us | total ms | % |\n|---|---|---|---|---|\n")
        for r in stats:
            f.write(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                    f"{float(r['TotalDurationNs']) / 1e6:.2f} | {float(r['Percentage']):.1f} |\n")
    with open(traffic_path(w.name, fp8), "w") as f:
        f.write(f"# HBM traffic per launch, {path_name}{w.name} (M={w.M}, H={w.H}, F_i={w.F_i}, t={w.t})\n\n")
        f.write("FETCH_SIZE and WRITE_SIZE (KiB per dispatch, L2-to-fabric traffic) from two rocprofv3 --pmc "
                "runs of one step, each scaled by what the same counter reads for a plain copy of "
                f"{mib} MiB through tpmlp_shard_sum (one part): fetch x{f_scale:.3f}, write x{w_scale:.3f}. "
                "A launch is one timed call of a kind: one kernel dispatch, or two where a product runs as "
                "whole waves of unsplit tiles plus a split tail (their bytes are added).\n\n")
        for k in ("fetch", "write", "copy_fetch", "copy_write"):
            f.write(f"```\n{cmd[k]}\n```\n")
        f.write("\n| kind | launches | fetch MB/launch | write MB/launch | algorithmic MB/launch | ratio |\n"
                "|---|---|---|---|---|---|\n")
        for kind, a in agg.items():
            fb, wb = a["fetch"] / a["n"], a["write"] / a["n"]
            al = alg.get(kind)
            f.write(f"| {kind} | {a['n']} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | "
                    f"{al / 1e6 if al else float('nan'):.1f} | {((fb + wb) / al) if al else float('nan'):.2f} |\n")
        f.write("\nMachine-readable (bytes per launch, fetch then write):\n\n```\n")
        f.write(f"source_sha256: {source_hash()}\n")
        for kind, a in agg.items():
            f.write(f"traffic_bytes {kind} {a['fetch'] / a['n']:.0f} {a['write'] / a['n']:.0f}\n")
        f.write("```\n")
    counters_md = _summarize_counters(d, w, cmd, order, agg, tag)
    print(f"wrote {PROFILES}/{w.name}{tag}_kernels.md and {traffic_path(w.name, fp8)}"
          + (f" and {counters_md}" if counters_md else ""))


def _summarize_counters(d, w, cmd, order, traffic, tag=""):
    """profiles/<workload>_counters.md: per kernel kind, the launch time (kernel trace),
    the shader clock and MFMA utilisation implied by GRBM_GUI_ACTIVE, the SQ MFMA-busy
    ratio, LDS bank conflicts per LDS instruction and HBM GB/s.  Needs the trace run's
    launch order and the SQ counter pass; returns None when they are absent."""
    trace_order_path = os.path.join(d, "trace_order.json")
    sq_csv = glob.glob(os.path.join(d, "sq", "*_counter_collection.csv"))
    trace_csv = glob.glob(os.path.join(d, "trace", "*_kernel_trace.csv"))
    if not (os.path.exists(trace_order_path) and sq_csv and trace_csv and "sq" in cmd):
        return None
    trace_order = _order_entries(json.load(open(trace_order_path)))
    disp = sorted((int(r["Dispatch_Id"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                  for r in csv.DictReader(open(trace_csv[0])) if "tpmlp" in r["Kernel_Name"])
    disp = disp[len(disp) - sum(n for _, n in trace_order):]  # the timed launches are the last ones
    dur, i = {}, 0
    for kind, n in trace_order:  # a record's time is the sum of its dispatches
        dur.setdefault(kind, []).append(sum(ns for _, ns in disp[i:i + n]))
        i += n
    sq = {}
    for kind, rec in _kernel_kinds_of(sq_csv[0], order):
        a = sq.setdefault(kind, {"n": 0})
        a["n"] += 1
        for c, v in rec["counters"].items():
            a[c] = a.get(c, 0.0) + v
    flops = gemm_flops(w)
    path = os.path.join(PROFILES, f"{w.name}{tag}_counters.md")
    peak_flop_clk = 8192 if tag == "_fp8" else 4096  # per CU: dense fp8 / bf16 MFMA
    with open(path, "w") as f:
        f.write(f"# Counters per kernel kind, {'FP8 path, ' if tag else ''}{w.name} "
                f"(M={w.M}, H={w.H}, F_i={w.F_i}, t={w.t})\n\n")
        f.write("Launch times from the kernel trace (the timed steps' dispatches), counters from one "
                "rocprofv3 --pmc pass over one step. A launch is one timed call of a kind: one kernel "
                "dispatch, or two where a product runs as whole waves of unsplit tiles plus a split tail "
                "(their times and counters are added):\n\n")
        f.write("```\n" + cmd["trace"] + "\n" + cmd["sq"] + "\n```\n\n")
        f.write("- cycles = GRBM_GUI_ACTIVE / 8 (the counter is summed over the 8 XCDs); clock = cycles / launch time "
                "(launches of 100 us or more only).\n"
                f"- MFMA util = the launch's algorithmic flops / (cycles x 256 CUs x {peak_flop_clk} "
                f"{'fp8' if tag else 'bf16'} flop/clk), i.e. the fraction of the MFMA peak at the clock the "
                "launch actually ran at.\n"
                "- SQ MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs).\n"
                "- LDS conflicts = SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS (conflict cycles per LDS instruction).\n"
                "- HBM GB/s = (FETCH_SIZE + WRITE_SIZE bytes, scaled as in the traffic file) / launch time.\n\n")
        f.write("| kind | launches | us | clock GHz | MFMA util | SQ MFMA busy | LDS conflicts / inst | HBM GB/s |\n"
                "|---|---|---|---|---|---|---|---|\n")
        for kind, a in sq.items():
            n = a["n"]
            us = (sum(dur.get(kind, [0])) / max(len(dur.get(kind, [])), 1)) / 1e3
            cyc = a.get("GRBM_GUI_ACTIVE", 0.0) / n / 8
            # The counter pass's dispatch is not the timed one; for short launches the two differ
            # too much for their ratio to be a clock.
            clock = cyc / (us * 1e3) if us >= 100 else float("nan")
            fl = flops[kind] * batch_factor(w, kind, n, 1) if kind in flops else 0.0
            util = (fl / (cyc * 256 * peak_flop_clk)) if kind in flops and cyc else float("nan")
            busy = a.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / n / (cyc * 1024) if cyc else float("nan")
            confl = a.get("SQ_LDS_BANK_CONFLICT", 0.0) / max(a.get("SQ_INSTS_LDS", 0.0), 1.0)
            t = traffic.get(kind)
            gbs = ((t["fetch"] + t["write"]) / t["n"]) / (us * 1e-6) / 1e9 if (t and us) else float("nan")
            f.write(f"| {kind} | {n} | {us:.1f} | {clock:.2f} | {util:.3f} | {busy:.3f} | {confl:.3f} | {gbs:.0f} |\n")
    return path


def measure(w, args, L, I, DeviceMLP, torch):
    """Warmup and timed steps of one workload; returns its numbers."""
    shards = list(w.shards_timed)
    driver = len(shards) == w.t
    log(f"[bench] workload {w.name}: M={w.M} H={w.H} F_i={w.F_i} t={w.t} shards={shards} "
        f"{'recompute' if w.recompute else 'store P'}; generating inputs")
    inp = I.make_inputs(w, shards=shards)
    if args.full_weights and not driver:
        print("--full-weights needs every shard of the workload", file=sys.stderr)
        sys.exit(2)
    d = DeviceMLP(inp, store_p=not w.recompute, driver=driver, full_weights=args.full_weights)
    del inp
    torch.cuda.synchronize()
    per_launch = gemm_flops(w)
    # Warmup, with every launch timed: the per-kind breakdown and the choice of
    # the dominant GEMM kind.  A timed launch delays the next kernel by a few
    # microseconds, so the timed steps below time only the dominant kind (all
    # kinds when a profiler run needs every launch's kind in order).
    log("[bench] inputs resident; warmup")
    warm_stats = None
    if args.warmup:
        L.tpmlp_timing_begin(16 * (len(shards) + 1) * args.warmup)
        for _ in range(args.warmup):
            d.step()
        torch.cuda.synchronize()
        warm_stats, _ = L.tpmlp_timing_end()
    torch.cuda.synchronize()

    n_launch = 16 * (len(shards) + 1) * max(args.steps, 1)
    dom = None
    graph = None
    if args.graph:
        if not warm_stats or args.trace_order:
            print("--graph needs warmup steps (their events give the per-kernel times) and no --trace-order",
                  file=sys.stderr)
            sys.exit(2)
        graph = d.capture()
        graph.replay()
        torch.cuda.synchronize()
        dom = max((n for n in per_launch if warm_stats.get(n, (0, 0))[0]), key=lambda n: warm_stats[n][1])
    elif warm_stats and not args.trace_order:
        dom = max((n for n in per_launch if warm_stats.get(n, (0, 0))[0]), key=lambda n: warm_stats[n][1])
        L.tpmlp_timing_begin_kinds(n_launch, [dom])
    else:
        L.tpmlp_timing_begin(n_launch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            d.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if graph is not None:
        stats, dropped = warm_stats, 0
    else:
        stats, dropped = L.tpmlp_timing_end()
    log(f"[bench] timed {args.steps} steps in {t1 - t0:.4f} s"
        + (" (graph replays; kernel times from the warmup)" if graph is not None
           else f" (launches of {dom} timed)" if dom else " (every launch timed)"))
    if args.trace_order:
        with open(args.trace_order, "w") as f:
            json.dump([[k, n] for (k, _), n in zip(L.tpmlp_timing_records(), L.tpmlp_timing_dispatches())], f)

    ms_per_step = (t1 - t0) * 1e3 / max(args.steps, 1)
    flops_step = w.model_flops_per_shard() * len(shards)
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    kernels = {}
    src = warm_stats if (dom or graph is not None) else stats
    src_steps = args.warmup if (dom or graph is not None) else args.steps
    log(f"[bench] {w.name} per kernel kind, {'warmup' if dom else 'timed'} steps:")
    for name, (count, total_ms) in src.items():
        if count:
            kernels[name] = {"launches": count, "avg_us": round(total_ms * 1e3 / count, 2),
                             "share": round(total_ms / sum(v[1] for v in src.values()), 4)}
            if name in per_launch:
                f = per_launch[name] * batch_factor(w, name, count, src_steps)
                kernels[name]["tflops"] = round(f / (total_ms * 1e-3 / count) / 1e12, 1)
                if f != per_launch[name]:
                    kernels[name]["shards_per_launch"] = round(f / per_launch[name], 2)
    for name, k in sorted(kernels.items(), key=lambda kv: -kv[1]["share"]):
        log(f"  {name:16s} {k}")
    if dom is None:
        dom = max((n for n in kernels if n in per_launch), key=lambda n: stats[n][1])
    avg_s = stats[dom][1] * 1e-3 / stats[dom][0]
    stat_steps = args.warmup if graph is not None else args.steps
    factor = batch_factor(w, dom, stats[dom][0], stat_steps)
    achieved = per_launch[dom] * factor / avg_s / 1e12
    traffic = read_traffic(w.name)
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": None, "avg_launch_us": round(avg_s * 1e6, 2),
                "alg_bytes": launch_alg_bytes(w, dom, factor, len(shards))}
    if factor != 1.0:
        roofline["shards_per_launch"] = round(factor, 2)
    if traffic and dom in traffic:
        fetch, write = traffic[dom]
        roofline["traffic"] = int(fetch + write)
        roofline["traffic_fetch"], roofline["traffic_write"] = int(fetch), int(write)
    log(f"[bench] {w.name}: {ms_per_step:.4f} ms per step, {value:.1f} TFLOP/s")
    cold = None
    if args.cold > 0 and graph is None:
        # Cold steps: before each, a 512 MiB fill evicts the 256 MB Infinity Cache;
        # events on the stream the library launches on bracket the step alone.
        scrub = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        events = []
        for i in range(args.cold):  # back to back, so that the GPU does not idle between steps
            scrub.fill_(i & 0x7F)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            d.step()
            e1.record()
            events.append((e0, e1))
        torch.cuda.synchronize()
        times = [e0.elapsed_time(e1) for e0, e1 in events]
        del scrub
        cold_ms = sorted(times)[len(times) // 2]
        cold = {"steps": args.cold, "ms_per_step_median": round(cold_ms, 4), "ms_per_step_min": round(min(times), 4),
                "value": round(flops_step / (cold_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                "scrub_bytes": 512 << 20}
        log(f"[bench] {w.name} cold (Infinity Cache evicted before each step): median {cold_ms:.4f} ms, "
            f"{cold['value']:.1f} TFLOP/s")
    del d
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"shards": len(shards), "ms_per_step": ms_per_step, "value": value, "roofline": roofline,
            "dropped": dropped, "cold": cold}


def measure_fp8(w, args, L, I, torch):
    """The FP8 path (E4M3 activations and weights, E5M2 gradients, per-tensor
    scaling) on the same workload and shards: warmup with every launch timed, then
    timed steps with the dominant product kind's launches timed."""
    from tensor_transformer_mlp_03_amd.device import DeviceFp8MLP
    shards = list(w.shards_timed)
    log(f"[bench] FP8 path on {w.name}, shards {shards}: generating inputs")
    inp = I.make_inputs(w, shards=shards)
    d = DeviceFp8MLP(inp, store_p=not w.recompute)
    del inp
    torch.cuda.synchronize()
    per_launch = gemm_flops(w)
    log("[bench] FP8 inputs resident; warmup")
    warm, dom = None, None
    if args.warmup:
        L.tpmlp_timing_begin(64 * (len(shards) + 1) * args.warmup)
        for _ in range(args.warmup):
            d.step()
        torch.cuda.synchronize()
        warm, _ = L.tpmlp_timing_end()
        dom = max((n for n in per_launch if warm.get(n, (0, 0))[0]), key=lambda n: warm[n][1])
    n_launch = 64 * (len(shards) + 1) * max(args.steps, 1)
    if dom is None or args.trace_order:  # every launch timed (a profiler run records their kinds in order)
        L.tpmlp_timing_begin(n_launch)
    else:
        L.tpmlp_timing_begin_kinds(n_launch, [dom])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        d.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stats, dropped = L.tpmlp_timing_end()
    if args.trace_order:
        with open(args.trace_order, "w") as f:
            json.dump([[k, n] for (k, _), n in zip(L.tpmlp_timing_records(), L.tpmlp_timing_dispatches())], f)
    if dom is None:
        dom = max((n for n in per_launch if stats.get(n, (0, 0))[0]), key=lambda n: stats[n][1])
    if warm is None:
        warm = stats
    ms = (t1 - t0) * 1e3 / max(args.steps, 1)
    value = w.model_flops_per_shard() * len(shards) / (ms * 1e-3) / 1e12
    avg_s = stats[dom][1] * 1e-3 / stats[dom][0]
    achieved = per_launch[dom] / avg_s / 1e12
    total = sum(v[1] for v in warm.values())
    kernels = {k: {"launches": c, "avg_us": round(ms_ * 1e3 / c, 2), "share": round(ms_ / total, 4),
                   **({"tflops": round(per_launch[k] / (ms_ * 1e-3 / c) / 1e12, 1)} if k in per_launch else {})}
               for k, (c, ms_) in warm.items() if c}
    for name, k in sorted(kernels.items(), key=lambda kv: -kv[1]["share"]):
        log(f"  fp8 {name:16s} {k}")
    log(f"[bench] FP8 {w.name}: {ms:.4f} ms per step, {value:.1f} TFLOP/s")
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": None,
                "avg_launch_us": round(avg_s * 1e6, 2), "alg_bytes": fp8_alg_bytes(w, fold=folds(w))[dom]}
    traffic = read_traffic(w.name, fp8=True)
    if traffic and dom in traffic:
        fetch, write = traffic[dom]
        roofline["traffic"] = int(fetch + write)
        roofline["traffic_fetch"], roofline["traffic_write"] = int(fetch), int(write)
    del d
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"workload": w.name, "formats": "E4M3 X, A_i, B_i, G_i; E5M2 dZ, dP_i; per-tensor current scaling",
            "shards_per_step": len(shards), "ms_per_step": round(ms, 4), "value": round(value, 2),
            "unit": "TFLOP/s", "frac_of_fp8_peak": round(value / PEAK_FP8_TFLOPS, 4),
            "roofline": roofline,
            "kernels_warmup": kernels, "timing_dropped": dropped}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, help="workload index 0-4 (default 3)")
    ap.add_argument("--also", type=int, default=4,
                    help="second workload timed in the same run and reported under \"workloads\" (default 4, "
                         "the 530B-class shard; -1 for none; skipped with --graph or --trace-order)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", type=int, default=0,
                    help="also time this many steps one at a time, each after a 512 MiB fill that evicts the "
                         "Infinity Cache (reported as `cold`; the headline stays the back-to-back steps)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8 path's measurement on the first workload (reported under \"fp8\")")
    ap.add_argument("--fp8-only", action="store_true",
                    help="time the FP8 path only (profiler runs of it; with --summarize: its summaries)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one step captured into a HIP graph (for launch-latency-bound "
                         "workloads); per-kernel times then come from the eager warmup steps")
    ap.add_argument("--full-weights", action="store_true",
                    help="run the t-shard driver over the whole weights A[H, t F_i], B[t F_i, H] (shards as views)")
    ap.add_argument("--trace-order", default="",
                    help="write [kernel kind, kernel dispatches] of the timed launches, in order, to this JSON file")
    ap.add_argument("--summarize", default="",
                    help="directory of rocprofv3 CSV outputs to summarize into profiles/ (no GPU needed)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain copy of this many MiB through tpmlp_shard_sum with one part "
                         "(reference dispatch for scaling HBM byte counters), then exit")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize, args.config, fp8=args.fp8_only)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the tensor-parallel "
              "ranks' shards run one after another on a single GPU).", file=sys.stderr)
        sys.exit(2)

    import torch
    from tensor_transformer_mlp_03_amd import _lib as L
    from tensor_transformer_mlp_03_amd import inputs as I
    from tensor_transformer_mlp_03_amd.device import DeviceMLP

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    L.lib()
    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            L.tpmlp_shard_sum([src], dst)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: 3 dispatches, each reads and writes {args.copy_probe_mib} MiB")
        return
    w = I.CONFIGS[args.config]
    if args.fp8_only:
        if not w.backward:
            print("--fp8-only needs a workload with a backward", file=sys.stderr)
            sys.exit(2)
        print(json.dumps({"workload": w.name, "fp8": measure_fp8(w, args, L, I, torch)}), flush=True)
        return
    m = measure(w, args, L, I, DeviceMLP, torch)
    extra = {}
    if args.also >= 0 and args.also != args.config and not (args.graph or args.trace_order or args.full_weights):
        # The second target workload, timed the same way in the same run, reported
        # in its own object; the headline stays the first and is printed whatever
        # happens here.
        w2 = I.CONFIGS[args.also]
        try:
            m2 = measure(w2, args, L, I, DeviceMLP, torch)
            extra[w2.name] = {
                "workload": w2.name, "M": w2.M, "H": w2.H, "F_i": w2.F_i, "t": w2.t,
                "shards_per_step": m2["shards"], "pre_activation": "recompute" if w2.recompute else "stored",
                "ms_per_step": round(m2["ms_per_step"], 4), "value": round(m2["value"], 2), "unit": "TFLOP/s",
                "frac_of_peak": round(m2["value"] / PEAK_BF16_TFLOPS, 4),
                "hfu_tflops": round(m2["value"] * (14.0 if w2.recompute else 12.0) / 12.0, 2),
                "roofline": m2["roofline"], "timing_dropped": m2["dropped"]}
            if m2["cold"]:
                extra[w2.name]["cold"] = m2["cold"]
        except Exception as e:
            log(f"[bench] {w2.name} failed: {e!r}")
            extra[w2.name] = {"workload": w2.name, "error": repr(e)}
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
    fp8 = None
    if not (args.no_fp8 or args.graph or args.trace_order or args.full_weights) and w.backward:
        try:
            fp8 = measure_fp8(w, args, L, I, torch)
        except Exception as e:  # the headline line is printed whatever happens here
            log(f"[bench] FP8 path failed: {e!r}")
            fp8 = {"workload": w.name, "error": repr(e)}
    shards, ms_per_step, value, roofline, dropped = m["shards"], m["ms_per_step"], m["value"], m["roofline"], \
        m["dropped"]

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "H": w.H, "F": w.F, "t": w.t, "F_i": w.F_i,
                   "shards_per_step": shards, "pre_activation": "recompute" if w.recompute else "stored",
                   "weights": "whole (shard views)" if args.full_weights else "per-shard buffers",
                   "launch": "HIP graph replay" if args.graph else "eager",
                   "saved_activation_bytes_per_rank": L.tpmlp_saved_activation_bytes(w.M, w.H, w.F_i, w.recompute),
                   "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
                   # hardware FLOPs: the recomputed product of the pre-activation counted too
                   "hfu_tflops": round(value * (14.0 if w.recompute else 12.0) / 12.0, 2) if w.backward else round(value, 2),
                   "timing_dropped": dropped},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if m["cold"]:
        result["cold"] = m["cold"]
    if extra:
        result["workloads"] = extra
    if fp8:
        if "value" in fp8:
            fp8["vs_bf16"] = round(fp8["value"] / value, 3)
        result["fp8"] = fp8
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a row sample")
        result["cpu_baseline"] = cpu_baseline(w)
        if fp8 and "value" in fp8:
            log("[bench] timing the FP8 CPU oracle on a row sample")
            fp8["cpu_baseline"] = cpu_baseline_fp8(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
