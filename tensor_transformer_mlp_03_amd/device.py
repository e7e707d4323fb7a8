"""Device-side setup of one workload for the library: uploads the seeded bf16
inputs, allocates outputs and the workspace with torch (memory only), and calls
the C ABI.  No arithmetic of the method happens here.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np

from . import _lib as L
from .inputs import Inputs


def to_device(bits: Optional[np.ndarray], device="cuda"):
    """uint16 bf16 bits -> an int16 device tensor holding the same bits."""
    import torch
    if bits is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)


def bits_of(t) -> np.ndarray:
    """Device int16/bf16 tensor -> uint16 numpy bits."""
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceMLP:
    """All buffers of one workload on the GPU.

    ``shards``: which weight shards to place (default: those generated in
    ``inputs``).  ``store_p``: keep the pre-activation from the forward (True) or
    recompute it in the backward (False).  ``driver``: run the shards through the
    t-shard driver (partials summed into Z and dX); otherwise each shard is one
    rank's ``tpmlp_fwd`` / ``tpmlp_bwd`` call with its own outputs.
    """

    def __init__(self, inputs: Inputs, store_p: bool = True, driver: bool = True, shards=None,
                 keep_partials: bool = False, device="cuda", full_weights: bool = False):
        import torch
        w = inputs.workload
        self.w, self.device, self.store_p, self.driver = w, device, store_p, driver
        self.full = full_weights
        if full_weights and (not driver or keep_partials):
            raise ValueError("full_weights runs the t-shard driver over whole weights, without per-shard partials")
        self.M, self.H, self.F = w.M, w.H, w.F_i
        self.shards = [i for i in range(w.t) if inputs.A[i] is not None] if shards is None else list(shards)
        if driver and len(self.shards) != w.t:
            raise ValueError("the t-shard driver needs every shard")
        f32 = dict(dtype=torch.float32, device=device)
        bf = dict(dtype=torch.int16, device=device)
        self.X = to_device(inputs.X, device)
        self.dZ = to_device(inputs.dZ, device) if w.backward else None
        self.A: List = [to_device(inputs.A[i], device) for i in self.shards]
        self.B: List = [to_device(inputs.B[i], device) for i in self.shards]
        n = len(self.shards)
        M, H, F = self.M, self.H, self.F
        self.P = [torch.empty((M, F), **bf) for _ in range(n)] if store_p else None
        self.Z_sh = [torch.empty((M, H), **f32) for _ in range(n)] if (keep_partials or not driver) else None
        self.Z = torch.empty((M, H), **f32) if driver else None
        if w.backward:
            self.dA = [torch.empty((H, F), **f32) for _ in range(n)]
            self.dB = [torch.empty((F, H), **f32) for _ in range(n)]
            self.dX_sh = [torch.empty((M, H), **f32) for _ in range(n)] if (keep_partials or not driver) else None
            self.dX = torch.empty((M, H), **f32) if driver else None
        if full_weights:
            # The whole weights A[H, t F_i] and B[t F_i, H]; the per-shard lists become
            # views into them (and into the whole P, dA and dB).
            self.Af = torch.cat(self.A, 1).contiguous()
            self.Bf = torch.cat(self.B, 0).contiguous()
            self.A = [self.Af[:, j * F:(j + 1) * F] for j in range(n)]
            self.B = [self.Bf[j * F:(j + 1) * F] for j in range(n)]
            if store_p:
                self.Pf = torch.empty((n, M, F), **bf)
                self.P = [self.Pf[j] for j in range(n)]
            if w.backward:
                self.dAf = torch.empty((H, n * F), **f32)
                self.dBf = torch.empty((n * F, H), **f32)
                self.dA = [self.dAf[:, j * F:(j + 1) * F] for j in range(n)]
                self.dB = [self.dBf[j * F:(j + 1) * F] for j in range(n)]
        if driver:
            ws = L.tpmlp_tp_workspace_bytes(n, M, H, F)
        else:
            ws = max(L.tpmlp_fwd_workspace_bytes(M, H, F), L.tpmlp_bwd_workspace_bytes(M, H, F, not store_p))
        self.ws = torch.empty(ws, dtype=torch.uint8, device=device)

    def forward(self, stream=None):
        if self.full:
            L.tpmlp_tp_fwd_full(self.X, self.Af, self.Bf, self.Pf if self.store_p else None, self.Z,
                                len(self.shards), self.ws, stream)
        elif self.driver:
            L.tpmlp_tp_fwd(self.X, self.A, self.B, self.P, self.Z_sh, self.Z, self.ws, stream)
        else:
            for j in range(len(self.shards)):
                L.tpmlp_fwd(self.X, self.A[j], self.B[j], self.Z_sh[j], self.P[j] if self.P else None, self.ws,
                            stream)

    def backward(self, stream=None):
        if self.full:
            L.tpmlp_tp_bwd_full(self.dZ, self.X, self.Af, self.Bf, self.Pf if self.store_p else None, self.dAf,
                                self.dBf, self.dX, len(self.shards), self.ws, stream)
        elif self.driver:
            L.tpmlp_tp_bwd(self.dZ, self.X, self.A, self.B, self.P, self.dA, self.dB, self.dX_sh, self.dX, self.ws,
                           stream)
        else:
            for j in range(len(self.shards)):
                L.tpmlp_bwd(self.dZ, self.X, self.A[j], self.B[j], self.P[j] if self.P else None, self.dX_sh[j],
                            self.dA[j], self.dB[j], self.ws, stream)

    def step(self, stream=None):
        self.forward(stream)
        if self.w.backward:
            self.backward(stream)

    def capture(self):
        """One step captured into a HIP graph (torch.cuda.CUDAGraph) on a side stream
        of default priority.  Replaying it reruns the step's kernel launches on the
        same buffers with no host work per launch, for workloads whose step time is
        launch latency.  The library's calls enqueue kernels only (no memset, no
        allocation, no host synchronisation), so the whole step can be captured."""
        import torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            self.step()
        torch.cuda.current_stream().wait_stream(s)
        return g


class DeviceFp8MLP:
    """Buffers of one workload for the FP8 path: bf16 inputs, float32 outputs, the
    stored bf16 pre-activations (unless recomputed) and the FP8 workspace; ``step``
    runs tpmlp_fp8_tp_fwd then tpmlp_fp8_tp_bwd over the placed shards (their
    partials summed into Z and dX)."""

    def __init__(self, inputs: Inputs, store_p: bool = True, device="cuda"):
        import torch
        w = inputs.workload
        self.shards = [i for i in range(w.t) if inputs.A[i] is not None]
        M, H, F = w.M, w.H, w.F_i
        n = len(self.shards)
        f32 = dict(dtype=torch.float32, device=device)
        self.X = to_device(inputs.X, device)
        self.dZ = to_device(inputs.dZ, device)
        self.A = [to_device(inputs.A[i], device) for i in self.shards]
        self.B = [to_device(inputs.B[i], device) for i in self.shards]
        self.P = [torch.empty((M, F), dtype=torch.int16, device=device) for _ in range(n)] if store_p else None
        self.Z = torch.empty((M, H), **f32)
        self.dX = torch.empty((M, H), **f32)
        self.dA = [torch.empty((H, F), **f32) for _ in range(n)]
        self.dB = [torch.empty((F, H), **f32) for _ in range(n)]
        self.ws = torch.empty(L.tpmlp_fp8_workspace_bytes(n, M, H, F), dtype=torch.uint8, device=device)

    def forward(self):
        L.tpmlp_fp8_tp_fwd(self.X, self.A, self.B, self.P, self.Z, self.ws)

    def backward(self):
        L.tpmlp_fp8_tp_bwd(self.dZ, self.X, self.A, self.B, self.P, self.dA, self.dB, self.dX, self.ws)

    def step(self):
        self.forward()
        self.backward()
