"""libtpmlp: one tensor-parallel rank's share of the transformer MLP on MI355X (gfx950).

The compute path is the HIP library ``libtpmlp.so`` (C ABI in ``include/tpmlp.h``);
``_lib`` binds it with ctypes.  Importing the package does not load the library;
the first call does, and fails loudly if it has not been built.
"""
from ._lib import (  # noqa: F401
    TpmlpError,
    lib,
    tpmlp_abi_version,
    tpmlp_bwd,
    tpmlp_bwd_workspace_bytes,
    tpmlp_fwd,
    tpmlp_fwd_workspace_bytes,
    tpmlp_kernel_name,
    tpmlp_shard_sum,
    tpmlp_status_str,
    tpmlp_timing_begin,
    tpmlp_timing_end,
    tpmlp_timing_records,
    tpmlp_tp_bwd,
    tpmlp_tp_fwd,
    tpmlp_tp_workspace_bytes,
)
