"""The C-ABI library loads, exports what include/tpmlp.h declares, and rejects bad
arguments before touching the GPU.

Every call here with made-up device addresses is invalid in at least one way
that the library checks before any HIP call, so none of them can reach a kernel.
"""
import ctypes
import os
import subprocess

import pytest

from tensor_transformer_mlp_03_amd import _lib as L

def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


# Host-side validation tests.  They run where no GPU is visible, so that even a
# validation bug could not send a made-up address to a kernel.
pytestmark = [
    pytest.mark.skipif(not __import__("os").path.exists(L.LIB_PATH), reason="libtpmlp.so not built"),
    pytest.mark.skipif(_gpu_visible(), reason="made-up device addresses are only passed where no GPU is visible"),
]

OK, NULL, SHAPE, ALIGN, WS, SHARDS, HIP, UNSUP, ALIAS, NO_FORWARD = range(10)


def test_exports_every_declared_function():
    declared = L.header_functions()
    assert "tpmlp_fwd" in declared and "tpmlp_tp_bwd" in declared
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    lib = L.lib()
    for f in declared:
        assert hasattr(lib, f)
    assert set(declared) == set(L._SIGS)


def test_header_is_plain_c_and_links(tmp_path):
    """include/tpmlp.h compiles as C99 with no HIP or torch header, and a C program
    that calls the host-only entry points links against the library and runs (no
    GPU needed: workspace queries, names, argument errors)."""
    import shutil
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    src.write_text(r"""
#include <stdio.h>
#include "tpmlp.h"
int main(void) {
  if (tpmlp_abi_version() != TPMLP_ABI_VERSION) return 1;
  if (tpmlp_fwd_workspace_bytes(64, 256, 512) == 0) return 2;
  if (tpmlp_fwd_workspace_bytes(60, 256, 512) != 0) return 3;
  if (tpmlp_fwd(0, 0, 0, 0, 0, 64, 256, 512, 0, 0, 0) != TPMLP_ERR_NULL) return 4;
  if (tpmlp_recompute_policy(2048, 20480, 10240, (size_t)1 << 40) != 0) return 5;
  printf("%s|%s\n", tpmlp_status_str(TPMLP_ERR_ALIAS), tpmlp_kernel_name(TPMLP_K_FWD_FUSED));
  return 0;
}
""")
    exe = tmp_path / "abi"
    lib_dir = os.path.dirname(L.LIB_PATH)
    subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(L.HEADER), str(src), "-o", str(exe),
                    "-L", lib_dir, "-ltpmlp", "-Wl,-rpath," + lib_dir], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, (out.returncode, out.stderr)
    assert out.stdout.strip() == f"{L.tpmlp_status_str(8)}|fwd_fused"


def test_last_error_is_per_thread():
    """Argument errors from concurrent threads each leave their own detail in
    tpmlp_last_error (thread-local), never another thread's."""
    import threading
    bad = {"X": dict(X=None), "ws": dict(ws=None), "shape": dict(M=60), "align": dict(A=_p(1) + 2)}
    want = {"X": (NULL, "X"), "ws": (NULL, "ws"), "shape": (SHAPE, "multiples of 8"), "align": (ALIGN, "A_i")}
    errors = []

    def run(name):
        for _ in range(200):
            st, msg = _fwd(**bad[name])
            code, text = want[name]
            if st != code or text not in msg:
                errors.append((name, st, msg))
                return

    threads = [threading.Thread(target=run, args=(n,)) for n in bad for _ in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]


def test_version_and_strings():
    assert L.tpmlp_abi_version() == 12
    assert L.tpmlp_status_str(0) == "ok"
    assert L.tpmlp_status_str(ALIAS) == "output overlaps another buffer"
    assert L.tpmlp_status_str(99) == "unknown status"
    assert L.tpmlp_kernel_name(0) == "fwd_gemm1_gelu"
    assert L.tpmlp_kernel_name(99) == "?"


def _align(x, a=256):
    return (x + a - 1) // a * a


def test_workspace_queries():
    M, H, F = 4096, 1024, 4096
    fwd = L.tpmlp_fwd_workspace_bytes(M, H, F)
    assert fwd >= M * F * 2
    assert L.tpmlp_bwd_workspace_bytes(M, H, F, True) >= L.tpmlp_bwd_workspace_bytes(M, H, F, False) + M * F * 2
    assert L.tpmlp_bwd_workspace_bytes(M, H, F, False) >= 2 * M * F * 2
    tp = L.tpmlp_tp_workspace_bytes(4, M, H, F)
    assert tp >= 4 * M * H * 4 + L.tpmlp_bwd_workspace_bytes(M, H, F, True)
    for bad in ((0, H, F), (M, 12, F), (M, H, -8), (1 << 25, H, F)):
        assert L.tpmlp_fwd_workspace_bytes(*bad) == 0
        assert L.tpmlp_bwd_workspace_bytes(*bad, 1) == 0
    assert L.tpmlp_tp_workspace_bytes(0, M, H, F) == 0
    assert L.tpmlp_tp_workspace_bytes(65, M, H, F) == 0


FAKE = 1 << 40  # an address never dereferenced: every call below fails validation first


def _p(i):
    return FAKE + i * (1 << 34)


def _fwd(**kw):
    a = dict(X=_p(0), A=_p(1), B=_p(2), Z=_p(3), P=None, M=64, H=256, F=512, ws=_p(4), wsb=1 << 30)
    a.update(kw)
    st = L.lib().tpmlp_fwd(a["X"], a["A"], a["B"], a["Z"], a["P"], a["M"], a["H"], a["F"], a["ws"], a["wsb"], None)
    return st, L.lib().tpmlp_last_error().decode()


def test_fwd_argument_errors():
    assert _fwd(X=None)[0] == NULL
    assert _fwd(ws=None)[0] == NULL
    assert _fwd(A=_p(1) + 2)[0] == ALIGN
    assert _fwd(P=_p(5) + 8)[0] == ALIGN
    for M, H, F in ((0, 256, 512), (60, 256, 512), (64, 250, 512), (64, 256, 0), (1 << 25, 256, 512)):
        st, msg = _fwd(M=M, H=H, F=F)
        assert st == SHAPE and "multiples of 8" in msg
    need = L.tpmlp_fwd_workspace_bytes(64, 256, 512)
    assert _fwd(wsb=need - 1)[0] == WS
    # outputs overlapping inputs or each other
    assert _fwd(Z=_p(0) + 64)[0] == ALIAS            # Z inside X
    assert _fwd(ws=_p(3) + 1024)[0] == ALIAS         # workspace inside Z
    assert _fwd(P=_p(2))[0] == ALIAS                 # P_save on B_i
    st, msg = _fwd(Z=_p(1))
    assert st == ALIAS and "Z_i" in msg


def _fwd_noalloc(**kw):
    a = dict(X=_p(0), A=_p(1), B=_p(2), Z=_p(3), P=None, M=64, H=256, F=512)
    a.update(kw)
    st = L.lib().tpmlp_fwd_noalloc(a["X"], a["A"], a["B"], a["Z"], a["P"], a["M"], a["H"], a["F"], None)
    return st, L.lib().tpmlp_last_error().decode()


def test_fwd_noalloc_argument_errors():
    """The no-allocation forward checks its arguments as tpmlp_fwd does, and rejects
    shapes whose forward workspace exceeds the scratch array's fixed size before
    any HIP call; a valid small shape gets as far as the device check."""
    assert _fwd_noalloc(X=None)[0] == NULL
    assert _fwd_noalloc(Z=_p(3) + 4)[0] == ALIGN
    assert _fwd_noalloc(M=60)[0] == SHAPE
    assert _fwd_noalloc(Z=_p(0) + 64)[0] == ALIAS
    for M, H, F in ((32768, 3584, 3584), (2048, 20480, 10240)):
        assert L.tpmlp_fwd_workspace_bytes(M, H, F) > L.NOALLOC_SCRATCH_BYTES
        st, msg = _fwd_noalloc(M=M, H=H, F=F)
        assert st == WS and "TPMLP_NOALLOC_SCRATCH_BYTES" in msg
    # the GPT-2-medium-like shape fits
    assert L.tpmlp_fwd_workspace_bytes(4096, 1024, 4096) <= L.NOALLOC_SCRATCH_BYTES
    assert _fwd_noalloc(M=4096, H=1024, F=4096)[0] in (HIP, UNSUP)  # no GPU here


def test_python_wrappers_check_tensors():
    """The binding rejects tensors of the wrong dtype, layout or shape before it
    calls the library (CPU tensors; nothing reaches a C entry point)."""
    torch = pytest.importorskip("torch")
    bf = dict(dtype=torch.bfloat16)
    M, H, F, t = 16, 32, 24, 2
    X = torch.zeros((M, H), **bf)
    A = torch.zeros((H, t * F), **bf)
    B = torch.zeros((t * F, H), **bf)
    Z = torch.zeros((M, H))
    ws = torch.zeros(8, dtype=torch.uint8)
    with pytest.raises(ValueError, match="multiple of t"):
        L.tpmlp_tp_fwd_full(X, A[:, :t * F - 1], B, None, Z, t, ws, stream=0)
    with pytest.raises(ValueError, match="shape"):
        L.tpmlp_tp_fwd_full(X, A, B[:-8], None, Z, t, ws, stream=0)
    with pytest.raises(TypeError, match="float32"):
        L.tpmlp_tp_fwd_full(X, A, B, None, Z.double(), t, ws, stream=0)
    shards_A = [A[:, i * F:(i + 1) * F] for i in range(t)]  # strided views
    shards_B = [B[i * F:(i + 1) * F] for i in range(t)]
    with pytest.raises(ValueError, match="contiguous"):
        L.tpmlp_tp_fwd(X, shards_A, shards_B, None, None, Z, ws, stream=0)
    shards_A = [a.contiguous() for a in shards_A]
    with pytest.raises(ValueError, match="shape"):
        L.tpmlp_tp_fwd(X, shards_A, [shards_B[0], shards_B[1][:8]], None, None, Z, ws, stream=0)
    with pytest.raises(ValueError, match="entries"):
        L.tpmlp_tp_fwd(X, shards_A, shards_B, [None], None, Z, ws, stream=0)
    with pytest.raises(ValueError, match="shape"):
        L.tpmlp_fwd(X, shards_A[0], shards_B[0], torch.zeros((M, H + 8)), None, ws, stream=0)


def _bwd(**kw):
    a = dict(dZ=_p(0), X=_p(1), A=_p(2), B=_p(3), P=None, dX=_p(4), dA=_p(5), dB=_p(6), M=64, H=256, F=512,
             ws=_p(7), wsb=1 << 30)
    a.update(kw)
    return L.lib().tpmlp_bwd(a["dZ"], a["X"], a["A"], a["B"], a["P"], a["dX"], a["dA"], a["dB"], a["M"], a["H"],
                             a["F"], a["ws"], a["wsb"], None)


def test_bwd_argument_errors():
    assert _bwd(dZ=None) == NULL
    assert _bwd(dB=None) == NULL
    assert _bwd(dA=_p(5) + 4) == ALIGN
    assert _bwd(M=7) == SHAPE
    # recompute needs more workspace than the stored pre-activation
    need_rc = L.tpmlp_bwd_workspace_bytes(64, 256, 512, True)
    need_st = L.tpmlp_bwd_workspace_bytes(64, 256, 512, False)
    assert _bwd(wsb=need_rc - 1) == WS
    assert _bwd(P=_p(8), wsb=need_st - 1) == WS
    assert _bwd(dA=_p(6)) == ALIAS                   # dA on dB
    assert _bwd(dX=_p(8), P=_p(8)) == ALIAS          # dX on P_saved
    assert _bwd(ws=_p(1)) == ALIAS                   # workspace on X


def _arr(ptrs):
    arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
    return ctypes.cast(arr, L._PP)


def test_tp_argument_errors():
    lib = L.lib()
    t, M, H, F = 4, 64, 256, 128
    A = _arr([_p(10 + i) for i in range(t)])
    B = _arr([_p(20 + i) for i in range(t)])
    assert lib.tpmlp_tp_fwd(_p(0), None, B, None, None, _p(1), t, M, H, F, _p(2), 1 << 40, None) == NULL
    assert lib.tpmlp_tp_fwd(_p(0), A, B, None, None, _p(1), 0, M, H, F, _p(2), 1 << 40, None) == SHARDS
    assert lib.tpmlp_tp_fwd(_p(0), A, B, None, None, _p(1), 65, M, H, F, _p(2), 1 << 40, None) == SHARDS
    need = L.tpmlp_tp_workspace_bytes(t, M, H, F)
    assert lib.tpmlp_tp_fwd(_p(0), A, B, None, None, _p(1), t, M, H, F, _p(2), need - 1, None) == WS
    Abad = _arr([_p(10), None, _p(12), _p(13)])
    assert lib.tpmlp_tp_fwd(_p(0), Abad, B, None, None, _p(1), t, M, H, F, _p(2), need, None) == NULL
    Bsame = _arr([_p(10)] + [_p(21 + i) for i in range(t - 1)])  # B_0 is A_0: fine, both inputs
    Zsh = _arr([_p(30), _p(30), None, None])                         # two partials on one buffer
    assert lib.tpmlp_tp_fwd(_p(0), A, Bsame, None, Zsh, _p(1), t, M, H, F, _p(2), need - 1, None) == WS
    assert lib.tpmlp_tp_fwd(_p(0), A, B, None, Zsh, _p(1), t, M, H, F, _p(2), need, None) == ALIAS
    dA = _arr([_p(40 + i) for i in range(t)])
    dB = _arr([_p(50 + i) for i in range(t)])
    assert lib.tpmlp_tp_bwd(_p(0), _p(3), A, B, None, dA, None, None, _p(1), t, M, H, F, _p(2), need, None) == NULL
    Pbad = _arr([_p(60), None, _p(62), _p(63)])
    assert lib.tpmlp_tp_bwd(_p(0), _p(3), A, B, Pbad, dA, dB, None, _p(1), t, M, H, F, _p(2), need, None) == NULL
    dBov = _arr([_p(40)] + [_p(51 + i) for i in range(t - 1)])       # dB_0 on dA_0
    assert lib.tpmlp_tp_bwd(_p(0), _p(3), A, B, None, dA, dBov, None, _p(1), t, M, H, F, _p(2), need, None) == ALIAS


def test_dimension_limit():
    """Dimensions up to 2^23 are accepted (workspace queries answer), one step more is
    not: operand offsets of up to 128 rows must fit the 2^31-byte buffer range."""
    assert L.tpmlp_fwd_workspace_bytes(8, 8, 1 << 23) > 0
    assert L.tpmlp_fwd_workspace_bytes(8, 8, (1 << 23) + 8) == 0
    assert L.tpmlp_bwd_workspace_bytes((1 << 23) + 8, 8, 8, 1) == 0
    assert _fwd(H=(1 << 23) + 8)[0] == SHAPE


def test_activation_accounting_and_policy():
    """Saved activations per rank: X always, P_i unless recomputed; the policy keeps
    P_i when it fits and recomputes only when the smaller footprint alone fits."""
    M, H, F = 2048, 20480, 10240  # a 530B-class rank shard
    x, p = M * H * 2, M * F * 2
    assert L.tpmlp_saved_activation_bytes(M, H, F, False) == x + p
    assert L.tpmlp_saved_activation_bytes(M, H, F, True) == x
    assert L.tpmlp_saved_activation_bytes(M, H, 12, True) == 0
    assert L.tpmlp_recompute_policy(M, H, F, x + p) == 0
    assert L.tpmlp_recompute_policy(M, H, F, x + p - 1) == 1
    assert L.tpmlp_recompute_policy(M, H, F, x) == 1
    assert L.tpmlp_recompute_policy(M, H, F, x - 1) == -1
    assert L.tpmlp_recompute_policy(0, H, F, 1 << 60) == -1


def test_tp_full_argument_errors():
    """The whole-weight drivers check their arguments before any HIP call."""
    lib = L.lib()
    t, M, H, F = 4, 64, 256, 128
    need = L.tpmlp_tp_workspace_bytes(t, M, H, F)
    X, A, B, Z, ws = _p(0), _p(1), _p(2), _p(3), _p(4)
    assert lib.tpmlp_tp_fwd_full(X, None, B, None, Z, t, M, H, F, ws, need, None) == NULL
    assert lib.tpmlp_tp_fwd_full(X, A, B, None, Z, 0, M, H, F, ws, need, None) == SHARDS
    assert lib.tpmlp_tp_fwd_full(X, A, B, None, Z, t, M, H, 12, ws, need, None) == SHAPE
    assert lib.tpmlp_tp_fwd_full(X, A, B, None, Z, 8, M, H, 1 << 21, ws, 1 << 62, None) == SHAPE  # t F_i > 2^23
    assert lib.tpmlp_tp_fwd_full(X, A, B, None, Z, t, M, H, F, ws, need - 1, None) == WS
    assert lib.tpmlp_tp_fwd_full(X, A + 8, B, None, Z, t, M, H, F, ws, need, None) == ALIGN
    # Z inside the whole A (H t F_i bf16 elements from A): overlap
    assert lib.tpmlp_tp_fwd_full(X, A, B, None, A + 1024 * 16, t, M, H, F, ws, need, None) == ALIAS
    dA, dB, dX = _p(5), _p(6), _p(7)
    assert lib.tpmlp_tp_bwd_full(X, X, A, B, None, None, dB, dX, t, M, H, F, ws, need, None) == NULL
    assert lib.tpmlp_tp_bwd_full(X, X, A, B, None, dA, dB, dX, 65, M, H, F, ws, need, None) == SHARDS
    # dB starting inside dA (H t F_i float32 elements): overlap
    assert lib.tpmlp_tp_bwd_full(X, X, A, B, None, dA, dA + 4096, dX, t, M, H, F, ws, need, None) == ALIAS
    # P inside dA: an input overlapping an output
    assert lib.tpmlp_tp_bwd_full(X, X, A, B, dA + 4096, dA, dB, dX, t, M, H, F, ws, need, None) == ALIAS


def test_shard_sum_argument_errors():
    lib = L.lib()
    parts = _arr([_p(0), _p(1)])
    assert lib.tpmlp_shard_sum(None, 2, _p(2), 1024, None) == NULL
    assert lib.tpmlp_shard_sum(parts, 0, _p(2), 1024, None) == SHARDS
    assert lib.tpmlp_shard_sum(parts, 2, _p(2), 1022, None) == SHAPE
    assert lib.tpmlp_shard_sum(parts, 2, _p(2) + 4, 1024, None) == ALIGN
    assert lib.tpmlp_shard_sum(parts, 2, _p(1) + 16, 1024, None) == ALIAS


def test_timing_argument_errors():
    lib = L.lib()
    assert lib.tpmlp_timing_begin(0) == SHAPE
    assert lib.tpmlp_timing_begin_kinds(8, 0) == SHAPE
    assert lib.tpmlp_timing_begin_kinds(8, 1 << L.KERNEL_COUNT) == SHAPE
    assert lib.tpmlp_timing_begin_kinds(0, 1) == SHAPE
    assert lib.tpmlp_timing_end(None, None, None) == NULL


def _sp(fn, t=2, M=128, H=64, F=64, **kw):
    arr = lambda base: L._ptr_array([_p(base + i) for i in range(t)], t)
    ws = kw.pop("ws", _p(40))
    wsb = kw.pop("wsb", 1 << 30)
    if fn == "fwd":
        a = dict(X=arr(0), A=arr(10), B=arr(20), P=None, Z=arr(30))
        a.update(kw)
        st = L.lib().tpmlp_sp_fwd(a["X"], a["A"], a["B"], a["P"], a["Z"], t, M, H, F, ws, wsb, None)
    else:
        a = dict(dZ=arr(0), X=arr(8), A=arr(16), B=arr(24), P=None, dA=arr(32), dB=arr(44), dX=arr(52))
        a.update(kw)
        st = L.lib().tpmlp_sp_bwd(a["dZ"], a["X"], a["A"], a["B"], a["P"], a["dA"], a["dB"], a["dX"], t, M, H, F,
                                  ws, wsb, None)
    return st, L.lib().tpmlp_last_error().decode()


def test_sp_argument_errors():
    """The sequence-parallel calls reject bad slices before any HIP call: NULL
    arrays and entries, token counts that do not split into slices of multiples
    of 8 rows, a short workspace, and overlapping outputs."""
    for fn in ("fwd", "bwd"):
        key = "X" if fn == "fwd" else "dZ"
        assert _sp(fn, **{key: None})[0] == NULL
        st, msg = _sp(fn, M=120, t=4)   # 30 rows per slice
        assert st == SHAPE and "row slices" in msg
        assert _sp(fn, M=96, t=4)[0] in (HIP, UNSUP)  # 24 rows per slice: valid, reaches the device check
        assert _sp(fn, t=0)[0] == SHARDS
        need = L.tpmlp_sp_workspace_bytes(2, 128, 64, 64)
        assert _sp(fn, wsb=need - 1)[0] == WS
    # an output slice on top of an input slice
    arr = L._ptr_array([_p(0), _p(30)], 2)
    st, msg = _sp("fwd", Z=arr)
    assert st == ALIAS and "Z_sl" in msg
    st, _ = _sp("fwd", H=(1 << 22) + 8)
    assert st == SHAPE


def test_sp_workspace_query():
    assert L.tpmlp_sp_workspace_bytes(4, 32768, 3584, 3584) > 0
    assert L.tpmlp_sp_workspace_bytes(4, 32768 + 8, 3584, 3584) == 0  # not a multiple of t
    assert L.tpmlp_sp_workspace_bytes(4, 96, 64, 64) > 0
    assert L.tpmlp_sp_workspace_bytes(3, 96, 64, 64) > 0     # 32 rows per slice
    assert L.tpmlp_sp_workspace_bytes(4, 48, 64, 64) == 0     # 12 rows per slice 


def _fp8(fn, t=2, M=128, H=64, F=96, **kw):
    arr = lambda base: L._ptr_array([_p(base + i) for i in range(t)], t)
    ws = kw.pop("ws", _p(60))
    wsb = kw.pop("wsb", 1 << 30)
    if fn == "fwd":
        a = dict(X=_p(0), A=arr(10), B=arr(20), P=None, Z=_p(30))
        a.update(kw)
        st = L.lib().tpmlp_fp8_tp_fwd(a["X"], a["A"], a["B"], a["P"], a["Z"], t, M, H, F, ws, wsb, None)
    else:
        a = dict(dZ=_p(0), X=_p(1), A=arr(10), B=arr(20), P=None, dA=arr(30), dB=arr(40), dX=_p(50))
        a.update(kw)
        st = L.lib().tpmlp_fp8_tp_bwd(a["dZ"], a["X"], a["A"], a["B"], a["P"], a["dA"], a["dB"], a["dX"], t, M, H,
                                      F, ws, wsb, None)
    return st, L.lib().tpmlp_last_error().decode()


def test_fp8_argument_errors():
    """The FP8 drivers check their arguments before any HIP call: NULL arrays and
    pointers, shard counts, dimensions that are not multiples of 16, a short
    workspace, misalignment and outputs that overlap inputs."""
    for fn in ("fwd", "bwd"):
        key = "X" if fn == "fwd" else "dZ"
        assert _fp8(fn, **{key: None})[0] == NULL
        assert _fp8(fn, A=None)[0] == NULL
        assert _fp8(fn, t=0)[0] == SHARDS
        st, msg = _fp8(fn, F=104)  # a multiple of 8 but not of 16
        assert st == SHAPE and "multiples of 16" in msg
        assert _fp8(fn, M=136)[0] == SHAPE
        need = L.tpmlp_fp8_workspace_bytes(2, 128, 64, 96)
        assert _fp8(fn, wsb=need - 1)[0] == WS
        assert _fp8(fn, ws=_p(60) + 8)[0] == ALIGN
    assert _fp8("fwd")[0] in (HIP, UNSUP)  # valid: reaches the device check
    # a backward needs the workspace of its forward (none has run here)
    st, msg = _fp8("bwd")
    assert st == NO_FORWARD and "no forward on this workspace" in msg
    st, msg = _fp8("fwd", Z=_p(0))  # Z on top of X
    assert st == ALIAS
    st, msg = _fp8("bwd", dX=_p(1))
    assert st == ALIAS
    # the quantizer
    q = lambda **kw: L.lib().tpmlp_fp8_quantize(kw.get("T", _p(0)), kw.get("R", 64), kw.get("C", 32),
                                                kw.get("fmt", 0), kw.get("tr", 0), kw.get("codes", _p(1)),
                                                kw.get("amax", _p(2)), None)
    assert q(T=None) == NULL and q(amax=None) == NULL
    assert q(R=40) == SHAPE and q(fmt=2) == SHAPE
    assert q(codes=_p(0)) == ALIAS
    assert q() in (HIP, UNSUP)


def test_fp8_workspace_query():
    assert L.tpmlp_fp8_workspace_bytes(4, 32768, 3584, 3584) > 0
    assert L.tpmlp_fp8_workspace_bytes(1, 64, 256, 512) > 0
    assert L.tpmlp_fp8_workspace_bytes(1, 64, 256, 520) == 0   # F_i not a multiple of 16
    assert L.tpmlp_fp8_workspace_bytes(0, 64, 256, 512) == 0
    assert L.tpmlp_fp8_workspace_bytes(65, 64, 256, 512) == 0
    # per shard the workspace keeps the weight codes in both layouts and G_i^T's
    # codes for the backward: 4 H F_i + M F_i bytes, plus four amax slots of 2 KiB
    grow = L.tpmlp_fp8_workspace_bytes(8, 2048, 4096, 2048) - L.tpmlp_fp8_workspace_bytes(1, 2048, 4096, 2048)
    per_shard = 4 * 4096 * 2048 + 2048 * 2048
    assert 7 * per_shard <= grow <= 7 * (per_shard + 4 * 2048) + 4096
