"""Host-only checks of the C ABI (no GPU needed).

The library must load, export every function declared in include/moe.h, and
reject invalid calls with the documented status before touching HIP.  Fake
device addresses are fine here: validation fails before anything is launched.
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import combine_router_top_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(M.LIB_PATH), reason="libmoe.so not built")

FAKE = 0x10000  # 16-byte aligned fake device address (never dereferenced)


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    L = ctypes.CDLL(M.LIB_PATH)
    names = declared_functions()
    assert set(names) == set(M.EXPORTED), names
    for n in names:
        assert hasattr(L, n), n
    assert M.lib().moe_version().startswith(b"libmoe")


def test_header_compiles_as_c():
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", HEADER],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def _p(**kw):
    base = dict(T=64, d=128, E=8, k=2, f=256, expert_lo=0, n_local=8, dtype=M.MOE_DTYPE_F32, flags=0)
    base.update(kw)
    return M.Problem(**base)


def _route(p, x=FAKE, wg=FAKE, idx=FAKE, w=FAKE, ws=FAKE, wsb=1 << 30):
    return M.lib().moe_route(ctypes.byref(p), x, wg, None, None, idx, w, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), M.MOE_ERR_INVALID_ARG),
    (dict(d=-8), M.MOE_ERR_INVALID_ARG),
    (dict(k=9), M.MOE_ERR_INVALID_ARG),            # k > E
    (dict(k=0), M.MOE_ERR_INVALID_ARG),
    (dict(expert_lo=4, n_local=5), M.MOE_ERR_INVALID_ARG),
    (dict(n_local=0), M.MOE_ERR_INVALID_ARG),
    (dict(expert_lo=-1), M.MOE_ERR_INVALID_ARG),
    (dict(flags=0x80), M.MOE_ERR_INVALID_ARG),
    (dict(d=100), M.MOE_ERR_UNSUPPORTED),          # d % 8
    (dict(f=12), M.MOE_ERR_UNSUPPORTED),           # f % 8
    (dict(E=64, k=33, n_local=64), M.MOE_ERR_UNSUPPORTED),
    (dict(E=1025, n_local=8), M.MOE_ERR_UNSUPPORTED),
    (dict(dtype=7), M.MOE_ERR_UNSUPPORTED),
])
def test_problem_validation(kw, status):
    assert _route(_p(**kw)) == status
    assert M.lib().moe_last_error()
    assert M.lib().moe_workspace_bytes(ctypes.byref(_p(**kw)), M.MOE_CALL_LAYER) == 0


def test_null_problem():
    assert M.lib().moe_route(None, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, 1 << 30, None) == \
        M.MOE_ERR_INVALID_ARG


def test_null_and_misaligned_pointers():
    p = _p()
    assert _route(p, x=0) == M.MOE_ERR_INVALID_ARG
    assert b"x is NULL" in M.lib().moe_last_error()
    assert _route(p, idx=0) == M.MOE_ERR_INVALID_ARG
    assert _route(p, x=FAKE + 2) == M.MOE_ERR_UNSUPPORTED
    assert b"aligned" in M.lib().moe_last_error()
    L = M.lib()
    assert L.moe_combine(ctypes.byref(p), FAKE, 0, FAKE, FAKE, None) == M.MOE_ERR_INVALID_ARG
    assert L.moe_expert_gemm(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, None, 0,
                             None) == M.MOE_ERR_INVALID_ARG
    assert L.moe_dispatch(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1 << 30,
                          None) == M.MOE_ERR_INVALID_ARG


def test_empty_batch_host():
    """T = 0 is a valid empty batch: no workspace, T-sized pointers may be
    NULL, and route / expert GEMM / combine return at once (nothing to launch;
    dispatch and the layer clear counts and offsets, covered on the GPU).  The
    weights are still checked; the padded calls reject T = 0 (no capacity in
    1 .. T)."""
    L = M.lib()
    p = _p(T=0)
    for call in range(M.MOE_CALL_ROUTE, M.MOE_CALL_EXPERT_GEMM_PADDED + 1):
        assert L.moe_workspace_bytes(ctypes.byref(p), call) == 0
        assert L.moe_last_error() == b""
    assert _route(p, x=0, idx=0, w=0, ws=0, wsb=0) == M.MOE_OK
    assert _route(p, x=0, wg=0, idx=0, w=0, ws=0, wsb=0) == M.MOE_ERR_INVALID_ARG
    assert L.moe_expert_gemm(ctypes.byref(p), 0, FAKE, FAKE, FAKE, FAKE, 0, 0, None, 0, None) == M.MOE_OK
    assert L.moe_expert_gemm(ctypes.byref(p), 0, FAKE, FAKE, FAKE, 0, 0, 0, None, 0, None) == \
        M.MOE_ERR_INVALID_ARG
    assert L.moe_combine(ctypes.byref(p), 0, 0, 0, 0, None) == M.MOE_OK
    assert L.moe_dispatch(ctypes.byref(p), 0, 0, 0, FAKE, 0, 0, 0, None, 0, None) == \
        M.MOE_ERR_INVALID_ARG                                    # counts_all is still required
    assert L.moe_dispatch_padded(ctypes.byref(p), 1, 0, 0, FAKE, FAKE, 0, 0, 0, None, 0, None) == \
        M.MOE_ERR_INVALID_ARG
    assert b"capacity" in L.moe_last_error()


def test_workspace_checks():
    p = _p()
    need = M.lib().moe_workspace_bytes(ctypes.byref(p), M.MOE_CALL_ROUTE)
    assert need >= 64 * 8 * 4
    assert _route(p, ws=0) == M.MOE_ERR_WORKSPACE
    assert _route(p, wsb=need - 1) == M.MOE_ERR_WORKSPACE
    assert _route(p, ws=FAKE + 16) == M.MOE_ERR_WORKSPACE       # not 256-byte aligned
    L = M.lib()
    lay = L.moe_workspace_bytes(ctypes.byref(p), M.MOE_CALL_LAYER)
    assert lay > need
    assert L.moe_layer(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                       lay - 1, None, None) == M.MOE_ERR_WORKSPACE
    assert L.moe_workspace_bytes(ctypes.byref(p), 99) == 0


def test_padded_calls_validate_capacity():
    """capacity must lie in [1, T]; the padded dispatch needs its workspace
    (the unpadded index plus the dispatch workspace); nothing is launched on
    an error."""
    p = _p()
    L = M.lib()
    need = L.moe_workspace_bytes(ctypes.byref(p), M.MOE_CALL_DISPATCH_PADDED)
    assert need >= L.moe_workspace_bytes(ctypes.byref(p), M.MOE_CALL_DISPATCH) + 64 * 2 * 4
    for cap in (0, -3, 65):
        assert L.moe_dispatch_padded(ctypes.byref(p), cap, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, need, None) == M.MOE_ERR_INVALID_ARG
        assert b"capacity" in L.moe_last_error()
        assert L.moe_expert_gemm_padded(ctypes.byref(p), cap, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        FAKE, None, 0, None) == M.MOE_ERR_INVALID_ARG
    assert L.moe_dispatch_padded(ctypes.byref(p), 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, need - 1, None) == M.MOE_ERR_WORKSPACE
    assert L.moe_dispatch_padded(ctypes.byref(p), 8, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE,
                                 FAKE, need, None) == M.MOE_ERR_INVALID_ARG
    assert L.moe_expert_gemm_padded(ctypes.byref(p), 8, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE,
                                    None, 0, None) == M.MOE_ERR_INVALID_ARG


def test_signal_calls_validate():
    """Shapes, pointers, epoch, scope, spin limit and workgroup count are
    checked on the host; nothing is launched on an error."""
    L = M.lib()
    assert L.moe_gemm_signal_tiles(300, 520) == 2 * 3
    assert L.moe_gemm_signal_tiles(0, 8) == 0
    ok = dict(M=300, N=520, K=264)
    def sig(M=300, N=520, K=264, A=FAKE, B=FAKE, C=FAKE, flags=FAKE, epoch=1, scope=0):
        return L.moe_gemm_signal(M, N, K, A, B, C, flags, epoch, scope, None)
    assert sig(M=0) == M.MOE_ERR_INVALID_ARG
    assert sig(N=100) == M.MOE_ERR_UNSUPPORTED
    assert sig(K=12) == M.MOE_ERR_UNSUPPORTED
    assert sig(K=1 << 20, N=1 << 11) == M.MOE_ERR_UNSUPPORTED   # B >= 2 GiB
    assert sig(flags=0) == M.MOE_ERR_INVALID_ARG
    assert sig(A=FAKE + 2) == M.MOE_ERR_UNSUPPORTED
    assert sig(epoch=0) == M.MOE_ERR_INVALID_ARG
    assert sig(scope=2) == M.MOE_ERR_INVALID_ARG
    def fwd(spin=100, wg=4, epoch=1, timeouts=FAKE, scope=0):
        return L.moe_tile_forward(300, 520, FAKE, FAKE, FAKE, epoch, spin, scope, timeouts, wg, None)
    assert fwd(spin=0) == M.MOE_ERR_INVALID_ARG
    assert fwd(wg=0) == M.MOE_ERR_INVALID_ARG and fwd(wg=2000) == M.MOE_ERR_INVALID_ARG
    assert fwd(epoch=0) == M.MOE_ERR_INVALID_ARG
    assert fwd(timeouts=0) == M.MOE_ERR_INVALID_ARG
    assert fwd(scope=-1) == M.MOE_ERR_INVALID_ARG


def test_write_logits_needs_buffer():
    p = _p(flags=M.MOE_F_WRITE_LOGITS)
    L = M.lib()
    lay = L.moe_workspace_bytes(ctypes.byref(p), M.MOE_CALL_LAYER)
    assert L.moe_layer(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, lay,
                       None, None) == M.MOE_ERR_INVALID_ARG


def test_workspace_sizes_cover_worst_case():
    """The layer workspace holds every intermediate at rows_max = T*min(k, n_local)."""
    for (T, d, E, k, f, lo, n, dt) in [(4096, 7168, 256, 8, 2048, 0, 32, 1),
                                       (16384, 4096, 8, 2, 14336, 0, 8, 1),
                                       (64, 128, 8, 2, 256, 0, 8, 0)]:
        p = M.Problem(T, d, E, k, f, lo, n, dt, 0)
        es = 2 if dt == 1 else 4
        rows = T * min(k, n)
        lay = M.lib().moe_workspace_bytes(ctypes.byref(p), M.MOE_CALL_LAYER)
        assert lay >= rows * (2 * d + f) * es + rows * 4 + 3 * T * k * 4


def test_hip_error_path_without_gpu():
    """A valid call on a machine with no GPU returns MOE_ERR_HIP with a message
    (run in a child process so the HIP runtime state stays out of this one)."""
    code = r"""
import ctypes, sys
sys.path.insert(0, %r)
import combine_router_top_amd as M
p = M.Problem(64, 128, 8, 2, 256, 0, 8, 0, 0)
L = M.lib()
n = L.moe_workspace_bytes(ctypes.byref(p), 0)
st = L.moe_route(ctypes.byref(p), 0x10000, 0x10000, None, None, 0x10000, 0x10000, 0x10000, n, None)
print(st, L.moe_last_error().decode())
""" % ROOT
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is visible")
    except ImportError:
        pass
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, HIP_VISIBLE_DEVICES=""))
    assert r.returncode == 0, r.stderr
    st, msg = r.stdout.split(" ", 1)
    assert int(st) == M.MOE_ERR_HIP and "moe_route" in msg


def test_dispatch_noalloc_rejects_oversize():
    """The allocation-free dispatch holds ceil(T*k/1024) * E int32 histograms in
    a 1 MiB static array: larger problems are rejected on the host, before any
    HIP call; so are missing pointers."""
    L = M.lib()
    big = M.Problem(1 << 17, 64, 1024, 8, 64, 0, 64, M.MOE_DTYPE_BF16, 0)  # 1024 chunks x 1024 experts
    assert L.moe_dispatch_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  None) == M.MOE_ERR_UNSUPPORTED
    assert b"scratch" in L.moe_last_error()
    fits = M.Problem(1 << 17, 64, 256, 8, 64, 0, 64, M.MOE_DTYPE_BF16, 0)  # 1024 chunks x 256 experts
    assert L.moe_dispatch_noalloc(ctypes.byref(fits), FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE,
                                  None) == M.MOE_ERR_INVALID_ARG       # perm is NULL
    assert b"perm is NULL" in L.moe_last_error()


def test_layer_ws_offset_and_fold_flag():
    """The layer workspace's h and y_packed offsets lie inside it, 256-byte
    aligned, y_packed after h; unknown regions and empty batches are errors;
    MOE_F_FOLD_WEIGHT is a valid flag."""
    L = M.lib()
    p = M.Problem(300, 128, 16, 4, 64, 0, 8, M.MOE_DTYPE_BF16, M.MOE_F_FOLD_WEIGHT)
    total = L.moe_workspace_bytes(ctypes.byref(p), M.MOE_CALL_LAYER)
    assert total > 0 and L.moe_last_error() == b""
    oh = L.moe_layer_ws_offset(ctypes.byref(p), M.MOE_WS_H)
    oy = L.moe_layer_ws_offset(ctypes.byref(p), M.MOE_WS_Y_PACKED)
    rows = 300 * 4
    assert oh % 256 == 0 and oy % 256 == 0
    assert oh + rows * 64 * 2 <= oy and oy + rows * 128 * 2 <= total
    bad = ctypes.c_size_t(-1).value
    assert L.moe_layer_ws_offset(ctypes.byref(p), 7) == bad and b"region" in L.moe_last_error()
    empty = M.Problem(0, 128, 16, 4, 64, 0, 8, M.MOE_DTYPE_BF16, 0)
    assert L.moe_layer_ws_offset(ctypes.byref(empty), M.MOE_WS_H) == bad


def test_layer_gemm_events_hook_host():
    """The measurement hook takes NULL events (records nothing) and needs no GPU."""
    assert M.lib().moe_layer_set_gemm_events(None, None) == M.MOE_OK
    M.layer_set_gemm_events(0, 0)
