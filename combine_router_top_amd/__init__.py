"""Python binding of libmoe (MI355X / gfx950 MoE-layer hot path).

A thin ctypes layer over the C ABI in ``include/moe.h``: it checks tensor
shapes and dtypes, passes ``data_ptr()`` and the current HIP stream, and turns
status codes into exceptions.  Every step of the layer runs in the library's
HIP kernels; there is no fallback.  If ``libmoe.so`` has not been built, every
call raises.

Functions (same names as the C calls):
    route(p, x, w_gate, bias=None, want_logits=False) -> (topk_idx, topk_w[, logits])
    dispatch(p, topk_idx, x) -> dict(counts_all, offsets, perm, inv, x_packed)
    dispatch_noalloc(p, topk_idx, x) -> the same, with no workspace (static scratch)
    expert_gemm(p, x_packed, offsets, w1, w3, w2) -> (h, y_packed)
    combine(p, y_packed, inv, topk_w) -> y
    layer(p, x, w_gate, bias, w1, w3, w2, routing=False, overlap=False, fold_weight=False, ...)
        -> y or (y, dict)
    layer_ws_offset(p, MOE_WS_H | MOE_WS_Y_PACKED) -> byte offset in the layer workspace
    dispatch_padded(p, capacity, topk_idx, x) -> dict(counts_all, offsets, perm, inv, x_packed)
    expert_gemm_padded(p, capacity, x_packed, offsets, w1, w3, w2) -> (h, y_packed)
    gemm_signal(A, B, flags, epoch) -> C          (C = rnd(A B), a flag per 256 x 256 tile)
    tile_forward(C, dst, flags, epoch, spin_limit, timeouts, workgroups)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Dict, Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, 1, 2, 3, 4
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
MOE_F_WRITE_LOGITS, MOE_F_OVERLAP, MOE_F_FOLD_WEIGHT = 1, 2, 4
MOE_WS_H, MOE_WS_Y_PACKED = 0, 1
MOE_CALL_ROUTE, MOE_CALL_DISPATCH, MOE_CALL_EXPERT_GEMM, MOE_CALL_COMBINE, MOE_CALL_LAYER = range(5)
MOE_CALL_DISPATCH_PADDED, MOE_CALL_EXPERT_GEMM_PADDED = 5, 6
MOE_SCOPE_AGENT, MOE_SCOPE_SYSTEM = 0, 1

EXPORTED = ["moe_last_error", "moe_version", "moe_workspace_bytes", "moe_route", "moe_dispatch",
            "moe_expert_gemm", "moe_combine", "moe_layer", "moe_dispatch_padded",
            "moe_expert_gemm_padded", "moe_gemm_signal_tiles", "moe_gemm_signal", "moe_tile_forward",
            "moe_dispatch_noalloc", "moe_layer_ws_offset", "moe_layer_set_gemm_events"]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libmoe status {status}: {msg}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("f", ctypes.c_int32), ("expert_lo", ctypes.c_int32),
                ("n_local", ctypes.c_int32), ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class RoutingOut(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_idx", "topk_w", "logits", "counts_all", "offsets", "perm", "inv")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not built; run python -m combine_router_top_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        P = ctypes.POINTER(Problem)
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_version.restype = ctypes.c_char_p
        L.moe_workspace_bytes.argtypes = [P, i32]
        L.moe_workspace_bytes.restype = sz
        L.moe_layer_ws_offset.argtypes = [P, i32]
        L.moe_layer_ws_offset.restype = sz
        L.moe_layer_set_gemm_events.argtypes = [vp, vp]
        L.moe_route.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_dispatch.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_dispatch_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_expert_gemm.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_combine.argtypes = [P, vp, vp, vp, vp, vp]
        L.moe_layer.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(RoutingOut), vp, sz,
                                vp, vp]
        L.moe_dispatch_padded.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_expert_gemm_padded.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_gemm_signal_tiles.argtypes = [i32, i32]
        L.moe_gemm_signal_tiles.restype = ctypes.c_int64
        u32 = ctypes.c_uint32
        L.moe_gemm_signal.argtypes = [i32, i32, i32, vp, vp, vp, vp, u32, i32, vp]
        L.moe_tile_forward.argtypes = [i32, i32, vp, vp, vp, u32, u32, i32, vp, i32, vp]
        for n in ("moe_route", "moe_dispatch", "moe_expert_gemm", "moe_combine", "moe_layer",
                  "moe_dispatch_padded", "moe_expert_gemm_padded", "moe_gemm_signal",
                  "moe_tile_forward", "moe_dispatch_noalloc"):
            getattr(L, n).restype = i32
        _lib = L
    return _lib


def _check(st: int):
    if st != MOE_OK:
        raise MoeError(st, lib().moe_last_error().decode())


@dataclass(frozen=True)
class Spec:
    """Problem description (mirrors moe_problem_t)."""
    T: int
    d: int
    E: int
    k: int
    f: int
    expert_lo: int
    n_local: int
    dtype: str  # "bf16" or "f32"
    flags: int = 0

    @property
    def rows_max(self) -> int:
        return self.T * min(self.k, self.n_local)

    def c(self) -> Problem:
        return Problem(self.T, self.d, self.E, self.k, self.f, self.expert_lo, self.n_local,
                       MOE_DTYPE_BF16 if self.dtype == "bf16" else MOE_DTYPE_F32, self.flags)

    @staticmethod
    def of(w, flags: int = 0) -> "Spec":
        """From any object with T, d, E, k, f, expert_lo, n_local, dtype fields."""
        return Spec(w.T, w.d, w.E, w.k, w.f, w.expert_lo, w.n_local, w.dtype, flags)


def workspace_bytes(p: Spec, call: int = MOE_CALL_LAYER) -> int:
    pc = p.c()
    n = lib().moe_workspace_bytes(ctypes.byref(pc), call)
    if n == 0 and lib().moe_last_error():
        raise MoeError(MOE_ERR_INVALID_ARG, lib().moe_last_error().decode())
    return int(n)


# ---------------------------------------------------------------------------
# torch helpers (device memory and streams only)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dt(p: Spec):
    t = _torch()
    return t.bfloat16 if p.dtype == "bf16" else t.float32


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    t = _torch()
    s = stream if stream is not None else t.cuda.current_stream()
    return s.cuda_stream


def _need(t, shape, dtype, name):
    torch = _torch()
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    return t


def alloc_workspace(p: Spec, call: int = MOE_CALL_LAYER, device="cuda"):
    torch = _torch()
    n = workspace_bytes(p, call)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device) if n else None


# ---------------------------------------------------------------------------
# the five calls
# ---------------------------------------------------------------------------
def route(p: Spec, x, w_gate, bias=None, want_logits: bool = False, workspace=None, stream=None,
          out=None):
    torch = _torch()
    dt = _dt(p)
    _need(x, (p.T, p.d), dt, "x")
    _need(w_gate, (p.d, p.E), dt, "w_gate")
    if bias is not None:
        _need(bias, (p.E,), torch.float32, "bias")
    dev = x.device
    idx = torch.empty((p.T, p.k), dtype=torch.int32, device=dev) if out is None else out[0]
    w = torch.empty((p.T, p.k), dtype=torch.float32, device=dev) if out is None else out[1]
    logits = torch.empty((p.T, p.E), dtype=torch.float32, device=dev) if want_logits else None
    ws = workspace if workspace is not None else alloc_workspace(p, MOE_CALL_ROUTE, dev)
    pc = p.c()
    _check(lib().moe_route(ctypes.byref(pc), _ptr(x), _ptr(w_gate), _ptr(bias), _ptr(logits),
                           _ptr(idx), _ptr(w), _ptr(ws), 0 if ws is None else ws.numel(),
                           _stream(stream)))
    return (idx, w, logits) if want_logits else (idx, w)


def _dispatch_out(p: Spec, topk_idx, x, out):
    torch = _torch()
    dt = _dt(p)
    _need(topk_idx, (p.T, p.k), torch.int32, "topk_idx")
    _need(x, (p.T, p.d), dt, "x")
    dev = x.device
    o = out if out is not None else {
        "counts_all": torch.empty(p.E, dtype=torch.int32, device=dev),
        "offsets": torch.empty(p.n_local + 1, dtype=torch.int32, device=dev),
        "perm": torch.full((p.rows_max,), -7, dtype=torch.int32, device=dev),
        "inv": torch.empty(p.T * p.k, dtype=torch.int32, device=dev),
        "x_packed": torch.zeros((p.rows_max, p.d), dtype=dt, device=dev),
    }
    _need(o["counts_all"], (p.E,), torch.int32, "counts_all")
    _need(o["offsets"], (p.n_local + 1,), torch.int32, "offsets")
    _need(o["perm"], (p.rows_max,), torch.int32, "perm")
    _need(o["inv"], (p.T * p.k,), torch.int32, "inv")
    _need(o["x_packed"], (p.rows_max, p.d), dt, "x_packed")
    return o


def dispatch(p: Spec, topk_idx, x, workspace=None, stream=None, out=None) -> Dict[str, object]:
    """Returns counts_all, offsets, perm, inv, x_packed.  Fresh outputs are
    pre-filled (perm with -7, x_packed with 0) so that untouched rows are
    visible; ``out`` (a dict of the same tensors) is written in place."""
    o = _dispatch_out(p, topk_idx, x, out)
    ws = workspace if workspace is not None else alloc_workspace(p, MOE_CALL_DISPATCH, x.device)
    pc = p.c()
    _check(lib().moe_dispatch(ctypes.byref(pc), _ptr(topk_idx), _ptr(x), _ptr(o["counts_all"]),
                              _ptr(o["offsets"]), _ptr(o["perm"]), _ptr(o["inv"]),
                              _ptr(o["x_packed"]), _ptr(ws), 0 if ws is None else ws.numel(),
                              _stream(stream)))
    return o


def dispatch_noalloc(p: Spec, topk_idx, x, stream=None, out=None) -> Dict[str, object]:
    """moe_dispatch_noalloc: the same outputs as ``dispatch`` with no
    workspace (the library's static per-device scratch; calls that overlap on
    one device race)."""
    o = _dispatch_out(p, topk_idx, x, out)
    pc = p.c()
    _check(lib().moe_dispatch_noalloc(ctypes.byref(pc), _ptr(topk_idx), _ptr(x),
                                      _ptr(o["counts_all"]), _ptr(o["offsets"]), _ptr(o["perm"]),
                                      _ptr(o["inv"]), _ptr(o["x_packed"]), _stream(stream)))
    return o


def expert_gemm(p: Spec, x_packed, offsets, w1, w3, w2, workspace=None, stream=None, out=None):
    torch = _torch()
    dt = _dt(p)
    _need(x_packed, (p.rows_max, p.d), dt, "x_packed")
    _need(offsets, (p.n_local + 1,), torch.int32, "offsets")
    _need(w1, (p.n_local, p.d, p.f), dt, "w1")
    _need(w3, (p.n_local, p.d, p.f), dt, "w3")
    _need(w2, (p.n_local, p.f, p.d), dt, "w2")
    dev = x_packed.device
    if out is None:
        h = torch.zeros((p.rows_max, p.f), dtype=dt, device=dev)
        yp = torch.zeros((p.rows_max, p.d), dtype=dt, device=dev)
    else:
        h, yp = out
    ws = workspace if workspace is not None else alloc_workspace(p, MOE_CALL_EXPERT_GEMM, dev)
    pc = p.c()
    _check(lib().moe_expert_gemm(ctypes.byref(pc), _ptr(x_packed), _ptr(offsets), _ptr(w1),
                                 _ptr(w3), _ptr(w2), _ptr(h), _ptr(yp), _ptr(ws),
                                 0 if ws is None else ws.numel(), _stream(stream)))
    return h, yp


def combine(p: Spec, y_packed, inv, topk_w, stream=None, out=None, rows: Optional[int] = None):
    """``rows``: rows of y_packed (default rows_max; n_local * capacity for
    the padded layout).  ``topk_w=None`` sums the rows unweighted."""
    torch = _torch()
    dt = _dt(p)
    _need(y_packed, (p.rows_max if rows is None else rows, p.d), dt, "y_packed")
    _need(inv, (p.T * p.k,), torch.int32, "inv")
    if topk_w is not None:
        _need(topk_w, (p.T, p.k), torch.float32, "topk_w")
    y = torch.empty((p.T, p.d), dtype=dt, device=y_packed.device) if out is None else out
    pc = p.c()
    _check(lib().moe_combine(ctypes.byref(pc), _ptr(y_packed), _ptr(inv), _ptr(topk_w), _ptr(y),
                             _stream(stream)))
    return y


def dispatch_padded(p: Spec, capacity: int, topk_idx, x, workspace=None, stream=None,
                    out=None) -> Dict[str, object]:
    """Padded fixed-capacity dispatch: n_local * capacity rows.  Fresh
    outputs are pre-filled (perm with -7, x_packed with ones) so that
    rows the call fails to write are visible."""
    torch = _torch()
    dt = _dt(p)
    _need(topk_idx, (p.T, p.k), torch.int32, "topk_idx")
    _need(x, (p.T, p.d), dt, "x")
    rows = p.n_local * int(capacity)
    dev = x.device
    o = out if out is not None else {
        "counts_all": torch.empty(p.E, dtype=torch.int32, device=dev),
        "offsets": torch.empty(p.n_local + 1, dtype=torch.int32, device=dev),
        "perm": torch.full((rows,), -7, dtype=torch.int32, device=dev),
        "inv": torch.empty(p.T * p.k, dtype=torch.int32, device=dev),
        "x_packed": torch.ones((rows, p.d), dtype=dt, device=dev),
    }
    _need(o["counts_all"], (p.E,), torch.int32, "counts_all")
    _need(o["offsets"], (p.n_local + 1,), torch.int32, "offsets")
    _need(o["perm"], (rows,), torch.int32, "perm")
    _need(o["inv"], (p.T * p.k,), torch.int32, "inv")
    _need(o["x_packed"], (rows, p.d), dt, "x_packed")
    ws = workspace if workspace is not None else alloc_workspace(p, MOE_CALL_DISPATCH_PADDED, dev)
    pc = p.c()
    _check(lib().moe_dispatch_padded(ctypes.byref(pc), int(capacity), _ptr(topk_idx), _ptr(x),
                                     _ptr(o["counts_all"]), _ptr(o["offsets"]), _ptr(o["perm"]),
                                     _ptr(o["inv"]), _ptr(o["x_packed"]), _ptr(ws),
                                     0 if ws is None else ws.numel(), _stream(stream)))
    return o


def expert_gemm_padded(p: Spec, capacity: int, x_packed, offsets, w1, w3, w2, workspace=None,
                       stream=None, out=None):
    torch = _torch()
    dt = _dt(p)
    rows = p.n_local * int(capacity)
    _need(x_packed, (rows, p.d), dt, "x_packed")
    _need(offsets, (p.n_local + 1,), torch.int32, "offsets")
    _need(w1, (p.n_local, p.d, p.f), dt, "w1")
    _need(w3, (p.n_local, p.d, p.f), dt, "w3")
    _need(w2, (p.n_local, p.f, p.d), dt, "w2")
    dev = x_packed.device
    if out is None:
        h = torch.ones((rows, p.f), dtype=dt, device=dev)
        yp = torch.ones((rows, p.d), dtype=dt, device=dev)
    else:
        h, yp = out
    ws = workspace if workspace is not None else alloc_workspace(p, MOE_CALL_EXPERT_GEMM_PADDED, dev)
    pc = p.c()
    _check(lib().moe_expert_gemm_padded(ctypes.byref(pc), int(capacity), _ptr(x_packed),
                                        _ptr(offsets), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(h),
                                        _ptr(yp), _ptr(ws), 0 if ws is None else ws.numel(),
                                        _stream(stream)))
    return h, yp


def gemm_signal_tiles(M: int, N: int) -> int:
    n = int(lib().moe_gemm_signal_tiles(int(M), int(N)))
    if n <= 0:
        raise MoeError(MOE_ERR_INVALID_ARG, lib().moe_last_error().decode())
    return n


def gemm_signal(A, B, flags, epoch: int, scope: int = MOE_SCOPE_AGENT, stream=None, out=None):
    """C = rnd(A B) (bf16 [M,K] x [K,N]); flags (int32 or uint32 device
    tensor of gemm_signal_tiles(M, N) entries) receive `epoch` per finished
    256 x 256 tile."""
    torch = _torch()
    M, K = A.shape
    N = B.shape[1]
    _need(A, (M, K), torch.bfloat16, "A")
    _need(B, (K, N), torch.bfloat16, "B")
    _need(flags, (gemm_signal_tiles(M, N),), flags.dtype, "flags")
    C = torch.empty((M, N), dtype=torch.bfloat16, device=A.device) if out is None else out
    _need(C, (M, N), torch.bfloat16, "C")
    _check(lib().moe_gemm_signal(M, N, K, _ptr(A), _ptr(B), _ptr(C), _ptr(flags), int(epoch),
                                 int(scope), _stream(stream)))
    return C


def tile_forward(C, dst, flags, epoch: int, spin_limit: int, timeouts, workgroups: int = 4,
                 scope: int = MOE_SCOPE_AGENT, stream=None):
    """Copies each 256 x 256 tile of C to dst once flags[tile] == epoch;
    adds 1 to timeouts[0] per tile whose flag did not arrive in spin_limit polls."""
    torch = _torch()
    M, N = C.shape
    _need(C, (M, N), torch.bfloat16, "C")
    _need(dst, (M, N), torch.bfloat16, "dst")
    _need(flags, (gemm_signal_tiles(M, N),), flags.dtype, "flags")
    _need(timeouts, (1,), timeouts.dtype, "timeouts")
    _check(lib().moe_tile_forward(M, N, _ptr(C), _ptr(dst), _ptr(flags), int(epoch),
                                  int(spin_limit), int(scope), _ptr(timeouts), int(workgroups),
                                  _stream(stream)))
    return dst


def layer_set_gemm_events(before: int, after: int) -> None:
    """The next layer() call on this thread records the two HIP events (raw
    hipEvent_t handles, timing enabled) on its launch stream around its expert
    GEMM."""
    _check(lib().moe_layer_set_gemm_events(ctypes.c_void_p(before or 0), ctypes.c_void_p(after or 0)))


def layer_ws_offset(p: Spec, what: int) -> int:
    """Byte offset of h (MOE_WS_H) or y_packed (MOE_WS_Y_PACKED) inside a
    moe_layer workspace of problem p."""
    pc = p.c()
    n = int(lib().moe_layer_ws_offset(ctypes.byref(pc), int(what)))
    if n == ctypes.c_size_t(-1).value:
        raise MoeError(MOE_ERR_INVALID_ARG, lib().moe_last_error().decode())
    return n


def layer(p: Spec, x, w_gate, bias, w1, w3, w2, routing: bool = False, want_logits: bool = False,
          overlap: bool = False, workspace=None, stream=None, stream2=None, out=None,
          fold_weight: bool = False):
    """The whole layer.  With ``routing`` also returns the routing/dispatch
    tensors; with ``overlap`` runs the two-stream dispatch overlap (needs
    ``stream2``, a torch.cuda.Stream, or creates none and runs one stream);
    with ``fold_weight`` the routing weights scale the expert output rows in
    the down projection and combine sums them unweighted."""
    torch = _torch()
    dt = _dt(p)
    _need(x, (p.T, p.d), dt, "x")
    _need(w_gate, (p.d, p.E), dt, "w_gate")
    if bias is not None:
        _need(bias, (p.E,), torch.float32, "bias")
    _need(w1, (p.n_local, p.d, p.f), dt, "w1")
    _need(w3, (p.n_local, p.d, p.f), dt, "w3")
    _need(w2, (p.n_local, p.f, p.d), dt, "w2")
    dev = x.device
    flags = (p.flags | (MOE_F_WRITE_LOGITS if want_logits else 0) | (MOE_F_OVERLAP if overlap else 0)
             | (MOE_F_FOLD_WEIGHT if fold_weight else 0))
    q = Spec(p.T, p.d, p.E, p.k, p.f, p.expert_lo, p.n_local, p.dtype, flags)
    y = torch.empty((p.T, p.d), dtype=dt, device=dev) if out is None else out
    r = None
    ro = None
    if routing or want_logits:
        r = {
            "topk_idx": torch.empty((p.T, p.k), dtype=torch.int32, device=dev),
            "topk_w": torch.empty((p.T, p.k), dtype=torch.float32, device=dev),
            "counts_all": torch.empty(p.E, dtype=torch.int32, device=dev),
            "offsets": torch.empty(p.n_local + 1, dtype=torch.int32, device=dev),
            "perm": torch.full((p.rows_max,), -7, dtype=torch.int32, device=dev),
            "inv": torch.empty(p.T * p.k, dtype=torch.int32, device=dev),
        }
        if want_logits:
            r["logits"] = torch.empty((p.T, p.E), dtype=torch.float32, device=dev)
        ro = RoutingOut(*[_ptr(r.get(n)) for n in
                          ("topk_idx", "topk_w", "logits", "counts_all", "offsets", "perm", "inv")])
    ws = workspace if workspace is not None else alloc_workspace(q, MOE_CALL_LAYER, dev)
    pc = q.c()
    s2 = _stream(stream2) if (overlap and stream2 is not None) else None
    _check(lib().moe_layer(ctypes.byref(pc), _ptr(x), _ptr(w_gate), _ptr(bias), _ptr(w1), _ptr(w3),
                           _ptr(w2), _ptr(y), ctypes.byref(ro) if ro is not None else None,
                           _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream), s2))
    return (y, r) if r is not None else y
