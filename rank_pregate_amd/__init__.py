"""rank_pregate_amd -- pre-gated multi-adapter low-rank projection on MI355X (gfx950).

Thin Python binding of librank_pregate.so (include/rank_pregate.h).  The
functions here only marshal torch tensors into pointers, sizes and the
current HIP stream; every step runs in the library's HIP kernels.  There is
no CPU fallback: if the library is not built, every call raises.

    pregate(x, Wg, k)                    -> topk_idx, topk_gate      (rp_pregate)
    segment(topk_idx, E)                 -> seg_offsets, pair_perm   (rp_segment)
    sgmm_fused(projs, x, E, r, ...)      -> list of y                (rp_sgmm_fused)

torch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
import weakref
from typing import List, Optional, Sequence, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librank_pregate.so")

RP_OK, RP_ERR_INVALID_ARG, RP_ERR_UNSUPPORTED, RP_ERR_WORKSPACE, RP_ERR_HIP, RP_ERR_DEVICE = range(6)
RP_F32, RP_BF16 = 0, 1
RP_MAX_K, RP_MAX_E, RP_MAX_PROJ = 8, 1024, 4

_STATUS_NAMES = {0: "RP_OK", 1: "RP_ERR_INVALID_ARG", 2: "RP_ERR_UNSUPPORTED", 3: "RP_ERR_WORKSPACE",
                 4: "RP_ERR_HIP", 5: "RP_ERR_DEVICE"}

EXPORTED = ("rp_pregate", "rp_segment", "rp_segment_workspace_size", "rp_sgmm_fused", "rp_sgmm_workspace_size",
            "rp_route_sgmm_fused", "rp_sgmm_step", "rp_sgmm_step_workspace_size", "rp_pack_w0", "rp_last_error", "rp_abi_version", "rp_util_stream_read", "rp_util_copy",
            "rp_workspace_status", "rp_sgmm_step_noalloc", "rp_adapter_apply", "rp_merge_adapters", "rp_rmsnorm",
            "rp_silu_mul")
RP_W0_ROWS, RP_W0_TILED = 0, 1
RP_ACT_NONE, RP_ACT_SILU_MUL = 0, 1


class RankPregateError(RuntimeError):
    def __init__(self, where: str, status: int, message: str):
        super().__init__(f"{where}: {_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class RpProj(ctypes.Structure):
    _fields_ = [("W0", ctypes.c_void_p), ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("d_out", ctypes.c_int64), ("ld_y", ctypes.c_int64), ("w0_layout", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("residual", ctypes.c_void_p)]


class RpGroup(ctypes.Structure):
    _fields_ = [("projs", ctypes.POINTER(RpProj)), ("n_proj", ctypes.c_int32), ("x_from_call", ctypes.c_int32),
                ("x", ctypes.c_void_p), ("d_in", ctypes.c_int64), ("ld_x", ctypes.c_int64), ("act", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m rank_pregate_amd.build` "
                           "(there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    L.rp_pregate.argtypes = [vp, i64, i64, i64, vp, i64, i32, ctypes.c_int, vp, vp, vp, vp]
    L.rp_segment.argtypes = [vp, i64, i32, i64, vp, vp, vp, sz, vp]
    L.rp_segment_workspace_size.argtypes = [i64, i32, i64]
    L.rp_segment_workspace_size.restype = sz
    L.rp_sgmm_fused.argtypes = [ctypes.POINTER(RpProj), i32, vp, i64, i64, i64, i64, i64, i32, vp, vp, vp, vp,
                                ctypes.c_int, vp, sz, vp]
    L.rp_route_sgmm_fused.argtypes = [ctypes.POINTER(RpProj), i32, vp, i64, i64, i64, vp, i64, i64, i32,
                                      ctypes.c_int, vp, vp, vp, vp, vp, sz, vp]
    L.rp_sgmm_step.argtypes = [ctypes.POINTER(RpGroup), i32, i64, i64, i64, i32, vp, vp, vp, vp, vp, ctypes.c_int, vp,
                               sz, vp]
    L.rp_sgmm_step_workspace_size.argtypes = [ctypes.POINTER(RpGroup), i32, i64, i64, i64, i32, ctypes.c_int]
    L.rp_sgmm_step_workspace_size.restype = sz
    L.rp_sgmm_workspace_size.argtypes = [i32, i64, i64, i64, i64, i64, i32, ctypes.c_int]
    L.rp_sgmm_workspace_size.restype = sz
    L.rp_last_error.argtypes = []
    L.rp_last_error.restype = ctypes.c_char_p
    L.rp_abi_version.argtypes = []
    L.rp_abi_version.restype = ctypes.c_int
    L.rp_pack_w0.argtypes = [vp, vp, i64, i64, ctypes.c_int, vp]
    L.rp_util_stream_read.argtypes = [vp, sz, vp, vp]
    L.rp_util_copy.argtypes = [vp, vp, sz, vp]
    L.rp_workspace_status.argtypes = [vp, sz, i32, ctypes.POINTER(i32), ctypes.POINTER(i32), vp]
    L.rp_adapter_apply.argtypes = [ctypes.POINTER(RpProj), i32, vp, i64, i64, i64, i64, i64, i32, i32, vp, vp, vp,
                                   ctypes.c_int, vp]
    L.rp_merge_adapters.argtypes = [vp, i32, i64, i64, vp, vp, i64, i64, vp, vp, i32, ctypes.c_float, ctypes.c_int,
                                    vp]
    L.rp_sgmm_step_noalloc.argtypes = [ctypes.POINTER(RpGroup), i32, i64, i64, i64, i32, vp, vp, vp, vp, vp,
                                       ctypes.c_int, vp]
    L.rp_rmsnorm.argtypes = [vp, i64, i64, i64, vp, ctypes.c_float, vp, i64, ctypes.c_int, vp]
    L.rp_silu_mul.argtypes = [vp, i64, vp, i64, i64, i64, vp, i64, ctypes.c_int, vp]
    for name in ("rp_pregate", "rp_segment", "rp_sgmm_fused", "rp_route_sgmm_fused", "rp_sgmm_step", "rp_pack_w0",
                 "rp_util_stream_read", "rp_util_copy", "rp_workspace_status", "rp_sgmm_step_noalloc",
                 "rp_adapter_apply", "rp_merge_adapters", "rp_rmsnorm", "rp_silu_mul"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def last_error() -> str:
    return lib().rp_last_error().decode()


def abi_version() -> int:
    return lib().rp_abi_version()


def _check(status: int, where: str) -> None:
    if status != RP_OK:
        raise RankPregateError(where, status, last_error())


# ----------------------------------------------------------------------------- torch marshalling

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return RP_BF16
    if t.dtype == torch.float32:
        return RP_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream, device) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _rows(t, name: str) -> int:
    """Leading dimension of a row-major 2-D view (unit stride along columns)."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a 2-D row-major tensor with unit column stride")
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def pregate(x, Wg, k: int, topk_idx=None, topk_gate=None, logits=None, stream=None):
    """rp_pregate on torch tensors: x [T, d_in], Wg [d_in, E] (dense), same dtype, on one GPU.

    Returns (topk_idx int32 [T, k], topk_gate float32 [T, k]); `logits`
    (float32 [T, E]) is filled when given.
    """
    torch = _torch()
    T, d_in = x.shape
    E = Wg.shape[1]
    if Wg.dtype != x.dtype or not Wg.is_contiguous() or Wg.shape[0] != d_in:
        raise ValueError("Wg must be a dense [d_in, E] tensor of x's dtype")
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    if topk_gate is None:
        topk_gate = torch.empty((T, k), dtype=torch.float32, device=x.device)
    st = lib().rp_pregate(_ptr(x), T, d_in, _rows(x, "x"), _ptr(Wg), E, k, _dtype_code(x), _ptr(topk_idx),
                          _ptr(topk_gate), _ptr(logits), _stream(stream, x.device))
    _check(st, "rp_pregate")
    return topk_idx, topk_gate


def segment_workspace_size(T: int, k: int, E: int) -> int:
    return lib().rp_segment_workspace_size(T, k, E)


def segment(topk_idx, E: int, seg_offsets=None, pair_perm=None, ws=None, stream=None):
    """rp_segment on torch tensors.  Returns (seg_offsets int32 [E+1], pair_perm int32 [T*k])."""
    torch = _torch()
    T, k = topk_idx.shape
    dev = topk_idx.device
    if seg_offsets is None:
        seg_offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    if pair_perm is None:
        pair_perm = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    nbytes = segment_workspace_size(T, k, E)
    if ws is None:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    st = lib().rp_segment(_ptr(topk_idx), T, k, E, _ptr(seg_offsets), _ptr(pair_perm), _ptr(ws), ws.numel(),
                          _stream(stream, dev))
    _check(st, "rp_segment")
    return seg_offsets, pair_perm


def sgmm_workspace_size(n_proj: int, T: int, d_in: int, sum_d_out: int, E: int, r: int, k: int,
                        dtype_code: int) -> int:
    return lib().rp_sgmm_workspace_size(n_proj, T, d_in, sum_d_out, E, r, k, dtype_code)


_tracked = weakref.WeakValueDictionary()


def track_workspace(ws):
    """Remember an SGMM workspace tensor (weakly) so check_workspaces() can read its status words."""
    _tracked[id(ws)] = ws
    return ws


class Workspace:
    """Zero-initialised device buffers reused across calls, one per (device, stream).

    The library keeps a buffer's control region consistent between calls, so a
    buffer only has to be zeroed when it is (re)allocated.  Calls on different
    streams get different buffers (calls that may overlap in time must not
    share one).  A new buffer is zero-filled on the current torch stream, which
    is then waited for, so the fill is complete before the call's stream uses
    it; pass an explicit workspace when recording a graph.
    """

    def __init__(self):
        self._buf = {}

    def get(self, nbytes: int, device, stream: int = 0):
        torch = _torch()
        key = (str(device), int(stream))
        b = self._buf.get(key)
        if b is None or b.numel() < nbytes:
            b = torch.zeros(max(nbytes, 1 << 16), dtype=torch.uint8, device=device)
            torch.cuda.current_stream(device).synchronize()
            self._buf[key] = track_workspace(b)
        return b


_default_ws = Workspace()


def workspace_status(ws, clear: bool = False, stream=None) -> Tuple[int, int]:
    """rp_workspace_status: (wait_overflow, bad_indices) of an SGMM workspace tensor.

    Waits for `stream` (default: the current one).  Raises RankPregateError
    (RP_ERR_DEVICE) when either word is nonzero."""
    wo, bad = ctypes.c_int32(0), ctypes.c_int32(0)
    st = lib().rp_workspace_status(_ptr(ws), ws.numel() * ws.element_size(), int(clear), ctypes.byref(wo),
                                   ctypes.byref(bad), _stream(stream, ws.device))
    _check(st, "rp_workspace_status")
    return wo.value, bad.value


def check_workspaces(clear: bool = True) -> int:
    """workspace_status on every tracked workspace still alive; returns how many were checked."""
    n = 0
    for ws in list(_tracked.values()):
        workspace_status(ws, clear=clear)
        n += 1
    return n


def _proj_array(projs: Sequence[Tuple], x):
    torch = _torch()
    T = x.shape[0]
    arr = (RpProj * len(projs))()
    ys = []
    sum_d_out = 0
    for i, pr in enumerate(projs):
        W0, A, B = pr[0], pr[1], pr[2]
        y = pr[3] if len(pr) > 3 else None
        res = pr[4] if len(pr) > 4 else None
        tiled = W0.dim() == 4
        d_out = W0.shape[0] * 16 if tiled else W0.shape[0]
        for name, t in (("W0", W0), ("A", A), ("B", B)):
            if t is not None and (t.dtype != x.dtype or not t.is_contiguous()):
                raise ValueError(f"projection {i}: {name} must be dense with x's dtype")
        if y is None:
            y = torch.empty((T, d_out), dtype=x.dtype, device=x.device)
        ys.append(y)
        if res is not None and (res.dtype != x.dtype or tuple(res.shape) != tuple(y.shape)
                                or _rows(res, "residual") != _rows(y, "y")):
            raise ValueError(f"projection {i}: residual must have y's dtype, shape and row stride")
        arr[i] = RpProj(_ptr(W0), _ptr(A), _ptr(B), _ptr(y), d_out, _rows(y, "y"),
                        RP_W0_TILED if tiled else RP_W0_ROWS, 0, _ptr(res))
        sum_d_out += d_out
    return arr, ys, sum_d_out


def route_sgmm_fused(projs: Sequence[Tuple], x, Wg, E: int, r: int, k: int, topk_idx=None, topk_gate=None,
                     seg_offsets=None, pair_perm=None, ws=None, stream=None):
    """rp_route_sgmm_fused on torch tensors: router, segmentation and the projections of `projs` on x.

    Returns (ys, topk_idx, topk_gate, seg_offsets, pair_perm); routing outputs that are None are allocated.
    """
    torch = _torch()
    T, d_in = x.shape
    dt = _dtype_code(x)
    if Wg.dtype != x.dtype or not Wg.is_contiguous() or tuple(Wg.shape) != (d_in, E):
        raise ValueError("Wg must be a dense [d_in, E] tensor with x's dtype")
    dev = x.device
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_gate is None:
        topk_gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    if seg_offsets is None:
        seg_offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    if pair_perm is None:
        pair_perm = torch.empty(max(1, T * k), dtype=torch.int32, device=dev)
    arr, ys, sum_d_out = _proj_array(projs, x)
    sh = _stream(stream, dev)
    if ws is None:
        ws = _default_ws.get(sgmm_workspace_size(len(projs), T, d_in, sum_d_out, E, r, k, dt), dev, sh)
    st = lib().rp_route_sgmm_fused(arr, len(projs), _ptr(x), T, d_in, _rows(x, "x"), _ptr(Wg), E, r, k, dt,
                                   _ptr(topk_idx), _ptr(topk_gate), _ptr(seg_offsets), _ptr(pair_perm), _ptr(ws),
                                   ws.numel(), sh)
    _check(st, "rp_route_sgmm_fused")
    return ys, topk_idx, topk_gate, seg_offsets, pair_perm


def sgmm_fused(projs: Sequence[Tuple], x, E: int, r: int, k: int, topk_idx=None, topk_gate=None, seg_offsets=None,
               pair_perm=None, ws=None, stream=None) -> List:
    """rp_sgmm_fused on torch tensors.

    projs: up to four tuples (W0, A [E, r, d_in], B [E, d_out, r], y [T, d_out] or None); W0 is either
    a dense [d_out, d_in] tensor or the 4-D tensor pack_w0 returns (tiled order).  Outputs that are
    None are allocated.  Returns the list of y tensors.
    """
    T, d_in = x.shape
    dt = _dtype_code(x)
    arr, ys, sum_d_out = _proj_array(projs, x)
    sh = _stream(stream, x.device)
    if ws is None:
        ws = _default_ws.get(sgmm_workspace_size(len(projs), T, d_in, sum_d_out, E, r, k, dt), x.device, sh)
    st = lib().rp_sgmm_fused(arr, len(projs), _ptr(x), T, d_in, _rows(x, "x"), E, r, k, _ptr(topk_idx),
                             _ptr(topk_gate), _ptr(seg_offsets), _ptr(pair_perm), dt, _ptr(ws), ws.numel(), sh)
    _check(st, "rp_sgmm_fused")
    return ys


def adapter_apply(projs: Sequence[Tuple], x, E: int, r: int, k: int, adapter: int, topk_gate, seg_offsets,
                  pair_perm, stream=None) -> None:
    """rp_adapter_apply on torch tensors: adds adapter `adapter`'s gated delta into each projection's y
    (projs as for sgmm_fused, with y given and already holding the base projection)."""
    T, d_in = x.shape
    if any(len(pr) < 4 or pr[3] is None for pr in projs):
        raise ValueError("adapter_apply updates y in place: every projection needs its y")
    arr, _, _ = _proj_array(projs, x)
    st = lib().rp_adapter_apply(arr, len(projs), _ptr(x), T, d_in, _rows(x, "x"), E, r, k, adapter,
                                _ptr(topk_gate), _ptr(seg_offsets), _ptr(pair_perm), _dtype_code(x),
                                _stream(stream, x.device))
    _check(st, "rp_adapter_apply")


def merge_adapters(W0, A, B, sel, weights, sign: float = 1.0, stream=None) -> None:
    """rp_merge_adapters: W0 += sign * sum_j weights[j] B[sel[j]] A[sel[j]] in place.

    W0: dense [d_out, d_in] or the 4-D tiled tensor pack_w0 returns; A [E, r, d_in]; B [E, d_out, r];
    sel int32 and weights float32 device tensors of n_sel entries."""
    tiled = W0.dim() == 4
    d_out = W0.shape[0] * 16 if tiled else W0.shape[0]
    E, r, d_in = A.shape
    if sel.dtype != _torch().int32 or weights.dtype != _torch().float32 or sel.numel() != weights.numel():
        raise ValueError("sel must be int32 and weights float32, with as many entries")
    st = lib().rp_merge_adapters(_ptr(W0), RP_W0_TILED if tiled else RP_W0_ROWS, d_out, d_in, _ptr(A), _ptr(B), E, r,
                                 _ptr(sel), _ptr(weights), sel.numel(), float(sign), _dtype_code(W0),
                                 _stream(stream, W0.device))
    _check(st, "rp_merge_adapters")


def _step_args(groups, E, k, Wg, topk_idx, topk_gate, seg_offsets, pair_perm):
    """Marshal sgmm_step's arguments: (group array, arrays to keep alive, ys, routing tensors, T, dt, dev)."""
    torch = _torch()
    x0 = groups[0][1]
    T = x0.shape[0]
    dt = _dtype_code(x0)
    dev = x0.device
    if Wg is not None:
        if Wg.dtype != x0.dtype or not Wg.is_contiguous() or tuple(Wg.shape) != (x0.shape[1], E):
            raise ValueError("Wg must be a dense [d_in, E] tensor with x's dtype")
        if topk_idx is None:
            topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        if topk_gate is None:
            topk_gate = torch.empty((T, k), dtype=torch.float32, device=dev)
        if seg_offsets is None:
            seg_offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        if pair_perm is None:
            pair_perm = torch.empty(max(1, T * k), dtype=torch.int32, device=dev)
    garr = (RpGroup * len(groups))()
    keep, ys = [], []
    for i, g in enumerate(groups):
        projs, x = g[0], g[1]
        from_call = int(g[2]) if len(g) > 2 else 0
        act = int(g[3]) if len(g) > 3 else RP_ACT_NONE
        if x.shape[0] != T or x.dtype != x0.dtype:
            raise ValueError(f"group {i}: x must have T rows and the first group's dtype")
        arr, gys, _ = _proj_array(projs, x)
        keep.append(arr)
        ys.append(gys)
        garr[i] = RpGroup(ctypes.cast(arr, ctypes.POINTER(RpProj)), len(projs), from_call, _ptr(x), x.shape[1],
                          _rows(x, "x"), act, 0)
    return garr, keep, ys, (topk_idx, topk_gate, seg_offsets, pair_perm), T, dt, dev


def sgmm_step(groups: Sequence[Tuple], E: int, r: int, k: int, Wg=None, topk_idx=None, topk_gate=None,
              seg_offsets=None, pair_perm=None, ws=None, stream=None):
    """rp_sgmm_step on torch tensors.

    groups: sequence of (projs, x), (projs, x, x_from_call) or (projs, x, x_from_call, act); projs as for
    sgmm_fused, each (W0, A, B[, y[, residual]]); act RP_ACT_SILU_MUL writes silu(y0) * y1 over y0.  With Wg the routing
    is computed from the first group's x into the four routing tensors (allocated when None); without it
    they are inputs.  Returns (list of y lists per group, topk_idx, topk_gate, seg_offsets, pair_perm).
    """
    garr, keep, ys, (topk_idx, topk_gate, seg_offsets, pair_perm), T, dt, dev = _step_args(
        groups, E, k, Wg, topk_idx, topk_gate, seg_offsets, pair_perm)
    sh = _stream(stream, dev)
    if ws is None:
        ws = _default_ws.get(lib().rp_sgmm_step_workspace_size(garr, len(groups), T, E, r, k, dt), dev, sh)
    st = lib().rp_sgmm_step(garr, len(groups), T, E, r, k, _ptr(Wg), _ptr(topk_idx), _ptr(topk_gate),
                            _ptr(seg_offsets), _ptr(pair_perm), dt, _ptr(ws), ws.numel(), sh)
    _check(st, "rp_sgmm_step")
    return ys, topk_idx, topk_gate, seg_offsets, pair_perm


def sgmm_step_noalloc(groups: Sequence[Tuple], E: int, r: int, k: int, Wg=None, topk_idx=None, topk_gate=None,
                      seg_offsets=None, pair_perm=None, stream=None):
    """rp_sgmm_step_noalloc on torch tensors: sgmm_step without a workspace argument (the library's
    static one serves).  Outputs and routing tensors that are None are allocated here by torch; pass
    them all to keep the call free of allocation."""
    garr, keep, ys, (topk_idx, topk_gate, seg_offsets, pair_perm), T, dt, dev = _step_args(
        groups, E, k, Wg, topk_idx, topk_gate, seg_offsets, pair_perm)
    st = lib().rp_sgmm_step_noalloc(garr, len(groups), T, E, r, k, _ptr(Wg), _ptr(topk_idx), _ptr(topk_gate),
                                    _ptr(seg_offsets), _ptr(pair_perm), dt, _stream(stream, dev))
    _check(st, "rp_sgmm_step_noalloc")
    return ys, topk_idx, topk_gate, seg_offsets, pair_perm


def step_workspace_size(groups: Sequence[Tuple], E: int, r: int, k: int) -> int:
    """rp_sgmm_step_workspace_size for groups given as sgmm_step takes them."""
    x0 = groups[0][1]
    garr = (RpGroup * len(groups))()
    keep = []
    for i, g in enumerate(groups):
        arr, _, _ = _proj_array(g[0], g[1])
        keep.append(arr)
        garr[i] = RpGroup(ctypes.cast(arr, ctypes.POINTER(RpProj)), len(g[0]), int(g[2]) if len(g) > 2 else 0,
                          _ptr(g[1]), g[1].shape[1], _rows(g[1], "x"), int(g[3]) if len(g) > 3 else RP_ACT_NONE, 0)
    return lib().rp_sgmm_step_workspace_size(garr, len(groups), x0.shape[0], E, r, k, _dtype_code(x0))


def rmsnorm(x, gamma, eps: float = 1e-5, out=None, stream=None):
    """rp_rmsnorm: out[t] = round(x[t] * gamma / sqrt(mean(x[t]^2) + eps)); out may be x."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(x)
    if gamma.dtype != x.dtype or not gamma.is_contiguous() or gamma.numel() != x.shape[1]:
        raise ValueError("gamma must be a dense [d] tensor with x's dtype")
    st = lib().rp_rmsnorm(_ptr(x), x.shape[0], x.shape[1], _rows(x, "x"), _ptr(gamma), float(eps), _ptr(out),
                          _rows(out, "out"), _dtype_code(x), _stream(stream, x.device))
    _check(st, "rp_rmsnorm")
    return out


def silu_mul(g, u, out=None, stream=None):
    """rp_silu_mul: out = round(silu(g) * u) elementwise in fp32; out may be g or u."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(g)
    if u.shape != g.shape or u.dtype != g.dtype:
        raise ValueError("g and u must have one shape and dtype")
    st = lib().rp_silu_mul(_ptr(g), _rows(g, "g"), _ptr(u), _rows(u, "u"), g.shape[0], g.shape[1], _ptr(out),
                           _rows(out, "out"), _dtype_code(g), _stream(stream, g.device))
    _check(st, "rp_silu_mul")
    return out


def pack_w0(W0, out=None, stream=None):
    """rp_pack_w0: repack a dense bf16 W0 [d_out, d_in] into the tiled order.

    Returns a [d_out/16, d_in/32, 64, 8] tensor (the shape marks the layout for sgmm_fused).
    """
    torch = _torch()
    d_out, d_in = W0.shape
    if out is None:
        out = torch.empty((d_out // 16, d_in // 32, 64, 8), dtype=W0.dtype, device=W0.device)
    st = lib().rp_pack_w0(_ptr(W0), _ptr(out), d_out, d_in, _dtype_code(W0), _stream(stream, W0.device))
    _check(st, "rp_pack_w0")
    return out


def stream_read(src, sink, stream=None) -> None:
    """rp_util_stream_read over the bytes of tensor `src`; `sink` is a float32 tensor of >= 1024 elements."""
    st = lib().rp_util_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                   _stream(stream, src.device))
    _check(st, "rp_util_stream_read")


def copy(dst, src, stream=None) -> None:
    st = lib().rp_util_copy(_ptr(dst), _ptr(src), src.numel() * src.element_size(), _stream(stream, src.device))
    _check(st, "rp_util_copy")


# the C names, for callers that mirror the header
rp_pregate, rp_segment, rp_sgmm_fused, rp_route_sgmm_fused = pregate, segment, sgmm_fused, route_sgmm_fused
rp_sgmm_step = sgmm_step
rp_workspace_status = workspace_status
rp_sgmm_step_noalloc = sgmm_step_noalloc
rp_adapter_apply = adapter_apply
rp_merge_adapters = merge_adapters
