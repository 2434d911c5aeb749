"""ctypes binding for libce_mi355x.so (include/ce_mi355x.h).

Argument marshalling only: it reads device pointers, shapes and strides from torch
tensors, allocates output tensors with torch, passes the current HIP stream, and
raises CEError on a negative status.  Every step of the computation runs in the
library's HIP kernels; there is no fallback of any kind, and a missing library is
an error.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libce_mi355x.so")

CE_F32, CE_F16, CE_BF16 = 0, 1, 2
DTYPE_CODE = {torch.float32: CE_F32, torch.float16: CE_F16, torch.bfloat16: CE_BF16}

STATUS = {
    0: "CE_OK", -1: "CE_ERR_NULL", -2: "CE_ERR_SHAPE", -3: "CE_ERR_DTYPE", -4: "CE_ERR_LAYOUT",
    -5: "CE_ERR_WORKSPACE", -6: "CE_ERR_LAUNCH", -7: "CE_ERR_ALIAS", -8: "CE_ERR_DEVICE", -9: "CE_ERR_OPTION",
}

CE_REDUCE = {"none": 0, "sum": 1, "mean": 2}
CE_NO_IGNORE = -(2 ** 31)

# every symbol include/ce_mi355x.h declares
EXPORTS = ("ce_forward", "ce_vjp", "ce_forward_vjp", "lce_workspace_size",
           "lce_forward", "lce_backward_workspace_size", "lce_backward_workspace_size_one_pass", "lce_backward",
           "kl_forward",
           "kl_vjp", "js_forward", "js_vjp",
           "ce_reduce_workspace_size", "ce_forward_ex", "ce_forward_ex_noalloc", "ce_vjp_ex", "ce_forward_probs",
           "ce_vjp_probs", "ce_status_string")
# the forced row-to-lane variants include/ce_mi355x_testing.h declares (tests and tuning)
TESTING_EXPORTS = ("ce_forward_lanes", "ce_vjp_lanes", "ce_forward_vjp_lanes", "kl_forward_lanes", "kl_vjp_lanes",
                   "js_forward_lanes", "js_vjp_lanes")


class CELayout(ctypes.Structure):
    _fields_ = [("rows_per_batch", ctypes.c_int64), ("row_stride", ctypes.c_int64),
                ("batch_stride", ctypes.c_int64)]


class CEOptions(ctypes.Structure):
    _fields_ = [("label_smoothing", ctypes.c_float), ("ignore_index", ctypes.c_int32), ("reduction", ctypes.c_int32)]


def options(label_smoothing: float = 0.0, ignore_index=None, reduction: str = "none") -> CEOptions:
    return CEOptions(float(label_smoothing), CE_NO_IGNORE if ignore_index is None else int(ignore_index),
                     CE_REDUCE[reduction] if isinstance(reduction, str) else int(reduction))


class CEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


_lib = None

_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.ce_forward.argtypes = [_vp, CELayout, ctypes.c_int, _vp, _i64, _i64, _vp, _vp, _vp]
        L.ce_forward_lanes.argtypes = [_vp, CELayout, ctypes.c_int, _vp, _i64, _i64, _vp, _vp, _i32, _vp]
        L.ce_vjp.argtypes = [_vp, CELayout, ctypes.c_int, _vp, _vp, _vp, _i64, _i64, _vp, CELayout, _vp]
        L.ce_vjp_lanes.argtypes = [_vp, CELayout, ctypes.c_int, _vp, _vp, _vp, _i64, _i64, _vp, CELayout,
                                   _i32, _vp]
        L.ce_forward_vjp.argtypes = [_vp, CELayout, ctypes.c_int, _vp, _vp, _i64, _i64, _vp, _vp, _vp, CELayout,
                                     _vp]
        L.ce_forward_vjp_lanes.argtypes = [_vp, CELayout, ctypes.c_int, _vp, _vp, _i64, _i64, _vp, _vp, _vp,
                                           CELayout, _i32, _vp]
        L.lce_workspace_size.argtypes = [_i64, _i64, _i64]
        L.lce_workspace_size.restype = _sz
        L.lce_forward.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _sz, _vp]
        L.lce_backward_workspace_size.argtypes = [_i64, _i64, _i64]
        L.lce_backward_workspace_size.restype = _sz
        L.lce_backward_workspace_size_one_pass.argtypes = [_i64, _i64, _i64]
        L.lce_backward_workspace_size_one_pass.restype = _sz
        L.lce_backward.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _sz, _vp]
        L.kl_forward.argtypes = [_vp, CELayout, _vp, CELayout, ctypes.c_int, _i64, _i64, _vp, _vp, _vp, _vp]
        L.kl_forward_lanes.argtypes = [_vp, CELayout, _vp, CELayout, ctypes.c_int, _i64, _i64, _vp, _vp, _vp,
                                       _i32, _vp]
        L.kl_vjp.argtypes = [_vp, CELayout, _vp, CELayout, ctypes.c_int, _vp, _vp, _vp, _i64, _i64, _vp,
                             CELayout, _vp]
        L.kl_vjp_lanes.argtypes = [_vp, CELayout, _vp, CELayout, ctypes.c_int, _vp, _vp, _vp, _i64, _i64, _vp,
                                   CELayout, _i32, _vp]
        L.js_forward.argtypes = [_vp, CELayout, _vp, CELayout, ctypes.c_int, _i64, _i64, _vp, _vp, _vp, _vp, _vp]
        L.js_forward_lanes.argtypes = [_vp, CELayout, _vp, CELayout, ctypes.c_int, _i64, _i64, _vp, _vp, _vp, _vp,
                                       _i32, _vp]
        L.js_vjp.argtypes = [_vp, CELayout, _vp, CELayout, ctypes.c_int, _vp, _vp, _vp, _vp, _i64, _i64, _vp,
                             CELayout, _vp]
        L.js_vjp_lanes.argtypes = [_vp, CELayout, _vp, CELayout, ctypes.c_int, _vp, _vp, _vp, _vp, _i64, _i64, _vp,
                                   CELayout, _i32, _vp]
        L.ce_reduce_workspace_size.argtypes = []
        L.ce_reduce_workspace_size.restype = _sz
        L.ce_forward_ex.argtypes = [_vp, CELayout, ctypes.c_int, _vp, _i64, _i64, CEOptions, _vp, _vp, _vp, _vp, _vp,
                                    _sz, _vp]
        L.ce_forward_ex_noalloc.argtypes = [_vp, CELayout, ctypes.c_int, _vp, _i64, _i64, CEOptions, _vp, _vp,
                                            _vp, _vp, _vp]
        L.ce_vjp_ex.argtypes = [_vp, CELayout, ctypes.c_int, _vp, _vp, _vp, _i64, _i64, CEOptions, _vp, _vp, CELayout,
                                _vp]
        L.ce_forward_probs.argtypes = [_vp, CELayout, ctypes.c_int, _vp, CELayout, _i64, _i64, CEOptions, _vp, _vp,
                                       _vp, _vp, _vp, _vp, _sz, _vp]
        L.ce_vjp_probs.argtypes = [_vp, CELayout, ctypes.c_int, _vp, CELayout, _vp, _vp, _vp, _i64, _i64, CEOptions,
                                   _vp, _vp, CELayout, _vp]
        L.ce_status_string.argtypes = [ctypes.c_int]
        L.ce_status_string.restype = ctypes.c_char_p
        for name in ("ce_forward", "ce_forward_lanes", "ce_vjp", "ce_vjp_lanes", "ce_forward_vjp",
                     "ce_forward_vjp_lanes", "lce_forward", "lce_backward",
                     "kl_forward", "kl_forward_lanes", "kl_vjp", "kl_vjp_lanes", "js_forward", "js_forward_lanes",
                     "js_vjp", "js_vjp_lanes", "ce_forward_ex", "ce_forward_ex_noalloc", "ce_vjp_ex",
                     "ce_forward_probs", "ce_vjp_probs"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().ce_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise CEError(status, where)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def rows_layout(t: torch.Tensor) -> tuple[CELayout, int, int]:
    """(layout, n_rows, V) of a [rows, V] or [B, L, V] view with unit column stride."""
    if t.dim() == 2:
        R, V = t.shape
        rs = t.stride(0)
        return CELayout(max(R, 1), rs, rs * max(R, 1)), R, V
    if t.dim() == 3:
        B, L, V = t.shape
        return CELayout(max(L, 1), t.stride(1), t.stride(0)), B * L, V
    raise ValueError("logits must be [rows, V] or [B, L, V]")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, dtype, n, name):
    if t.dtype != dtype or not t.is_contiguous() or t.numel() != n:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of {n} elements")


def ce_forward(logits: torch.Tensor, targets: torch.Tensor, loss=None, lse=None, lanes_per_row: int = 0):
    """Per-row (loss [n], lse [n, 2]) of a [rows, V] or [B, L, V] logits view."""
    if logits.stride(-1) != 1 and logits.shape[-1] > 1:
        raise ValueError("logits need unit column stride")
    lay, n, V = rows_layout(logits)
    _need(targets, torch.int32, n, "targets")
    if loss is None:
        loss = torch.empty(n, dtype=torch.float32, device=logits.device)
    if lse is None:
        lse = torch.empty(n, 2, dtype=torch.float32, device=logits.device)
    _need(loss, torch.float32, n, "loss")
    _need(lse, torch.float32, 2 * n, "lse")
    args = (_ptr(logits), lay, DTYPE_CODE[logits.dtype], _ptr(targets), n, V, _ptr(loss), _ptr(lse))
    if lanes_per_row == 0:
        st = lib().ce_forward(*args, _stream(logits))
    else:
        st = lib().ce_forward_lanes(*args, int(lanes_per_row), _stream(logits))
    _check(st, "ce_forward")
    return loss, lse


def ce_vjp(logits: torch.Tensor, targets: torch.Tensor, lse: torch.Tensor, g: torch.Tensor, dlogits=None,
           lanes_per_row: int = 0):
    """dlogits = g * (softmax(logits) - onehot(targets)) from the saved lse; same shape as logits."""
    if logits.stride(-1) != 1 and logits.shape[-1] > 1:
        raise ValueError("logits need unit column stride")
    lay, n, V = rows_layout(logits)
    _need(targets, torch.int32, n, "targets")
    _need(lse, torch.float32, 2 * n, "lse")
    _need(g, torch.float32, n, "g")
    if dlogits is None:
        dlogits = torch.empty(logits.shape, dtype=logits.dtype, device=logits.device)
    if dlogits.dtype != logits.dtype or dlogits.shape != logits.shape:
        raise ValueError("dlogits must match logits in dtype and shape")
    if dlogits.stride(-1) != 1 and V > 1:
        raise ValueError("dlogits need unit column stride")
    olay, _, _ = rows_layout(dlogits)
    args = (_ptr(logits), lay, DTYPE_CODE[logits.dtype], _ptr(targets), _ptr(lse), _ptr(g), n, V, _ptr(dlogits),
            olay)
    if lanes_per_row == 0:
        st = lib().ce_vjp(*args, _stream(logits))
    else:
        st = lib().ce_vjp_lanes(*args, int(lanes_per_row), _stream(logits))
    _check(st, "ce_vjp")
    return dlogits


def ce_forward_vjp(logits: torch.Tensor, targets: torch.Tensor, g: torch.Tensor, loss=None, lse=None, dlogits=None,
                   lanes_per_row: int = 0):
    """(loss [n], lse [n, 2], dlogits) of ce_forward then ce_vjp with g, in one kernel."""
    if logits.stride(-1) != 1 and logits.shape[-1] > 1:
        raise ValueError("logits need unit column stride")
    lay, n, V = rows_layout(logits)
    _need(targets, torch.int32, n, "targets")
    _need(g, torch.float32, n, "g")
    if loss is None:
        loss = torch.empty(n, dtype=torch.float32, device=logits.device)
    if lse is None:
        lse = torch.empty(n, 2, dtype=torch.float32, device=logits.device)
    _need(loss, torch.float32, n, "loss")
    _need(lse, torch.float32, 2 * n, "lse")
    if dlogits is None:
        dlogits = torch.empty(logits.shape, dtype=logits.dtype, device=logits.device)
    if dlogits.dtype != logits.dtype or dlogits.shape != logits.shape:
        raise ValueError("dlogits must match logits in dtype and shape")
    if dlogits.stride(-1) != 1 and V > 1:
        raise ValueError("dlogits need unit column stride")
    olay, _, _ = rows_layout(dlogits)
    args = (_ptr(logits), lay, DTYPE_CODE[logits.dtype], _ptr(targets), _ptr(g), n, V, _ptr(loss), _ptr(lse),
            _ptr(dlogits), olay)
    if lanes_per_row == 0:
        st = lib().ce_forward_vjp(*args, _stream(logits))
    else:
        st = lib().ce_forward_vjp_lanes(*args, int(lanes_per_row), _stream(logits))
    _check(st, "ce_forward_vjp")
    return loss, lse, dlogits


def js_forward(q: torch.Tensor, p: torch.Tensor, js=None, lse_q=None, lse_p=None, hq=None, lanes_per_row: int = 0):
    """Per-row (js [n], lse_q [n, 2], lse_p [n, 2], hq [n]) of the student q and teacher p."""
    if q.dtype != p.dtype or q.shape != p.shape:
        raise ValueError("q and p must have the same dtype and shape")
    ql, n, V = _view(q, "q")
    pl, _, _ = _view(p, "p")
    dev = q.device
    js = torch.empty(n, dtype=torch.float32, device=dev) if js is None else js
    lse_q = torch.empty(n, 2, dtype=torch.float32, device=dev) if lse_q is None else lse_q
    lse_p = torch.empty(n, 2, dtype=torch.float32, device=dev) if lse_p is None else lse_p
    hq = torch.empty(n, dtype=torch.float32, device=dev) if hq is None else hq
    _need(js, torch.float32, n, "js")
    _need(lse_q, torch.float32, 2 * n, "lse_q")
    _need(lse_p, torch.float32, 2 * n, "lse_p")
    _need(hq, torch.float32, n, "hq")
    args = (_ptr(q), ql, _ptr(p), pl, DTYPE_CODE[q.dtype], n, V, _ptr(js), _ptr(lse_q), _ptr(lse_p), _ptr(hq))
    if lanes_per_row == 0:
        st = lib().js_forward(*args, _stream(q))
    else:
        st = lib().js_forward_lanes(*args, int(lanes_per_row), _stream(q))
    _check(st, "js_forward")
    return js, lse_q, lse_p, hq


def js_vjp(q: torch.Tensor, p: torch.Tensor, lse_q: torch.Tensor, lse_p: torch.Tensor, hq: torch.Tensor,
           g: torch.Tensor, dq=None, lanes_per_row: int = 0):
    """dq = g * Q * (h - H) from js_forward's outputs; same shape and dtype as q."""
    if q.dtype != p.dtype or q.shape != p.shape:
        raise ValueError("q and p must have the same dtype and shape")
    ql, n, V = _view(q, "q")
    pl, _, _ = _view(p, "p")
    _need(lse_q, torch.float32, 2 * n, "lse_q")
    _need(lse_p, torch.float32, 2 * n, "lse_p")
    _need(hq, torch.float32, n, "hq")
    _need(g, torch.float32, n, "g")
    if dq is None:
        dq = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if dq.dtype != q.dtype or dq.shape != q.shape:
        raise ValueError("dq must match q in dtype and shape")
    dl, _, _ = _view(dq, "dq")
    args = (_ptr(q), ql, _ptr(p), pl, DTYPE_CODE[q.dtype], _ptr(lse_q), _ptr(lse_p), _ptr(hq), _ptr(g), n, V,
            _ptr(dq), dl)
    if lanes_per_row == 0:
        st = lib().js_vjp(*args, _stream(q))
    else:
        st = lib().js_vjp_lanes(*args, int(lanes_per_row), _stream(q))
    _check(st, "js_vjp")
    return dq


def ce_reduce_workspace_size() -> int:
    return int(lib().ce_reduce_workspace_size())


def _rows_view(t: torch.Tensor, name: str):
    if t.stride(-1) != 1 and t.shape[-1] > 1:
        raise ValueError(f"{name} needs unit column stride")
    return rows_layout(t)


def _reduce_outputs(dev, reduction, total, count, workspace):
    if reduction == "none":
        return total, count, workspace
    if total is None:
        total = torch.empty(1, dtype=torch.float32, device=dev)
    if count is None:
        count = torch.empty(1, dtype=torch.int64, device=dev)
    if workspace is None:
        workspace = torch.empty(ce_reduce_workspace_size(), dtype=torch.uint8, device=dev)
    _need(total, torch.float32, 1, "total")
    _need(count, torch.int64, 1, "count")
    return total, count, workspace


def _upstream(g, n, reduction):
    _need(g, torch.float32, n if reduction == "none" else 1, "g")


def ce_forward_ex(logits: torch.Tensor, targets: torch.Tensor, label_smoothing: float = 0.0, ignore_index=None,
                  reduction: str = "none", loss=None, lse=None, total=None, count=None, workspace=None):
    """(loss [n], lse [n, 2], total [1] or None, count [1] or None) with the cross-entropy options."""
    lay, n, V = _rows_view(logits, "logits")
    _need(targets, torch.int32, n, "targets")
    dev = logits.device
    loss = torch.empty(n, dtype=torch.float32, device=dev) if loss is None else loss
    lse = torch.empty(n, 2, dtype=torch.float32, device=dev) if lse is None else lse
    _need(loss, torch.float32, n, "loss")
    _need(lse, torch.float32, 2 * n, "lse")
    total, count, workspace = _reduce_outputs(dev, reduction, total, count, workspace)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().ce_forward_ex(_ptr(logits), lay, DTYPE_CODE[logits.dtype], _ptr(targets), n, V,
                             options(label_smoothing, ignore_index, reduction), _ptr(loss), _ptr(lse), _ptr(total),
                             _ptr(count), _ptr(workspace), ws_bytes, _stream(logits))
    _check(st, "ce_forward_ex")
    return loss, lse, total, count


def ce_forward_ex_noalloc(logits: torch.Tensor, targets: torch.Tensor, label_smoothing: float, ignore_index,
                          reduction: str, loss: torch.Tensor, lse: torch.Tensor, total=None, count=None):
    """ce_forward_ex with the library's fixed per-GPU reduction scratch: the caller passes
    every output (total and count for a sum or mean) and nothing is allocated."""
    lay, n, V = _rows_view(logits, "logits")
    _need(targets, torch.int32, n, "targets")
    _need(loss, torch.float32, n, "loss")
    _need(lse, torch.float32, 2 * n, "lse")
    if reduction != "none":
        _need(total, torch.float32, 1, "total")
        _need(count, torch.int64, 1, "count")
    st = lib().ce_forward_ex_noalloc(_ptr(logits), lay, DTYPE_CODE[logits.dtype], _ptr(targets), n, V,
                                     options(label_smoothing, ignore_index, reduction), _ptr(loss), _ptr(lse),
                                     _ptr(total), _ptr(count), _stream(logits))
    _check(st, "ce_forward_ex_noalloc")
    return loss, lse, total, count


def ce_vjp_ex(logits: torch.Tensor, targets: torch.Tensor, lse: torch.Tensor, g: torch.Tensor,
              label_smoothing: float = 0.0, ignore_index=None, reduction: str = "none", count=None, dlogits=None):
    """Gradient of ce_forward_ex's loss: g per row ('none') or g [1] of the total."""
    lay, n, V = _rows_view(logits, "logits")
    _need(targets, torch.int32, n, "targets")
    _need(lse, torch.float32, 2 * n, "lse")
    _upstream(g, n, reduction)
    if dlogits is None:
        dlogits = torch.empty(logits.shape, dtype=logits.dtype, device=logits.device)
    if dlogits.dtype != logits.dtype or dlogits.shape != logits.shape:
        raise ValueError("dlogits must match logits in dtype and shape")
    olay, _, _ = _rows_view(dlogits, "dlogits")
    st = lib().ce_vjp_ex(_ptr(logits), lay, DTYPE_CODE[logits.dtype], _ptr(targets), _ptr(lse), _ptr(g), n, V,
                         options(label_smoothing, ignore_index, reduction), _ptr(count), _ptr(dlogits), olay,
                         _stream(logits))
    _check(st, "ce_vjp_ex")
    return dlogits


def ce_forward_probs(logits: torch.Tensor, probs: torch.Tensor, label_smoothing: float = 0.0,
                     reduction: str = "none", loss=None, lse=None, wsum=None, total=None, count=None,
                     workspace=None):
    """(loss [n], lse [n, 2], wsum [n], total, count) with probability targets of the logits' dtype."""
    lay, n, V = _rows_view(logits, "logits")
    if probs.dtype != logits.dtype or probs.shape != logits.shape:
        raise ValueError("probs must match logits in dtype and shape")
    play, _, _ = _rows_view(probs, "probs")
    dev = logits.device
    loss = torch.empty(n, dtype=torch.float32, device=dev) if loss is None else loss
    lse = torch.empty(n, 2, dtype=torch.float32, device=dev) if lse is None else lse
    wsum = torch.empty(n, dtype=torch.float32, device=dev) if wsum is None else wsum
    _need(loss, torch.float32, n, "loss")
    _need(lse, torch.float32, 2 * n, "lse")
    _need(wsum, torch.float32, n, "wsum")
    total, count, workspace = _reduce_outputs(dev, reduction, total, count, workspace)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().ce_forward_probs(_ptr(logits), lay, DTYPE_CODE[logits.dtype], _ptr(probs), play, n, V,
                                options(label_smoothing, None, reduction), _ptr(loss), _ptr(lse), _ptr(wsum),
                                _ptr(total), _ptr(count), _ptr(workspace), ws_bytes, _stream(logits))
    _check(st, "ce_forward_probs")
    return loss, lse, wsum, total, count


def ce_vjp_probs(logits: torch.Tensor, probs: torch.Tensor, lse: torch.Tensor, wsum: torch.Tensor, g: torch.Tensor,
                 label_smoothing: float = 0.0, reduction: str = "none", count=None, dlogits=None):
    """Gradient of ce_forward_probs's loss: g (W p - w)."""
    lay, n, V = _rows_view(logits, "logits")
    if probs.dtype != logits.dtype or probs.shape != logits.shape:
        raise ValueError("probs must match logits in dtype and shape")
    play, _, _ = _rows_view(probs, "probs")
    _need(lse, torch.float32, 2 * n, "lse")
    _need(wsum, torch.float32, n, "wsum")
    _upstream(g, n, reduction)
    if dlogits is None:
        dlogits = torch.empty(logits.shape, dtype=logits.dtype, device=logits.device)
    if dlogits.dtype != logits.dtype or dlogits.shape != logits.shape:
        raise ValueError("dlogits must match logits in dtype and shape")
    olay, _, _ = _rows_view(dlogits, "dlogits")
    st = lib().ce_vjp_probs(_ptr(logits), lay, DTYPE_CODE[logits.dtype], _ptr(probs), play, _ptr(lse), _ptr(wsum),
                            _ptr(g), n, V, options(label_smoothing, None, reduction), _ptr(count), _ptr(dlogits),
                            olay, _stream(logits))
    _check(st, "ce_vjp_probs")
    return dlogits


def lce_workspace_size(N: int, D: int, V: int) -> int:
    return int(lib().lce_workspace_size(N, D, V))


def lce_forward(H: torch.Tensor, W: torch.Tensor, targets: torch.Tensor, loss=None, lse=None, workspace=None):
    """Per-row (loss [N], lse [N, 2]) of H.W^T for bf16 H [N, D] and W [V, D]."""
    if H.dtype != torch.bfloat16 or W.dtype != torch.bfloat16 or H.dim() != 2 or W.dim() != 2:
        raise ValueError("H and W must be 2-D bfloat16 tensors")
    if not H.is_contiguous() or not W.is_contiguous() or H.shape[1] != W.shape[1]:
        raise ValueError("H [N, D] and W [V, D] must be contiguous with the same D")
    N, D = H.shape
    V = W.shape[0]
    _need(targets, torch.int32, N, "targets")
    if loss is None:
        loss = torch.empty(N, dtype=torch.float32, device=H.device)
    if lse is None:
        lse = torch.empty(N, 2, dtype=torch.float32, device=H.device)
    need = lce_workspace_size(N, D, V)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=H.device)
    st = lib().lce_forward(_ptr(H), _ptr(W), _ptr(targets), N, D, V, _ptr(loss), _ptr(lse), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(H))
    _check(st, "lce_forward")
    return loss, lse


def lce_backward_workspace_size(N: int, D: int, V: int) -> int:
    return int(lib().lce_backward_workspace_size(N, D, V))


def lce_backward_workspace_size_one_pass(N: int, D: int, V: int) -> int:
    return int(lib().lce_backward_workspace_size_one_pass(N, D, V))


def lce_backward(H: torch.Tensor, W: torch.Tensor, targets: torch.Tensor, lse: torch.Tensor, g: torch.Tensor,
                 dH=None, dW=None, workspace=None, one_pass: bool = False):
    """(dH [N, D], dW [V, D]) float32 of sum_i g_i loss_i, from lce_forward's lse [N, 2].
    Without a workspace, one of lce_backward_workspace_size bytes is allocated (chunks of
    8192 columns), or of lce_backward_workspace_size_one_pass bytes with one_pass."""
    if H.dtype != torch.bfloat16 or W.dtype != torch.bfloat16 or H.dim() != 2 or W.dim() != 2:
        raise ValueError("H and W must be 2-D bfloat16 tensors")
    if not H.is_contiguous() or not W.is_contiguous() or H.shape[1] != W.shape[1]:
        raise ValueError("H [N, D] and W [V, D] must be contiguous with the same D")
    N, D = H.shape
    V = W.shape[0]
    _need(targets, torch.int32, N, "targets")
    _need(g, torch.float32, N, "g")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (N, 2) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of shape [N, 2]")
    if dH is None:
        dH = torch.empty(N, D, dtype=torch.float32, device=H.device)
    if dW is None:
        dW = torch.empty(V, D, dtype=torch.float32, device=H.device)
    need = (lce_backward_workspace_size_one_pass if one_pass else lce_backward_workspace_size)(N, D, V)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=H.device)
    st = lib().lce_backward(_ptr(H), _ptr(W), _ptr(targets), _ptr(lse), _ptr(g), N, D, V, _ptr(dH), _ptr(dW),
                            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(H))
    _check(st, "lce_backward")
    return dH, dW


def _view(t: torch.Tensor, name: str):
    if t.stride(-1) != 1 and t.shape[-1] > 1:
        raise ValueError(f"{name} needs unit column stride")
    return rows_layout(t)


def kl_forward(q: torch.Tensor, p: torch.Tensor, kl=None, lse_q=None, lse_p=None, lanes_per_row: int = 0):
    """Per-row (kl [n], lse_q [n, 2], lse_p [n, 2]) of the teacher p from the student q."""
    if q.dtype != p.dtype or q.shape != p.shape:
        raise ValueError("q and p must have the same dtype and shape")
    ql, n, V = _view(q, "q")
    pl, _, _ = _view(p, "p")
    dev = q.device
    kl = torch.empty(n, dtype=torch.float32, device=dev) if kl is None else kl
    lse_q = torch.empty(n, 2, dtype=torch.float32, device=dev) if lse_q is None else lse_q
    lse_p = torch.empty(n, 2, dtype=torch.float32, device=dev) if lse_p is None else lse_p
    _need(kl, torch.float32, n, "kl")
    _need(lse_q, torch.float32, 2 * n, "lse_q")
    _need(lse_p, torch.float32, 2 * n, "lse_p")
    args = (_ptr(q), ql, _ptr(p), pl, DTYPE_CODE[q.dtype], n, V, _ptr(kl), _ptr(lse_q), _ptr(lse_p))
    if lanes_per_row == 0:
        st = lib().kl_forward(*args, _stream(q))
    else:
        st = lib().kl_forward_lanes(*args, int(lanes_per_row), _stream(q))
    _check(st, "kl_forward")
    return kl, lse_q, lse_p


def kl_vjp(q: torch.Tensor, p: torch.Tensor, lse_q: torch.Tensor, lse_p: torch.Tensor, g: torch.Tensor, dq=None,
           lanes_per_row: int = 0):
    """dq = g * (softmax(q) - softmax(p)) from the saved pairs; same shape and dtype as q."""
    if q.dtype != p.dtype or q.shape != p.shape:
        raise ValueError("q and p must have the same dtype and shape")
    ql, n, V = _view(q, "q")
    pl, _, _ = _view(p, "p")
    _need(lse_q, torch.float32, 2 * n, "lse_q")
    _need(lse_p, torch.float32, 2 * n, "lse_p")
    _need(g, torch.float32, n, "g")
    if dq is None:
        dq = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if dq.dtype != q.dtype or dq.shape != q.shape:
        raise ValueError("dq must match q in dtype and shape")
    dl, _, _ = _view(dq, "dq")
    args = (_ptr(q), ql, _ptr(p), pl, DTYPE_CODE[q.dtype], _ptr(lse_q), _ptr(lse_p), _ptr(g), n, V, _ptr(dq), dl)
    if lanes_per_row == 0:
        st = lib().kl_vjp(*args, _stream(q))
    else:
        st = lib().kl_vjp_lanes(*args, int(lanes_per_row), _stream(q))
    _check(st, "kl_vjp")
    return dq

