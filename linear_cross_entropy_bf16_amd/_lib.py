"""ctypes view of libflce.so (declarations mirror include/flce.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of the loss anywhere in the package.
"""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

FLCE_OK = 0
FLCE_ERR_INVALID_ARGUMENT = 1
FLCE_ERR_UNSUPPORTED = 2
FLCE_ERR_WORKSPACE_TOO_SMALL = 3
FLCE_ERR_TARGET_OUT_OF_RANGE = 4
FLCE_ERR_DEVICE = 5

DTYPE_BF16 = 0
DTYPE_F32 = 1

REDUCTIONS = {"mean": 0, "sum": 1, "none": 2}

EXPORTS = ("flce_workspace_size", "flce_forward", "flce_forward_metrics", "flce_backward",
           "flce_fused_fwd_bwd", "flce_ce_workspace_size", "flce_ce_forward", "flce_ce_forward_metrics",
           "flce_ce_backward", "flce_ce_fused_fwd_bwd", "flce_stored_workspace_size",
           "flce_fused_fwd_bwd_stored", "flce_fused_fwd_bwd_noalloc",
           "flce_check_status", "flce_status_string", "flce_version")


class Params(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int64),
        ("d", ctypes.c_int64),
        ("v", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("ignore_index", ctypes.c_int32),
        ("label_smoothing", ctypes.c_float),
        ("lse_square_scale", ctypes.c_float),
        ("softcap", ctypes.c_float),
        ("reduction", ctypes.c_int32),
        ("vocab_slice", ctypes.c_int32),
        ("token_chunk", ctypes.c_int32),
        ("dw_bf16", ctypes.c_int32),
        ("class_weight", ctypes.c_void_p),
    ]


class FLCEError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})" if what
                         else f"{status_string(status)} (status {status})")


_lib = None
_P = ctypes.c_void_p


def load():
    """Load libflce.so once; raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m linear_cross_entropy_bf16_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    pp = ctypes.POINTER(Params)
    lib.flce_workspace_size.argtypes = [pp, ctypes.c_int]
    lib.flce_workspace_size.restype = ctypes.c_size_t
    lib.flce_forward.argtypes = [pp, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.flce_forward.restype = ctypes.c_int
    lib.flce_forward_metrics.argtypes = [pp, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.flce_forward_metrics.restype = ctypes.c_int
    lib.flce_ce_forward_metrics.argtypes = [pp, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.flce_ce_forward_metrics.restype = ctypes.c_int
    lib.flce_backward.argtypes = [pp, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.flce_backward.restype = ctypes.c_int
    lib.flce_fused_fwd_bwd.argtypes = [pp, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.flce_fused_fwd_bwd.restype = ctypes.c_int
    lib.flce_stored_workspace_size.argtypes = [pp]
    lib.flce_stored_workspace_size.restype = ctypes.c_size_t
    lib.flce_fused_fwd_bwd_stored.argtypes = [pp, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                              _P]
    lib.flce_fused_fwd_bwd_stored.restype = ctypes.c_int
    lib.flce_fused_fwd_bwd_noalloc.argtypes = [pp, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.flce_fused_fwd_bwd_noalloc.restype = ctypes.c_int
    lib.flce_ce_workspace_size.argtypes = [pp]
    lib.flce_ce_workspace_size.restype = ctypes.c_size_t
    lib.flce_ce_forward.argtypes = [pp, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.flce_ce_forward.restype = ctypes.c_int
    lib.flce_ce_backward.argtypes = [pp, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.flce_ce_backward.restype = ctypes.c_int
    lib.flce_ce_fused_fwd_bwd.argtypes = [pp, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.flce_ce_fused_fwd_bwd.restype = ctypes.c_int
    lib.flce_check_status.argtypes = [_P, _P]
    lib.flce_check_status.restype = ctypes.c_int
    lib.flce_status_string.argtypes = [ctypes.c_int]
    lib.flce_status_string.restype = ctypes.c_char_p
    lib.flce_version.argtypes = []
    lib.flce_version.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load().flce_status_string(int(status)).decode()
    except RuntimeError:
        return f"status {status}"


def make_params(n, d, v, dtype, ignore_index=-100, label_smoothing=0.0, lse_square_scale=0.0,
                softcap=0.0, reduction="mean", vocab_slice=0, token_chunk=0, dw_bf16=0,
                class_weight=None) -> Params:
    """``reduction`` is 'mean', 'sum', 'none' or the raw enum value;
    ``class_weight`` a device address of fp32 [v] weights, or None."""
    if isinstance(reduction, str):
        if reduction not in REDUCTIONS:
            raise ValueError(f"reduction must be one of {tuple(REDUCTIONS)}, got {reduction!r}")
        reduction = REDUCTIONS[reduction]
    return Params(int(n), int(d), int(v), int(dtype), int(ignore_index), float(label_smoothing),
                  float(lse_square_scale), float(softcap), int(reduction), int(vocab_slice),
                  int(token_chunk), int(dw_bf16), class_weight)


def workspace_size(params: Params, with_backward: bool) -> int:
    return int(load().flce_workspace_size(ctypes.byref(params), 1 if with_backward else 0))


def forward(params, x, w, bias, targets, loss, lse, row_loss, ws, ws_bytes, stream) -> int:
    return load().flce_forward(ctypes.byref(params), x, w, bias, targets, loss, lse, row_loss, ws,
                               ws_bytes, stream)


def forward_metrics(params, x, w, bias, targets, loss, lse, row_loss, pred, accuracy, ws, ws_bytes,
                    stream) -> int:
    return load().flce_forward_metrics(ctypes.byref(params), x, w, bias, targets, loss, lse, row_loss,
                                       pred, accuracy, ws, ws_bytes, stream)


def ce_forward_metrics(params, logits, targets, loss, lse, row_loss, pred, accuracy, ws, ws_bytes,
                       stream) -> int:
    return load().flce_ce_forward_metrics(ctypes.byref(params), logits, targets, loss, lse, row_loss,
                                          pred, accuracy, ws, ws_bytes, stream)


def backward(params, x, w, bias, targets, lse, grad_output, dx, dw, dbias, ws, ws_bytes, stream) -> int:
    return load().flce_backward(ctypes.byref(params), x, w, bias, targets, lse, grad_output, dx, dw,
                                dbias, ws, ws_bytes, stream)


def fused_fwd_bwd(params, x, w, bias, targets, loss, lse, dx, dw, dbias, ws, ws_bytes, stream) -> int:
    return load().flce_fused_fwd_bwd(ctypes.byref(params), x, w, bias, targets, loss, lse, dx, dw,
                                     dbias, ws, ws_bytes, stream)


def stored_workspace_size(params: Params) -> int:
    return int(load().flce_stored_workspace_size(ctypes.byref(params)))


def fused_fwd_bwd_stored(params, x, w, bias, targets, loss, lse, dx, dw, dbias, ws, ws_bytes,
                         stream) -> int:
    return load().flce_fused_fwd_bwd_stored(ctypes.byref(params), x, w, bias, targets, loss, lse, dx,
                                            dw, dbias, ws, ws_bytes, stream)


NOALLOC_MAX_BYTES = 128 << 20   # the library's scratch array (include/flce.h)


def fused_fwd_bwd_noalloc(params, x, w, bias, targets, loss, lse, dx, dw, dbias, stream) -> int:
    return load().flce_fused_fwd_bwd_noalloc(ctypes.byref(params), x, w, bias, targets, loss, lse, dx,
                                             dw, dbias, stream)


def ce_workspace_size(params: Params) -> int:
    return int(load().flce_ce_workspace_size(ctypes.byref(params)))


def ce_forward(params, logits, targets, loss, lse, row_loss, ws, ws_bytes, stream) -> int:
    return load().flce_ce_forward(ctypes.byref(params), logits, targets, loss, lse, row_loss, ws,
                                  ws_bytes, stream)


def ce_backward(params, logits, targets, lse, grad_output, dlogits, ws, ws_bytes, stream) -> int:
    return load().flce_ce_backward(ctypes.byref(params), logits, targets, lse, grad_output, dlogits,
                                   ws, ws_bytes, stream)


def ce_fused_fwd_bwd(params, logits, targets, loss, lse, dlogits, ws, ws_bytes, stream) -> int:
    return load().flce_ce_fused_fwd_bwd(ctypes.byref(params), logits, targets, loss, lse, dlogits, ws,
                                        ws_bytes, stream)


def check_status(ws, stream) -> int:
    return load().flce_check_status(ws, stream)


def version() -> int:
    return int(load().flce_version())
