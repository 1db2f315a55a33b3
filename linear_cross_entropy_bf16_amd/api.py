"""PyTorch-facing API of the fused linear cross-entropy.

Argument marshalling only: torch supplies device memory and the current HIP
stream, every step of the computation runs in libflce.so.  Tensors must live
on a ROCm GPU; there is no CPU path.

    loss = linear_cross_entropy(x, weight, target, bias=None, ignore_index=-100,
                                label_smoothing=0.0, lse_square_scale=0.0,
                                softcap=0.0, reduction="mean")

``weight`` is the LM-head matrix in nn.Linear layout [V, D]; ``x`` is [..., D]
(leading dimensions are flattened into tokens); ``target`` holds class ids with
the same leading shape.
"""
from __future__ import annotations

import functools
from typing import Optional, Tuple

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.DTYPE_BF16, torch.float32: _lib.DTYPE_F32}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _on_tensor_device(fn):
    """Run ``fn`` with the first argument's GPU as the current device: the
    library launches on the current HIP device."""
    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        first = args[0] if args else None
        if isinstance(first, torch.Tensor) and first.device.type == "cuda":
            with torch.cuda.device(first.device):
                return fn(*args, **kwargs)
        return fn(*args, **kwargs)   # the argument checks raise
    return wrapper


def _check(status: int, what: str) -> None:
    if status != _lib.FLCE_OK:
        raise _lib.FLCEError(status, what)


def _prepare(x, weight, target, bias):
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise ValueError("x must be a tensor on a ROCm GPU (device 'cuda')")
    if x.dtype not in _DTYPES:
        raise TypeError(f"x must be bfloat16 or float32, got {x.dtype}")
    if weight.dtype != x.dtype or (bias is not None and bias.dtype != x.dtype):
        raise TypeError("x, weight and bias must share one dtype")
    if weight.dim() != 2 or weight.shape[1] != x.shape[-1]:
        raise ValueError(f"weight must be [V, D] with D = x.shape[-1]; got {tuple(weight.shape)}")
    dev = x.device
    for name, t in (("weight", weight), ("target", target), ("bias", bias)):
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, x on {dev}")
    d = x.shape[-1]
    x2 = x.reshape(-1, d).contiguous()
    t2 = target.reshape(-1)
    if t2.numel() != x2.shape[0]:
        raise ValueError("target must have one entry per row of x")
    t2 = t2.to(torch.int32).contiguous()
    w2 = weight.contiguous()
    b2 = bias.contiguous() if bias is not None else None
    if b2 is not None and b2.shape != (w2.shape[0],):
        raise ValueError("bias must be [V]")
    return x2, w2, t2, b2


def _check_buffer(t, name, shape, dtype, device):
    """A caller-supplied buffer must match what the library will write."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_params(n, d, v, dtype, ignore_index=-100, label_smoothing=0.0, lse_square_scale=0.0,
                softcap=0.0, reduction="mean", vocab_slice=0, token_chunk=0,
                dw_bf16=False, class_weight=None) -> _lib.Params:
    """``class_weight``: None, or a contiguous fp32 [v] tensor on the device
    (the caller keeps it alive while the call runs)."""
    return _lib.make_params(n, d, v, _DTYPES[dtype], ignore_index, label_smoothing,
                            lse_square_scale, softcap, reduction, vocab_slice, token_chunk,
                            1 if dw_bf16 else 0, _ptr(class_weight))


def _weights(class_weight, v, device):
    if class_weight is None:
        return None
    if class_weight.numel() != v:
        raise ValueError(f"class_weight must have V = {v} entries, got {class_weight.numel()}")
    return class_weight.detach().to(device=device, dtype=torch.float32).reshape(v).contiguous()


def workspace_bytes(n, d, v, dtype=torch.bfloat16, with_backward=True, stored_logits=False,
                    **opts) -> int:
    """Workspace of the calls for these sizes and options (``make_params``
    keywords); ``stored_logits``: of the three-contraction schedule."""
    p = make_params(n, d, v, dtype, **opts)
    return _lib.stored_workspace_size(p) if stored_logits else _lib.workspace_size(p, with_backward)


def _workspace(params, with_backward, device) -> Tuple[torch.Tensor, int]:
    nbytes = _lib.workspace_size(params, with_backward)
    if nbytes == 0:
        raise _lib.FLCEError(_lib.FLCE_ERR_INVALID_ARGUMENT, "workspace size")
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


@_on_tensor_device
def forward(x, weight, target, bias=None, *, ignore_index=-100, label_smoothing=0.0,
            lse_square_scale=0.0, softcap=0.0, reduction="mean", vocab_slice=0,
            check_targets=False, return_metrics=False, class_weight=None):
    """Returns (loss, lse, row_loss): loss is a 0-d tensor ([N] for 'none'),
    lse and row_loss are fp32 [N].  With ``return_metrics`` also the predicted
    tokens (int32 [N], -1 on ignored rows) and the token accuracy (0-d fp32)."""
    x2, w2, t2, b2 = _prepare(x, weight, target, bias)
    n, d = x2.shape
    v = w2.shape[0]
    cw = _weights(class_weight, v, x2.device)
    p = make_params(n, d, v, x2.dtype, ignore_index, label_smoothing, lse_square_scale, softcap,
                    reduction, vocab_slice, class_weight=cw)
    dev = x2.device
    ws, nbytes = _workspace(p, False, dev)
    loss = torch.empty(n if reduction == "none" else 1, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)
    row_loss = torch.empty(n, dtype=torch.float32, device=dev)
    st = _stream(dev)
    if return_metrics:
        pred = torch.empty(n, dtype=torch.int32, device=dev)
        acc = torch.empty(1, dtype=torch.float32, device=dev)
        _check(_lib.forward_metrics(p, _ptr(x2), _ptr(w2), _ptr(b2), _ptr(t2), _ptr(loss), _ptr(lse),
                                    _ptr(row_loss), _ptr(pred), _ptr(acc), _ptr(ws), nbytes, st),
               "flce_forward_metrics")
    else:
        _check(_lib.forward(p, _ptr(x2), _ptr(w2), _ptr(b2), _ptr(t2), _ptr(loss), _ptr(lse),
                            _ptr(row_loss), _ptr(ws), nbytes, st), "flce_forward")
    if check_targets:
        _check(_lib.check_status(_ptr(ws), st), "target check")
    out = ((loss if reduction == "none" else loss[0]), lse, row_loss)
    return out + (pred, acc[0]) if return_metrics else out


@_on_tensor_device
def backward(x, weight, target, lse, grad_output=None, bias=None, *, ignore_index=-100,
             label_smoothing=0.0, lse_square_scale=0.0, softcap=0.0, reduction="mean",
             vocab_slice=0, token_chunk=0, dw_bf16=False, class_weight=None):
    """Returns (dx, dw, db): dx in x's dtype, dw fp32 (bf16 with ``dw_bf16``)
    and db fp32 (db None without bias).  grad_output is a device scalar
    (None = 1.0).  ``token_chunk`` > 0 runs the backward over that many packed
    rows at a time."""
    x2, w2, t2, b2 = _prepare(x, weight, target, bias)
    n, d = x2.shape
    v = w2.shape[0]
    cw = _weights(class_weight, v, x2.device)
    p = make_params(n, d, v, x2.dtype, ignore_index, label_smoothing, lse_square_scale, softcap,
                    reduction, vocab_slice, token_chunk, dw_bf16, cw)
    dev = x2.device
    ws, nbytes = _workspace(p, True, dev)
    g = None
    if grad_output is not None:
        g = grad_output.detach().reshape(1).to(device=dev, dtype=torch.float32).contiguous()
    lse = lse.detach().to(torch.float32).contiguous()
    dx = torch.empty((n, d), dtype=x2.dtype, device=dev)
    dw = torch.empty((v, d), dtype=torch.bfloat16 if dw_bf16 else torch.float32, device=dev)
    db = torch.empty(v, dtype=torch.float32, device=dev) if b2 is not None else None
    _check(_lib.backward(p, _ptr(x2), _ptr(w2), _ptr(b2), _ptr(t2), _ptr(lse), _ptr(g), _ptr(dx),
                         _ptr(dw), _ptr(db), _ptr(ws), nbytes, _stream(dev)), "flce_backward")
    return dx.reshape(x.shape), dw, db


@_on_tensor_device
def fused_fwd_bwd(x, weight, target, bias=None, *, ignore_index=-100, label_smoothing=0.0,
                  lse_square_scale=0.0, softcap=0.0, reduction="mean", vocab_slice=0,
                  token_chunk=0, dw_bf16=False, workspace: Optional[torch.Tensor] = None, out=None,
                  stored_logits=False, class_weight=None):
    """One call computing (loss, lse, dx, dw, db) with grad_output = 1.
    ``workspace`` and ``out`` (a tuple of preallocated loss, lse, dx, dw, db)
    let a caller reuse buffers across steps; ``token_chunk`` and ``dw_bf16``
    as for ``backward``.  ``stored_logits`` selects the three-contraction
    schedule (each token chunk's logits kept instead of recomputed)."""
    x2, w2, t2, b2 = _prepare(x, weight, target, bias)
    n, d = x2.shape
    v = w2.shape[0]
    cw = _weights(class_weight, v, x2.device)
    p = make_params(n, d, v, x2.dtype, ignore_index, label_smoothing, lse_square_scale, softcap,
                    reduction, vocab_slice, token_chunk, dw_bf16, cw)
    dev = x2.device
    nbytes = _lib.stored_workspace_size(p) if stored_logits else _lib.workspace_size(p, True)
    if nbytes == 0:
        raise _lib.FLCEError(_lib.FLCE_ERR_INVALID_ARGUMENT, "workspace size")
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    else:
        _check_buffer(workspace, "workspace", (workspace.numel(),), torch.uint8, dev)
        if workspace.numel() < nbytes:
            raise _lib.FLCEError(_lib.FLCE_ERR_WORKSPACE_TOO_SMALL, "fused_fwd_bwd")
        nbytes = workspace.numel()
    dw_dtype = torch.bfloat16 if dw_bf16 else torch.float32
    if out is None:
        loss = torch.empty(1, dtype=torch.float32, device=dev)
        lse = torch.empty(n, dtype=torch.float32, device=dev)
        dx = torch.empty((n, d), dtype=x2.dtype, device=dev)
        dw = torch.empty((v, d), dtype=dw_dtype, device=dev)
        db = torch.empty(v, dtype=torch.float32, device=dev) if b2 is not None else None
    else:
        loss, lse, dx, dw, db = out
        # the library writes through these pointers with the sizes above: a
        # short or mistyped buffer would be overrun on the device
        _check_buffer(loss, "out loss", (1,), torch.float32, dev)
        _check_buffer(lse, "out lse", (n,), torch.float32, dev)
        _check_buffer(dx, "out dx", (n, d), x2.dtype, dev)
        _check_buffer(dw, "out dw", (v, d), dw_dtype, dev)
        if b2 is not None:
            _check_buffer(db, "out db", (v,), torch.float32, dev)
    call = _lib.fused_fwd_bwd_stored if stored_logits else _lib.fused_fwd_bwd
    _check(call(p, _ptr(x2), _ptr(w2), _ptr(b2), _ptr(t2), _ptr(loss), _ptr(lse), _ptr(dx), _ptr(dw),
                _ptr(db), _ptr(workspace), nbytes, _stream(dev)),
           "flce_fused_fwd_bwd_stored" if stored_logits else "flce_fused_fwd_bwd")
    return loss[0], lse, dx, dw, db


class LinearCrossEntropyFunction(torch.autograd.Function):
    """Autograd wrapper: the forward keeps only the per-row LSE; the backward
    recomputes the softmax from it inside the library."""

    @staticmethod
    def forward(ctx, x, weight, target, bias, ignore_index, label_smoothing, lse_square_scale,
                softcap, reduction, class_weight=None):
        loss, lse, _ = forward(x, weight, target, bias, ignore_index=ignore_index,
                               label_smoothing=label_smoothing, lse_square_scale=lse_square_scale,
                               softcap=softcap, reduction=reduction, class_weight=class_weight)
        ctx.save_for_backward(x, weight, target, bias, lse)
        ctx.opts = dict(ignore_index=ignore_index, label_smoothing=label_smoothing,
                        lse_square_scale=lse_square_scale, softcap=softcap, reduction=reduction,
                        class_weight=class_weight)
        ctx.mark_non_differentiable(lse)
        return loss, lse

    @staticmethod
    def backward(ctx, grad_loss, grad_lse=None):   # lse is not differentiable
        x, weight, target, bias, lse = ctx.saved_tensors
        if ctx.opts["reduction"] == "none":
            raise RuntimeError("reduction='none' has no backward in the fused kernel; "
                               "use 'mean' or 'sum'")
        # a bf16 weight gets its gradient in bf16 straight from the dW kernel
        # (one rounding of the fp32 sum, as a cast would do, without the fp32 copy)
        dx, dw, db = backward(x, weight, target, lse, grad_output=grad_loss, bias=bias,
                              dw_bf16=weight.dtype == torch.bfloat16, **ctx.opts)
        return (dx.to(x.dtype), dw.to(weight.dtype), None,
                db.to(bias.dtype) if db is not None else None, None, None, None, None, None, None)


def linear_cross_entropy(x, weight, target, bias=None, ignore_index=-100, label_smoothing=0.0,
                         lse_square_scale=0.0, softcap=0.0, reduction="mean", class_weight=None,
                         return_lse=False):
    """Fused LM-head projection + cross-entropy; differentiable in x, weight
    and bias (reduction 'mean' or 'sum'; 'none' is forward-only).
    ``class_weight``: optional [V] per-class weights (torch's weighted
    cross-entropy; not differentiated).  ``return_lse``: also return the
    per-row log-sum-exp (fp32 [N], 0 on ignored rows; not differentiable)."""
    loss, lse = LinearCrossEntropyFunction.apply(x, weight, target, bias, ignore_index,
                                                 label_smoothing, lse_square_scale, softcap,
                                                 reduction, class_weight)
    return (loss, lse) if return_lse else loss


class LinearCrossEntropyLoss(torch.nn.Module):
    """Module form of ``linear_cross_entropy`` for an LM head: holds the
    loss options; ``forward(x, weight, target, bias=None)`` with ``weight``
    the head's [V, D] matrix (for example ``lm_head.weight``)."""

    def __init__(self, ignore_index=-100, label_smoothing=0.0, lse_square_scale=0.0, softcap=0.0,
                 reduction="mean", class_weight=None):
        super().__init__()
        if reduction not in ("mean", "sum", "none"):
            raise ValueError(f"reduction must be 'mean', 'sum' or 'none', got {reduction!r}")
        if not 0.0 <= label_smoothing <= 1.0:
            raise ValueError(f"label_smoothing must lie in [0, 1], got {label_smoothing}")
        self.ignore_index = ignore_index
        self.label_smoothing = label_smoothing
        self.lse_square_scale = lse_square_scale
        self.softcap = softcap
        self.reduction = reduction
        self.register_buffer("class_weight", class_weight, persistent=False)

    def forward(self, x, weight, target, bias=None):
        return linear_cross_entropy(x, weight, target, bias, self.ignore_index, self.label_smoothing,
                                    self.lse_square_scale, self.softcap, self.reduction,
                                    self.class_weight)

    def extra_repr(self):
        return (f"ignore_index={self.ignore_index}, label_smoothing={self.label_smoothing}, "
                f"lse_square_scale={self.lse_square_scale}, softcap={self.softcap}, "
                f"reduction={self.reduction!r}")


# ------------------------------------------------- cross-entropy on logits

def _prepare_logits(logits, target):
    if not isinstance(logits, torch.Tensor) or logits.device.type != "cuda":
        raise ValueError("logits must be a tensor on a ROCm GPU (device 'cuda')")
    if logits.dtype not in _DTYPES:
        raise TypeError(f"logits must be bfloat16 or float32, got {logits.dtype}")
    if target.device != logits.device:
        raise ValueError(f"target is on {target.device}, logits on {logits.device}")
    v = logits.shape[-1]
    r2 = logits.reshape(-1, v).contiguous()
    if r2.data_ptr() % 16:
        r2 = r2.clone()                      # a fresh allocation is 16-byte aligned
    t2 = target.reshape(-1)
    if t2.numel() != r2.shape[0]:
        raise ValueError("target must have one entry per row of logits")
    return r2, t2.to(torch.int32).contiguous()


def _ce_params(r2, ignore_index, label_smoothing, lse_square_scale, softcap, reduction):
    n, v = r2.shape
    return make_params(n, 8, v, r2.dtype, ignore_index, label_smoothing, lse_square_scale, softcap,
                       reduction)


def _ce_workspace(p, device):
    nbytes = _lib.ce_workspace_size(p)
    if nbytes == 0:
        raise _lib.FLCEError(_lib.FLCE_ERR_INVALID_ARGUMENT, "workspace size")
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


@_on_tensor_device
def cross_entropy_forward(logits, target, *, ignore_index=-100, label_smoothing=0.0,
                          lse_square_scale=0.0, softcap=0.0, reduction="mean", check_targets=False,
                          return_metrics=False):
    """Cross-entropy on given logits [..., V]: returns (loss, lse, row_loss)
    like ``forward`` (plus predicted tokens and token accuracy with
    ``return_metrics``)."""
    r2, t2 = _prepare_logits(logits, target)
    p = _ce_params(r2, ignore_index, label_smoothing, lse_square_scale, softcap, reduction)
    n = r2.shape[0]
    dev = r2.device
    ws, nbytes = _ce_workspace(p, dev)
    loss = torch.empty(n if reduction == "none" else 1, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)
    row_loss = torch.empty(n, dtype=torch.float32, device=dev)
    st = _stream(dev)
    if return_metrics:
        pred = torch.empty(n, dtype=torch.int32, device=dev)
        acc = torch.empty(1, dtype=torch.float32, device=dev)
        _check(_lib.ce_forward_metrics(p, _ptr(r2), _ptr(t2), _ptr(loss), _ptr(lse), _ptr(row_loss),
                                       _ptr(pred), _ptr(acc), _ptr(ws), nbytes, st),
               "flce_ce_forward_metrics")
    else:
        _check(_lib.ce_forward(p, _ptr(r2), _ptr(t2), _ptr(loss), _ptr(lse), _ptr(row_loss),
                               _ptr(ws), nbytes, st), "flce_ce_forward")
    if check_targets:
        _check(_lib.check_status(_ptr(ws), st), "target check")
    out = ((loss if reduction == "none" else loss[0]), lse, row_loss)
    return out + (pred, acc[0]) if return_metrics else out


@_on_tensor_device
def cross_entropy_backward(logits, target, lse, grad_output=None, *, ignore_index=-100,
                           label_smoothing=0.0, lse_square_scale=0.0, softcap=0.0,
                           reduction="mean", inplace=False):
    """dL/dlogits in the logits' dtype and shape; ``inplace`` overwrites the
    logits (when they are already a contiguous, 16-byte aligned tensor)."""
    r2, t2 = _prepare_logits(logits, target)
    p = _ce_params(r2, ignore_index, label_smoothing, lse_square_scale, softcap, reduction)
    dev = r2.device
    ws, nbytes = _ce_workspace(p, dev)
    g = None
    if grad_output is not None:
        g = grad_output.detach().reshape(1).to(device=dev, dtype=torch.float32).contiguous()
    lse = lse.detach().to(torch.float32).contiguous()
    out = r2 if inplace else torch.empty_like(r2)
    _check(_lib.ce_backward(p, _ptr(r2), _ptr(t2), _ptr(lse), _ptr(g), _ptr(out), _ptr(ws), nbytes,
                            _stream(dev)), "flce_ce_backward")
    return out.reshape(logits.shape)


@_on_tensor_device
def cross_entropy_fused_fwd_bwd(logits, target, *, ignore_index=-100, label_smoothing=0.0,
                                lse_square_scale=0.0, softcap=0.0, reduction="mean", inplace=False,
                                workspace: Optional[torch.Tensor] = None, out=None):
    """(loss, lse, dlogits) in one pass per row, grad_output = 1.  ``out`` is
    an optional (loss [1], lse [N], dlogits) tuple to reuse."""
    r2, t2 = _prepare_logits(logits, target)
    p = _ce_params(r2, ignore_index, label_smoothing, lse_square_scale, softcap, reduction)
    n = r2.shape[0]
    dev = r2.device
    nbytes = _lib.ce_workspace_size(p)
    if workspace is None:
        workspace, nbytes = _ce_workspace(p, dev)
    elif workspace.numel() < nbytes:
        raise _lib.FLCEError(_lib.FLCE_ERR_WORKSPACE_TOO_SMALL, "cross_entropy_fused_fwd_bwd")
    else:
        nbytes = workspace.numel()
    if out is None:
        loss = torch.empty(1, dtype=torch.float32, device=dev)
        lse = torch.empty(n, dtype=torch.float32, device=dev)
        grad = r2 if inplace else torch.empty_like(r2)
    else:
        loss, lse, grad = out
    _check(_lib.ce_fused_fwd_bwd(p, _ptr(r2), _ptr(t2), _ptr(loss), _ptr(lse), _ptr(grad),
                                 _ptr(workspace), nbytes, _stream(dev)), "flce_ce_fused_fwd_bwd")
    return loss[0], lse, grad.reshape(logits.shape)


class CrossEntropyFunction(torch.autograd.Function):
    """Autograd wrapper of the logits path: keeps only the per-row LSE."""

    @staticmethod
    def forward(ctx, logits, target, ignore_index, label_smoothing, lse_square_scale, softcap,
                reduction):
        loss, lse, _ = cross_entropy_forward(logits, target, ignore_index=ignore_index,
                                             label_smoothing=label_smoothing,
                                             lse_square_scale=lse_square_scale, softcap=softcap,
                                             reduction=reduction)
        ctx.save_for_backward(logits, target, lse)
        ctx.opts = dict(ignore_index=ignore_index, label_smoothing=label_smoothing,
                        lse_square_scale=lse_square_scale, softcap=softcap, reduction=reduction)
        ctx.mark_non_differentiable(lse)
        return loss, lse

    @staticmethod
    def backward(ctx, grad_loss, grad_lse=None):   # lse is not differentiable
        logits, target, lse = ctx.saved_tensors
        if ctx.opts["reduction"] == "none":
            raise RuntimeError("reduction='none' is forward-only; use 'mean' or 'sum'")
        g = cross_entropy_backward(logits, target, lse, grad_output=grad_loss, **ctx.opts)
        return g, None, None, None, None, None, None


def cross_entropy(logits, target, ignore_index=-100, label_smoothing=0.0, lse_square_scale=0.0,
                  softcap=0.0, reduction="mean", return_lse=False):
    """Cross-entropy of given logits [..., V]; differentiable in the logits
    (reduction 'mean' or 'sum'; 'none' is forward-only).  ``return_lse``: also
    return the per-row log-sum-exp (fp32 [N], not differentiable)."""
    loss, lse = CrossEntropyFunction.apply(logits, target, ignore_index, label_smoothing,
                                           lse_square_scale, softcap, reduction)
    return (loss, lse) if return_lse else loss
