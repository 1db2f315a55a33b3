"""Fused linear cross-entropy for AMD Instinct MI355X (gfx950).

The computation lives in libflce.so (hand-written HIP kernels behind a C ABI,
include/flce.h); this package is its thin PyTorch binding.
"""
from .api import (CrossEntropyFunction, LinearCrossEntropyFunction, LinearCrossEntropyLoss,
                  backward, cross_entropy, cross_entropy_backward, cross_entropy_forward,
                  cross_entropy_fused_fwd_bwd, forward, fused_fwd_bwd, linear_cross_entropy,
                  workspace_bytes)
from ._lib import FLCEError

__all__ = ["linear_cross_entropy", "LinearCrossEntropyFunction", "LinearCrossEntropyLoss",
           "forward", "backward", "fused_fwd_bwd", "workspace_bytes", "cross_entropy",
           "CrossEntropyFunction", "cross_entropy_forward", "cross_entropy_backward",
           "cross_entropy_fused_fwd_bwd", "FLCEError"]
