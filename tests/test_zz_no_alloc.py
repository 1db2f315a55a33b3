"""flce_fused_fwd_bwd_noalloc through the C ABI (needs an MI355X): the
library's own scratch array in place of a caller workspace.  Two calls in a
row, the second smaller, each against flce_fused_fwd_bwd on the same inputs
with a caller workspace, at the acceptance bars (and bit for bit, since the
kernels are the same); a problem too large for the array is refused on the
host before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from linear_cross_entropy_bf16_amd import _lib, workloads as W
from oracle import flce_oracle as O
from tests import gpu_utils as U

pytestmark = pytest.mark.gpu


def _problem(n, d, v, seed, bias):
    rng = np.random.default_rng(seed)
    x = W.f32_to_bf16_bits(rng.standard_normal((n, d), dtype=np.float32))
    w = W.f32_to_bf16_bits(rng.standard_normal((v, d), dtype=np.float32) * np.float32(1 / np.sqrt(d)))
    b = W.f32_to_bf16_bits(rng.standard_normal(v, dtype=np.float32) * np.float32(0.1)) if bias else None
    t = rng.integers(0, v, n).astype(np.int32)
    t[rng.choice(n, n // 10, replace=False)] = -100
    return dict(x=x, w=w, bias=b, targets=t)


def _outputs(n, d, v, bias):
    f32 = dict(dtype=torch.float32, device="cuda")
    return dict(loss=torch.full((1,), np.nan, **f32), lse=torch.full((n,), np.nan, **f32),
                dx=torch.full((n, d), np.nan, dtype=torch.bfloat16, device="cuda"),
                dw=torch.full((v, d), np.nan, **f32),
                db=torch.full((v,), np.nan, **f32) if bias else None)


def _call(inp, params, noalloc):
    n, d = inp["x"].shape
    v = inp["w"].shape[0]
    x = U.dev_tensor(inp["x"], "bf16")
    w = U.dev_tensor(inp["w"], "bf16")
    b = U.dev_tensor(inp["bias"], "bf16") if inp["bias"] is not None else None
    t = torch.from_numpy(inp["targets"]).cuda()
    o = _outputs(n, d, v, b is not None)
    ptr = lambda a: None if a is None else a.data_ptr()
    stream = torch.cuda.current_stream().cuda_stream
    args = (params, ptr(x), ptr(w), ptr(b), ptr(t), ptr(o["loss"]), ptr(o["lse"]), ptr(o["dx"]),
            ptr(o["dw"]), ptr(o["db"]))
    torch.cuda.synchronize()
    if noalloc:
        before = torch.cuda.memory_allocated()
        st = _lib.fused_fwd_bwd_noalloc(*args, stream)
        assert torch.cuda.memory_allocated() == before
    else:
        nbytes = _lib.workspace_size(params, True)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        st = _lib.fused_fwd_bwd(*args, ptr(ws), nbytes, stream)
    torch.cuda.synchronize()
    assert st == _lib.FLCE_OK, _lib.status_string(st)
    return {k: (None if a is None else a.clone()) for k, a in o.items()}


@pytest.mark.parametrize("bias", [False, True])
def test_noalloc_matches_the_workspace_call(bias):
    cases = [(2048, 512, 8000, 16), (700, 256, 3001, 16)]     # second call smaller than the first
    opts = dict(label_smoothing=0.1, lse_square_scale=1e-4, softcap=20.0)
    for n, d, v, seed in cases:
        print(f"\n[noalloc] n={n} d={d} v={v} bias={bias}", flush=True)
        inp = _problem(n, d, v, seed + n, bias)
        params = _lib.make_params(n, d, v, _lib.DTYPE_BF16, vocab_slice=1024, **opts)
        assert 0 < _lib.workspace_size(params, True) <= _lib.NOALLOC_MAX_BYTES
        got = _call(inp, params, noalloc=True)
        ref = _call(inp, params, noalloc=False)
        U.assert_loss(float(got["loss"].item()), float(ref["loss"].item()))
        U.assert_lse(U.host(got["lse"]), U.host(ref["lse"]))
        for k in ("dx", "dw", "db"):
            if ref[k] is not None:
                U.assert_close(U.host(got[k]), U.host(ref[k]), k)
                assert torch.equal(got[k], ref[k]), f"{k}: same kernels, same inputs, bit for bit"
        assert torch.equal(got["lse"], ref["lse"]) and torch.equal(got["loss"], ref["loss"])
        # and both against the oracle
        o = O.LossOptions(**opts)
        want = O.forward_backward(inp["x"], inp["w"], inp["bias"], inp["targets"], o)
        U.assert_loss(float(got["loss"].item()), want.loss)
        U.assert_close(U.host(got["dw"]), want.dw, "dW vs oracle")


def test_noalloc_refuses_problems_beyond_the_scratch_array():
    n, d, v = 4096, 2048, 32000                               # default slices: ~240 MB of workspace
    params = _lib.make_params(n, d, v, _lib.DTYPE_BF16)
    assert _lib.workspace_size(params, True) > _lib.NOALLOC_MAX_BYTES
    x = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((v, d), dtype=torch.bfloat16, device="cuda")
    t = torch.zeros(n, dtype=torch.int32, device="cuda")
    o = _outputs(n, d, v, False)
    st = _lib.fused_fwd_bwd_noalloc(params, x.data_ptr(), w.data_ptr(), None, t.data_ptr(),
                                    o["loss"].data_ptr(), o["lse"].data_ptr(), o["dx"].data_ptr(),
                                    o["dw"].data_ptr(), None, torch.cuda.current_stream().cuda_stream)
    assert st == _lib.FLCE_ERR_WORKSPACE_TOO_SMALL
    assert torch.isnan(o["loss"]).all()                       # nothing ran
