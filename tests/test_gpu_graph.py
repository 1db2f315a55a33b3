"""A whole step captured in a HIP graph (needs an MI355X).

The library only launches kernels on the caller's stream (no allocation, no
synchronisation, no memset), so one fused call can be captured with
torch.cuda.graph and replayed.  Each test replays the graph several times,
with unrelated eager work and a change of the inputs between replays, and
checks every replay bit for bit against an eager call on the same inputs (the
kernels are deterministic)."""
import numpy as np
import pytest
import torch

from linear_cross_entropy_bf16_amd import api, workloads as W
from tests import gpu_utils as U

pytestmark = pytest.mark.gpu

IGN = -100


def problem(n, d, v, seed, bias=True):
    rng = np.random.default_rng(seed)
    x = W.f32_to_bf16_bits(rng.standard_normal((n, d), dtype=np.float32))
    w = W.f32_to_bf16_bits(rng.standard_normal((v, d), dtype=np.float32) * np.float32(1 / np.sqrt(d)))
    b = W.f32_to_bf16_bits(rng.standard_normal(v, dtype=np.float32) * np.float32(0.3)) if bias else None
    t = rng.integers(0, v, n).astype(np.int32)
    t[rng.choice(n, n // 10, replace=False)] = IGN
    return (U.dev_tensor(x, "bf16"), U.dev_tensor(w, "bf16"),
            U.dev_tensor(b, "bf16") if b is not None else None, torch.from_numpy(t).cuda())


def unrelated_eager_work():
    a = torch.randn(512, 512, device="cuda")
    (a @ a).sum().item()


def capture(fn):
    """Warm up on a side stream, then capture one call of fn."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def check_replays(g, outs, eager_fn, inputs, new_inputs):
    """Replays 1-2 on the captured inputs, replay 3 after the inputs were
    overwritten in place; each against an eager call."""
    want = [o.clone() for o in eager_fn()]
    for rep in range(3):
        if rep == 2:
            for dst, src in zip(inputs, new_inputs):
                dst.copy_(src)
            want = [o.clone() for o in eager_fn()]
        for o in outs:
            o.fill_(float("nan")) if o.is_floating_point() else o.zero_()
        unrelated_eager_work()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, ref) in enumerate(zip(outs, want)):
            assert torch.equal(got, ref), f"replay {rep}: output {i} differs from the eager call"


@pytest.mark.parametrize("stored", [False, True])
def test_fused_step_graph(stored):
    print(f"\n[gpu-graph] fused step stored={stored}", flush=True)
    n, d, v = 1000, 136, 3000
    x, w, b, t = problem(n, d, v, seed=11)
    x2, _, _, t2 = problem(n, d, v, seed=12)
    opts = dict(label_smoothing=0.1, lse_square_scale=1e-3, softcap=20.0)
    opts.update(dict(stored_logits=True, token_chunk=256) if stored else dict(vocab_slice=512))
    nbytes = api.workspace_bytes(n, d, v, torch.bfloat16, stored_logits=stored,
                                 **{k: opts[k] for k in opts if k in ("label_smoothing", "lse_square_scale",
                                                                     "softcap", "vocab_slice",
                                                                     "token_chunk")})
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = (torch.empty(1, device="cuda"), torch.empty(n, device="cuda"), torch.empty_like(x),
           torch.empty((v, d), device="cuda"), torch.empty(v, device="cuda"))

    def step():
        return api.fused_fwd_bwd(x, w, t, b, workspace=ws, out=out, **opts)

    def eager():
        loss, *rest = api.fused_fwd_bwd(x, w, t, b, **opts)
        return (loss.reshape(1), *rest)

    g = capture(step)
    check_replays(g, out, eager, (x, t), (x2, t2))


def test_logits_step_graph():
    print("\n[gpu-graph] logits step", flush=True)
    n, v = 300, 5001
    rng = np.random.default_rng(3)
    r = U.dev_tensor(W.f32_to_bf16_bits(rng.standard_normal((n, v), dtype=np.float32)), "bf16")
    r2 = U.dev_tensor(W.f32_to_bf16_bits(2 * rng.standard_normal((n, v), dtype=np.float32)), "bf16")
    t = torch.from_numpy(rng.integers(0, v, n).astype(np.int32)).cuda()
    t[::7] = IGN
    opts = dict(label_smoothing=0.1, softcap=10.0)
    out = (torch.empty(1, device="cuda"), torch.empty(n, device="cuda"), torch.empty_like(r))
    p = api._ce_params(r.view(-1, v), ignore_index=IGN, lse_square_scale=0.0, reduction="mean", **opts)
    from linear_cross_entropy_bf16_amd import _lib
    ws = torch.empty(max(_lib.ce_workspace_size(p), 1), dtype=torch.uint8, device="cuda")

    def step():
        return api.cross_entropy_fused_fwd_bwd(r, t, workspace=ws, out=out, **opts)

    def eager():
        loss, *rest = api.cross_entropy_fused_fwd_bwd(r, t, **opts)
        return (loss.reshape(1), *rest)

    g = capture(step)
    check_replays(g, out, eager, (r,), (r2,))


def test_calls_follow_the_current_stream():
    """A call made while a side stream is current is enqueued there: its
    results, read after that stream is synchronised, equal a call on the
    default stream bit for bit."""
    print("\n[gpu-graph] side stream", flush=True)
    n, d, v = 600, 72, 2000
    x, w, b, t = problem(n, d, v, seed=21)
    opts = dict(label_smoothing=0.1, softcap=12.0)
    want = api.fused_fwd_bwd(x, w, t, b, **opts)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = api.fused_fwd_bwd(x, w, t, b, **opts)
        lse_side = api.forward(x, w, t, b, **opts)[1]
    side.synchronize()
    for a, c in zip(got, want):
        assert torch.equal(a, c)
    assert torch.equal(lse_side, want[1])
