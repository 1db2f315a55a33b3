"""Seeded sweep over option combinations (needs an MI355X).

Each case draws its sizes and options from its own seed: ragged N, D and V,
bf16 or fp32, bias, label smoothing, z-loss, softcap, mean or sum, a share of
ignored rows, class weights, bf16 dW, and the schedule (recompute with a
vocabulary slice and token chunks, or stored logits).  Every output of the fused
call is compared with the fp64 oracle element by element, at the same bars as
the other parity tests."""
import numpy as np
import pytest
import torch

from linear_cross_entropy_bf16_amd import api, workloads as W
from oracle import flce_oracle as O
from tests import gpu_utils as U

pytestmark = pytest.mark.gpu

IGN = -100
N_CASES = 120


def draw_case(seed):
    """Sizes and options of one case; V >= 2 so that no loss is a pure
    cancellation of fp32 terms."""
    rng = np.random.default_rng(seed)
    case = dict(
        n=int(rng.integers(1, 700)),
        d=8 * int(rng.integers(1, 41)),
        v=int(rng.integers(2, 3000)),
        dtype=str(rng.choice(["bf16", "f32"])),
        bias=bool(rng.random() < 0.5),
        label_smoothing=float(rng.choice([0.0, 0.0, 0.1, 0.3])),
        lse_square_scale=float(rng.choice([0.0, 0.0, 1e-3])),
        softcap=float(rng.choice([0.0, 0.0, 4.0, 30.0])),
        reduction=str(rng.choice(["mean", "sum"])),
        ignore_frac=float(rng.choice([0.0, 0.1, 0.5])),
        weights=bool(rng.random() < 0.3),
        schedule=str(rng.choice(["recompute", "recompute", "stored"])),
        vocab_slice=int(rng.choice([0, 256, 512])),
        token_chunk=int(rng.choice([0, 0, 256])),
        dw_bf16=bool(rng.random() < 0.25),
    )
    return case


def make_inputs(c, seed):
    rng = np.random.default_rng(seed + 7)
    n, d, v = c["n"], c["d"], c["v"]
    x = rng.standard_normal((n, d), dtype=np.float32)
    w = rng.standard_normal((v, d), dtype=np.float32) * np.float32(1.5 / np.sqrt(d))
    b = rng.standard_normal(v, dtype=np.float32) * np.float32(0.3) if c["bias"] else None
    t = rng.integers(0, v, n).astype(np.int32)
    k = int(round(c["ignore_frac"] * n))
    if k:
        t[rng.choice(n, k, replace=False)] = IGN
    cw = rng.uniform(0.2, 2.5, v) if c["weights"] else None
    if c["dtype"] == "bf16":
        x, w = W.f32_to_bf16_bits(x), W.f32_to_bf16_bits(w)
        b = W.f32_to_bf16_bits(b) if b is not None else None
    return dict(x=x, w=w, bias=b, targets=t), cw


@pytest.mark.parametrize("case", range(N_CASES))
def test_option_sweep(case):
    seed = 4000 + case
    c = draw_case(seed)
    print(f"\n[gpu-sweep] case {case} seed {seed}: {c}", flush=True)
    inp, cw = make_inputs(c, seed)
    o = O.LossOptions(label_smoothing=c["label_smoothing"], lse_square_scale=c["lse_square_scale"],
                      softcap=c["softcap"], reduction=c["reduction"], class_weight=cw)
    dtype = c["dtype"]
    x = U.dev_tensor(inp["x"], dtype)
    w = U.dev_tensor(inp["w"], dtype)
    b = U.dev_tensor(inp["bias"], dtype) if inp["bias"] is not None else None
    t = torch.from_numpy(inp["targets"]).to("cuda")
    kw = dict(**U.lib_opts(o))
    if cw is not None:
        kw["class_weight"] = torch.tensor(cw, dtype=torch.float32, device="cuda")
    if c["schedule"] == "stored":
        kw.update(stored_logits=True, token_chunk=c["token_chunk"], dw_bf16=c["dw_bf16"])
    else:
        kw.update(vocab_slice=c["vocab_slice"], token_chunk=c["token_chunk"], dw_bf16=c["dw_bf16"])
    loss, lse, dx, dw, db = api.fused_fwd_bwd(x, w, t, b, **kw)
    torch.cuda.synchronize()
    got = dict(loss=float(loss.item()), lse=U.host(lse), dx=U.host(dx), dw=U.host(dw),
               db=None if db is None else U.host(db))
    ref = O.forward_backward(inp["x"], inp["w"], inp["bias"], inp["targets"], o)
    U.assert_loss(got["loss"], ref.loss)
    valid = inp["targets"] != IGN
    U.assert_lse(got["lse"][valid], ref.lse[valid])
    assert np.all(got["lse"][~valid] == 0.0), "ignored rows must have lse 0"
    if valid.any():
        U.assert_close(got["dx"], ref.dx, "dX")
        U.assert_close(got["dw"], ref.dw, "dW")
        if c["bias"]:
            U.assert_close(got["db"], ref.db, "db")
    else:
        assert np.all(got["dx"] == 0.0) and np.all(got["dw"] == 0.0)
    assert np.all(got["dx"][~valid] == 0.0), "ignored rows must have zero dX"


def draw_ce_case(seed):
    """Sizes and options of one cross-entropy-on-logits case (V >= 2)."""
    rng = np.random.default_rng(seed)
    return dict(
        n=int(rng.integers(0, 300)),
        v=int(rng.integers(2, 5000)),
        dtype=str(rng.choice(["bf16", "f32"])),
        label_smoothing=float(rng.choice([0.0, 0.0, 0.1, 0.3])),
        lse_square_scale=float(rng.choice([0.0, 0.0, 1e-3])),
        softcap=float(rng.choice([0.0, 0.0, 4.0, 30.0])),
        reduction=str(rng.choice(["mean", "sum"])),
        ignore_frac=float(rng.choice([0.0, 0.1, 0.5])),
        mode=str(rng.choice(["fused", "separate"])),
        inplace=bool(rng.random() < 0.3),
        spread=float(rng.choice([1.0, 3.0])),
    )


@pytest.mark.parametrize("case", range(N_CASES))
def test_logits_option_sweep(case):
    seed = 9000 + case
    c = draw_ce_case(seed)
    print(f"\n[gpu-sweep] logits case {case} seed {seed}: {c}", flush=True)
    rng = np.random.default_rng(seed + 3)
    n, v = c["n"], c["v"]
    r = rng.standard_normal((n, v), dtype=np.float32) * np.float32(c["spread"])
    t = rng.integers(0, v, n).astype(np.int32)
    k = int(round(c["ignore_frac"] * n))
    if k:
        t[rng.choice(n, k, replace=False)] = IGN
    if c["dtype"] == "bf16":
        r = W.f32_to_bf16_bits(r)
    o = O.LossOptions(label_smoothing=c["label_smoothing"], lse_square_scale=c["lse_square_scale"],
                      softcap=c["softcap"], reduction=c["reduction"])
    logits = U.dev_tensor(r, c["dtype"])
    tt = torch.from_numpy(t).to("cuda")
    if c["mode"] == "fused":
        loss, lse, g = api.cross_entropy_fused_fwd_bwd(logits, tt, inplace=c["inplace"], **U.lib_opts(o))
    else:
        loss, lse, _ = api.cross_entropy_forward(logits, tt, check_targets=True, **U.lib_opts(o))
        g = api.cross_entropy_backward(logits, tt, lse, None, inplace=c["inplace"], **U.lib_opts(o))
    torch.cuda.synchronize()
    ref = O.cross_entropy_on_logits(r, t, o)
    U.assert_loss(float(loss.item()), ref.loss)
    valid = t != IGN
    got_lse, got_g = U.host(lse), U.host(g)
    U.assert_lse(got_lse[valid], ref.lse[valid])
    assert np.all(got_lse[~valid] == 0.0) and np.all(got_g[~valid] == 0.0)
    if valid.any():
        U.assert_close(got_g, ref.dx, "dlogits")


@pytest.mark.parametrize("case", range(60))
def test_separate_calls_sweep(case):
    """flce_forward (with predicted tokens and accuracy in half the cases)
    then flce_backward with an upstream gradient other than 1, over the same
    kinds of random options as the fused sweep (token chunks, bf16 dW, class
    weights): every output against the oracle."""
    seed = 7000 + case
    c = draw_case(seed)
    rng = np.random.default_rng(seed + 11)
    metrics = bool(rng.random() < 0.5)
    g_out = float(rng.choice([0.5, 2.0, -1.5]))
    print(f"\n[gpu-sweep] separate calls case {case} seed {seed}: {c} metrics={metrics} g={g_out}",
          flush=True)
    inp, cw = make_inputs(c, seed)
    o = O.LossOptions(label_smoothing=c["label_smoothing"], lse_square_scale=c["lse_square_scale"],
                      softcap=c["softcap"], reduction=c["reduction"], class_weight=cw)
    dtype = c["dtype"]
    x = U.dev_tensor(inp["x"], dtype)
    w = U.dev_tensor(inp["w"], dtype)
    b = U.dev_tensor(inp["bias"], dtype) if inp["bias"] is not None else None
    t = torch.from_numpy(inp["targets"]).to("cuda")
    cwt = torch.tensor(cw, dtype=torch.float32, device="cuda") if cw is not None else None
    opts = U.lib_opts(o)
    out = api.forward(x, w, t, b, return_metrics=metrics, class_weight=cwt, **opts)
    loss, lse, row_loss = out[:3]
    go = torch.tensor([g_out], dtype=torch.float32, device="cuda")
    dx, dw, db = api.backward(x, w, t, lse, go, b, vocab_slice=c["vocab_slice"],
                              token_chunk=c["token_chunk"], dw_bf16=c["dw_bf16"], class_weight=cwt,
                              **opts)
    torch.cuda.synchronize()
    ref = O.forward_backward(inp["x"], inp["w"], inp["bias"], inp["targets"], o, grad_output=g_out)
    U.assert_loss(float(loss.item()), ref.loss)
    valid = inp["targets"] != IGN
    U.assert_lse(U.host(lse)[valid], ref.lse[valid])
    if valid.any():
        U.assert_close(U.host(dx), ref.dx, "dX")
        U.assert_close(U.host(dw), ref.dw, "dW")
        if c["bias"]:
            U.assert_close(U.host(db), ref.db, "db")
    if metrics:
        pred, acc = out[3], out[4]
        z = O.logits(O.to_f64(inp["x"]), O.to_f64(inp["w"]), O.to_f64(inp["bias"]), o.softcap)
        U.check_predictions(pred.cpu().numpy(), float(acc), z, inp["targets"], o)
