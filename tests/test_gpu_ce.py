"""Cross-entropy on given logits (flce_ce_*) against the fp64 oracle (needs an
MI355X).

Full element-by-element comparison on the small and the fp32 feature
workloads and on edge cases (every V residue of the 16-byte row split, empty
and fully ignored batches, in-place gradients); the Llama-3-8B sequence is run
at full size and checked on 256 sampled rows plus properties that hold at any
size."""
import numpy as np
import pytest
import torch

from linear_cross_entropy_bf16_amd import api, workloads as W
from linear_cross_entropy_bf16_amd._lib import FLCE_ERR_TARGET_OUT_OF_RANGE, FLCEError
from oracle import flce_oracle as O
from tests import gpu_utils as U

pytestmark = pytest.mark.gpu

IGN = -100


def banner(msg):
    print(f"\n[gpu-ce] {msg}", flush=True)


def logits_problem(n, v, dtype="bf16", ignore_frac=0.1, seed=0, spread=1.0):
    rng = np.random.default_rng(seed)
    r = rng.standard_normal((n, v), dtype=np.float32) * np.float32(spread)
    t = rng.integers(0, v, n).astype(np.int32)
    k = int(round(ignore_frac * n))
    if k:
        t[rng.choice(n, k, replace=False)] = IGN
    if dtype == "bf16":
        r = W.f32_to_bf16_bits(r)
    return dict(logits=r, targets=t)


def run_ce(inp, dtype, o, mode="fused", inplace=False):
    r = U.dev_tensor(inp["logits"], dtype)
    t = torch.from_numpy(inp["targets"]).to("cuda")
    if mode == "fused":
        loss, lse, g = api.cross_entropy_fused_fwd_bwd(r, t, inplace=inplace, **U.lib_opts(o))
        row_loss = None
    else:
        loss, lse, row_loss = api.cross_entropy_forward(r, t, check_targets=True, **U.lib_opts(o))
        g = api.cross_entropy_backward(r, t, lse, None, inplace=inplace, **U.lib_opts(o))
    torch.cuda.synchronize()
    if inplace:
        assert g.data_ptr() == r.data_ptr()
    return dict(loss=float(loss.item()), lse=U.host(lse), grad=U.host(g),
                row_loss=None if row_loss is None else U.host(row_loss))


def compare(inp, dtype, o, **kw):
    got = run_ce(inp, dtype, o, **kw)
    ref = O.cross_entropy_on_logits(inp["logits"], inp["targets"], o)
    U.assert_loss(got["loss"], ref.loss)
    U.assert_lse(got["lse"], ref.lse)
    U.assert_close(got["grad"], ref.dx, "dlogits")
    if got["row_loss"] is not None:
        assert np.abs(got["row_loss"] - ref.row_loss).max() <= 2 * U.LSE_ABS
    return got, ref


@pytest.mark.parametrize("mode", ["fused", "separate"])
@pytest.mark.parametrize("name", ["ce_logits_small", "ce_logits_features_f32"])
def test_workload_full(name, mode):
    wl = W.CE_WORKLOADS[name]
    banner(f"{wl.name} {mode}")
    inp = W.generate_logits(wl)
    compare(inp, wl.dtype, U.options(wl), mode=mode)


FEATURES = [dict(), dict(label_smoothing=0.1), dict(lse_square_scale=1e-3), dict(softcap=5.0),
            dict(label_smoothing=0.2, lse_square_scale=1e-3, softcap=3.0, reduction="sum")]


@pytest.mark.parametrize("feats", FEATURES, ids=lambda f: "-".join(f"{k}={v}" for k, v in f.items()) or "plain")
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_features(dtype, feats):
    inp = logits_problem(300, 1000, dtype, seed=3, spread=2.0)
    banner(f"features {dtype} {feats}")
    compare(inp, dtype, O.LossOptions(**feats))
    compare(inp, dtype, O.LossOptions(**feats), mode="separate")


@pytest.mark.parametrize("v", [1, 2, 3, 7, 8, 9, 15, 17, 255, 257, 1000, 4097])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_row_split_residues(dtype, v):
    """Every residue of V against the 16-byte vector: rows start misaligned by
    every possible amount, so heads, bodies and tails of all lengths occur."""
    inp = logits_problem(37, v, dtype, seed=v, ignore_frac=0.1)
    banner(f"row split {dtype} v={v}")
    compare(inp, dtype, O.LossOptions(label_smoothing=0.05, lse_square_scale=1e-3, softcap=4.0))


@pytest.mark.parametrize("mode", ["fused", "separate"])
@pytest.mark.parametrize("dtype,v", [("bf16", 256000), ("f32", 200003)])
def test_rows_longer_than_the_register_cache(dtype, v, mode):
    """Rows longer than what the fused kernel holds in registers (129024 bf16
    or 64512 fp32 entries per row): the rest of the row streams through its
    second loop in both passes; fp32 with an odd V also leaves most rows
    unaligned.  Every output against the oracle."""
    inp = logits_problem(24, v, dtype, seed=v % 101, spread=2.0)
    banner(f"long rows {dtype} v={v} {mode}")
    compare(inp, dtype, O.LossOptions(label_smoothing=0.1, lse_square_scale=1e-3, softcap=8.0), mode=mode)
    compare(inp, dtype, O.LossOptions(), mode=mode, inplace=True)


@pytest.mark.parametrize("mode", ["fused", "separate"])
def test_in_place_gradient(mode):
    inp = logits_problem(129, 999, "bf16", seed=5)
    banner(f"in place {mode}")
    compare(inp, "bf16", O.LossOptions(label_smoothing=0.1), mode=mode, inplace=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_empty_and_all_ignored(dtype):
    banner(f"empty / all ignored {dtype}")
    empty = logits_problem(0, 100, dtype)
    for red in ("mean", "sum"):
        got = run_ce(empty, dtype, O.LossOptions(reduction=red))
        assert got["loss"] == 0.0 and got["lse"].size == 0 and got["grad"].shape == (0, 100)
    ign = logits_problem(50, 333, dtype, seed=2)
    ign["targets"][:] = IGN
    for red in ("mean", "sum"):
        for mode in ("fused", "separate"):
            got = run_ce(ign, dtype, O.LossOptions(reduction=red), mode=mode)
            assert got["loss"] == 0.0
            assert np.all(got["lse"] == 0.0) and np.all(got["grad"] == 0.0)


def test_reduction_none_forward():
    inp = logits_problem(200, 777, "bf16", seed=8)
    o = O.LossOptions(reduction="none", label_smoothing=0.1)
    r = U.dev_tensor(inp["logits"], "bf16")
    t = torch.from_numpy(inp["targets"]).to("cuda")
    loss, lse, row_loss = api.cross_entropy_forward(r, t, **U.lib_opts(o))
    ref = O.cross_entropy_on_logits(inp["logits"], inp["targets"], o, want_grad=False)
    assert np.abs(U.host(loss) - ref.loss).max() <= 2 * U.LSE_ABS
    assert torch.equal(loss, row_loss)
    with pytest.raises(FLCEError):
        api.cross_entropy_fused_fwd_bwd(r, t, **U.lib_opts(o))


def test_target_out_of_range_is_reported():
    inp = logits_problem(64, 500, "bf16", seed=9, ignore_frac=0.0)
    inp["targets"][7] = 500 + 5
    inp["targets"][9] = -3
    r = U.dev_tensor(inp["logits"], "bf16")
    t = torch.from_numpy(inp["targets"]).to("cuda")
    with pytest.raises(FLCEError) as e:
        api.cross_entropy_forward(r, t, check_targets=True)
    assert e.value.status == FLCE_ERR_TARGET_OUT_OF_RANGE
    api.cross_entropy_fused_fwd_bwd(r, t)       # still no out-of-bounds access
    torch.cuda.synchronize()


def test_deterministic_bitwise():
    inp = logits_problem(256, 5000, "bf16", seed=4)
    a = run_ce(inp, "bf16", O.LossOptions(label_smoothing=0.1))
    b = run_ce(inp, "bf16", O.LossOptions(label_smoothing=0.1))
    assert a["loss"] == b["loss"]
    assert np.array_equal(a["lse"], b["lse"]) and np.array_equal(a["grad"], b["grad"])


def test_autograd_function_and_grad_output():
    inp = logits_problem(96, 640, "f32", seed=6)
    o = O.LossOptions(lse_square_scale=1e-3)
    r = U.dev_tensor(inp["logits"], "f32").requires_grad_(True)
    t = torch.from_numpy(inp["targets"]).to("cuda")
    loss = api.cross_entropy(r.view(8, 12, 640), t.view(8, 12), **U.lib_opts(o))
    (3.0 * loss).backward()
    torch.cuda.synchronize()
    ref = O.cross_entropy_on_logits(inp["logits"], inp["targets"], o, grad_output=3.0)
    U.assert_loss(float(loss.item()), ref.loss)
    loss2, lse = api.cross_entropy(r.detach(), t, return_lse=True, **U.lib_opts(o))
    assert float(loss2) == float(loss.detach()) and not lse.requires_grad
    U.assert_lse(U.host(lse), ref.lse)
    U.assert_close(U.host(r.grad), ref.dx, "dlogits via autograd")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("mode", ["fused", "separate"])
def test_llama3_seq_sampled_rows(mode):
    """Full-size 8192 x 128256 bf16 logits: 256 sampled rows of lse and
    gradient against the oracle (with the full batch's n_valid); the loss
    equals the reduction of all row losses; ignored rows are exactly 0; each
    gradient row sums to 0 without z-loss and softcap."""
    wl = W.CE_WORKLOADS["ce_logits_llama3_8b_seq"]
    banner(f"full-size {wl.name} {mode}")
    inp = W.generate_logits(wl)
    o = U.options(wl)
    r = U.dev_tensor(inp["logits"], wl.dtype)
    t = torch.from_numpy(inp["targets"]).to("cuda")
    if mode == "fused":
        loss, lse, g = api.cross_entropy_fused_fwd_bwd(r, t, **U.lib_opts(o))
    else:
        loss, lse, _ = api.cross_entropy_forward(r, t, check_targets=True, **U.lib_opts(o))
        g = api.cross_entropy_backward(r, t, lse, None, **U.lib_opts(o))
    torch.cuda.synchronize()
    valid = inp["targets"] != wl.ignore_index
    n_valid = int(valid.sum())
    rows = W.sample_rows(wl, 256)
    ref = O.cross_entropy_on_logits(inp["logits"][rows], inp["targets"][rows], o, n_valid=n_valid)
    rows_d = torch.from_numpy(rows).cuda()
    U.assert_lse(U.host(lse[rows_d]), ref.lse)
    U.assert_close(U.host(g[rows_d]), ref.dx, "dlogits rows")
    # the loss against the oracle's loss of all rows, computed block by block
    full = O.cross_entropy_on_logits(inp["logits"], inp["targets"], o, want_grad=False)
    U.assert_loss(float(loss.item()), full.loss)
    U.assert_lse(U.host(lse), full.lse)
    ign = torch.from_numpy(np.nonzero(~valid)[0]).cuda()
    assert torch.all(lse[ign] == 0) and torch.all(g[ign] == 0)
    # each row's entries sum to 0 up to the bf16 rounding of each entry
    gd = g.double()
    assert torch.all(gd.sum(dim=1).abs() <= 2.0 ** -8 * gd.abs().sum(dim=1))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("v", [1, 7, 1000, 4097])
def test_forward_metrics(dtype, v):
    inp = logits_problem(129, v, dtype, seed=v + 1, spread=2.0)
    o = O.LossOptions(softcap=5.0, label_smoothing=0.1)
    banner(f"metrics {dtype} v={v}")
    r = U.dev_tensor(inp["logits"], dtype)
    t = torch.from_numpy(inp["targets"]).to("cuda")
    loss, lse, rl, pred, acc = api.cross_entropy_forward(r, t, return_metrics=True, **U.lib_opts(o))
    loss0, lse0, rl0 = api.cross_entropy_forward(r, t, **U.lib_opts(o))
    torch.cuda.synchronize()
    assert torch.equal(lse, lse0) and torch.equal(rl, rl0) and float(loss) == float(loss0)
    z = O.to_f64(inp["logits"])
    z = o.softcap * np.tanh(z / o.softcap)
    U.check_predictions(pred.cpu().numpy(), float(acc), z, inp["targets"], o)
    # exact ties resolve to the lowest index
    r2 = torch.zeros_like(r)
    _, _, _, p2, _ = api.cross_entropy_forward(r2, t, return_metrics=True)
    valid = inp["targets"] != IGN
    assert np.all(p2.cpu().numpy()[valid] == 0)
