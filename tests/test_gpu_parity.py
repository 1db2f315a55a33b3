"""HIP path against the fp64 oracle (needs an MI355X).

Full element-by-element comparison on the tiny fp32 and small LM-head
workloads and on edge cases; the large workloads are checked on a seeded
512-row sub-batch (its own call) and on 256 sampled rows of the full-size run.
"""
import numpy as np
import pytest
import torch

from linear_cross_entropy_bf16_amd import api, workloads as W
from linear_cross_entropy_bf16_amd._lib import FLCE_ERR_TARGET_OUT_OF_RANGE, FLCEError
from oracle import flce_oracle as O
from tests import gpu_utils as U

pytestmark = pytest.mark.gpu

IGN = -100


def small_problem(n, d, v, dtype="bf16", bias=False, ignore_frac=0.1, seed=0, w_std=None):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d), dtype=np.float32)
    w = rng.standard_normal((v, d), dtype=np.float32) * np.float32(w_std or 1.0 / np.sqrt(d))
    b = (rng.standard_normal(v, dtype=np.float32) * np.float32(0.3)) if bias else None
    t = rng.integers(0, v, n).astype(np.int32)
    k = int(round(ignore_frac * n))
    if k:
        t[rng.choice(n, k, replace=False)] = IGN
    if dtype == "bf16":
        x, w = W.f32_to_bf16_bits(x), W.f32_to_bf16_bits(w)
        b = W.f32_to_bf16_bits(b) if b is not None else None
    return dict(x=x, w=w, bias=b, targets=t)


def banner(msg):
    print(f"\n[gpu] {msg}", flush=True)


# ----------------------------------------------------------------- workloads
def test_tiny_f32_full():
    wl = W.WORKLOADS["tiny_f32"]
    banner(f"{wl}")
    U.compare_full(W.generate(wl), wl.dtype, U.options(wl))


def test_small_lm_head_full():
    wl = W.WORKLOADS["small_lm_head"]
    banner(f"{wl}")
    U.compare_full(W.generate(wl), wl.dtype, U.options(wl))


LARGE = ["llama3_8b_seq", "llama3_8b_batch8", "wide_vocab_features"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", LARGE)
def test_large_subbatch(name):
    """A seeded 512-row sub-batch of the workload as its own call: every
    output compared, dW streamed by vocabulary blocks."""
    wl = W.WORKLOADS[name]
    banner(f"sub-batch of {wl}")
    full = W.generate(wl)
    rows = W.sample_rows(wl, 512, salt=1)
    inp = dict(x=full["x"][rows], w=full["w"], bias=full["bias"], targets=full["targets"][rows])
    del full
    o = U.options(wl)
    got = U.run_fused(inp, wl.dtype, o)
    ref = O.forward(inp["x"], inp["w"], inp["bias"], inp["targets"], o)
    U.assert_loss(got["loss"], ref.loss)
    U.assert_lse(got["lse"], ref.lse)
    acc = U.FrobAccumulator()
    xr = O.to_f64(inp["x"])
    wr = O.to_f64(inp["w"])
    br = O.to_f64(inp["bias"])
    z = O.logits(xr, wr, br, o.softcap)
    lse = O.log_sum_exp(z)
    g = O.grad_logits(z, lse, inp["targets"], o) * O.grad_scale(o, ref.n_valid, 1.0)
    del z
    U.assert_close(got["dx"], g @ wr, "dX")
    for v0 in range(0, wl.v, 16384):
        v1 = min(wl.v, v0 + 16384)
        acc.add(got["dw"][v0:v1], g[:, v0:v1].T @ xr)
    acc.check("dW")
    if got["db"] is not None:
        U.assert_close(got["db"], g.sum(axis=0), "db")


def oracle_forward_columns(inp, o, cols, row_block=512):
    """The oracle's forward over every row of a workload, block by block:
    LSE, row losses, and the columns ``cols`` of the final logits (enough to
    form those columns of G, hence those rows of dW and db, for the whole
    batch without the [N, V] logits).  Returns (lse, row_loss, z_cols, X fp64)."""
    xf, wf, bf = O.to_f64(inp["x"]), O.to_f64(inp["w"]), O.to_f64(inp["bias"])
    t = inp["targets"]
    n = xf.shape[0]
    valid = O.valid_rows(t, o)
    lse, rl, zc = np.zeros(n), np.zeros(n), np.empty((n, len(cols)))
    for r0 in range(0, n, row_block):
        sl = slice(r0, min(n, r0 + row_block))
        z = O.logits(xf[sl], wf, bf, o.softcap)
        l = O.log_sum_exp(z)
        rl[sl] = O.row_losses(z, l, t[sl], o)
        lse[sl] = np.where(valid[sl], l, 0.0)
        zc[sl] = z[:, cols]
    return lse, rl, zc, xf


def sampled_vocab_rows(wl, targets, count=48):
    """The 16 most frequent targets, the last vocabulary entry (ragged tail)
    and seeded uniform picks: rows of dW whose contraction over all tokens
    includes many target hits and many none."""
    valid = targets[targets >= 0]
    freq = np.bincount(valid, minlength=wl.v)
    top = np.argsort(-freq, kind="stable")[:16]
    rng = np.random.default_rng(wl.seed + 123)
    rest = rng.choice(wl.v, count - 17, replace=False)
    return np.unique(np.concatenate([top, [wl.v - 1], rest]))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", LARGE)
def test_large_sampled_rows(name):
    """Full-size forward and backward through the two separate entry points,
    against the oracle's forward over every row: the loss and every row's
    LSE; 256 sampled rows of row loss and dX; 48 sampled vocabulary rows of
    dW and db (each a contraction over all N tokens: the most frequent
    targets, the last entry, random picks); ignored rows exactly zero; the
    column sums of dW within G's bf16 rounding (no z-loss, no softcap)."""
    wl = W.WORKLOADS[name]
    banner(f"full-size {wl}")
    inp = W.generate(wl)
    o = U.options(wl)
    x = U.dev_tensor(inp["x"], wl.dtype)
    w = U.dev_tensor(inp["w"], wl.dtype)
    b = U.dev_tensor(inp["bias"], wl.dtype) if inp["bias"] is not None else None
    t = torch.from_numpy(inp["targets"]).to("cuda")
    loss, lse, row_loss = api.forward(x, w, t, b, check_targets=True, **U.lib_opts(o))
    dx, dw, db = api.backward(x, w, t, lse, None, b, **U.lib_opts(o))
    torch.cuda.synchronize()
    valid = inp["targets"] != wl.ignore_index
    n_valid = int(valid.sum())
    cols = sampled_vocab_rows(wl, inp["targets"])
    banner(f"oracle forward over all {wl.n} rows")
    lse_ref, rl_ref, zc, xf = oracle_forward_columns(inp, o, cols)
    U.assert_loss(float(loss.item()), O.reduce_loss(rl_ref, n_valid, o))
    U.assert_lse(U.host(lse), lse_ref)
    rows = W.sample_rows(wl, 256)
    ref = O.forward_backward(inp["x"][rows], inp["w"], inp["bias"], inp["targets"][rows], o,
                             n_valid=n_valid, want_dw=False)
    rows_d = torch.from_numpy(rows).cuda()
    rl = U.host(row_loss)
    assert np.abs(rl[rows] - ref.row_loss).max() <= U.LSE_ABS * 2
    U.assert_close(U.host(dx[rows_d]), ref.dx, "dX rows")
    # vocabulary rows of dW and db: contractions over every token
    scale = O.grad_scale(o, n_valid, 1.0)
    g_cols = O.grad_logits_columns(zc, cols, wl.v, lse_ref, inp["targets"], o) * scale
    cols_d = torch.from_numpy(cols).cuda()
    U.assert_close(U.host(dw[cols_d]), g_cols.T @ xf, "dW sampled vocabulary rows")
    if db is not None:
        U.assert_close(U.host(db[cols_d]), g_cols.sum(axis=0), "db sampled vocabulary rows")
    del zc, g_cols
    # ignored rows: exactly zero
    ign = ~valid
    if ign.any():
        it = torch.from_numpy(np.nonzero(ign)[0]).cuda()
        assert torch.all(lse[it] == 0) and torch.all(row_loss[it] == 0)
        assert torch.all(dx[it] == 0)
    if wl.lse_square_scale == 0 and wl.softcap == 0:
        U.assert_dw_column_sums(dw, xf[valid], scale)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("bias", [False, True])
def test_llama3_seq_full_against_oracle(bias):
    """8192 x 4096 x 128256 (the per-GPU share of the headline batch under
    8-way data parallelism) through the fused call: loss, LSE, dX and the
    whole dW (the contraction over all tokens) element by element against
    the oracle; with a bias N(0, 0.02^2) also db."""
    wl = W.WORKLOADS["llama3_8b_seq"]
    banner(f"{wl} in full, bias={bias}")
    inp = W.generate(wl)
    if bias:
        b = np.random.default_rng(wl.seed + 7).standard_normal(wl.v).astype(np.float32) * np.float32(0.02)
        inp["bias"] = W.f32_to_bf16_bits(b)
    U.compare_full(inp, wl.dtype, U.options(wl))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_vocab_with_multi_tile_chunks(dtype):
    """Enough tiles for four vocabulary tiles per forward workgroup (bf16; the
    fp32 register-staged path at this size runs two), and V not a multiple of
    256: the whole tiles and the partial last tile come from two launches
    whose partials are merged.  256 sampled rows of LSE, row loss and dX
    against the oracle; bias, softcap and label smoothing on."""
    n, d, v = (16384, 256, 65535) if dtype == "bf16" else (8192, 64, 65537)
    banner(f"ragged vocabulary, multi-tile chunks {dtype} n={n} d={d} v={v}")
    inp = small_problem(n, d, v, dtype, bias=True, seed=11)
    o = O.LossOptions(IGN, 0.1, 1e-4, 20.0, "mean")
    x, w = U.dev_tensor(inp["x"], dtype), U.dev_tensor(inp["w"], dtype)
    b = U.dev_tensor(inp["bias"], dtype)
    t = torch.from_numpy(inp["targets"]).to("cuda")
    loss, lse, row_loss = api.forward(x, w, t, b, check_targets=True, **U.lib_opts(o))
    dx, dw, db = api.backward(x, w, t, lse, None, b, **U.lib_opts(o))
    torch.cuda.synchronize()
    rows = np.random.default_rng(5).choice(n, 256, replace=False)
    rows.sort()
    n_valid = int((inp["targets"] != IGN).sum())
    ref = O.forward_backward(inp["x"][rows], inp["w"], inp["bias"], inp["targets"][rows], o,
                             n_valid=n_valid, want_dw=False)
    rows_d = torch.from_numpy(rows).cuda()
    U.assert_lse(U.host(lse[rows_d]), ref.lse)
    rl = U.host(row_loss)
    assert np.abs(rl[rows] - ref.row_loss).max() <= U.LSE_ABS * 2
    U.assert_close(U.host(dx[rows_d]), ref.dx, "dX rows")
    U.assert_loss(float(loss.item()), rl.sum() / n_valid, "loss vs its row losses")


# ----------------------------------------------------------------- features
FEATURES = [
    dict(),
    dict(label_smoothing=0.1),
    dict(lse_square_scale=1e-3),
    dict(softcap=2.0),
    dict(reduction="sum"),
    dict(label_smoothing=0.2, lse_square_scale=1e-2, softcap=1.5, reduction="sum"),
]


@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("feats", FEATURES, ids=lambda f: "-".join(f"{k}={v}" for k, v in f.items()) or "plain")
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_features(dtype, feats, bias):
    inp = small_problem(300, 136, 1000, dtype, bias=bias, seed=3, w_std=0.3)
    banner(f"features {dtype} {feats} bias={bias}")
    U.compare_full(inp, dtype, O.LossOptions(**feats))


@pytest.mark.parametrize("n,d,v,slice_", [
    (1, 8, 1, 0), (2, 8, 2, 0), (257, 264, 257, 0), (300, 72, 1000, 256), (513, 200, 1000, 512),
    (64, 1024, 3000, 1024), (1000, 64, 33, 0), (256, 256, 256, 0), (255, 8, 4097, 1024),
])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_shapes(dtype, n, d, v, slice_):
    """Tails in every dimension, several vocabulary slices with a ragged last
    slice, K not a multiple of the 64-wide slab, single-class and two-class
    vocabularies."""
    inp = small_problem(n, d, v, dtype, bias=True, seed=n + d + v)
    banner(f"ragged {dtype} n={n} d={d} v={v} slice={slice_}")
    U.compare_full(inp, dtype, O.LossOptions(label_smoothing=0.05, lse_square_scale=1e-3),
                   vocab_slice=slice_)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("n,d,v", [(40, 1 << 20, 300), (1 << 22, 8, 20)])
def test_maximum_sizes(n, d, v):
    """The largest hidden size and batch the library accepts (D = 2^20: the
    K-major row offsets of a tile reach 2^29 bytes; N = 2^22: the largest
    packed-row and token-tile counts), with small other dimensions so the
    oracle stays quick: loss, LSE, dX and dW against the oracle (sampled rows
    for N = 2^22)."""
    banner(f"maximum sizes n={n} d={d} v={v}")
    inp = small_problem(n, d, v, "bf16", bias=True, seed=n % 97 + d % 89, ignore_frac=0.1)
    o = O.LossOptions(label_smoothing=0.1, lse_square_scale=1e-3)
    if n <= 4096:
        U.compare_full(inp, "bf16", o)
        return
    x = U.dev_tensor(inp["x"], "bf16")
    w = U.dev_tensor(inp["w"], "bf16")
    b = U.dev_tensor(inp["bias"], "bf16")
    t = torch.from_numpy(inp["targets"]).to("cuda")
    loss, lse, dx, dw, db = api.fused_fwd_bwd(x, w, t, b, **U.lib_opts(o))
    torch.cuda.synchronize()
    ref = O.forward_backward(inp["x"], inp["w"], inp["bias"], inp["targets"], o)
    U.assert_loss(float(loss), ref.loss)
    rows = np.random.default_rng(1).choice(n, 4096, replace=False)
    rows_d = torch.from_numpy(rows).cuda()
    U.assert_lse(U.host(lse[rows_d]), ref.lse[rows])
    U.assert_close(U.host(dx[rows_d]), ref.dx[rows], "dX rows")
    U.assert_close(U.host(dw), ref.dw, "dW")
    U.assert_close(U.host(db), ref.db, "db")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_empty_batch(dtype):
    inp = small_problem(0, 64, 100, dtype, bias=True)
    for red in ("mean", "sum"):
        got = U.run_fused(inp, dtype, O.LossOptions(reduction=red))
        assert got["loss"] == 0.0 and got["lse"].size == 0 and got["dx"].shape == (0, 64)
        assert np.all(got["dw"] == 0) and np.all(got["db"] == 0)


@pytest.mark.parametrize("red", ["mean", "sum"])
def test_all_rows_ignored(red):
    inp = small_problem(100, 64, 500, "bf16", bias=True, ignore_frac=1.0)
    got = U.run_fused(inp, "bf16", O.LossOptions(reduction=red))
    assert got["loss"] == 0.0
    assert np.all(got["lse"] == 0) and np.all(got["dx"] == 0)
    assert np.all(got["dw"] == 0) and np.all(got["db"] == 0)


def test_ignore_index_inside_vocabulary():
    inp = small_problem(200, 64, 500, "bf16", ignore_frac=0.0, seed=5)
    inp["targets"][::7] = 3
    U.compare_full(inp, "bf16", O.LossOptions(ignore_index=3))


def test_reduction_none_forward():
    inp = small_problem(300, 64, 700, "bf16", seed=6)
    x, w = U.dev_tensor(inp["x"], "bf16"), U.dev_tensor(inp["w"], "bf16")
    t = torch.from_numpy(inp["targets"]).cuda()
    loss, lse, row_loss = api.forward(x, w, t, reduction="none", label_smoothing=0.1)
    ref = O.forward(inp["x"], inp["w"], None, inp["targets"],
                    O.LossOptions(reduction="none", label_smoothing=0.1))
    assert np.abs(U.host(loss) - ref.loss).max() <= U.LSE_ABS
    assert np.array_equal(U.host(loss), U.host(row_loss))
    with pytest.raises(FLCEError):
        api.backward(x, w, t, lse, reduction="none")


def test_target_out_of_range_is_reported():
    inp = small_problem(100, 64, 500, "bf16", seed=7)
    inp["targets"][10] = 500
    x, w = U.dev_tensor(inp["x"], "bf16"), U.dev_tensor(inp["w"], "bf16")
    t = torch.from_numpy(inp["targets"]).cuda()
    with pytest.raises(FLCEError) as e:
        api.forward(x, w, t, check_targets=True)
    assert e.value.status == FLCE_ERR_TARGET_OUT_OF_RANGE
    inp["targets"][10] = -7
    with pytest.raises(FLCEError):
        api.forward(x, w, torch.from_numpy(inp["targets"]).cuda(), check_targets=True)
    inp["targets"][10] = 499
    api.forward(x, w, torch.from_numpy(inp["targets"]).cuda(), check_targets=True)


# ----------------------------------------------------------------- API layers
def test_deterministic_bitwise():
    inp = small_problem(700, 264, 3000, "bf16", bias=True, seed=8)
    o = O.LossOptions(label_smoothing=0.1, softcap=5.0)
    a = U.run_fused(inp, "bf16", o, vocab_slice=1024)
    b = U.run_fused(inp, "bf16", o, vocab_slice=1024)
    for k in ("lse", "dx", "dw", "db"):
        assert np.array_equal(a[k], b[k]), k
    assert a["loss"] == b["loss"]


def test_repeat_calls_bitwise_with_work_queues():
    """The forward, G and dX launches hand their tiles out through per-XCD
    work counters (which workgroup computes which tile changes from run to
    run); the results must not.  A shape with thousands of forward items and
    G tiles per slice, so the queues' tails are in use, called three times."""
    inp = small_problem(12000, 512, 40000, "bf16", bias=True, seed=21)
    o = O.LossOptions(label_smoothing=0.05, lse_square_scale=1e-4)
    runs = [U.run_fused(inp, "bf16", o) for _ in range(3)]
    for r in runs[1:]:
        assert r["loss"] == runs[0]["loss"]
        for k in ("lse", "dx", "dw", "db"):
            assert np.array_equal(r[k], runs[0][k]), k


def test_fused_equals_separate_calls():
    inp = small_problem(500, 128, 2000, "bf16", bias=True, seed=9)
    o = O.LossOptions(label_smoothing=0.1, lse_square_scale=1e-3)
    a = U.run_fused(inp, "bf16", o, vocab_slice=768)
    x, w = U.dev_tensor(inp["x"], "bf16"), U.dev_tensor(inp["w"], "bf16")
    b_ = U.dev_tensor(inp["bias"], "bf16")
    t = torch.from_numpy(inp["targets"]).cuda()
    loss, lse, _ = api.forward(x, w, t, b_, vocab_slice=768, **U.lib_opts(o))
    dx, dw, db = api.backward(x, w, t, lse, None, b_, vocab_slice=768, **U.lib_opts(o))
    assert a["loss"] == float(loss.item())
    assert np.array_equal(a["dx"], U.host(dx)) and np.array_equal(a["dw"], U.host(dw))
    assert np.array_equal(a["db"], U.host(db))


def test_fused_call_checks_caller_buffers():
    """Preallocated outputs and workspace that do not match the call are
    refused before the library runs; matching ones are written in place."""
    inp = small_problem(300, 64, 700, "bf16", bias=True, seed=12)
    x, w = U.dev_tensor(inp["x"], "bf16"), U.dev_tensor(inp["w"], "bf16")
    b = U.dev_tensor(inp["bias"], "bf16")
    t = torch.from_numpy(inp["targets"]).cuda()
    f32 = dict(dtype=torch.float32, device="cuda")
    good = (torch.empty(1, **f32), torch.empty(300, **f32),
            torch.empty((300, 64), dtype=torch.bfloat16, device="cuda"),
            torch.empty((700, 64), **f32), torch.empty(700, **f32))
    loss, lse, dx, dw, db = api.fused_fwd_bwd(x, w, t, b, out=good)
    assert dx.data_ptr() == good[2].data_ptr() and dw.data_ptr() == good[3].data_ptr()
    ref = U.run_fused(inp, "bf16", O.LossOptions())
    assert np.array_equal(U.host(dw), ref["dw"]) and float(loss) == ref["loss"]
    for i, bad in ((2, torch.empty((299, 64), dtype=torch.bfloat16, device="cuda")),
                   (3, torch.empty((700, 64), dtype=torch.bfloat16, device="cuda")),
                   (1, torch.empty(300, dtype=torch.float16, device="cuda")),
                   (4, torch.empty(699, **f32))):
        out = list(good)
        out[i] = bad
        with pytest.raises(ValueError):
            api.fused_fwd_bwd(x, w, t, b, out=tuple(out))
    with pytest.raises(ValueError):
        api.fused_fwd_bwd(x, w, t, b, workspace=torch.empty(1 << 20, dtype=torch.float32, device="cuda"))


def test_autograd_function_and_grad_output():
    """Not-last-layer use: the loss is scaled before backward, so the upstream
    gradient reaches the library as a device scalar."""
    inp = small_problem(256, 128, 1500, "bf16", bias=True, seed=10)
    x = U.dev_tensor(inp["x"], "bf16").requires_grad_(True)
    w = U.dev_tensor(inp["w"], "bf16").requires_grad_(True)
    b = U.dev_tensor(inp["bias"], "bf16").requires_grad_(True)
    t = torch.from_numpy(inp["targets"]).cuda()
    loss, lse = api.linear_cross_entropy(x, w, t, b, label_smoothing=0.1, return_lse=True)
    assert not lse.requires_grad
    (2.5 * loss).backward()
    o = O.LossOptions(label_smoothing=0.1)
    ref = O.forward_backward(inp["x"], inp["w"], inp["bias"], inp["targets"], o, grad_output=2.5)
    U.assert_loss(float(loss.item()), ref.loss)
    U.assert_lse(U.host(lse), ref.lse)
    U.assert_close(U.host(x.grad), ref.dx, "dX")
    U.assert_close(U.host(w.grad), ref.dw, "dW")
    U.assert_close(U.host(b.grad), ref.db, "db")


@pytest.mark.parametrize("stored", [False, True])
def test_class_weights_with_zeros(stored):
    """Class weights that are 0 for half the vocabulary (rows whose target
    has weight 0 add nothing), and all 0: then the weighted mean divides by
    0, which gives loss 0 and zero gradients, as with no valid row."""
    n, d, v = 400, 72, 900
    inp = small_problem(n, d, v, "bf16", bias=True, seed=31)
    x = U.dev_tensor(inp["x"], "bf16")
    w = U.dev_tensor(inp["w"], "bf16")
    b = U.dev_tensor(inp["bias"], "bf16")
    t = torch.from_numpy(inp["targets"]).to("cuda")
    kw = dict(stored_logits=True, token_chunk=256) if stored else dict(vocab_slice=256)
    half = np.where(np.arange(v) % 2 == 0, 0.0, 1.5)
    for cw in (half, np.zeros(v)):
        o = O.LossOptions(label_smoothing=0.1, class_weight=cw)
        banner(f"class weights with zeros stored={stored} all_zero={not cw.any()}")
        loss, lse, dx, dw, db = api.fused_fwd_bwd(x, w, t, b, class_weight=torch.tensor(cw, device="cuda"),
                                                  **U.lib_opts(o), **kw)
        torch.cuda.synchronize()
        ref = O.forward_backward(inp["x"], inp["w"], inp["bias"], inp["targets"], o)
        U.assert_lse(U.host(lse), ref.lse)
        if cw.any():
            U.assert_loss(float(loss.item()), ref.loss)
            U.assert_close(U.host(dx), ref.dx, "dX")
            U.assert_close(U.host(dw), ref.dw, "dW")
            U.assert_close(U.host(db), ref.db, "db")
        else:
            assert ref.loss == 0.0 and float(loss.item()) == 0.0
            assert torch.all(dx == 0) and torch.all(dw == 0) and torch.all(db == 0)


def test_loss_module_on_an_lm_head():
    """The module form on an nn.Linear head: [B, T, D] hidden states, the
    head's weight and bias, class weights held as a buffer, gradients through
    autograd into the head's parameters."""
    inp = small_problem(2 * 150, 96, 700, "bf16", bias=True, seed=21)
    cw = np.random.default_rng(2).uniform(0.5, 2.0, 700)
    head = torch.nn.Linear(96, 700, bias=True).to(device="cuda", dtype=torch.bfloat16)
    with torch.no_grad():
        head.weight.copy_(U.dev_tensor(inp["w"], "bf16"))
        head.bias.copy_(U.dev_tensor(inp["bias"], "bf16"))
    crit = api.LinearCrossEntropyLoss(label_smoothing=0.1, softcap=15.0,
                                      class_weight=torch.tensor(cw, dtype=torch.float32)).cuda()
    x = U.dev_tensor(inp["x"], "bf16").view(2, 150, 96).requires_grad_(True)
    t = torch.from_numpy(inp["targets"]).cuda().view(2, 150)
    loss = crit(x, head.weight, t, head.bias)
    loss.backward()
    o = O.LossOptions(label_smoothing=0.1, softcap=15.0, class_weight=cw)
    ref = O.forward_backward(inp["x"], inp["w"], inp["bias"], inp["targets"], o)
    U.assert_loss(float(loss.item()), ref.loss)
    U.assert_close(U.host(x.grad).reshape(300, 96), ref.dx, "dX")
    U.assert_close(U.host(head.weight.grad), ref.dw, "dW")
    U.assert_close(U.host(head.bias.grad), ref.db, "db")


def test_noncontiguous_and_batched_inputs():
    inp = small_problem(240, 64, 800, "bf16", seed=11)
    ref = O.forward(inp["x"], inp["w"], None, inp["targets"], O.LossOptions())
    x = U.dev_tensor(inp["x"], "bf16")
    w = U.dev_tensor(inp["w"], "bf16")
    t = torch.from_numpy(inp["targets"]).cuda()
    wide = torch.zeros((240, 128), dtype=torch.bfloat16, device="cuda")
    wide[:, 32:96] = x
    xs = wide[:, 32:96]                         # rows strided by 128 elements
    assert not xs.is_contiguous()
    U.assert_loss(float(api.linear_cross_entropy(xs, w, t).item()), ref.loss, "strided x")
    wt = w.t().contiguous().t()                 # column-major weight
    assert not wt.is_contiguous()
    U.assert_loss(float(api.linear_cross_entropy(x, wt, t).item()), ref.loss, "column-major W")
    loss3 = api.linear_cross_entropy(x.reshape(4, 60, 64), w, t.reshape(4, 60).long())
    U.assert_loss(float(loss3.item()), ref.loss, "batched x")


# ------------------------------------------------- predicted tokens, accuracy

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n,d,v,feats", [
    (300, 136, 1000, dict()), (513, 64, 4097, dict(softcap=3.0, label_smoothing=0.1)),
    (257, 264, 257, dict(lse_square_scale=1e-3)), (64, 1024, 3000, dict(softcap=30.0)),
])
def test_forward_metrics(dtype, n, d, v, feats):
    """Predicted tokens and token accuracy from the forward epilogue: equal
    to the fp64 argmax except at near-ties, -1 on ignored rows, accuracy the
    hit rate; the loss and lse equal the plain forward's bit for bit."""
    inp = small_problem(n, d, v, dtype, bias=True, seed=n + v, w_std=0.5)
    o = O.LossOptions(**feats)
    banner(f"metrics {dtype} n={n} d={d} v={v} {feats}")
    x = U.dev_tensor(inp["x"], dtype)
    w = U.dev_tensor(inp["w"], dtype)
    b = U.dev_tensor(inp["bias"], dtype)
    t = torch.from_numpy(inp["targets"]).to("cuda")
    loss, lse, rl, pred, acc = api.forward(x, w, t, b, return_metrics=True, **U.lib_opts(o))
    loss0, lse0, rl0 = api.forward(x, w, t, b, **U.lib_opts(o))
    torch.cuda.synchronize()
    assert torch.equal(lse, lse0) and torch.equal(rl, rl0) and float(loss) == float(loss0)
    z = O.logits(O.to_f64(inp["x"]), O.to_f64(inp["w"]), O.to_f64(inp["bias"]), o.softcap)
    U.check_predictions(pred.cpu().numpy(), float(acc), z, inp["targets"], o)


def test_forward_metrics_exact_ties():
    """Equal logits resolve to the lowest index, also across vocabulary tiles
    and chunks: W = 0 predicts 0 everywhere; a row of W duplicated at a higher
    index (another tile) and made the largest predicts the lower copy."""
    n, d, v = 200, 64, 2000
    inp = small_problem(n, d, v, "bf16", seed=7)
    x = U.dev_tensor(inp["x"], "bf16")
    t = torch.from_numpy(inp["targets"]).to("cuda")
    w0 = torch.zeros((v, d), dtype=torch.bfloat16, device="cuda")
    _, _, _, pred, acc = api.forward(x, w0, t, None, return_metrics=True)
    valid = inp["targets"] != IGN
    p = pred.cpu().numpy()
    assert np.all(p[valid] == 0) and np.all(p[~valid] == -1)
    assert abs(float(acc) - ((inp["targets"] == 0) & valid).sum() / valid.sum()) <= 1e-6
    wd = U.dev_tensor(inp["w"], "bf16").clone()
    wd[300] = U.dev_tensor(inp["x"], "bf16")[0] * 4      # row 0's best class by far
    wd[1700] = wd[300]                                  # a tied copy in a later tile
    _, _, _, pred, _ = api.forward(x, wd, t, None, return_metrics=True)
    p = pred.cpu().numpy()
    assert not np.any(p == 1700)                        # always tied with 300, never chosen
    if valid[0]:
        assert p[0] == 300


@pytest.mark.timeout(900)
def test_forward_metrics_full_size():
    """8192 x 4096 x 128256 (one data-parallel share of the headline batch):
    the predicted token of every row against the argmax of the fp64 logits
    (a row may differ only inside the fp32 near-tie window, and only on
    0.1% of the rows), ignored rows -1 everywhere, the accuracy equal to the
    hits of the whole returned prediction array and to the oracle's up to
    those rows, and the forward's other outputs unchanged by the metrics."""
    wl = W.WORKLOADS["llama3_8b_seq"]
    banner(f"forward metrics {wl}")
    inp = W.generate(wl)
    inp["targets"][::17] = IGN                        # some ignored rows as well
    o = U.options(wl)
    x = U.dev_tensor(inp["x"], wl.dtype)
    w = U.dev_tensor(inp["w"], wl.dtype)
    t = torch.from_numpy(inp["targets"]).to("cuda")
    loss, lse, rl, pred, acc = api.forward(x, w, t, None, return_metrics=True, **U.lib_opts(o))
    loss0, lse0, rl0 = api.forward(x, w, t, None, **U.lib_opts(o))
    torch.cuda.synchronize()
    assert torch.equal(lse, lse0) and torch.equal(rl, rl0) and float(loss) == float(loss0)
    p = pred.cpu().numpy()
    valid = inp["targets"] != IGN
    assert np.all(p[~valid] == -1) and np.all((p[valid] >= 0) & (p[valid] < wl.v))
    hits = int(((p == inp["targets"]) & valid).sum())
    assert abs(float(acc) - hits / int(valid.sum())) <= 1e-6
    ref, gap, zabs = U.fp64_argmax_gaps(inp["x"], inp["w"], None, o.softcap, p)
    differ = U.check_prediction_gaps(p, float(acc), ref, gap, U.tie_window(zabs, o.softcap),
                                     inp["targets"], o)
    banner(f"{differ} of {int(valid.sum())} rows differ from the fp64 argmax (near-ties)")


# ------------------------------------------------- token chunks, bf16 dW

def _fused_opts(inp, dtype, o, to_host=True, **kw):
    x = U.dev_tensor(inp["x"], dtype)
    w = U.dev_tensor(inp["w"], dtype)
    b = U.dev_tensor(inp["bias"], dtype) if inp.get("bias") is not None else None
    t = torch.from_numpy(inp["targets"]).to("cuda")
    loss, lse, dx, dw, db = api.fused_fwd_bwd(x, w, t, b, **U.lib_opts(o), **kw)
    torch.cuda.synchronize()
    out = dict(loss=float(loss.item()), lse=U.host(lse), dx_raw=dx, dw_raw=dw)
    if to_host:
        out.update(dx=U.host(dx), dw=U.host(dw), db=None if db is None else U.host(db))
    return out


@pytest.mark.parametrize("dw_bf16", [False, True])
@pytest.mark.parametrize("n,chunk,ignore", [(1000, 256, 0.1), (1000, 512, 0.0), (700, 256, 0.6),
                                            (300, 1024, 0.1)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_token_chunks(dtype, n, chunk, ignore, dw_bf16):
    """The backward over chunks of packed rows (the last one ragged; with 60%
    ignored rows the later chunks start past n_valid and hold nothing), dW and
    db accumulated over the chunks, dW optionally bf16: every output against
    the oracle; dX bit for bit equal to the single-pass schedule."""
    inp = small_problem(n, 136, 1000, dtype, bias=True, ignore_frac=ignore, seed=n + chunk)
    o = O.LossOptions(label_smoothing=0.05, lse_square_scale=1e-3)
    banner(f"token chunks {dtype} n={n} chunk={chunk} ignore={ignore} dw_bf16={dw_bf16}")
    got = _fused_opts(inp, dtype, o, token_chunk=chunk, dw_bf16=dw_bf16, vocab_slice=256)
    assert got["dw_raw"].dtype == (torch.bfloat16 if dw_bf16 else torch.float32)
    U.compare_full(inp, dtype, o, got=got)
    one = _fused_opts(inp, dtype, o, vocab_slice=256)
    assert torch.equal(got["dx_raw"], one["dx_raw"])
    assert got["loss"] == one["loss"] and np.array_equal(got["lse"], one["lse"])


@pytest.mark.timeout(600)
def test_token_chunks_llama3_seq():
    """One Llama-3-8B sequence (8192 x 4096 x 128256) in chunks of 2048 with
    bf16 dW against the single-pass fp32 run: same loss and dX bit for bit,
    dW within bf16 rounding."""
    wl = W.WORKLOADS["llama3_8b_seq"]
    banner(f"token chunks {wl}")
    inp = W.generate(wl)
    o = U.options(wl)
    a = _fused_opts(inp, wl.dtype, o, to_host=False, token_chunk=2048, dw_bf16=True)
    b = _fused_opts(inp, wl.dtype, o, to_host=False)
    assert a["loss"] == b["loss"] and torch.equal(a["dx_raw"], b["dx_raw"])
    dwa, dwb = a["dw_raw"].double(), b["dw_raw"].double()
    rel = (torch.linalg.norm(dwa - dwb) / torch.linalg.norm(dwb)).item()
    assert rel <= 4e-3, rel


# ------------------------------------------------- stored-logits schedule

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n,d,v,chunk,feats", [
    (1000, 136, 1000, 256, dict(label_smoothing=0.05, lse_square_scale=1e-3)),
    (700, 64, 4097, 512, dict(softcap=3.0)),
    (300, 264, 257, 0, dict(label_smoothing=0.1, reduction="sum")),
    (1, 8, 1, 0, dict()),
])
def test_stored_logits(dtype, n, d, v, chunk, feats):
    """Three contractions (logits kept per token chunk): every output against
    the oracle; loss and lse bit for bit those of the recompute schedule (the
    forward is the same)."""
    inp = small_problem(n, d, v, dtype, bias=True, seed=n + v + 1)
    o = O.LossOptions(**feats)
    banner(f"stored logits {dtype} n={n} d={d} v={v} chunk={chunk} {feats}")
    got = _fused_opts(inp, dtype, o, stored_logits=True, token_chunk=chunk)
    U.compare_full(inp, dtype, o, got=got)
    ref = _fused_opts(inp, dtype, o)
    assert got["loss"] == ref["loss"] and np.array_equal(got["lse"], ref["lse"])


def test_stored_logits_empty_and_ignored():
    for n in (0, 40):
        inp = small_problem(n, 64, 300, "bf16", bias=True, seed=5)
        inp["targets"][:] = IGN
        got = _fused_opts(inp, "bf16", O.LossOptions(), stored_logits=True)
        assert got["loss"] == 0.0
        assert np.all(got["dx"] == 0) and np.all(got["dw"] == 0) and np.all(got["db"] == 0)


@pytest.mark.timeout(600)
def test_stored_logits_llama3_seq():
    """One Llama-3-8B sequence: the stored-logits schedule (chunks of 4096, so
    dW accumulates) against the recompute schedule; G is the same bf16 tensor
    in both, so dX and dW differ only by fp32 summation order."""
    wl = W.WORKLOADS["llama3_8b_seq"]
    banner(f"stored logits {wl}")
    inp = W.generate(wl)
    o = U.options(wl)
    a = _fused_opts(inp, wl.dtype, o, to_host=False, stored_logits=True, token_chunk=4096)
    b = _fused_opts(inp, wl.dtype, o, to_host=False)
    assert a["loss"] == b["loss"] and np.array_equal(a["lse"], b["lse"])
    # dX leaves in bf16, where an fp32 difference in the last bits can flip an
    # element by one bf16 ulp (2^-8): a looser bound than for the fp32 dW
    for k, bound in (("dx_raw", 1e-3), ("dw_raw", 1e-4)):
        x1, x2 = a[k].double(), b[k].double()
        rel = (torch.linalg.norm(x1 - x2) / torch.linalg.norm(x2)).item()
        assert rel <= bound, (k, rel)


@pytest.mark.timeout(900)
def test_headline_schedules_sampled_rows():
    """65536 x 4096 x 128256, the benchmark's shape, through the two other
    schedules the benchmark times: the stored-logits schedule against the
    oracle on 256 sampled rows (lse, row-wise dX, with the full batch's
    n_valid) plus the column sums of dW; the chunked backward with bf16 dW
    against the single-pass schedule (dX bit for bit, dW within bf16
    rounding)."""
    wl = W.WORKLOADS["llama3_8b_batch8"]
    banner(f"headline schedules {wl}")
    inp = W.generate(wl)
    o = U.options(wl)
    x = U.dev_tensor(inp["x"], wl.dtype)
    w = U.dev_tensor(inp["w"], wl.dtype)
    t = torch.from_numpy(inp["targets"]).to("cuda")
    loss, lse, dx, dw, _ = api.fused_fwd_bwd(x, w, t, None, stored_logits=True, **U.lib_opts(o))
    torch.cuda.synchronize()
    valid = inp["targets"] != wl.ignore_index
    n_valid = int(valid.sum())
    rows = W.sample_rows(wl, 256, salt=3)
    ref = O.forward_backward(inp["x"][rows], inp["w"], None, inp["targets"][rows], o,
                             n_valid=n_valid, want_dw=False)
    rows_d = torch.from_numpy(rows).cuda()
    U.assert_lse(U.host(lse[rows_d]), ref.lse)
    U.assert_close(U.host(dx[rows_d]), ref.dx, "stored: dX rows")
    U.assert_dw_column_sums(dw, O.to_f64(inp["x"])[valid], O.grad_scale(o, n_valid, 1.0),
                            "stored: dW column sums")
    del dw
    # chunked backward with bf16 dW against the single pass
    loss1, lse1, dx1, dw1, _ = api.fused_fwd_bwd(x, w, t, None, **U.lib_opts(o))
    loss2, lse2, dx2, dw2, _ = api.fused_fwd_bwd(x, w, t, None, token_chunk=16384, dw_bf16=True,
                                                 **U.lib_opts(o))
    torch.cuda.synchronize()
    assert float(loss1) == float(loss2) == float(loss) and torch.equal(lse1, lse2)
    assert torch.equal(lse1, lse)
    assert torch.equal(dx1, dx2)
    rel = (torch.linalg.norm(dw2.double() - dw1.double()) / torch.linalg.norm(dw1.double())).item()
    assert rel <= 4e-3, rel


@pytest.mark.timeout(900)
def test_wide_vocab_stored_sampled_rows():
    """16384 x 8192 x 256000 with bias, softcap, smoothing, z-loss, sum and
    25% ignored rows through the stored-logits schedule (two 8192-row chunks
    of fp32 logits): the loss and LSE against the recompute schedule, 256
    sampled rows of LSE and dX against the oracle, ignored rows exactly zero,
    and db equal to the recompute schedule's (the same bf16 G summed over two
    chunks instead of one; the recompute schedule's db is compared with the
    oracle on sampled vocabulary rows in test_large_sampled_rows)."""
    wl = W.WORKLOADS["wide_vocab_features"]
    banner(f"stored schedule {wl}")
    inp = W.generate(wl)
    o = U.options(wl)
    x = U.dev_tensor(inp["x"], wl.dtype)
    w = U.dev_tensor(inp["w"], wl.dtype)
    b = U.dev_tensor(inp["bias"], wl.dtype)
    t = torch.from_numpy(inp["targets"]).to("cuda")
    loss, lse, dx, dw, db = api.fused_fwd_bwd(x, w, t, b, stored_logits=True, **U.lib_opts(o))
    torch.cuda.synchronize()
    del dw
    loss_r, lse_r, _ = api.forward(x, w, t, b, **U.lib_opts(o))
    _, dw_r, db_r = api.backward(x, w, t, lse_r, None, b, **U.lib_opts(o))
    torch.cuda.synchronize()
    del dw_r
    assert torch.equal(lse, lse_r)
    U.assert_loss(float(loss), float(loss_r), "stored vs recompute loss")
    rel = (torch.linalg.norm(db.double() - db_r.double()) / torch.linalg.norm(db_r.double())).item()
    assert rel <= 1e-5, f"db: stored vs recompute rel err {rel:.3e}"
    valid = inp["targets"] != wl.ignore_index
    rows = W.sample_rows(wl, 256, salt=5)
    ref = O.forward_backward(inp["x"][rows], inp["w"], inp["bias"], inp["targets"][rows], o,
                             n_valid=int(valid.sum()), want_dw=False)
    rows_d = torch.from_numpy(rows).cuda()
    U.assert_lse(U.host(lse[rows_d]), ref.lse)
    U.assert_close(U.host(dx[rows_d]), ref.dx, "stored: dX rows")
    ign = torch.from_numpy(np.nonzero(~valid)[0]).cuda()
    assert torch.all(lse[ign] == 0) and torch.all(dx[ign] == 0)


# ------------------------------------------------- class weights

@pytest.mark.parametrize("stored", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("feats", [dict(), dict(label_smoothing=0.1), dict(lse_square_scale=1e-3, softcap=5.0),
                                   dict(label_smoothing=0.2, lse_square_scale=1e-3, softcap=3.0,
                                        reduction="sum")],
                         ids=lambda f: "-".join(f"{k}={v}" for k, v in f.items()) or "plain")
def test_class_weights(feats, dtype, stored):
    """Per-class weights (torch's weighted cross-entropy): every output of the
    fused call against the oracle, in both schedules, over several vocabulary
    slices and a ragged vocabulary."""
    n, d, v = 600, 136, 1000
    inp = small_problem(n, d, v, dtype, bias=True, seed=17)
    cw = np.random.default_rng(5).uniform(0.1, 3.0, v)
    o = O.LossOptions(class_weight=cw, **feats)
    banner(f"class weights {dtype} stored={stored} {feats}")
    kw = dict(stored_logits=True, token_chunk=256) if stored else dict(vocab_slice=256)
    got = _fused_opts(inp, dtype, o, class_weight=torch.tensor(cw, dtype=torch.float32, device="cuda"),
                      **kw)
    U.compare_full(inp, dtype, o, got=got)
    # the forward alone, and the weighted mean's denominator
    x = U.dev_tensor(inp["x"], dtype)
    w = U.dev_tensor(inp["w"], dtype)
    b = U.dev_tensor(inp["bias"], dtype)
    t = torch.from_numpy(inp["targets"]).to("cuda")
    loss, lse, rl = api.forward(x, w, t, b, class_weight=torch.tensor(cw, device="cuda"), **U.lib_opts(o))
    ref = O.forward(inp["x"], inp["w"], inp["bias"], inp["targets"], o)
    U.assert_loss(float(loss), ref.loss)
    assert np.abs(U.host(rl) - ref.row_loss).max() <= 2 * U.LSE_ABS * max(1.0, cw.max())
