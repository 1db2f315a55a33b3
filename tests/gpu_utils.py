"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
call the library through its binding, compare against the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

from linear_cross_entropy_bf16_amd import api
from oracle import flce_oracle as O

# Acceptance bars of the method (bf16 inputs, fp32 accumulation).
LOSS_REL = 1e-4
LSE_ABS = 2e-3
FROB_REL = 5e-3
MAX_REL = 2e-2


def dev_tensor(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


def options(wl, **override) -> O.LossOptions:
    kw = dict(ignore_index=wl.ignore_index, label_smoothing=wl.label_smoothing,
              lse_square_scale=wl.lse_square_scale, softcap=wl.softcap, reduction=wl.reduction)
    kw.update(override)
    return O.LossOptions(**kw)


def lib_opts(o: O.LossOptions) -> dict:
    return dict(ignore_index=o.ignore_index, label_smoothing=o.label_smoothing,
                lse_square_scale=o.lse_square_scale, softcap=o.softcap, reduction=o.reduction)


def assert_loss(got: float, ref: float, what="loss"):
    err = abs(got - ref)
    assert err <= LOSS_REL * max(abs(ref), 1e-30) or (ref == 0.0 and got == 0.0), \
        f"{what}: got {got!r}, oracle {ref!r}, rel err {err / max(abs(ref), 1e-30):.3e}"


def assert_lse(got: np.ndarray, ref: np.ndarray, what="lse"):
    err = np.abs(got - ref)
    assert err.size == 0 or err.max() <= LSE_ABS, f"{what}: max abs err {err.max():.3e}"


def assert_close(got: np.ndarray, ref: np.ndarray, what: str):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    nref = np.linalg.norm(ref)
    nerr = np.linalg.norm(got - ref)
    if nref == 0.0:
        assert nerr == 0.0, f"{what}: reference is 0, got norm {nerr:.3e}"
        return
    assert nerr <= FROB_REL * nref, f"{what}: rel Frobenius err {nerr / nref:.3e}"
    mx = np.abs(ref).max()
    assert np.abs(got - ref).max() <= MAX_REL * mx, \
        f"{what}: max elementwise err {np.abs(got - ref).max():.3e} vs max|ref| {mx:.3e}"


class FrobAccumulator:
    """Relative Frobenius and max-elementwise errors accumulated block by
    block (for weight gradients too large to hold in fp64 at once)."""

    def __init__(self):
        self.err2 = 0.0
        self.ref2 = 0.0
        self.max_err = 0.0
        self.max_ref = 0.0

    def add(self, got, ref):
        d = np.asarray(got, np.float64) - ref
        self.err2 += float((d * d).sum())
        self.ref2 += float((ref * ref).sum())
        self.max_err = max(self.max_err, float(np.abs(d).max()))
        self.max_ref = max(self.max_ref, float(np.abs(ref).max()))

    def check(self, what):
        assert self.ref2 > 0, what
        rel = (self.err2 / self.ref2) ** 0.5
        assert rel <= FROB_REL, f"{what}: rel Frobenius err {rel:.3e}"
        assert self.max_err <= MAX_REL * self.max_ref, \
            f"{what}: max elementwise err {self.max_err:.3e} vs max|ref| {self.max_ref:.3e}"


def assert_dw_column_sums(dw, x_valid, scale, what="dW column sums"):
    """Without z-loss and softcap every row of G sums to 0, so each column of
    dW = scale G^T X sums to 0 over the vocabulary, up to two roundings:
    G is rounded to bf16 (relative error at most 2^-8, unbiased under
    round-to-nearest-even) before the dW contraction, which leaves row n of
    G a sum e_n of standard deviation at most 2^-8 sqrt(1/3) |G_n| <=
    2^-8 sqrt(2/3) (|G_n|^2 <= sum p^2 + 1 <= 2), and column d of dW a sum of
    scale e_n X[n, d] of standard deviation at most
    scale 2^-8 sqrt(2/3) |X[:, d]| over the valid rows; and every fp32 dW
    element carries a few ulp per sqrt of its K/16 accumulation steps, summed
    over V elements.  Bound: 6 standard deviations of each.
    ``dw`` is a device tensor [V, D]; ``x_valid`` the valid rows of X (fp64)."""
    v = dw.shape[0]
    k = x_valid.shape[0]
    colsum = dw.double().sum(dim=0).cpu().numpy()
    max_dw = dw.double().abs().max().item()
    bf16 = 6.0 * scale * 2.0 ** -8 * np.sqrt(2.0 / 3.0) * np.linalg.norm(x_valid, axis=0)
    fp32 = 6.0 * np.sqrt(v) * np.sqrt(max(k, 16) / 16.0) * 2.0 ** -24 * max_dw
    bound = bf16 + fp32
    worst = int(np.argmax(np.abs(colsum) - bound))
    assert np.all(np.abs(colsum) <= bound), \
        f"{what}: column {worst} sums to {colsum[worst]:.3e}, bound {bound[worst]:.3e}"


def run_fused(inp, dtype, o: O.LossOptions, vocab_slice=0):
    x = dev_tensor(inp["x"], dtype)
    w = dev_tensor(inp["w"], dtype)
    b = dev_tensor(inp["bias"], dtype) if inp.get("bias") is not None else None
    t = torch.from_numpy(inp["targets"]).to("cuda")
    loss, lse, dx, dw, db = api.fused_fwd_bwd(x, w, t, b, vocab_slice=vocab_slice, **lib_opts(o))
    torch.cuda.synchronize()
    return dict(loss=float(loss.item()), lse=host(lse), dx=host(dx), dw=host(dw),
                db=None if db is None else host(db))


def compare_full(inp, dtype, o: O.LossOptions, vocab_slice=0, got=None):
    """Every output of one fused call against the oracle, element by element."""
    if got is None:
        got = run_fused(inp, dtype, o, vocab_slice)
    ref = O.forward_backward(inp["x"], inp["w"], inp.get("bias"), inp["targets"], o)
    assert_loss(got["loss"], ref.loss)
    assert_lse(got["lse"], ref.lse)
    assert_close(got["dx"], ref.dx, "dX")
    assert_close(got["dw"], ref.dw, "dW")
    if ref.db is not None and got["db"] is not None:
        assert_close(got["db"], ref.db, "db")
    return got, ref


TIE_ULPS = 256          # near-tie window of an fp32 argmax, in ulp of the largest |logit|
MAX_TIE_FRAC = 1e-3     # at most this fraction of the valid rows may take a near-tie's other side


def tie_window(zabs_max: float, softcap: float = 0.0) -> float:
    """Window within which an argmax decided in fp32 may differ from the
    fp64 one.  A GPU logit carries the fp32 rounding of its contraction: a
    few ulp of the partial sums, whose magnitude stays at the scale of the
    largest |logit| (unit-scale data), so 256 ulp of max|z| covers it with a
    wide margin; under a softcap c the tanh adds c times a few ulp of 1."""
    z = np.float32(max(float(zabs_max), np.finfo(np.float32).tiny))
    return float(TIE_ULPS * np.spacing(z)) + 8.0 * 2.0 ** -24 * float(softcap)


def check_prediction_gaps(pred, acc, ref, gap, window, targets, o: O.LossOptions, n_valid=None):
    """Predicted tokens ``pred`` (GPU) against the fp64 argmax ``ref`` of the
    same rows; ``gap[i]`` = z[i, ref[i]] - z[i, pred[i]] in fp64.  A row may
    differ from the fp64 argmax only inside the near-tie ``window`` and only
    on at most MAX_TIE_FRAC of the valid rows (at least 2); ignored rows must
    hold -1.  The accuracy must be the GPU's own hit rate (``n_valid``
    overrides the denominator for sampled rows: then only the predictions are
    checked).  Returns the number of rows that differ."""
    valid = np.asarray(targets) != o.ignore_index
    assert np.all(pred[~valid] == -1), "ignored rows must predict -1"
    rows = np.nonzero(valid & (pred != ref))[0]
    for i in rows:
        assert 0 <= gap[i] <= window, (f"row {i}: predicted {int(pred[i])}, fp64 argmax {int(ref[i])}, "
                                       f"gap {gap[i]:.3e} outside the near-tie window {window:.3e}")
    nv_rows = int(valid.sum())
    cap = max(2, int(MAX_TIE_FRAC * nv_rows))
    assert len(rows) <= cap, f"{len(rows)} of {nv_rows} rows differ from the fp64 argmax (cap {cap})"
    if n_valid is None:
        hits = int(((pred == targets) & valid).sum())
        want = hits / nv_rows if nv_rows else 0.0
        assert abs(acc - want) <= 1e-6, (acc, want)
        # and the oracle's accuracy, up to the near-tie rows
        ref_acc = O.token_accuracy(np.where(valid, ref, -1), targets, o)
        assert abs(acc - ref_acc) <= len(rows) / max(nv_rows, 1) + 1e-6, (acc, ref_acc)
    return len(rows)


def check_predictions(pred: np.ndarray, acc: float, z: np.ndarray, targets: np.ndarray,
                      o: O.LossOptions, n_valid=None):
    """``check_prediction_gaps`` with the fp64 logits ``z`` of the rows."""
    ref = np.argmax(z, axis=1)
    p = np.clip(pred, 0, z.shape[1] - 1)
    assert np.all((pred == -1) | ((pred >= 0) & (pred < z.shape[1]))), "prediction outside the vocabulary"
    gap = z[np.arange(len(ref)), ref] - z[np.arange(len(ref)), p]
    return check_prediction_gaps(pred, acc, ref, gap, tie_window(np.abs(z).max(), o.softcap), targets, o,
                                 n_valid)


def fp64_argmax_gaps(x, w, bias, softcap, pred, row_block=512):
    """Row by row block over the fp64 logits of (x, w, bias, softcap): the
    argmax, the gap z[argmax] - z[pred] of a given prediction and max|z|,
    without holding all logits."""
    xf, wf, bf = O.to_f64(x), O.to_f64(w), O.to_f64(bias)
    n = xf.shape[0]
    ref = np.empty(n, dtype=np.int64)
    gap = np.zeros(n)
    zabs = 0.0
    for r0 in range(0, n, row_block):
        sl = slice(r0, min(n, r0 + row_block))
        z = O.logits(xf[sl], wf, bf, softcap)
        ref[sl] = np.argmax(z, axis=1)
        idx = np.arange(z.shape[0])
        p = np.clip(pred[sl], 0, z.shape[1] - 1)
        gap[sl] = z[idx, ref[sl]] - z[idx, p]
        zabs = max(zabs, float(np.abs(z).max()))
    return ref, gap, zabs
