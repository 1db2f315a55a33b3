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


def check_predictions(pred: np.ndarray, acc: float, z: np.ndarray, targets: np.ndarray,
                      o: O.LossOptions, n_valid=None, tie_tol: float = 1e-3):
    """Predicted tokens against the fp64 logits ``z`` of the same rows.  The
    argmax is an integer decided in fp32 on the GPU: where it differs from the
    fp64 argmax, the two logits must be a near-tie (within ``tie_tol`` of the
    row's logit scale); ignored rows must hold -1.  The accuracy must be the
    GPU's own hit rate (``n_valid`` overrides the denominator for sampled
    rows: then only the predictions are checked)."""
    valid = np.asarray(targets) != o.ignore_index
    assert np.all(pred[~valid] == -1), "ignored rows must predict -1"
    ref = np.argmax(z, axis=1)
    rows = np.nonzero(valid & (pred != ref))[0]
    scale = max(1.0, float(np.abs(z).max()))
    for i in rows:
        p = int(pred[i])
        assert 0 <= p < z.shape[1], f"row {i}: predicted {p} outside the vocabulary"
        gap = z[i, ref[i]] - z[i, p]
        assert gap <= tie_tol * scale, f"row {i}: predicted {p}, fp64 argmax {ref[i]}, gap {gap:.3e}"
    if n_valid is None:
        nv = int(valid.sum())
        hits = int(((pred == targets) & valid).sum())
        want = hits / nv if nv else 0.0
        assert abs(acc - want) <= 1e-6, (acc, want)
        # and the oracle's accuracy, up to the near-tie rows
        ref_acc = O.token_accuracy(np.where(valid, ref, -1), targets, o)
        assert abs(acc - ref_acc) <= len(rows) / max(nv, 1) + 1e-6, (acc, ref_acc)
    return len(rows)
