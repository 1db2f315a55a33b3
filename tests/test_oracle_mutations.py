"""Plant plausible mistakes in a private copy of the oracle and check that at
least one pin catches each of them (CPU only; the real oracle is untouched)."""
import importlib.util
import os
import sys

import numpy as np
import pytest

from tests import oracle_pins as P

ORACLE_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "oracle", "flce_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("flce_oracle_mutant", ORACLE_PATH)
    m = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = m          # dataclasses look their module up here
    spec.loader.exec_module(m)
    return m


def mut_drop_smoothing_sum(m):
    orig = m.row_losses

    def row_losses(z, lse, targets, opts):
        o2 = m.LossOptions(opts.ignore_index, 0.0, opts.lse_square_scale, opts.softcap, opts.reduction)
        valid = m.valid_rows(targets, opts)
        t = np.where(valid, targets, 0)
        zt = z[np.arange(z.shape[0]), t]
        base = orig(z, lse, targets, o2)
        return np.where(valid, base + opts.label_smoothing * zt, 0.0)   # forgot -(eps/V) sum z
    m.row_losses = row_losses


def mut_zloss_grad_sign(m):
    orig = m.grad_logits

    def grad_logits(z, lse, targets, opts):
        g = orig(z, lse, targets, opts)
        s = opts.lse_square_scale
        if s:
            p = np.exp(z - lse[:, None])
            fac = 1.0 - (z / opts.softcap) ** 2 if opts.softcap > 0 else 1.0
            valid = m.valid_rows(targets, opts)
            g = g - (4.0 * s * lse[:, None] * p * fac) * valid[:, None]   # 1 - 2 s lse
        return g
    m.grad_logits = grad_logits


def mut_no_softcap_derivative(m):
    orig = m.grad_logits

    def grad_logits(z, lse, targets, opts):
        g = orig(z, lse, targets, opts)
        if opts.softcap > 0:
            with np.errstate(divide="ignore", invalid="ignore"):
                g = np.where(g != 0, g / (1.0 - (z / opts.softcap) ** 2), 0.0)
        return g
    m.grad_logits = grad_logits


def mut_target_off_by_one(m):
    orig = m.grad_logits

    def grad_logits(z, lse, targets, opts):
        t = np.asarray(targets).copy()
        v = z.shape[1]
        ok = t != opts.ignore_index
        t[ok] = (t[ok] + 1) % v
        return orig(z, lse, t, opts)
    m.grad_logits = grad_logits


def mut_lse_missing_max(m):
    def log_sum_exp(z):
        mx = z.max(axis=1)
        return np.log(np.exp(z - mx[:, None]).sum(axis=1))
    m.log_sum_exp = log_sum_exp


def mut_mean_over_all_rows(m):
    orig = m.reduce_loss

    def reduce_loss(row_loss, n_valid, opts):
        if opts.reduction == "mean":
            return float(row_loss.sum() / row_loss.size)
        return orig(row_loss, n_valid, opts)
    m.reduce_loss = reduce_loss


def mut_online_no_rescale(m):
    def log_sum_exp_online(z, block):
        n, v = z.shape
        mx = np.full(n, -np.inf)
        d = np.zeros(n)
        for v0 in range(0, v, block):
            blk = z[:, v0:v0 + block]
            m_new = np.maximum(mx, blk.max(axis=1))
            d = d + np.exp(blk - m_new[:, None]).sum(axis=1)
            mx = m_new
        return mx + np.log(d)
    m.log_sum_exp_online = log_sum_exp_online


def mut_smoothing_over_v_minus_1(m):
    orig = m.grad_logits

    def grad_logits(z, lse, targets, opts):
        g = orig(z, lse, targets, opts)
        v = z.shape[1]
        eps = opts.label_smoothing
        if eps and v > 1:
            valid = m.valid_rows(targets, opts)
            g = g + (eps / v - eps / (v - 1)) * valid[:, None]
        return g
    m.grad_logits = grad_logits


def mut_transposed_dw(m):
    orig = m.forward_backward

    def forward_backward(*a, **k):
        r = orig(*a, **k)
        if r.dw is not None and r.dw.shape[0] == r.dw.shape[1]:
            r.dw = r.dw.T.copy()
        elif r.dw is not None:
            r.dw = r.dw[::-1].copy()          # rows attributed to the wrong class
        return r
    m.forward_backward = forward_backward


def mut_logits_ignore_softcap(m):
    orig = m.cross_entropy_on_logits

    def cross_entropy_on_logits(r, targets, opts, *a, **k):
        o2 = m.LossOptions(opts.ignore_index, opts.label_smoothing, opts.lse_square_scale, 0.0,
                           opts.reduction)
        return orig(r, targets, o2, *a, **k)            # softcap option dropped on this path
    m.cross_entropy_on_logits = cross_entropy_on_logits


def mut_logits_unscaled_grad(m):
    orig = m.cross_entropy_on_logits

    def cross_entropy_on_logits(r, targets, opts, grad_output=1.0, n_valid=None, want_grad=True,
                                **k):
        res = orig(r, targets, opts, grad_output, n_valid, want_grad, **k)
        if want_grad and res.n_valid and opts.reduction == "mean":
            res.dx = res.dx * res.n_valid                  # forgot the 1 / n_valid of the mean
        return res
    m.cross_entropy_on_logits = cross_entropy_on_logits


def mut_megatron_plain_eps(m):
    m.megatron_smoothing = lambda eps, v: eps               # forgot the V / (V - 1)


def mut_argmax_last_tie(m):
    def predicted_tokens(z, targets, opts):
        pred = (z.shape[1] - 1 - np.argmax(z[:, ::-1], axis=1)).astype(np.int32)   # last maximum
        return np.where(m.valid_rows(targets, opts), pred, -1).astype(np.int32)
    m.predicted_tokens = predicted_tokens


def mut_accuracy_over_all_rows(m):
    def token_accuracy(pred, targets, opts, n_valid=None):
        return float((pred == np.asarray(targets)).sum()) / len(targets)
    m.token_accuracy = token_accuracy


def mut_weighted_mean_over_rows(m):
    orig = m.mean_denominator

    def mean_denominator(targets, opts):
        if opts.class_weight is None:
            return orig(targets, opts)
        return int(m.valid_rows(targets, opts).sum())           # forgot the weights in the mean
    m.mean_denominator = mean_denominator


def mut_weighted_smoothing_unweighted(m):
    orig = m.grad_logits

    def grad_logits(z, lse, targets, opts):
        g = orig(z, lse, targets, opts)
        if opts.class_weight is not None and opts.label_smoothing:
            w = np.asarray(opts.class_weight, dtype=np.float64)
            valid = m.valid_rows(targets, opts)
            fac = 1.0 - (z / opts.softcap) ** 2 if opts.softcap > 0 else 1.0
            g = g + (opts.label_smoothing / z.shape[1]) * (w[None, :] - 1.0) * fac * valid[:, None]
        return g                                                  # eps/V instead of eps w_c / V
    m.grad_logits = grad_logits


def mut_bf16_as_fp16(m):
    orig = m.to_f64

    def to_f64(a):
        if a is not None and a.dtype == np.uint16:
            return a.view(np.float16).astype(np.float64)          # the bits read as IEEE half
        return orig(a)
    m.to_f64 = to_f64


def mut_columns_smoothing_over_held(m):
    orig = m.grad_logits_columns

    def grad_logits_columns(z_cols, cols, v, lse, targets, opts):
        return orig(z_cols, cols, len(cols), lse, targets, opts)   # eps / (columns held), not eps / V
    m.grad_logits_columns = grad_logits_columns


def mut_columns_target_by_position(m):
    orig = m.grad_logits_columns

    def grad_logits_columns(z_cols, cols, v, lse, targets, opts):
        return orig(z_cols, np.arange(len(cols)), v, lse, targets, opts)   # one-hot by position
    m.grad_logits_columns = grad_logits_columns


MUTATIONS = [mut_drop_smoothing_sum, mut_zloss_grad_sign, mut_no_softcap_derivative,
             mut_target_off_by_one, mut_lse_missing_max, mut_mean_over_all_rows,
             mut_online_no_rescale, mut_smoothing_over_v_minus_1, mut_transposed_dw,
             mut_logits_ignore_softcap, mut_logits_unscaled_grad, mut_megatron_plain_eps,
             mut_argmax_last_tie, mut_accuracy_over_all_rows, mut_weighted_mean_over_rows,
             mut_weighted_smoothing_unweighted, mut_bf16_as_fp16,
             mut_columns_smoothing_over_held, mut_columns_target_by_position]


@pytest.mark.parametrize("mutate", MUTATIONS, ids=lambda f: f.__name__)
def test_mutation_is_caught(mutate):
    m = fresh_oracle()
    mutate(m)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(m)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught {mutate.__name__}"
