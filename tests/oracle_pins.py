"""Checks that pin the fp64 oracle to facts other than itself.

Each ``pin_*`` function raises AssertionError when the oracle module it is
given disagrees with a closed form, an invariant, a library special case,
finite differences or a brute-force evaluation of the definition.  They take
the module as an argument so ``test_oracle_mutations.py`` can show that
plausible mistakes planted in a patched copy of the oracle are caught.
"""
from __future__ import annotations

import math

import numpy as np

IGN = -100


def _problem(n=24, d=16, v=40, seed=0, bias=False, ignore=3, scale_w=None):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d))
    w = rng.standard_normal((v, d)) * (scale_w if scale_w is not None else 1.0 / math.sqrt(d))
    b = rng.standard_normal(v) * 0.3 if bias else None
    t = rng.integers(0, v, n).astype(np.int32)
    if ignore:
        t[rng.choice(n, ignore, replace=False)] = IGN
    return x, w, b, t


def _opts(O, **kw):
    return O.LossOptions(**kw)


FEATURE_SETS = [
    dict(),
    dict(label_smoothing=0.1),
    dict(lse_square_scale=1e-2),
    dict(softcap=2.0),
    dict(label_smoothing=0.2, lse_square_scale=3e-2, softcap=1.5),
    dict(reduction="sum"),
    dict(reduction="sum", label_smoothing=0.1, lse_square_scale=1e-2, softcap=3.0),
]


# ------------------------------------------------------------ closed forms

def pin_uniform_logits(O):
    """W = 0, b = 0: every logit is 0, softmax is uniform, lse = ln V, the
    per-row loss is ln V (+ s ln^2 V) whatever eps and c, dX = 0 exactly."""
    for v in (1024, 32000):
        n, d = 8, 16
        x = np.random.default_rng(1).standard_normal((n, d))
        w = np.zeros((v, d))
        t = np.arange(n, dtype=np.int32) * 7 % v
        for feats in FEATURE_SETS:
            o = _opts(O, **feats)
            r = O.forward_backward(x, w, None, t, o)
            ln_v = math.log(v)
            expect = ln_v + o.lse_square_scale * ln_v * ln_v
            assert np.allclose(r.lse, ln_v, rtol=0, atol=1e-12), feats
            assert np.allclose(r.row_loss, expect, rtol=0, atol=1e-12), feats
            total = expect * n
            want = total if o.reduction == "sum" else total / n
            assert abs(r.loss - want) <= 1e-10 * abs(want), feats
            assert np.all(r.dx == 0.0), feats
            # uniform softmax: G[n, v] = 1/V (1 + 2 s ln V) - (1-eps) [v = t] - eps/V
            z = O.logits(x, w, None, o.softcap)
            g = O.grad_logits(z, O.log_sum_exp(z), t, o)
            base = (1.0 + 2.0 * o.lse_square_scale * ln_v) / v - o.label_smoothing / v
            off = np.ones((n, v), bool)
            off[np.arange(n), t] = False
            assert np.allclose(g[off], base, rtol=0, atol=1e-15), feats
            assert np.allclose(g[~off], base - (1.0 - o.label_smoothing), rtol=0, atol=1e-15), feats


def pin_single_class(O):
    """V = 1: softmax is 1 and lse = z_0, so the cross-entropy term vanishes
    and the loss is s z_0^2; G = 2 s z_0 on every valid row."""
    n, d = 6, 5
    rng = np.random.default_rng(2)
    x = rng.standard_normal((n, d))
    w = rng.standard_normal((1, d))
    t = np.zeros(n, np.int32)
    s = 0.05
    o = _opts(O, lse_square_scale=s, label_smoothing=0.3, reduction="sum")
    r = O.forward_backward(x, w, None, t, o)
    z0 = x @ w[0]
    assert np.allclose(r.lse, z0, atol=1e-13)
    assert np.allclose(r.row_loss, s * z0 ** 2, atol=1e-13)
    assert np.allclose(r.dx, (2 * s * z0)[:, None] * w[0][None, :], atol=1e-13)


def pin_two_classes(O):
    """V = 2 with eps = s = 0: the loss is softplus(z_other - z_target),
    evaluated with scalar math.log1p / math.exp, with and without softcap."""
    n, d = 10, 7
    rng = np.random.default_rng(3)
    x = rng.standard_normal((n, d))
    w = rng.standard_normal((2, d))
    t = rng.integers(0, 2, n).astype(np.int32)
    for c in (0.0, 1.3):
        o = _opts(O, softcap=c, reduction="none")
        r = O.forward(x, w, None, t, o)
        for i in range(n):
            raw = [float(np.dot(x[i], w[k])) for k in range(2)]
            z = [c * math.tanh(q / c) for q in raw] if c > 0 else raw
            m = z[1 - t[i]] - z[t[i]]
            sp = m + math.log1p(math.exp(-m)) if m > 0 else math.log1p(math.exp(m))
            assert abs(r.row_loss[i] - sp) <= 1e-13, (c, i)


# ------------------------------------------------------------ invariants

def pin_gradient_row_sums(O):
    """Each row of G sums to 0 without z-loss and softcap (softmax sums to 1,
    the smoothed target distribution sums to 1), so sum_v dW[v, :] = 0 and
    sum_v db = 0; with z-loss the row sum is 2 s lse."""
    x, w, b, t = _problem(bias=True)
    for eps in (0.0, 0.15):
        o = _opts(O, label_smoothing=eps)
        z = O.logits(x, w, b, 0.0)
        g = O.grad_logits(z, O.log_sum_exp(z), t, o)
        assert np.allclose(g.sum(axis=1), 0.0, atol=1e-14)
        r = O.forward_backward(x, w, b, t, o)
        assert np.allclose(r.dw.sum(axis=0), 0.0, atol=1e-14)
        assert abs(r.db.sum()) <= 1e-14
    s = 0.04
    o = _opts(O, lse_square_scale=s)
    z = O.logits(x, w, b, 0.0)
    lse = O.log_sum_exp(z)
    g = O.grad_logits(z, lse, t, o)
    valid = t != IGN
    assert np.allclose(g.sum(axis=1)[valid], 2 * s * lse[valid], atol=1e-13)
    assert np.all(g[~valid] == 0.0)


def pin_shift_invariance(O):
    """Adding the same vector u to every vocabulary row of W shifts every
    logit of row n by x_n.u: softmax, the loss, dX, dW and db are unchanged
    (s = c = 0), and lse moves by exactly x_n.u."""
    x, w, b, t = _problem(bias=True)
    u = np.random.default_rng(9).standard_normal(w.shape[1]) * 0.7
    for eps in (0.0, 0.1):
        o = _opts(O, label_smoothing=eps, reduction="sum")
        r0 = O.forward_backward(x, w, b, t, o)
        r1 = O.forward_backward(x, w + u[None, :], b, t, o)
        valid = t != IGN
        assert np.allclose(r1.lse[valid], r0.lse[valid] + (x @ u)[valid], atol=1e-12)
        assert abs(r1.loss - r0.loss) <= 1e-11
        assert np.allclose(r1.dx, r0.dx, atol=1e-12)
        assert np.allclose(r1.dw, r0.dw, atol=1e-12)
        assert np.allclose(r1.db, r0.db, atol=1e-12)


def pin_batch_additivity(O):
    """Under sum reduction the loss and the weight gradient of a batch are
    the sums over any partition of its rows (the micro-batching identity)."""
    x, w, b, t = _problem(n=30, bias=True)
    o = _opts(O, reduction="sum", label_smoothing=0.1, lse_square_scale=1e-2, softcap=2.5)
    full = O.forward_backward(x, w, b, t, o)
    parts = [slice(0, 7), slice(7, 19), slice(19, 30)]
    loss = sum(O.forward_backward(x[p], w, b, t[p], o).loss for p in parts)
    dw = sum(O.forward_backward(x[p], w, b, t[p], o).dw for p in parts)
    db = sum(O.forward_backward(x[p], w, b, t[p], o).db for p in parts)
    assert abs(loss - full.loss) <= 1e-11 * abs(full.loss)
    assert np.allclose(dw, full.dw, atol=1e-13)
    assert np.allclose(db, full.db, atol=1e-13)


def pin_vocab_permutation(O):
    """Relabelling the vocabulary (permuting rows of W and b and mapping the
    targets) leaves the loss, lse and dX unchanged and permutes dW and db."""
    x, w, b, t = _problem(bias=True)
    v = w.shape[0]
    perm = np.random.default_rng(5).permutation(v)      # new row j = old row perm[j]
    inv = np.argsort(perm)
    t2 = np.where(t == IGN, IGN, inv[np.where(t == IGN, 0, t)]).astype(np.int32)
    o = _opts(O, label_smoothing=0.1, lse_square_scale=1e-2, softcap=2.0)
    r0 = O.forward_backward(x, w, b, t, o)
    r1 = O.forward_backward(x, w[perm], b[perm], t2, o)
    assert abs(r0.loss - r1.loss) <= 1e-12
    assert np.allclose(r0.lse, r1.lse, atol=1e-12)
    assert np.allclose(r0.dx, r1.dx, atol=1e-13)
    assert np.allclose(r0.dw[perm], r1.dw, atol=1e-13)
    assert np.allclose(r0.db[perm], r1.db, atol=1e-13)


def pin_online_merge(O):
    """The blocked online-softmax recurrence reaches the two-pass LSE, also
    with a ragged last block and with blocks whose maximum falls."""
    rng = np.random.default_rng(6)
    z = rng.standard_normal((16, 1000)) * 4.0
    z[:, 500:] -= 30.0          # later blocks have smaller maxima
    z[3, 999] = 60.0            # a late maximum forces a rescale
    ref = O.log_sum_exp(z)
    for blk in (1, 7, 64, 333, 1000, 4096):
        assert np.allclose(O.log_sum_exp_online(z, blk), ref, rtol=0, atol=1e-12), blk


def pin_no_valid_rows(O):
    """All rows ignored: mean loss is 0 (declared, no 0/0), grads are 0."""
    x, w, b, _ = _problem(bias=True, ignore=0)
    t = np.full(x.shape[0], IGN, np.int32)
    for red in ("mean", "sum"):
        r = O.forward_backward(x, w, b, t, _opts(O, reduction=red))
        assert r.loss == 0.0 and r.n_valid == 0
        assert np.all(r.dx == 0) and np.all(r.dw == 0) and np.all(r.db == 0)
        assert np.all(r.lse == 0) and np.all(r.row_loss == 0)


def pin_softcap_limits(O):
    """A very large cap reproduces the uncapped loss; capped logits stay
    inside [-c, c]."""
    x, w, b, t = _problem(bias=True, scale_w=1.0)
    r0 = O.forward_backward(x, w, b, t, _opts(O))
    r1 = O.forward_backward(x, w, b, t, _opts(O, softcap=1e7))
    assert abs(r0.loss - r1.loss) <= 1e-9 * abs(r0.loss)
    assert np.allclose(r0.dw, r1.dw, atol=1e-9)
    z = O.logits(x, w, b, 0.5)
    assert np.all(np.abs(z) <= 0.5)


# ------------------------------------------------------------ library case

def pin_torch_cross_entropy(O):
    """Without softcap and z-loss the method is torch's cross-entropy of the
    materialised logits: loss (mean over non-ignored rows, sum or none, with
    label smoothing) and autograd gradients, all in float64 on the CPU."""
    import torch
    import torch.nn.functional as F

    for bias in (False, True):
        x, w, b, t = _problem(n=40, d=12, v=57, bias=bias, ignore=5, seed=11)
        for eps in (0.0, 0.1):
            for red in ("mean", "sum", "none"):
                o = _opts(O, label_smoothing=eps, reduction=red)
                xt = torch.tensor(x, requires_grad=True)
                wt = torch.tensor(w, requires_grad=True)
                bt = torch.tensor(b, requires_grad=True) if bias else None
                lg = xt @ wt.T + (bt if bias else 0.0)
                lt = F.cross_entropy(lg, torch.tensor(t, dtype=torch.long),
                                     ignore_index=IGN, label_smoothing=eps,
                                     reduction=red)
                if red == "none":
                    r = O.forward(x, w, b, t, o)
                    assert np.allclose(r.loss, lt.detach().numpy(), rtol=0, atol=1e-13)
                    continue
                lt.backward()
                r = O.forward_backward(x, w, b, t, o)
                assert abs(r.loss - lt.item()) <= 1e-13 * max(1.0, abs(lt.item()))
                assert np.allclose(r.dx, xt.grad.numpy(), rtol=0, atol=1e-14)
                assert np.allclose(r.dw, wt.grad.numpy(), rtol=0, atol=1e-14)
                if bias:
                    assert np.allclose(r.db, bt.grad.numpy(), rtol=0, atol=1e-14)


# ------------------------------------------------------------ calculus

def pin_finite_differences(O, n=256, d=128, v=1024, directions=16, seed=21):
    """Central differences of the loss along random directions in X, W, b and
    along W restricted to the target rows agree with the analytic gradient to
    1e-7 of the gradient's norm, for every feature combination."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d))
    w = rng.standard_normal((v, d)) / math.sqrt(d)
    b = rng.standard_normal(v) * 0.02
    t = rng.integers(0, v, n).astype(np.int32)
    t[rng.choice(n, n // 20, replace=False)] = IGN
    h = 1e-5
    for feats in FEATURE_SETS:
        o = _opts(O, **feats)
        r = O.forward_backward(x, w, b, t, o)

        def loss_at(xx, ww, bb):
            return O.forward(xx, ww, bb, t, o).loss

        for k in range(directions):
            which = k % 4
            if which == 0:
                dxv = rng.standard_normal(x.shape)
                dxv /= np.linalg.norm(dxv)
                fd = (loss_at(x + h * dxv, w, b) - loss_at(x - h * dxv, w, b)) / (2 * h)
                an, gn = float((r.dx * dxv).sum()), np.linalg.norm(r.dx)
            elif which in (1, 3):
                dwv = rng.standard_normal(w.shape)
                if which == 3:           # only the target rows of W
                    mask = np.zeros(v, bool)
                    mask[t[t != IGN]] = True
                    dwv[~mask] = 0.0
                dwv /= np.linalg.norm(dwv)
                fd = (loss_at(x, w + h * dwv, b) - loss_at(x, w - h * dwv, b)) / (2 * h)
                an, gn = float((r.dw * dwv).sum()), np.linalg.norm(r.dw)
            else:
                dbv = rng.standard_normal(v)
                dbv /= np.linalg.norm(dbv)
                fd = (loss_at(x, w, b + h * dbv) - loss_at(x, w, b - h * dbv)) / (2 * h)
                an, gn = float((r.db * dbv).sum()), np.linalg.norm(r.db)
            assert abs(fd - an) <= 1e-7 * gn + 1e-12, (feats, k, fd, an, gn)


# ------------------------------------------------------------ brute force

def _brute_row(xr, W, br, t, eps, s, c):
    """Cross-entropy -sum_v q_v log p_v of one row by plain Python loops,
    straight from the definition of cross-entropy between two distributions
    (no LSE rewriting): p = softmax(z), q = (1-eps) onehot_t + eps/V."""
    V = len(W)
    z = []
    for j in range(V):
        acc = 0.0
        for k in range(len(xr)):
            acc += xr[k] * W[j][k]
        if br is not None:
            acc += br[j]
        if c > 0:
            acc = c * math.tanh(acc / c)
        z.append(acc)
    mx = max(z)
    ex = [math.exp(q - mx) for q in z]
    tot = sum(ex)
    p = [e / tot for e in ex]
    ce = 0.0
    for j in range(V):
        q = (1.0 - eps) * (1.0 if j == t else 0.0) + eps / V
        ce -= q * math.log(p[j])
    zlse = mx + math.log(tot)
    return ce + s * zlse * zlse, zlse


def pin_brute_force(O):
    """Tiny problems (N = 5, D = 4, V = 6) evaluated row by row with plain
    Python loops from the cross-entropy definition, every feature on."""
    rng = np.random.default_rng(13)
    n, d, v = 5, 4, 6
    x = rng.standard_normal((n, d))
    w = rng.standard_normal((v, d))
    b = rng.standard_normal(v) * 0.5
    t = np.array([0, 5, IGN, 2, 3], np.int32)
    for eps, s, c, red in ((0.0, 0.0, 0.0, "mean"), (0.25, 0.0, 0.0, "sum"),
                           (0.0, 0.07, 0.0, "mean"), (0.0, 0.0, 1.1, "sum"),
                           (0.3, 0.05, 2.0, "mean"), (0.3, 0.05, 2.0, "none")):
        o = _opts(O, label_smoothing=eps, lse_square_scale=s, softcap=c, reduction=red)
        r = O.forward(x, w, b, t, o)
        rows = []
        for i in range(n):
            if t[i] == IGN:
                rows.append(0.0)
                assert r.lse[i] == 0.0
                continue
            l, zl = _brute_row(list(x[i]), [list(q) for q in w], list(b), int(t[i]), eps, s, c)
            rows.append(l)
            assert abs(r.lse[i] - zl) <= 1e-13
        rows = np.array(rows)
        assert np.allclose(r.row_loss, rows, rtol=0, atol=1e-13)
        nv = int((t != IGN).sum())
        want = rows.sum() / nv if red == "mean" else (rows.sum() if red == "sum" else rows)
        assert np.allclose(r.loss, want, rtol=0, atol=1e-13)


def pin_gaussian_lse_level(O):
    """Statistical sanity, not a tolerance: with unit-variance Gaussian logits
    E[exp z] = e^(1/2), so the mean LSE sits near ln V + 1/2."""
    rng = np.random.default_rng(17)
    n, d, v = 64, 256, 4096
    x = rng.standard_normal((n, d))
    w = rng.standard_normal((v, d)) / math.sqrt(d)
    t = rng.integers(0, v, n).astype(np.int32)
    r = O.forward(x, w, None, t, _opts(O))
    assert abs(r.lse.mean() - (math.log(v) + 0.5)) < 0.05


# ------------------------------------------------- cross-entropy on logits

def _logits_problem(n=30, v=47, seed=31, ignore=4, spread=1.5):
    rng = np.random.default_rng(seed)
    r = rng.standard_normal((n, v)) * spread
    t = rng.integers(0, v, n).astype(np.int32)
    if ignore:
        t[rng.choice(n, ignore, replace=False)] = IGN
    return r, t


def pin_logits_identity_linear(O):
    """Cross-entropy on given logits r is the fused problem with X = r and W =
    the identity (logits X.W^T = r), whose dX = G.W is then dL/dr, for every
    feature combination; the fused oracle is pinned independently above."""
    r, t = _logits_problem()
    eye = np.eye(r.shape[1])
    for feats in FEATURE_SETS:
        o = _opts(O, **feats)
        a = O.cross_entropy_on_logits(r, t, o, grad_output=0.7)
        b = O.forward_backward(r, eye, None, t, o, grad_output=0.7)
        assert abs(a.loss - b.loss) <= 1e-13 * max(1.0, abs(b.loss)), feats
        assert np.allclose(a.lse, b.lse, rtol=0, atol=1e-13), feats
        assert np.allclose(a.row_loss, b.row_loss, rtol=0, atol=1e-13), feats
        assert np.allclose(a.dx, b.dx, rtol=0, atol=1e-15), feats


def pin_logits_torch(O):
    """Without softcap and z-loss: torch's cross_entropy on the same logits
    (mean over non-ignored rows, sum, none; label smoothing) and its autograd
    gradient, float64 on the CPU."""
    import torch
    import torch.nn.functional as F

    r, t = _logits_problem(n=33, v=61, seed=5)
    for eps in (0.0, 0.15):
        for red in ("mean", "sum", "none"):
            o = _opts(O, label_smoothing=eps, reduction=red)
            rt = torch.tensor(r, requires_grad=True)
            lt = F.cross_entropy(rt, torch.tensor(t, dtype=torch.long), ignore_index=IGN,
                                 label_smoothing=eps, reduction=red)
            if red == "none":
                a = O.cross_entropy_on_logits(r, t, o, want_grad=False)
                assert np.allclose(a.loss, lt.detach().numpy(), rtol=0, atol=1e-13)
                continue
            lt.backward()
            a = O.cross_entropy_on_logits(r, t, o)
            assert abs(a.loss - lt.item()) <= 1e-13 * max(1.0, abs(lt.item()))
            assert np.allclose(a.dx, rt.grad.numpy(), rtol=0, atol=1e-15)


def pin_logits_finite_differences(O, directions=12, seed=8):
    """Central differences of the loss along random directions of the logits
    agree with dL/dr to 1e-7 of its norm, for every feature combination (the
    softcap derivative and the z-loss term included)."""
    rng = np.random.default_rng(seed)
    r, t = _logits_problem(n=64, v=300, seed=seed, ignore=6)
    h = 1e-5
    for feats in FEATURE_SETS:
        o = _opts(O, **feats)
        a = O.cross_entropy_on_logits(r, t, o)
        gn = np.linalg.norm(a.dx)
        for _ in range(directions):
            dv = rng.standard_normal(r.shape)
            dv /= np.linalg.norm(dv)
            fp = O.cross_entropy_on_logits(r + h * dv, t, o, want_grad=False).loss
            fm = O.cross_entropy_on_logits(r - h * dv, t, o, want_grad=False).loss
            fd = (fp - fm) / (2 * h)
            an = float((a.dx * dv).sum())
            assert abs(fd - an) <= 1e-7 * gn + 1e-12, (feats, fd, an, gn)


def pin_megatron_smoothing(O):
    """The Megatron form that the TransformerEngine cross-entropy kernels
    follow, written out here from its own description: smoothing = eps V / (V-1),
    loss = (1 - smoothing)(-log p_t) - smoothing mean_v log p_v and gradient
    softmax - (1 - smoothing) onehot - smoothing / V.  It equals the oracle at
    eps' = megatron_smoothing(eps, V); its target distribution keeps 1 - eps on
    the target and eps / (V - 1) on every other class."""
    r, t = _logits_problem(n=20, v=37, seed=9, ignore=0)
    n, v = r.shape
    for eps in (0.05, 0.3):
        sm = eps * v / (v - 1)
        assert abs(O.megatron_smoothing(eps, v) - sm) <= 1e-15
        assert abs((1 - sm + sm / v) - (1 - eps)) <= 1e-15 and abs(sm / v - eps / (v - 1)) <= 1e-15
        m = r.max(axis=1, keepdims=True)
        logp = r - m - np.log(np.exp(r - m).sum(axis=1, keepdims=True))
        rows = -(1 - sm) * logp[np.arange(n), t] - sm * logp.mean(axis=1)
        grad = np.exp(logp)
        grad[np.arange(n), t] -= 1 - sm
        grad -= sm / v
        a = O.cross_entropy_on_logits(r, t, _opts(O, label_smoothing=O.megatron_smoothing(eps, v),
                                                  reduction="sum"))
        assert np.allclose(a.row_loss, rows, rtol=0, atol=1e-13)
        assert np.allclose(a.dx, grad, rtol=0, atol=1e-15)


# ------------------------------------------------- predicted tokens, accuracy

def pin_predicted_tokens(O):
    """Predicted tokens by brute force (a Python loop keeping the first
    strict maximum), torch.argmax on the same logits, ties at W = 0 (every
    valid row predicts 0), invariance under the monotonic softcap, and the
    accuracy as hits over valid rows on a constructed case."""
    import torch

    x, w, b, t = _problem(n=40, d=10, v=33, bias=True, ignore=6, seed=41)
    o = _opts(O)
    pred, acc = O.forward_metrics(x, w, b, t, o)
    z = x @ w.T + b
    for i in range(len(t)):
        if t[i] == IGN:
            assert pred[i] == -1
            continue
        best, arg = -math.inf, -1
        for v in range(w.shape[0]):
            zv = sum(float(x[i, k]) * float(w[v, k]) for k in range(x.shape[1])) + float(b[v])
            if zv > best:
                best, arg = zv, v
        assert pred[i] == arg
    tz = torch.argmax(torch.tensor(z), dim=1).numpy()
    valid = t != IGN
    assert np.array_equal(pred[valid], tz[valid])
    assert acc == float(((tz == t) & valid).sum()) / valid.sum()
    for c in (0.5, 3.0):
        pc, _ = O.forward_metrics(x, w, b, t, _opts(O, softcap=c))
        assert np.array_equal(pc, pred)
    # W = 0: all logits tie, the lowest index wins
    p0, a0 = O.forward_metrics(x, np.zeros_like(w), None, t, o)
    assert np.all(p0[valid] == 0) and np.all(p0[~valid] == -1)
    assert a0 == float(((t == 0) & valid).sum()) / valid.sum()
    # constructed: X = identity rows pick class k with logit 1, others 0
    n = 12
    xe = np.eye(n)
    we = np.eye(n)
    te = np.arange(n, dtype=np.int32)
    te[[1, 4, 7]] = [0, 0, 0]                          # three misses
    te[10] = IGN
    pe, ae = O.forward_metrics(xe, we, None, te, o)
    assert np.array_equal(pe[te != IGN], np.arange(n)[te != IGN])
    assert ae == 8 / 11
    # no valid row: accuracy 0
    assert O.token_accuracy(pe, np.full(n, IGN, np.int32), o) == 0.0
    # the logits entry point agrees with the fused one at W = identity
    pl, al = O.logits_metrics(x @ w.T + b, t, o)
    assert np.array_equal(pl, pred) and al == acc


# ------------------------------------------------- class weights

def pin_class_weight_torch(O):
    """Per-class weights without softcap and z-loss are torch's weighted
    cross-entropy of the materialised logits: loss (mean over the sum of the
    valid rows' target weights, sum, none; with label smoothing) and autograd
    gradients through the linear layer, float64 on the CPU."""
    import torch
    import torch.nn.functional as F

    x, w, b, t = _problem(n=36, d=10, v=23, bias=True, ignore=4, seed=13)
    cw = np.random.default_rng(3).uniform(0.1, 3.0, w.shape[0])
    for eps in (0.0, 0.15):
        for red in ("mean", "sum", "none"):
            o = _opts(O, label_smoothing=eps, reduction=red, class_weight=cw)
            xt = torch.tensor(x, requires_grad=True)
            wt = torch.tensor(w, requires_grad=True)
            bt = torch.tensor(b, requires_grad=True)
            lt = F.cross_entropy(xt @ wt.T + bt, torch.tensor(t, dtype=torch.long),
                                 weight=torch.tensor(cw), ignore_index=IGN, label_smoothing=eps,
                                 reduction=red)
            if red == "none":
                r = O.forward(x, w, b, t, o)
                assert np.allclose(r.loss, lt.detach().numpy(), rtol=0, atol=1e-13)
                continue
            lt.backward()
            r = O.forward_backward(x, w, b, t, o)
            assert abs(r.loss - lt.item()) <= 1e-13 * max(1.0, abs(lt.item())), (eps, red)
            assert np.allclose(r.dx, xt.grad.numpy(), rtol=0, atol=1e-14)
            assert np.allclose(r.dw, wt.grad.numpy(), rtol=0, atol=1e-14)
            assert np.allclose(r.db, bt.grad.numpy(), rtol=0, atol=1e-14)


def pin_class_weight_unit_and_fd(O, directions=8, seed=29):
    """Unit weights give the unweighted problem exactly, for every feature
    combination; with random weights, softcap and z-loss (outside torch's
    reach) central differences along X and W agree with the gradient."""
    x, w, b, t = _problem(n=40, d=12, v=50, bias=True, ignore=5, seed=seed)
    ones = np.ones(w.shape[0])
    for feats in FEATURE_SETS:
        a = O.forward_backward(x, w, b, t, _opts(O, **feats))
        c = O.forward_backward(x, w, b, t, _opts(O, class_weight=ones, **feats))
        assert abs(a.loss - c.loss) <= 1e-13 * max(1.0, abs(a.loss)), feats
        assert np.allclose(a.dx, c.dx, rtol=0, atol=1e-15) and np.allclose(a.dw, c.dw, rtol=0, atol=1e-15)
    rng = np.random.default_rng(seed)
    cw = rng.uniform(0.2, 2.5, w.shape[0])
    h = 1e-5
    for feats in (dict(softcap=2.0, lse_square_scale=3e-2, label_smoothing=0.2),
                  dict(lse_square_scale=1e-2, reduction="sum"), dict(label_smoothing=0.1)):
        o = _opts(O, class_weight=cw, **feats)
        r = O.forward_backward(x, w, b, t, o)
        for k in range(directions):
            if k % 2 == 0:
                dv = rng.standard_normal(x.shape)
                dv /= np.linalg.norm(dv)
                fd = (O.forward(x + h * dv, w, b, t, o).loss - O.forward(x - h * dv, w, b, t, o).loss) / (2 * h)
                an, gn = float((r.dx * dv).sum()), np.linalg.norm(r.dx)
            else:
                dv = rng.standard_normal(w.shape)
                dv /= np.linalg.norm(dv)
                fd = (O.forward(x, w + h * dv, b, t, o).loss - O.forward(x, w - h * dv, b, t, o).loss) / (2 * h)
                an, gn = float((r.dw * dv).sum()), np.linalg.norm(r.dw)
            assert abs(fd - an) <= 1e-7 * gn + 1e-12, (feats, k, fd, an)


def pin_gradient_columns(O):
    """Columns of G from only those columns of the logits equal the columns
    of the full G (every feature set, class weights, unsorted and repeated
    target columns) and torch's autograd gradient of its cross-entropy."""
    import torch
    import torch.nn.functional as F

    x, w, b, t = _problem(n=30, d=12, v=37, seed=17, bias=True)
    v = w.shape[0]
    cols = np.array([0, 5, int(t[t >= 0][0]), 36, 11, int(t[t >= 0][1])])
    cw = np.random.default_rng(4).uniform(0.2, 2.0, v)
    for feats in FEATURE_SETS + [dict(class_weight=cw), dict(class_weight=cw, label_smoothing=0.1,
                                                             lse_square_scale=1e-2, softcap=2.0)]:
        o = _opts(O, **{k: val for k, val in feats.items() if k != "reduction"})
        z = O.logits(x, w, b, o.softcap)
        lse = O.log_sum_exp(z)
        full = O.grad_logits(z, lse, t, o)
        part = O.grad_logits_columns(z[:, cols], cols, v, lse, t, o)
        assert np.allclose(part, full[:, cols], rtol=1e-13, atol=1e-15), feats
    for eps in (0.0, 0.15):
        o = _opts(O, label_smoothing=eps)
        z = O.logits(x, w, b, 0.0)
        zt = torch.tensor(z, requires_grad=True)
        tt = torch.tensor(t, dtype=torch.long)
        F.cross_entropy(zt, tt, ignore_index=IGN, label_smoothing=eps, reduction="sum").backward()
        part = O.grad_logits_columns(z[:, cols], cols, v, O.log_sum_exp(z), t, o)
        assert np.allclose(part, zt.grad.numpy()[:, cols], rtol=1e-12, atol=1e-14), eps


def pin_target_validation(O):
    """Targets outside [0, V) that are not ignore_index are refused; the
    ignore index itself is accepted even when it lies inside [0, V), and then
    those rows are the ignored ones."""
    x, w, b, t = _problem(n=12, d=8, v=10, seed=4, ignore=0)
    for bad in (10, -3):
        tb = t.copy()
        tb[5] = bad
        try:
            O.forward(x, w, b, tb, _opts(O))
        except ValueError:
            pass
        else:
            raise AssertionError(f"target {bad} accepted")
    o = _opts(O, ignore_index=3)
    t2 = t.copy()
    t2[:4] = 3
    r = O.forward(x, w, b, t2, o)
    assert np.all(r.row_loss[t2 == 3] == 0.0) and r.n_valid == int((t2 != 3).sum())


def pin_bf16_widening(O):
    """The exact widening of stored bf16 bit patterns (uint16) agrees with
    torch's bfloat16 -> float64 conversion on random values and on zeros,
    infinities, the largest and smallest normals and subnormals; fp32 arrays
    widen unchanged."""
    import torch
    g = torch.Generator().manual_seed(13)
    vals = torch.cat([torch.randn(4096, generator=g) * 10.0 ** torch.randint(-30, 30, (4096,), generator=g),
                      torch.tensor([0.0, -0.0, float("inf"), float("-inf"), 3.3895e38, -3.3895e38,
                                    1.1755e-38, 9.2e-41, -9.2e-41, 1.0, -2.0])])
    b = vals.to(torch.bfloat16)
    bits = b.view(torch.int16).numpy().view(np.uint16)
    got = O.to_f64(bits)
    want = b.to(torch.float64).numpy()
    assert got.dtype == np.float64
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))
    f = np.random.default_rng(3).standard_normal(100).astype(np.float32)
    assert np.array_equal(O.to_f64(f), f.astype(np.float64))
    assert O.to_f64(None) is None


ALL_PINS = [
    pin_uniform_logits, pin_single_class, pin_two_classes, pin_gradient_row_sums,
    pin_shift_invariance, pin_batch_additivity, pin_vocab_permutation,
    pin_online_merge, pin_no_valid_rows, pin_softcap_limits,
    pin_torch_cross_entropy, pin_finite_differences, pin_brute_force,
    pin_gaussian_lse_level, pin_logits_identity_linear, pin_logits_torch,
    pin_logits_finite_differences, pin_megatron_smoothing, pin_predicted_tokens,
    pin_class_weight_torch, pin_class_weight_unit_and_fd, pin_bf16_widening,
    pin_target_validation, pin_gradient_columns,
]
