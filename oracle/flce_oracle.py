"""Plain fp64 CPU oracle for fused linear cross-entropy (FLCE).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library.

What it computes is the plain definition of the loss on materialised logits,
because the fused method reaches exactly that result (up to rounding order) and
only avoids storing the [N, V] logits:

* page "Cutting LLM Memory by 84%: A Deep Dive into Fused Kernels",
  section "The maths behind Fused Linear Cross-Entropy / Definition and Forward
  Pass": with a one-hot target the cross-entropy of softmax(x.W) collapses to
  LSE(logits) - (target logit), evaluated with the row maximum subtracted;
* same page, "Backward Pass": matmul gradients dX = G.W^T, dW = X^T.G
  (section "Matrix Multiplication"), the cross-entropy gradient
  softmax - onehot (section "Cross-Entropy"), their chain-rule product
  (section "Fused Linear Cross-Entropy") and the batch reduction of the weight
  gradient by sum or mean (the note that closes that section);
* same page, "Kernel Implementation", step 1: rows whose target equals
  ignore_index (default -100) contribute a loss of 0;
* page "[CuteDSL] FLCE: 2-SM online-softmax fast path (Blackwell)" (Liger-Kernel
  PR #1291), Summary: the option set bias, softcap, label_smoothing, z-loss
  (lse_square_scale), ignore_index, mean/sum reduction and forward-only
  reduction='none';
* page "Add efficient Cross-Entropy by cuda kernel" (TransformerEngine PR #995),
  review of the backward kernel: label smoothing subtracts a uniform term from
  the softmax gradient.

Readings taken where the pages are silent or their equations were lost (every
displayed equation of the first page is missing from the extracted text):

* W is stored [V, D] (nn.Linear layout); logits r = X.W^T + b.
* softcap c > 0: z = c * tanh(r / c), applied after the bias and before the
  LSE, target logit, smoothing and z-loss; c <= 0 means off.
* label smoothing eps: target distribution q = (1 - eps) onehot + eps / V
  (PyTorch convention; the Megatron form on the TransformerEngine page is the
  same family with eps' = eps V / (V - 1)).
* z-loss: + s * lse^2 per valid row, reduced like the cross-entropy term.
* mean divides by n_valid (rows whose target is not ignore_index); with
  n_valid = 0 the loss and every gradient are 0.
* ignored rows report lse = 0 and row_loss = 0.
* grad_output g scales every gradient; scale = g / n_valid (mean) or g (sum).
* class weights w [V] (option ``class_weight``; page "[CuteDSL] FLCE",
  Summary, names ce_weight): torch's weighted cross-entropy, i.e. row loss
  (1-eps) w_t (lse - z_t) + (eps/V) sum_c w_c (lse - z_c), the mean taken over
  sum_valid w_t instead of n_valid; the z-loss term is weighted by w_t too (so
  w = 1 is the unweighted loss).

Parity status of each function is stated in its docstring; every function is
pinned by tests in ``tests/test_oracle_pins.py`` except where a docstring says
"parity unpinned".
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

ROW_BLOCK = 1024


@dataclasses.dataclass(frozen=True)
class LossOptions:
    ignore_index: int = -100
    label_smoothing: float = 0.0
    lse_square_scale: float = 0.0
    softcap: float = 0.0
    reduction: str = "mean"
    class_weight: object = None      # [V] per-class weights, or None


# --------------------------------------------------------------------- inputs

def to_f64(a: Optional[np.ndarray]) -> Optional[np.ndarray]:
    """Exact widening of the stored inputs: uint16 arrays hold bf16 bit
    patterns (the upper half of an IEEE fp32), float arrays widen as is."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        wide = a.astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------- pieces

def logits(x: np.ndarray, w: np.ndarray, bias: Optional[np.ndarray],
           softcap: float) -> np.ndarray:
    """Logits of a block of rows: z = X.W^T (+ b), then the optional softcap
    z = c tanh(z / c).  Pinned: closed forms at W = 0, the torch special case,
    finite differences, brute force."""
    r = x @ w.T
    if bias is not None:
        r = r + bias[None, :]
    if softcap > 0.0:
        r = softcap * np.tanh(r / softcap)
    return r


def log_sum_exp(z: np.ndarray) -> np.ndarray:
    """Row-wise LSE with the row maximum subtracted first (numerically stable
    softmax, page "Cutting LLM Memory by 84%", "Definition and Forward
    Pass").  Pinned: ln V at W = 0, the online merge, brute force."""
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def log_sum_exp_online(z: np.ndarray, block: int) -> np.ndarray:
    """The same LSE reached by the online-softmax recurrence over vocabulary
    blocks (page "Cutting LLM Memory by 84%", "Definition and Forward Pass",
    step 2: a running maximum m and a running sum of exponentials d, the sum
    rescaled by exp(m_old - m_new) whenever the maximum grows).  Used only to
    pin the merge rule that the GPU epilogue relies on."""
    n, v = z.shape
    m = np.full(n, -np.inf)
    d = np.zeros(n)
    for v0 in range(0, v, block):
        blk = z[:, v0:v0 + block]
        m_new = np.maximum(m, blk.max(axis=1))
        d = d * np.exp(m - m_new) + np.exp(blk - m_new[:, None]).sum(axis=1)
        m = m_new
    return m + np.log(d)


def valid_rows(targets: np.ndarray, opts: LossOptions) -> np.ndarray:
    return np.asarray(targets) != opts.ignore_index


def mean_denominator(targets: np.ndarray, opts: LossOptions) -> float:
    """What 'mean' divides by: n_valid, or with class weights the sum of the
    valid rows' target weights."""
    valid = valid_rows(targets, opts)
    if opts.class_weight is None:
        return int(valid.sum())
    w = np.asarray(opts.class_weight, dtype=np.float64)
    return float(w[np.asarray(targets)[valid]].sum())


def check_targets(targets: np.ndarray, v: int, opts: LossOptions) -> None:
    t = np.asarray(targets)
    bad = (t != opts.ignore_index) & ((t < 0) | (t >= v))
    if bad.any():
        raise ValueError("target outside [0, V) and not ignore_index")


def row_losses(z: np.ndarray, lse: np.ndarray, targets: np.ndarray,
               opts: LossOptions) -> np.ndarray:
    """Per-row loss of valid rows: the cross-entropy between the smoothed
    target distribution q = (1-eps) onehot_t + eps/V and softmax(z),
    -sum_v q_v (z_v - lse) = lse - (1-eps) z_t - (eps/V) sum_v z_v, plus the
    z-loss s lse^2.  Ignored rows get 0."""
    n, v = z.shape
    valid = valid_rows(targets, opts)
    t = np.where(valid, targets, 0)
    zt = z[np.arange(n), t]
    eps = opts.label_smoothing
    if opts.class_weight is not None:
        w = np.asarray(opts.class_weight, dtype=np.float64)
        wt = w[t]
        out = (1.0 - eps) * wt * (lse - zt)
        if eps != 0.0:
            out = out + (eps / v) * (w.sum() * lse - z @ w)
        if opts.lse_square_scale != 0.0:
            out = out + opts.lse_square_scale * wt * lse * lse
        return np.where(valid, out, 0.0)
    out = lse - (1.0 - eps) * zt
    if eps != 0.0:
        out = out - (eps / v) * z.sum(axis=1)
    if opts.lse_square_scale != 0.0:
        out = out + opts.lse_square_scale * lse * lse
    return np.where(valid, out, 0.0)


def grad_logits(z: np.ndarray, lse: np.ndarray, targets: np.ndarray,
                opts: LossOptions) -> np.ndarray:
    """d(row_loss)/d(pre-softcap logit), unscaled:
    G = [softmax(z) (1 + 2 s lse) - (1-eps) onehot_t - eps/V] * dz/dr, with
    dz/dr = 1 - (z/c)^2 under the softcap; zero rows for ignored targets.
    (page "Cutting LLM Memory by 84%", "Cross-Entropy": prediction minus
    ground truth.)  Pinned: finite differences, torch autograd, row sums."""
    n, v = z.shape
    valid = valid_rows(targets, opts)
    t = np.where(valid, targets, 0)
    p = np.exp(z - lse[:, None])
    s = opts.lse_square_scale
    if opts.class_weight is not None:
        # d/dz_c of the weighted row: p_c [(1-eps) w_t + (eps/V) sum w + 2 s w_t lse]
        #   - (1-eps) w_t [c = t] - (eps/V) w_c
        w = np.asarray(opts.class_weight, dtype=np.float64)
        wt = w[t]
        eps = opts.label_smoothing
        fac = (1.0 - eps) * wt + (eps / v) * w.sum() + 2.0 * s * wt * lse
        g = p * fac[:, None]
        g[np.arange(n), t] -= (1.0 - eps) * wt
        if eps != 0.0:
            g -= (eps / v) * w[None, :]
        if opts.softcap > 0.0:
            g *= 1.0 - (z / opts.softcap) ** 2
        g[~valid] = 0.0
        return g
    g = p * (1.0 + 2.0 * s * lse)[:, None] if s != 0.0 else p
    g[np.arange(n), t] -= (1.0 - opts.label_smoothing)
    if opts.label_smoothing != 0.0:
        g -= opts.label_smoothing / v
    if opts.softcap > 0.0:
        g *= 1.0 - (z / opts.softcap) ** 2
    g[~valid] = 0.0
    return g


def grad_logits_columns(z_cols: np.ndarray, cols: np.ndarray, v: int, lse: np.ndarray,
                        targets: np.ndarray, opts: LossOptions) -> np.ndarray:
    """Columns ``cols`` of ``grad_logits`` when only those columns of the
    rows' final logits are held: ``z_cols = z[:, cols]``, ``lse`` the rows'
    full LSE and ``v`` the vocabulary size.  The same formula column by
    column: p_c = exp(z_c - lse) times (1 + 2 s lse), less (1 - eps) where
    c is the target, less eps / V, times 1 - (z_c / c)^2 under the softcap;
    with class weights the weighted form of ``grad_logits``.  Lets a test
    check a few rows of dW = G^T X over a whole batch without the [N, V]
    logits.  Pinned: equals the columns of ``grad_logits`` and of torch's
    autograd gradient."""
    cols = np.asarray(cols)
    n = z_cols.shape[0]
    valid = valid_rows(targets, opts)
    t = np.where(valid, targets, -1)
    hit = t[:, None] == cols[None, :]
    p = np.exp(z_cols - lse[:, None])
    s = opts.lse_square_scale
    eps = opts.label_smoothing
    if opts.class_weight is not None:
        w = np.asarray(opts.class_weight, dtype=np.float64)
        wt = w[np.where(valid, targets, 0)]
        fac = (1.0 - eps) * wt + (eps / v) * w.sum() + 2.0 * s * wt * lse
        g = p * fac[:, None] - np.where(hit, ((1.0 - eps) * wt)[:, None], 0.0)
        g = g - (eps / v) * w[cols][None, :]
    else:
        g = p * (1.0 + 2.0 * s * lse)[:, None] - np.where(hit, 1.0 - eps, 0.0) - eps / v
    if opts.softcap > 0.0:
        g = g * (1.0 - (z_cols / opts.softcap) ** 2)
    g[~valid] = 0.0
    assert g.shape == (n, len(cols))
    return g


def grad_scale(opts: LossOptions, n_valid: int, grad_output: float) -> float:
    """Scale from the unscaled per-row gradient to d(loss): g / n_valid for
    mean (0 when no row is valid), g for sum.  reduction 'none' has no
    backward (refused, page "[CuteDSL] FLCE", Summary)."""
    if opts.reduction == "mean":
        return grad_output / n_valid if n_valid > 0 else 0.0
    if opts.reduction == "sum":
        return grad_output
    raise ValueError("reduction='none' has no backward")


def reduce_loss(row_loss: np.ndarray, n_valid: int, opts: LossOptions):
    if opts.reduction == "mean":
        return float(row_loss.sum() / n_valid) if n_valid > 0 else 0.0
    if opts.reduction == "sum":
        return float(row_loss.sum())
    if opts.reduction == "none":
        return row_loss.copy()
    raise ValueError(f"unknown reduction {opts.reduction!r}")


# ------------------------------------------------------------- whole problem

@dataclasses.dataclass
class Result:
    loss: object                     # float, or [N] array for 'none'
    lse: np.ndarray                  # [N], 0 on ignored rows
    row_loss: np.ndarray             # [N]
    n_valid: int
    dx: Optional[np.ndarray] = None  # [N, D]
    dw: Optional[np.ndarray] = None  # [V, D]
    db: Optional[np.ndarray] = None  # [V]


def forward(x, w, bias, targets, opts: LossOptions,
            n_valid: Optional[int] = None, row_block: int = ROW_BLOCK) -> Result:
    """Loss, per-row LSE and per-row loss.  ``n_valid`` overrides the mean
    denominator (sampled rows of a larger batch use the full batch's count,
    or with class weights its sum of target weights)."""
    x, w, bias = to_f64(x), to_f64(w), to_f64(bias)
    targets = np.asarray(targets)
    check_targets(targets, w.shape[0], opts)
    n = x.shape[0]
    valid = valid_rows(targets, opts)
    nv = mean_denominator(targets, opts) if n_valid is None else n_valid
    lse = np.zeros(n)
    rl = np.zeros(n)
    for r0 in range(0, n, row_block):
        sl = slice(r0, min(n, r0 + row_block))
        z = logits(x[sl], w, bias, opts.softcap)
        l = log_sum_exp(z)
        rl[sl] = row_losses(z, l, targets[sl], opts)
        lse[sl] = np.where(valid[sl], l, 0.0)
    return Result(reduce_loss(rl, nv, opts), lse, rl, nv)


def forward_backward(x, w, bias, targets, opts: LossOptions,
                     grad_output: float = 1.0, n_valid: Optional[int] = None,
                     want_dw: bool = True, row_block: int = ROW_BLOCK) -> Result:
    """Forward plus dX = scale G.W, dW = scale G^T.X and db = scale sum_n G,
    logits computed once per block of rows (page "Cutting LLM Memory by 84%",
    "Fused Linear Cross-Entropy": the chain rule through the linear layer)."""
    x, w, bias = to_f64(x), to_f64(w), to_f64(bias)
    targets = np.asarray(targets)
    check_targets(targets, w.shape[0], opts)
    n, d = x.shape
    v = w.shape[0]
    valid = valid_rows(targets, opts)
    nv = mean_denominator(targets, opts) if n_valid is None else n_valid
    scale = grad_scale(opts, nv, grad_output)
    lse = np.zeros(n)
    rl = np.zeros(n)
    dx = np.zeros((n, d))
    dw = np.zeros((v, d)) if want_dw else None
    db = np.zeros(v)
    for r0 in range(0, n, row_block):
        sl = slice(r0, min(n, r0 + row_block))
        z = logits(x[sl], w, bias, opts.softcap)
        l = log_sum_exp(z)
        rl[sl] = row_losses(z, l, targets[sl], opts)
        lse[sl] = np.where(valid[sl], l, 0.0)
        g = grad_logits(z, l, targets[sl], opts) * scale
        dx[sl] = g @ w
        if want_dw:
            dw += g.T @ x[sl]
        db += g.sum(axis=0)
    return Result(reduce_loss(rl, nv, opts), lse, rl, nv, dx, dw, db)


# ------------------------------------------------- cross-entropy on logits

def cross_entropy_on_logits(r, targets, opts: LossOptions, grad_output: float = 1.0,
                            n_valid: Optional[int] = None, want_grad: bool = True,
                            row_block: int = ROW_BLOCK) -> Result:
    """The same loss on logits given directly (no linear layer): the forward
    "sum-exp" and "mean-log" passes and the backward of the cross-entropy
    kernels on materialised logits (page "Add efficient Cross-Entropy by cuda
    kernel", TransformerEngine PR #995: Changes, and the review of the
    backward kernel, where smoothing subtracts a uniform term).  ``r`` holds
    the pre-softcap logits [N, V] (bf16 bit patterns or floats); the result's
    ``dx`` field carries dL/dr = scale * G.  Same readings as the fused
    problem; the smoothing eps is the PyTorch one (the Megatron form on that
    page is eps' = eps V / (V - 1), see ``megatron_smoothing``).  Pinned:
    equals ``forward_backward`` with X = r and W = identity, torch's
    cross_entropy with autograd, finite differences, the Megatron form."""
    r = to_f64(r)
    targets = np.asarray(targets)
    n, v = r.shape
    check_targets(targets, v, opts)
    valid = valid_rows(targets, opts)
    nv = mean_denominator(targets, opts) if n_valid is None else n_valid
    scale = grad_scale(opts, nv, grad_output) if want_grad else 0.0
    lse = np.zeros(n)
    rl = np.zeros(n)
    grad = np.zeros((n, v)) if want_grad else None
    for r0 in range(0, n, row_block):
        sl = slice(r0, min(n, r0 + row_block))
        z = r[sl]
        if opts.softcap > 0.0:
            z = opts.softcap * np.tanh(z / opts.softcap)
        l = log_sum_exp(z)
        rl[sl] = row_losses(z, l, targets[sl], opts)
        lse[sl] = np.where(valid[sl], l, 0.0)
        if want_grad:
            grad[sl] = grad_logits(z, l, targets[sl], opts) * scale
    return Result(reduce_loss(rl, nv, opts), lse, rl, nv, dx=grad)


def megatron_smoothing(eps: float, v: int) -> float:
    """The smoothing factor of the Megatron cross-entropy that the
    TransformerEngine kernels follow (review of the backward kernel there:
    smoothing = label_smoothing * V / (V - 1)); with it the target keeps
    1 - eps and every other class gets eps / (V - 1).  Under this module's
    convention that is the target distribution of eps' = eps V / (V - 1)."""
    return eps * v / (v - 1)


# ------------------------------------------------- predicted tokens, accuracy

def predicted_tokens(z: np.ndarray, targets: np.ndarray, opts: LossOptions) -> np.ndarray:
    """Argmax over the vocabulary of each row's final logits z (after bias and
    softcap), the lowest index among equal maxima; -1 on ignored rows (page
    "[CuteDSL] FLCE", Summary: the predicted-tokens and token-accuracy
    outputs of the option set; the pages give no formula, this is the plain
    reading).  Pinned: brute force, ties at W = 0, torch.argmax, invariance
    under the (monotonic) softcap."""
    pred = np.argmax(z, axis=1).astype(np.int32)     # first occurrence of the maximum
    return np.where(valid_rows(targets, opts), pred, -1).astype(np.int32)


def token_accuracy(pred: np.ndarray, targets: np.ndarray, opts: LossOptions,
                   n_valid: Optional[int] = None) -> float:
    """Fraction of valid rows whose predicted token is the target (0 when no
    row is valid)."""
    valid = valid_rows(targets, opts)
    nv = int(valid.sum()) if n_valid is None else int(n_valid)
    hits = int(((pred == np.asarray(targets)) & valid).sum())
    return hits / nv if nv > 0 else 0.0


def forward_metrics(x, w, bias, targets, opts: LossOptions,
                    row_block: int = ROW_BLOCK) -> Tuple[np.ndarray, float]:
    """(predicted tokens [N], token accuracy) of the fused problem."""
    x, w, bias = to_f64(x), to_f64(w), to_f64(bias)
    targets = np.asarray(targets)
    pred = np.empty(x.shape[0], dtype=np.int32)
    for r0 in range(0, x.shape[0], row_block):
        sl = slice(r0, min(x.shape[0], r0 + row_block))
        pred[sl] = predicted_tokens(logits(x[sl], w, bias, opts.softcap), targets[sl], opts)
    return pred, token_accuracy(pred, targets, opts)


def logits_metrics(r, targets, opts: LossOptions) -> Tuple[np.ndarray, float]:
    """(predicted tokens [N], token accuracy) on logits given directly."""
    z = to_f64(r)
    if opts.softcap > 0.0:
        z = opts.softcap * np.tanh(z / opts.softcap)
    targets = np.asarray(targets)
    pred = predicted_tokens(z, targets, opts)
    return pred, token_accuracy(pred, targets, opts)
