"""The predicted-token check of the GPU tests, on the CPU: it accepts a
prediction that differs from the fp64 argmax only inside the fp32 near-tie
window and only on a few rows, and rejects a second-best prediction outside
the window, too many near-tie rows, and ignored rows that predict a class."""
import numpy as np
import pytest

from oracle import flce_oracle as O
from tests import gpu_utils as U


def logits(n=400, v=300, seed=0, scale=3.0):
    return np.random.default_rng(seed).standard_normal((n, v)) * scale


def test_window_scales_with_the_logits():
    assert U.tie_window(1.0) == pytest.approx(256 * 2.0 ** -23)
    assert U.tie_window(1000.0) == pytest.approx(256 * 2.0 ** -14)
    assert U.tie_window(1.0, softcap=30.0) > U.tie_window(1.0)


def test_exact_predictions_pass():
    z = logits()
    t = np.argmax(z, axis=1).astype(np.int32)
    t[::5] = -100
    pred = np.where(t == -100, -1, np.argmax(z, axis=1)).astype(np.int32)
    acc = float(((pred == t) & (t != -100)).sum() / (t != -100).sum())
    assert U.check_predictions(pred, acc, z, t, O.LossOptions()) == 0


def _near_tie(z, row, delta):
    """Make the second-best class of `row` trail the best by `delta`."""
    order = np.argsort(z[row])
    best, second = order[-1], order[-2]
    z[row, second] = z[row, best] - delta
    return best, second


def test_second_best_inside_the_window_passes():
    z = logits()
    best, second = _near_tie(z, 7, 0.25 * U.tie_window(np.abs(z).max()))
    t = np.zeros(len(z), dtype=np.int32)
    pred = np.argmax(z, axis=1).astype(np.int32)
    pred[7] = second
    acc = float((pred == t).mean())
    assert U.check_predictions(pred, acc, z, t, O.LossOptions()) == 1


def test_second_best_outside_the_window_is_rejected():
    z = logits()
    w = U.tie_window(np.abs(z).max())
    best, second = _near_tie(z, 7, 4.0 * w)       # a near-tie by the old 1e-3 max|z| rule, not by fp32's
    assert 4.0 * w < 1e-3 * np.abs(z).max()
    t = np.zeros(len(z), dtype=np.int32)
    pred = np.argmax(z, axis=1).astype(np.int32)
    pred[7] = second
    with pytest.raises(AssertionError, match="outside the near-tie window"):
        U.check_predictions(pred, float((pred == t).mean()), z, t, O.LossOptions())


def test_too_many_near_tie_rows_are_rejected():
    z = logits(n=400)
    w = U.tie_window(np.abs(z).max())
    pred = np.argmax(z, axis=1).astype(np.int32)
    for row in range(3):                          # cap is max(2, 0.1% of 400 rows) = 2
        _, pred[row] = _near_tie(z, row, 0.1 * w)
    t = np.zeros(len(z), dtype=np.int32)
    with pytest.raises(AssertionError, match="rows differ"):
        U.check_predictions(pred, float((pred == t).mean()), z, t, O.LossOptions())


def test_ignored_rows_must_predict_minus_one():
    z = logits()
    t = np.zeros(len(z), dtype=np.int32)
    t[3] = -100
    pred = np.argmax(z, axis=1).astype(np.int32)
    with pytest.raises(AssertionError, match="ignored rows"):
        U.check_predictions(pred, 0.0, z, t, O.LossOptions())


def test_blockwise_gaps_match_the_dense_ones():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((70, 16))
    w = rng.standard_normal((50, 16))
    b = rng.standard_normal(50)
    pred = rng.integers(0, 50, 70)
    ref, gap, zabs = U.fp64_argmax_gaps(x, w, b, 5.0, pred, row_block=16)
    z = O.logits(x, w, b, 5.0)
    assert np.array_equal(ref, np.argmax(z, axis=1))
    assert np.allclose(gap, z[np.arange(70), ref] - z[np.arange(70), pred])
    assert zabs == pytest.approx(np.abs(z).max())
