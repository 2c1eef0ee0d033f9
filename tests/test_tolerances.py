"""The GPU parity tests' comparison helpers, on the CPU: the gradient bar
(element bound with its column floor, column norm bound, fixed-point slack)
rejects what it must, including a NaN on one side only."""
import numpy as np
import pytest

from gpu_util import assert_colour_close, assert_grad_close, assert_stats_close, grad_ratios


def _grads(seed=0, n=200):
    rng = np.random.default_rng(seed)
    g = rng.normal(size=(n, 12)) * np.logspace(-6, -2, 12)[None, :]
    g[:, 10:] = 0.0
    return g


def test_grad_bar_accepts_small_errors():
    ref = _grads()
    gpu = ref * (1 + 0.5e-4 * np.sign(np.random.default_rng(1).normal(size=ref.shape)))
    assert_grad_close(gpu.astype(np.float64), ref, "half the bar")


def test_grad_bar_rejects_one_large_relative_error():
    ref = _grads()
    gpu = ref.copy()
    k = np.argmax(np.abs(ref[:, 3]))
    gpu[k, 3] *= 1 + 2e-4
    with pytest.raises(AssertionError, match="out of tolerance"):
        assert_grad_close(gpu, ref, "one entry at twice the bar")


def test_grad_bar_floor_is_relative_to_the_column_maximum():
    ref = _grads()
    ref[5, 2] = 1e-9 * np.abs(ref[:, 2]).max()
    gpu = ref.copy()
    gpu[5, 2] += 0.5 * 1e-4 * 1e-3 * np.abs(ref[:, 2]).max()  # below the floor's bound
    assert_grad_close(gpu, ref, "tiny entry within the floor")
    gpu[5, 2] += 1e-4 * 1e-3 * np.abs(ref[:, 2]).max()  # now 1.5x the floor's bound
    with pytest.raises(AssertionError, match="out of tolerance"):
        assert_grad_close(gpu, ref, "tiny entry past the floor")


def test_grad_bar_rejects_a_column_norm_error():
    ref = _grads()
    gpu = ref * (1 + 0.99e-4)  # every element and the column norm at 0.99 of the bound
    assert_grad_close(gpu, ref, "uniform 0.99e-4")
    ratio, norm = grad_ratios(gpu, ref)
    assert np.all(ratio <= 1.0) and np.all(norm < 1.0)
    # one site carries the column's only non-zero gradient; the others, at
    # zero, may each be off by up to the floor's 1e-4 x 1e-3 of it, yet the
    # sum of squares of ~1.1M such errors exceeds 1e-4 of the column norm
    n = 1_100_000
    ref2 = np.zeros((n, 10))
    ref2[0, :] = 1.0
    gpu2 = ref2.copy()
    gpu2[1:, 4] = 0.99e-7
    ratio, norm = grad_ratios(gpu2, ref2)
    assert ratio.max() <= 1.0 and norm[4] > 1.0
    with pytest.raises(AssertionError, match="norm error"):
        assert_grad_close(gpu2, ref2, "many errors at the floor")


def test_grad_bar_rejects_nan_on_one_side():
    ref = _grads()
    gpu = ref.copy()
    gpu[7, 0] = np.nan
    with pytest.raises(AssertionError):
        assert_grad_close(gpu, ref, "NaN from the GPU")
    gpu = ref.copy()
    ref_nan = ref.copy()
    ref_nan[7, 0] = np.nan
    with pytest.raises(AssertionError):
        assert_grad_close(gpu, ref_nan, "NaN from the oracle")
    gpu[7, 0] = np.nan
    assert_grad_close(gpu, ref_nan, "NaN on both sides")


def test_grad_bar_rejects_infinities():
    ref = _grads()
    gpu = ref.copy()
    gpu[3, 8] = np.inf
    with pytest.raises(AssertionError):
        assert_grad_close(gpu, ref, "inf from the GPU")


def test_grad_bar_fixed_point_slack_counts_listings():
    ref = _grads(n=4)
    topk = np.full((2, 2, 8), 0xFFFFFFFF, np.uint32)
    topk[0, 0, 0] = 1
    topk[0, 1, 0] = 1
    gpu = ref.copy()
    gpu[1, :10] += 1.5 * 1e-4 * np.maximum(np.abs(ref[1, :10]), 1e-3 * np.abs(ref[:, :10]).max(0))
    with pytest.raises(AssertionError):
        assert_grad_close(gpu, ref, "no slack")
    res = np.abs(ref[:, :10]).max() * 1e-3  # two listings of site 1 x res covers the excess
    assert_grad_close(gpu, ref, "slack", topk, (2, 2), res)


def test_stats_and_colour_checks_reject_nan():
    ref = np.ones((3, 8))
    gpu = ref.copy()
    gpu[1, 1] = np.nan
    topk = np.zeros((1, 1, 8), np.uint32)
    with pytest.raises(AssertionError):
        assert_stats_close(gpu, ref, np.ones_like(ref), topk, (1, 1))
    img = np.zeros((2, 2, 3))
    bad = img.copy()
    bad[0, 0, 0] = np.nan
    with pytest.raises(AssertionError):
        assert_colour_close(bad.astype(np.float32), img)
