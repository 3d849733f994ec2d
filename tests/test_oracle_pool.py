"""Pins of oracle.pool (SnapKV 1D pooling) against library routines and closed forms."""

import numpy as np
import pytest
from scipy.ndimage import maximum_filter1d

import oracle
from oracle.pool import AVG, MAX


@pytest.mark.parametrize("kernel", [1, 3, 7, 31])
def test_avg_is_box_convolution(kernel):
    # zero-padded box filter / k == numpy's 'same' convolution with ones(k)/k
    x = np.random.default_rng(kernel).standard_normal(200)
    ref = np.convolve(x, np.ones(kernel) / kernel, mode="same")
    assert np.allclose(oracle.pool.pool_row(x, kernel, AVG), ref, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("kernel", [1, 5, 9, 63])
def test_max_is_maximum_filter(kernel):
    x = np.random.default_rng(100 + kernel).standard_normal(300)
    ref = maximum_filter1d(x, size=kernel, mode="constant", cval=-np.inf)
    assert np.array_equal(oracle.pool.pool_row(x, kernel, MAX), ref)


def test_closed_forms():
    n, k = 50, 7
    c = np.full(n, 0.25)
    avg = oracle.pool.pool_row(c, k, AVG)
    assert np.allclose(avg[3:-3], 0.25)                          # interior keeps the constant
    assert np.allclose(avg[:3], 0.25 * np.array([4, 5, 6]) / 7)   # zero padding at the edge
    hot = np.zeros(n)
    hot[20] = 1.0
    mx = oracle.pool.pool_row(hot, k, MAX)
    assert np.array_equal(np.nonzero(mx)[0], np.arange(17, 24))   # plateau of width k
    # kernel 1 is the identity; pooling preserves a head's total up to edge losses
    x = np.random.default_rng(3).random(n)
    assert np.array_equal(oracle.pool.pool_row(x, 1, AVG), x)
    assert np.array_equal(oracle.pool.pool_row(x, 1, MAX), x)
    y = np.zeros(n)
    y[10:40] = np.random.default_rng(4).random(30)
    assert np.isclose(oracle.pool.pool_row(y, k, AVG).sum(), y.sum())


def test_rejects_even_kernel():
    with pytest.raises(ValueError):
        oracle.pool.pool_row(np.zeros(4), 4, AVG)


@pytest.mark.parametrize("mode", [AVG, MAX])
@pytest.mark.parametrize("lead", [(2, 3), (3,)])
def test_pool_multi_row_keeps_each_row_apart(mode, lead):
    # importance [2, 3, n] (layers, heads) or [3, n] (heads): row r holds one spike of
    # height r+1 at its own position p = 7r + 3, so each pooled row must show that row's
    # plateau [p - h, p + h] at that row's height (ZigZagKV page, SnapKV section: pooling
    # runs along the keys of each head separately), nothing else, and the shape is kept.
    n, k = 40, 5
    h = k // 2
    x = np.zeros(lead + (n,))
    rows = x.reshape(-1, n)
    for r in range(rows.shape[0]):
        rows[r, 7 * r + 3] = r + 1
    out = oracle.pool.pool(x, k, mode)
    assert out.shape == x.shape
    got = out.reshape(-1, n)
    for r in range(rows.shape[0]):
        p, v = 7 * r + 3, r + 1
        want = np.zeros(n)
        want[p - h:p + h + 1] = v / k if mode == AVG else v
        assert np.allclose(got[r], want, rtol=0, atol=1e-15), r


def test_pool_single_row_input_stays_one_dimensional():
    x = np.arange(9, dtype=np.float64)
    out = oracle.pool.pool(x, 3, AVG)
    assert out.shape == (9,)
    assert np.allclose(out[1:-1], x[1:-1])          # a linear ramp is kept by a centred box
    assert np.isclose(out[0], (0 + 1) / 3) and np.isclose(out[-1], (7 + 8) / 3)
