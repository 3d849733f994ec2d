"""Pins for the oracle's threshold selection and packed gather (CPU only).

* Top-k equivalence: with distinct scores, theta = the k-th largest candidate
  score keeps exactly the set the (independently written) top-k selection
  keeps with budget k + r.
* Closed form: scores a * rho^j in a shuffled order keep
  floor(log(theta / a) / log(rho)) + 1 candidates, the largest ones.
* Extremes: theta = -inf keeps every candidate, +inf only the recent window;
  raising theta never adds a position; a score equal to theta is kept, NaN
  never; the window tokens between S - w and S - r are never candidates.
* The kept count follows the prompt (the page's dynamic ratio): at one theta a
  flat score row keeps every candidate and a peaked one keeps few.
* Packed gather against the per-head gather of ``compact``.
"""

import math

import numpy as np
import pytest

from oracle import compact, select, threshold


def _distinct_scores(rng, n):
    return rng.permutation(np.linspace(1.0, 2.0, n)) * rng.uniform(0.5, 1.5)


@pytest.mark.parametrize("S,w,recent,k", [(300, 20, 20, 37), (257, 16, 40, 1), (500, 64, 8, 200), (64, 8, 0, 56)])
def test_topk_equivalence(S, w, recent, k):
    rng = np.random.default_rng(S + k)
    c = select.candidates(S, w, recent)
    v = _distinct_scores(rng, c)
    theta = np.sort(v)[::-1][k - 1]
    got = threshold.select_threshold(v, S=S, w=w, recent=recent, theta=theta)
    ref = select.select(v, S=S, w=w, recent=recent, budget=k + recent)
    assert np.array_equal(np.sort(got), ref)
    assert np.all(np.diff(got) > 0)


def test_geometric_closed_form():
    rng = np.random.default_rng(5)
    a, rho, c = 1.0, 0.5, 40
    perm = rng.permutation(c)
    v = np.empty(c, dtype=np.float32)
    v[perm] = (a * rho ** np.arange(c)).astype(np.float32)        # exact in float32
    for theta in [0.01, 0.3, 0.9, 1e-9]:
        cnt = min(c, math.floor(math.log(theta / a) / math.log(rho)) + 1)
        got = threshold.select_threshold(v, S=c + 4, w=4, recent=4, theta=np.float32(theta))
        assert got.size == cnt + 4
        assert np.array_equal(got[:cnt], np.sort(perm[:cnt]))
        assert np.array_equal(got[cnt:], np.arange(c, c + 4))


def test_extremes_and_monotone():
    rng = np.random.default_rng(7)
    S, w, r = 400, 32, 16
    c = select.candidates(S, w, r)
    v = rng.exponential(size=c)
    allc = threshold.select_threshold(v, S=S, w=w, recent=r, theta=-np.inf)
    assert np.array_equal(allc, np.concatenate([np.arange(c), np.arange(S - r, S)]))
    none = threshold.select_threshold(v, S=S, w=w, recent=r, theta=np.inf)
    assert np.array_equal(none, np.arange(S - r, S))
    prev = set(allc.tolist())
    for theta in np.linspace(0, 4, 17):
        cur = set(threshold.select_threshold(v, S=S, w=w, recent=r, theta=theta).tolist())
        assert cur <= prev
        prev = cur


def test_equality_nan_and_window_rule():
    v = np.array([0.5, np.nan, 0.25, 0.5, 0.75, 9.0, 9.0], dtype=np.float32)
    # S = 7, w = 2 (window tokens 5, 6 are not candidates), r = 1
    got = threshold.select_threshold(v, S=7, w=2, recent=1, theta=np.float32(0.5))
    assert got.tolist() == [0, 3, 4, 6]
    # r > w: the recent tokens leave the candidates
    got = threshold.select_threshold(v, S=7, w=1, recent=3, theta=np.float32(0.0))
    assert got.tolist() == [0, 2, 3, 4, 5, 6]


def test_kept_count_follows_the_prompt():
    c, G = 1000, 4
    flat = np.full(c, G / c)
    peaked = G * np.exp(-np.arange(c) / 20.0)
    peaked /= peaked.sum() / G
    theta = G / c
    nf = threshold.select_threshold(flat, S=c + 8, w=8, recent=8, theta=theta).size - 8
    npk = threshold.select_threshold(peaked, S=c + 8, w=8, recent=8, theta=theta).size - 8
    assert nf == c and npk < c // 10


def test_packed_heads_and_gather():
    rng = np.random.default_rng(9)
    Hkv, S, w, r, D = 4, 300, 24, 24, 16
    c = select.candidates(S, w, r)
    sc = rng.exponential(size=(Hkv, c)).astype(np.float32)
    sc[2] *= 0.01                                   # head 2 keeps only its recent window
    theta = np.float32(1.0)
    idx, off = threshold.select_threshold_heads(sc, S=S, w=w, recent=r, theta=theta)
    assert off[0] == 0 and off.size == Hkv + 1 and off[-1] == idx.size
    assert off[3] - off[2] == r
    x = rng.integers(0, 2 ** 16, size=(Hkv, S, D), dtype=np.uint16)
    out = threshold.compact_ragged(x, idx, off)
    for g in range(Hkv):
        rows = idx[off[g]:off[g + 1]]
        assert np.all(np.diff(rows) > 0)
        ref = compact.compact(x[g:g + 1], rows[None])[0]
        assert np.array_equal(out[off[g]:off[g + 1]], ref)
