"""Pins for the oracle's selection and compaction (CPU only).

* Selection: a rank-count characterisation (token j is kept iff fewer than
  k_top candidates beat it under (score desc, position asc)), brute force on
  tiny inputs; invariants from the pages: the last window is always kept
  (ZigZagKV page, SnapKV section; Keyformer page, prompt phase), output size
  is the budget, positions ascending and unique.
* Compaction: rows that encode their own (head, position) come out at the
  kept positions.
"""

import numpy as np
import pytest

from oracle import compact, select


def _rank_select(v, S, w, r, budget):
    c = min(S - w, S - r)
    k = budget - r
    keep = []
    for j in range(c):
        beats = sum(1 for jj in range(c) if v[jj] > v[j] or (v[jj] == v[j] and jj < j))
        if beats < k:
            keep.append(j)
    return sorted(keep + list(range(S - r, S)))


@pytest.mark.parametrize("seed", range(30))
def test_select_matches_rank_brute_force(seed):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(4, 14))
    w = int(rng.integers(1, S))
    r = int(rng.integers(0, S))
    c = min(S - w, S - r)
    if c < 0:
        pytest.skip("no candidates")
    k = int(rng.integers(0, c + 1))
    v = rng.integers(0, 4, S - w).astype(float) / 3.0     # plenty of ties
    out = select.select(v, S=S, w=w, recent=r, budget=k + r)
    assert out.tolist() == _rank_select(v, S, w, r, k + r)


def test_select_invariants_large():
    rng = np.random.default_rng(1)
    S, w, r, B = 5000, 128, 64, 700
    v = rng.exponential(size=S - w)
    out = select.select(v, S=S, w=w, recent=r, budget=B)
    assert out.size == B
    assert np.all(np.diff(out) > 0)
    assert set(range(S - r, S)) <= set(out.tolist())
    # window tokens that are not recent are dropped (r < w)
    assert not np.any((out >= S - w) & (out < S - r))
    # every kept candidate scores at least as much as every dropped one
    c = min(S - w, S - r)
    kept = out[out < c]
    dropped = np.setdiff1d(np.arange(c), kept)
    assert v[kept].min() >= v[dropped].max()


def test_select_edge_budgets():
    v = np.array([0.5, 0.1, 0.4])
    assert select.select(v, S=5, w=2, recent=2, budget=2).tolist() == [3, 4]        # k_top = 0
    assert select.select(v, S=5, w=2, recent=2, budget=5).tolist() == [0, 1, 2, 3, 4]
    with pytest.raises(ValueError):
        select.select(v, S=5, w=2, recent=2, budget=6)
    with pytest.raises(ValueError):
        select.select(v, S=5, w=2, recent=2, budget=1)


def test_select_recent_longer_than_window():
    # r > w: the recent tokens leave the candidate set
    v = np.array([1.0, 2.0, 3.0, 4.0, 5.0, 6.0])    # n = 6 (S=8, w=2)
    out = select.select(v, S=8, w=2, recent=4, budget=6)
    assert out.tolist() == [2, 3, 4, 5, 6, 7]


def test_compact_gathers_rows():
    Hkv, S, D = 3, 50, 4
    x = np.zeros((Hkv, S, D), dtype=np.uint16)
    for g in range(Hkv):
        for j in range(S):
            x[g, j, :] = g * 1000 + j
    rng = np.random.default_rng(0)
    idx = np.stack([np.sort(rng.choice(S, 9, replace=False)) for _ in range(Hkv)])
    out = compact.compact(x, idx)
    for g in range(Hkv):
        assert np.all(out[g, :, 0] == g * 1000 + idx[g])
        assert np.all(out[g] == out[g, :, :1])


def test_select_heads_per_row():
    # head g scores its own candidates (4g + 1, 4g + 2) highest, so with k_top = 2 each
    # row of the result must be exactly those two plus the recent window, in that head's
    # row (ZigZagKV page, SnapKV section: per-head top-K plus the last window).
    Hkv, S, w, r = 5, 40, 6, 3
    c = min(S - w, S - r)
    imp = np.full((Hkv, S - w), 0.01)
    for g in range(Hkv):
        imp[g, 4 * g + 1] = 1.0 + g
        imp[g, 4 * g + 2] = 0.5 + g
    out = select.select_heads(imp, S=S, w=w, recent=r, budget=2 + r)
    assert out.shape == (Hkv, 2 + r)
    for g in range(Hkv):
        assert out[g].tolist() == [4 * g + 1, 4 * g + 2, S - 3, S - 2, S - 1], g
    assert c == S - w


def test_select_heads_rows_are_independent():
    # reversing the heads reverses the rows of the result
    rng = np.random.default_rng(5)
    imp = rng.exponential(size=(4, 300))
    a = select.select_heads(imp, S=340, w=40, recent=16, budget=80)
    b = select.select_heads(imp[::-1], S=340, w=40, recent=16, budget=80)
    assert np.array_equal(a[::-1], b)
    assert not np.array_equal(a[0], a[1])
