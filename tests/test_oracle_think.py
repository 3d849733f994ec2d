"""Pins for the oracle's ThinK channel pruning and size arithmetic (CPU only).

* T = floor((1 - lambda) D) = 76 at lambda 0.4, D 128, and the total-memory
  fraction (T + D) / 2D is about 0.8, the 20% saving the ThinK page reports
  for lambda 0.4 (golden page figures).
* Channel norms equal numpy.linalg.norm (library); outlier channels are always
  kept; ties go to the lower channel; the gather keeps the selected columns.
* KV-cache size formula against the two sizes the pages print (13 GB on the
  ThinK page, about 335 GB on the KVzap page).
* Query-driven score (outer-product Frobenius norm) against the rank-1
  identity ||q k^T||_F = ||q|| ||k||, a case the query side decides, the
  contiguous query-head grouping (one group's loud channels do not reach the
  other) and recent rows not voting.
* Value-channel score: one key (output rows = that value row) and zero
  queries (uniform attention: output rows = the mean value row) in closed
  form, exact linearity in each value channel, explicit loops on a tiny case,
  and per-group selection with recent rows not voting.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import sizes, think

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_kept_channels_and_saving():
    g = GOLD["think_lambda_0_4"]
    assert sizes.think_channels(g["D"], g["lambda"]) == g["T"]
    assert abs((1 - sizes.think_total_fraction(g["D"], g["lambda"])) - g["printed_total_saving"]) < 0.005
    assert sizes.think_channels(128, 0.5) == 64
    assert sizes.think_channels(128, 0.3) == 89
    assert sizes.think_channels(128, 0.0) == 128


def test_kv_cache_sizes_match_pages():
    a = GOLD["kv_cache_llama2_7b"]
    m = a["model"]
    b = sizes.kv_cache_bytes(a["B"], a["S"], m["L"], m["N"], m["D"], m["elem_bytes"])
    assert round(b / 2 ** 30) == a["printed_GB"]
    c = GOLD["kv_cache_llama1_65b"]
    m = c["model"]
    b = sizes.kv_cache_bytes(c["B"], c["S"], m["L"], m["N"], m["D"], m["elem_bytes"])
    assert abs(b / 1e9 - c["printed_GB"]) < 1.0     # the page gives about 335 GB; the formula gives 335.5e9 bytes


@pytest.mark.parametrize("p", [1, 2])
def test_norms_match_numpy(p):
    rng = np.random.default_rng(p)
    x = rng.standard_normal((300, 128))
    assert np.allclose(think.channel_norms(x, p), np.linalg.norm(x, ord=p, axis=0), rtol=1e-13, atol=0)


def test_outliers_always_kept_and_gather():
    rng = np.random.default_rng(3)
    Hkv, B, r, D = 4, 90, 10, 128
    kc = rng.standard_normal((Hkv, B, D))
    outl = [3, 40, 77, 120]
    kc[:, :, outl] *= 8
    chans, mask, pruned, norms = think.think_prune(kc, recent=r, lam=0.4, p=2)
    assert chans.shape == (Hkv, 76) and pruned.shape == (Hkv, B - r, 76)
    for g in range(Hkv):
        assert set(outl) <= set(chans[g].tolist())
        assert np.all(np.diff(chans[g]) > 0)
        assert mask[g].sum() == 76 and np.all(mask[g, chans[g]] == 1)
        assert np.array_equal(pruned[g], kc[g, :B - r][:, chans[g]])
        # every kept channel's norm >= every pruned channel's norm
        kept = norms[g][chans[g]]
        gone = np.delete(norms[g], chans[g])
        assert kept.min() >= gone.max()


def test_recent_rows_do_not_vote():
    Hkv, B, r, D = 1, 20, 5, 8
    kc = np.ones((Hkv, B, D))
    kc[0, B - r:, 7] = 1000.0          # huge, but only in recent rows
    chans, _, _, _ = think.think_prune(kc, recent=r, lam=0.5, p=2)
    assert chans[0].tolist() == [0, 1, 2, 3]   # all norms equal -> lowest channels


def test_channel_ties_go_to_lower_index():
    kc = np.ones((1, 6, 16))
    chans, _, _, _ = think.think_prune(kc, recent=0, lam=0.75, p=1)
    assert chans[0].tolist() == [0, 1, 2, 3]


def test_query_score_is_product_of_column_norms():
    # rank-1 Frobenius identity: ||q k^T||_F = ||q||_2 ||k||_2, per channel
    rng = np.random.default_rng(11)
    q = rng.standard_normal((12, 16))
    k = rng.standard_normal((40, 16))
    got = think.query_scores(q, k)
    assert np.allclose(got, np.linalg.norm(q, axis=0) * np.linalg.norm(k, axis=0), rtol=1e-12)


def test_query_driven_prefers_channels_the_queries_use():
    # equal key norms everywhere: the query side alone decides; a channel with no
    # query energy is never kept, the loud query channels always are
    rng = np.random.default_rng(12)
    Hkv, G, w, B, D, recent = 2, 2, 3, 20, 16, 4
    kc = np.sign(rng.standard_normal((Hkv, B, D)))          # |K| = 1: every key column has norm sqrt(rows)
    q = rng.standard_normal((Hkv * G, w, D)) * 0.1
    q[:, :, 5] = 0.0
    loud = {0: [2, 9], 1: [4, 7]}                             # group g = query heads [g*G, g*G + G)
    for g, cols in loud.items():
        q[g * G:(g + 1) * G][:, :, cols] *= 100.0
    ch, mask, pruned, sc = think.think_prune_query(kc, q, recent=recent, lam=0.5)
    assert ch.shape == (Hkv, 8)
    for g in range(Hkv):
        assert 5 not in ch[g] and set(loud[g]) <= set(ch[g].tolist())
        assert np.array_equal(pruned[g], kc[g, :B - recent][:, ch[g]])
        assert mask[g].sum() == 8


def test_value_score_single_key_and_uniform_attention():
    rng = np.random.default_rng(21)
    R, D = 12, 16
    q = rng.standard_normal((R, D))
    k1, v1 = rng.standard_normal((1, D)), rng.standard_normal((1, D))
    # one key: every softmax row is [1], the output rows are V[0]
    assert np.allclose(think.value_scores(q, k1, v1, 0.3), np.sqrt(R) * np.abs(v1[0]), rtol=1e-13)
    # zero queries: uniform attention, the output rows are the mean value row
    k, v = rng.standard_normal((9, D)), rng.standard_normal((9, D))
    got = think.value_scores(np.zeros((R, D)), k, v, 0.3)
    assert np.allclose(got, np.sqrt(R) * np.abs(v.mean(axis=0)), rtol=1e-12)


def test_value_score_is_linear_in_each_value_channel():
    rng = np.random.default_rng(22)
    q, k, v = rng.standard_normal((10, 8)), rng.standard_normal((30, 8)), rng.standard_normal((30, 8))
    base = think.value_scores(q, k, v, 0.5)
    v2 = v.copy()
    v2[:, 3] *= -4.0
    got = think.value_scores(q, k, v2, 0.5)
    assert np.isclose(got[3], 4.0 * base[3], rtol=1e-12)
    assert np.allclose(np.delete(got, 3), np.delete(base, 3), rtol=1e-12)


def test_value_score_brute_force():
    rng = np.random.default_rng(23)
    R, U, D, a = 3, 4, 5, 0.7
    q, k, v = rng.standard_normal((R, D)), rng.standard_normal((U, D)), rng.standard_normal((U, D))
    want = []
    for d in range(D):
        tot = 0.0
        for i in range(R):
            w = [math.exp(a * sum(q[i, e] * k[j, e] for e in range(D))) for j in range(U)]
            o = sum(w[j] * v[j, d] for j in range(U)) / sum(w)
            tot += o * o
        want.append(math.sqrt(tot))
    assert np.allclose(think.value_scores(q, k, v, a), want, rtol=1e-12)


def test_value_pruning_grouping_and_gather():
    # uniform attention per group (zero queries): the score is sqrt(G*w) * |mean of
    # the non-recent V rows|, so each group keeps the channels its own values make loud
    rng = np.random.default_rng(24)
    Hkv, G, w, B, D, recent = 2, 3, 2, 24, 16, 4
    kc = rng.standard_normal((Hkv, B, D))
    vc = rng.standard_normal((Hkv, B, D)) * 0.01
    vc[0, :B - recent, [1, 6]] += 5.0
    vc[1, :B - recent, [2, 11]] += 5.0
    vc[:, B - recent:, 9] = 100.0                            # recent rows do not vote
    ch, mask, pruned, sc = think.think_prune_value(kc, vc, np.zeros((Hkv * G, w, D)), recent=recent, lam=0.75,
                                                   scale=0.25)
    assert {1, 6} <= set(ch[0].tolist())
    assert {2, 11} <= set(ch[1].tolist()) and 9 not in ch[0] and 9 not in ch[1]
    assert np.allclose(sc[1], np.sqrt(G * w) * np.abs(vc[1, :B - recent].mean(axis=0)), rtol=1e-12)
    for g in range(Hkv):
        assert np.array_equal(pruned[g], vc[g, :B - recent][:, ch[g]]) and mask[g].sum() == 4


def test_query_driven_group_is_contiguous_and_recent_rows_do_not_vote():
    # each group's own loud query channels dominate its scores; the other
    # group's loud channels (other query heads) do not reach it
    rng = np.random.default_rng(25)
    Hkv, G, w, B, D, recent = 2, 2, 3, 20, 16, 4
    kc = np.sign(rng.standard_normal((Hkv, B, D)))
    q = rng.standard_normal((Hkv * G, w, D)) * 0.1
    loud = {0: [2, 9], 1: [4, 7]}
    for g, cols in loud.items():
        q[g * G:(g + 1) * G][:, :, cols] *= 100.0
    _, _, _, sc = think.think_prune_query(kc, q, recent=recent, lam=0.5)
    for g in range(Hkv):
        assert sc[g][loud[g]].min() > 10.0 * sc[g][loud[1 - g]].max()
    # equal key and query energy in every channel except a huge value in the
    # recent rows of channel 7: the recent rows do not vote, so ties -> 0..T-1
    kc2 = np.ones((1, 12, 16))
    kc2[0, 8:, 7] = 1000.0
    ch, _, _, _ = think.think_prune_query(kc2, np.ones((1, 2, 16)), recent=4, lam=0.75)
    assert ch[0].tolist() == [0, 1, 2, 3]
