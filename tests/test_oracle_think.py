"""Pins for the oracle's ThinK channel pruning and size arithmetic (CPU only).

* T = floor((1 - lambda) D) = 76 at lambda 0.4, D 128, and the total-memory
  fraction (T + D) / 2D is about 0.8, the 20% saving the ThinK page reports
  for lambda 0.4 (golden page figures).
* Channel norms equal numpy.linalg.norm (library); outlier channels are always
  kept; ties go to the lower channel; the gather keeps the selected columns.
* KV-cache size formula against the two sizes the pages print (13 GB on the
  ThinK page, about 335 GB on the KVzap page).
* Query-driven score (outer-product Frobenius norm) against the rank-1
  identity ||q k^T||_F = ||q|| ||k||, and a case the query side decides.
"""

import json
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
