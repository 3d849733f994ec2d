"""Pins for the oracle's Keyformer decode step (CPU only).

* tau = inf: every step score is G / (B + 1), so with zero initial scores the
  prompt tokens (present since the first step) hold the smallest scores and
  leave in order of position, one per step (closed form).
* The step scores of a KV head sum to G (one softmax per query head).
* tau -> 0: the step score is one-hot at the key with the largest noisy logit
  (Gumbel-max), here a key made to dominate.
* Permuting the cache slots permutes the result and evicts the same token
  (the noise is keyed by position, not slot).
* Tokens in the recent window are never evicted, whatever their score; a
  token at exactly t - recent is outside it and may leave.
* Brute force on a tiny cache: the evicted slot has the smallest (score,
  position) among the non-recent entries.
* initial_scores reads the prompt importance at kept prefix positions.
"""

import numpy as np

from oracle import decode
from kv_cache_compression_bf16_amd import workload as wk


def _state(rng, Hkv, G, B, D, t):
    kc = wk.f32_to_bf16_bits(rng.standard_normal((Hkv, B, D), dtype=np.float32))
    vc = wk.f32_to_bf16_bits(rng.standard_normal((Hkv, B, D), dtype=np.float32))
    pos = np.stack([np.sort(rng.choice(t, size=B, replace=False)) for _ in range(Hkv)])
    return kc, vc, pos


def _new(rng, Hkv, G, D):
    q = rng.standard_normal((Hkv * G, D))
    kn = wk.f32_to_bf16_bits(rng.standard_normal((Hkv, D), dtype=np.float32))
    vn = wk.f32_to_bf16_bits(rng.standard_normal((Hkv, D), dtype=np.float32))
    return q, kn, vn


def test_uniform_scores_evict_oldest_prompt_tokens():
    rng = np.random.default_rng(31)
    Hkv, G, B, D, recent, t0 = 2, 2, 12, 8, 4, 100
    kc, vc, pos = _state(rng, Hkv, G, B, D, t0)
    pos[:, -recent:] = np.arange(t0 - recent, t0)            # the prompt's own recent window
    acc = np.zeros((Hkv, B))
    start = pos.copy()
    for m in range(recent):                                   # while prompt tokens score lowest
        q, kn, vn = _new(rng, Hkv, G, D)
        kc, vc, pos, acc, ev = decode.decode_step(kc, vc, pos, acc, q, kn, vn, t=t0 + m, recent=recent,
                                                  scale=0.3, tau=np.inf, seed=5)
        for g in range(Hkv):
            assert not (set(start[g, :m + 1].tolist()) & set(pos[g].tolist()))   # oldest m + 1 gone
            assert t0 + m in pos[g]
    # every slot that has been present s steps holds s * G / (B + 1)
    assert np.allclose(np.sort(np.unique(np.round(acc * (B + 1) / G, 9))), np.arange(1, recent + 1))


def test_step_scores_sum_to_G_and_gumbel_max_limit():
    rng = np.random.default_rng(32)
    G, N, D = 3, 40, 16
    keys = rng.standard_normal((N, D))
    q = rng.standard_normal((G, D))
    p = rng.choice(1000, size=N, replace=False)
    s = decode.step_scores(keys, p, q, t=1000, heads=[0, 1, 2], scale=0.2, tau=1.0, seed=9)
    assert np.isclose(s.sum(), G, rtol=1e-12) and np.all(s > 0)
    keys[7] = 50.0 * q.sum(axis=0) / np.linalg.norm(q.sum(axis=0))    # dominant logit for every head
    s0 = decode.step_scores(keys, p, q, t=1000, heads=[0, 1, 2], scale=1.0, tau=1e-6, seed=9)
    assert np.isclose(s0[7], G) and np.allclose(np.delete(s0, 7), 0.0)


def test_slot_permutation_invariance_and_recent_window():
    rng = np.random.default_rng(33)
    Hkv, G, B, D, recent, t = 2, 2, 16, 8, 5, 500
    kc, vc, pos = _state(rng, Hkv, G, B, D, t)
    pos[:, -3:] = [t - 3, t - 2, t - 1]                      # three tokens inside the recent window
    acc = rng.exponential(size=(Hkv, B))
    acc[:, -3:] = 0.0                                         # lowest scores, but recent
    q, kn, vn = _new(rng, Hkv, G, D)
    a = decode.decode_step(kc, vc, pos, acc, q, kn, vn, t=t, recent=recent, scale=0.25, tau=1.0, seed=3)
    for g in range(Hkv):
        assert a[4][g] < B - 3                                # a recent token is never evicted
    perm = rng.permutation(B)
    b = decode.decode_step(kc[:, perm], vc[:, perm], pos[:, perm], acc[:, perm], q, kn, vn, t=t, recent=recent,
                           scale=0.25, tau=1.0, seed=3)
    for g in range(Hkv):
        assert pos[g, a[4][g]] == pos[g, perm][b[4][g]]      # the same token leaves
        assert np.allclose(b[3][g], a[3][g][perm], rtol=1e-12)
        assert np.array_equal(b[2][g], a[2][g][perm])


def test_eviction_brute_force():
    rng = np.random.default_rng(34)
    Hkv, G, B, D, recent, t = 1, 1, 6, 4, 2, 50
    kc, vc, pos = _state(rng, Hkv, G, B, D, t)
    acc = np.array([[0.5, 0.25, 0.75, 0.25, 1.0, 0.1]])
    q, kn, vn = _new(rng, Hkv, G, D)
    new = decode.decode_step(kc, vc, pos, acc, q, kn, vn, t=t, recent=recent, scale=0.5, tau=2.0, seed=1)
    s = decode.step_scores(np.concatenate([decode.bf16_bits_to_f64(kc[0]), decode.bf16_bits_to_f64(kn[0])[None]]),
                           np.concatenate([pos[0], [t]]), q, t=t, heads=[0], scale=0.5, tau=2.0, seed=1)
    best = None
    for j in range(B):
        if pos[0, j] > t - recent:
            continue
        key = (acc[0, j] + s[j], pos[0, j])
        if best is None or key < best[0]:
            best = (key, j)
    assert new[4][0] == best[1]
    assert new[2][0, best[1]] == t and np.isclose(new[3][0, best[1]], s[B])


def test_initial_scores():
    imp = np.array([[0.1, 0.2, 0.3, 0.4], [1.0, 2.0, 3.0, 4.0]])
    idx = np.array([[0, 3, 5], [2, 4, 6]])
    assert np.allclose(decode.initial_scores(imp, idx, 4), [[0.1, 0.4, 0.0], [3.0, 0.0, 0.0]])


def test_token_at_the_window_edge_may_leave():
    # the recent window is the positions > t - recent: a token at exactly
    # t - recent is outside it and, with the lowest score, is the one evicted
    rng = np.random.default_rng(35)
    Hkv, G, B, D, recent, t = 1, 1, 8, 4, 3, 100
    kc, vc, _ = _state(rng, Hkv, G, B, D, t)
    pos = np.array([[10, 20, 30, 40, 50, t - recent, t - 2, t - 1]])
    acc = np.array([[5.0, 5.0, 5.0, 5.0, 5.0, 0.0, 0.0, 0.0]])
    q, kn, vn = _new(rng, Hkv, G, D)
    new = decode.decode_step(kc, vc, pos, acc, q, kn, vn, t=t, recent=recent, scale=0.5, tau=1.0, seed=2)
    assert new[4][0] == 5 and new[2][0, 5] == t
