"""Pins for the oracle's causal (whole-prompt) scoring (CPU only).

* tau = inf: row i sees P + 1 keys with equal weight, so
  I[j] = (G / w) * sum over rows with P >= j of 1 / (P + 1) (harmonic sums).
* Each row sums to 1: every KV head's importance sums to G; with w = S the
  last key is seen only by the last row and the first key by every row.
* Explicit loops (exp, sums) agree on a tiny case, noise included.
"""

import math

import numpy as np

from oracle import philox, score


def test_uniform_is_harmonic():
    rng = np.random.default_rng(41)
    Hkv, G, S, w, D = 2, 3, 40, 12, 8
    q = rng.standard_normal((Hkv * G, w, D))
    k = rng.standard_normal((Hkv, S, D))
    got = score.importance_causal(q, k, S=S, w=w, scale=0.3, gumbel=True, tau=np.inf, seed=1)
    want = np.array([G / w * sum(1.0 / (S - w + i + 1) for i in range(w) if S - w + i >= j) for j in range(S)])
    assert np.allclose(got, want[None], rtol=1e-12)


def test_sums_and_edge_keys():
    rng = np.random.default_rng(42)
    Hkv, G, S, D = 2, 2, 30, 8
    w = S
    q = rng.standard_normal((Hkv * G, w, D))
    k = rng.standard_normal((Hkv, S, D))
    imp = score.importance_causal(q, k, S=S, w=w, scale=0.5, gumbel=True, tau=1.0, seed=3)
    assert np.allclose(imp.sum(axis=1), G, rtol=1e-12)
    # the first row (position 0) sees only key 0: it contributes G/w there
    assert np.all(imp[:, 0] >= G / w - 1e-15)
    # the last key is seen only by the last row of each query head
    last = sum(score.head_causal_mean(q[h], k[0], S=S, w=w, scale=0.5, gumbel=True, seed=3, head=h, tau=1.0,
                                      rows=[w - 1])[S - 1] for h in range(G))
    assert np.isclose(imp[0, S - 1], last, rtol=1e-12)


def test_brute_force_with_noise():
    rng = np.random.default_rng(43)
    S, w, D, a, tau, seed = 7, 4, 3, 0.8, 2.0, 11
    q = rng.standard_normal((1, w, D))
    k = rng.standard_normal((1, S, D))
    want = [0.0] * S
    for i in range(w):
        P = S - w + i
        ys = []
        for j in range(P + 1):
            x = a * sum(q[0, i, e] * k[0, j, e] for e in range(D))
            zeta = float(philox.keyformer_noise(seed, 0, P, j))
            ys.append((x + zeta) / tau)
        m = max(ys)
        tot = sum(math.exp(y - m) for y in ys)
        for j in range(P + 1):
            want[j] += math.exp(ys[j] - m) / tot / w
    got = score.importance_causal(q, k, S=S, w=w, scale=a, gumbel=True, tau=tau, seed=seed)[0]
    assert np.allclose(got, want, rtol=1e-12)
