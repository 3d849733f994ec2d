"""Keyformer's decode phase: score accumulation over the compressed cache, and eviction.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: Keyformer blog page, the closing paragraphs on the two phases: decoding
runs on the reduced KV cache, and each step's score is added to the score
carried from before; the cache keeps the w most recent tokens and the k - w
other tokens with the highest score.  The step's score is the Gumbel-noised,
tempered softmax of the Gumbel-distribution and temperature sections,
f(y_j) = e^{(x_j + zeta_j)/tau} / sum e^{(x_l + zeta_l)/tau}.

Readings (the page gives the rule, not its bookkeeping):

* one step for one layer: the new token at position t has a query per query
  head and a key and a value per KV head; it attends over the B cache slots and
  itself (B + 1 keys);
* the step score of key j for KV head g sums that softmax over the G query
  heads of the group; x = scale * <q_h, k_j>; zeta is the Keyformer noise for
  query position t and key position pos_j (the prompt phase's counter), and
  tau = inf gives a uniform softmax;
* acc_j += score_j for the cached slots; the new token's accumulated score is
  its own step score;
* the recent window is the positions p > t - recent (the new token included);
  among the other entries the lowest accumulated score is evicted (ties: the
  smaller position), and the new token's key, value, position and score take
  that slot.  recent < B, so some entry can always be evicted;
* the prompt phase hands over the kept positions and, as initial accumulated
  scores, the prompt importance of kept prefix tokens (0 for the window's own
  tokens, which the prompt phase does not score) -- ``initial_scores``.

Parity: pinned by the tau = inf closed form (uniform scores: the oldest prompt
tokens go first), the per-group sum G of the step scores, the tau -> 0 one-hot
limit, invariance under a permutation of the slots, the recent-window rule and
a brute-force eviction on a tiny case (``tests/test_oracle_decode.py``).
"""

import numpy as np

from . import philox
from .score import bf16_bits_to_f64


def initial_scores(importance, indices, n):
    """acc[g, t] = importance[g, indices[g, t]] for prefix positions (< n), else 0."""
    imp = np.asarray(importance, dtype=np.float64)
    idx = np.asarray(indices, dtype=np.int64)
    out = np.zeros(idx.shape)
    for g in range(idx.shape[0]):
        pre = idx[g] < n
        out[g, pre] = imp[g, idx[g, pre]]
    return out


def step_scores(keys, positions, q_group, *, t, heads, scale, tau, seed):
    """Step score of each of the given keys: sum over the group's query heads of
    the noisy tempered softmax over these keys.  keys [N, D] float64,
    positions [N] int, q_group [G, D] float64, heads: the query-head ids."""
    s = np.zeros(len(positions))
    for q, h in zip(q_group, heads):
        x = scale * (keys @ q)
        if np.isinf(tau):
            y = np.zeros_like(x)
        else:
            y = (x + philox.keyformer_noise(seed, h, t, np.asarray(positions, dtype=np.int64))) / tau
        e = np.exp(y - y.max())
        s += e / e.sum()
    return s


def decode_step(kc, vc, pos, acc, q, k_new, v_new, *, t, recent, scale, tau, seed):
    """One step for one layer.

    kc, vc: [Hkv, B, D] uint16 bf16 bits (the cache slots); pos [Hkv, B] int;
    acc [Hkv, B] float64; q [H, D] float64 (H = G * Hkv, head h in group h // G);
    k_new, v_new [Hkv, D] uint16 bits.  Returns the new (kc, vc, pos, acc) and
    the evicted slot of each KV head.
    """
    kc, vc = np.array(kc), np.array(vc)
    pos, acc = np.array(pos, dtype=np.int64), np.array(acc, dtype=np.float64)
    Hkv, B, D = kc.shape
    G = q.shape[0] // Hkv
    if not 0 < recent < B:
        raise ValueError("the recent window must be shorter than the cache")
    evicted = np.empty(Hkv, dtype=np.int64)
    for g in range(Hkv):
        keys = np.concatenate([bf16_bits_to_f64(kc[g]), bf16_bits_to_f64(k_new[g])[None]])
        p = np.concatenate([pos[g], [t]])
        s = step_scores(keys, p, q[g * G:(g + 1) * G], t=t, heads=range(g * G, (g + 1) * G), scale=scale,
                        tau=tau, seed=seed)
        a = acc[g] + s[:B]
        cand = np.nonzero(pos[g] <= t - recent)[0]
        e = cand[np.lexsort((pos[g][cand], a[cand]))[0]]       # lowest score, then smaller position
        evicted[g] = e
        a[e] = s[B]
        acc[g] = a
        kc[g, e], vc[g, e], pos[g, e] = k_new[g], v_new[g], t
    return kc, vc, pos, acc, evicted
