"""Pins for the oracle's observation-window scoring (CPU only).

What fixes each part, independently of the oracle's own code:

* closed forms: a two-key problem whose softmax is the logistic function;
  alpha = 0 and tau = inf give the uniform distribution (the Keyformer page's
  tau -> infinity limit, 1/k for every token);
* library routine: the softmax step equals scipy.special.softmax;
* invariants: each query head's window mean sums to 1 over the prefix and a
  KV head's importance sums to G; keys outside the prefix do not matter;
  permuting prefix keys permutes the importance; grouped-query heads
  h -> floor(h/G) (checked against the MHA problem with duplicated KV heads);
* limits and statistics: tau -> 0 gives one-hot rows at argmax(x + zeta)
  (Keyformer page, temperature paragraph); averaged over many seeds the
  tau -> 0 importance converges to the noiseless softmax importance
  (Gumbel-max theorem, textbook).
"""

import math

import numpy as np
import pytest
import scipy.special

from oracle import philox, score

RNG = np.random.default_rng(7)


def _rand(*shape):
    return RNG.standard_normal(shape)


def test_row_sums_and_group_sums():
    H, Hkv, w, S, D = 6, 2, 5, 37, 16
    q, k = _rand(H, w, D), _rand(Hkv, S, D)
    I = score.importance(q, k, S=S, w=w, scale=1 / math.sqrt(D))
    assert I.shape == (Hkv, S - w)
    assert np.allclose(I.sum(axis=1), H // Hkv, rtol=0, atol=1e-12)
    assert np.all(I > 0)
    for h in range(H):
        a = score.head_window_mean(q[h], k[h // 3], n=S - w, scale=1 / math.sqrt(D))
        assert abs(a.sum() - 1.0) < 1e-12


def test_two_key_logistic_closed_form():
    D, w, S = 128, 1, 3          # prefix = keys 0 and 1; key 2 is the window position
    q = np.zeros((1, w, D)); q[0, 0, 5] = 3.0
    k = np.zeros((1, S, D)); k[0, 0, 5] = 2.0; k[0, 2, :] = 99.0
    alpha = 1 / math.sqrt(D)
    I = score.importance(q, k, S=S, w=w, scale=alpha)
    x0 = alpha * 6.0
    assert I[0, 0] == pytest.approx(1 / (1 + math.exp(-x0)), rel=1e-14)
    assert I[0, 1] == pytest.approx(math.exp(-x0) / (1 + math.exp(-x0)), rel=1e-14)


def test_softmax_step_matches_scipy():
    y = _rand(9, 31) * 4
    assert np.allclose(score.softmax_rows(y), scipy.special.softmax(y, axis=1), rtol=1e-13, atol=0)


def test_zero_scale_and_infinite_tau_are_uniform():
    H, w, S, D = 2, 4, 29, 8
    q, k = _rand(H, w, D), _rand(H, S, D)
    n = S - w
    I0 = score.importance(q, k, S=S, w=w, scale=0.0)
    assert np.allclose(I0, 1.0 / n, rtol=1e-14, atol=0)
    Iinf = score.importance(q, k, S=S, w=w, scale=0.3, gumbel=True, tau=math.inf, seed=3)
    assert np.allclose(Iinf, 1.0 / n, rtol=1e-14, atol=0)
    # tau = 1e12: n * I = 1 to 1e-9 (the Keyformer page's large-tau limit)
    Ibig = score.importance(q, k, S=S, w=w, scale=0.3, gumbel=True, tau=1e12, seed=3)
    assert np.allclose(Ibig * n, 1.0, rtol=0, atol=1e-9)


def test_keys_after_prefix_are_ignored():
    H, w, S, D = 2, 3, 20, 8
    q, k = _rand(H, w, D), _rand(H, S, D)
    k2 = k.copy(); k2[:, S - w:, :] = 1e6
    assert np.array_equal(score.importance(q, k, S=S, w=w, scale=0.5),
                          score.importance(q, k2, S=S, w=w, scale=0.5))


def test_prefix_permutation_equivariance():
    H, w, S, D = 3, 4, 30, 8
    q, k = _rand(H, w, D), _rand(H, S, D)
    n = S - w
    perm = RNG.permutation(n)
    kp = k.copy(); kp[:, :n] = k[:, perm]
    I = score.importance(q, k, S=S, w=w, scale=0.4)
    Ip = score.importance(q, kp, S=S, w=w, scale=0.4)
    assert np.allclose(Ip, I[:, perm], rtol=1e-13, atol=0)


def test_gqa_head_mapping_is_contiguous_groups():
    H, Hkv, w, S, D = 4, 2, 3, 25, 8
    q, k = _rand(H, w, D), _rand(Hkv, S, D)
    Igqa = score.importance(q, k, S=S, w=w, scale=0.35)
    kdup = np.stack([k[0], k[0], k[1], k[1]])
    Imha = score.importance(q, kdup, S=S, w=w, scale=0.35)
    assert np.allclose(Igqa[0], Imha[0] + Imha[1], rtol=1e-13, atol=0)
    assert np.allclose(Igqa[1], Imha[2] + Imha[3], rtol=1e-13, atol=0)


def test_single_row_importance_orders_like_logits():
    D, w, S = 8, 1, 40
    q, k = _rand(1, w, D), _rand(1, S, D)
    I = score.importance(q, k, S=S, w=w, scale=0.5)[0]
    x = 0.5 * (k[0, :S - w] @ q[0, 0])
    assert np.array_equal(np.argsort(I, kind="stable"), np.argsort(x, kind="stable"))


def test_small_tau_is_one_hot_at_noisy_argmax():
    H, w, S, D, seed = 2, 6, 40, 8, 11
    q, k = _rand(H, w, D), _rand(H, S, D)
    n = S - w
    tau = 1e-8
    I = score.importance(q, k, S=S, w=w, scale=0.5, gumbel=True, tau=tau, seed=seed)
    for h in range(H):
        x = 0.5 * (q[h] @ k[h, :n].T)
        pos = (S - w + np.arange(w))[:, None]
        zeta = philox.keyformer_noise(seed, h, pos, np.arange(n)[None, :])
        top2 = np.sort(x + zeta, axis=1)[:, -2:]
        assert np.all(top2[:, 1] - top2[:, 0] > 1e-6)     # no near-tie rows in this draw
        am = np.argmax(x + zeta, axis=1)
        expect = np.bincount(am, minlength=n) / w
        assert np.allclose(I[h], expect, rtol=0, atol=1e-12)


def test_gumbel_max_average_converges_to_softmax():
    # Gumbel-max theorem: argmax_j (x_j + zeta_j) is distributed as softmax(x).
    H, w, S, D = 1, 2, 8, 4
    q, k = _rand(H, w, D), _rand(H, S, D)
    n = S - w
    seeds = 3000
    acc = np.zeros(n)
    for s in range(seeds):
        acc += score.importance(q, k, S=S, w=w, scale=0.7, gumbel=True, tau=1e-6, seed=s)[0]
    acc /= seeds
    ref = score.importance(q, k, S=S, w=w, scale=0.7)[0]
    # each entry is a mean of w*seeds Bernoulli draws / w (rows independent given seed)
    sd = np.sqrt(ref * (1 - ref) / (w * seeds))
    assert np.all(np.abs(acc - ref) < 5 * sd + 1e-12)


def test_bf16_decode_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x4049, 0x7F7F], dtype=np.uint16)
    v = score.bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -1.0 and v[2] == 0.0
    assert v[3] == 3.140625
    assert v[4] == (2 - 2 ** -7) * 2.0 ** 127
