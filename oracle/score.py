"""Observation-window scoring: logits, optional Gumbel noise and temperature,
softmax over the prefix, window mean and grouped-query sum.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources (all on the pages; no code is printed there):

* ZigZagKV blog page (qidao123 thread 109074), SnapKV section: the prompt's
  last window of queries (the observation window) attends to every earlier
  (prefix) token, per attention head; the mean over the window's rows of
  those attention scores is the prefix token's importance, giving an
  [heads, prefix] matrix from which each head picks its top-K.
* ThinK page (papercache summary of arXiv 2407.21018), section on
  query-driven pruning: attention = softmax(Q K^T / sqrt(D)) V.
* Keyformer blog page, section on the Gumbel distribution: x_i = Q K^T/sqrt(d_k),
  y_i = x_i + zeta_i with Gumbel noise, then softmax((x + zeta)/tau).
* KVzap news page, section on architectural compression: grouped-query
  attention, several query heads share one KV head.

Readings where the pages are silent (each also listed in the design notes):

* the softmax runs over the prefix keys j in [0, n), n = S - w, only (the
  importance row of a head then sums to 1);
* the window mean is the arithmetic mean over the w window rows;
* with H query heads and Hkv KV heads (G = H/Hkv), query head h reads KV head
  floor(h/G), and the importance of KV head g is the SUM of its G query heads'
  window means (so a row sums to G);
* noise is added before dividing by tau; tau = +inf gives y = 0 (uniform);
* the Gumbel generator is the one in ``oracle.philox``.

``importance_causal`` is the other reading of Keyformer's prompt phase (full,
causal attention); its pins are a harmonic-sum closed form at tau = inf, the
row and group sums, and explicit loops on a tiny case.
"""

import numpy as np

from . import philox


def bf16_bits_to_f64(bits):
    """Decode raw bf16 bit patterns (uint16) to float64 exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def logits(q_h, k_g, n, scale):
    """x[i, j] = scale * <Q_obs[h, i, :], K[g, j, :]> for the n prefix keys.

    q_h: [w, D] float64; k_g: [>=n, D] float64.  Returns [w, n] float64.
    """
    return scale * (q_h @ k_g[:n].T)


def noisy_tempered(x, *, seed, head, S, w, tau):
    """y = (x + zeta) / tau with zeta the Keyformer Gumbel noise for query head
    ``head`` (window query i sits at absolute position S - w + i)."""
    wn, n = x.shape
    pos = (S - w + np.arange(wn, dtype=np.int64))[:, None]
    j = np.arange(n, dtype=np.int64)[None, :]
    zeta = philox.keyformer_noise(seed, head, pos, j)
    if np.isinf(tau):
        return np.zeros_like(x)
    return (x + zeta) / tau


def softmax_rows(y):
    """p[i, j] = exp(y[i, j] - max_j y[i, :]) / sum_j exp(y[i, j] - max_j y[i, :])."""
    m = y.max(axis=1, keepdims=True)
    e = np.exp(y - m)
    return e / e.sum(axis=1, keepdims=True)


def head_window_mean(q_h, k_g, *, n, scale, gumbel=False, seed=0, head=0, S=None, w=None,
                     tau=1.0):
    """a[j] = (1/w) * sum_i p[i, j] for one query head.  Returns [n] float64."""
    x = logits(q_h, k_g, n, scale)
    y = noisy_tempered(x, seed=seed, head=head, S=S, w=w, tau=tau) if gumbel else x
    p = softmax_rows(y)
    return p.mean(axis=0)


def importance(q_obs, k, *, S, w, scale, gumbel=False, tau=1.0, seed=0, kv_heads=None):
    """Importance I[g, j] for j in [0, S-w): sum over the query heads of KV
    head g of their window means.

    q_obs: [H, w, D] float64 (the last w queries of the prompt);
    k:     [Hkv, >=S-w, D] float64;
    kv_heads: optional iterable of KV heads to compute (others left NaN).
    Returns [Hkv, S-w] float64.
    """
    H = q_obs.shape[0]
    Hkv = k.shape[0]
    if H % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = H // Hkv
    n = S - w
    out = np.full((Hkv, n), np.nan)
    for g in (range(Hkv) if kv_heads is None else kv_heads):
        acc = np.zeros(n)
        for h in range(g * G, (g + 1) * G):
            acc += head_window_mean(q_obs[h], k[g], n=n, scale=scale, gumbel=gumbel, seed=seed,
                                    head=h, S=S, w=w, tau=tau)
        out[g] = acc
    return out


# ---- Keyformer's other reading: causal scoring over the whole prompt
#
# Keyformer blog page, closing paragraphs: the prompt phase is a full attention
# pass with the Gumbel noise added, from which the key tokens are picked.  Read
# as causal attention: window query i sits at position P = S - w + i and sees
# the keys j <= P (with w = S every prompt position is a query).  Its noisy
# tempered softmax runs over those P + 1 keys; the importance of key j is the
# mean over the w query rows (0 for the rows that cannot see it), summed over
# the G query heads of the KV head, for every j in [0, S).

def head_causal_mean(q_h, k_g, *, S, w, scale, gumbel=False, seed=0, head=0, tau=1.0, rows=None):
    """a[j] = (1/w) * sum over the given window rows i (default: all) of p[i, j],
    p the causal softmax of row i.  Returns [S] float64."""
    out = np.zeros(S)
    for i in (range(w) if rows is None else rows):
        P = S - w + i
        x = scale * (k_g[:P + 1] @ q_h[i])
        if gumbel:
            x = np.zeros_like(x) if np.isinf(tau) else (x + philox.keyformer_noise(seed, head, P, np.arange(P + 1))) / tau
        e = np.exp(x - x.max())
        out[:P + 1] += e / e.sum()
    return out / w


def importance_causal(q_obs, k, *, S, w, scale, gumbel=False, tau=1.0, seed=0, kv_heads=None):
    """Causal importance I[g, j], j in [0, S).  q_obs: [H, w, D] float64 (the
    last w prompt queries), k: [Hkv, >= S, D] float64.  Returns [Hkv, S]."""
    H, Hkv = q_obs.shape[0], k.shape[0]
    G = H // Hkv
    out = np.full((Hkv, S), np.nan)
    for g in (range(Hkv) if kv_heads is None else kv_heads):
        acc = np.zeros(S)
        for h in range(g * G, (g + 1) * G):
            acc += head_causal_mean(q_obs[h], k[g], S=S, w=w, scale=scale, gumbel=gumbel, seed=seed, head=h,
                                    tau=tau)
        out[g] = acc
    return out
