"""ThinK key-channel pruning: magnitude-based and query-driven.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: ThinK page (papercache summary of arXiv 2407.21018, ICLR 2025):

* section on magnitude-based pruning: M_{n,d} = ||K[n, :, d]||_p for head n and
  channel d; with pruning ratio lambda every head keeps T = floor((1 - lambda) D)
  channels, I = Top_T(M, T), I in Z^{N x T};
* section on THINK's implementation: recent tokens' keys are not pruned, and a
  binary mask records which channels were pruned;
* sections on query-driven pruning, the greedy algorithm and the observation
  window: channel j of head i scores Score_i[j] = ||Q_i[-S_obs:, j] K_i[:, j]^T||_F
  (the Frobenius norm of the outer product of the channel's window-query column
  and key column), and the T highest-scoring channels are kept.

* supplementary section on value-cache pruning: channel j of the value cache
  scores Score_v[j] = ||softmax(Q[-S_obs:] K^T / sqrt(D)) V[:, j]||_F and the
  T highest-scoring value channels are kept.

Readings: the norm runs over the non-recent kept rows (the rows that get
pruned), i.e. the first budget - r rows of the compacted cache, whose positions
all precede the recent window; ties in M go to the lower channel; the kept
channel list is ascending.  For the query-driven score of a KV head shared by
G query heads, the window queries of those G heads are stacked (G*w rows); the
key side is the same non-recent kept rows.  Value pruning (a separate call)
takes K and V over those same rows U: the softmax of each stacked query row is
normalised over U, with the logit scale given (1/sqrt(D) on the page).
"""

import numpy as np

from .sizes import think_channels as kept_channels


def channel_norms(kc_head_rows, p=2):
    """M[d] = (sum_t |K[t, d]|^p)^(1/p) over the given rows.  kc_head_rows: [rows, D] float64."""
    a = np.abs(np.asarray(kc_head_rows, dtype=np.float64))
    return (a ** p).sum(axis=0) ** (1.0 / p)


def think_prune(kc, *, recent, lam, p=2):
    """kc: [Hkv, B, D] float64 values of the compacted keys (recent rows last).

    Returns (channels [Hkv, T] int64 ascending, mask [Hkv, D] uint8,
             pruned [Hkv, B - recent, T] float64, norms [Hkv, D] float64).
    """
    Hkv, B, D = kc.shape
    T = kept_channels(D, lam)
    rows = B - recent
    chans = np.empty((Hkv, T), dtype=np.int64)
    mask = np.zeros((Hkv, D), dtype=np.uint8)
    norms = np.empty((Hkv, D))
    pruned = np.empty((Hkv, rows, T))
    for g in range(Hkv):
        M = channel_norms(kc[g, :rows], p)
        norms[g] = M
        d = np.arange(D)
        order = np.lexsort((d, -M))
        c = np.sort(order[:T])
        chans[g] = c
        mask[g, c] = 1
        pruned[g] = kc[g, :rows][:, c]
    return chans, mask, pruned, norms


def query_scores(q_group, kc_head_rows):
    """Score[d] = ||Q[:, d] K[:, d]^T||_F, straight from the definition.

    q_group: [G*w, D] window queries of the KV head's query heads; kc_head_rows:
    [rows, D] non-recent kept keys (both float64).  Returns float64 [D].
    """
    q = np.asarray(q_group, dtype=np.float64)
    k = np.asarray(kc_head_rows, dtype=np.float64)
    return np.array([np.linalg.norm(np.outer(q[:, d], k[:, d]), "fro") for d in range(q.shape[1])])


def think_prune_query(kc, q_obs, *, recent, lam):
    """Query-driven ThinK.  kc: [Hkv, B, D] float64 compacted keys (recent rows
    last); q_obs: [H, w, D] float64 window queries, H = G * Hkv, head h in group h // G.

    Returns (channels [Hkv, T] ascending, mask [Hkv, D], pruned [Hkv, B - recent, T], scores [Hkv, D]).
    """
    Hkv, B, D = kc.shape
    H = q_obs.shape[0]
    G = H // Hkv
    T = kept_channels(D, lam)
    rows = B - recent
    chans = np.empty((Hkv, T), dtype=np.int64)
    mask = np.zeros((Hkv, D), dtype=np.uint8)
    scores = np.empty((Hkv, D))
    pruned = np.empty((Hkv, rows, T))
    for g in range(Hkv):
        qg = q_obs[g * G:(g + 1) * G].reshape(-1, D)
        sc = query_scores(qg, kc[g, :rows])
        scores[g] = sc
        order = np.lexsort((np.arange(D), -sc))
        c = np.sort(order[:T])
        chans[g] = c
        mask[g, c] = 1
        pruned[g] = kc[g, :rows][:, c]
    return chans, mask, pruned, scores


def value_scores(q_group, kc_rows, vc_rows, scale):
    """Score_v[d] = ||softmax(scale * Q K^T) V[:, d]||_2 over the stacked query rows.

    q_group [R, D], kc_rows / vc_rows [U, D] (float64).  The softmax of each
    query row runs over the U keys.  Returns float64 [D].
    """
    q = np.asarray(q_group, dtype=np.float64)
    k = np.asarray(kc_rows, dtype=np.float64)
    v = np.asarray(vc_rows, dtype=np.float64)
    x = scale * (q @ k.T)                                   # [R, U] logits
    x -= x.max(axis=1, keepdims=True)
    e = np.exp(x)
    P = e / e.sum(axis=1, keepdims=True)                    # row softmax
    O = P @ v                                               # [R, D] attention output
    return np.sqrt((O * O).sum(axis=0))                     # Frobenius norm per channel


def think_prune_value(kc, vc, q_obs, *, recent, lam, scale):
    """Value-channel pruning.  kc, vc: [Hkv, B, D] float64 compacted cache
    (recent rows last); q_obs: [H, w, D] float64, head h in group h // G.

    Returns (channels [Hkv, T] ascending, mask [Hkv, D], pruned values
    [Hkv, B - recent, T], scores [Hkv, D]).
    """
    Hkv, B, D = vc.shape
    G = q_obs.shape[0] // Hkv
    T = kept_channels(D, lam)
    rows = B - recent
    chans = np.empty((Hkv, T), dtype=np.int64)
    mask = np.zeros((Hkv, D), dtype=np.uint8)
    scores = np.zeros((Hkv, D))
    pruned = np.empty((Hkv, rows, T))
    for g in range(Hkv):
        if rows > 0:
            qg = q_obs[g * G:(g + 1) * G].reshape(-1, D)
            scores[g] = value_scores(qg, kc[g, :rows], vc[g, :rows], scale)
        order = np.lexsort((np.arange(D), -scores[g]))
        c = np.sort(order[:T])
        chans[g] = c
        mask[g, c] = 1
        pruned[g] = vc[g, :rows][:, c]
    return chans, mask, pruned, scores
