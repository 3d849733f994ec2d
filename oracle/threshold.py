"""Threshold selection with a sliding window, and the packed (ragged) gather.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: KVzap news page, inference section (thresholding and a sliding
window): at inference the entries whose score falls below a threshold are
removed, a window of the most recent tokens is always kept, and so the number
of kept tokens, hence the compression ratio, follows the prompt.

Readings (the page gives the rule, not its details):

* the score is any per-head score over the candidates C = [0, min(S - w, S - r))
  (the same candidate set as the top-k selection; here the window importance,
  optionally pooled);
* a candidate is kept when score >= theta; a NaN score is never kept;
* the comparison is made in the precision of the scores handed in: float32
  scores are compared with theta rounded to float32 (as the kernel does);
* the recent window [S - r, S) is always kept and follows the kept
  candidates, so each head's positions are ascending;
* heads are packed one after the other: head g's positions are
  indices[offsets[g]:offsets[g + 1]], offsets[0] = 0.

Parity: pinned by the top-k equivalence (theta = the k-th largest of distinct
scores keeps exactly the top-k set of ``select``), a closed-form count on a
geometric score sequence, the -inf/+inf extremes, monotonicity in theta and
the NaN / equality rules (``tests/test_oracle_threshold.py``).
"""

import numpy as np

from .select import candidates


def keep_candidates(score_row, c, theta):
    """Positions j in [0, c) with score_row[j] >= theta, ascending."""
    v = np.asarray(score_row)[:c]
    th = np.asarray(theta, dtype=v.dtype) if v.dtype.kind == "f" else theta
    return np.flatnonzero(v >= th)        # NaN >= x is False: never kept


def select_threshold(score_row, *, S, w, recent, theta):
    """One head: kept candidate positions, then the recent window (int64, ascending)."""
    c = candidates(S, w, recent)
    if recent < 0 or recent > S or c < 0:
        raise ValueError("invalid window / recent sizes")
    kept = keep_candidates(score_row, c, theta)
    return np.concatenate([kept, np.arange(S - recent, S)]).astype(np.int64)


def select_threshold_heads(scores, *, S, w, recent, theta):
    """All heads, packed.  Returns (indices int64 [total], offsets int64 [Hkv + 1])."""
    rows = [select_threshold(r, S=S, w=w, recent=recent, theta=theta) for r in scores]
    offsets = np.zeros(len(rows) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum([len(r) for r in rows])
    idx = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)
    return idx, offsets


def compact_ragged(x, indices, offsets):
    """x: [Hkv, S, D] (any dtype, raw bits preserved).  Row t of the packed
    output is x[g, indices[t]] for the head g with offsets[g] <= t < offsets[g + 1]."""
    x = np.asarray(x)
    out = np.empty((int(offsets[-1]),) + x.shape[2:], dtype=x.dtype)
    for g in range(x.shape[0]):
        a, b = int(offsets[g]), int(offsets[g + 1])
        out[a:b] = x[g][np.asarray(indices[a:b], dtype=np.int64)]
    return out
