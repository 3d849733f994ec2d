"""Per-head token selection: top-k by importance plus the recent window.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources:

* ZigZagKV blog page, SnapKV section: each head keeps the top-K prefix tokens
  by averaged score, plus every token of the last window; ZigZagKV's token
  selection section: the same rule with each head's K taken from its
  layer's quota;
* Keyformer blog page, prompt-phase paragraph: keep the w most recent tokens
  and k - w of the remaining n - w, forming the new k-sized cache.

Readings: candidates are C = [0, min(S - w, S - r)) (with r < w the window
tokens in [S-w, S-r) are dropped, with r > w the recent tokens leave C); the
order is (importance descending, position ascending); k_top = budget - r;
the output lists the kept positions ascending; a budget beyond |C| + r is an
error.
"""

import numpy as np


def candidates(S, w, recent):
    return min(S - w, S - recent)


def select(importance_row, *, S, w, recent, budget):
    """importance_row: [>= candidates] scores of the prefix tokens.
    Returns int64 [budget] ascending positions."""
    c = candidates(S, w, recent)
    k_top = budget - recent
    if recent < 0 or recent > S or k_top < 0 or c < 0 or k_top > c:
        raise ValueError("invalid budget / recent window")
    v = np.asarray(importance_row, dtype=np.float64)[:c]
    j = np.arange(c)
    order = np.lexsort((j, -v))          # primary: -v ascending, then j ascending
    top = order[:k_top]
    keep = np.concatenate([top, np.arange(S - recent, S)])
    return np.sort(keep).astype(np.int64)


def select_heads(importance, *, S, w, recent, budget):
    return np.stack([select(row, S=S, w=w, recent=recent, budget=budget) for row in importance])
