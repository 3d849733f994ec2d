"""ThinK magnitude-based key-channel pruning.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: ThinK page (papercache summary of arXiv 2407.21018, ICLR 2025):

* section on magnitude-based pruning: M_{n,d} = ||K[n, :, d]||_p for head n and
  channel d; with pruning ratio lambda every head keeps T = floor((1 - lambda) D)
  channels, I = Top_T(M, T), I in Z^{N x T};
* section on THINK's implementation: recent tokens' keys are not pruned, and a
  binary mask records which channels were pruned.

Readings: the norm runs over the non-recent kept rows (the rows that get
pruned), i.e. the first budget - r rows of the compacted cache, whose positions
all precede the recent window; ties in M go to the lower channel; the kept
channel list is ascending; V is not touched.
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
