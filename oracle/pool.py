"""SnapKV's 1D pooling of the importance along the prefix keys.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: ZigZagKV blog page, SnapKV section (after the window-averaged scores
are computed, a 1D pooling clusters them so that the neighbours of a strong
token are kept together with it).  The page gives neither the kernel size nor
the pooling type.

Readings: pooling runs along the key axis of each head's importance vector
[0, n), stride 1, odd kernel size k, window [j - k//2, j + k//2] ('same'
output length).  Average pooling treats positions outside [0, n) as zeros and
always divides by k; max pooling takes the maximum over the positions of the
window that lie in [0, n).  Written straight from that definition, one output
at a time.
"""

import numpy as np

AVG, MAX = 0, 1


def pool_row(x, kernel, mode):
    """x: [n] scores (any float); returns float64 [n]."""
    if kernel < 1 or kernel % 2 == 0:
        raise ValueError("kernel size must be odd and >= 1")
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    h = kernel // 2
    out = np.empty(n, dtype=np.float64)
    for j in range(n):
        lo, hi = max(0, j - h), min(n, j + h + 1)
        window = x[lo:hi]
        out[j] = window.sum() / kernel if mode == AVG else window.max()
    return out


def pool(importance, kernel, mode):
    """importance: [..., n]; pools every row."""
    imp = np.asarray(importance, dtype=np.float64)
    flat = imp.reshape(-1, imp.shape[-1])
    return np.stack([pool_row(r, kernel, mode) for r in flat]).reshape(imp.shape)
