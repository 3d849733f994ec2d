"""Compaction: gather the kept rows of K and V into a dense per-head cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources: Keyformer blog page, prompt-phase paragraph (the kept tokens form the
new, smaller KV cache); KVzap news page, first section (the cache holds keys
and values per layer and head, shape (2, L, H, T, D)).  The copy is of raw
bf16 bit patterns, so the result is bit-exact by construction.
"""

import numpy as np


def compact(x, indices):
    """x: [Hkv, S, D] (any dtype, raw bits preserved); indices: [Hkv, B].
    Returns [Hkv, B, D] with out[g, t] = x[g, indices[g, t]]."""
    x = np.asarray(x)
    idx = np.asarray(indices, dtype=np.int64)
    out = np.empty((idx.shape[0], idx.shape[1]) + x.shape[2:], dtype=x.dtype)
    for g in range(idx.shape[0]):
        out[g] = x[g][idx[g]]
    return out
