"""Shared helpers for the GPU-vs-oracle parity tests.

Tolerances (fixed here, used by every parity test):

* importance: |I_gpu - I_or| <= 1e-3 * I_or (absolute floor 1e-30) per element;
  each KV head's row sums to G within 1e-5 relative;
* kept indices: bit-exact unless the oracle's k-th and (k+1)-th candidate
  scores are within 1e-3 relative; in that tie case the GPU set must have the
  right size, be unique, ascending and in range, contain the recent window,
  contain every candidate scoring >= s_k (1 + 1e-3), none scoring
  <= s_{k+1} (1 - 1e-3), and retain attention mass (sum of the oracle's scores
  over the kept candidates) within 1e-3 of the oracle's set;
* compacted K/V: bit-exact against the gather at the GPU's indices;
* ThinK channels: bit-exact unless the T-th and (T+1)-th norms are within
  1e-3 relative, else the kept norm mass within 1e-3; pruned keys bit-exact
  against the gather at the GPU's channels.
"""

import numpy as np
import torch

from kv_cache_compression_bf16_amd import pipeline

REL = 1e-3


def dev():
    return torch.device("cuda:0")


def to_dev(bits):
    return pipeline.bf16_to_device(bits, dev())


def bits_of(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check_importance(gpu, ref, G, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, what
    tol = np.maximum(REL * ref, 1e-30)
    err = np.abs(gpu - ref)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err / tol), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} elements off; worst at {i}: gpu {gpu[i]!r} ref {ref[i]!r}")
    sums = gpu.reshape(-1, gpu.shape[-1]).sum(axis=1)
    assert np.allclose(sums, G, rtol=1e-5, atol=0), f"{what}: row sums {sums.min()}..{sums.max()} != {G}"
    return float((err / np.maximum(ref, 1e-30)).max())


def check_selection(gpu_idx, ref_scores, ref_idx, *, S, w, recent, budget):
    """Tie-aware comparison of one head's kept positions.  Returns 'exact' or 'tie'."""
    gpu_idx = np.asarray(gpu_idx, dtype=np.int64)
    c = min(S - w, S - recent)
    k = budget - recent
    if np.array_equal(gpu_idx, ref_idx):
        return "exact"
    v = np.asarray(ref_scores, dtype=np.float64)[:c]
    order = np.lexsort((np.arange(c), -v))
    sk = v[order[k - 1]] if k > 0 else np.inf
    sk1 = v[order[k]] if k < c else -np.inf
    assert k > 0 and k < c and sk - sk1 <= REL * sk, \
        f"selection differs outside a tie (s_k={sk}, s_k+1={sk1})"
    assert gpu_idx.size == budget and np.all(np.diff(gpu_idx) > 0)
    assert gpu_idx.min() >= 0 and gpu_idx.max() < S
    assert set(range(S - recent, S)) <= set(gpu_idx.tolist())
    cand = gpu_idx[gpu_idx < c]
    assert cand.size == k and np.all(gpu_idx[k:] >= S - recent)
    must = np.nonzero(v >= sk * (1 + REL))[0]
    assert set(must.tolist()) <= set(cand.tolist()), "a clear winner was dropped"
    never = np.nonzero(v <= sk1 * (1 - REL))[0]
    assert not (set(never.tolist()) & set(cand.tolist())), "a clear loser was kept"
    m_gpu = v[cand].sum()
    m_ref = v[ref_idx[ref_idx < c]].sum()
    assert abs(m_gpu - m_ref) <= REL * m_ref, f"retained mass {m_gpu} vs {m_ref}"
    return "tie"


def check_channels(gpu_ch, norms, ref_ch, T):
    gpu_ch = np.asarray(gpu_ch, dtype=np.int64)
    if np.array_equal(gpu_ch, ref_ch):
        return "exact"
    order = np.lexsort((np.arange(norms.size), -norms))
    mT, mT1 = norms[order[T - 1]], norms[order[T]]
    assert mT - mT1 <= REL * mT, "channel choice differs outside a tie"
    assert np.all(np.diff(gpu_ch) > 0) and gpu_ch.size == T
    assert abs(norms[gpu_ch].sum() - norms[ref_ch].sum()) <= REL * norms[ref_ch].sum()
    return "tie"
