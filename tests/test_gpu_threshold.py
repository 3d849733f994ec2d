"""kvc_select_threshold and kvc_compact_ragged on the GPU against the oracle,
in isolation on identical fp32 scores (the keep decision is an fp32 compare on
both sides, so the packed indices and offsets must be bit-exact), including
the degenerate cases: nothing or everything kept, no candidates, NaN scores,
scores equal to the threshold, truncation of the gather at max_rows."""

import numpy as np
import pytest
import torch

import oracle

from _parity import bits_of, dev, to_dev

pytestmark = pytest.mark.gpu


def _kvc():
    from kv_cache_compression_bf16_amd import kvc
    return kvc


def _gpu_threshold(sc32, *, S, w, recent, theta, pad=0):
    kvc = _kvc()
    Hkv, n = sc32.shape
    full = np.zeros((Hkv, n + pad), dtype=np.float32)
    full[:, :n] = sc32
    t = torch.from_numpy(full).to(dev())[:, :n]            # row stride n + pad
    c = min(S - w, S - recent)
    idx = torch.full((Hkv * (c + recent),), -7, dtype=torch.int32, device=dev())
    off = torch.full((Hkv + 1,), -7, dtype=torch.int32, device=dev())
    kvc.kvc_select_threshold(t, idx, off, S=S, w=w, recent=recent, threshold=theta)
    torch.cuda.synchronize()
    off_h = off.cpu().numpy()
    return idx.cpu().numpy()[:max(off_h[-1], 0)], off_h


def _check(sc32, *, S, w, recent, theta, pad=0):
    print(f"[threshold] Hkv={sc32.shape[0]} S={S} w={w} r={recent} theta={theta}", flush=True)
    gi, go = _gpu_threshold(sc32, S=S, w=w, recent=recent, theta=theta, pad=pad)
    ri, ro = oracle.threshold.select_threshold_heads(sc32, S=S, w=w, recent=recent, theta=np.float32(theta))
    assert np.array_equal(go, ro), (go, ro)
    assert np.array_equal(gi, ri)
    return go


@pytest.mark.parametrize("Hkv,S,w,recent,q", [
    (8, 5000, 128, 64, 0.9),              # c = 4872: one full chunk and a ragged tail
    (3, 3 * 4096 + 200 + 32, 32, 32, 0.5),   # three full chunks + 200
    (5, 4097 + 16, 16, 16, 0.0),          # theta at the minimum: every candidate kept
    (4, 2000, 100, 300, 0.7),             # recent > w: the recent tokens leave the candidates
    (2, 300, 20, 0, 0.95),                # no recent window
    (1, 129, 1, 1, 0.5),
])
def test_threshold_bit_exact(Hkv, S, w, recent, q):
    rng = np.random.default_rng(S + Hkv)
    n = S - w
    sc = rng.exponential(size=(Hkv, n)).astype(np.float32)
    c = min(S - w, S - recent)
    theta = float(np.quantile(sc[:, :c], q)) if c else 0.0
    _check(sc, S=S, w=w, recent=recent, theta=theta)


def test_threshold_extremes_and_degenerate():
    rng = np.random.default_rng(3)
    Hkv, S, w, r = 6, 9000, 64, 64
    sc = rng.exponential(size=(Hkv, S - w)).astype(np.float32)
    sc[2] *= 1e-6                                         # head 2 keeps only its recent window
    off = _check(sc, S=S, w=w, recent=r, theta=1.0)
    assert off[3] - off[2] == r
    _check(sc, S=S, w=w, recent=r, theta=-np.inf)         # everything
    off = _check(sc, S=S, w=w, recent=r, theta=np.inf)    # only the recent windows
    assert np.array_equal(np.diff(off), np.full(Hkv, r))
    _check(sc, S=S, w=w, recent=S, theta=0.0)             # c = 0: no candidates at all
    off = _check(sc, S=S, w=w, recent=0, theta=np.inf)    # nothing kept anywhere
    assert np.all(off == 0)


def test_threshold_nan_equal_and_stride():
    rng = np.random.default_rng(4)
    Hkv, S, w, r = 40, 6000, 128, 32
    sc = rng.integers(0, 8, size=(Hkv, S - w)).astype(np.float32) * 0.25     # many scores equal theta
    sc[rng.random(sc.shape) < 0.01] = np.nan
    _check(sc, S=S, w=w, recent=r, theta=1.0, pad=37)                           # odd row stride


@pytest.mark.parametrize("D,with_v", [(128, True), (64, False), (256, True)])
def test_compact_ragged_bit_exact(D, with_v):
    kvc = _kvc()
    rng = np.random.default_rng(D)
    Hkv, S, w, r = 5, 3000, 64, 64
    sc = rng.exponential(size=(Hkv, S - w)).astype(np.float32)
    sc[1] *= 1e-6
    gi, go = _gpu_threshold(sc, S=S, w=w, recent=r, theta=1.5)
    total = int(go[-1])
    k = rng.integers(0, 2 ** 16, size=(Hkv, S, D), dtype=np.uint16)
    v = rng.integers(0, 2 ** 16, size=(Hkv, S, D), dtype=np.uint16)
    idx_t = torch.from_numpy(gi.astype(np.int32)).to(dev())
    off_t = torch.from_numpy(go.astype(np.int32)).to(dev())
    for max_rows in (total, total - 37):                   # exact size, then truncated
        print(f"[compact_ragged] D={D} v={with_v} rows={max_rows}/{total}", flush=True)
        big_k = torch.full((total + 8, D), -1, dtype=torch.int16, device=dev())
        big_v = torch.full((total + 8, D), -1, dtype=torch.int16, device=dev())
        ko, vo = big_k[:max_rows], (big_v[:max_rows] if with_v else None)
        kvc.kvc_compact_ragged(to_dev(k), to_dev(v) if with_v else None, idx_t[:max_rows], off_t, ko, vo, S=S)
        torch.cuda.synchronize()
        ref_k = oracle.threshold.compact_ragged(k, gi, go)
        got = bits_of(big_k)
        assert np.array_equal(got[:max_rows], ref_k[:max_rows])
        assert np.all(got[max_rows:] == 0xFFFF)             # nothing written past max_rows
        if with_v:
            ref_v = oracle.threshold.compact_ragged(v, gi, go)
            gv = bits_of(big_v)
            assert np.array_equal(gv[:max_rows], ref_v[:max_rows])
            assert np.all(gv[max_rows:] == 0xFFFF)
