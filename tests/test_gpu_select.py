"""kvc_select_topk, kvc_compact, kvc_lmba_budget and kvc_channel_prune on the
GPU against the oracle, each in isolation on identical inputs (so every
integer result must be bit-exact), including the degenerate cases."""

import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_bf16_amd import workload as wk

from _parity import bits_of, check_channels, dev, to_dev

pytestmark = pytest.mark.gpu


def _kvc():
    from kv_cache_compression_bf16_amd import kvc
    return kvc


# ---------------------------------------------------------------- select
def _gpu_select(imp32, *, S, w, recent, budget):
    kvc = _kvc()
    t = torch.from_numpy(np.ascontiguousarray(imp32)).to(dev())
    idx = torch.full((imp32.shape[0], budget), -7, dtype=torch.int32, device=dev())
    kvc.kvc_select_topk(t, idx, S=S, w=w, recent=recent, budget=budget)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


def _ref_select(imp32, **kw):
    return oracle.select.select_heads(imp32.astype(np.float64), **kw)


@pytest.mark.parametrize("Hkv,S,w,recent,budget,kind", [
    (8, 2048, 32, 32, 256, "exp"),
    (8, 5000, 128, 64, 700, "exp"),
    (3, 1025 + 16, 16, 16, 300, "ties3"),       # n = 1025: one element past a 1024 chunk
    (4, 4000, 100, 300, 900, "exp"),            # recent > w: recent tokens leave the candidates
    (4, 4000, 300, 100, 900, "exp"),            # recent < w: window-only tokens are dropped
    (2, 3000, 10, 10, 10, "exp"),               # k_top = 0
    (2, 3000, 10, 10, 3000, "exp"),             # k_top = |C|: keep everything
    (2, 3000, 10, 10, 2999, "exp"),             # all but one
    (2, 3000, 10, 0, 500, "equal"),             # all scores equal -> lowest positions
    (2, 3000, 10, 5, 700, "zeros_denorm"),      # zeros and denormals
    (8, 131072, 64, 64, 26214, "exp"),          # the 131072-token long-context shape
    (4, 40000, 64, 64, 5000, "narrow"),         # near-uniform scores: a tiny key range, 2 rounds
    (4, 9000, 64, 64, 2000, "signed"),          # negative and positive scores
    (2, 9000, 64, 64, 1000, "wide"),            # keys spanning all 32 bits, +-inf included
    (2, 70016, 16, 16, 30000, "ties3"),         # three rounds; equal keys straddle round borders
    (3, 40016, 16, 16, 9000, "equal"),          # chunked path: one key everywhere -> lowest positions
    (2, 50064, 64, 64, 7000, "wide"),           # chunked path: full key range, +-inf
    (2, 45000, 10, 5, 20000, "zeros_denorm"),   # chunked path: zeros and denormals
    (8, 32768, 128, 64, 2048, "exp"),           # 32K-token GQA shape: the bin of T is ranked directly
    (4, 32768, 128, 64, 2048, "dups"),          # ~6 copies of each value: ties inside the ranked bin
    (2, 32768, 128, 64, 2048, "ties3"),         # the bin of T holds ~11K keys: every radix level
    (2, 32768, 128, 64, 2048, "narrow"),        # a tiny key range in one workgroup
    (2, 32768, 128, 0, 30000, "exp"),           # k_top close to the candidate count
    (3, 32767 + 128, 128, 0, 5, "dups"),        # 32767 candidates: the last wave part-filled
    (2, 32769 + 128, 128, 0, 3000, "exp"),      # 32769 candidates: the first count on the chunked path
    (2, 9000, 64, 64, 6000, "signed_zeros"),    # +0 and -0 tied at the threshold (one workgroup)
    (2, 40064, 64, 64, 26000, "signed_zeros"),  # the same on the chunked path
])
def test_select_bit_exact(Hkv, S, w, recent, budget, kind):
    rng = np.random.default_rng(S + budget)
    n = S - w
    if kind == "exp":
        imp = rng.exponential(size=(Hkv, n)).astype(np.float32)
    elif kind == "ties3":
        imp = (rng.integers(0, 3, size=(Hkv, n)) / 7.0).astype(np.float32)
    elif kind == "dups":
        imp = (rng.integers(0, 5000, size=(Hkv, n)) / 5000.0).astype(np.float32)
    elif kind == "equal":
        imp = np.full((Hkv, n), 1.0 / n, dtype=np.float32)
    elif kind == "narrow":
        imp = ((1.0 + 1e-4 * rng.standard_normal(size=(Hkv, n))) / n).astype(np.float32)
    elif kind == "signed":
        imp = rng.standard_normal(size=(Hkv, n)).astype(np.float32)
    elif kind == "signed_zeros":
        # half positive, a third +0.0, the rest -0.0: the kept set ends inside
        # the zeros, which count as equal (position order)
        imp = rng.exponential(size=(Hkv, n)).astype(np.float32)
        u = rng.random(size=(Hkv, n))
        imp[u < 0.5] = 0.0
        imp[u < 0.15] = -0.0
    elif kind == "wide":
        imp = rng.choice(np.array([-np.inf, -1e30, -1.0, -0.0, 0.0, 1e-30, 1.0, 1e30, np.inf],
                                  dtype=np.float32), size=(Hkv, n))
    else:
        imp = rng.choice(np.array([0.0, 1e-42, 3e-40, 1e-38, 0.5], dtype=np.float32), size=(Hkv, n))
    gpu = _gpu_select(imp, S=S, w=w, recent=recent, budget=budget)
    ref = _ref_select(imp, S=S, w=w, recent=recent, budget=budget)
    assert np.array_equal(gpu, ref)


def test_select_reads_only_candidates_with_head_stride():
    kvc = _kvc()
    Hkv, S, w, recent, budget = 3, 2000, 50, 100, 400
    n = S - w
    rng = np.random.default_rng(4)
    big = rng.exponential(size=(Hkv, n + 37)).astype(np.float32)
    big[:, S - recent:] = 1e9          # beyond the candidates (r > w): must be ignored
    t = torch.from_numpy(big).to(dev())[:, :n]
    idx = torch.empty((Hkv, budget), dtype=torch.int32, device=dev())
    kvc.kvc_select_topk(t, idx, S=S, w=w, recent=recent, budget=budget)
    ref = _ref_select(big[:, :n], S=S, w=w, recent=recent, budget=budget)
    assert np.array_equal(idx.cpu().numpy(), ref)


# ---------------------------------------------------------------- pooling
@pytest.mark.parametrize("rows,n,kernel,mode", [
    (8, 32640, 7, 0), (8, 32640, 7, 1),
    (3, 1025, 1, 0), (3, 1025, 255, 0), (3, 1025, 255, 1),   # identity and the widest window
    (2, 5, 9, 0), (2, 5, 9, 1),                              # window wider than the row
    (5, 131008, 31, 0),
])
def test_pool_matches_oracle(rows, n, kernel, mode):
    kvc = _kvc()
    rng = np.random.default_rng(n + kernel + mode)
    x = rng.exponential(size=(rows, n)).astype(np.float32) / n
    if mode == 1:
        x -= np.float32(1.0 / n)                             # signed values: max must ignore the padding
    t = torch.from_numpy(x).to(dev())
    out = torch.full_like(t, float("nan"))
    kvc.kvc_pool_importance(t, out, kernel=kernel, mode=mode)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = oracle.pool.pool(x.astype(np.float64), kernel, mode)
    if mode == 1:
        assert np.array_equal(got, ref)                      # a max picks an input value exactly
    else:
        # fp32: kernel - 1 sequential additions of positive terms and one division
        rel = (kernel + 2) * 2.0 ** -24
        assert np.all(np.abs(got - ref) <= rel * np.abs(ref) + 1e-38)


# ---------------------------------------------------------------- compact
@pytest.mark.parametrize("D", [128, 96, 8])   # 4-rows-per-thread path (128, 8) and chunk path (96)
def test_compact_bit_exact_and_bad_index_fill(D):
    kvc = _kvc()
    rng = np.random.default_rng(0)
    Hkv, S, B = 4, 3000, 333
    k = rng.integers(0, 65536, size=(Hkv, S + 10, D), dtype=np.uint16)
    v = rng.integers(0, 65536, size=(Hkv, S, D), dtype=np.uint16)
    idx = np.stack([np.sort(rng.choice(S, B, replace=False)) for _ in range(Hkv)]).astype(np.int32)
    idx[2, 5] = S + 3                  # out of range -> NaN row, no read
    kd, vd = to_dev(k), to_dev(v)
    idd = torch.from_numpy(idx).to(dev())
    ko = torch.empty((Hkv, B, D), dtype=torch.bfloat16, device=dev())
    vo = torch.empty((Hkv, B, D), dtype=torch.bfloat16, device=dev())
    kvc.kvc_compact(kd, vd, idd, ko, vo, S=S)
    kob, vob = bits_of(ko), bits_of(vo)
    good = idx.copy(); good[2, 5] = 0
    ref_k = oracle.compact.compact(k, good)
    ref_v = oracle.compact.compact(v, good)
    ref_k[2, 5] = 0xFFFF
    ref_v[2, 5] = 0xFFFF
    assert np.array_equal(kob, ref_k) and np.array_equal(vob, ref_v)
    ko2 = torch.empty_like(ko)
    kvc.kvc_compact(kd, None, idd, ko2, None, S=S)
    assert np.array_equal(bits_of(ko2), ref_k)


# ---------------------------------------------------------------- lmba budgets
def _rows(L, Hkv, n, seed):
    rng = np.random.default_rng(seed)
    conc = rng.uniform(0.2, 6.0, size=(L, 1, 1))
    x = rng.standard_normal((L, Hkv, n)) * conc
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def _gpu_budget(imp, **kw):
    kvc = _kvc()
    L, Hkv, n = imp.shape
    t = torch.from_numpy(imp).to(dev())
    b = torch.empty(L, dtype=torch.int32, device=dev())
    m = torch.empty((L, Hkv), dtype=torch.int32, device=dev())
    kvc.kvc_lmba_budget(t, b, mba=m, **kw)
    torch.cuda.synchronize()
    return m.cpu().numpy(), b.cpu().numpy()


@pytest.mark.parametrize("L,Hkv,n,total,floor,cap,seed", [
    (32, 8, 16256, 32 * 1024, 128, 16384, 0),
    (5, 3, 1000, 2000, 50, 1000, 1),
    (1, 2, 77, 40, 10, 77, 2),
    (7, 4, 4096, 7 * 3000, 100, 3500, 3),     # forces capacity clamping
    (3, 9, 500, 3 * 200, 50, 500, 5),         # nine KV heads: two steps of MBA loads per layer
    (70, 9, 300, 70 * 100, 20, 300, 4),       # more layers than one wave allocates
    (2, 3, 20000, 2 * 6000, 100, 20000, 6),   # rows longer than the MBA kernel keeps in registers
])
def test_budgets_bit_exact(L, Hkv, n, total, floor, cap, seed):
    imp = _rows(L, Hkv, n, seed)
    mba, bud = _gpu_budget(imp, total_budget=total, floor_per_layer=floor, capacity=cap)
    ref_mba, ref_b = oracle.budget.zigzag_budgets(imp.astype(np.float64), total_budget=total, floor=floor,
                                                  capacity=cap)
    assert np.array_equal(mba, np.array(ref_mba))
    assert bud.tolist() == ref_b
    assert bud.sum() == total and bud.min() >= floor and bud.max() <= cap


def test_budget_degenerate_rows():
    n = 1000
    imp = np.zeros((4, 2, n), dtype=np.float32)
    imp[0] = 1.0 / n                     # uniform: ceil(0.9 n) = 900
    imp[1, :, 17] = 1.0                  # one-hot: 1
    imp[2, 0, :] = 0.0                   # all zero: 0
    imp[2, 1, :10] = 0.1                 # ten equal values: 9
    imp[3] = np.float32(1e-40)           # denormals only
    mba, bud = _gpu_budget(imp, total_budget=1000, floor_per_layer=100, capacity=n)
    ref_mba, ref_b = oracle.budget.zigzag_budgets(imp.astype(np.float64), total_budget=1000, floor=100,
                                                  capacity=n)
    assert mba.tolist() == ref_mba
    assert bud.tolist() == ref_b


def test_budget_mixed_magnitudes():
    # the 90% crossing lands among thousands of tiny scores below one large one,
    # and rows span many decades (the MBA search keeps masses in 64-bit fixed point)
    n = 16256
    rng = np.random.default_rng(7)
    imp = np.zeros((3, 4, n), dtype=np.float32)
    imp[0, :, :] = 3e-5
    imp[0, :, 123] = 0.5
    imp[1] = (10.0 ** rng.uniform(-12, 0, size=(4, n))).astype(np.float32)
    imp[2] = rng.exponential(size=(4, n)).astype(np.float32) ** 6
    imp /= imp.sum(axis=-1, keepdims=True)
    mba, bud = _gpu_budget(imp, total_budget=3 * 4000, floor_per_layer=128, capacity=n)
    ref_mba, ref_b = oracle.budget.zigzag_budgets(imp.astype(np.float64), total_budget=3 * 4000, floor=128,
                                                  capacity=n)
    assert mba.tolist() == ref_mba
    assert bud.tolist() == ref_b


@pytest.mark.parametrize("mass", [1.0, 0.5])
def test_budgets_other_mass_fractions(mass):
    # mass = 1 needs every score whose fixed-point mass is nonzero (the target is the exact
    # total); mass = 0.5 crosses well inside the row
    if mass == 1.0:
        # well-conditioned rows: every nonzero score is far above both the fixed-point
        # resolution and the fp64 rounding of the oracle's total, and some scores are 0
        rng = np.random.default_rng(11)
        imp = rng.uniform(0.1, 1.0, size=(4, 3, 3000))
        imp[rng.random(imp.shape) < 0.2] = 0.0
        imp = (imp / imp.sum(axis=-1, keepdims=True)).astype(np.float32)
    else:
        imp = _rows(4, 3, 3000, 12)
    mba, bud = _gpu_budget(imp, total_budget=4 * 1200, floor_per_layer=64, capacity=3000, mass=mass)
    ref_mba, ref_b = oracle.budget.zigzag_budgets(imp.astype(np.float64), total_budget=4 * 1200, floor=64,
                                                  capacity=3000, mass=mass)
    assert np.array_equal(mba, np.array(ref_mba))
    assert bud.tolist() == ref_b
    if mass == 1.0:
        assert np.array_equal(mba, (imp > 0).sum(axis=-1))


def test_budget_negative_zero_is_zero():
    # -0.0 is a zero score, not the largest key
    n = 500
    imp = _rows(2, 2, n, 13)
    imp[:, :, ::7] = np.float32(-0.0)
    imp[1, 1, :] = np.float32(-0.0)
    imp[1, 1, 42] = 1.0
    mba, bud = _gpu_budget(imp, total_budget=2 * 200, floor_per_layer=10, capacity=n)
    ref_mba, ref_b = oracle.budget.zigzag_budgets(imp.astype(np.float64), total_budget=2 * 200, floor=10,
                                                  capacity=n)
    assert np.array_equal(mba, np.array(ref_mba))
    assert mba[1, 1] == 1
    assert bud.tolist() == ref_b


def test_budget_equal_lmba_is_uniform():
    imp = np.tile(_rows(1, 4, 2048, 9), (6, 1, 1))
    _, bud = _gpu_budget(imp, total_budget=6 * 500, floor_per_layer=64, capacity=2048)
    assert bud.tolist() == [500] * 6


# ---------------------------------------------------------------- ThinK
@pytest.mark.parametrize("Hkv,B,recent,lam,p", [
    (8, 2000, 64, 0.4, 2),
    (4, 1500, 32, 0.5, 1),
    (2, 513, 1, 0.3, 2),
    (3, 100, 100, 0.4, 2),      # no prunable rows
    (2, 700, 0, 0.0, 2),        # lambda 0 keeps every channel
])
def test_channel_prune_bit_exact(Hkv, B, recent, lam, p):
    kvc = _kvc()
    rng = np.random.default_rng(B)
    x = rng.standard_normal((Hkv, B, 128), dtype=np.float32)
    x[:, :, [5, 66, 99, 127]] *= 8
    kc = wk.f32_to_bf16_bits(x)
    T = oracle.sizes.think_channels(128, lam)
    rows = B - recent
    ch = torch.empty((Hkv, T), dtype=torch.int32, device=dev())
    mask = torch.empty((Hkv, 128), dtype=torch.uint8, device=dev())
    kp = torch.empty((Hkv, rows, T), dtype=torch.bfloat16, device=dev())
    kvc.kvc_channel_prune(to_dev(kc), ch, kp, recent=recent, lam=lam, p=p, mask=mask)
    torch.cuda.synchronize()
    ref_ch, ref_mask, _, norms = oracle.think.think_prune(oracle.score.bf16_bits_to_f64(kc), recent=recent,
                                                         lam=lam, p=p)
    gch = ch.cpu().numpy()
    for g in range(Hkv):
        check_channels(gch[g], norms[g], ref_ch[g], T)
        assert np.array_equal(mask.cpu().numpy()[g], np.isin(np.arange(128), gch[g]).astype(np.uint8))
    kpb = bits_of(kp)
    for g in range(Hkv):
        assert np.array_equal(kpb[g], kc[g, :rows][:, gch[g]])


@pytest.mark.parametrize("Hkv,G,w,wpad,B,recent,lam,loud", [
    (8, 4, 32, 0, 2000, 64, 0.4, False),
    (2, 1, 17, 0, 513, 1, 0.3, False),        # w not a multiple of the 16 row lanes
    (3, 2, 8, 0, 100, 100, 0.4, False),       # no prunable rows: every score is 0, lowest channels win
    (2, 8, 16, 0, 700, 0, 0.0, False),        # lambda 0 keeps every channel
    (4, 4, 24, 40, 1500, 32, 0.5, True),      # window rows a slice of a longer query block; per-group loud channels
])
def test_channel_prune_query(Hkv, G, w, wpad, B, recent, lam, loud):
    kvc = _kvc()
    rng = np.random.default_rng(B + w)
    x = rng.standard_normal((Hkv, B, 128), dtype=np.float32)
    x[:, :, [5, 66, 99, 127]] *= 8
    qf = rng.standard_normal((Hkv * G, w + wpad, 128), dtype=np.float32)
    if loud:
        qf[:, :, 66] = 0.0                                    # an outlier key channel no query uses
        for g in range(Hkv):
            qf[g * G:(g + 1) * G, :, [10 + g, 40 + 2 * g]] *= 16.0
    kc, qb = wk.f32_to_bf16_bits(x), wk.f32_to_bf16_bits(qf)
    T = oracle.sizes.think_channels(128, lam)
    rows = B - recent
    ch = torch.empty((Hkv, T), dtype=torch.int32, device=dev())
    mask = torch.empty((Hkv, 128), dtype=torch.uint8, device=dev())
    kp = torch.empty((Hkv, rows, T), dtype=torch.bfloat16, device=dev())
    qd = to_dev(qb)[:, wpad:, :]                              # head stride (w + wpad) * D
    kvc.kvc_channel_prune_query(to_dev(kc), qd, ch, kp, recent=recent, lam=lam, mask=mask)
    torch.cuda.synchronize()
    ref_ch, _, _, scores = oracle.think.think_prune_query(oracle.score.bf16_bits_to_f64(kc),
                                                          oracle.score.bf16_bits_to_f64(qb[:, wpad:, :]),
                                                          recent=recent, lam=lam)
    gch = ch.cpu().numpy()
    gmask = mask.cpu().numpy()
    kpb = bits_of(kp)
    for g in range(Hkv):
        check_channels(gch[g], scores[g], ref_ch[g], T)
        assert np.array_equal(gmask[g], np.isin(np.arange(128), gch[g]).astype(np.uint8))
        assert np.array_equal(kpb[g], kc[g, :rows][:, gch[g]])
        if loud:
            assert 66 not in gch[g] and {10 + g, 40 + 2 * g} <= set(gch[g].tolist())


@pytest.mark.parametrize("Hkv,G,w,B,recent,lam,loud", [
    (8, 4, 32, 2000, 64, 0.4, False),      # 1936 rows: 4 key splits, ragged last tile
    (2, 1, 17, 513, 1, 0.3, False),        # a partial query block
    (3, 2, 8, 100, 100, 0.4, False),       # no prunable rows: every score is 0, lowest channels win
    (2, 8, 64, 700, 0, 0.0, False),        # R = 512: several query groups; lambda 0 keeps every channel
    (4, 4, 24, 1500, 32, 0.5, True),       # loud value channels are always kept
])
def test_channel_prune_value(Hkv, G, w, B, recent, lam, loud):
    kvc = _kvc()
    print(f"[value prune] Hkv={Hkv} G={G} w={w} B={B} r={recent} lam={lam}", flush=True)
    rng = np.random.default_rng(B + 7 * w)
    k = rng.standard_normal((Hkv, B, 128), dtype=np.float32)
    v = rng.standard_normal((Hkv, B, 128), dtype=np.float32)
    q = rng.standard_normal((Hkv * G, w, 128), dtype=np.float32)
    loud_ch = [3, 50, 97]
    if loud:
        v[:, :, loud_ch] *= 8.0
    kb, vb, qb = wk.f32_to_bf16_bits(k), wk.f32_to_bf16_bits(v), wk.f32_to_bf16_bits(q)
    T = oracle.sizes.think_channels(128, lam)
    rows = B - recent
    ch = torch.empty((Hkv, T), dtype=torch.int32, device=dev())
    mask = torch.empty((Hkv, 128), dtype=torch.uint8, device=dev())
    vp = torch.empty((Hkv, rows, T), dtype=torch.bfloat16, device=dev())
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    kvc.kvc_channel_prune_value(to_dev(kb), to_dev(vb), to_dev(qb), ch, vp, recent=recent, lam=lam, scale=scale,
                                mask=mask)
    torch.cuda.synchronize()
    f64 = oracle.score.bf16_bits_to_f64
    ref_ch, _, _, scores = oracle.think.think_prune_value(f64(kb), f64(vb), f64(qb), recent=recent, lam=lam,
                                                          scale=scale)
    gch, gmask, vpb = ch.cpu().numpy(), mask.cpu().numpy(), bits_of(vp)
    kinds = []
    for g in range(Hkv):
        kinds.append(check_channels(gch[g], scores[g], ref_ch[g], T))
        assert np.array_equal(gmask[g], np.isin(np.arange(128), gch[g]).astype(np.uint8))
        assert np.array_equal(vpb[g], vb[g, :rows][:, gch[g]])
        if loud:
            assert set(loud_ch) <= set(gch[g].tolist())
    print("channels:", kinds)


def test_select_and_compact_layers_batched():
    # all layers in one launch each, budgets on the device: identical to per-layer calls
    kvc = _kvc()
    rng = np.random.default_rng(61)
    L, Hkv, S, w, recent, D = 5, 3, 3000, 64, 64, 128
    n = S - w
    imp = rng.exponential(size=(L, Hkv, n)).astype(np.float32)
    imp[1, 1, :500] = 1.0                                    # ties across the cut in one row
    budgets = np.array([64, 500, 1, 2936 + 64, 130], dtype=np.int32)   # incl. k_top = 0 and k_top = c
    budgets[2] = 64                                          # (k_top = 0)
    tot = int(budgets.sum())
    k = wk.f32_to_bf16_bits(rng.standard_normal((L, Hkv, S, D), dtype=np.float32))
    v = wk.f32_to_bf16_bits(rng.standard_normal((L, Hkv, S, D), dtype=np.float32))
    imp_t = torch.from_numpy(imp).to(dev())
    b_t = torch.from_numpy(budgets).to(dev())
    idx = torch.full((Hkv * tot + 7,), -9, dtype=torch.int32, device=dev())
    ko = torch.zeros((Hkv * tot + 7, D), dtype=torch.int16, device=dev())
    vo = torch.zeros((Hkv * tot + 7, D), dtype=torch.int16, device=dev())
    kvc.kvc_select_topk_layers(imp_t, b_t, idx, S=S, w=w, recent=recent, total_budget=tot)
    kvc.kvc_compact_layers(to_dev(k), to_dev(v), b_t, idx, ko, vo, S=S, total_budget=tot)
    torch.cuda.synchronize()
    gi, gk, gv = idx.cpu().numpy(), bits_of(ko), bits_of(vo)
    off = 0
    for l in range(L):
        B = int(budgets[l])
        ref = _ref_select(imp[l], S=S, w=w, recent=recent, budget=B)
        got = gi[off * Hkv:(off + B) * Hkv].reshape(Hkv, B)
        assert np.array_equal(got, ref), f"layer {l}"
        assert np.array_equal(gk[off * Hkv:(off + B) * Hkv].reshape(Hkv, B, D), oracle.compact.compact(k[l], ref))
        assert np.array_equal(gv[off * Hkv:(off + B) * Hkv].reshape(Hkv, B, D), oracle.compact.compact(v[l], ref))
        off += B
    assert np.all(gi[Hkv * tot:] == -9)                     # nothing past the blocks
    assert np.all(gk[Hkv * tot:] == 0)
