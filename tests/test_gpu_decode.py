"""Keyformer decode step and score hand-over on the GPU against the oracle.

Each step runs on the GPU from a host state and the oracle steps from the same
state: the evicted slot must be the oracle's (or, in a tie, a valid candidate
whose accumulated score is within 1e-5 of the oracle's choice), positions and
K/V bits must then match exactly, and the accumulated scores agree within
2e-6 relative (fp32 against fp64).  The next step starts from the GPU's state.
"""

import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_bf16_amd import workload as wk

from _parity import bits_of, dev, to_dev

pytestmark = pytest.mark.gpu


def _kvc():
    from kv_cache_compression_bf16_amd import kvc
    return kvc


def _random_state(rng, Hkv, B, D, t0, recent):
    kc = wk.f32_to_bf16_bits(rng.standard_normal((Hkv, B, D), dtype=np.float32))
    vc = wk.f32_to_bf16_bits(rng.standard_normal((Hkv, B, D), dtype=np.float32))
    pos = np.stack([np.sort(rng.choice(t0 - recent, size=B - recent, replace=False)) for _ in range(Hkv)])
    pos = np.concatenate([pos, np.tile(np.arange(t0 - recent, t0), (Hkv, 1))], axis=1)   # the prompt's window
    return kc, vc, pos.astype(np.int32)


def _gpu_step(state, q, kn, vn, *, t, recent, tau, seed, scale):
    kvc = _kvc()
    kc, vc, pos, acc = state
    kc_t, vc_t = to_dev(kc), to_dev(vc)
    pos_t = torch.from_numpy(pos.astype(np.int32)).to(dev())
    acc_t = torch.from_numpy(acc.astype(np.float32)).to(dev())
    ev = torch.full((kc.shape[0],), -7, dtype=torch.int32, device=dev())
    kvc.kvc_keyformer_decode_step(to_dev(q), to_dev(kn), to_dev(vn), kc_t, vc_t, pos_t, acc_t, t=t, recent=recent,
                                  tau=tau, seed=seed, scale=scale, evicted=ev)
    torch.cuda.synchronize()
    return (bits_of(kc_t), bits_of(vc_t), pos_t.cpu().numpy(), acc_t.cpu().numpy()), ev.cpu().numpy()


def _run_steps(rng, *, Hkv, G, B, recent, steps, tau, acc0, seed=11):
    D, t0 = 128, 20000
    scale = float(np.float32(1.0 / np.sqrt(D)))
    kc, vc, pos = _random_state(rng, Hkv, B, D, t0, recent)
    state = (kc, vc, pos, acc0(rng, Hkv, B).astype(np.float32))
    kinds = []
    for s in range(steps):
        t = t0 + s
        print(f"[decode] Hkv={Hkv} G={G} B={B} r={recent} tau={tau} step {s}", flush=True)
        q = wk.f32_to_bf16_bits(rng.standard_normal((Hkv * G, D), dtype=np.float32))
        kn = wk.f32_to_bf16_bits(rng.standard_normal((Hkv, D), dtype=np.float32))
        vn = wk.f32_to_bf16_bits(rng.standard_normal((Hkv, D), dtype=np.float32))
        new, ev = _gpu_step(state, q, kn, vn, t=t, recent=recent, tau=tau, seed=seed, scale=scale)
        kc, vc, pos, acc = state
        f64 = oracle.score.bf16_bits_to_f64
        rk, rv, rp, ra, rev = oracle.decode.decode_step(kc, vc, pos, acc.astype(np.float64), f64(q), kn, vn, t=t,
                                                        recent=recent, scale=scale, tau=tau, seed=seed)
        for g in range(Hkv):
            if ev[g] != rev[g]:
                # tie: both candidates' accumulated scores (oracle) within 1e-5
                keys = np.concatenate([f64(kc[g]), f64(kn[g])[None]])
                sc = oracle.decode.step_scores(keys, np.concatenate([pos[g], [t]]), f64(q[g * G:(g + 1) * G]),
                                               t=t, heads=range(g * G, (g + 1) * G), scale=scale, tau=tau,
                                               seed=seed)
                a = acc[g].astype(np.float64) + sc[:B]
                assert pos[g, ev[g]] <= t - recent, "a recent token was evicted"
                assert abs(a[ev[g]] - a[rev[g]]) <= 1e-5 * max(a[rev[g]], 1e-30), \
                    f"head {g}: evicted slot {ev[g]} vs {rev[g]} outside a tie"
                kinds.append("tie")
                continue
            kinds.append("exact")
            assert np.array_equal(new[2][g], rp[g])
            assert np.array_equal(new[0][g], rk[g]) and np.array_equal(new[1][g], rv[g])
            assert np.allclose(new[3][g], ra[g], rtol=2e-6, atol=1e-9)
        state = new
    return kinds


@pytest.mark.parametrize("Hkv,G,B,recent,steps,tau", [
    (4, 2, 600, 32, 12, 1.0),
    (2, 1, 4096, 512, 4, 1.0e4),       # Keyformer's cache and window sizes, the other temperature
    (3, 8, 4095, 100, 2, 1.0),         # G = 8, the widest query group
    (2, 8, 6000, 64, 2, 1.0),          # G * (B + 1) = 48008 logits per head, 24 key chunks
    (2, 4, 257, 1, 6, 0.5),            # window of one token
    (2, 2, 5000, 128, 3, 1.0),         # 4096 < B <= 8192 with G <= 4: eight slots per update thread
    (1, 1, 9000, 64, 2, 1.0),          # B > 8192: the update's strided loops
])
def test_decode_steps_match_oracle(Hkv, G, B, recent, steps, tau):
    rng = np.random.default_rng(B + G)
    kinds = _run_steps(rng, Hkv=Hkv, G=G, B=B, recent=recent, steps=steps, tau=tau,
                       acc0=lambda r, h, b: r.exponential(size=(h, b)) * 1e-3)
    print("evictions:", kinds)


def test_decode_uniform_scores_are_fifo():
    # tau = inf and zero initial scores: every slot gains G / (B + 1) per step and
    # the oldest prompt tokens leave first, identically on both sides
    rng = np.random.default_rng(77)
    kinds = _run_steps(rng, Hkv=2, G=2, B=300, recent=20, steps=10, tau=np.inf,
                       acc0=lambda r, h, b: np.zeros((h, b)))
    assert set(kinds) == {"exact"}


def test_decode_init_scores_bit_exact():
    kvc = _kvc()
    rng = np.random.default_rng(5)
    Hkv, n, B = 5, 3000, 700
    imp = rng.random((Hkv, n + 13), dtype=np.float32)
    idx = np.stack([np.sort(rng.choice(n + 100, size=B, replace=False)) for _ in range(Hkv)]).astype(np.int32)
    acc = torch.full((Hkv, B), -1.0, dtype=torch.float32, device=dev())
    imp_t = torch.from_numpy(imp).to(dev())[:, :n + 13]
    kvc.kvc_decode_init_scores(imp_t, torch.from_numpy(idx).to(dev()), acc, n=n)
    torch.cuda.synchronize()
    ref = oracle.decode.initial_scores(imp.astype(np.float64), idx, n)
    assert np.array_equal(acc.cpu().numpy().astype(np.float64), ref)
