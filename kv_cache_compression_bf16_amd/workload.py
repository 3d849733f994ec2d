"""Seeded synthetic workloads for prompt KV-cache compression.

This module only draws random inputs; it holds none of the compression
arithmetic.  Both the HIP path (through the tests and the bench) and the CPU
oracle consume exactly these arrays.

Recipe (per tensor): numpy ``Generator(PCG64(SeedSequence([seed, cfg_id,
tensor_id, layer])))``, ``standard_normal(dtype=float32)``, rounded to bf16 with
round-to-nearest-even and kept as raw uint16 bit patterns.  tensor_id: Q=0,
K=1, V=2, per-layer logit scales=3, outlier key channels=4; decode-phase rows of
step s (layer = s): query=5, key=6, value=7.

* Only the observation-window queries Q_obs [H, w, D] are drawn (the prefix
  queries are never used by the method).
* Outlier key channels (the key-magnitude imbalance the ThinK page observes):
  ``outliers`` distinct channels, shared by all heads and layers, multiplied by
  ``outlier_gain`` (a power of two, so the scaling is exact in bf16).
* Per-layer logit scale (the 32-layer ZigZag workload): s_l ~ U[lo, hi) in
  float64, passed on as alpha_l = float32(s_l / sqrt(D)), so attention
  concentration and LMBA vary by layer.
"""

from dataclasses import dataclass, field, replace
import math

import numpy as np

Q_ID, K_ID, V_ID, SCALE_ID, OUTLIER_ID = 0, 1, 2, 3, 4
DEC_Q_ID, DEC_K_ID, DEC_V_ID = 5, 6, 7


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    L: int
    H: int
    Hkv: int
    S: int
    w: int
    recent: int
    D: int = 128
    budget: int = 0                 # tokens per KV head incl. recent (uniform budgets)
    total_budget: int = 0           # ZigZag: sum over layers of per-head budgets
    floor: int = 0                  # ZigZag per-layer floor
    mass: float = 0.9               # MBA attention-mass fraction
    outliers: int = 0
    outlier_gain: float = 8.0
    scale_range: tuple = ()         # (lo, hi) for per-layer logit scales, else ()
    gumbel: bool = False
    taus: tuple = (1.0,)
    noise_seed: int = 0
    think_lambda: float = -1.0      # < 0: no channel pruning
    think_p: int = 2
    think_query: bool = False       # query-driven ThinK score (window queries x keys) instead of l_p norms
    think_value_lambda: float = -1.0   # >= 0: ThinK value-channel pruning after the key pruning
    pool_kernel: int = 0            # SnapKV 1D pooling of the importance before top-k (0: off)
    pool_mode: int = 0              # 0: average (zero padding, / kernel), 1: max
    threshold: float = 0.0          # > 0: KVzap threshold selection at threshold * G / (S - w), not top-k
    decode_steps: int = 0           # > 0: Keyformer decode steps after the prompt phase (positions S, S+1, ...)
    causal: bool = False            # causal scoring: window row i (position S - w + i) over keys [0, S)
    seed: int = 0
    notes: str = field(default="", compare=False)

    @property
    def G(self):
        return self.H // self.Hkv

    @property
    def n(self):
        return self.S - self.w

    @property
    def imp_len(self):
        """Keys an importance row covers: the prefix, or (causal) the whole prompt."""
        return self.S if self.causal else self.S - self.w

    @property
    def select_w(self):
        """The window argument of the selection: candidates [0, min(S - select_w, S - recent))."""
        return self.recent if self.causal else self.w

    @property
    def n_candidates(self):
        return min(self.S - self.select_w, self.S - self.recent)

    @property
    def capacity(self):
        return self.n_candidates + self.recent

    @property
    def theta(self):
        """The threshold in importance units (float32), for threshold selection."""
        return float(np.float32(self.threshold * self.G / self.n))

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    "snapkv_mha8_s2048": Workload(
        name="snapkv_mha8_s2048", cfg_id=0, L=1, H=8, Hkv=8, S=2048, w=32, recent=32, budget=256,
        notes="tiny SnapKV, MHA 8 heads, uniform budget 256 incl. 32 recent"),
    "gqa32x8_s32768": Workload(
        name="gqa32x8_s32768", cfg_id=1, L=1, H=32, Hkv=8, S=32768, w=128, recent=64, budget=2048,
        outliers=4,
        notes="Llama-3-8B-shaped layer, GQA 32/8, 4 outlier key channels x8, budget 2048 incl. 64 recent"),
    "gqa32x8_s32768_pool7": Workload(
        name="gqa32x8_s32768_pool7", cfg_id=1, L=1, H=32, Hkv=8, S=32768, w=128, recent=64, budget=2048,
        outliers=4, pool_kernel=7, pool_mode=0,
        notes="the GQA layer above (same inputs) with SnapKV's average pooling (kernel 7) before top-k"),
    "think_s131072_kv": Workload(
        name="think_s131072_kv", cfg_id=4, L=1, H=8, Hkv=8, S=131072, w=64, recent=64,
        budget=int(0.2 * 131072), outliers=4, think_lambda=0.3, think_query=True, think_value_lambda=0.3,
        notes="the long-context case above (same inputs) with query-driven key and value channel pruning, "
              "lambda 0.3 each"),
    "gqa32x8_s32768_thr2": Workload(
        name="gqa32x8_s32768_thr2", cfg_id=1, L=1, H=32, Hkv=8, S=32768, w=128, recent=64,
        outliers=4, threshold=2.0,
        notes="the GQA layer above (same inputs) with KVzap's threshold rule at twice the uniform share, "
              "packed per-head output"),
    "zigzag_l32_s16384": Workload(
        name="zigzag_l32_s16384", cfg_id=2, L=32, H=8, Hkv=8, S=16384, w=128, recent=128,
        total_budget=32 * 1024, floor=128, scale_range=(0.5, 3.0),
        notes="ZigZag 32 layers x 8 KV heads, LMBA allocation, floor 128"),
    "keyformer_mha32_s8192": Workload(
        name="keyformer_mha32_s8192", cfg_id=3, L=1, H=32, Hkv=32, S=8192, w=512, recent=512,
        budget=4096, gumbel=True, taus=(1.0, 1.0e4),
        notes="Keyformer MHA 32, Gumbel noise, tau 1 and 1e4, 512 recent + 3584 top"),
    "keyformer_mha32_s8192_causal": Workload(
        name="keyformer_mha32_s8192_causal", cfg_id=3, L=1, H=32, Hkv=32, S=8192, w=8192, recent=512,
        budget=4096, gumbel=True, taus=(1.0,), causal=True,
        notes="Keyformer's full-attention reading of the prompt phase: all 8192 positions are queries, causal, "
              "Gumbel noise tau 1; 512 recent + 3584 top of the other 7680 (same keys as the MHA 32 case)"),
    "keyformer_mha32_s8192_decode": Workload(
        name="keyformer_mha32_s8192_decode", cfg_id=3, L=1, H=32, Hkv=32, S=8192, w=512, recent=512,
        budget=4096, gumbel=True, taus=(1.0,), decode_steps=64,
        notes="the Keyformer prompt phase above (same inputs, tau 1), then decode steps on the 4096-token cache: "
              "score accumulation and eviction of one token per step"),
    "think_s131072": Workload(
        name="think_s131072", cfg_id=4, L=1, H=8, Hkv=8, S=131072, w=64, recent=64,
        budget=int(0.2 * 131072), outliers=4, think_lambda=0.4, think_p=2,
        notes="long context, top 20% then ThinK l2 key-channel pruning lambda 0.4"),
    "think_s131072_query": Workload(
        name="think_s131072_query", cfg_id=4, L=1, H=8, Hkv=8, S=131072, w=64, recent=64,
        budget=int(0.2 * 131072), outliers=4, think_lambda=0.4, think_query=True,
        notes="the long-context case above (same inputs) with ThinK's query-driven channel score"),
}


def _rng(seed, cfg_id, tensor_id, layer):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg_id, tensor_id, layer])))


def f32_to_bf16_bits(x):
    """Round float32 values to bf16 (round to nearest, ties to even); raw uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def outlier_channels(wl):
    if wl.outliers <= 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(wl.seed, wl.cfg_id, OUTLIER_ID, 0).choice(wl.D, size=wl.outliers, replace=False))


def layer_scales(wl):
    """float32 logit scale per layer."""
    base = 1.0 / math.sqrt(wl.D)
    if not wl.scale_range:
        return np.full(wl.L, base, dtype=np.float32)
    lo, hi = wl.scale_range
    s = _rng(wl.seed, wl.cfg_id, SCALE_ID, 0).uniform(lo, hi, wl.L)
    return (s * base).astype(np.float32)


def _normal_bf16(wl, tensor_id, layer, shape, gain_channels=None):
    x = _rng(wl.seed, wl.cfg_id, tensor_id, layer).standard_normal(size=shape, dtype=np.float32)
    if gain_channels is not None and len(gain_channels):
        x[..., gain_channels] *= np.float32(wl.outlier_gain)
    return f32_to_bf16_bits(x)


def gen_q(wl, layer=0):
    return _normal_bf16(wl, Q_ID, layer, (wl.H, wl.w, wl.D))


def gen_k(wl, layer=0):
    return _normal_bf16(wl, K_ID, layer, (wl.Hkv, wl.S, wl.D), outlier_channels(wl))


def gen_v(wl, layer=0):
    return _normal_bf16(wl, V_ID, layer, (wl.Hkv, wl.S, wl.D))


def gen_decode(wl, step):
    """Raw bf16 bits of decode step `step` (the token at position S + step):
    q [H, D], k [Hkv, D], v [Hkv, D]."""
    return (_normal_bf16(wl, DEC_Q_ID, step, (wl.H, wl.D)), _normal_bf16(wl, DEC_K_ID, step, (wl.Hkv, wl.D)),
            _normal_bf16(wl, DEC_V_ID, step, (wl.Hkv, wl.D)))


def gen_layer(wl, layer=0):
    """Raw bf16 bits: q [H, w, D], k [Hkv, S, D], v [Hkv, S, D]."""
    return gen_q(wl, layer), gen_k(wl, layer), gen_v(wl, layer)


def scaled_down(wl, S, **kw):
    """Same structure at a smaller prompt length (for oracle-sized parity runs)."""
    return wl.with_(S=S, **kw)
