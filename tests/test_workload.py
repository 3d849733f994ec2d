"""The seeded synthetic input generator (CPU only)."""

import math

import numpy as np
import torch

from kv_cache_compression_bf16_amd import workload as wk


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 65504.0, 1e-30],
                                 dtype=np.float32)])
    ours = wk.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_generation_is_deterministic_and_shaped():
    w = wk.WORKLOADS["snapkv_mha8_s2048"]
    q1, k1, v1 = wk.gen_layer(w)
    q2, k2, v2 = wk.gen_layer(w)
    assert q1.shape == (8, 32, 128) and k1.shape == (8, 2048, 128) and v1.shape == k1.shape
    assert q1.dtype == np.uint16
    assert np.array_equal(q1, q2) and np.array_equal(k1, k2) and np.array_equal(v1, v2)
    assert not np.array_equal(k1, v1)


def test_outlier_channels_scaled_exactly():
    w = wk.WORKLOADS["gqa32x8_s32768"].with_(S=512)
    ch = wk.outlier_channels(w)
    assert len(set(ch.tolist())) == 4
    k = wk.bf16_bits_to_f32(wk.gen_k(w))
    plain = wk.bf16_bits_to_f32(wk.gen_k(w.with_(outliers=0)))
    mask = np.zeros(128, bool); mask[ch] = True
    assert np.array_equal(k[..., ~mask], plain[..., ~mask])
    assert np.array_equal(k[..., mask], plain[..., mask] * 8)


def test_layer_scales_range():
    w = wk.WORKLOADS["zigzag_l32_s16384"]
    s = wk.layer_scales(w) * math.sqrt(128)
    assert s.shape == (32,) and s.dtype == np.float32
    assert np.all((s >= 0.5 - 1e-6) & (s < 3.0 + 1e-6))
    assert s.std() > 0.3


def test_workload_shapes():
    w = wk.WORKLOADS["think_s131072"]
    assert w.budget == 26214 and w.n == 131008 and w.capacity == 131072
    z = wk.WORKLOADS["zigzag_l32_s16384"]
    assert z.capacity == 16384 and z.total_budget == 32768
