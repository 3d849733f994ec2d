"""kvc_score_noalloc (the scoring entry point whose workspace is the library's
static per-device scratch) against kvc_score on the same inputs: two calls in a
row, the second smaller, each bit-identical to kvc_score (same kernels, fixed
reduction order) and within the importance tolerance of the oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_bf16_amd import workload as wk

from _parity import check_importance, dev, to_dev

pytestmark = pytest.mark.gpu


def _draw(H, Hkv, w, S, seed):
    rng = np.random.default_rng(seed)
    q = wk.f32_to_bf16_bits(rng.standard_normal((H, w, 128), dtype=np.float32))
    k = wk.f32_to_bf16_bits(rng.standard_normal((Hkv, S, 128), dtype=np.float32))
    return q, k


def test_noalloc_matches_kvc_score_two_calls_second_smaller():
    from kv_cache_compression_bf16_amd import kvc

    alpha = float(np.float32(1 / math.sqrt(128)))
    for H, Hkv, w, S in [(32, 8, 128, 4096 + 77), (8, 4, 20, 1000)]:
        print(f"[no_alloc] H={H} Hkv={Hkv} w={w} S={S}", flush=True)
        qb, kb = _draw(H, Hkv, w, S, seed=H + S)
        q, k = to_dev(qb), to_dev(kb)
        ref_gpu = torch.full((Hkv, S - w), float("nan"), dtype=torch.float32, device=dev())
        out = torch.full((Hkv, S - w), float("nan"), dtype=torch.float32, device=dev())
        kvc.kvc_score(q, k, ref_gpu, w=w, S=S)
        kvc.kvc_score_noalloc(q, k, out, w=w, S=S)
        torch.cuda.synchronize()
        a, b = out.cpu().numpy(), ref_gpu.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "differs from kvc_score"
        ref = oracle.score.importance(oracle.score.bf16_bits_to_f64(qb), oracle.score.bf16_bits_to_f64(kb),
                                      S=S, w=w, scale=alpha)
        check_importance(a, ref, H // Hkv, f"noalloc H={H} S={S}")


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    from kv_cache_compression_bf16_amd import kvc

    # 32 layers of 8 heads x 512 rows over 16K keys: partials far beyond 16 MiB
    q = torch.empty((32, 32, 128, 128), dtype=torch.bfloat16, device=dev())
    k = torch.empty((32, 8, 16384, 128), dtype=torch.bfloat16, device=dev())
    a = kvc.score_args(q, k, w=128, S=16384)
    assert kvc.lib.kvc_score_workspace_size(a) > kvc.lib.kvc_score_noalloc_max_workspace()
    imp = torch.empty((32, 8, 16384 - 128), dtype=torch.float32, device=dev())
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_score_noalloc(q, k, imp, w=128, S=16384)
    assert e.value.status == kvc.KVC_E_WORKSPACE
