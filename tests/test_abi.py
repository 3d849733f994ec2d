"""The C ABI without a GPU: libkvc.so loads, exports every function that
include/kvc.h declares, and rejects invalid arguments on the host before
anything is enqueued (these calls never reach a kernel launch)."""

import ctypes
import json
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")

kvc = pytest.importorskip("kv_cache_compression_bf16_amd.kvc",
                          reason="libkvc.so not built (run __graft_entry__.build())")
lib = kvc.lib
E = kvc


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), f"{n} declared in kvc.h but not exported"


def test_status_strings_and_version():
    for s in range(6):
        assert lib.kvc_status_str(s).decode().startswith("KVC")
    assert lib.kvc_status_str(99).decode().startswith("KVC")
    assert lib.kvc_abi_version() == 1


def test_cache_bytes_against_page_figures():
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "page_figures.json")))
    a = gold["kv_cache_llama2_7b"]
    m = a["model"]
    b = kvc.kvc_cache_bytes(a["B"], a["S"], m["L"], m["N"], m["D"], m["elem_bytes"])
    assert round(b / 2 ** 30) == a["printed_GB"]
    c = gold["kv_cache_llama1_65b"]
    m = c["model"]
    assert abs(kvc.kvc_cache_bytes(c["B"], c["S"], m["L"], m["N"], m["D"], m["elem_bytes"]) / 1e9 - 335) < 1
    assert kvc.kvc_cache_bytes(-1, 1, 1, 1, 1, 2) == -1
    assert kvc.kvc_cache_bytes(2 ** 40, 2 ** 40, 1, 1, 1, 2) == -1


def test_think_channels():
    assert kvc.kvc_think_channels(128, 0.4) == 76
    assert kvc.kvc_think_channels(128, 0.5) == 64
    assert kvc.kvc_think_channels(128, 0.3) == 89
    assert kvc.kvc_think_channels(128, 1.0) == -1
    assert kvc.kvc_think_channels(128, -0.1) == -1
    assert kvc.kvc_think_channels(128, float("nan")) == -1


def _args(**over):
    a = kvc.ScoreArgs()
    a.L, a.H, a.Hkv, a.w, a.S, a.D = 1, 8, 8, 32, 2048, 128
    a.q_head_stride, a.q_layer_stride = 32 * 128, 8 * 32 * 128
    a.k_head_stride, a.k_layer_stride = 2048 * 128, 8 * 2048 * 128
    a.scale, a.layer_scales, a.gumbel, a.tau, a.seed = 1 / math.sqrt(128), None, 0, 1.0, 0
    for k, v in over.items():
        setattr(a, k, v)
    return a


FAKE = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced: validation fails first
FAKE2 = ctypes.c_void_p(1 << 21)


@pytest.mark.parametrize("over,status", [
    (dict(H=6), E.KVC_E_SHAPE),          # H % Hkv
    (dict(w=2048), E.KVC_E_SHAPE),       # w >= S
    (dict(w=0), E.KVC_E_ARG),
    (dict(D=64, q_head_stride=32 * 64, k_head_stride=2048 * 64), E.KVC_E_UNSUPPORTED),
    (dict(scale=0.0), E.KVC_E_ARG),
    (dict(scale=float("inf")), E.KVC_E_ARG),
    (dict(gumbel=1, tau=0.0), E.KVC_E_ARG),
    (dict(gumbel=1, tau=float("nan")), E.KVC_E_ARG),
    (dict(k_head_stride=100), E.KVC_E_SHAPE),
    (dict(q_head_stride=32 * 128 + 4), E.KVC_E_ARG),
    # 65535 layers of 65535 KV heads: more units of work than 32-bit counters hold
    (dict(L=65535, H=65535, Hkv=65535, q_layer_stride=65535 * 32 * 128, k_layer_stride=65535 * 2048 * 128),
     E.KVC_E_SHAPE),
])
def test_score_validation(over, status):
    a = _args(**over)
    st = lib.kvc_score(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == status


def test_score_workspace_checks():
    a = _args()
    need = lib.kvc_score_workspace_size(ctypes.byref(a))
    assert need > 0
    assert lib.kvc_score(ctypes.byref(a), FAKE, FAKE, FAKE, None, need, None) == E.KVC_E_WORKSPACE
    assert lib.kvc_score(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, need - 1, None) == E.KVC_E_WORKSPACE
    assert lib.kvc_score(ctypes.byref(a), None, FAKE, FAKE, FAKE, need, None) == E.KVC_E_ARG
    misaligned = ctypes.c_void_p((1 << 20) + 2)
    assert lib.kvc_score(ctypes.byref(a), misaligned, FAKE, FAKE, FAKE, need, None) == E.KVC_E_ARG
    assert lib.kvc_score(None, FAKE, FAKE, FAKE, FAKE, need, None) == E.KVC_E_ARG
    assert lib.kvc_score_workspace_size(ctypes.byref(_args(H=6))) == 0


@pytest.mark.parametrize("S,w,recent,budget,status", [
    (100, 10, 10, 9, E.KVC_E_ARG),        # budget < recent
    (100, 10, 10, 101, E.KVC_E_ARG),      # beyond capacity c + recent = 100
    (100, 10, 101, 101, E.KVC_E_ARG),     # recent > S
    (100, 100, 10, 20, E.KVC_E_ARG),      # w >= S
    (100, 10, -1, 20, E.KVC_E_ARG),
])
def test_select_validation(S, w, recent, budget, status):
    st = lib.kvc_select_topk(FAKE, S - w, 4, S, w, recent, budget, FAKE, None, 0, None)
    assert st == status


def test_select_workspace():
    # up to 32768 candidates per head: one workgroup per head, no workspace
    assert lib.kvc_select_topk_workspace_size(8, 32640) == 0
    need = lib.kvc_select_topk_workspace_size(8, 131008)
    assert need > 0 and lib.kvc_select_topk_workspace_size(0, 100) == 0
    # the size for n covers every smaller candidate count (the chunking is not monotone in c)
    for Hkv in (1, 3, 8, 32):
        big = lib.kvc_select_topk_workspace_size(Hkv, 140000)
        assert all(lib.kvc_select_topk_workspace_size(Hkv, n) <= big for n in range(1, 140000, 997))
    # too small or missing: rejected before anything is enqueued
    args = (FAKE, 131008, 8, 131072, 64, 64, 26214, FAKE)
    assert lib.kvc_select_topk(*args, None, need, None) == E.KVC_E_WORKSPACE
    assert lib.kvc_select_topk(*args, FAKE, 4, None) == E.KVC_E_WORKSPACE


@pytest.mark.parametrize("rows,n,kernel,mode,status", [
    (0, 10, 3, 0, E.KVC_E_ARG),
    (2, 0, 3, 0, E.KVC_E_ARG),
    (2, 10, 4, 0, E.KVC_E_ARG),        # even kernel
    (2, 10, 257, 0, E.KVC_E_ARG),      # beyond 255
    (2, 10, 3, 2, E.KVC_E_ARG),        # unknown mode
])
def test_pool_validation(rows, n, kernel, mode, status):
    assert lib.kvc_pool_importance(FAKE, n, FAKE2, n, rows, n, kernel, mode, None) == status


def test_pool_aliasing_and_strides():
    assert lib.kvc_pool_importance(FAKE, 10, FAKE, 10, 2, 10, 3, 0, None) == E.KVC_E_ARG     # in == out
    assert lib.kvc_pool_importance(FAKE, 9, FAKE2, 10, 2, 10, 3, 0, None) == E.KVC_E_SHAPE   # stride < n


def test_compact_validation():
    assert lib.kvc_compact(FAKE, FAKE, 4, 100, 12, 1200, 1200, FAKE, 10, FAKE, FAKE, None) == E.KVC_E_ARG
    assert lib.kvc_compact(FAKE, None, 4, 100, 128, 12800, 0, FAKE, 10, FAKE, FAKE, None) == E.KVC_E_ARG
    assert lib.kvc_compact(FAKE, FAKE, 4, 100, 128, 100, 12800, FAKE, 10, FAKE, FAKE, None) == E.KVC_E_SHAPE
    assert lib.kvc_compact(None, FAKE, 4, 100, 128, 12800, 12800, FAKE, 10, FAKE, FAKE, None) == E.KVC_E_ARG


def test_lmba_validation():
    f = lib.kvc_lmba_budget
    assert f(FAKE, 4, 8, 1000, 0.9, 3, 1, 100, FAKE, FAKE, None, 0, None) == E.KVC_E_ARG   # total < L*floor
    assert f(FAKE, 4, 8, 1000, 0.9, 500, 1, 100, FAKE, FAKE, None, 0, None) == E.KVC_E_ARG  # total > L*cap
    assert f(FAKE, 4, 8, 1000, 0.0, 100, 1, 100, FAKE, FAKE, None, 0, None) == E.KVC_E_ARG  # mass
    assert f(FAKE, 4, 8, 1000, 1.5, 100, 1, 100, FAKE, FAKE, None, 0, None) == E.KVC_E_ARG
    assert f(FAKE, 4, 8, 1000, 0.9, 100, 50, 40, FAKE, FAKE, None, 0, None) == E.KVC_E_ARG  # floor > cap
    assert f(FAKE, 4, 8, 1000, 0.9, 100, 1, 100, None, FAKE, None, 0, None) == E.KVC_E_WORKSPACE
    assert f(FAKE, 2000, 8, 1000, 0.9, 4000, 1, 100, FAKE, FAKE, None, 0, None) == E.KVC_E_ARG  # L limit


def test_channel_prune_validation():
    f = lib.kvc_channel_prune
    ws = lib.kvc_channel_prune_workspace_size(8, 100, 128)
    assert ws > 0
    assert f(FAKE, 8, 100, 128, 101, 0.4, 2, FAKE, None, FAKE, FAKE, ws, None) == E.KVC_E_ARG
    assert f(FAKE, 8, 100, 128, 10, 1.0, 2, FAKE, None, FAKE, FAKE, ws, None) == E.KVC_E_ARG
    assert f(FAKE, 8, 100, 128, 10, 0.4, 3, FAKE, None, FAKE, FAKE, ws, None) == E.KVC_E_ARG
    assert f(FAKE, 8, 100, 64, 10, 0.4, 2, FAKE, None, FAKE, FAKE, ws, None) == E.KVC_E_UNSUPPORTED
    assert f(FAKE, 8, 100, 128, 10, 0.4, 2, FAKE, None, FAKE, None, ws, None) == E.KVC_E_WORKSPACE
    assert f(FAKE, 8, 100, 128, 10, 0.999, 2, FAKE, None, FAKE, FAKE, ws, None) == E.KVC_E_ARG  # T = 0


def _named_call(f, names, ok):
    def call(**kw):
        a = dict(zip(names, ok))
        a.update(kw)
        return f(*[a[n] for n in names])
    return call


def test_select_threshold_validation():
    ws = lib.kvc_select_threshold_workspace_size(8, 1000, 32, 32)
    assert ws >= 8 * 4 and lib.kvc_select_threshold_workspace_size(8, 1000, 1000, 32) == 0
    names = ["s", "hs", "Hkv", "S", "w", "r", "th", "idx", "off", "ws", "nb", "st"]
    call = _named_call(lib.kvc_select_threshold, names,
                       (FAKE, 1000, 8, 1000, 32, 32, 0.5, FAKE, FAKE, FAKE, ws, None))
    assert call(w=0) == E.KVC_E_ARG
    assert call(w=1000) == E.KVC_E_ARG
    assert call(r=1001) == E.KVC_E_ARG
    assert call(th=float("nan")) == E.KVC_E_ARG
    assert call(hs=100) == E.KVC_E_SHAPE                                  # stride < S - w
    assert call(Hkv=70000) == E.KVC_E_SHAPE
    assert call(Hkv=65535, S=40000, hs=40000) == E.KVC_E_SHAPE             # Hkv * (c + r) >= 2^31
    assert call(idx=None) == E.KVC_E_ARG
    assert call(off=None) == E.KVC_E_ARG
    assert call(s=None) == E.KVC_E_ARG
    assert call(s=ctypes.c_void_p((1 << 20) + 2)) == E.KVC_E_ARG           # misaligned scores
    assert call(ws=None) == E.KVC_E_WORKSPACE
    assert call(nb=8 * 4 - 4) == E.KVC_E_WORKSPACE


def test_compact_ragged_validation():
    names = ["k", "v", "Hkv", "S", "D", "khs", "vhs", "idx", "off", "rows", "ko", "vo", "st"]
    call = _named_call(lib.kvc_compact_ragged, names,
                       (FAKE, FAKE, 8, 1000, 128, 1000 * 128, 1000 * 128, FAKE, FAKE, 4000, FAKE, FAKE, None))
    assert call(D=100) == E.KVC_E_ARG
    assert call(D=48, khs=1000 * 48, vhs=1000 * 48) == E.KVC_E_UNSUPPORTED    # 256 % (48 / 8) != 0
    assert call(rows=-1) == E.KVC_E_ARG
    assert call(off=None) == E.KVC_E_ARG
    assert call(idx=None) == E.KVC_E_ARG
    assert call(vo=None) == E.KVC_E_ARG                                    # v without v_out
    assert call(khs=999 * 128) == E.KVC_E_SHAPE
    assert call(k=ctypes.c_void_p((1 << 20) + 8)) == E.KVC_E_ARG
    assert call(off=ctypes.c_void_p((1 << 20) + 2)) == E.KVC_E_ARG
    assert call(rows=1 << 30) == E.KVC_E_SHAPE                             # max_rows * D / 8 >= 2^31
    assert call(rows=0) == E.KVC_OK                                        # nothing to gather: no launch


def test_channel_prune_value_validation():
    ws = lib.kvc_channel_prune_value_workspace_size(8, 4, 16, 100, 10, 128)
    assert ws > 0
    assert lib.kvc_channel_prune_value_workspace_size(8, 4, 16, 100, 101, 128) == 0
    assert lib.kvc_channel_prune_value_workspace_size(8, 4, 16, 100, 10, 64) == 0
    names = ["k", "v", "q", "Hkv", "G", "w", "qs", "budget", "D", "recent", "lam", "scale", "ch", "mask", "vp",
             "ws", "nb", "st"]
    call = _named_call(lib.kvc_channel_prune_value, names,
                       (FAKE, FAKE, FAKE, 8, 4, 16, 16 * 128, 100, 128, 10, 0.4, 0.088, FAKE, None, FAKE, FAKE, ws,
                        None))
    assert call(v=None) == E.KVC_E_ARG
    assert call(q=None) == E.KVC_E_ARG
    assert call(v=ctypes.c_void_p((1 << 20) + 8)) == E.KVC_E_ARG           # v not 16-byte aligned
    assert call(scale=0.0) == E.KVC_E_ARG
    assert call(scale=float("inf")) == E.KVC_E_ARG
    assert call(scale=float("nan")) == E.KVC_E_ARG
    assert call(lam=1.0) == E.KVC_E_ARG
    assert call(recent=101) == E.KVC_E_ARG
    assert call(D=64) == E.KVC_E_UNSUPPORTED
    assert call(G=4, w=20000, qs=20000 * 128) == E.KVC_E_SHAPE             # G * w > 65536
    assert call(qs=16 * 128 - 8) == E.KVC_E_SHAPE
    assert call(ws=None) == E.KVC_E_WORKSPACE
    assert call(nb=ws - 256) == E.KVC_E_WORKSPACE


def test_decode_validation():
    names = ["q", "qs", "kn", "vn", "kc", "vc", "pos", "acc", "Hkv", "G", "B", "D", "t", "recent", "scale", "tau",
             "seed", "ev", "ws", "nb", "st"]
    ws = lib.kvc_keyformer_decode_step_workspace_size(32, 1, 4096)
    assert ws >= 32 * 4097 * 4 and lib.kvc_keyformer_decode_step_workspace_size(32, 9, 4096) == 0
    call = _named_call(lib.kvc_keyformer_decode_step, names,
                       (FAKE, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 32, 1, 4096, 128, 9000, 512, 0.088, 1.0, 0,
                        None, FAKE, ws, None))
    assert call(recent=4096) == E.KVC_E_ARG                   # the window must be shorter than the cache
    assert call(recent=0) == E.KVC_E_ARG
    assert call(t=-1) == E.KVC_E_ARG
    assert call(scale=0.0) == E.KVC_E_ARG
    assert call(tau=0.0) == E.KVC_E_ARG
    assert call(tau=float("nan")) == E.KVC_E_ARG
    assert call(D=64) == E.KVC_E_UNSUPPORTED
    assert call(G=9, Hkv=4) == E.KVC_E_UNSUPPORTED
    assert call(B=(1 << 28) + 1) == E.KVC_E_SHAPE
    assert call(ws=None) == E.KVC_E_WORKSPACE
    assert call(nb=ws - 256) == E.KVC_E_WORKSPACE
    assert call(qs=100) == E.KVC_E_SHAPE
    assert call(acc=None) == E.KVC_E_ARG
    assert call(kc=ctypes.c_void_p((1 << 20) + 8)) == E.KVC_E_ARG
    assert call(ev=ctypes.c_void_p((1 << 20) + 2)) == E.KVC_E_ARG
    f = lib.kvc_decode_init_scores
    assert f(FAKE, 100, FAKE, 4, 10, -1, FAKE, None) == E.KVC_E_ARG
    assert f(FAKE, 50, FAKE, 4, 10, 100, FAKE, None) == E.KVC_E_SHAPE
    assert f(None, 100, FAKE, 4, 10, 100, FAKE, None) == E.KVC_E_ARG
    assert f(FAKE, 100, FAKE, 4, 0, 100, FAKE, None) == E.KVC_OK   # nothing to do: no launch


def test_score_causal_validation():
    a = kvc.ScoreArgs()
    a.L, a.H, a.Hkv, a.w, a.S, a.D = 1, 32, 32, 8192, 8192, 128
    a.q_head_stride, a.q_layer_stride = 8192 * 128, 32 * 8192 * 128
    a.k_head_stride, a.k_layer_stride = 8192 * 128, 32 * 8192 * 128
    a.scale, a.gumbel, a.tau = 0.088, 1, 1.0
    ws = lib.kvc_score_causal_workspace_size(ctypes.byref(a))
    assert ws > 0                                                # w == S is allowed here
    assert lib.kvc_score_workspace_size(ctypes.byref(a)) == 0    # but not for the window scoring
    f = lib.kvc_score_causal
    assert f(ctypes.byref(a), FAKE, FAKE, FAKE, None, ws, None) == E.KVC_E_WORKSPACE
    a.w = 8191
    assert f(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, ws, None) == E.KVC_E_SHAPE   # w % 32 != 0
    a.w = 8224
    assert f(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, ws, None) == E.KVC_E_SHAPE   # w > S
    a.w, a.tau = 8192, 0.0
    assert f(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, ws, None) == E.KVC_E_ARG


def test_layers_batched_validation():
    f = lib.kvc_select_topk_layers
    #         imp   hs     ls          L   Hkv  S      w    r    budgets tot   idx   stream
    ok = [FAKE, 16256, 8 * 16256, 32, 8, 16384, 128, 128, FAKE, 32768, FAKE, None]
    call = _named_call(f, list("abcdefghijkl"), ok)
    assert call(f=70000, g=128) == E.KVC_E_UNSUPPORTED        # c > 32768: not the one-workgroup path
    assert call(g=16384) == E.KVC_E_ARG                        # w >= S
    assert call(c=16256 * 7) == E.KVC_E_SHAPE                  # layer stride < Hkv * head stride
    assert call(i=None) == E.KVC_E_ARG
    assert call(k=None) == E.KVC_E_ARG
    assert call(j=-1) == E.KVC_E_ARG
    assert call(j=0) == E.KVC_OK                               # nothing to select: no launch
    g = lib.kvc_compact_layers
    okc = [FAKE, FAKE, 32, 8, 16384, 128, 16384 * 128, 8 * 16384 * 128, 16384 * 128, 8 * 16384 * 128, FAKE, 32768,
           FAKE, FAKE, FAKE, None]
    callc = _named_call(g, list("abcdefghijklmnop"), okc)
    assert callc(f=48, g=16384 * 48, h=8 * 16384 * 48, i=16384 * 48, j=8 * 16384 * 48) == E.KVC_E_UNSUPPORTED
    assert callc(h=16384 * 128) == E.KVC_E_SHAPE               # k layer stride too small
    assert callc(c=10000) == E.KVC_E_SHAPE                     # Hkv * L > 65535
    assert callc(k=None) == E.KVC_E_ARG
    assert callc(o=None) == E.KVC_E_ARG                        # v without v_out
    assert callc(l=0) == E.KVC_OK                              # nothing to gather: no launch


def test_channel_prune_query_validation():
    f = lib.kvc_channel_prune_query
    ws = lib.kvc_channel_prune_query_workspace_size(8, 4, 100, 128)
    assert ws >= lib.kvc_channel_prune_workspace_size(8, 100, 128) + 8 * 4 * 128 * 4
    assert lib.kvc_channel_prune_query_workspace_size(8, 0, 100, 128) == 0
    assert lib.kvc_channel_prune_query_workspace_size(8, 4, 100, 64) == 0
    qs = 16 * 128
    ok = (FAKE, FAKE, 8, 4, 16, qs, 100, 128, 10, 0.4, FAKE, None, FAKE, FAKE, ws, None)

    def call(**kw):
        names = ["k", "q", "Hkv", "G", "w", "qs", "budget", "D", "recent", "lam", "ch", "mask", "kp", "ws",
                 "nbytes", "stream"]
        a = dict(zip(names, ok))
        a.update(kw)
        return f(*[a[n] for n in names])

    assert call(q=None) == E.KVC_E_ARG
    assert call(q=ctypes.c_void_p((1 << 21) + 8)) == E.KVC_E_ARG   # q not 16-byte aligned
    assert call(G=0) == E.KVC_E_ARG
    assert call(w=0) == E.KVC_E_ARG
    assert call(qs=16 * 128 - 8) == E.KVC_E_SHAPE              # window rows overlap the next head
    assert call(qs=16 * 128 + 4) == E.KVC_E_SHAPE              # head stride not a multiple of 8
    assert call(Hkv=8192, G=16) == E.KVC_E_SHAPE               # Hkv * G > 65535
    assert call(recent=101) == E.KVC_E_ARG
    assert call(lam=1.0) == E.KVC_E_ARG
    assert call(D=64) == E.KVC_E_UNSUPPORTED
    assert call(ws=None) == E.KVC_E_WORKSPACE
    assert call(nbytes=ws - 256) == E.KVC_E_WORKSPACE          # the magnitude path's size is not enough


def test_timing_api_without_launches():
    assert lib.kvc_timing_enable(1) == E.KVC_OK
    assert lib.kvc_timing_count() == 0
    assert lib.kvc_timing_enable(0) == E.KVC_OK


def test_peak_probe_library_exports_its_header():
    # the benchmark's probe library (libkvc_peak.so, include/kvc_peak.h) loads and
    # exports every function its header declares; bad arguments are rejected on
    # the host (return 1) before any launch
    from kv_cache_compression_bf16_amd import build_lib
    if not os.path.exists(build_lib.PEAK_LIB):
        pytest.skip("libkvc_peak.so not built")
    peak = ctypes.CDLL(build_lib.PEAK_LIB)
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "kvc_peak.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(kvc_peak_[a-z0-9_]+)\s*\(", src)))
    assert len(names) >= 9
    for n in names:
        assert hasattr(peak, n), f"{n} declared in kvc_peak.h but not exported"
    peak.kvc_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    peak.kvc_peak_valu.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    assert peak.kvc_peak_read(None, 16, None, None) == 1
    assert peak.kvc_peak_valu(0, None, 1, None) == 1
