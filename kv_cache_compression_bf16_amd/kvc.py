"""Thin Python binding of libkvc.so (C ABI declared in include/kvc.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libkvc.so.  Tensors are torch tensors on the GPU (torch provides device memory
and the stream); each function takes the same name as the C entry point it
calls.  Importing this module fails loudly if the library is missing; there is
no CPU fallback.
"""

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# KVC_LIBRARY may name an alternative build of the same library (A/B timing).
LIB_PATH = os.environ.get("KVC_LIBRARY") or os.path.join(_PKG, "libkvc.so")

KVC_OK, KVC_E_ARG, KVC_E_SHAPE, KVC_E_WORKSPACE, KVC_E_DEVICE, KVC_E_UNSUPPORTED = range(6)


class KvcError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {_lib.kvc_status_str(status).decode()}")


class ScoreArgs(ctypes.Structure):
    _fields_ = [
        ("L", ctypes.c_int32), ("H", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("w", ctypes.c_int32), ("S", ctypes.c_int32), ("D", ctypes.c_int32),
        ("q_head_stride", ctypes.c_int64), ("q_layer_stride", ctypes.c_int64),
        ("k_head_stride", ctypes.c_int64), ("k_layer_stride", ctypes.c_int64),
        ("scale", ctypes.c_float), ("layer_scales", ctypes.c_void_p),
        ("gumbel", ctypes.c_int32), ("tau", ctypes.c_float), ("seed", ctypes.c_uint64),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m kv_cache_compression_bf16_amd.build_lib` "
                          "(or __graft_entry__.build()) first -- there is no CPU fallback")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_double
    sig = {
        "kvc_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "kvc_abi_version": (ctypes.c_int, []),
        "kvc_cache_bytes": (I64, [I64, I64, I64, I64, I64, I64]),
        "kvc_think_channels": (ctypes.c_int, [ctypes.c_int, F64]),
        "kvc_score_workspace_size": (SZ, [ctypes.POINTER(ScoreArgs)]),
        "kvc_score": (ctypes.c_int, [ctypes.POINTER(ScoreArgs), P, P, P, P, SZ, P]),
        "kvc_score_noalloc_max_workspace": (SZ, []),
        "kvc_score_noalloc": (ctypes.c_int, [ctypes.POINTER(ScoreArgs), P, P, P, P]),
        "kvc_score_causal_workspace_size": (SZ, [ctypes.POINTER(ScoreArgs)]),
        "kvc_score_causal": (ctypes.c_int, [ctypes.POINTER(ScoreArgs), P, P, P, P, SZ, P]),
        "kvc_lmba_budget_workspace_size": (SZ, [I32, I32, I32]),
        "kvc_lmba_budget": (ctypes.c_int, [P, I32, I32, I32, F64, I64, I32, I32, P, P, P, SZ, P]),
        "kvc_pool_importance": (ctypes.c_int, [P, I64, P, I64, I32, I32, I32, I32, P]),
        "kvc_select_topk_workspace_size": (SZ, [I32, I32]),
        "kvc_select_topk": (ctypes.c_int, [P, I64, I32, I32, I32, I32, I32, P, P, SZ, P]),
        "kvc_compact": (ctypes.c_int, [P, P, I32, I32, I32, I64, I64, P, I32, P, P, P]),
        "kvc_select_topk_layers": (ctypes.c_int, [P, I64, I64, I32, I32, I32, I32, I32, P, I32, P, P]),
        "kvc_compact_layers": (ctypes.c_int, [P, P, I32, I32, I32, I32, I64, I64, I64, I64, P, I32, P, P, P, P]),
        "kvc_select_threshold_workspace_size": (SZ, [I32, I32, I32, I32]),
        "kvc_select_threshold": (ctypes.c_int, [P, I64, I32, I32, I32, I32, ctypes.c_float, P, P, P, SZ, P]),
        "kvc_compact_ragged": (ctypes.c_int, [P, P, I32, I32, I32, I64, I64, P, P, I32, P, P, P]),
        "kvc_channel_prune_workspace_size": (SZ, [I32, I32, I32]),
        "kvc_channel_prune": (ctypes.c_int, [P, I32, I32, I32, I32, F64, I32, P, P, P, P, SZ, P]),
        "kvc_channel_prune_query_workspace_size": (SZ, [I32, I32, I32, I32]),
        "kvc_channel_prune_value_workspace_size": (SZ, [I32, I32, I32, I32, I32, I32]),
        "kvc_channel_prune_value": (ctypes.c_int, [P, P, P, I32, I32, I32, I64, I32, I32, I32, F64, ctypes.c_float,
                                                   P, P, P, P, SZ, P]),
        "kvc_channel_prune_query": (ctypes.c_int, [P, P, I32, I32, I32, I64, I32, I32, I32, F64, P, P, P, P, SZ,
                                                   P]),
        "kvc_decode_init_scores": (ctypes.c_int, [P, I64, P, I32, I32, I32, P, P]),
        "kvc_keyformer_decode_step_workspace_size": (SZ, [I32, I32, I32]),
        "kvc_keyformer_decode_step": (ctypes.c_int, [P, I64, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32,
                                                     ctypes.c_float, ctypes.c_float, ctypes.c_uint64, P, P, SZ,
                                                     P]),
        "kvc_timing_enable": (ctypes.c_int, [I32]),
        "kvc_timing_count": (I32, []),
        "kvc_timing_read": (ctypes.c_int, [I32, ctypes.c_char_p, I32, ctypes.POINTER(I32),
                                           ctypes.POINTER(F64)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
lib = _lib


def _check(status, where):
    if status != KVC_OK:
        raise KvcError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _workspace(nbytes, device, ws, stream):
    if nbytes == 0:
        return ws, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        if stream is not None:
            # allocated on the current stream, used on `stream`: without this the
            # allocator could hand the block to a later call while the kernels
            # queued on `stream` still use it
            ws.record_stream(stream)
    return ws, ws.numel() * ws.element_size()


def _bf16(t, name):
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold raw bf16 (torch.bfloat16 / int16), got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")


# ---------------------------------------------------------------- helpers
def kvc_abi_version():
    return _lib.kvc_abi_version()


def kvc_cache_bytes(B, S, L, N, D, elem_bytes):
    return _lib.kvc_cache_bytes(B, S, L, N, D, elem_bytes)


def kvc_think_channels(D, lam):
    return _lib.kvc_think_channels(D, lam)


# ---------------------------------------------------------------- kvc_score
def score_args(q_obs, k, *, w, S, scale=None, layer_scales=None, gumbel=False, tau=1.0, seed=0):
    """ScoreArgs from tensors shaped q_obs [L?, H, w, D], k [L?, Hkv, S_alloc, D]."""
    q4 = q_obs if q_obs.dim() == 4 else q_obs.unsqueeze(0)
    k4 = k if k.dim() == 4 else k.unsqueeze(0)
    L, H, wq, D = q4.shape
    Lk, Hkv, Sk, Dk = k4.shape
    if Lk != L or Dk != D or wq != w or Sk < S:
        raise ValueError(f"shape mismatch: q_obs {tuple(q_obs.shape)}, k {tuple(k.shape)}, w={w}, S={S}")
    if q4.stride(3) != 1 or q4.stride(2) != D or k4.stride(3) != 1 or k4.stride(2) != D:
        raise ValueError("rows of q_obs and k must be contiguous with stride D")
    a = ScoreArgs()
    a.L, a.H, a.Hkv, a.w, a.S, a.D = L, H, Hkv, w, S, D
    a.q_head_stride, a.q_layer_stride = q4.stride(1), q4.stride(0)
    a.k_head_stride, a.k_layer_stride = k4.stride(1), k4.stride(0)
    a.scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    a.layer_scales = None if layer_scales is None else layer_scales.data_ptr()
    a.gumbel = 1 if gumbel else 0
    a.tau = float(tau)
    a.seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return a


def kvc_score_workspace_size(args):
    return _lib.kvc_score_workspace_size(ctypes.byref(args))


def kvc_score(q_obs, k, importance, *, w, S, scale=None, layer_scales=None, gumbel=False, tau=1.0, seed=0,
              workspace=None, stream=None):
    """Observation-window importance into ``importance`` (fp32 [L?, Hkv, S-w])."""
    _bf16(q_obs, "q_obs")
    _bf16(k, "k")
    if layer_scales is not None and (layer_scales.dtype != torch.float32 or not layer_scales.is_cuda):
        raise TypeError("layer_scales must be a float32 GPU tensor")
    a = score_args(q_obs, k, w=w, S=S, scale=scale, layer_scales=layer_scales, gumbel=gumbel, tau=tau,
                   seed=seed)
    if importance.dtype != torch.float32 or not importance.is_contiguous() \
            or importance.numel() != a.L * a.Hkv * (S - w):
        raise ValueError("importance must be contiguous float32 with L*Hkv*(S-w) elements")
    ws, nbytes = _workspace(_lib.kvc_score_workspace_size(ctypes.byref(a)), k.device, workspace, stream)
    _check(_lib.kvc_score(ctypes.byref(a), _ptr(q_obs), _ptr(k), _ptr(importance), _ptr(ws), nbytes,
                          _stream(stream, k.device)), "kvc_score")
    return importance


def kvc_score_noalloc(q_obs, k, importance, *, w, S, scale=None, layer_scales=None, gumbel=False, tau=1.0,
                      seed=0, stream=None):
    """kvc_score with the library's per-device static scratch as its workspace (no
    device allocation by the library or here); calls that overlap on one device race."""
    _bf16(q_obs, "q_obs")
    _bf16(k, "k")
    if layer_scales is not None and (layer_scales.dtype != torch.float32 or not layer_scales.is_cuda):
        raise TypeError("layer_scales must be a float32 GPU tensor")
    a = score_args(q_obs, k, w=w, S=S, scale=scale, layer_scales=layer_scales, gumbel=gumbel, tau=tau,
                   seed=seed)
    if importance.dtype != torch.float32 or not importance.is_contiguous() \
            or importance.numel() != a.L * a.Hkv * (S - w):
        raise ValueError("importance must be contiguous float32 with L*Hkv*(S-w) elements")
    _check(_lib.kvc_score_noalloc(ctypes.byref(a), _ptr(q_obs), _ptr(k), _ptr(importance),
                                  _stream(stream, k.device)), "kvc_score_noalloc")
    return importance


def kvc_score_causal(q_obs, k, importance, *, w, S, scale=None, layer_scales=None, gumbel=False, tau=1.0, seed=0,
                     workspace=None, stream=None):
    """Causal importance into ``importance`` (fp32 [L?, Hkv, S]): window row i sits at
    position S - w + i and sees the keys at positions <= its own (w <= S, w % 32 == 0)."""
    _bf16(q_obs, "q_obs")
    _bf16(k, "k")
    if layer_scales is not None and (layer_scales.dtype != torch.float32 or not layer_scales.is_cuda):
        raise TypeError("layer_scales must be a float32 GPU tensor")
    a = score_args(q_obs, k, w=w, S=S, scale=scale, layer_scales=layer_scales, gumbel=gumbel, tau=tau,
                   seed=seed)
    if importance.dtype != torch.float32 or not importance.is_contiguous() \
            or importance.numel() != a.L * a.Hkv * S:
        raise ValueError("importance must be contiguous float32 with L*Hkv*S elements")
    ws, nbytes = _workspace(_lib.kvc_score_causal_workspace_size(ctypes.byref(a)), k.device, workspace, stream)
    _check(_lib.kvc_score_causal(ctypes.byref(a), _ptr(q_obs), _ptr(k), _ptr(importance), _ptr(ws), nbytes,
                                 _stream(stream, k.device)), "kvc_score_causal")
    return importance


# ---------------------------------------------------------------- kvc_lmba_budget
def kvc_lmba_budget(importance, budgets, *, total_budget, floor_per_layer, capacity, mass=0.9, mba=None,
                    workspace=None, stream=None):
    """ZigZag budgets (int32 [L]) and optionally MBA (int32 [L, Hkv]) from importance [L, Hkv, n]."""
    L, Hkv, n = importance.shape
    if not importance.is_contiguous() or importance.dtype != torch.float32:
        raise ValueError("importance must be contiguous float32 [L, Hkv, n]")
    ws, nbytes = (workspace, 0)
    if mba is None:
        ws, nbytes = _workspace(_lib.kvc_lmba_budget_workspace_size(L, Hkv, n), importance.device, workspace, stream)
    _check(_lib.kvc_lmba_budget(_ptr(importance), L, Hkv, n, float(mass), int(total_budget),
                                int(floor_per_layer), int(capacity), _ptr(mba), _ptr(budgets), _ptr(ws),
                                nbytes, _stream(stream, importance.device)), "kvc_lmba_budget")
    return budgets


# ---------------------------------------------------------------- kvc_pool_importance
POOL_AVG, POOL_MAX = 0, 1


def kvc_pool_importance(importance, pooled, *, kernel, mode=POOL_AVG, stream=None):
    """SnapKV 1D pooling along the keys of every row of importance [..., n] into pooled (same shape)."""
    if importance.dtype != torch.float32 or pooled.dtype != torch.float32:
        raise ValueError("importance and pooled must be float32")
    if importance.shape != pooled.shape or importance.stride(-1) != 1 or pooled.stride(-1) != 1:
        raise ValueError("importance and pooled must have the same shape and unit-stride rows")
    n = importance.shape[-1]
    src = importance.reshape(-1, n)
    dst = pooled.view(-1, n)
    _check(_lib.kvc_pool_importance(_ptr(src), src.stride(0), _ptr(dst), dst.stride(0), src.shape[0], n,
                                    int(kernel), int(mode), _stream(stream, importance.device)),
           "kvc_pool_importance")
    return pooled


# ---------------------------------------------------------------- kvc_select_topk
def kvc_select_topk(importance, indices, *, S, w, recent, budget, workspace=None, stream=None):
    """Per-head kept positions (int32 [Hkv, budget], ascending) from importance [Hkv, n]."""
    Hkv = importance.shape[0]
    if importance.dtype != torch.float32 or importance.stride(-1) != 1:
        raise ValueError("importance rows must be float32 with unit stride")
    if indices.dtype != torch.int32 or not indices.is_contiguous() or indices.numel() != Hkv * budget:
        raise ValueError("indices must be contiguous int32 [Hkv, budget]")
    ws, nbytes = _workspace(_lib.kvc_select_topk_workspace_size(Hkv, S - w), importance.device, workspace, stream)
    _check(_lib.kvc_select_topk(_ptr(importance), importance.stride(0), Hkv, S, w, recent, budget,
                                _ptr(indices), _ptr(ws), nbytes, _stream(stream, importance.device)),
           "kvc_select_topk")
    return indices


SELECT_ONE_WORKGROUP_MAX = 32768   # candidates per row up to which kvc_select_topk_layers applies


def kvc_select_topk_layers(importance, budgets, indices, *, S, w, recent, total_budget, stream=None):
    """All layers at once: importance [L, Hkv, n] fp32, budgets int32 [L] (device),
    indices int32 with Hkv * total_budget entries (layer blocks packed in order)."""
    if importance.dtype != torch.float32 or importance.dim() != 3 or importance.stride(2) != 1:
        raise ValueError("importance must be float32 [L, Hkv, n] with unit stride along n")
    if budgets.dtype != torch.int32 or indices.dtype != torch.int32 or not indices.is_contiguous():
        raise TypeError("budgets and indices must be int32 (indices contiguous)")
    L, Hkv, _ = importance.shape
    if budgets.numel() != L or indices.numel() < Hkv * total_budget:
        raise ValueError("budgets needs L entries and indices Hkv * total_budget")
    _check(_lib.kvc_select_topk_layers(_ptr(importance), importance.stride(1), importance.stride(0), L, Hkv, S, w,
                                       recent, _ptr(budgets), int(total_budget), _ptr(indices),
                                       _stream(stream, importance.device)), "kvc_select_topk_layers")
    return indices


# ---------------------------------------------------------------- kvc_compact
def kvc_compact(k, v, indices, k_out, v_out, *, S, stream=None):
    """k_out[g, t] = k[g, indices[g, t]] (and v likewise); k, v [Hkv, S_alloc, D]."""
    _bf16(k, "k")
    Hkv, _, D = k.shape
    budget = indices.shape[1]
    if k.stride(2) != 1 or k.stride(1) != D or not k_out.is_contiguous():
        raise ValueError("k rows must be contiguous; k_out contiguous")
    if v is not None and (v.stride(2) != 1 or v.stride(1) != D or not v_out.is_contiguous()):
        raise ValueError("v rows must be contiguous; v_out contiguous")
    _check(_lib.kvc_compact(_ptr(k), _ptr(v), Hkv, S, D, k.stride(0), 0 if v is None else v.stride(0),
                            _ptr(indices), budget, _ptr(k_out), _ptr(v_out), _stream(stream, k.device)),
           "kvc_compact")
    return k_out, v_out


def kvc_compact_layers(k, v, budgets, indices, k_out, v_out, *, S, total_budget, stream=None):
    """All layers at once: k, v [L, Hkv, S_alloc, D]; outputs [Hkv * total_budget, D] rows, layer blocks packed."""
    _bf16(k, "k")
    L, Hkv, _, D = k.shape
    if k.stride(2) != D or k.stride(3) != 1 or not k_out.is_contiguous() or k_out.shape[-1] != D:
        raise ValueError("k rows must be contiguous with stride D and k_out contiguous [rows, D]")
    if k_out.numel() < Hkv * total_budget * D or indices.numel() < Hkv * total_budget or budgets.numel() != L:
        raise ValueError("outputs and indices need Hkv * total_budget rows and budgets L entries")
    if v is not None:
        _bf16(v, "v")
        if v.shape != k.shape or v.stride(2) != D or v_out.shape != k_out.shape or not v_out.is_contiguous():
            raise ValueError("v / v_out must match k / k_out")
    _check(_lib.kvc_compact_layers(_ptr(k), _ptr(v), L, Hkv, S, D, k.stride(1), k.stride(0),
                                   0 if v is None else v.stride(1), 0 if v is None else v.stride(0),
                                   _ptr(budgets), int(total_budget), _ptr(indices), _ptr(k_out), _ptr(v_out),
                                   _stream(stream, k.device)), "kvc_compact_layers")
    return k_out, v_out


# ---------------------------------------------------------------- kvc_select_threshold
def kvc_select_threshold(scores, indices, offsets, *, S, w, recent, threshold, workspace=None, stream=None):
    """Keep candidates with score >= threshold plus the recent window; packed heads.
    scores [Hkv, >= S - w] fp32; indices int32 with Hkv * (c + recent) entries; offsets int32 [Hkv + 1]."""
    if scores.dtype != torch.float32 or indices.dtype != torch.int32 or offsets.dtype != torch.int32:
        raise TypeError("scores must be float32, indices and offsets int32")
    if scores.dim() != 2 or scores.stride(1) != 1:
        raise ValueError("scores must be [Hkv, n] with unit stride along n")
    Hkv = scores.shape[0]
    c = min(S - w, S - recent)
    if offsets.numel() != Hkv + 1 or indices.numel() < Hkv * (c + recent):
        raise ValueError(f"offsets needs {Hkv + 1} entries and indices {Hkv * (c + recent)}")
    ws, nbytes = _workspace(_lib.kvc_select_threshold_workspace_size(Hkv, S, w, recent), scores.device,
                            workspace, stream)
    _check(_lib.kvc_select_threshold(_ptr(scores), scores.stride(0), Hkv, S, w, recent, float(threshold),
                                     _ptr(indices), _ptr(offsets), _ptr(ws), nbytes,
                                     _stream(stream, scores.device)), "kvc_select_threshold")
    return indices, offsets


def kvc_compact_ragged(k, v, indices, offsets, k_out, v_out, *, S, stream=None):
    """Gather packed heads: k [Hkv, S_alloc, D] -> k_out [max_rows, D] (v likewise, or None)."""
    _bf16(k, "k")
    Hkv, _, D = k.shape
    max_rows = k_out.shape[0]
    if k.stride(1) != D or k.stride(2) != 1 or not k_out.is_contiguous() or k_out.shape[-1] != D:
        raise ValueError("k rows must be contiguous with stride D and k_out [max_rows, D] contiguous")
    if indices.numel() < max_rows or offsets.numel() != Hkv + 1:
        raise ValueError("indices needs max_rows entries and offsets Hkv + 1")
    if v is not None:
        _bf16(v, "v")
        if v.shape != k.shape or v.stride(1) != D or v_out.shape != k_out.shape or not v_out.is_contiguous():
            raise ValueError("v / v_out must match k / k_out")
    _check(_lib.kvc_compact_ragged(_ptr(k), _ptr(v), Hkv, S, D, k.stride(0), 0 if v is None else v.stride(0),
                                   _ptr(indices), _ptr(offsets), max_rows, _ptr(k_out), _ptr(v_out),
                                   _stream(stream, k.device)), "kvc_compact_ragged")
    return k_out, v_out


# ---------------------------------------------------------------- kvc_channel_prune
def kvc_channel_prune(k_c, channels, k_pruned, *, recent, lam, p=2, mask=None, workspace=None, stream=None):
    """ThinK pruning of the compacted keys k_c [Hkv, budget, D]."""
    _bf16(k_c, "k_c")
    Hkv, budget, D = k_c.shape
    if not k_c.is_contiguous():
        raise ValueError("k_c must be contiguous")
    ws, nbytes = _workspace(_lib.kvc_channel_prune_workspace_size(Hkv, budget, D), k_c.device, workspace, stream)
    _check(_lib.kvc_channel_prune(_ptr(k_c), Hkv, budget, D, recent, float(lam), int(p), _ptr(channels),
                                  _ptr(mask), _ptr(k_pruned), _ptr(ws), nbytes, _stream(stream, k_c.device)),
           "kvc_channel_prune")
    return channels, k_pruned


def kvc_channel_prune_query(k_c, q_obs, channels, k_pruned, *, recent, lam, mask=None, workspace=None,
                            stream=None):
    """Query-driven ThinK pruning of k_c [Hkv, budget, D] by the window queries q_obs [H, w, D]."""
    _bf16(k_c, "k_c")
    _bf16(q_obs, "q_obs")
    Hkv, budget, D = k_c.shape
    H, w, Dq = q_obs.shape
    if not k_c.is_contiguous():
        raise ValueError("k_c must be contiguous")
    if Dq != D or H % Hkv or q_obs.stride(1) != D or q_obs.stride(2) != 1:
        raise ValueError(f"shape mismatch: q_obs {tuple(q_obs.shape)}, k_c {tuple(k_c.shape)}")
    G = H // Hkv
    ws, nbytes = _workspace(_lib.kvc_channel_prune_query_workspace_size(Hkv, G, budget, D), k_c.device,
                            workspace, stream)
    _check(_lib.kvc_channel_prune_query(_ptr(k_c), _ptr(q_obs), Hkv, G, w, q_obs.stride(0), budget, D, recent,
                                        float(lam), _ptr(channels), _ptr(mask), _ptr(k_pruned), _ptr(ws), nbytes,
                                        _stream(stream, k_c.device)), "kvc_channel_prune_query")
    return channels, k_pruned


def kvc_channel_prune_value(k_c, v_c, q_obs, channels, v_pruned, *, recent, lam, scale=None, mask=None,
                            workspace=None, stream=None):
    """ThinK value-channel pruning of v_c [Hkv, budget, D], scored with k_c and the window queries q_obs [H, w, D]."""
    for t, n in ((k_c, "k_c"), (v_c, "v_c"), (q_obs, "q_obs")):
        _bf16(t, n)
    Hkv, budget, D = k_c.shape
    H, w, Dq = q_obs.shape
    if not (k_c.is_contiguous() and v_c.is_contiguous()) or v_c.shape != k_c.shape:
        raise ValueError("k_c and v_c must be contiguous [Hkv, budget, D] tensors of one shape")
    if Dq != D or H % Hkv or q_obs.stride(1) != D or q_obs.stride(2) != 1:
        raise ValueError(f"shape mismatch: q_obs {tuple(q_obs.shape)}, k_c {tuple(k_c.shape)}")
    G = H // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    ws, nbytes = _workspace(_lib.kvc_channel_prune_value_workspace_size(Hkv, G, w, budget, recent, D), k_c.device,
                            workspace, stream)
    _check(_lib.kvc_channel_prune_value(_ptr(k_c), _ptr(v_c), _ptr(q_obs), Hkv, G, w, q_obs.stride(0), budget, D,
                                        recent, float(lam), float(scale), _ptr(channels), _ptr(mask),
                                        _ptr(v_pruned), _ptr(ws), nbytes, _stream(stream, k_c.device)),
           "kvc_channel_prune_value")
    return channels, v_pruned


# ---------------------------------------------------------------- Keyformer decode phase
def kvc_decode_init_scores(importance, indices, acc, *, n, stream=None):
    """acc [Hkv, B] = importance [Hkv, >= n] at the kept prefix indices [Hkv, B], else 0."""
    if importance.dtype != torch.float32 or acc.dtype != torch.float32 or indices.dtype != torch.int32:
        raise TypeError("importance and acc must be float32, indices int32")
    Hkv, B = indices.shape
    if acc.shape != indices.shape or not acc.is_contiguous() or not indices.is_contiguous():
        raise ValueError("acc and indices must be contiguous [Hkv, B]")
    if importance.dim() != 2 or importance.stride(1) != 1 or importance.shape[0] != Hkv:
        raise ValueError("importance must be [Hkv, n] with unit stride along n")
    _check(_lib.kvc_decode_init_scores(_ptr(importance), importance.stride(0), _ptr(indices), Hkv, B, int(n),
                                       _ptr(acc), _stream(stream, acc.device)), "kvc_decode_init_scores")
    return acc


def kvc_keyformer_decode_step(q, k_new, v_new, k_cache, v_cache, pos, acc, *, t, recent, tau=1.0, seed=0,
                              scale=None, evicted=None, workspace=None, stream=None):
    """One Keyformer decode step: q [H, D], k_new / v_new [Hkv, D], caches [Hkv, B, D] (in place),
    pos int32 / acc float32 [Hkv, B] (in place), optional evicted int32 [Hkv]."""
    for x, nme in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _bf16(x, nme)
    Hkv, B, D = k_cache.shape
    H = q.shape[0]
    if H % Hkv or q.shape[-1] != D or q.stride(-1) != 1 or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between q and the caches")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous() and k_new.is_contiguous() and v_new.is_contiguous()):
        raise ValueError("caches and new rows must be contiguous")
    if pos.dtype != torch.int32 or acc.dtype != torch.float32 or pos.shape != (Hkv, B) or acc.shape != (Hkv, B):
        raise ValueError("pos must be int32 and acc float32, both [Hkv, B]")
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    ws, nbytes = _workspace(_lib.kvc_keyformer_decode_step_workspace_size(Hkv, H // Hkv, B), k_cache.device,
                            workspace, stream)
    _check(_lib.kvc_keyformer_decode_step(_ptr(q), q.stride(0), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                          _ptr(v_cache), _ptr(pos), _ptr(acc), Hkv, H // Hkv, B, D, int(t),
                                          int(recent), float(scale), float(tau), int(seed) & (2 ** 64 - 1),
                                          _ptr(evicted), _ptr(ws), nbytes, _stream(stream, k_cache.device)),
           "kvc_keyformer_decode_step")
    return evicted


# ---------------------------------------------------------------- timing
def kvc_timing_enable(enable=True):
    _check(_lib.kvc_timing_enable(1 if enable else 0), "kvc_timing_enable")


def kvc_timing_read():
    """{kernel name: (launches, total_ms)} for launches since kvc_timing_enable."""
    n = _lib.kvc_timing_count()
    if n < 0:
        raise KvcError(KVC_E_DEVICE, "kvc_timing_count")
    out = {}
    buf = ctypes.create_string_buffer(128)
    for i in range(n):
        cnt, ms = ctypes.c_int32(), ctypes.c_double()
        _check(_lib.kvc_timing_read(i, buf, 128, ctypes.byref(cnt), ctypes.byref(ms)), "kvc_timing_read")
        out[buf.value.decode()] = (cnt.value, ms.value)
    return out
