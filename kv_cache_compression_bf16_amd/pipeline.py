"""Composition of the C-ABI calls into whole compression passes.

Each pass is a fixed sequence of libkvc calls on one stream: score ->
[SnapKV pooling] -> [ZigZag budgets] -> select (top-k, or KVzap's threshold with packed
heads) -> compact -> [ThinK: key channels by norms or by the window queries; value
channels].  Buffers are allocated once
per plan (through torch) so a pass itself allocates nothing on the device.
No arithmetic happens here.
"""

import numpy as np
import torch

from . import kvc


def bf16_to_device(bits, device):
    """Raw bf16 bit patterns (numpy uint16) -> torch.bfloat16 tensor on ``device``."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


class CompressionPlan:
    """Buffers and call sequence for one workload (see ``workload.Workload``)."""

    def __init__(self, wl, device, tau=1.0):
        self.wl = wl
        self.device = device
        self.tau = tau
        f32, i32, bf = torch.float32, torch.int32, torch.bfloat16
        L, Hkv, n, D = wl.L, wl.Hkv, wl.n, wl.D
        self.importance = torch.empty((L, Hkv, wl.imp_len), dtype=f32, device=device)
        # scores the selection ranks: the importance, or its SnapKV pooling
        self.pooled = torch.empty_like(self.importance) if wl.pool_kernel else None
        self.scores = self.pooled if wl.pool_kernel else self.importance
        self.zigzag = bool(wl.total_budget)
        # workspace for kvc_score sized from a representative ScoreArgs
        a = kvc.ScoreArgs()
        a.L, a.H, a.Hkv, a.w, a.S, a.D = L, wl.H, Hkv, wl.w, wl.S, D
        a.q_head_stride, a.q_layer_stride = wl.w * D, wl.H * wl.w * D
        a.k_head_stride, a.k_layer_stride = wl.S * D, Hkv * wl.S * D
        a.scale, a.gumbel, a.tau = 1.0, 1 if wl.gumbel else 0, 1.0
        nb = kvc.lib.kvc_score_causal_workspace_size(a) if wl.causal else kvc.kvc_score_workspace_size(a)
        self.ws_score = torch.empty(max(nb, 256), dtype=torch.uint8, device=device)
        sel_ws = kvc.lib.kvc_select_topk_workspace_size(Hkv, wl.S - wl.select_w)
        self.ws_select = torch.empty(max(sel_ws, 256), dtype=torch.uint8, device=device)
        if self.zigzag:
            self.budgets = torch.empty(L, dtype=i32, device=device)
            self.mba = torch.empty((L, Hkv), dtype=i32, device=device)
            tot = wl.total_budget
            self.indices_flat = torch.empty(Hkv * tot, dtype=i32, device=device)
            self.kc_flat = torch.empty(Hkv * tot * D, dtype=bf, device=device)
            self.vc_flat = torch.empty(Hkv * tot * D, dtype=bf, device=device)
        elif wl.threshold > 0:
            cap = Hkv * wl.capacity                  # the most a threshold can keep
            self.ws_thr = torch.empty(max(kvc.lib.kvc_select_threshold_workspace_size(Hkv, wl.S, wl.w, wl.recent),
                                          256), dtype=torch.uint8, device=device)
            self.indices_flat = torch.empty(cap, dtype=i32, device=device)
            self.offsets = torch.empty(Hkv + 1, dtype=i32, device=device)
            self.kc_flat = torch.empty((cap, D), dtype=bf, device=device)
            self.vc_flat = torch.empty((cap, D), dtype=bf, device=device)
        else:
            B = wl.budget
            self.indices = torch.empty((Hkv, B), dtype=i32, device=device)
            self.kc = torch.empty((Hkv, B, D), dtype=bf, device=device)
            self.vc = torch.empty((Hkv, B, D), dtype=bf, device=device)
        self.think = wl.think_lambda >= 0
        if self.think:
            T = kvc.kvc_think_channels(D, wl.think_lambda)
            rows = wl.budget - wl.recent
            self.channels = torch.empty((Hkv, T), dtype=i32, device=device)
            self.mask = torch.empty((Hkv, D), dtype=torch.uint8, device=device)
            self.kp = torch.empty((Hkv, rows, T), dtype=bf, device=device)
            if wl.think_query:
                nb = kvc.lib.kvc_channel_prune_query_workspace_size(Hkv, wl.G, wl.budget, D)
            else:
                nb = kvc.lib.kvc_channel_prune_workspace_size(Hkv, wl.budget, D)
            self.ws_think = torch.empty(max(nb, 256), dtype=torch.uint8, device=device)
        self.think_value = wl.think_value_lambda >= 0
        if self.think_value:
            Tv = kvc.kvc_think_channels(D, wl.think_value_lambda)
            rows = wl.budget - wl.recent
            self.channels_v = torch.empty((Hkv, Tv), dtype=i32, device=device)
            self.mask_v = torch.empty((Hkv, D), dtype=torch.uint8, device=device)
            self.vp = torch.empty((Hkv, rows, Tv), dtype=bf, device=device)
            nb = kvc.lib.kvc_channel_prune_value_workspace_size(Hkv, wl.G, wl.w, wl.budget, wl.recent, D)
            self.ws_think_v = torch.empty(max(nb, 256), dtype=torch.uint8, device=device)

    def decode_init(self, stream=None):
        """Hand the prompt phase's cache to the decode phase: slot positions are the
        kept indices, accumulated scores the prompt importance of kept prefix tokens."""
        wl = self.wl
        self.pos = self.indices.clone()
        self.acc = torch.empty(self.indices.shape, dtype=torch.float32, device=self.device)
        self.evicted = torch.empty(wl.Hkv, dtype=torch.int32, device=self.device)
        nb = kvc.lib.kvc_keyformer_decode_step_workspace_size(wl.Hkv, wl.G, wl.budget)
        self.ws_decode = torch.empty(max(nb, 256), dtype=torch.uint8, device=self.device)
        kvc.kvc_decode_init_scores(self.importance[0], self.indices, self.acc, n=wl.n, stream=stream)

    def decode_step(self, q, k_new, v_new, t, stream=None):
        """One Keyformer decode step on the compacted cache (in place)."""
        wl = self.wl
        kvc.kvc_keyformer_decode_step(q, k_new, v_new, self.kc, self.vc, self.pos, self.acc, t=t, recent=wl.recent,
                                      tau=self.tau, seed=wl.noise_seed, evicted=self.evicted,
                                      workspace=self.ws_decode, stream=stream)

    def score(self, q, k, layer_scales=None, stream=None):
        wl = self.wl
        (kvc.kvc_score_causal if wl.causal else kvc.kvc_score)(q, k, self.importance if wl.L > 1 else self.importance[0], w=wl.w, S=wl.S,
                      layer_scales=layer_scales, gumbel=wl.gumbel, tau=self.tau, seed=wl.noise_seed,
                      workspace=self.ws_score, stream=stream)

    def run(self, q, k, v, layer_scales=None, stream=None):
        """One whole pass.  q [L?, H, w, D], k/v [L?, Hkv, S, D] (bf16 on device)."""
        wl = self.wl
        self.score(q, k, layer_scales, stream)
        if wl.pool_kernel:
            kvc.kvc_pool_importance(self.importance, self.pooled, kernel=wl.pool_kernel, mode=wl.pool_mode,
                                    stream=stream)
        if wl.threshold > 0:
            kvc.kvc_select_threshold(self.scores[0], self.indices_flat, self.offsets, S=wl.S, w=wl.w,
                                     recent=wl.recent, threshold=wl.theta, workspace=self.ws_thr, stream=stream)
            kvc.kvc_compact_ragged(k if k.dim() == 3 else k[0], v if v.dim() == 3 else v[0], self.indices_flat,
                                   self.offsets, self.kc_flat, self.vc_flat, S=wl.S, stream=stream)
            return
        if not self.zigzag:
            kvc.kvc_select_topk(self.scores[0], self.indices, S=wl.S, w=wl.select_w, recent=wl.recent,
                                budget=wl.budget, workspace=self.ws_select, stream=stream)
            kvc.kvc_compact(k if k.dim() == 3 else k[0], v if v.dim() == 3 else v[0], self.indices, self.kc,
                            self.vc, S=wl.S, stream=stream)
            if self.think and wl.think_query:
                kvc.kvc_channel_prune_query(self.kc, q if q.dim() == 3 else q[0], self.channels, self.kp,
                                            recent=wl.recent, lam=wl.think_lambda, mask=self.mask,
                                            workspace=self.ws_think, stream=stream)
            elif self.think:
                kvc.kvc_channel_prune(self.kc, self.channels, self.kp, recent=wl.recent, lam=wl.think_lambda,
                                      p=wl.think_p, mask=self.mask, workspace=self.ws_think, stream=stream)
            if self.think_value:
                kvc.kvc_channel_prune_value(self.kc, self.vc, q if q.dim() == 3 else q[0], self.channels_v, self.vp,
                                            recent=wl.recent, lam=wl.think_value_lambda, mask=self.mask_v,
                                            workspace=self.ws_think_v, stream=stream)
            return
        kvc.kvc_lmba_budget(self.importance, self.budgets, total_budget=wl.total_budget,
                            floor_per_layer=wl.floor, capacity=wl.capacity, mass=wl.mass, mba=self.mba,
                            stream=stream)
        if wl.n_candidates <= kvc.SELECT_ONE_WORKGROUP_MAX:
            # every layer in one launch each, budgets read on the device: no host round trip
            kvc.kvc_select_topk_layers(self.scores, self.budgets, self.indices_flat, S=wl.S, w=wl.w,
                                       recent=wl.recent, total_budget=wl.total_budget, stream=stream)
            kvc.kvc_compact_layers(k, v, self.budgets, self.indices_flat, self.kc_flat.view(-1, wl.D),
                                   self.vc_flat.view(-1, wl.D), S=wl.S, total_budget=wl.total_budget,
                                   stream=stream)
            return
        # long prompts: one call per layer, sized from the budgets on the host
        for l, (B, idx, kc, vc) in enumerate(self.zigzag_layers(stream)):
            kvc.kvc_select_topk(self.scores[l], idx, S=wl.S, w=wl.w, recent=wl.recent, budget=B,
                                workspace=self.ws_select, stream=stream)
            kvc.kvc_compact(k[l], v[l], idx, kc, vc, S=wl.S, stream=stream)

    def zigzag_layers(self, stream=None):
        """Per-layer (budget, indices, K, V) views of the ZigZag outputs.  Reads the
        budgets back to the host after synchronising ``stream`` (the one the budget
        kernel was enqueued on; None: torch's current stream of the device)."""
        wl = self.wl
        Hkv, D = wl.Hkv, wl.D
        (stream if stream is not None else torch.cuda.current_stream(self.device)).synchronize()
        out, off = [], 0
        for B in self.budgets.cpu().tolist():
            idx = self.indices_flat[off * Hkv:(off + B) * Hkv].view(Hkv, B)
            kc = self.kc_flat[off * Hkv * D:(off + B) * Hkv * D].view(Hkv, B, D)
            vc = self.vc_flat[off * Hkv * D:(off + B) * Hkv * D].view(Hkv, B, D)
            out.append((B, idx, kc, vc))
            off += B
        return out
