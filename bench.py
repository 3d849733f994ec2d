"""Benchmark: prompt KV tokens compressed per second on one MI355X.

One step = one whole compression pass (score -> [ZigZag budgets] -> select ->
compact -> [ThinK]) over one synthetic prompt of the chosen workload, inputs
already resident in HBM.  Default workload: the Llama-3-8B-shaped GQA layer
(32 query / 8 KV heads, D 128, 32768-token prompt, window 128, budget 2048 per
KV head incl. 64 recent, 4 outlier key channels x8).

Prints ONE JSON line.  ``value`` = prompt tokens (layers x S) per second.
The input set rotates over enough copies to exceed the 256 MB Infinity Cache,
so every step reads its keys from HBM.  Per-kernel durations come from HIP
events that libkvc records around each launch on the launch stream
(kvc_timing_enable), in a second timed pass of the same steps.
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prompt KV tokens compressed/sec (score+top-k+gather); % of HBM roofline"
DECODE_METRIC = "Keyformer decode tokens/sec for one layer (score accumulation + eviction on the kept cache)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
CLOCK_HZ = 2.4e9                # MI355X peak engine clock, published
# Vector ALU roof in lane instructions: the published unpacked fp32 rate,
# 78.6 TFLOP/s, counts an FMA as 2 flops, i.e. 256 CUs x 4 SIMDs x 16 lanes x
# 2.4 GHz = 39.3 T lane-FMAs/s.  Other instruction classes are converted to
# FMA-equivalents by their cost per wave64 instruction relative to v_fma_f32,
# measured on the box by libkvc_peak in the same run (measure_peaks).
VALU_PEAK_TLANE = 256 * 4 * 16 * CLOCK_HZ / 1e12
# Lane instructions per noisy tempered logit of the Gumbel passes, by class:
#   philox_pair -- Philox4x32-10: 10 rounds x (2 v_mad_u64_u32 + 2 v_bitop3_b32)
#                  per 4 samples = 5 (product, three-input xor) pairs per sample;
#   trans       -- the two logs of -ln(-ln u) and the exp2 of the softmax;
#   simple      -- the uniform from a word (3), two scalings of the noise (2),
#                  (x c + g) / tau (2), and the softmax's max, shift and add in
#                  pass 1 (3) or shift and add in pass 2 (2).
GUMBEL_MIX_PASS1 = {"philox_pair": 5, "trans": 3, "simple": 10}
GUMBEL_MIX_PASS2 = {"philox_pair": 5, "trans": 3, "simple": 9}
MALL_BYTES = 256 * 2 ** 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa32x8_s32768")
    ap.add_argument("--tau", type=float, default=1.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline leg")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU oracle sample time")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (counter calibration)")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure the on-box peaks (and read bandwidth over buffer sizes)")
    return ap.parse_args()


def calibrate_copy(mib):
    """A plain copy of known size, for scaling FETCH_SIZE / WRITE_SIZE counter readings."""
    import torch

    n = mib * 2 ** 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}))


def _mix(mix, logits):
    """Lane instructions per class for `logits` noisy tempered logits."""
    return {c: n * logits for c, n in mix.items()}


def fma_equivalents(mix_counts, peaks):
    """Lane instructions of several classes -> v_fma_f32 equivalents, each class
    weighted by its measured cycles per wave64 instruction relative to FMA."""
    cyc = peaks["valu_cycles_per_wave_instr"]
    cost = {"simple": 1.0, "trans": cyc["exp2"] / cyc["fma"], "philox_pair": cyc["mad_u64+bitop3"] / cyc["fma"]}
    return sum(n * cost[c] for c, n in mix_counts.items())


def measure_peaks(dev, stream, sweep=False):
    """On-box peaks from libkvc_peak (its own probe kernels, timed with events on
    `stream`): HBM read stream over 2 GiB, Infinity Cache read over 96 MiB, dense
    bf16 MFMA, and the issue cost of each vector instruction class."""
    import ctypes

    import torch

    from kv_cache_compression_bf16_amd import build_lib

    lib = ctypes.CDLL(build_lib.PEAK_LIB)
    P, SZ, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.kvc_peak_read.argtypes = [P, SZ, P, P]
    lib.kvc_peak_mfma.argtypes = [P, I, P]
    lib.kvc_peak_valu.argtypes = [I, P, I, P]
    for f in ("kvc_peak_read_sink_words", "kvc_peak_mfma_sink_words", "kvc_peak_valu_sink_words"):
        getattr(lib, f).restype = SZ
    lib.kvc_peak_mfma_flops.restype = ctypes.c_double
    lib.kvc_peak_valu_wave_instructions.restype = ctypes.c_double
    lib.kvc_peak_mfma_flops.argtypes = [I]
    lib.kvc_peak_valu_wave_instructions.argtypes = [I]
    sp = ctypes.c_void_p(stream.cuda_stream)
    cus = lib.kvc_peak_cus()

    def timed(launch, reps):
        assert launch() == 0
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / 1e3          # seconds per launch

    out = {"cus": cus}
    sink = torch.empty(max(lib.kvc_peak_read_sink_words(), lib.kvc_peak_mfma_sink_words(),
                           lib.kvc_peak_valu_sink_words()), dtype=torch.int32, device=dev)
    big = 2 << 30
    buf = torch.empty(big, dtype=torch.uint8, device=dev)
    t = timed(lambda: lib.kvc_peak_read(P(buf.data_ptr()), big, P(sink.data_ptr()), sp), 5)
    out["hbm_read_GBs"] = big / t / 1e9
    small = 96 << 20
    t = timed(lambda: lib.kvc_peak_read(P(buf.data_ptr()), small, P(sink.data_ptr()), sp), 20)
    out["infinity_cache_read_GBs"] = small / t / 1e9
    del buf
    iters = 4096
    t = timed(lambda: lib.kvc_peak_mfma(P(sink.data_ptr()), iters, sp), 3)
    out["mfma_bf16_TFLOPs"] = lib.kvc_peak_mfma_flops(iters) / t / 1e12
    cyc = {}
    for op, name in enumerate(("fma", "add", "exp2", "log2", "mad_u64+bitop3", "bitop3")):
        it = 2048
        t = timed(lambda: lib.kvc_peak_valu(op, P(sink.data_ptr()), it, sp), 3)
        per_simd = lib.kvc_peak_valu_wave_instructions(it) / (cus * 4)
        cyc[name] = t * CLOCK_HZ / per_simd             # at the published 2.4 GHz clock
    out["valu_cycles_per_wave_instr"] = cyc
    out["valu_fma_Tlane"] = 64 * 4 * cus * CLOCK_HZ / cyc["fma"] / 1e12
    if sweep:
        # read bandwidth against the buffer size: L2 (4 MB per XCD), Infinity Cache
        # (256 MB), HBM
        buf = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
        out["read_GBs_by_MiB"] = {}
        for mib in (16, 32, 64, 128, 192, 256, 512, 1024, 2048):
            n = mib << 20
            t = timed(lambda: lib.kvc_peak_read(P(buf.data_ptr()), n, P(sink.data_ptr()), sp), max(3, 2048 // mib))
            out["read_GBs_by_MiB"][mib] = round(n / t / 1e9)
        del buf
    return out


def algorithmic(wl, kept_rows=None):
    """Algorithmic bytes and flops of one step, and per-kernel figures.  kept_rows:
    the kept (head, token) rows of a threshold selection, which depend on the data."""
    L, H, Hkv, S, w, D, G = wl.L, wl.H, wl.Hkv, wl.S, wl.w, wl.D, wl.G
    n = S - w
    R = G * w
    q_bytes = L * H * w * D * 2
    k_prefix = L * Hkv * n * D * 2
    imp = L * Hkv * n * 4
    if wl.threshold > 0:
        B_total = kept_rows
    else:
        B_total = wl.total_budget * Hkv if wl.total_budget else L * Hkv * wl.budget
    rows = B_total * D * 2
    flops_pass = 2.0 * L * Hkv * R * n * D
    if wl.causal:
        # every key up to the row's position: w (S - w) + w (w + 1) / 2 (row, key) pairs per query head
        n = S
        k_prefix = L * Hkv * n * D * 2
        imp = L * Hkv * n * 4
        flops_pass = 2.0 * D * L * H * (w * (S - w) + w * (w + 1) / 2)
    step_bytes = q_bytes + k_prefix + 2 * imp + B_total * 4 + 2 * rows * 2
    if wl.think_lambda >= 0:
        T = int(math.floor((1 - wl.think_lambda) * D))
        kr = Hkv * (wl.budget - wl.recent)
        step_bytes += kr * D * 2 + kr * T * 2
    if wl.think_lambda >= 0 and wl.think_query:
        step_bytes += q_bytes
    if wl.pool_kernel:
        step_bytes += 2 * imp
    if wl.decode_steps:
        # one decode step: the cache keys once, pos and acc read and written, new rows, queries
        B = wl.budget
        dec_bytes = Hkv * B * D * 2 + Hkv * B * 12 + 2 * Hkv * D * 2 * 2 + H * D * 2
        logits = H * (B + 1) * 4        # the step's tempered logits, written then read once
        return dec_bytes, 0.0, {
            "keyformer_decode_logits": ("hbm", 0.0, Hkv * (B + 1) * D * 2 + Hkv * B * 4 + H * D * 2 + logits),
            "keyformer_decode_update": ("hbm", 0.0, logits + Hkv * B * 12 + 2 * Hkv * D * 2 * 2),
        }
    # per step (bench divides by the launches per step): bound, flops, algorithmic
    # bytes[, vector operations]
    logits = flops_pass / (2.0 * D)
    per_kernel = {
        "score_pass1": ("mfma", flops_pass, q_bytes + k_prefix),
        "score_pass2": ("mfma", flops_pass, q_bytes + k_prefix + imp),
        "score_pass1_gumbel": ("mfma", flops_pass, q_bytes + k_prefix, _mix(GUMBEL_MIX_PASS1, logits)),
        "score_pass2_gumbel": ("mfma", flops_pass, q_bytes + k_prefix + imp, _mix(GUMBEL_MIX_PASS2, logits)),
        "score_causal_pass1_gumbel": ("mfma", flops_pass, q_bytes + k_prefix, _mix(GUMBEL_MIX_PASS1, logits)),
        "score_causal_pass2_gumbel": ("mfma", flops_pass, q_bytes + k_prefix + imp, _mix(GUMBEL_MIX_PASS2, logits)),
        "score_causal_pass1": ("mfma", flops_pass, q_bytes + k_prefix),
        "score_causal_pass2": ("mfma", flops_pass, q_bytes + k_prefix + imp),
        "select_topk": ("hbm", 0.0, imp + B_total * 4),
        "threshold_count": ("hbm", 0.0, imp),
        "threshold_emit": ("hbm", 0.0, imp + B_total * 4),
        "compact_ragged": ("hbm", 0.0, 2 * rows * 2 + B_total * 4),
        "compact": ("hbm", 0.0, 2 * rows * 2 + B_total * 4),
        "lmba_mba": ("hbm", 0.0, imp),
        "pool_importance": ("hbm", 0.0, 2 * imp),
    }
    if wl.think_lambda >= 0:
        T = int(math.floor((1 - wl.think_lambda) * D))
        kr = Hkv * (wl.budget - wl.recent)
        per_kernel["think_partial"] = ("hbm", 0.0, kr * D * 2)
        per_kernel["think_gather"] = ("hbm", 0.0, kr * D * 2 + kr * T * 2)
        if wl.think_query:
            per_kernel["think_qpartial"] = ("hbm", 0.0, q_bytes)
    if wl.think_value_lambda >= 0:
        Tv = int(math.floor((1 - wl.think_value_lambda) * D))
        U = wl.budget - wl.recent
        kr = Hkv * U
        step_bytes += 2 * kr * D * 2 + q_bytes + kr * D * 2 + kr * Tv * 2
        # softmax constants over U (pass 1 of the scoring path), then S = K Q^T and O = P V
        per_kernel["think_rowc_pass1"] = ("mfma", 2.0 * Hkv * R * U * D, q_bytes + kr * D * 2)
        per_kernel["think_vpartial"] = ("mfma", 4.0 * Hkv * R * U * D, q_bytes + 2 * kr * D * 2)
        per_kernel["think_gather_v"] = ("hbm", 0.0, kr * D * 2 + kr * Tv * 2)
    return step_bytes, flops_pass, per_kernel


KERNEL_SOURCE = {"score": "score.hip", "select": "select.hip", "compact": "compact.hip", "lmba": "budget.hip",
                 "pool": "pool.hip", "threshold": "threshold.hip", "keyformer": "decode.hip", "decode": "decode.hip",
                 "think": "think.hip"}


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (profiles/hbm_traffic_<workload>.md), or None if there is none or the kernel's
    source (common.h, philox.h for the scoring and decode kernels, its .hip file)
    has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    csrc = os.path.join(ROOT, "kv_cache_compression_bf16_amd", "csrc")
    h = hashlib.sha256()
    src = KERNEL_SOURCE[kernel.split("_")[0]]
    for f in ("common.h",) + (("philox.h",) if src in ("score.hip", "decode.hip") else ()) + (src,):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    for line in open(path):
        m = re.match(r"traffic kernel=(\S+) read_bytes=(\d+) write_bytes=(\d+) source=\S+ sha256_16=([0-9a-f]+)", line)
        if m and m.group(1) == kernel:
            if m.group(4) != h.hexdigest()[:16]:
                return None
            return int(m.group(2)) + int(m.group(3))
    return None


# ---- CPU oracle baseline ----------------------------------------------------
# Workers are forked before anything touches the GPU and hold the host inputs
# copy-on-write; each runs the oracle with BLAS pinned to one thread.
_CPU = {}


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits

    _CPU["limits"] = threadpool_limits(1)


def _causal_row(wl, u):
    """The query row of causal unit u: rows visited with an odd stride, so a short
    sample spreads over short and long rows alike."""
    return ((u // wl.H) * 4099) % wl.w


def _cpu_unit(u):
    """One unit of oracle work: a whole KV head of layer 0 (score [+ pool] + select
    + compact [+ ThinK]), or one causal query row.  Returns the unit index."""
    import numpy as np
    import oracle

    wl, (q, k, v), tau = _CPU["wl"], _CPU["data"], _CPU["tau"]
    scale = float(np.float32(1.0 / math.sqrt(wl.D)))
    if wl.causal:
        h, i = u % wl.H, _causal_row(wl, u)
        oracle.score.head_causal_mean(oracle.score.bf16_bits_to_f64(q[h]),
                                      oracle.score.bf16_bits_to_f64(k[h // wl.G]), S=wl.S, w=wl.w, scale=scale,
                                      gumbel=wl.gumbel, seed=wl.noise_seed, head=h, tau=tau, rows=[i])
        return u
    q0 = q if wl.L == 1 else q[0]
    kraw = k if wl.L == 1 else k[0]
    vraw = v if wl.L == 1 else v[0]
    g = u % wl.Hkv
    qf = oracle.score.bf16_bits_to_f64(q0[g * wl.G:(g + 1) * wl.G])
    kf = oracle.score.bf16_bits_to_f64(kraw[g])
    B = wl.budget if wl.budget else wl.total_budget // wl.L
    # KV head g's importance: the sum of its query heads' window means (the noise keyed
    # by the true query-head index)
    imp = sum(oracle.score.head_window_mean(qf[i], kf, n=wl.n, scale=scale, gumbel=wl.gumbel, seed=wl.noise_seed,
                                            head=g * wl.G + i, S=wl.S, w=wl.w, tau=tau) for i in range(wl.G))
    sc = oracle.pool.pool(imp[None], wl.pool_kernel, wl.pool_mode)[0] if wl.pool_kernel else imp
    if wl.threshold > 0:
        idx = oracle.threshold.select_threshold(sc, S=wl.S, w=wl.w, recent=wl.recent, theta=wl.theta)
    else:
        idx = oracle.select.select(sc, S=wl.S, w=wl.w, recent=wl.recent, budget=B)
    kc = oracle.compact.compact(kraw[g:g + 1], idx[None])
    vc = oracle.compact.compact(vraw[g:g + 1], idx[None])
    if wl.think_value_lambda >= 0:
        oracle.think.think_prune_value(oracle.score.bf16_bits_to_f64(kc), oracle.score.bf16_bits_to_f64(vc), qf,
                                       recent=wl.recent, lam=wl.think_value_lambda, scale=scale)
    if wl.think_lambda >= 0 and wl.think_query:
        oracle.think.think_prune_query(oracle.score.bf16_bits_to_f64(kc), qf, recent=wl.recent,
                                       lam=wl.think_lambda)
    elif wl.think_lambda >= 0:
        oracle.think.think_prune(oracle.score.bf16_bits_to_f64(kc), recent=wl.recent, lam=wl.think_lambda,
                                 p=wl.think_p)
    return u


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(wl, data, target_s, tau, max_workers=16):
    """The oracle, as it stands, on a bounded sample of the same workload, spread
    over a process pool of one worker per available host core (at most
    ``max_workers``, the host share of one GPU), BLAS pinned to one thread each."""
    import multiprocessing as mp

    import numpy as np
    import oracle

    cores = max(1, min(len(os.sched_getaffinity(0)), max_workers))
    if wl.decode_steps:
        # decode steps depend on each other: one process, BLAS pinned to one thread,
        # from a kept cache of the workload's own rows (the prompt's recent window
        # plus evenly spaced prefix tokens, zero scores)
        from threadpoolctl import threadpool_limits

        from kv_cache_compression_bf16_amd import workload as wk
        q, k, v = data
        B, r = wl.budget, wl.recent
        pos = np.concatenate([np.linspace(0, wl.S - r - 1, B - r).astype(np.int64), np.arange(wl.S - r, wl.S)])
        kc, vc = k[:, pos], v[:, pos]
        pos = np.tile(pos, (wl.Hkv, 1))
        acc = np.zeros((wl.Hkv, B))
        scale = float(np.float32(1.0 / math.sqrt(wl.D)))
        steps, t0 = 0, time.perf_counter()
        with threadpool_limits(1):
            while time.perf_counter() - t0 < target_s:
                qd, kn, vn = wk.gen_decode(wl, steps)
                kc, vc, pos, acc, _ = oracle.decode.decode_step(kc, vc, pos, acc, oracle.score.bf16_bits_to_f64(qd),
                                                                kn, vn, t=wl.S + steps, recent=r, scale=scale,
                                                                tau=tau, seed=wl.noise_seed)
                steps += 1
        dt = time.perf_counter() - t0
        return {"value": steps / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle", "cpu_model": _cpu_model(),
                "sample": f"{steps} decode steps of all {wl.Hkv} KV heads from a kept cache of the workload's rows "
                          f"(fp64 numpy, one process: the steps are sequential), {dt:.1f} s"}
    _CPU.update(wl=wl, data=data, tau=tau)
    done, t0 = 0, time.perf_counter()
    with mp.get_context("fork").Pool(cores, initializer=_cpu_worker_init) as pool:
        # rounds of one unit per worker until the time target; whole rounds only
        while time.perf_counter() - t0 < target_s:
            done += len(pool.map(_cpu_unit, range(done, done + cores), chunksize=1))
        dt = time.perf_counter() - t0
    if wl.causal:
        # whole causal query rows (row i of every head in turn); scaled by the share of
        # the layer's (row, key) pairs done
        total_pairs = wl.H * (wl.w * (wl.S - wl.w) + wl.w * (wl.w + 1) / 2)
        pairs = sum(wl.S - wl.w + _causal_row(wl, u) + 1 for u in range(done))
        return {"value": wl.S * (pairs / total_pairs) / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
                "cpu_model": _cpu_model(),
                "sample": f"{done} causal query rows ({pairs} of the layer's {int(total_pairs)} (row, key) pairs; "
                          f"scoring only, fp64 numpy), {cores} worker processes x 1 BLAS thread, {dt:.1f} s"}
    steps = "+".join(["score"] + (["pool"] if wl.pool_kernel else [])
                     + (["threshold", "compact"] if wl.threshold > 0 else ["select", "compact"])
                     + (["think"] if wl.think_lambda >= 0 else [])
                     + (["think_value"] if wl.think_value_lambda >= 0 else []))
    return {"value": wl.S * done / wl.Hkv / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"{done} KV-head passes over layer 0 ({wl.Hkv} heads per layer; {steps}, fp64 numpy), "
                      f"{cores} worker processes x 1 BLAS thread, {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(heads, layers and sequence blocks would shard over GPUs, but no collective is built); "
              "rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.peaks:
        import torch

        dev = torch.device("cuda:0")
        print(json.dumps({"measured_peaks": measure_peaks(dev, torch.cuda.current_stream(dev), sweep=True)}))
        return

    import numpy as np
    import torch

    from kv_cache_compression_bf16_amd import kvc, pipeline
    from kv_cache_compression_bf16_amd import workload as wk

    dev = torch.device("cuda:0")
    wl = wk.WORKLOADS[args.workload]
    print(f"[bench] workload {wl.name}: generating inputs", file=sys.stderr, flush=True)
    if wl.L == 1:
        host = wk.gen_layer(wl)
    else:
        qs, ks, vs = zip(*(wk.gen_layer(wl, l) for l in range(wl.L)))
        host = (np.stack(qs), np.stack(ks), np.stack(vs))
    cpu = None
    if not args.no_cpu:
        # before anything touches the GPU: the oracle's worker processes are forked here
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, host, args.cpu_seconds, args.tau)
    set_bytes = sum(x.nbytes for x in host)
    copies = max(1, min(8, math.ceil(2 * MALL_BYTES / set_bytes)))
    base = [pipeline.bf16_to_device(x, dev) for x in host]
    sets = [base] + [[t.clone() for t in base] for _ in range(copies - 1)]
    ls = torch.from_numpy(wk.layer_scales(wl)).to(dev) if wl.scale_range else None
    plan = pipeline.CompressionPlan(wl, dev, tau=args.tau)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        q, k, v = sets[i % copies]
        plan.run(q, k, v, layer_scales=ls, stream=stream)

    if wl.decode_steps:
        # decode workload: the prompt phase once (untimed), then one timed step is
        # one decode step of the layer (the token at position S + i)
        step(0)
        plan.decode_init(stream=stream)
        n_dec = args.warmup + 2 * args.steps
        dec = [[pipeline.bf16_to_device(x, dev) for x in wk.gen_decode(wl, i)] for i in range(n_dec)]
        torch.cuda.synchronize()

        def step(i):   # noqa: F811 -- the decode workload's step
            q, kn, vn = dec[i]
            plan.decode_step(q, kn, vn, wl.S + i, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    i_next = args.warmup

    # ---- timed region: exactly `steps` steps between two events on the launch stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        step(i_next + i)   # decode positions keep increasing
    e1.record(stream)
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps

    # ---- per-kernel durations: same steps again with libkvc's per-launch events
    kvc.kvc_timing_enable(True)
    for i in range(args.steps):
        step(i_next + args.steps + i)
    torch.cuda.synchronize()
    kt = kvc.kvc_timing_read()
    kvc.kvc_timing_enable(False)

    peaks = measure_peaks(dev, stream)
    tokens = 1 if wl.decode_steps else wl.L * wl.S    # decode: one token of one layer per step
    value = tokens / (ms_step / 1e3)
    kept_rows = int(plan.offsets[-1].item()) if wl.threshold > 0 else None   # after the timed region
    step_bytes, flops_pass, per_kernel = algorithmic(wl, kept_rows)
    kernels = {name: {"launches": c, "avg_us": 1e3 * ms / c} for name, (c, ms) in kt.items()}
    dom = max(kt.items(), key=lambda kv: kv[1][1])[0]
    avg_s = kernels[dom]["avg_us"] / 1e6
    per_launch = args.steps / kernels[dom]["launches"]     # one step's figure -> one launch's
    bound, flops, nbytes, mix = (per_kernel.get(dom, ("hbm", 0.0, 0)) + ({},))[:4]
    ops = fma_equivalents(mix, peaks) if mix else 0.0
    # the roofline that binds this kernel: the longest of its MFMA, HBM and
    # vector-ALU times at peak (a scoring pass over few query rows moves more
    # bytes per flop than the chip's ratio and is HBM-bound; the Gumbel passes
    # spend more on Philox and logs than on their MFMA work)
    t_roof = {"mfma": flops / (MFMA_BF16_PEAK_TFLOPS * 1e12), "hbm": nbytes / (HBM_PEAK_GBS * 1e9),
              "alu": ops / (VALU_PEAK_TLANE * 1e12)}
    if bound == "mfma":
        bound = max(t_roof, key=t_roof.get)
    traffic = measured_traffic(dom, wl.name)
    if bound == "alu":
        achieved = ops * per_launch / avg_s / 1e12
        roof = {"bound": "alu", "achieved": achieved, "peak": VALU_PEAK_TLANE, "unit": "T lane-FMA-equivalents/s",
                "frac": achieved / VALU_PEAK_TLANE, "traffic": traffic, "measured_peak": peaks["valu_fma_Tlane"]}
    elif bound == "mfma":
        achieved = flops * per_launch / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic,
                "measured_peak": peaks["mfma_bf16_TFLOPs"]}
    else:
        achieved = nbytes * per_launch / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "measured_peak": peaks["hbm_read_GBs"]}
    roof["frac_of_measured_peak"] = roof["achieved"] / roof["measured_peak"]
    roof["kernel"] = dom
    roof["alg_bytes_per_launch"] = nbytes * per_launch
    for name, kk in kernels.items():
        b, f, nb, mx = (per_kernel.get(name, ("", 0.0, 0)) + ({},))[:4]
        pl = args.steps / kk["launches"]
        kk["alg_TFLOPs"] = round(f * pl / (kk["avg_us"] / 1e6) / 1e12, 2) if f else None
        kk["alg_GBs"] = round(nb * pl / (kk["avg_us"] / 1e6) / 1e9, 1) if nb else None
        if mx:
            kk["alg_T_lane_fma_eq"] = round(fma_equivalents(mx, peaks) * pl / (kk["avg_us"] / 1e6) / 1e12, 2)
        kk["avg_us"] = round(kk["avg_us"], 2)

    config = {"workload": wl.name, "layers": wl.L, "q_heads": wl.H, "kv_heads": wl.Hkv, "seq_len": wl.S,
              "head_dim": wl.D, "window": wl.w, "recent": wl.recent,
              "budget_per_kv_head": wl.budget or None, "total_budget": wl.total_budget or None,
              "gumbel_tau": args.tau if wl.gumbel else None, "pool_kernel": wl.pool_kernel or None,
              "threshold_x_uniform": wl.threshold or None, "kept_rows": kept_rows,
              "input_copies_rotated": copies}
    out = {
        "metric": DECODE_METRIC if wl.decode_steps else METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) bf16, workload recipe)",
        "config": config,
        "hbm_frac_step": step_bytes / (ms_step / 1e3) / (HBM_PEAK_GBS * 1e9),
        "alg_bytes_step": step_bytes, "alg_flops_score_pass": flops_pass,
        "roofline": roof, "kernels": kernels, "cpu_baseline": cpu,
        "measured_peaks": peaks,
        "published_peaks": {"hbm_GBs": HBM_PEAK_GBS, "mfma_bf16_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                            "valu_T_lane_fma": VALU_PEAK_TLANE},
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
