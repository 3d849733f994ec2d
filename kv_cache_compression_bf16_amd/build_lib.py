"""Build libkvc.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m kv_cache_compression_bf16_amd.build_lib`` or ``build()``.
Objects go to ``kv_cache_compression_bf16_amd/_build/``; the shared library to
``kv_cache_compression_bf16_amd/libkvc.so``.  Always recompiles.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvc.so")

SOURCES = ["kvc_common.hip", "score.hip", "pool.hip", "select.hip", "threshold.hip", "compact.hip", "budget.hip",
           "think.hip", "decode.hip"]
# the benchmark's peak probes: a library of their own, not part of the path
PEAK_SOURCES = ["peak.hip"]
PEAK_LIB = os.path.join(PKG, "libkvc_peak.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",          # explicit fmaf only: both score passes round identically
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",  # MFMA results stay in VGPRs: no AGPR copies before the exp epilogue
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkvc.so)")


def _compile(src, extra=(), build_dir=BUILD):
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose=False, jobs=None, extra_flags=(), out=LIB, build_dir=BUILD, peak=True):
    """Compile every source and link ``out`` (and, with ``peak``, the probe
    library libkvc_peak.so); ``extra_flags`` (e.g. -D switches) build an
    alternative variant of the library for A/B measurements."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = SOURCES + (PEAK_SOURCES if peak else [])
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda src: _compile(src, extra_flags, build_dir), srcs))
    objs = dict(zip(srcs, (o for o, _ in results)))
    if verbose:
        for (_, err), src in zip(results, srcs):
            warn = "\n".join(l for l in err.splitlines() if "packed-fp32-ops" not in l and l.strip())
            if warn:
                print(f"[{src}] {warn}", file=sys.stderr)
    _link([objs[s] for s in SOURCES], out)
    if peak:
        _link([objs[s] for s in PEAK_SOURCES], PEAK_LIB)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
