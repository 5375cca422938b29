"""Build libpagedkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_320_amd.build        # or build() from Python

Every HIP source is compiled for gfx950 only. Packed fp32 instructions are
switched off for device code (-packed-fp32-ops); hipcc's host pass warns that
it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpagedkv.so")
# (source, object, extra flags): decode_inst.hip is compiled once per (key/value format,
# query/output format, head_dim) instance set
DECODE_INSTANCES = [(kt, qt, d) for kt, qt in (("PA_F32", "PA_F32"), ("PA_F16", "PA_F16"),
                                               ("PA_BF16", "PA_BF16"), ("PA_FP8_E4M3", "PA_F16"),
                                               ("PA_FP8_E4M3", "PA_BF16"))
                    for d in (64, 128)]
# The matrix-core decode keeps its accumulators in ordinary VGPRs: left to its heuristics the
# compiler put 64 of them in AGPRs and copied them back and forth around every rescale (about
# 500 accvgpr moves per two chunks); in VGPRs the 8-query-head decode of the Llama-2-70B-shaped
# step went from 104.5-106.9 to 95.9-98.1 us per op.
MFMA_VGPR = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
UNITS = [(src, os.path.splitext(src)[0], []) for src in
         ("api.cpp", "allocator.cpp", "cache_ops.hip", "decode.hip", "prefill.hip", "probe.hip")] + \
        [("decode_inst.hip", f"decode_inst_{kt}_{qt}_d{d}".lower(),
          [f"-DPA_INST_KT={kt}", f"-DPA_INST_QT={qt}", f"-DPA_INST_D={d}", *MFMA_VGPR])
         for kt, qt, d in DECODE_INSTANCES]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpagedkv.so)")


def flags() -> list:
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument"]


def _compile(cc: str, src: str, obj: str, extra: list, verbose: bool) -> None:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [cc, *flags(), *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source (in parallel) and link libpagedkv.so next to this file."""
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, name + ".o") for _, name, _ in UNITS]
    jobs = jobs or max(1, min(len(UNITS), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        futs = [pool.submit(_compile, cc, src, obj, extra, verbose)
                for (src, _, extra), obj in zip(UNITS, objs)]
        for f in futs:
            f.result()
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libpagedkv.so failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
