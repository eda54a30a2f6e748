"""Build ``libkvpop.so`` in-tree with hipcc for gfx950.

    python -m fixed_budget_learned_amd.build [--timeline]

``--timeline`` builds ``libkvpop_timeline.so`` instead: the same library with
the decode kernel's device-clock stamps compiled in (``-DKVPOP_TIMELINE``),
read by ``python -m fixed_budget_learned_amd.timeline``.

Every source is compiled every time (a few seconds per file); the objects go
to ``_build/`` at the repository root and the library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libkvpop.so")
TIMELINE_LIB_PATH = os.path.join(PKG, "libkvpop_timeline.so")
ARCH = "gfx950"

SOURCES = ["kvpop_abi.cpp", "kvpop_prefill.hip", "kvpop_decode.hip", "kvpop_thresholds.hip",
           "kvpop_future.hip", "kvpop_prune.hip"]

# Packed-FP32 instructions are disabled for all device code.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]

# Per-file additions.  The MFMA kernels keep their accumulators in ordinary
# VGPRs: the softmax reads every accumulator element, and from AGPRs each
# read would be one more VALU instruction.
FILE_FLAGS = {"kvpop_future.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libkvpop.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops" not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)


def build(verbose: bool = False, timeline: bool = False) -> str:
    hipcc = _hipcc()
    bdir = os.path.join(BUILD_DIR, "timeline") if timeline else BUILD_DIR
    out = TIMELINE_LIB_PATH if timeline else LIB_PATH
    extra = ["-DKVPOP_TIMELINE"] if timeline else []
    os.makedirs(bdir, exist_ok=True)
    jobs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        jobs.append([hipcc] + COMMON_FLAGS + extra + FILE_FLAGS.get(src, []) + lang +
                    ["-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        for f in [ex.submit(_run, j, verbose) for j in jobs]:
            f.result()
    tmp = out + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:], timeline="--timeline" in sys.argv[1:]))
