"""Build libmarca.so in-tree: hipcc for the gfx950 kernels, g++ for the host ABI.

Run as ``python -m cache_aware_attention_amd.build`` or through
``__graft_entry__.build()``.  Objects go to ``_build/`` next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD = PKG / "_build"
LIB = PKG / "libmarca.so"

HIP_SOURCES = ["cache_attn.hip", "kv_scatter.hip", "refresh_topk.hip", "cos_gate.hip",
               "cfg_residual.hip"]
# Measurement kernels (include/mar_bench.h), a library of their own: the
# decoding path never loads it.
BENCH_SOURCES = ["bench_kernels.hip"]
BENCH_LIB = PKG / "libmarca_bench.so"
CPP_SOURCES = ["abi.cpp", "schedule.cpp"]
# Per-file device flags.  The attention kernels assume NaN-free inputs (a
# documented precondition of the ABI), which lets the compiler take maxima of
# matrix-core results without quieting them first.
HIP_EXTRA_FLAGS = {"cache_attn.hip": ["-fno-honor-nans"]}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmarca)")


def hip_flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
            # no packed fp32 instructions in device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass warns about the device-only feature flag; drop that noise
    msg = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if msg.strip():
        print(msg, file=sys.stderr)


def build(verbose: bool = False) -> Path:
    BUILD.mkdir(exist_ok=True)
    jobs = []
    for src in HIP_SOURCES + BENCH_SOURCES:
        obj = BUILD / (src + ".o")
        jobs.append([hipcc(), *hip_flags(), *HIP_EXTRA_FLAGS.get(src, []), "-c", str(CSRC / src),
                     "-o", str(obj)])
    for src in CPP_SOURCES:
        obj = BUILD / (src + ".o")
        jobs.append(["g++", "-O2", "-fPIC", "-std=c++17", "-Wall", "-Wextra",
                     f"-I{INCLUDE}", f"-I{CSRC}", "-c", str(CSRC / src), "-o", str(obj)])
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        list(ex.map(_run, jobs))
    for lib, sources in ((LIB, HIP_SOURCES + CPP_SOURCES), (BENCH_LIB, BENCH_SOURCES)):
        objs = [str(BUILD / (s + ".o")) for s in sources]
        tmp = lib.with_suffix(f".so.tmp{os.getpid()}")
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *objs])
        os.replace(tmp, lib)
        if verbose:
            print(f"built {lib}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
