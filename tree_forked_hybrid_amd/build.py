"""Build libflide.so (HIP kernels for gfx950 + C ABI) in-tree with hipcc.

    python -m tree_forked_hybrid_amd.build            # incremental
    python -m tree_forked_hybrid_amd.build --force    # rebuild everything
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libflide.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")

SOURCES = [
    "plan.cpp",
    "store.cpp",
    "api.cpp",
    "meta_kernels.hip",
    "attn_kernels.hip",
    "gdn_kernels.hip",
    "gdn_chunk_kernels.hip",
    "readout_kernels.hip",
    "noalloc.hip",
    "peak_kernels.hip",
    "stack_kernels.hip",
]
HEADERS = ["flide_internal.hpp", "device_common.hpp"]

ARCH = "gfx950"
# Packed fp32 VALU ops are disabled for every HIP translation unit.
FLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", f"-I{INCLUDE}"]


# Per-source flags.  attn_kernels.hip: no NaN reaches the attention arithmetic (masked scores are -inf,
# never NaN), so max() over MFMA results needs no quieting of signaling NaNs (one canonicalising
# v_max per operand otherwise).
SOURCE_FLAGS = {"attn_kernels.hip": ["-fno-honor-nans"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libflide.so)")


def _newest_dep() -> float:
    deps = [os.path.join(CSRC, h) for h in HEADERS] + [os.path.join(INCLUDE, "flide.h")]
    return max(os.path.getmtime(p) for p in deps)


def _compile(src: str, force: bool, dep_time: float) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src.replace(".", "_") + ".o")
    if (not force and os.path.exists(obj) and os.path.getmtime(obj) >= os.path.getmtime(path)
            and os.path.getmtime(obj) >= dep_time):
        return obj
    cmd = [_hipcc(), *FLAGS, *SOURCE_FLAGS.get(src, []), "-x", "hip", "-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(force: bool = True, jobs: int = 8) -> str:
    """Compile every source for gfx950 and link libflide.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    dep_time = _newest_dep()
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, force, dep_time), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--force", action="store_true")
    ap.add_argument("-j", type=int, default=8)
    a = ap.parse_args()
    print(build(force=a.force, jobs=a.j))
