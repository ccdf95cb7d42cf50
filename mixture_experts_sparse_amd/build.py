"""Builds libmoe.so in-tree with hipcc for gfx950.

    python -m mixture_experts_sparse_amd.build [-v]

Every HIP source is compiled with packed-fp32 instruction generation off
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass warns
that it does not know the feature, which is harmless.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libmoe.so")
ARCH = "gfx950"

SOURCES = ["moe_api.cpp", "route_dispatch.hip", "expert_gemm.hip", "expert_gemm_small.hip", "combine.hip",
           "routing_stats.hip", "backward.hip", "noalloc.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe.so)")


def _compile(src: str, verbose: bool, defines=(), tag: str = "") -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + tag + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src),
           "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    lines = [ln for ln in out.splitlines() if noise not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)
    return obj


def build(verbose: bool = False, defines=(), lib_path: str = LIB_PATH) -> str:
    """Compiles every source and links libmoe.so (or ``lib_path``); returns its
    path. ``defines`` are extra -D flags (tuning variants)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        tag = "" if not defines else "_" + "_".join(d.replace("=", "") for d in defines)
        objs = list(ex.map(lambda s: _compile(s, verbose, defines, tag), SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
