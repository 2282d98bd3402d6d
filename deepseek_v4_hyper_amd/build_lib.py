"""Build libds4hc.so (gfx950) in-tree with hipcc.

    python -m deepseek_v4_hyper_amd.build_lib          # from the repository root

All HIP code is built with packed-FP32 instruction selection turned off
(``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libds4hc.so")
SOURCES = ["hc_kernels.hip", "ds4hc_api.cpp"]
# the plain device copy bench.py measures beside the op (not part of the op's ABI)
LIB_BW = os.path.join(PKG, "libds4hc_bw.so")
SOURCES_BW = ["bw_copy.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def source_paths():
    return [os.path.join(CSRC, s) for s in SOURCES]


def _stale(obj: str) -> bool:
    if not os.path.exists(obj):
        return True
    deps = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(INCLUDE, "ds4hc.h")]
    return any(os.path.getmtime(p) > os.path.getmtime(obj) for p in deps)


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source and link the shared libraries (the op's and the copy
    bench.py measures beside it). Returns the op library's path.
    With incremental=True, objects newer than every source and header are reused."""
    _link(SOURCES_BW, LIB_BW, verbose, incremental)
    return _link(SOURCES, LIB, verbose, incremental)


def _link(sources, lib, verbose, incremental):
    objs = []
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    for src in [os.path.join(CSRC, s) for s in sources]:
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        objs.append(obj)
        if incremental and not _stale(obj):
            continue
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc()] + HIPCC_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c"] + lang + [src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv))
