"""Builds libgg.so (the HIP library behind include/gg.h) in-tree for gfx950.

``python -m moe_expert_grouped_ragged_amd._build`` or ``build()`` from Python.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgg.so")

SOURCES = ["gg_api.cpp", "gg_kernels.hip", "gg_noalloc.hip"]
HEADERS = ["gg_kernels.h"]

# Packed-fp32 VALU ops are disabled for all device code.
HIP_FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
             "-Wall", "-Werror", "-Wno-unused-command-line-argument",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wl,-z,defs"]   # every symbol resolved at link time


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, extra_flags=()) -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), *HIP_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only target feature above and
    # says so; that is expected and harmless.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
