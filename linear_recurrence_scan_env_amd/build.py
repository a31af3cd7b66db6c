"""Build liblrs.so (the gfx950 HIP kernels + C ABI) in place with hipcc.

    python -m linear_recurrence_scan_env_amd.build [--resource-usage]

Flags: gfx950 only; packed-fp32 instruction selection disabled; -O3; no
fast-math (the kernels rely on IEEE fma/min semantics).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "lrs.hip")
DEPS = [SRC, os.path.join(PKG, "csrc", "scan_core.hpp"), os.path.join(PKG, "csrc", "estimators.hpp"),
        os.path.join(ROOT, "include", "lrs.h")]
LIB = os.path.join(PKG, "liblrs.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liblrs.so)")


def flags(resource_usage: bool = False):
    f = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument",
         "-I", os.path.join(ROOT, "include")]
    if resource_usage:
        f += ["-Rpass-analysis=kernel-resource-usage"]
    return f


def build(resource_usage: bool = False, quiet: bool = True) -> str:
    """Always recompiles; writes liblrs.so atomically."""
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + flags(resource_usage) + [SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}) building {LIB}")
    if not quiet or resource_usage:
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(d) > t for d in DEPS)


if __name__ == "__main__":
    build(resource_usage="--resource-usage" in sys.argv, quiet=False)
    print(LIB)
