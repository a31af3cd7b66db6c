"""Build liblrs.so (the gfx950 HIP kernels + C ABI) in place with hipcc.

    python -m linear_recurrence_scan_env_amd.build [--resource-usage]

Flags: gfx950 only; packed-fp32 instruction selection disabled; -O3; no
fast-math (the kernels rely on IEEE fma/min semantics); the compiler's
atomic optimizer off.  Every atomic here is already issued by one lane; the
optimizer would still rewrite a returning one into a wave-wide form whose
result is broadcast at once, which waits for the atomic's round trip right
after it (a block's look-back count then held back its data loads).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
# One translation unit per group of entry points, compiled in parallel.
SOURCES = [os.path.join(CSRC, f) for f in ("abi.hip", "noalloc.hip", "floor.hip")] + [
    os.path.join(CSRC, f"{group}{sfx}.hip")
    for group in ("returns", "offpolicy", "forward", "affine") for sfx in ("", "_bf16", "_f16")]
HEADERS = [os.path.join(CSRC, f)
           for f in ("launch.hpp", "scan_core.hpp", "estimators.hpp", "entries.hpp",
                     "timemajor.hpp")] + \
    [os.path.join(ROOT, "include", "lrs.h")]
DEPS = SOURCES + HEADERS
LIB = os.path.join(PKG, "liblrs.so")
OBJ_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liblrs.so)")


def flags(resource_usage: bool = False):
    f = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
         "-Wall", "-Wno-unused-command-line-argument",
         "-I", os.path.join(ROOT, "include")]
    if resource_usage:
        f += ["-Rpass-analysis=kernel-resource-usage"]
    return f


def build(resource_usage: bool = False, quiet: bool = True) -> str:
    """Always recompiles every source (in parallel), links liblrs.so atomically."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    cc = hipcc()
    jobs = max(1, min(16, os.cpu_count() or 1))
    procs, failed, pending = [], [], list(SOURCES)

    def reap(entry):
        src, obj, p = entry
        out, err = p.communicate()
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(out + err)
        elif not quiet or resource_usage:
            sys.stderr.write(err)

    running = []
    while pending or running:
        while pending and len(running) < jobs:
            src = pending.pop(0)
            obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
            cmd = [cc] + flags(resource_usage) + ["-c", src, "-o", obj]
            entry = (src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.PIPE, text=True))
            running.append(entry)
            procs.append(entry)
        reap(running.pop(0))
    if failed:
        raise RuntimeError(f"hipcc failed on {', '.join(map(os.path.basename, failed))}")
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + [o for _, o, _ in procs] + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}) linking {LIB}")
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
