"""Build libmlaq.so (the HIP kernels and the C ABI) in-tree for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmlaq.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("api.cpp", "decode.hip", "quant.hip", "extend.hip", "extend_attn.hip", "probe.hip")]
HEADERS = [os.path.join(HERE, "csrc", f) for f in ("device_common.h", "mlaq_kernels.h")] + \
    [os.path.join(ROOT, "include", "mlaq.h")]


def hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the mlaq library needs ROCm's hipcc to build")


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 into libmlaq.so next to this file (always rebuilds)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-o", tmp] + SOURCES
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
