"""Build libgdn_hip.so (HIP kernels + C ABI) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgdn_hip.so")
SOURCES = [os.path.join(CSRC, f) for f in ("gdn_kernels.hip", "gdn_check.cpp")]
HEADERS = [os.path.join(CSRC, "gdn_internal.h"), os.path.join(INCLUDE, "gdn.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed FP32 instructions are kept out of the device code on purpose.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def command(out: str = LIB, extra=()):
    return ([HIPCC, "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Wall", "-I", INCLUDE, "-I", CSRC] + DEVICE_FLAGS + list(extra)
            + ["-o", out] + SOURCES)


def build(verbose: bool = False) -> str:
    """Compile every source into the package directory (always recompiles)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
