"""Build libgdn_hip.so (HIP kernels + C ABI) in-tree with hipcc for gfx950."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgdn_hip.so")
SOURCES = [os.path.join(CSRC, f) for f in
           ("gdn_decode.hip", "gdn_scan.hip", "gdn_chunk.hip", "gdn_gates.hip", "gdn_conv.hip",
            "gdn_calib.hip", "gdn_noalloc.hip", "gdn_api.cpp", "gdn_check.cpp")]
HEADERS = [os.path.join(CSRC, f) for f in ("gdn_device.h", "gdn_launch.h", "gdn_internal.h")] + [
    os.path.join(INCLUDE, "gdn.h"), os.path.join(INCLUDE, "gdn_calib.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed FP32 instructions are kept out of the device code on purpose.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE,
          "-I", CSRC]


def compile_cmd(src: str, obj: str):
    return [HIPCC] + COMMON + DEVICE_FLAGS + ["-c", src, "-o", obj]


def link_cmd(objs, out: str):
    return [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", out] + list(objs)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source (in parallel) and link into the package directory.

    Always recompiles; the previous library is replaced atomically."""
    tmpdir = tempfile.mkdtemp(prefix="gdn_build_")
    try:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in SOURCES]
        cmds = [compile_cmd(s, o) for s, o in zip(SOURCES, objs)]
        with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
            futs = []
            for c in cmds:
                if verbose:
                    print(" ".join(c), flush=True)
                futs.append(ex.submit(subprocess.run, c, capture_output=True, text=True))
            for c, f in zip(cmds, futs):
                r = f.result()
                if r.returncode != 0:
                    sys.stderr.write(r.stdout + r.stderr)
                    raise subprocess.CalledProcessError(r.returncode, c)
        tmp = LIB + ".tmp%d" % os.getpid()
        lc = link_cmd(objs, tmp)
        if verbose:
            print(" ".join(lc), flush=True)
        subprocess.check_call(lc)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
