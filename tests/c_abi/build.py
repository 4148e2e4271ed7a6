"""Build tests/c_abi/libgdn_demo.so, the C++ caller of libgdn_hip.so's C ABI
that tests/test_gpu_c_abi.py loads and runs.  Linked against the in-tree
library (built first) with an rpath relative to itself, so it loads from any
copy of the tree.  Called by __graft_entry__.build(); the GPU test only runs
it."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "linear_attention_recurrence_recurrent_amd")
SRC = os.path.join(HERE, "gdn_demo.cpp")
LIB = os.path.join(HERE, "libgdn_demo.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-Wall", "-shared", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), SRC, "-o", tmp,
           "-L", PKG, "-lgdn_hip",
           "-Wl,-rpath,$ORIGIN/../../linear_attention_recurrence_recurrent_amd"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
