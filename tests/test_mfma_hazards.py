"""Matrix-core dependencies in the gfx950 code hipcc emits for the library (CPU only).

On gfx950 a matrix instruction that takes the result of a matrix instruction of
another shape as an operand needs wait states between the two.  With the ROCm
7.2 compiler, a 16x16x16 bf16 product that accumulates onto the result of a
16x16x32 bf16 product issued right before it got none and read a stale
accumulator: a one-wave check of that pair gave results wrong by a factor of
about 160, and correct ones with 14 or more wait states between the two
products (or with the value passed through a vector instruction).  The kernels
are written so that no product takes a product of the other shape as its
accumulator back to back; this test compiles every HIP source to gfx950
assembly and checks, in straight-line order, that each matrix instruction
reading registers an earlier matrix instruction of another opcode wrote has at
least MIN_WAIT wait states (instructions between, an s_nop N counting N + 1)
after it: 14 for a 16x16x16 product after a 16x16x32 one (the fewest found
correct on the hardware), 12 otherwise (what the compiler itself inserts for
the other order, which the GPU parity tests cover).
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_recurrence_recurrent_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
MIN_WAIT = {("v_mfma_f32_16x16x32_bf16", "v_mfma_f32_16x16x16_bf16"): 14}
DEFAULT_WAIT = 12
WINDOW = 24

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return m.group(1), set(range(int(m.group(2)), int(m.group(3)) + 1))
    m = re.match(r"([va])(\d+)$", tok)
    if m:
        return m.group(1), {int(m.group(2))}
    return None, set()


def scan(asm):
    """(matrix instructions, [(function, instruction, earlier opcode, wait states)])"""
    found, n, fn, recent = [], 0, "?", []
    for line in asm.split("\n"):
        if re.match(r"^_Z\w+:", line):
            fn, recent = line.split(":")[0], []
            continue
        s = line.split(";")[0].strip()
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        op = s.split()[0]
        if op == "s_endpgm":
            recent = []
            continue
        m = re.match(r"s_nop\s+(\d+)", s)
        w = int(m.group(1)) + 1 if m else 1
        if op.startswith("v_mfma"):
            n += 1
            ops = [o.strip() for o in s.split(None, 1)[1].split(",")]
            dst, srcs = _regs(ops[0]), [_regs(o) for o in ops[1:4]]
            for pop, kind, pregs, dist in recent:
                if pop != op and any(k == kind and r & pregs for k, r in srcs):
                    if dist < MIN_WAIT.get((pop, op), DEFAULT_WAIT):
                        found.append((fn, s, pop, dist))
            recent = [(a, b, c, d + w) for a, b, c, d in recent if d + w < WINDOW]
            recent.append((op, dst[0], dst[1], 0))
        else:
            recent = [(a, b, c, d + w) for a, b, c, d in recent if d + w < WINDOW]
    return n, found


def test_scan_flags_a_back_to_back_mixed_pair():
    asm = """_Zk:
        v_mfma_f32_16x16x32_bf16 v[4:7], v[2:5], v[10:13], v[6:9]
        v_mfma_f32_16x16x16_bf16 v[0:3], v[2:3], v[0:1], v[4:7]
        s_endpgm
_Zk2:
        v_mfma_f32_16x16x32_bf16 v[4:7], v[2:5], v[10:13], v[6:9]
        s_nop 7
        s_nop 7
        v_mfma_f32_16x16x16_bf16 v[0:3], v[2:3], v[0:1], v[4:7]
        v_mfma_f32_16x16x16_bf16 v[8:11], v[2:3], v[0:1], v[8:11]
        s_endpgm
"""
    n, found = scan(asm)
    assert n == 5
    assert [(f, d) for f, _, _, d in found] == [("_Zk", 0)]


@pytest.mark.parametrize("src", sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")))
def test_no_mixed_shape_matrix_dependency_without_wait_states(src, tmp_path):
    out = str(tmp_path / "k.s")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17",
                        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "--cuda-device-only", "-S", "-o", out, os.path.join(CSRC, src)],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    n, found = scan(open(out).read())
    assert not found, "%d matrix instructions read another shape's result too early, e.g. %s" % (
        len(found), found[:3])
