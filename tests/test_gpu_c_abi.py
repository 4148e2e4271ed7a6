"""The C ABI from C++ code that uses no Python and no torch.

tests/c_abi/gdn_demo.cpp (built into tests/c_abi/libgdn_demo.so by
__graft_entry__.build(), and called here through its one C entry point in this
process) owns its buffers
(hipMalloc), sizes and passes the block form's workspace, runs a gated scan
(B=2 T=37 Hk=2 Hv=4 D=64, bf16: the few-head block kernel and its separate
norm) on a stream it created, then one decode step that updates the scan's
final state in place, and checks that a bad descriptor is refused.  It writes
the bytes it used and what it got; here the float64 oracle runs on those bytes:
the scan's y and state, the step against the oracle from the program's own
scan state, and scan plus step against the oracle's T+1-token scan.  Bar:
3e-3 * (1 + |ref|), the tolerance for 16-bit operands.
"""
import ctypes
import os

import numpy as np
import pytest

from oracle import gdn_oracle as orc

pytestmark = pytest.mark.gpu

DEMO = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "libgdn_demo.so")
TOL = 3e-3


def _close(got, ref, what):
    err = np.abs(got - ref) / (1.0 + np.abs(ref))
    assert np.all(np.isfinite(got)), what + ": non-finite"
    assert float(err.max()) <= TOL, "%s: max rel err %.3e" % (what, float(err.max()))


class _Reader:
    def __init__(self, buf):
        self.buf, self.off = buf, 0

    def take(self, shape, dtype):
        n = int(np.prod(shape))
        a = np.frombuffer(self.buf, dtype=dtype, count=n, offset=self.off).reshape(shape)
        self.off += n * np.dtype(dtype).itemsize
        if dtype == np.uint16:  # bfloat16 bytes -> float64, exactly
            return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return a.astype(np.float64)


def test_c_program_scan_and_step_match_the_oracle(tmp_path):
    assert os.path.exists(DEMO), "tests/c_abi/libgdn_demo.so is not built (__graft_entry__.build())"
    out = tmp_path / "demo.bin"
    print("c_abi: running gdn_demo_run from %s" % DEMO, flush=True)
    run = ctypes.CDLL(DEMO).gdn_demo_run
    run.restype, run.argtypes = ctypes.c_int, [ctypes.c_char_p]
    assert run(str(out).encode()) == 0, "gdn_demo_run failed (its reason is on stderr)"
    rd = _Reader(out.read_bytes())
    B, T, Hk, Hv, D = (int(x) for x in rd.take((5,), np.int64))
    u16, f32 = np.uint16, np.float32
    q, k = rd.take((B, T, Hk, D), u16), rd.take((B, T, Hk, D), u16)
    v, z = rd.take((B, T, Hv, D), u16), rd.take((B, T, Hv, D), u16)
    g, be = rd.take((B, T, Hv), u16), rd.take((B, T, Hv), u16)
    w, s0 = rd.take((D,), u16), rd.take((B, Hv, D, D), f32)
    q1, k1 = rd.take((B, 1, Hk, D), u16), rd.take((B, 1, Hk, D), u16)
    v1, z1 = rd.take((B, 1, Hv, D), u16), rd.take((B, 1, Hv, D), u16)
    g1, be1 = rd.take((B, 1, Hv), u16), rd.take((B, 1, Hv), u16)
    y, s_scan = rd.take((B, T, Hv, D), f32), rd.take((B, Hv, D, D), f32)
    y1, s_step = rd.take((B, 1, Hv, D), f32), rd.take((B, Hv, D, D), f32)
    assert rd.off == len(rd.buf)

    yr, sr = orc.scan(q, k, v, g, be, s0, z, w)
    _close(y, yr, "scan y")
    _close(s_scan, sr, "scan state")
    y1r, s1r = orc.step(q1, k1, v1, g1, be1, s_scan, z1, w)  # from the program's own state
    _close(y1, y1r, "step y")
    _close(s_step, s1r, "step state")
    cat = lambda a, b: np.concatenate([a, b], axis=1)  # noqa: E731
    ya, sa = orc.scan(cat(q, q1), cat(k, k1), cat(v, v1), cat(g, g1), cat(be, be1), s0,
                      cat(z, z1), w)
    _close(np.concatenate([y, y1], axis=1), ya, "scan and step against a T+1 scan")
    _close(s_step, sa, "state after scan and step")
