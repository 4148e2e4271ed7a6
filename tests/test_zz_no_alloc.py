"""gdn_scan_noalloc (static device scratch, no allocation) through the C ABI,
checked against gdn_scan with a caller-owned workspace.

Two calls in a row share the GPU's static scratch: the first on the prefill
workload (B=1 T=4096 Hk=16 Hv=32 bf16, whose records fill exactly half of the
64 MiB), the second on a smaller input, so a stale or misplaced record from
the first call would show in the second.  Then a 256-head shape (the other
block-form kernel, norm fused), the raw output, the one-token and empty
cases, and the rejection of a shape whose records exceed the scratch.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

from linear_attention_recurrence_recurrent_amd import (_desc, _native, scan, scan_noalloc,
                                                       scan_workspace_bytes, synth)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"f32": 1e-4, "f16": 3e-3, "bf16": 3e-3}
DT = {"f32": 0, "f16": 1, "bf16": 2}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _noalloc(ops, B, T, Hk, Hv, dtype, head_major, gated):
    """One gdn_scan_noalloc call on the current stream; returns (status, y, s_out)."""
    desc = _desc(B, T, Hk, Hv, 128, 128, head_major, DT[dtype], DT[dtype], True, True, 1e-6,
                 1e-6)
    y = torch.full(ops["v"].shape, float("nan"), dtype=torch.float32, device=DEV)
    s_out = torch.full_like(ops["s0"], float("nan"))
    vp = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    z, w = (ops["z"], ops["w"]) if gated else (None, None)
    rc = _native.lib().gdn_scan_noalloc(
        ctypes.byref(desc), vp(ops["q"]), vp(ops["k"]), vp(ops["v"]), vp(ops["log_decay"]),
        vp(ops["beta"]), vp(ops["s0"]), vp(z), vp(w), vp(y), vp(s_out),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return rc, y, s_out


def _compare(case, gated=True):
    B, T, Hk, Hv, dtype, hm = case
    say("noalloc vs gdn_scan: %s gated=%s" % (case, gated))
    ops = {n: t.to(DEV) for n, t in synth.random_operands(
        B, T, Hk, Hv, 128, 128, dtype=dtype, head_major=hm, seed=B * 1000 + T).items()}
    rc, y, s = _noalloc(ops, B, T, Hk, Hv, dtype, hm, gated)
    assert rc == 0, _native.last_error()
    z, w = (ops["z"], ops["w"]) if gated else (None, None)
    yr, sr = scan(ops["q"], ops["k"], ops["v"], ops["log_decay"], ops["beta"], ops["s0"], z, w,
                  head_major=hm)
    torch.cuda.synchronize()
    for got, ref, what in ((y, yr, "y"), (s, sr, "final state")):
        g, r = got.double().cpu().numpy(), ref.double().cpu().numpy()
        assert np.all(np.isfinite(g)), what + ": not every output was written"
        err = float((np.abs(g - r) / (1 + np.abs(r))).max())
        assert err <= TOL[dtype], "%s: %.3e" % (what, err)
        assert torch.equal(got, ref), what + ": the same kernels should give the same bits"


def test_noalloc_two_calls_second_smaller():
    desc = _desc(1, 4096, 16, 32, 128, 128, False, 2, 2, True, True, 1e-6, 1e-6)
    assert scan_workspace_bytes(desc) == 32 << 20  # half of the static scratch
    _compare((1, 4096, 16, 32, "bf16", False))   # the prefill workload, few-head kernel
    _compare((1, 100, 2, 4, "f16", True))        # smaller, right after, other layout


def test_noalloc_many_heads_raw_and_trivial_lengths():
    _compare((8, 45, 16, 32, "bf16", True))               # 256 heads: whole-head kernel
    _compare((2, 37, 2, 6, "f32", False), gated=False)    # raw o
    _compare((3, 1, 2, 4, "bf16", False))                 # one token: the decode kernel
    B, T, Hk, Hv = 2, 0, 2, 4                             # empty time axis: s_out = s0
    ops = {n: t.to(DEV) for n, t in synth.random_operands(B, T, Hk, Hv, 128, 128,
                                                          dtype="bf16", seed=3).items()}
    rc, _, s = _noalloc(ops, B, T, Hk, Hv, "bf16", False, True)
    torch.cuda.synchronize()
    assert rc == 0 and torch.equal(s, ops["s0"])
    # the Python binding of the same entry point
    ops = {n: t.to(DEV) for n, t in synth.random_operands(1, 70, 2, 4, 128, 128, dtype="bf16",
                                                          seed=5).items()}
    a = (ops["q"], ops["k"], ops["v"], ops["log_decay"], ops["beta"], ops["s0"], ops["z"],
         ops["w"])
    y0, s0 = scan(*a)
    y1, s1 = scan_noalloc(*a)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(s0, s1)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    """The head-major workload (B=16 T=1024 Hv=32) needs 80 MiB of records: rejected
    with a reason before anything is enqueued (the outputs keep their NaN fill)."""
    B, T, Hk, Hv = 16, 1024, 16, 32
    desc = _desc(B, T, Hk, Hv, 128, 128, True, 1, 1, True, True, 1e-6, 1e-6)
    assert scan_workspace_bytes(desc) > _native.GDN_NOALLOC_SCRATCH_BYTES
    ops = {n: t.to(DEV) for n, t in synth.random_operands(B, T, Hk, Hv, 128, 128, dtype="f16",
                                                          head_major=True, seed=4).items()}
    rc, y, s = _noalloc(ops, B, T, Hk, Hv, "f16", True, True)
    torch.cuda.synchronize()
    assert rc == 9 and "static" in _native.last_error()
    assert torch.isnan(y).all() and torch.isnan(s).all()
