"""The streaming and clock reference kernels (include/gdn_calib.h) on the GPU: every
variant's copy is exact and its in-place update is buf * 1.0000001 + 1e-7 to
within one float32 rounding (the kernels fuse the multiply-add), on a size
that leaves a ragged last workgroup, and nothing outside the buffer is
touched.  These kernels set the streaming ceiling bench.py reports beside the
decode, so a lost or misplaced store would inflate it."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from linear_attention_recurrence_recurrent_amd import _native

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N4 = 1024 * 16 * 3 + 37  # 16-byte vectors: three of the largest chunks and a ragged tail
PAD = 64                 # guard floats on each side


def _call(op, v, src, dst, nbytes):
    rc = _native.lib().gdn_calib_stream(op, v, ctypes.c_void_p(src), ctypes.c_void_p(dst), nbytes,
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, _native.last_error()


@pytest.mark.parametrize("variant", range(_native.GDN_CALIB_VARIANTS))
def test_stream_variant_results(variant):
    name = _native.lib().gdn_calib_variant_name(variant).decode()
    print("calib variant %d: %s" % (variant, name), flush=True)
    sys.stdout.flush()
    g = torch.Generator(device=DEV)
    g.manual_seed(variant)
    n = 4 * N4
    a = torch.empty(n + 2 * PAD, dtype=torch.float32, device=DEV)
    a.copy_(torch.randn(n + 2 * PAD, generator=g, device=DEV))
    b = torch.full((n + 2 * PAD,), -7.0, dtype=torch.float32, device=DEV)
    x0 = a.cpu().numpy()
    # copy
    _call(_native.GDN_CALIB_COPY, variant, a.data_ptr() + 4 * PAD, b.data_ptr() + 4 * PAD, 16 * N4)
    # in place
    _call(_native.GDN_CALIB_RMW, variant, a.data_ptr() + 4 * PAD, a.data_ptr() + 4 * PAD, 16 * N4)
    torch.cuda.synchronize()
    got_b, got_a = b.cpu().numpy(), a.cpu().numpy()
    assert np.array_equal(got_b[PAD:PAD + n], x0[PAD:PAD + n]), "copy"
    assert np.all(got_b[:PAD] == -7.0) and np.all(got_b[PAD + n:] == -7.0), "copy wrote outside"
    assert np.array_equal(got_a[:PAD], x0[:PAD]) and np.array_equal(got_a[PAD + n:], x0[PAD + n:])
    want = (x0[PAD:PAD + n].astype(np.float64) * np.float64(np.float32(1.0000001))
            + np.float64(np.float32(1e-7)))
    ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got_a[PAD:PAD + n] - want) <= ulp), "in-place update"


@pytest.mark.parametrize("waves,iters", [(4, 1000), (1024, 20000), (8192, 2000)])
def test_clock_reference(waves, iters):
    """The clock reference writes four words per wave and nothing past them:
    positive shader cycles and real-time ticks whose ratio is a plausible
    shader clock (0.3 to 3 GHz against the constant 100 MHz counter), the
    chains' float sum (finite), and a zero; the ticks match the HIP events'
    duration of the launch at 100 MHz."""
    print("clock reference: %d waves x %d rounds" % (waves, iters), flush=True)
    L = _native.lib()
    stream = torch.cuda.current_stream()
    out = torch.full((4 * waves + 8,), -7, dtype=torch.int64, device="cuda:0")
    for _ in range(3):  # clocks up first
        assert L.gdn_calib_clock(waves, iters, ctypes.c_void_p(out.data_ptr()),
                                 ctypes.c_void_p(stream.cuda_stream)) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    assert L.gdn_calib_clock(waves, iters, ctypes.c_void_p(out.data_ptr()),
                             ctypes.c_void_p(stream.cuda_stream)) == 0
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3
    o = out.cpu().numpy()
    assert np.all(o[4 * waves:] == -7)
    w = o[:4 * waves].reshape(waves, 4)
    assert np.all(w[:, 0] > 0) and np.all(w[:, 1] > 0) and np.all(w[:, 3] == 0)
    sums = w[:, 2].astype(np.uint32).view(np.float32)
    assert np.all(np.isfinite(sums))
    ghz = w[:, 0].sum() / w[:, 1].sum() * 0.1
    assert 0.3 < ghz < 3.0, ghz
    if iters * waves >= 1 << 24:  # long enough for the launch overhead not to matter
        mhz = w[:, 1].max() / us
        assert 70 < mhz < 130, (mhz, us)
