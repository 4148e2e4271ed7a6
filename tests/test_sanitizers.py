"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host C/C++ code (CPU only).

The float64 oracle (oracle/gdn_oracle.c) and the C ABI's validation
(csrc/gdn_check.cpp) are built with -fsanitize=address,undefined (any report
aborts the run) together with a small driver each (tests/sanitize/).  The
oracle driver runs every oracle entry point, including the threaded scan,
on operands written by this test, and its outputs must equal the ordinary
build's; the validation driver runs accepted and rejected arguments through
gdn_check, gdn_scan_workspace_size and the gate and conv checks.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import gdn_oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-static-libasan", "-g"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:strict_string_checks=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="needs gcc and g++")


@pytest.fixture(scope="module")
def oracle_exe(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("san") / "oracle_driver")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off"] + SAN + [
        "-o", exe, os.path.join(ROOT, "oracle", "gdn_oracle.c"),
        os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm", "-lpthread"])
    return exe


def _run(exe, args, arrays, tmp_path, n_out):
    fin, fout = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    with open(fin, "wb") as f:
        for a in arrays:
            np.ascontiguousarray(a, dtype=np.float64).tofile(f)
    r = subprocess.run([exe] + [str(a) for a in args] + [fin, fout], env=ENV,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    out = np.fromfile(fout, dtype=np.float64)
    assert out.size == n_out
    return out


@pytest.mark.parametrize("shape", [
    # (B, T, Hk, Hv, Dk, Dv, flags, gated, threads)
    (2, 9, 2, 6, 16, 16, 3, True, 3),
    (1, 5, 1, 2, 8, 12, 1, False, 1),     # Dv != Dk, no q scale
    (3, 0, 2, 2, 16, 16, 3, True, 2),     # empty time axis
    (0, 4, 1, 1, 16, 16, 3, False, 4),    # empty batch
    (1, 6, 2, 4, 32, 32, 0, True, 8),     # no folds, more threads than heads
])
def test_oracle_scan_under_sanitizers(oracle_exe, tmp_path, shape):
    B, T, Hk, Hv, Dk, Dv, flags, gated, threads = shape
    r = np.random.default_rng(B * 100 + T)
    q = r.standard_normal((B, T, Hk, Dk))
    k = r.standard_normal((B, T, Hk, Dk))
    if not flags & 1:
        q /= np.linalg.norm(q, axis=-1, keepdims=True) + 1e-300
        k /= np.linalg.norm(k, axis=-1, keepdims=True) + 1e-300
    v = r.standard_normal((B, T, Hv, Dv))
    g = -np.logaddexp(0, r.standard_normal((B, T, Hv)))
    be = 1 / (1 + np.exp(-r.standard_normal((B, T, Hv))))
    s0 = 0.1 * r.standard_normal((B, Hv, Dv, Dk))
    z = r.standard_normal((B, T, Hv, Dv)) if gated else None
    w = 1 + 0.1 * r.standard_normal(Dv) if gated else None
    arrays = [q, k, v, g, be, s0] + ([z, w] if gated else [])
    ny, ns = B * T * Hv * Dv, B * Hv * Dv * Dk
    out = _run(oracle_exe, ["scan", B, T, Hk, Hv, Dk, Dv, flags, int(gated), threads], arrays,
               tmp_path, ny + ns)
    yr, sr = orc.scan(q, k, v, g, be, s0, z, w, fold_qk_l2norm=bool(flags & 1),
                      fold_q_scale=bool(flags & 2))
    np.testing.assert_allclose(out[:ny].reshape(yr.shape), yr, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(out[ny:].reshape(sr.shape), sr, rtol=1e-13, atol=1e-13)


def test_oracle_producers_and_norms_under_sanitizers(oracle_exe, tmp_path):
    r = np.random.default_rng(7)
    n = 1001
    a = np.concatenate([r.standard_normal(n - 3) * 4, [0.0, 700.0, -700.0]])
    b = np.concatenate([r.standard_normal(n - 3) * 4, [0.0, 800.0, -800.0]])
    out = _run(oracle_exe, ["gates", n, 0.25], [a, b], tmp_path, 2 * n)
    ld, bt = orc.gates(a, b, decay_scale=0.25)
    np.testing.assert_array_equal(out[:n], ld)
    np.testing.assert_array_equal(out[n:], bt)
    for (B, T, C, W, bias, state) in ((2, 7, 5, 4, True, True), (1, 2, 3, 4, False, True),
                                      (2, 0, 4, 3, True, True), (1, 5, 6, 1, False, False)):
        x = r.standard_normal((B, T, C))
        wt = r.standard_normal((C, W))
        bb = r.standard_normal(C) if bias else None
        st = r.standard_normal((B, C, W - 1)) if state else None
        arrays = [x, wt] + ([bb] if bias else []) + ([st] if state else [])
        ny, nst = B * T * C, B * C * (W - 1)
        out = _run(oracle_exe, ["conv", B, T, C, W, 1, int(bias), int(state)], arrays, tmp_path,
                   ny + nst)
        yr, sr = orc.conv_silu(x, wt, bb, st)
        np.testing.assert_array_equal(out[:ny].reshape(yr.shape), yr)
        np.testing.assert_array_equal(out[ny:].reshape(sr.shape), sr)
    rows, n = 6, 24
    x, z, w = r.standard_normal((rows, n)), r.standard_normal((rows, n)), r.standard_normal(n)
    out = _run(oracle_exe, ["norms", rows, n], [x, z, w], tmp_path, 2 * rows * n)
    np.testing.assert_array_equal(out[:rows * n].reshape(rows, n), orc.l2norm(x))
    want = np.stack([orc.gated_rmsnorm(x[i], z[i], w if i & 1 else None) for i in range(rows)])
    np.testing.assert_array_equal(out[rows * n:].reshape(rows, n), want)


def test_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "check_driver")
    csrc = os.path.join(ROOT, "linear_attention_recurrence_recurrent_amd", "csrc")
    subprocess.check_call(["g++", "-O1", "-std=c++17"] + SAN + [
        "-I", os.path.join(ROOT, "include"), "-I", csrc, "-o", exe,
        os.path.join(csrc, "gdn_check.cpp"),
        os.path.join(ROOT, "tests", "sanitize", "check_driver.cpp")])
    r = subprocess.run([exe], env=ENV, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "check_driver ok" in r.stdout, r.stdout + r.stderr
