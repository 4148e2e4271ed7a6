"""A seeded random sweep of the scan (and, at T = 1, the decode step) against
the float64 oracle, through the C ABI.

The hand-picked cases in test_gpu_parity.py aim at known corners; this sweep
draws the combinations they do not list: head dims 16 to 256, one to eight
value heads per key head, fewer and more than 256 value heads (the two
block-form kernels), token counts on and around the 16-token block edges and
longer ragged ones, every operand dtype with the gates in the operand dtype or
in f32, both layouts, gated and raw output, every form of the time loop and
both product modes, and gates from strong to slow decay with low and high
beta.  Bars as everywhere: |gpu - ref| <= tol * (1 + |ref|) on y and the
final state, tol = 1e-4 for f32 operands and 3e-3 for 16-bit ones.  Sizes are
bounded so that the oracle runs each case in about a second.
"""
import math
import sys

import numpy as np
import pytest
import torch

from linear_attention_recurrence_recurrent_amd import recurrent_step, scan, synth
from oracle import gdn_oracle as orc

TOL = {"f32": 1e-4, "f16": 3e-3, "bf16": 3e-3}
DEV = "cuda:0"
N_CASES = 256


def _draw_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        D = int(rng.choice([16, 32, 64, 128, 256], p=[0.1, 0.2, 0.2, 0.35, 0.15]))
        G = int(rng.choice([1, 2, 3, 4, 8]))
        many = D <= 128 and rng.random() < 0.25
        if many:  # at least 256 value heads: the whole-head block kernel
            Hk = int(rng.choice([8, 16, 32])) // G or 1
            Hv = Hk * G
            B = math.ceil(256 / Hv) + int(rng.integers(0, 2))
            T = int(rng.choice([1, 2, 15, 16, 17, 33, int(rng.integers(34, 64))]))
        else:
            Hk = int(rng.integers(1, 4))
            Hv = Hk * G
            B = int(rng.integers(1, 4))
            t_max = 200 if D == 256 else 700
            T = int(rng.choice([1, 2, 15, 16, 17, 31, 32, 33, 48, 49]
                               + [int(x) for x in rng.integers(50, t_max, 3)]))
        dtype = str(rng.choice(["f32", "bf16", "f16"]))
        gate_dtype = "f32" if rng.random() < 0.3 else None
        forms = [None, "per_token"] + (["block"] if D >= 32 else [])
        form = forms[int(rng.integers(0, len(forms)))]
        exact = dtype != "f32" and form != "per_token" and bool(rng.random() < 0.4)
        cases.append(dict(
            B=B, T=T, Hk=Hk, Hv=Hv, D=D, dtype=dtype, gate_dtype=gate_dtype,
            head_major=bool(rng.random() < 0.5), gated=bool(rng.random() < 0.6),
            form=form, exact=exact,
            decay_scale=float(rng.choice([1.0, 0.01, 5.0])),
            beta_mean=float(rng.choice([0.0, 2.0, -2.0])),
            s0_std=float(rng.choice([0.02, 0.5, 0.0])),
            seed=1000 + i))
    return cases


CASES = _draw_cases(N_CASES, 20261202)


def _id(c):
    return "B%dT%dHk%dHv%dD%d-%s%s-%s-%s-%s%s" % (
        c["B"], c["T"], c["Hk"], c["Hv"], c["D"], c["dtype"],
        "/f32gates" if c["gate_dtype"] else "", "hm" if c["head_major"] else "tm",
        "gated" if c["gated"] else "raw", c["form"] or "default", "-exact" if c["exact"] else "")


def test_sweep_reaches_every_kind():
    """The drawn cases cover what the sweep claims (on the CPU: the draw alone)."""
    kinds = {(c["D"], c["dtype"]) for c in CASES}
    assert {c["D"] for c in CASES} == {16, 32, 64, 128, 256}
    assert {d for _, d in kinds} == {"f32", "bf16", "f16"}
    assert any(c["B"] * c["Hv"] >= 256 for c in CASES)
    assert any(c["Hv"] // c["Hk"] == 8 for c in CASES)
    assert any(c["T"] == 1 for c in CASES) and any(c["T"] > 48 for c in CASES)
    assert {c["form"] for c in CASES} == {None, "per_token", "block"}
    assert any(c["exact"] for c in CASES) and any(c["head_major"] for c in CASES)
    assert any(c["gate_dtype"] for c in CASES) and any(not c["gated"] for c in CASES)


def _close(got, ref, tol, what):
    got = got.detach().double().cpu().numpy()
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    err = np.abs(got - ref) / (1.0 + np.abs(ref))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, "%s: max |gpu-ref|/(1+|ref|) = %.3e > %.1e at %s" % (
        what, worst, tol, np.unravel_index(int(err.argmax()), err.shape))


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=_id)
def test_sweep_case(case):
    c = case
    print("sweep %s" % _id(c), flush=True)
    sys.stdout.flush()
    ops = synth.random_operands(c["B"], c["T"], c["Hk"], c["Hv"], c["D"], c["D"],
                                dtype=c["dtype"], gate_dtype=c["gate_dtype"],
                                head_major=c["head_major"], seed=c["seed"],
                                decay_scale=c["decay_scale"], beta_mean=c["beta_mean"],
                                s0_std=c["s0_std"])
    d = {n: t.to(DEV) for n, t in ops.items()}
    z, w = (d["z"], d["w"]) if c["gated"] else (None, None)
    y, s = scan(d["q"], d["k"], d["v"], d["log_decay"], d["beta"], d["s0"], z, w,
                head_major=c["head_major"], form=c["form"], exact=c["exact"])
    torch.cuda.synchronize()
    yr, sr = orc.scan(ops["q"], ops["k"], ops["v"], ops["log_decay"], ops["beta"], ops["s0"],
                      ops["z"] if c["gated"] else None, ops["w"] if c["gated"] else None,
                      head_major=c["head_major"])
    tol = TOL[c["dtype"]]
    assert y.dtype == torch.float32 and s.dtype == torch.float32
    _close(y, yr, tol, "y")
    _close(s, sr, tol, "final_state")
    if c["T"] == 1:  # the decode step on the same token
        y1, s1 = recurrent_step(d["q"], d["k"], d["v"], d["log_decay"], d["beta"], d["s0"], z, w,
                                head_major=c["head_major"])
        torch.cuda.synchronize()
        _close(y1, yr, tol, "step y")
        _close(s1, sr, tol, "step final_state")
