"""Buffers past 2^31 elements on the GPU, through the C ABI.

The kernels address operands, outputs, records and the state with 64-bit
offsets; 32-bit ones appear only inside a 16-token block, where the descriptor
check bounds them.  Each case here puts heads or tokens past element 2^31 of a
buffer and compares them elementwise with the float64 oracle at the 3e-3 bar,
gated and with the raw o:
  - the decode step and a 20-token scan (both forms; the block form's kernel
    with a workgroup per head) with B = 4100, Hk 16, Hv 32, D 128: the state has
    2^31 + 2^21 elements.  Heads are independent through the recurrence ("Module
    gdn" page, module description: one memory per value head), so the oracle
    computes the first head, the heads around element 2^31 and the last ones;
  - the few-head scan (B = 1, Hk 16, Hv 32, D 128, the block form's kernel with
    a workgroup per 16 state rows, and the per-token form) over T = 524,328
    tokens, whose v, z and y have 2^31 + 163,840 elements, in both layouts.  A
    token with alpha = 0 forty tokens from the end sets S = beta v k^T whatever
    came before, so the oracle runs the last forty tokens alone and the GPU's
    outputs there, and its final state, must match.
Inputs are drawn on the GPU by torch's seeded generator with the workloads'
recipe (q, k, v, z ~ N(0, 1) in bf16, log_decay = -softplus(N(0, 1)),
beta = sigmoid(N(0, 1)), s0 ~ N(0, 0.02) in f32, w = 1 + 0.1 N(0, 1)); the
oracle reads the same bytes back.
"""
import sys

import numpy as np
import pytest
import torch

from linear_attention_recurrence_recurrent_amd import recurrent_step, scan
from oracle import gdn_oracle as orc

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 3e-3
BIG = 1 << 31
HK, HV, D = 16, 32, 128
G = HV // HK


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _operands(q_shape, v_shape, g_shape, s_shape, seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)

    def normal(shape, dtype, scale=1.0, shift=0.0):
        x = torch.randn(shape, generator=gen, device=DEV, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        if shift != 0.0:
            x.add_(shift)
        return x if dtype == torch.float32 else x.to(dtype)

    bf = torch.bfloat16
    ops = dict(q=normal(q_shape, bf), k=normal(q_shape, bf), v=normal(v_shape, bf),
               z=normal(v_shape, bf))
    ops["log_decay"] = torch.nn.functional.softplus(normal(g_shape, torch.float32)).neg_().to(bf)
    ops["beta"] = torch.sigmoid(normal(g_shape, torch.float32)).to(bf)
    ops["s0"] = normal(s_shape, torch.float32, scale=0.02)
    ops["w"] = normal((D,), bf, scale=0.1, shift=1.0)
    return ops


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def _close(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref) / (1.0 + np.abs(ref))
    assert np.all(np.isfinite(got)), what + ": non-finite"
    worst = float(err.max())
    assert worst <= TOL, "%s: max rel err %.3e at %s" % (
        what, worst, np.unravel_index(int(err.argmax()), err.shape))


# ------------------------------------------------------------------ many heads, state > 2^31
B_MANY = 4100  # B * Hv * D * D = 2^31 + 2^21
# heads (b * Hv + hv): the first, the three around element 2^31, the last
HEADS = [0, BIG // (D * D) - 1, BIG // (D * D), BIG // (D * D) + 1, B_MANY * HV - 1]


def _head_oracle(ops, h, gated, T):
    """The oracle on value head h = (b, hv) alone (token-major operands)."""
    b, hv = divmod(h, HV)
    hk = hv // G
    sub = dict(q=ops["q"][b:b + 1, :, hk:hk + 1], k=ops["k"][b:b + 1, :, hk:hk + 1],
               v=ops["v"][b:b + 1, :, hv:hv + 1], z=ops["z"][b:b + 1, :, hv:hv + 1],
               log_decay=ops["log_decay"][b:b + 1, :, hv:hv + 1],
               beta=ops["beta"][b:b + 1, :, hv:hv + 1], s0=ops["s0"][b:b + 1, hv:hv + 1])
    sub = {n: _host(t) for n, t in sub.items()}
    assert sub["q"].shape == (1, T, 1, D)
    return orc.scan(sub["q"], sub["k"], sub["v"], sub["log_decay"], sub["beta"], sub["s0"],
                    sub["z"] if gated else None, _host(ops["w"]) if gated else None)


@pytest.fixture(scope="module")
def many_heads():
    say("large: drawing B=%d T=20 operands, state %d elements" % (B_MANY, B_MANY * HV * D * D))
    ops = _operands((B_MANY, 20, HK, D), (B_MANY, 20, HV, D), (B_MANY, 20, HV),
                    (B_MANY, HV, D, D), seed=31)
    yield ops
    del ops
    torch.cuda.empty_cache()


@pytest.mark.parametrize("gated", [True, False])
def test_decode_state_past_2_31_elements(many_heads, gated):
    ops = {n: (t[:, :1].contiguous() if n in ("q", "k", "v", "z", "log_decay", "beta") else t)
           for n, t in many_heads.items()}
    say("large: decode step B=%d, state past 2^31 elements, gated=%s" % (B_MANY, gated))
    y, s = recurrent_step(ops["q"], ops["k"], ops["v"], ops["log_decay"], ops["beta"], ops["s0"],
                          ops["z"] if gated else None, ops["w"] if gated else None)
    torch.cuda.synchronize()
    for h in HEADS:
        b, hv = divmod(h, HV)
        yr, sr = _head_oracle(ops, h, gated, T=1)
        _close(_host(y[b:b + 1, :, hv:hv + 1]), yr, "decode y, head %d" % h)
        _close(_host(s[b:b + 1, hv:hv + 1]), sr, "decode state, head %d" % h)
    del y, s
    torch.cuda.empty_cache()


@pytest.mark.parametrize("gated", [True, False])
@pytest.mark.parametrize("form", [None, "per_token"], ids=["block", "per_token"])
def test_scan_state_past_2_31_elements(many_heads, form, gated):
    ops = many_heads
    say("large: scan B=%d T=20, state past 2^31 elements, form %s, gated=%s" % (
        B_MANY, form, gated))
    y, s = scan(ops["q"], ops["k"], ops["v"], ops["log_decay"], ops["beta"], ops["s0"],
                ops["z"] if gated else None, ops["w"] if gated else None, form=form)
    torch.cuda.synchronize()
    for h in HEADS:
        b, hv = divmod(h, HV)
        yr, sr = _head_oracle(ops, h, gated, T=20)
        _close(_host(y[b:b + 1, :, hv:hv + 1]), yr, "scan y, head %d" % h)
        _close(_host(s[b:b + 1, hv:hv + 1]), sr, "scan state, head %d" % h)
    del y, s
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ few heads, y > 2^31
T_LONG = BIG // (HV * D) + 40  # 524,328 tokens: v, z, y have 2^31 + 163,840 elements
TAIL = 40


@pytest.mark.parametrize("head_major", [False, True], ids=["token_major", "head_major"])
def test_long_scan_outputs_past_2_31_elements(head_major):
    j = T_LONG - TAIL
    if head_major:
        shapes = ((1, HK, T_LONG, D), (1, HV, T_LONG, D), (1, HV, T_LONG))
    else:
        shapes = ((1, T_LONG, HK, D), (1, T_LONG, HV, D), (1, T_LONG, HV))
    say("large: few-head scan T=%d (%s), outputs past 2^31 elements" % (
        T_LONG, "head-major" if head_major else "token-major"))
    ops = _operands(*shapes, (1, HV, D, D), seed=41 + int(head_major))
    tdim = 2 if head_major else 1
    ops["log_decay"].select(tdim, j).fill_(float("-inf"))  # alpha = 0: S = beta v k^T
    tail = {n: _host(ops[n].narrow(tdim, j, TAIL)) for n in ("q", "k", "v", "z")}
    tail.update({n: _host(ops[n].narrow(tdim, j, TAIL)) for n in ("log_decay", "beta")})
    w = _host(ops["w"])
    zero = np.zeros((1, HV, D, D))  # any s0: alpha = 0 at the tail's first token
    want = {g: orc.scan(tail["q"], tail["k"], tail["v"], tail["log_decay"], tail["beta"], zero,
                        tail["z"] if g else None, w if g else None, head_major=head_major)
            for g in (True, False)}
    for form in (None, "per_token"):
        for gated in (True, False):
            say("large: T=%d form %s gated=%s" % (T_LONG, form, gated))
            y, s = scan(ops["q"], ops["k"], ops["v"], ops["log_decay"], ops["beta"], ops["s0"],
                        ops["z"] if gated else None, ops["w"] if gated else None,
                        head_major=head_major, form=form)
            torch.cuda.synchronize()
            assert y.numel() > BIG
            yr, sr = want[gated]
            _close(_host(y.narrow(tdim, j, TAIL)), yr, "y over the last %d tokens" % TAIL)
            _close(_host(s), sr, "final state")
            del y, s
            torch.cuda.empty_cache()
    del ops
    torch.cuda.empty_cache()
