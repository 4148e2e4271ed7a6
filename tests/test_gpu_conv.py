"""Parity of the conv + silu producer (gdn_conv_silu through the C ABI) with the
float64 oracle, element by element.  The producer's output is in the operand
dtype (it feeds the recurrence), so the bar is the final rounding plus the f32
arithmetic before it: |gpu - ref| <= u * |ref| + 1e-5 * (1 + |ref|) with u the
unit roundoff of the output dtype (2^-8 bfloat16, 2^-11 float16), and
1e-4 * (1 + |ref|) for float32.  The carried state is an exact copy of inputs,
so it must match bit for bit."""
import sys

import numpy as np
import pytest
import torch

from linear_attention_recurrence_recurrent_amd import GdnError, conv_silu, synth
from oracle import gdn_oracle as orc

pytestmark = pytest.mark.gpu

UNIT_ROUNDOFF = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def operands(B, T, C, W, dtype, *, seed, bias=True, state=True):
    g = torch.Generator().manual_seed(seed)
    dt = synth.DTYPES[dtype]
    x = torch.randn((B, T, C), generator=g, dtype=torch.float64).to(dt)
    w = (torch.randn((C, W), generator=g, dtype=torch.float64) / W ** 0.5).to(dt)
    b = torch.randn((C,), generator=g, dtype=torch.float64).to(dt) if bias else None
    s = torch.randn((B, C, W - 1), generator=g, dtype=torch.float64).to(dt) if state else None
    return x, w, b, s


def check_close(got, ref, dtype, what):
    got = got.detach().double().cpu().numpy()
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    if dtype == "f32":
        bound = 1e-4 * (1.0 + np.abs(ref))
    else:
        bound = UNIT_ROUNDOFF[dtype] * np.abs(ref) + 1e-5 * (1.0 + np.abs(ref))
    ratio = np.abs(got - ref) / bound
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= 1.0, "%s: error reaches %.3f of the bound at %s" % (
        what, worst, np.unravel_index(int(ratio.argmax()), ratio.shape))


def run_both(B, T, C, W, dtype, *, seed, bias=True, state=True, apply_silu=True, offset=0):
    x, w, b, s = operands(B, T, C, W, dtype, seed=seed, bias=bias, state=state)
    dx = x.to(DEV)
    if offset:  # a base address that is not 16-byte aligned: the scalar path
        buf = torch.empty(x.numel() + offset, dtype=x.dtype, device=DEV)
        dx = buf[offset:].view(x.shape)
        dx.copy_(x.to(DEV))
    y, st = conv_silu(dx, w.to(DEV), None if b is None else b.to(DEV),
                      None if s is None else s.to(DEV), apply_silu=apply_silu)
    torch.cuda.synchronize()
    yr, sr = orc.conv_silu(x, w, b, s, apply_silu=apply_silu)
    check_close(y, yr, dtype, "y")
    assert np.array_equal(st.double().cpu().numpy(), sr), "state"
    return x, w, b, s, y, st


CASES = [
    # (B, T, C, W, dtype, bias, state)
    (2, 37, 96, 4, "bf16", True, True),    # vector path, ragged token tile
    (3, 130, 64, 3, "f32", False, True),   # many token tiles
    (1, 5, 130, 4, "f16", True, False),    # C % 4 != 0: scalar path, no context
    (2, 70, 12, 1, "bf16", True, True),    # width one (no context)
    (1, 65, 8, 8, "f32", True, True),      # widest filter, ragged last tile
    (4, 1, 256, 4, "bf16", False, True),   # decode: one token with its context
    (2, 2, 40, 4, "f16", True, True),      # fewer tokens than the context
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dT%dC%dW%d-%s%s%s" % (
    c[0], c[1], c[2], c[3], c[4], "-b" if c[5] else "", "-s" if c[6] else ""))
def test_conv_small_cases(case):
    B, T, C, W, dt, bias, state = case
    say("conv %s" % (case,))
    run_both(B, T, C, W, dt, seed=B * 7 + T, bias=bias, state=state)


def test_conv_without_silu_and_unaligned_base():
    say("conv no-silu / unaligned")
    run_both(2, 40, 64, 4, "f32", seed=3, apply_silu=False)
    run_both(2, 40, 64, 4, "bf16", seed=4, offset=2)


def test_conv_time_chaining_and_in_place_state():
    """conv over T1 + T2 tokens equals conv over T1 then T2 with the carried
    state, bit for bit (each output is computed in the same order whatever the
    tiling); the in-place state update equals the out-of-place one."""
    say("conv chaining")
    x, w, b, s = operands(2, 150, 64, 4, "bf16", seed=11)
    dx, dw, db, ds = (t.to(DEV) for t in (x, w, b, s))
    y, st = conv_silu(dx, dw, db, ds)
    for T1 in (1, 3, 64, 100):
        y1, s1 = conv_silu(dx[:, :T1].contiguous(), dw, db, ds)
        s1c = s1.clone()
        y2, s2 = conv_silu(dx[:, T1:].contiguous(), dw, db, s1c, inplace=True)
        torch.cuda.synchronize()
        assert s2.data_ptr() == s1c.data_ptr()
        assert torch.equal(torch.cat([y1, y2], dim=1), y)
        assert torch.equal(s2, st)


def test_conv_empty_time_axis_copies_the_context():
    say("conv T=0")
    x, w, b, s = operands(3, 0, 16, 4, "f16", seed=5)
    y, st = conv_silu(x.to(DEV), w.to(DEV), b.to(DEV), s.to(DEV))
    y0, st0 = conv_silu(x.to(DEV), w.to(DEV), b.to(DEV), None)
    torch.cuda.synchronize()
    assert y.shape == (3, 0, 16) and torch.equal(st.cpu(), s)
    assert torch.all(st0 == 0)


def test_conv_rejections_raise():
    x = torch.zeros((1, 4, 8), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((8, 9), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(GdnError, match="GDN_EUNSUPPORTED"):
        conv_silu(x, w)
    with pytest.raises(GdnError):
        conv_silu(x, w[:, :4].float())


def test_conv_qwen_prefill_full_size():
    """The prefill producer at full size (B=1, T=4096, C = 2*16*128 + 32*128 =
    8192 channels, W=4, bf16), every output against the oracle."""
    say("conv full size")
    run_both(1, 4096, 8192, 4, "bf16", seed=21, bias=False, state=True)
