"""torch custom ops: the fake kernels give the promoted float32 output (CPU, meta
tensors), and on the GPU the ops equal the direct C-ABI calls and pass opcheck."""
import pytest
import torch

from linear_attention_recurrence_recurrent_amd import scan, synth
from linear_attention_recurrence_recurrent_amd.torch_op import recurrent_step_op, scan_op


def _meta(ops):
    return {n: t.to("meta") for n, t in ops.items()}


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("head_major", [False, True])
def test_fake_kernel_promotes_to_f32(dtype, head_major):
    ops = _meta(synth.random_operands(2, 5, 2, 4, 64, 64, dtype=dtype, head_major=head_major))
    from torch._subclasses.fake_tensor import FakeTensorMode
    with FakeTensorMode(allow_non_fake_inputs=True):
        y, s = scan_op(ops["q"], ops["k"], ops["v"], ops["log_decay"], ops["beta"], ops["s0"],
                       ops["z"], ops["w"], head_major)
    assert y.dtype == torch.float32 and tuple(y.shape) == tuple(ops["v"].shape)
    assert s.dtype == torch.float32 and tuple(s.shape) == tuple(ops["s0"].shape)


def test_fake_kernel_step():
    ops = _meta(synth.random_operands(3, 1, 2, 4, 32, 32, dtype="bf16"))
    from torch._subclasses.fake_tensor import FakeTensorMode
    with FakeTensorMode(allow_non_fake_inputs=True):
        y, s = recurrent_step_op(ops["q"], ops["k"], ops["v"], ops["log_decay"], ops["beta"],
                                 ops["s0"])
    assert y.dtype == torch.float32 and tuple(y.shape) == (3, 1, 4, 32)


@pytest.mark.gpu
def test_op_equals_direct_call_and_opcheck():
    ops = {n: t.cuda() for n, t in synth.random_operands(2, 9, 2, 4, 64, 64, dtype="bf16",
                                                         seed=3).items()}
    y, s = scan(ops["q"], ops["k"], ops["v"], ops["log_decay"], ops["beta"], ops["s0"], ops["z"],
                ops["w"])
    yo, so = scan_op(ops["q"], ops["k"], ops["v"], ops["log_decay"], ops["beta"], ops["s0"],
                     ops["z"], ops["w"], False)
    torch.cuda.synchronize()
    assert torch.equal(y, yo) and torch.equal(s, so)
    torch.library.opcheck(scan_op, (ops["q"], ops["k"], ops["v"], ops["log_decay"], ops["beta"],
                                    ops["s0"], ops["z"], ops["w"], False),
                          test_utils=("test_schema", "test_faketensor"))
