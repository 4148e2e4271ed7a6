"""Seeded synthetic operands for the Gated DeltaNet recurrence.

This module is the one piece of code that both the HIP path's callers (tests,
bench) and the CPU oracle's callers share.  It draws random numbers and casts
them; it holds none of the recurrence's arithmetic (no normalisation, no
decay, no state update, no gating).  The distribution transforms used to shape
the gate operands (``-softplus`` for ``log_decay``, ``sigmoid`` for ``beta``)
belong to the workload recipe, not to the operator, which takes both gates as
given.

q and k are drawn as plain N(0, 1).  The operator folds the q/k L2
normalisation and the 1/sqrt(Dk) scale in itself (torch-to-nnef page,
``native_gdn_reject_reason``: the fused decode operator folds the q/k l2-norm
and the output scale), and L2 normalisation removes any positive pre-scale, so
an input that was already normalised outside gives the same result up to the
eps term.  Drawing raw vectors keeps this module free of the method's
arithmetic.

Draws are made in float64 with ``numpy.random.default_rng(seed)`` in a fixed
order (q, k, v, z, log-decay pre-activation, beta pre-activation, s0, w) and in
the operand's own layout, then cast to the operand dtype (float64 -> float32
round-to-nearest-even -> float16/bfloat16 round-to-nearest-even).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic workload."""

    name: str
    B: int
    T: int
    Hk: int
    Hv: int
    Dk: int
    Dv: int
    dtype: str = "bf16"          # q, k, v, z, w
    gate_dtype: Optional[str] = None  # log_decay, beta (None: same as dtype)
    head_major: bool = False
    decay_scale: float = 1.0     # log_decay = -softplus(N(0,1)) * decay_scale
    beta_mean: float = 0.0       # beta = sigmoid(N(beta_mean, 1))
    s0_std: float = 0.02         # s0 ~ N(0, s0_std) in f32; 0 -> zeros
    gated: bool = True           # draw z and w
    seed: int = 0
    steps: int = 1               # decode workloads: number of chained steps

    @property
    def G(self) -> int:
        return self.Hv // self.Hk


# The five workloads of the benchmark description.  Decode workloads (steps)
# are drawn with T = steps and consumed one token at a time.
WORKLOADS: Dict[int, Workload] = {
    0: Workload("tiny scan f32 B1 H2 D16 T8", B=1, T=8, Hk=2, Hv=2, Dk=16, Dv=16,
                dtype="f32", s0_std=0.0, seed=0),
    1: Workload("decode step bf16 B1 Hk16 Hv32 D128", B=1, T=1, Hk=16, Hv=32, Dk=128,
                Dv=128, dtype="bf16", seed=1, steps=1),
    2: Workload("decode bf16 B64 Hk16 Hv32 D128 x100 chained steps", B=64, T=100, Hk=16,
                Hv=32, Dk=128, Dv=128, dtype="bf16", seed=2, steps=100),
    3: Workload("prefill scan bf16 B1 T4096 Hk16 Hv32 D128 token-major", B=1, T=4096,
                Hk=16, Hv=32, Dk=128, Dv=128, dtype="bf16", seed=3),
    4: Workload("head-major scan f16 B16 T1024 Hk16 Hv32 D128 slow decay", B=16, T=1024,
                Hk=16, Hv=32, Dk=128, Dv=128, dtype="f16", head_major=True,
                decay_scale=0.01, beta_mean=2.0, seed=4),
}


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.float32)
    return t.to(DTYPES[dtype]).contiguous()


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def operand_shapes(B, T, Hk, Hv, Dk, Dv, head_major):
    """Shapes of (q, k, v, gates) in the chosen layout.

    Token-major is [B, T, H, D] / [B, T, Hv]; head-major is [B, H, T, D] /
    [B, Hv, T] (torch-to-nnef page, ``emit_native_gdn_recurrent``)."""
    if head_major:
        return (B, Hk, T, Dk), (B, Hv, T, Dv), (B, Hv, T)
    return (B, T, Hk, Dk), (B, T, Hv, Dv), (B, T, Hv)


def make(w: Workload, *, T: Optional[int] = None, B: Optional[int] = None,
         seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Draw the operands of workload ``w`` as CPU tensors.

    Returns q, k, v, log_decay, beta, s0 and, when ``w.gated``, z and w.
    q/k/v/z/w take ``w.dtype``; gates take ``w.gate_dtype or w.dtype``; s0 is
    float32 [B, Hv, Dv, Dk]."""
    B = w.B if B is None else B
    T = w.T if T is None else T
    rng = np.random.default_rng(w.seed if seed is None else seed)
    qk_shape, v_shape, g_shape = operand_shapes(B, T, w.Hk, w.Hv, w.Dk, w.Dv, w.head_major)
    gdt = w.gate_dtype or w.dtype
    out: Dict[str, torch.Tensor] = {}
    out["q"] = _cast(rng.standard_normal(qk_shape), w.dtype)
    out["k"] = _cast(rng.standard_normal(qk_shape), w.dtype)
    out["v"] = _cast(rng.standard_normal(v_shape), w.dtype)
    z = rng.standard_normal(v_shape) if w.gated else None
    a = rng.standard_normal(g_shape)
    b = rng.standard_normal(g_shape) + w.beta_mean
    out["log_decay"] = _cast(-_softplus(a) * w.decay_scale, gdt)
    out["beta"] = _cast(_sigmoid(b), gdt)
    if w.s0_std > 0:
        out["s0"] = _cast(rng.standard_normal((B, w.Hv, w.Dv, w.Dk)) * w.s0_std, "f32")
    else:
        out["s0"] = torch.zeros((B, w.Hv, w.Dv, w.Dk), dtype=torch.float32)
    if w.gated:
        out["z"] = _cast(z, w.dtype)
        out["w"] = _cast(1.0 + 0.1 * rng.standard_normal((w.Dv,)), w.dtype)
    return out


def random_operands(B, T, Hk, Hv, Dk, Dv, *, dtype="f32", gate_dtype=None, head_major=False,
                    gated=True, seed=0, decay_scale=1.0, beta_mean=0.0, s0_std=0.5):
    """Operands for an ad-hoc shape (tests): same recipe as ``make``."""
    w = Workload("adhoc", B=B, T=T, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, dtype=dtype,
                 gate_dtype=gate_dtype, head_major=head_major, decay_scale=decay_scale,
                 beta_mean=beta_mean, s0_std=s0_std, gated=gated, seed=seed)
    return make(w)


def step_slices(ops: Dict[str, torch.Tensor], head_major: bool):
    """Split operands drawn with T = steps into per-step dense tensors.

    Each returned dict holds q/k/v/log_decay/beta (and z) with T = 1, copied
    into dense storage so that a step call sees contiguous operands."""
    t_axis = 2 if head_major else 1
    steps = ops["q"].shape[t_axis]
    res = []
    for t in range(steps):
        d = {}
        for name in ("q", "k", "v", "z"):
            if name in ops:
                d[name] = ops[name].narrow(t_axis, t, 1).contiguous()
        for name in ("log_decay", "beta"):
            d[name] = ops[name].narrow(t_axis, t, 1).contiguous()
        res.append(d)
    return res
