"""Python face of the float64 CPU oracle (``gdn_oracle.c``).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It does not import the HIP package
and the HIP package does not import it.

``scan`` computes the Gated DeltaNet recurrence over the time axis with the
three literal passes per token ("Module gdn" page, module description and
"The fusion"), the folded q/k L2 norm and q scale ("gated_delta" page,
native_gdn_reject_reason and l2norm) and, when ``z`` is given, the gated
RMSNorm applied gate-first ("Module gdn" page, last equation).  Head-major
operands ([B, H, S, ...], "gated_delta" page, emit_native_gdn_recurrent) are
transposed to token-major before the call and the output is transposed back.

Inputs may be numpy arrays or torch tensors of any float dtype; they are
widened to float64 exactly.  Outputs are float64 numpy arrays.

``gates`` and ``conv_silu`` are the two producers next to the recurrence
("Module gdn" page, QWEN38_KERNELS): both gates from their pre-activations,
and the causal convolution with silu that produces q, k and v.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
LIB = os.path.join(HERE, "libgdn_oracle.so")

FOLD_QK_L2NORM = 1
FOLD_Q_SCALE = 2

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                               "-o", tmp, SRC, "-lm", "-lpthread"])
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.gdn_oracle_scan.restype = ctypes.c_int
        lib.gdn_oracle_scan.argtypes = [i64] * 6 + [ctypes.c_uint32, ctypes.c_double,
                                                    ctypes.c_double] + [dp] * 10 + [ctypes.c_int]
        lib.gdn_oracle_l2norm.restype = None
        lib.gdn_oracle_l2norm.argtypes = [dp, i64, ctypes.c_double]
        lib.gdn_oracle_gates.restype = None
        lib.gdn_oracle_gates.argtypes = [i64, dp, dp, ctypes.c_double, dp, dp]
        lib.gdn_oracle_conv.restype = None
        lib.gdn_oracle_conv.argtypes = [i64, i64, i64, i64, ctypes.c_int] + [dp] * 6
        lib.gdn_oracle_gated_rmsnorm.restype = None
        lib.gdn_oracle_gated_rmsnorm.argtypes = [dp, dp, dp, i64, ctypes.c_double, dp]
        _lib = lib
    return _lib


def _f64(x) -> Optional[np.ndarray]:
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: widen exactly on the CPU
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def scan(q, k, v, log_decay, beta, s0, z=None, w=None, *, head_major: bool = False,
         fold_qk_l2norm: bool = True, fold_q_scale: bool = True, qk_eps: float = 1e-6,
         norm_eps: float = 1e-6, threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Return (y, final_state) in float64.

    q, k: [B,T,Hk,Dk] (head-major: [B,Hk,T,Dk]); v, z: [B,T,Hv,Dv] (or
    [B,Hv,T,Dv]); log_decay, beta: [B,T,Hv] (or [B,Hv,T]); s0: [B,Hv,Dv,Dk];
    w: [Dv].  y has v's layout."""
    q, k, v, g, bt, s0, z, w = map(_f64, (q, k, v, log_decay, beta, s0, z, w))
    if (z is None) != (w is None) and z is None:
        raise ValueError("w given without z")
    if head_major:
        q, k, v = (np.ascontiguousarray(x.transpose(0, 2, 1, 3)) for x in (q, k, v))
        g, bt = (np.ascontiguousarray(x.transpose(0, 2, 1)) for x in (g, bt))
        if z is not None:
            z = np.ascontiguousarray(z.transpose(0, 2, 1, 3))
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    assert k.shape == q.shape and v.shape[:2] == (B, T) and g.shape == (B, T, Hv)
    assert bt.shape == g.shape and s0.shape == (B, Hv, Dv, Dk)
    if z is not None:
        assert z.shape == v.shape
        if w is None:
            w = np.ones((Dv,), dtype=np.float64)
        assert w.shape == (Dv,)
    y = np.empty((B, T, Hv, Dv), dtype=np.float64)
    s_out = np.empty_like(s0)
    flags = (FOLD_QK_L2NORM if fold_qk_l2norm else 0) | (FOLD_Q_SCALE if fold_q_scale else 0)
    rc = _load().gdn_oracle_scan(B, T, Hk, Hv, Dk, Dv, flags, qk_eps, norm_eps, _ptr(q), _ptr(k),
                                 _ptr(v), _ptr(g), _ptr(bt), _ptr(s0), _ptr(z), _ptr(w), _ptr(y),
                                 _ptr(s_out), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the shapes")
    if head_major:
        y = np.ascontiguousarray(y.transpose(0, 2, 1, 3))
    return y, s_out


def step(q, k, v, log_decay, beta, s0, z=None, w=None, **kw):
    """One decode step: the scan at T == 1 (operands carry T == 1)."""
    return scan(q, k, v, log_decay, beta, s0, z, w, **kw)


def l2norm(x, eps: float = 1e-6) -> np.ndarray:
    """L2-normalise the last axis (the oracle's own routine, for its pins)."""
    x = _f64(x).copy()
    lib = _load()
    flat = x.reshape(-1, x.shape[-1])
    for r in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[r])
        lib.gdn_oracle_l2norm(_ptr(row), row.shape[0], eps)
        flat[r] = row
    return flat.reshape(x.shape)


def gated_rmsnorm(o, z, w=None, eps: float = 1e-6) -> np.ndarray:
    """Gate-first RMSNorm over the last axis (the oracle's own routine)."""
    o, z, w = _f64(o), _f64(z), _f64(w)
    n = o.shape[-1]
    of, zf = o.reshape(-1, n), z.reshape(-1, n)
    y = np.empty_like(of)
    lib = _load()
    for r in range(of.shape[0]):
        orow, zrow = np.ascontiguousarray(of[r]), np.ascontiguousarray(zf[r])
        yrow = np.empty(n)
        lib.gdn_oracle_gated_rmsnorm(_ptr(orow), _ptr(zrow), _ptr(w), n, eps, _ptr(yrow))
        y[r] = yrow
    return y.reshape(o.shape)


def gates(a, b, decay_scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """Gate producer: (log_decay, beta) = (-decay_scale*softplus(a), sigmoid(b)), float64."""
    a, b = _f64(a), _f64(b)
    assert a.shape == b.shape
    ld = np.empty_like(a)
    be = np.empty_like(b)
    _load().gdn_oracle_gates(a.size, _ptr(a), _ptr(b), decay_scale, _ptr(ld), _ptr(be))
    return ld, be


def conv_silu(x, weight, bias=None, state=None, *, apply_silu: bool = True):
    """Causal depthwise convolution over time, then silu ("Module gdn" page,
    QWEN38_KERNELS: the convolution carries the silu).  x: [B, T, C]; weight:
    [C, W] (tap W-1 on the current token); bias: [C]; state: [B, C, W-1], the
    W-1 inputs before x (zeros when None).  Returns (y [B, T, C], state_out
    [B, C, W-1] = the last W-1 inputs), float64."""
    x, weight, bias, state = map(_f64, (x, weight, bias, state))
    B, T, C = x.shape
    W = weight.shape[1]
    assert weight.shape == (C, W) and W >= 1
    if bias is not None:
        assert bias.shape == (C,)
    if state is not None:
        assert state.shape == (B, C, W - 1)
    y = np.empty((B, T, C), dtype=np.float64)
    st = np.empty((B, C, W - 1), dtype=np.float64)
    _load().gdn_oracle_conv(B, T, C, W, int(bool(apply_silu)), _ptr(x), _ptr(weight), _ptr(bias),
                            _ptr(state), _ptr(y), _ptr(st))
    return y, st
