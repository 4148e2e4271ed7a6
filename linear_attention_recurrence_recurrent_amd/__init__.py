"""MI355X (gfx950) Gated DeltaNet recurrence: thin Python binding of libgdn_hip.so.

``recurrent_step`` (single-token decode) and ``scan`` (the whole time axis)
follow the operator contract of the "gated_delta" page (torch-to-nnef op
reference): operands (q, k, v, log_decay, beta, s0), token-major
[B, S, H, W] or head-major [B, H, S, W] layout, outputs (y, final_state) with
y in float32 whatever the input dtype.  The recurrence and the optional
gate-first RMSNorm are those of the "Module gdn" page (logicaffeine
codegen_cuda/gdn).  torch supplies device memory and the current stream; all
arithmetic runs in the HIP kernels.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _native
from ._native import (GDN_FOLD_Q_SCALE, GDN_FOLD_QK_L2NORM, GDN_SCAN_BLOCK, GDN_SCAN_EXACT,
                      GDN_SCAN_PER_TOKEN, GdnDesc)

__all__ = ["recurrent_step", "recurrent_step_three_pass", "scan", "scan_noalloc",
           "scan_workspace_bytes", "gates",
           "conv_silu", "check", "abi_version", "GdnError"]

_DT = {torch.float32: _native.GDN_F32, torch.float16: _native.GDN_F16,
       torch.bfloat16: _native.GDN_BF16}


class GdnError(ValueError):
    """A call the library rejected; ``status`` is the gdn_status name."""

    def __init__(self, status: int, reason: str):
        self.status = _native.STATUS.get(status, str(status))
        super().__init__("%s: %s" % (self.status, reason))


def abi_version() -> int:
    return _native.lib().gdn_abi_version()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _desc(B, T, Hk, Hv, Dk, Dv, head_major, dtype, gate_dtype, fold_qk_l2norm, fold_q_scale,
          qk_eps, norm_eps, form=None, exact=False) -> GdnDesc:
    flags = (GDN_FOLD_QK_L2NORM if fold_qk_l2norm else 0) | (GDN_FOLD_Q_SCALE if fold_q_scale else 0)
    if exact:
        flags |= GDN_SCAN_EXACT
    if form == "per_token":
        flags |= GDN_SCAN_PER_TOKEN
    elif form == "block":
        flags |= GDN_SCAN_BLOCK
    elif form is not None:
        raise GdnError(1, "form must be None, 'per_token' or 'block'")
    return GdnDesc(B, T, Hk, Hv, Dk, Dv, int(bool(head_major)), dtype, gate_dtype, flags,
                   float(qk_eps), float(norm_eps))


def _dtype_code(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _DT:
        raise GdnError(3, "%s has unsupported dtype %s" % (name, t.dtype))
    return _DT[t.dtype]


def _prepare(q, k, v, log_decay, beta, s0, z, w, head_major, T_expected=None):
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4:
        raise GdnError(2, "q, k must be 4-d with equal shapes and v 4-d")
    if head_major:
        B, Hk, T, Dk = q.shape
        Bv, Hv, Tv, Dv = v.shape
        gshape = (B, Hv, T)
    else:
        B, T, Hk, Dk = q.shape
        Bv, Tv, Hv, Dv = v.shape
        gshape = (B, T, Hv)
    if (Bv, Tv) != (B, T):
        raise GdnError(2, "v batch/time %s do not match q %s" % ((Bv, Tv), (B, T)))
    if tuple(log_decay.shape) != gshape or tuple(beta.shape) != gshape:
        raise GdnError(2, "log_decay and beta must have shape %s" % (gshape,))
    if z is not None and z.shape != v.shape:
        raise GdnError(2, "z must have v's shape")
    if (z is None) != (w is None):
        raise GdnError(1, "z and w must be given together")
    if w is not None and tuple(w.shape) != (Dv,):
        raise GdnError(2, "w must have shape (%d,)" % Dv)
    dev = q.device
    if dev.type != "cuda":
        raise GdnError(8, "operands must be on a GPU device")
    tensors = dict(q=q, k=k, v=v, log_decay=log_decay, beta=beta, z=z, w=w, s0=s0)
    for n, t in tensors.items():
        if t is None:
            continue
        if t.device != dev:
            raise GdnError(1, "%s is on %s, q on %s" % (n, t.device, dev))
        if not t.is_contiguous():
            raise GdnError(1, "%s must be contiguous" % n)
    dt = _dtype_code(q, "q")
    for n in ("k", "v", "z", "w"):
        t = tensors[n]
        if t is not None and _DT.get(t.dtype) != dt:
            raise GdnError(3, "%s dtype %s differs from q's %s" % (n, t.dtype, q.dtype))
    gdt = _dtype_code(log_decay, "log_decay")
    if _DT.get(beta.dtype) != gdt:
        raise GdnError(3, "beta dtype must equal log_decay dtype")
    if s0 is not None:
        if s0.dtype != torch.float32 or tuple(s0.shape) != (B, Hv, Dv, Dk):
            raise GdnError(2, "s0 must be float32 [%d, %d, %d, %d]" % (B, Hv, Dv, Dk))
    return B, T, Hk, Hv, Dk, Dv, dt, gdt


def _check_out(t: torch.Tensor, name: str, shape, dev) -> None:
    """A caller-supplied output must be float32, contiguous, on q's device and
    of the exact shape the kernels write (the library sizes its writes from
    the descriptor, not from the tensor)."""
    if t.dtype != torch.float32:
        raise GdnError(3, "%s must be float32 (got %s)" % (name, t.dtype))
    if t.device != dev:
        raise GdnError(1, "%s is on %s, q on %s" % (name, t.device, dev))
    if tuple(t.shape) != tuple(shape):
        raise GdnError(2, "%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise GdnError(1, "%s must be contiguous" % name)


def _outputs(q, v, s0, out, state_out, B, Hv, Dv, Dk):
    if out is not None:
        _check_out(out, "out", v.shape, q.device)
    if state_out is not None:
        _check_out(state_out, "state_out", (B, Hv, Dv, Dk), q.device)
    y = out if out is not None else torch.empty(v.shape, dtype=torch.float32, device=q.device)
    return y


def _raise(rc: int) -> None:
    reason = _native.last_error()
    if rc == 8:
        raise RuntimeError("%s: %s" % (_native.STATUS[rc], reason))
    raise GdnError(rc, reason)


def scan_workspace_bytes(desc: GdnDesc) -> int:
    """Device workspace gdn_scan needs for ``desc`` (gdn_scan_workspace_size)."""
    n = ctypes.c_uint64(0)
    rc = _native.lib().gdn_scan_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if rc != 0:
        _raise(rc)
    return int(n.value)


def _call(fn_name, desc, q, k, v, log_decay, beta, s0, z, w, y, s_out):
    L = _native.lib()
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        rc = getattr(L, fn_name)(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_decay),
                                 _ptr(beta), _ptr(s0), _ptr(z), _ptr(w), _ptr(y), _ptr(s_out),
                                 ctypes.c_void_p(stream))
    if rc != 0:
        _raise(rc)


def scan(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_decay: torch.Tensor,
         beta: torch.Tensor, s0: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
         w: Optional[torch.Tensor] = None, *, head_major: bool = False,
         fold_qk_l2norm: bool = True, fold_q_scale: bool = True, qk_eps: float = 1e-6,
         norm_eps: float = 1e-6, out: Optional[torch.Tensor] = None,
         state_out: Optional[torch.Tensor] = None, form: Optional[str] = None,
         exact: bool = False,
         workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Gated DeltaNet recurrence over the time axis; returns (y, final_state).

    q, k: [B, T, Hk, D] (head-major: [B, Hk, T, D]); v, z: [B, T, Hv, D]
    ([B, Hv, T, D]); log_decay, beta: [B, T, Hv] ([B, Hv, T]); s0:
    float32 [B, Hv, D, D] (None: zeros); w: [D].  y is float32 in v's layout;
    final_state is float32 [B, Hv, D, D] (``state_out`` may be ``s0`` for an
    in-place update).  ``form`` picks the time loop: "per_token" (vector units,
    any D), "block" (16 tokens at a time on the matrix cores; D of 32, 64, 128
    or 256), or None for the library's choice for the shape (the block form
    wherever it runs, for T of 2 or more).  ``exact`` makes the block
    form's products with the f32 state exact f32 products for 16-bit q and k
    (three bf16 parts of the state instead of two rounded ones, whose terms
    are within 2^-16 relative).  The block form's workspace
    (``scan_workspace_bytes``) is allocated here with torch on the current
    stream unless ``workspace`` (a contiguous uint8 device tensor at least
    that large) is passed."""
    B, T, Hk, Hv, Dk, Dv, dt, gdt = _prepare(q, k, v, log_decay, beta, s0, z, w, head_major)
    if s0 is None:
        s0 = torch.zeros((B, Hv, Dv, Dk), dtype=torch.float32, device=q.device)
    y = _outputs(q, v, s0, out, state_out, B, Hv, Dv, Dk)
    s_out = state_out if state_out is not None else torch.empty_like(s0)
    desc = _desc(B, T, Hk, Hv, Dk, Dv, head_major, dt, gdt, fold_qk_l2norm, fold_q_scale,
                 qk_eps, norm_eps, form, exact)
    need = scan_workspace_bytes(desc)
    ws = None
    if need:
        if workspace is None:
            ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        else:
            if workspace.dtype != torch.uint8 or workspace.device != q.device or \
                    not workspace.is_contiguous():
                raise GdnError(1, "workspace must be a contiguous uint8 tensor on q's device")
            ws = workspace
    L = _native.lib()
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        rc = L.gdn_scan(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_decay),
                        _ptr(beta), _ptr(s0), _ptr(z), _ptr(w), _ptr(y), _ptr(s_out), _ptr(ws),
                        ws.numel() if ws is not None else 0, ctypes.c_void_p(stream))
    if rc != 0:
        _raise(rc)
    return y, s_out


def scan_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_decay: torch.Tensor,
                 beta: torch.Tensor, s0: torch.Tensor, z: Optional[torch.Tensor] = None,
                 w: Optional[torch.Tensor] = None, *, head_major: bool = False,
                 fold_qk_l2norm: bool = True, fold_q_scale: bool = True, qk_eps: float = 1e-6,
                 norm_eps: float = 1e-6, out: Optional[torch.Tensor] = None,
                 state_out: Optional[torch.Tensor] = None, form: Optional[str] = None,
                 exact: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """``scan`` through gdn_scan_noalloc: the library takes no workspace and
    allocates nothing (the block form's records go to its static per-GPU
    scratch, at most 64 MiB of them; larger shapes raise GdnError).  Calls
    that overlap on one GPU race on that scratch.  Pass ``out`` and
    ``state_out`` to keep this call free of allocations on the torch side too."""
    B, T, Hk, Hv, Dk, Dv, dt, gdt = _prepare(q, k, v, log_decay, beta, s0, z, w, head_major)
    if s0 is None:
        raise GdnError(1, "scan_noalloc needs s0")
    y = _outputs(q, v, s0, out, state_out, B, Hv, Dv, Dk)
    s_out = state_out if state_out is not None else torch.empty_like(s0)
    desc = _desc(B, T, Hk, Hv, Dk, Dv, head_major, dt, gdt, fold_qk_l2norm, fold_q_scale,
                 qk_eps, norm_eps, form, exact)
    _call("gdn_scan_noalloc", desc, q, k, v, log_decay, beta, s0, z, w, y, s_out)
    return y, s_out


def recurrent_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_decay: torch.Tensor,
                   beta: torch.Tensor, s0: torch.Tensor, z: Optional[torch.Tensor] = None,
                   w: Optional[torch.Tensor] = None, *, head_major: bool = False,
                   inplace: bool = False, fold_qk_l2norm: bool = True, fold_q_scale: bool = True,
                   qk_eps: float = 1e-6, norm_eps: float = 1e-6,
                   out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """One decode step.  Operands carry T == 1 ([B, 1, H, D] etc., or the
    head-major equivalent); ``inplace`` writes the new state into ``s0``."""
    B, T, Hk, Hv, Dk, Dv, dt, gdt = _prepare(q, k, v, log_decay, beta, s0, z, w, head_major)
    if s0 is None:
        raise GdnError(1, "recurrent_step needs s0")
    y = _outputs(q, v, s0, out, None, B, Hv, Dv, Dk)
    s_out = s0 if inplace else torch.empty_like(s0)
    desc = _desc(B, T, Hk, Hv, Dk, Dv, head_major, dt, gdt, fold_qk_l2norm, fold_q_scale,
                 qk_eps, norm_eps)
    _call("gdn_recurrent_step", desc, q, k, v, log_decay, beta, s0, z, w, y, s_out)
    return y, s_out


def recurrent_step_three_pass(q, k, v, log_decay, beta, s0, z=None, w=None, *,
                              head_major: bool = False, inplace: bool = False,
                              fold_qk_l2norm: bool = True, fold_q_scale: bool = True,
                              qk_eps: float = 1e-6, norm_eps: float = 1e-6, out=None):
    """The decode step in its literal three-pass form (u = S.k, the update,
    o = S.q as three launches, "Module gdn" page, "The fusion"); same results
    as ``recurrent_step``, kept to measure the fusion's saving.  D == 128 only."""
    B, T, Hk, Hv, Dk, Dv, dt, gdt = _prepare(q, k, v, log_decay, beta, s0, z, w, head_major)
    if s0 is None:
        raise GdnError(1, "recurrent_step_three_pass needs s0")
    y = _outputs(q, v, s0, out, None, B, Hv, Dv, Dk)
    s_out = s0 if inplace else torch.empty_like(s0)
    desc = _desc(B, T, Hk, Hv, Dk, Dv, head_major, dt, gdt, fold_qk_l2norm, fold_q_scale,
                 qk_eps, norm_eps)
    _call("gdn_recurrent_step_three_pass", desc, q, k, v, log_decay, beta, s0, z, w, y, s_out)
    return y, s_out


def gates(a: torch.Tensor, b: torch.Tensor, *, decay_scale: float = 1.0,
          out_dtype: Optional[torch.dtype] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Gate producer (one launch): log_decay = -decay_scale*softplus(a),
    beta = sigmoid(b), elementwise; outputs in ``out_dtype`` (default a's)."""
    if a.shape != b.shape or a.dtype != b.dtype or a.device != b.device:
        raise GdnError(2, "a and b must match in shape, dtype and device")
    if a.device.type != "cuda":
        raise GdnError(8, "operands must be on a GPU device")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise GdnError(1, "a and b must be contiguous")
    odt = out_dtype or a.dtype
    ld = torch.empty(a.shape, dtype=odt, device=a.device)
    be = torch.empty(a.shape, dtype=odt, device=a.device)
    L = _native.lib()
    stream = torch.cuda.current_stream(a.device).cuda_stream
    with torch.cuda.device(a.device):
        rc = L.gdn_gates(a.numel(), _ptr(a), _ptr(b), _dtype_code(a, "a"), float(decay_scale),
                         _ptr(ld), _ptr(be), _DT[odt], ctypes.c_void_p(stream))
    if rc != 0:
        _raise(rc)
    return ld, be


def conv_silu(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
              state: Optional[torch.Tensor] = None, *, apply_silu: bool = True,
              inplace: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """Causal depthwise convolution over time with silu, one launch: the
    producer of q, k and v ("Module gdn" page, QWEN38_KERNELS).  x: [B, T, C];
    weight: [C, W] (tap W-1 on the current token); bias: [C]; state: the
    [B, C, W-1] inputs before x (None: zeros).  Returns (y [B, T, C] in x's
    dtype, new state [B, C, W-1] = the last W-1 inputs); ``inplace`` writes the
    new state into ``state``."""
    if x.dim() != 3 or weight.dim() != 2 or weight.shape[0] != x.shape[2]:
        raise GdnError(2, "x must be [B, T, C] and weight [C, W]")
    B, T, C = x.shape
    W = weight.shape[1]
    if x.device.type != "cuda":
        raise GdnError(8, "operands must be on a GPU device")
    for n, t in (("weight", weight), ("bias", bias), ("state", state)):
        if t is not None and (t.dtype != x.dtype or t.device != x.device):
            raise GdnError(3, "%s must match x in dtype and device" % n)
    if bias is not None and tuple(bias.shape) != (C,):
        raise GdnError(2, "bias must have shape (%d,)" % C)
    if state is not None and tuple(state.shape) != (B, C, W - 1):
        raise GdnError(2, "state must have shape %s" % ((B, C, W - 1),))
    for n, t in (("x", x), ("weight", weight), ("bias", bias), ("state", state)):
        if t is not None and not t.is_contiguous():
            raise GdnError(1, "%s must be contiguous" % n)
    if inplace and state is None:
        raise GdnError(1, "inplace needs a state")
    y = torch.empty_like(x)
    new_state = state if inplace else torch.empty((B, C, W - 1), dtype=x.dtype, device=x.device)
    L = _native.lib()
    stream = torch.cuda.current_stream(x.device).cuda_stream
    with torch.cuda.device(x.device):
        rc = L.gdn_conv_silu(B, T, C, W, _dtype_code(x, "x"), int(bool(apply_silu)), _ptr(x),
                             _ptr(weight), _ptr(bias), _ptr(state), _ptr(y), _ptr(new_state),
                             ctypes.c_void_p(stream))
    if rc != 0:
        _raise(rc)
    return y, new_state


def check(desc: GdnDesc, q=None, k=None, v=None, log_decay=None, beta=None, s0=None, z=None,
          w=None, y=None, s_out=None, workspace=None, workspace_bytes=0) -> Tuple[int, str]:
    """Host-only validation (gdn_check) on raw integer addresses; returns (status, reason)."""
    L = _native.lib()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    rc = L.gdn_check(ctypes.byref(desc), vp(q), vp(k), vp(v), vp(log_decay), vp(beta), vp(s0),
                     vp(z), vp(w), vp(y), vp(s_out), vp(workspace), int(workspace_bytes))
    return rc, (_native.last_error() if rc else "")
