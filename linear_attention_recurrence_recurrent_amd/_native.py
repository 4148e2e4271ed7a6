"""ctypes view of libgdn_hip.so (the C ABI declared in include/gdn.h).

Argument marshalling only: every step of the recurrence runs in the HIP
kernels behind these symbols.  There is no fallback: if the library is not
built, loading raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgdn_hip.so")

GDN_F32, GDN_F16, GDN_BF16 = 0, 1, 2
GDN_FOLD_QK_L2NORM = 1
GDN_FOLD_Q_SCALE = 2
GDN_SCAN_PER_TOKEN = 4
GDN_SCAN_BLOCK = 8
GDN_SCAN_EXACT = 16
STATUS = {0: "GDN_OK", 1: "GDN_EINVAL", 2: "GDN_ESHAPE", 3: "GDN_EDTYPE", 4: "GDN_EGROUP",
          5: "GDN_EUNSUPPORTED", 6: "GDN_EALIGN", 7: "GDN_EALIAS", 8: "GDN_EDEVICE",
          9: "GDN_EWORKSPACE"}
ABI_VERSION = 2

# Every symbol include/gdn.h and include/gdn_calib.h declare.
EXPORTS = ("gdn_recurrent_step", "gdn_recurrent_step_three_pass", "gdn_scan",
           "gdn_scan_workspace_size", "gdn_scan_noalloc", "gdn_gates", "gdn_conv_silu", "gdn_check",
           "gdn_last_error", "gdn_status_str", "gdn_abi_version", "gdn_calib_stream",
           "gdn_calib_variant_name", "gdn_calib_clock")
GDN_CALIB_RMW, GDN_CALIB_COPY, GDN_CALIB_VARIANTS = 0, 1, 15
GDN_NOALLOC_SCRATCH_BYTES = 64 << 20


class GdnDesc(ctypes.Structure):
    """Mirror of ``gdn_desc`` (same field order and C alignment)."""

    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("Hk", ctypes.c_int64),
                ("Hv", ctypes.c_int64), ("Dk", ctypes.c_int64), ("Dv", ctypes.c_int64),
                ("head_major", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("gate_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("qk_eps", ctypes.c_float), ("norm_eps", ctypes.c_float)]


_lib = None


def lib():
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libgdn_hip.so is not built (run `python -m "
                "linear_attention_recurrence_recurrent_amd.build` or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        dp = ctypes.POINTER(GdnDesc)
        for name in ("gdn_recurrent_step", "gdn_recurrent_step_three_pass", "gdn_scan_noalloc"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [dp] + [vp] * 11
        # (desc, q, k, v, log_decay, beta, s0, z, w, y, s_out, workspace, workspace_bytes, stream)
        L.gdn_scan.restype = ctypes.c_int
        L.gdn_scan.argtypes = [dp] + [vp] * 11 + [ctypes.c_uint64, vp]
        L.gdn_scan_workspace_size.restype = ctypes.c_int
        L.gdn_scan_workspace_size.argtypes = [dp, ctypes.POINTER(ctypes.c_uint64)]
        L.gdn_gates.restype = ctypes.c_int
        L.gdn_gates.argtypes = [ctypes.c_int64, vp, vp, ctypes.c_int32, ctypes.c_float, vp, vp,
                                ctypes.c_int32, vp]
        L.gdn_conv_silu.restype = ctypes.c_int
        L.gdn_conv_silu.argtypes = [ctypes.c_int64] * 3 + [ctypes.c_int32] * 3 + [vp] * 7
        L.gdn_check.restype = ctypes.c_int
        L.gdn_check.argtypes = [dp] + [vp] * 11 + [ctypes.c_uint64]
        L.gdn_last_error.restype = ctypes.c_char_p
        L.gdn_last_error.argtypes = []
        L.gdn_status_str.restype = ctypes.c_char_p
        L.gdn_status_str.argtypes = [ctypes.c_int]
        L.gdn_abi_version.restype = ctypes.c_int
        L.gdn_abi_version.argtypes = []
        L.gdn_calib_stream.restype = ctypes.c_int
        L.gdn_calib_stream.argtypes = [ctypes.c_int32, ctypes.c_int32, vp, vp, ctypes.c_uint64,
                                       vp]
        L.gdn_calib_variant_name.restype = ctypes.c_char_p
        L.gdn_calib_variant_name.argtypes = [ctypes.c_int32]
        L.gdn_calib_clock.restype = ctypes.c_int
        L.gdn_calib_clock.argtypes = [ctypes.c_int32, ctypes.c_int32, vp, vp]
        _lib = L
    return _lib


def last_error() -> str:
    return lib().gdn_last_error().decode()
