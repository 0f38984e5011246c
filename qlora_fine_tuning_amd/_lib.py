"""ctypes binding of libqlora_mi355x.so (the C ABI in include/qlora.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their device pointers and torch's current HIP stream are passed
to the library, and every step of the computation runs in the library's
gfx950 kernels. There is no fallback: if the library is missing or a call
fails, a RuntimeError is raised.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# QLORA_LIB_PATH selects another build of the same library (the host-code
# sanitizer build that the tests make); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("QLORA_LIB_PATH") or os.path.join(PKG, "libqlora_mi355x.so")

QLORA_OK = 0
STATUS = {0: "QLORA_OK", -1: "QLORA_EINVAL", -2: "QLORA_ESHAPE", -3: "QLORA_EWORKSPACE",
          -4: "QLORA_EHIP", -5: "QLORA_ENOTIMPL"}
ACT = {"swiglu": 0, "geglu_tanh": 1}
MODE = {"auto": 0, "fused": 1, "staged": 2}

c_i64 = ctypes.c_int64
c_vp = ctypes.c_void_p


class Nf4(ctypes.Structure):
    _fields_ = [("codes", c_vp), ("absmax", c_vp), ("n", c_i64), ("k", c_i64),
                ("absmax_q", c_vp), ("absmax_scale", c_vp), ("absmax_offset", c_vp)]


class MlpWeights(ctypes.Structure):
    _fields_ = [("gate", Nf4), ("up", Nf4), ("down", Nf4),
                ("a_gate", c_vp), ("b_gate", c_vp), ("a_up", c_vp), ("b_up", c_vp),
                ("a_down", c_vp), ("b_down", c_vp),
                ("d", c_i64), ("h", c_i64), ("r", c_i64), ("s", ctypes.c_float), ("act", ctypes.c_int)]


class Mlp16Weights(ctypes.Structure):
    _fields_ = [("gate", c_vp), ("up", c_vp), ("down", c_vp),
                ("a_gate", c_vp), ("b_gate", c_vp), ("a_up", c_vp), ("b_up", c_vp),
                ("a_down", c_vp), ("b_down", c_vp),
                ("d", c_i64), ("h", c_i64), ("r", c_i64), ("s", ctypes.c_float), ("act", ctypes.c_int)]


class QkvWeights(ctypes.Structure):
    _fields_ = [("q", Nf4), ("k", Nf4), ("v", Nf4),
                ("a_q", c_vp), ("b_q", c_vp), ("a_k", c_vp), ("b_k", c_vp), ("a_v", c_vp),
                ("b_v", c_vp), ("r", c_i64), ("s", ctypes.c_float)]


class Qkv16Weights(ctypes.Structure):
    _fields_ = [("q", c_vp), ("k", c_vp), ("v", c_vp),
                ("d", c_i64), ("n_q", c_i64), ("n_k", c_i64), ("n_v", c_i64),
                ("a_q", c_vp), ("b_q", c_vp), ("a_k", c_vp), ("b_k", c_vp), ("a_v", c_vp),
                ("b_v", c_vp), ("r", c_i64), ("s", ctypes.c_float)]


class QkvGrads(ctypes.Structure):
    _fields_ = [("a_q", c_vp), ("b_q", c_vp), ("a_k", c_vp), ("b_k", c_vp), ("a_v", c_vp),
                ("b_v", c_vp)]


class MlpGrads(ctypes.Structure):
    _fields_ = [("a_gate", c_vp), ("b_gate", c_vp), ("a_up", c_vp), ("b_up", c_vp),
                ("a_down", c_vp), ("b_down", c_vp)]


_LIB = None


def lib() -> ctypes.CDLL:
    """Load the HIP library once; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m qlora_fine_tuning_amd.build` "
                "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        L.qlora_status_string.restype = ctypes.c_char_p
        L.qlora_status_string.argtypes = [ctypes.c_int]
        L.qlora_last_error.restype = ctypes.c_char_p
        L.qlora_last_error.argtypes = []
        L.qlora_version.restype = ctypes.c_char_p
        L.qlora_version.argtypes = []
        L.qlora_gemm_split_count.restype = ctypes.c_int
        L.qlora_gemm_split_count.argtypes = [ctypes.c_int64] * 3
        L.qlora_nf4_levels.restype = None
        L.qlora_nf4_levels.argtypes = [ctypes.POINTER(ctypes.c_float)]
        L.qlora_nf4_dequant.restype = ctypes.c_int
        L.qlora_nf4_dequant.argtypes = [Nf4, c_vp, c_vp]
        L.qlora_absmax_dq_quantize.restype = ctypes.c_int
        L.qlora_absmax_dq_quantize.argtypes = [c_vp, c_i64, c_vp, c_vp, c_vp, c_vp]
        L.qlora_absmax_dq_dequant.restype = ctypes.c_int
        L.qlora_absmax_dq_dequant.argtypes = [c_vp, c_vp, c_vp, c_i64, c_vp, c_vp]
        L.qlora_nf4_quantize.restype = ctypes.c_int
        L.qlora_nf4_quantize.argtypes = [c_vp, c_i64, c_i64, c_vp, c_vp, c_vp]
        L.qlora_linear_workspace_bytes.restype = ctypes.c_size_t
        L.qlora_linear_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, c_i64, ctypes.c_int]
        L.qlora_linear_fwd.restype = ctypes.c_int
        L.qlora_linear_fwd.argtypes = [c_vp, c_i64, Nf4, c_vp, c_vp, c_i64, ctypes.c_float,
                                       c_vp, c_vp, ctypes.c_int, c_vp, ctypes.c_size_t, c_vp]
        L.qlora_linear_fwd_noalloc_max_bytes.restype = ctypes.c_size_t
        L.qlora_linear_fwd_noalloc_max_bytes.argtypes = []
        L.qlora_linear_fwd_noalloc.restype = ctypes.c_int
        L.qlora_linear_fwd_noalloc.argtypes = [c_vp, c_i64, Nf4, c_vp, c_vp, c_i64, ctypes.c_float,
                                               c_vp, c_vp, ctypes.c_int, c_vp]
        L.qlora_linear_bwd.restype = ctypes.c_int
        L.qlora_linear_bwd.argtypes = [c_vp, c_vp, c_vp, c_i64, Nf4, c_vp, c_vp, c_i64,
                                       ctypes.c_float, c_vp, c_vp, c_vp, ctypes.c_int, c_vp,
                                       ctypes.c_size_t, c_vp]
        L.qlora_mlp_workspace_bytes.restype = ctypes.c_size_t
        L.qlora_mlp_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, c_i64, ctypes.c_int]
        L.qlora_mlp_fwd.restype = ctypes.c_int
        L.qlora_mlp_fwd.argtypes = [c_vp, c_i64, ctypes.POINTER(MlpWeights), c_vp, c_vp, c_vp,
                                    c_vp, c_vp, c_vp, ctypes.c_int, c_vp, ctypes.c_size_t, c_vp]
        L.qlora_mlp_bwd.restype = ctypes.c_int
        L.qlora_mlp_bwd.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64,
                                    ctypes.POINTER(MlpWeights), c_vp, ctypes.POINTER(MlpGrads),
                                    ctypes.c_int, c_vp, ctypes.c_size_t, c_vp]
        L.qlora_linear16_workspace_bytes.restype = ctypes.c_size_t
        L.qlora_linear16_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, c_i64]
        L.qlora_linear16_fwd.restype = ctypes.c_int
        L.qlora_linear16_fwd.argtypes = [c_vp, c_i64, c_vp, c_i64, c_i64, c_vp, c_vp, c_i64,
                                         ctypes.c_float, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]
        L.qlora_linear16_bwd.restype = ctypes.c_int
        L.qlora_linear16_bwd.argtypes = [c_vp, c_vp, c_vp, c_i64, c_vp, c_i64, c_i64, c_vp, c_vp,
                                         c_i64, ctypes.c_float, c_vp, c_vp, c_vp, c_vp,
                                         ctypes.c_size_t, c_vp]
        L.qlora_mlp16_workspace_bytes.restype = ctypes.c_size_t
        L.qlora_mlp16_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, c_i64]
        L.qlora_mlp16_fwd.restype = ctypes.c_int
        L.qlora_mlp16_fwd.argtypes = [c_vp, c_i64, ctypes.POINTER(Mlp16Weights), c_vp, c_vp, c_vp,
                                      c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]
        L.qlora_mlp16_bwd.restype = ctypes.c_int
        L.qlora_mlp16_bwd.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64,
                                      ctypes.POINTER(Mlp16Weights), c_vp, ctypes.POINTER(MlpGrads),
                                      c_vp, ctypes.c_size_t, c_vp]
        L.qlora_qkv_workspace_bytes.restype = ctypes.c_size_t
        L.qlora_qkv_workspace_bytes.argtypes = [c_i64] * 6
        for name, wt in (("qlora_qkv_fwd", QkvWeights), ("qlora_qkv16_fwd", Qkv16Weights)):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [c_vp, c_i64, ctypes.POINTER(wt), c_vp, c_i64, c_vp, c_i64, c_vp, c_i64,
                          c_vp, c_vp, ctypes.c_size_t, c_vp]
        for name, wt in (("qlora_qkv_bwd", QkvWeights), ("qlora_qkv16_bwd", Qkv16Weights)):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [c_vp, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_i64,
                          ctypes.POINTER(wt), c_vp, ctypes.POINTER(QkvGrads), c_vp,
                          ctypes.c_size_t, c_vp]
        c_f = ctypes.c_float
        for name, args in (
                ("qlora_rmsnorm_fwd", [c_vp, c_i64, c_i64, c_vp, c_f, ctypes.c_int, c_vp, c_vp, c_vp]),
                ("qlora_rmsnorm_bwd", [c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, ctypes.c_int, c_vp, c_vp]),
                ("qlora_rope_fwd", [c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_f, c_vp, c_i64, c_vp]),
                ("qlora_rope_bwd", [c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_f, c_vp, c_i64, c_vp]),
                ("qlora_cross_entropy_fwd", [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp,
                                             c_vp]),
                ("qlora_cross_entropy_bwd", [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp,
                                             c_i64, c_vp]),
                ("qlora_cross_entropy_fused", [c_vp, c_i64, c_i64, c_i64, c_vp, c_f, c_vp, c_vp, c_vp,
                                               c_vp, c_vp, c_i64, c_vp])):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = args
        L.qlora_probe_mfma_peak.restype = ctypes.c_int
        L.qlora_probe_mfma_peak.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                            ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
        L.qlora_trace_enable.restype = ctypes.c_int
        L.qlora_trace_enable.argtypes = [ctypes.c_int]
        L.qlora_trace_read.restype = ctypes.c_int
        L.qlora_trace_read.argtypes = [ctypes.POINTER(c_i64), ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_double)]
        _LIB = L
    return _LIB


def check(status: int, what: str) -> None:
    if status != QLORA_OK:
        L = lib()
        msg = L.qlora_status_string(status).decode()
        extra = L.qlora_last_error().decode() if status == -4 else ""
        raise RuntimeError(f"{what}: {STATUS.get(status, status)}: {msg} {extra}".strip())


EXPORTED = [
    "qlora_status_string", "qlora_last_error", "qlora_version", "qlora_nf4_levels",
    "qlora_gemm_split_count",
    "qlora_nf4_dequant", "qlora_nf4_quantize", "qlora_absmax_dq_quantize", "qlora_absmax_dq_dequant", "qlora_linear_workspace_bytes", "qlora_linear_fwd", "qlora_linear_bwd",
    "qlora_linear_fwd_noalloc_max_bytes", "qlora_linear_fwd_noalloc",
    "qlora_mlp_workspace_bytes", "qlora_mlp_fwd", "qlora_mlp_bwd",
    "qlora_trace_enable", "qlora_trace_read", "qlora_probe_mfma_peak",
    "qlora_linear16_workspace_bytes", "qlora_linear16_fwd", "qlora_linear16_bwd",
    "qlora_mlp16_workspace_bytes", "qlora_mlp16_fwd", "qlora_mlp16_bwd",
    "qlora_qkv_workspace_bytes", "qlora_qkv_fwd", "qlora_qkv_bwd", "qlora_qkv16_fwd",
    "qlora_qkv16_bwd", "qlora_rmsnorm_fwd", "qlora_rmsnorm_bwd", "qlora_rope_fwd", "qlora_rope_bwd",
    "qlora_cross_entropy_fwd", "qlora_cross_entropy_bwd", "qlora_cross_entropy_fused",
]
