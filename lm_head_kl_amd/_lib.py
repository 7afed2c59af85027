"""ctypes loader for libkdkl.so and the C structures of include/kdkl.h.

Loading needs no GPU: the library links the HIP runtime, which is installed on every host
of this image. Compute calls need a gfx950 device.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkdkl.so")

KD_FP32, KD_BF16 = 0, 1
KD_VALIDATE_IDX, KD_ACCUMULATE_DW, KD_SKIP_DW, KD_LOW_MEMORY = 0x1, 0x2, 0x4, 0x8
KD_NOALLOC_SCRATCH_BYTES = 64 << 20

STATUS = {
    0: "KD_OK",
    1: "KD_ERR_NULL",
    2: "KD_ERR_SHAPE",
    3: "KD_ERR_DTYPE",
    4: "KD_ERR_VALUE",
    5: "KD_ERR_WORKSPACE",
    6: "KD_ERR_INDEX",
    7: "KD_ERR_HIP",
    8: "KD_ERR_INTERNAL",
}

# Every symbol include/kdkl.h declares.
EXPORTS = (
    "kd_abi_version",
    "kd_status_str",
    "kd_fused_workspace_bytes",
    "kd_fused_kl_fwd",
    "kd_fused_kl_fwd_noalloc",
    "kd_fused_kl_bwd",
    "kd_dense_workspace_bytes",
    "kd_dense_kl",
    "kd_chunked_workspace_bytes",
    "kd_chunked_kl",
    "kd_chunked_logits",
    "kd_fused_fwdbwd_workspace_bytes",
    "kd_fused_kl_fwdbwd",
    "kd_topk_cache",
    "kd_validate_ids",
    "kd_timing_enable",
    "kd_timing_kinds",
    "kd_timing_name",
    "kd_timing_read",
    "kd_timing_reset",
)


class KdProblem(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int64),
        ("d", ctypes.c_int64),
        ("V", ctypes.c_int64),
        ("K", ctypes.c_int64),
        ("chunk", ctypes.c_int64),
        ("T", ctypes.c_float),
        ("n_norm", ctypes.c_float),
        ("act", ctypes.c_int32),
        ("tlogit", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


class KdError(RuntimeError):
    def __init__(self, code: int, where: str, text: str):
        super().__init__(f"{where}: {STATUS.get(code, code)} ({text})")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library. Raises if it has not been built: there is no fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libkdkl.so not found at {LIB_PATH}; build it with "
                          f"`python -m lm_head_kl_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, P = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(KdProblem)
    L.kd_abi_version.restype = ctypes.c_int
    L.kd_abi_version.argtypes = []
    L.kd_status_str.restype = ctypes.c_char_p
    L.kd_status_str.argtypes = [ctypes.c_int]
    L.kd_fused_workspace_bytes.restype = sz
    L.kd_fused_workspace_bytes.argtypes = [P]
    L.kd_dense_workspace_bytes.restype = sz
    L.kd_dense_workspace_bytes.argtypes = [P]
    L.kd_fused_kl_fwd.restype = ctypes.c_int
    L.kd_fused_kl_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.kd_fused_kl_fwd_noalloc.restype = ctypes.c_int
    L.kd_fused_kl_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.kd_fused_kl_bwd.restype = ctypes.c_int
    L.kd_fused_kl_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.kd_dense_kl.restype = ctypes.c_int
    L.kd_dense_kl.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    for name in ("kd_chunked_workspace_bytes", "kd_fused_fwdbwd_workspace_bytes"):
        getattr(L, name).restype = sz
        getattr(L, name).argtypes = [P]
    for name in ("kd_chunked_kl", "kd_fused_kl_fwdbwd"):
        getattr(L, name).restype = ctypes.c_int
        getattr(L, name).argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    i64 = ctypes.c_int64
    L.kd_chunked_logits.restype = ctypes.c_int
    L.kd_chunked_logits.argtypes = [P, vp, sz, ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(i64)]
    L.kd_topk_cache.restype = ctypes.c_int
    L.kd_topk_cache.argtypes = [vp, ctypes.c_int32, i64, i64, i64, i64, vp, vp, vp]
    L.kd_validate_ids.restype = ctypes.c_int
    L.kd_validate_ids.argtypes = [vp, i64, i64, i64, vp, vp]
    L.kd_timing_enable.restype = ctypes.c_int
    L.kd_timing_enable.argtypes = [ctypes.c_int]
    L.kd_timing_kinds.restype = ctypes.c_int
    L.kd_timing_kinds.argtypes = []
    L.kd_timing_name.restype = ctypes.c_char_p
    L.kd_timing_name.argtypes = [ctypes.c_int]
    L.kd_timing_read.restype = ctypes.c_int
    L.kd_timing_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]
    L.kd_timing_reset.restype = None
    L.kd_timing_reset.argtypes = []
    _lib = L
    return L


def check(code: int, where: str) -> None:
    if code != 0:
        raise KdError(code, where, lib().kd_status_str(code).decode())
