"""ctypes declarations of liblbq's C ABI (include/lbq.h).

Loading fails loudly when the shared library has not been built: there is no
fallback implementation anywhere in the package.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblbq.so")

LBQ_MINMAX = 0
LBQ_NF4 = 1
LBQ_META_F32 = 0
LBQ_META_COMPACT = 1
LBQ_MAX_GROUP = 8

STATUS = {
    0: "LBQ_OK", 1: "LBQ_E_NULL", 2: "LBQ_E_SHAPE", 3: "LBQ_E_FORMAT", 4: "LBQ_E_ALIGN",
    5: "LBQ_E_WORKSPACE", 6: "LBQ_E_UNSUPPORTED", 7: "LBQ_E_HIP",
}
STATUS_CODE = {v: k for k, v in STATUS.items()}

EXPORTED = (
    "lbq_layout", "lbq_quantize", "lbq_dequant", "lbq_linear_workspace_bytes",
    "lbq_linear_fwd", "lbq_linear_fwd_noalloc", "lbq_linear_fwd_grouped_workspace_bytes", "lbq_linear_fwd_grouped",
    "lbq_linear_bwd_dx", "lbq_linear_bwd_dx_grouped", "lbq_lora_workspace_bytes", "lbq_lora_fwd",
    "lbq_lora_bwd_workspace_bytes", "lbq_lora_bwd",
    "lbq_serialized_bytes", "lbq_serialize", "lbq_blob_desc", "lbq_deserialize",
    "lbq_nf4_codebook", "lbq_strerror", "lbq_last_error_detail", "lbq_version",
)


class Desc(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("double_quant", ctypes.c_int32), ("dq_block", ctypes.c_int32),
                ("meta", ctypes.c_int32), ("n", ctypes.c_int64), ("k", ctypes.c_int64)]


class QTensor(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p),
                ("absmax", ctypes.c_void_p), ("absmax_q", ctypes.c_void_p),
                ("absmax_scale", ctypes.c_void_p), ("out_rows", ctypes.c_void_p)]


class Sizes(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_size_t), ("scales", ctypes.c_size_t), ("zeros", ctypes.c_size_t),
                ("absmax", ctypes.c_size_t), ("absmax_q", ctypes.c_size_t),
                ("absmax_scale", ctypes.c_size_t)]


class LbqError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{func}: {self.name}: {detail}")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m group_wise_minmax_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    DP, QP = ctypes.POINTER(Desc), ctypes.POINTER(QTensor)
    sig = {
        "lbq_layout": (I32, [DP, ctypes.POINTER(Sizes)]),
        "lbq_quantize": (I32, [DP, P, QP, P]),
        "lbq_dequant": (I32, [DP, QP, P, P]),
        "lbq_linear_workspace_bytes": (SZ, [DP, I64]),
        "lbq_linear_fwd": (I32, [DP, QP, P, I64, P, I64, P, SZ, P]),
        "lbq_linear_fwd_noalloc": (I32, [DP, QP, P, I64, P, I64, P]),
        "lbq_linear_fwd_grouped_workspace_bytes": (SZ, [I32, DP, I64]),
        "lbq_linear_fwd_grouped": (I32, [I32, DP, QP, P, I64, ctypes.POINTER(P), ctypes.POINTER(I64), P, SZ, P]),
        "lbq_linear_bwd_dx": (I32, [DP, QP, P, I64, P, P]),
        "lbq_linear_bwd_dx_grouped": (I32, [I32, DP, QP, ctypes.POINTER(P), I64, P, P]),
        "lbq_lora_workspace_bytes": (SZ, [DP, I64, I32]),
        "lbq_lora_fwd": (I32, [DP, QP, P, I64, P, P, I32, ctypes.c_float, P, I64, P, SZ, P]),
        "lbq_lora_bwd_workspace_bytes": (SZ, [DP, I64, I32]),
        "lbq_lora_bwd": (I32, [DP, QP, P, P, I64, P, P, I32, ctypes.c_float, P, P, P, P, SZ, P]),
        "lbq_serialized_bytes": (SZ, [DP]),
        "lbq_serialize": (I32, [DP, QP, P, SZ, P]),
        "lbq_blob_desc": (I32, [P, SZ, DP]),
        "lbq_deserialize": (I32, [P, SZ, QP, P]),
        "lbq_nf4_codebook": (None, [ctypes.POINTER(ctypes.c_float)]),
        "lbq_strerror": (ctypes.c_char_p, [I32]),
        "lbq_last_error_detail": (ctypes.c_char_p, []),
        "lbq_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def check(status: int, func: str) -> None:
    if status != 0:
        raise LbqError(status, func, lib.lbq_last_error_detail().decode())
