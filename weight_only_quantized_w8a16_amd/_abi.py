"""ctypes view of libqgemm.so (include/qgemm.h), with the same names.

Argument marshalling only: every computation runs in the library's HIP
kernels.  The library is loaded on first use; if it has not been built the
call fails loudly rather than falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqgemm.so")

QG_OK = 0
STATUS_NAMES = {
    0: "QG_OK", 1: "QG_ERR_NULL", 2: "QG_ERR_SHAPE", 3: "QG_ERR_GROUP", 4: "QG_ERR_DTYPE",
    5: "QG_ERR_ALIGN", 6: "QG_ERR_WORKSPACE", 7: "QG_ERR_UNSUPPORTED", 8: "QG_ERR_HIP",
    9: "QG_ERR_MODE",
}
QG_NONE, QG_BF16, QG_FP16, QG_FP32 = 0, 1, 2, 3
QG_W8A8_PER_TENSOR, QG_W8A8_PER_CHANNEL, QG_W8A8_PER_TOKEN = 0, 1, 2
QG_LAYOUT_PORTABLE, QG_LAYOUT_TILED = 0, 1
QG_MOE_NORM_NONE, QG_MOE_RENORMALIZE = 0, 1

_P = ctypes.c_void_p
_INT = ctypes.c_int
_SZ = ctypes.c_size_t
_ST = ctypes.c_int

# name -> (restype, argtypes), in the order of include/qgemm.h
SIGNATURES = {
    "qg_strerror": (ctypes.c_char_p, [_ST]),
    "qg_version": (_INT, []),
    "qg_set_override": (_ST, [ctypes.c_char_p]),
    "qrepack_w4": (_ST, [_P, _P, _INT, _INT, _P]),
    "qunrepack_w4": (_ST, [_P, _P, _INT, _INT, _P]),
    "qrepack_w8": (_ST, [_P, _P, _INT, _INT, _P]),
    "qunrepack_w8": (_ST, [_P, _P, _INT, _INT, _P]),
    "qrepack_w8_kn": (_ST, [_P, _P, _INT, _INT, _P]),
    "qunrepack_w8_kn": (_ST, [_P, _P, _INT, _INT, _P]),
    "qquantize_w4": (_ST, [_P, _P, _P, _P, _INT, _INT, _INT, _INT, _INT, _P]),
    "qdequant_w4": (_ST, [_P, _P, _P, _P, _INT, _INT, _INT, _INT, _INT, _P]),
    "qdequant_w8": (_ST, [_P, _P, _P, _INT, _INT, _INT, _INT, _INT, _P]),
    "qgemm_workspace_size": (_SZ, [_INT, _INT, _INT, _INT, _INT]),
    "qgemm_w4a16": (_ST, [_P, _P, _P, _P, _P, _P, _INT, _INT, _INT, _INT, _INT, _INT, _P, _SZ, _P]),
    "qgemm_w8a16": (_ST, [_P, _P, _P, _P, _P, _INT, _INT, _INT, _INT, _INT, _INT, _P, _SZ, _P]),
    "qgemm_w8a8_workspace_size": (_SZ, [_INT, _INT, _INT]),
    "qgemm_w8a8": (_ST, [_P, _P, _INT, _P, _P, _P, _INT, _INT, _INT, _INT, _P, _SZ, _P]),
    "qembed_w4": (_ST, [_P, _INT, _P, _INT, _P, _P, _P, _INT, _INT, _INT, _INT, _INT, _P]),
    "qembed_w8": (_ST, [_P, _INT, _P, _INT, _P, _P, _INT, _INT, _INT, _INT, _INT, _P]),
    "qg_read_probe_blocks": (_SZ, [_SZ]),
    "qg_read_probe": (_ST, [_P, _SZ, _P, _P]),
    "qg_lds_probe": (_ST, [ctypes.c_int, ctypes.c_int, ctypes.c_int, _P, _P]),
    "qmoe_workspace_size": (_SZ, [_INT, _INT, _INT, _INT, _INT]),
    "qmoe_grouped": (_ST, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _INT, _INT, _INT, _INT, _INT, _INT,
                           _INT, _P, _P, _P, _SZ, _P]),
    "qmoe_grouped_noalloc": (_ST, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _INT, _INT, _INT, _INT, _INT,
                                   _INT, _INT, _P, _P, _P]),
    "qmoe_grouped_ex": (_ST, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _INT, _INT, _INT,
                              _INT, _INT, _INT, _INT, _INT, _P, _P, _P, _SZ, _P]),
}

_lock = threading.Lock()
_lib = None


class QGemmError(RuntimeError):
    """A library call returned a non-OK status, or the library is missing."""

    def __init__(self, func: str, status: int, detail: str = ""):
        self.func = func
        self.status = status
        name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{func}: {name}" + (f" ({detail})" if detail else ""))


def lib() -> ctypes.CDLL:
    """The loaded libqgemm (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise QGemmError("load", -1, f"{LIB_PATH} is missing; build it with "
                                     "`python -m weight_only_quantized_w8a16_amd.build`")
                handle = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in SIGNATURES.items():
                    fn = getattr(handle, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = handle
    return _lib


def check(func: str, status: int) -> None:
    if status != QG_OK:
        msg = lib().qg_strerror(status)
        raise QGemmError(func, status, msg.decode() if msg else "")
