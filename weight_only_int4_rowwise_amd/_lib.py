"""ctypes loader for libw4a16.so (the gfx950 HIP library).

There is no fallback: if the library is missing or cannot be loaded, every
entry point raises.  Build it with ``python -m weight_only_int4_rowwise_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libw4a16.so")

# Status codes of include/w4a16.h
OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_HIP, ERR_DEVICE = range(6)

# Every symbol include/w4a16.h, include/w8a16.h and include/w4a16_zp.h declare.
EXPORTS = (
    "quantize_rowwise_int4",
    "w4a16_linear",
    "w4a16_geglu_linear",
    "w4a16_prepacked_bytes",
    "w4a16_prepack",
    "w4a16_linear_prepacked",
    "w4a16_geglu_linear_prepacked",
    "w4a16_status_string",
    "w4a16_last_error",
    "w4a16_abi_version",
    "quantize_rowwise_int8",
    "w8a16_linear",
    "w8a16_geglu_linear",
    "w8a16_prepacked_bytes",
    "w8a16_prepack",
    "w8a16_linear_prepacked",
    "w8a16_geglu_linear_prepacked",
    "quantize_rowwise_int4_zp",
    "w4a16_zp_linear",
    "w4a16_zp_geglu_linear",
    "w4a16_zp_linear_prepacked",
    "w4a16_zp_geglu_linear_prepacked",
    "w4a16_read_probe",
)

ABI_VERSION = 1

_lib = None


class W4A16Error(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        msg = f"{where}: status {status}"
        if _lib is not None:
            msg += f" ({_lib.w4a16_status_string(status).decode()})"
        if detail:
            msg += f": {detail}"
        super().__init__(msg)


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m weight_only_int4_rowwise_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I = ctypes.c_void_p, ctypes.c_int64
    lib.quantize_rowwise_int4.argtypes = [P, I, I, P, P, P]
    lib.quantize_rowwise_int4.restype = ctypes.c_int
    lib.w4a16_linear.argtypes = [P, I, I, P, P, I, P, P, P]
    lib.w4a16_linear.restype = ctypes.c_int
    lib.w4a16_geglu_linear.argtypes = [P, I, I, P, P, I, P, P, P]
    lib.w4a16_geglu_linear.restype = ctypes.c_int
    lib.w4a16_prepacked_bytes.argtypes = [I, I]
    lib.w4a16_prepacked_bytes.restype = ctypes.c_int64
    lib.w4a16_prepack.argtypes = [P, I, I, P, P]
    lib.w4a16_prepack.restype = ctypes.c_int
    lib.w4a16_linear_prepacked.argtypes = [P, I, I, P, P, I, P, P, P]
    lib.w4a16_linear_prepacked.restype = ctypes.c_int
    lib.w4a16_geglu_linear_prepacked.argtypes = [P, I, I, P, P, I, P, P, P]
    lib.w4a16_geglu_linear_prepacked.restype = ctypes.c_int
    lib.quantize_rowwise_int8.argtypes = [P, I, I, P, P, P]
    lib.quantize_rowwise_int8.restype = ctypes.c_int
    for fn in ("w8a16_linear", "w8a16_geglu_linear", "w8a16_linear_prepacked",
               "w8a16_geglu_linear_prepacked"):
        getattr(lib, fn).argtypes = [P, I, I, P, P, I, P, P, P]
        getattr(lib, fn).restype = ctypes.c_int
    lib.w8a16_prepacked_bytes.argtypes = [I, I]
    lib.w8a16_prepacked_bytes.restype = ctypes.c_int64
    lib.w8a16_prepack.argtypes = [P, I, I, P, P]
    lib.w8a16_prepack.restype = ctypes.c_int
    lib.quantize_rowwise_int4_zp.argtypes = [P, I, I, P, P, P, P]
    lib.quantize_rowwise_int4_zp.restype = ctypes.c_int
    for fn in ("w4a16_zp_linear", "w4a16_zp_geglu_linear", "w4a16_zp_linear_prepacked",
               "w4a16_zp_geglu_linear_prepacked"):
        getattr(lib, fn).argtypes = [P, I, I, P, P, P, I, P, P, P]
        getattr(lib, fn).restype = ctypes.c_int
    lib.w4a16_read_probe.argtypes = [P, I, P, P]
    lib.w4a16_read_probe.restype = ctypes.c_int
    lib.w4a16_status_string.argtypes = [ctypes.c_int]
    lib.w4a16_status_string.restype = ctypes.c_char_p
    lib.w4a16_last_error.argtypes = []
    lib.w4a16_last_error.restype = ctypes.c_char_p
    lib.w4a16_abi_version.argtypes = []
    lib.w4a16_abi_version.restype = ctypes.c_int
    if lib.w4a16_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH}: ABI version {lib.w4a16_abi_version()} != {ABI_VERSION}")
    _lib = lib
    return lib


def check(status: int, where: str) -> None:
    if status != OK:
        detail = _lib.w4a16_last_error().decode() if status in (ERR_HIP, ERR_DEVICE) else ""
        raise W4A16Error(status, where, detail)
