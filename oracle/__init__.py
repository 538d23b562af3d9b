"""CPU oracle for weight-only INT4 row-wise quantization and the W4A16 linear,
for the INT8 row-wise variant (W8A16: divisor 127, one code per byte), and for
the zero-point INT4 variant (min/max range, 15 steps, integer zero point).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only users.  The GPU library never imports, links or
calls this package, and this package imports nothing from it.

The arithmetic lives in ``w4a16_oracle.c`` (plain C, binary64, plain loops),
built with gcc by :func:`build`.  This module only marshals numpy arrays.
All fp16 tensors cross the boundary as their raw uint16 bit patterns.

Sources: the GLM-130B paper card (wikillm.com), sections "Method" (weight-only
INT4 quantization and its forward pseudocode), "Paper vs code" (scale divisor
2^(b-1)-1 = 7 computed per output row in FP16, int8 packing) and
"Hyperparameters" (GeGLU FFN); the paperlayer.ai summary, "INT4 Quantization
for RTX 3090s/2080s" (FP16 activations, weights turned back into FP16 at run
time) and section B.3 (GeGLU).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4a16_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

ERRORS = {
    0: "ok",
    1: "bad argument",
    2: "non-finite weight",
    3: "odd row length",
    4: "host FPU not in round-to-nearest-even",
}


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (no HIP, no shared code with the GPU path)."""
    stale = (not os.path.exists(_LIB_PATH)
             or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC))
    if force or stale:
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        build(force=False)                 # compiles only if missing or older than the source
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_half_to_double.restype = ctypes.c_double
        lib.oracle_double_to_half.argtypes = [ctypes.c_double]
        lib.oracle_double_to_half.restype = ctypes.c_uint16
        lib.oracle_gelu.argtypes = [ctypes.c_double]
        lib.oracle_gelu.restype = ctypes.c_double
        lib.oracle_gelu_n.argtypes = [P, I, P]
        lib.oracle_quantize_codes.argtypes = [P, I, I, P, P]
        lib.oracle_quantize_rowwise_int4.argtypes = [P, I, I, P, P]
        lib.oracle_unpack_int4.argtypes = [P, I, I, P]
        lib.oracle_linear.argtypes = [P, I, I, P, P, I, P, P, P]
        lib.oracle_linear_at.argtypes = [P, I, P, P, P, P, P, I, P, P]
        lib.oracle_geglu.argtypes = [P, I, I, P, P, I, P, P, P, P, P, P]
        lib.oracle_geglu_at.argtypes = [P, I, P, P, I, P, P, P, I, P, P, P, P, P]
        lib.oracle_quantize_rowwise_int8.argtypes = [P, I, I, P, P]
        lib.oracle_linear_int8.argtypes = [P, I, I, P, P, I, P, P, P]
        lib.oracle_linear_int8_at.argtypes = [P, I, P, P, P, P, P, I, P, P]
        lib.oracle_geglu_int8.argtypes = [P, I, I, P, P, I, P, P, P, P, P, P]
        lib.oracle_geglu_int8_at.argtypes = [P, I, P, P, I, P, P, P, I, P, P, P, P, P]
        lib.oracle_quantize_codes_zp.argtypes = [P, I, I, P, P, P]
        lib.oracle_quantize_rowwise_int4_zp.argtypes = [P, I, I, P, P, P]
        lib.oracle_linear_zp.argtypes = [P, I, I, P, P, P, I, P, P, P]
        lib.oracle_geglu_zp.argtypes = [P, I, I, P, P, P, I, P, P, P, P, P, P]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(st):
    if st != 0:
        raise OracleError(ERRORS.get(st, f"status {st}"))


def _bits16(a) -> np.ndarray:
    """fp16 data as a C-contiguous uint16 array of its bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected float16 or uint16 bit patterns, got {a.dtype}")
    return np.ascontiguousarray(a)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def half_to_double(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.oracle_half_to_double(int(v)) for v in b], dtype=np.float64)


def double_to_half(values) -> np.ndarray:
    lib = _load()
    v = np.asarray(values, dtype=np.float64).ravel()
    return np.array([lib.oracle_double_to_half(float(t)) for t in v], dtype=np.uint16)


def gelu(t: float) -> float:
    return float(_load().oracle_gelu(float(t)))


def gelu_n(t) -> np.ndarray:
    """GELU of every entry of a float64 array (same shape)."""
    t = np.ascontiguousarray(t, dtype=np.float64)
    out = np.empty_like(t)
    _load().oracle_gelu_n(_ptr(t), t.size, _ptr(out))
    return out


def quantize_codes(w):
    """W fp16 [n][k] -> (codes int8 [n][k], scale bits uint16 [n])."""
    w = _bits16(w)
    n, k = w.shape
    codes = np.empty((n, k), dtype=np.int8)
    scales = np.empty(n, dtype=np.uint16)
    _check(_load().oracle_quantize_codes(_ptr(w), n, k, _ptr(codes), _ptr(scales)))
    return codes, scales


def quantize_rowwise_int4(w):
    """W fp16 [n][k] -> (packed uint8 [n][k/2], scale bits uint16 [n])."""
    w = _bits16(w)
    n, k = w.shape
    packed = np.empty((n, k // 2), dtype=np.uint8)
    scales = np.empty(n, dtype=np.uint16)
    _check(_load().oracle_quantize_rowwise_int4(_ptr(w), n, k, _ptr(packed), _ptr(scales)))
    return packed, scales


def unpack_int4(packed, k: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    codes = np.empty((n, k), dtype=np.int8)
    _check(_load().oracle_unpack_int4(_ptr(packed), n, k, _ptr(codes)))
    return codes


def linear(x, packed, scales, bias=None):
    """y = x . (s*q)^T (+ bias) in binary64.  Returns (y [m][n], mag [m][n])."""
    x = _bits16(x)
    m, k = x.shape
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = _bits16(scales)
    n = packed.shape[0]
    if packed.shape[1] * 2 != k or scales.shape[0] != n:
        raise ValueError("shape mismatch")
    b = None if bias is None else _bits16(bias)
    y = np.empty((m, n), dtype=np.float64)
    mag = np.empty((m, n), dtype=np.float64)
    _check(_load().oracle_linear(_ptr(x), m, k, _ptr(packed), _ptr(scales), n,
                                 _ptr(b), _ptr(y), _ptr(mag)))
    return y, mag


def linear_at(x, packed, scales, mi, ni, bias=None):
    """Selected outputs y[mi[t], ni[t]] in binary64.  Returns (y, mag)."""
    x = _bits16(x)
    k = x.shape[1]
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = _bits16(scales)
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    if mi.shape != ni.shape:
        raise ValueError("index shape mismatch")
    if mi.size and (mi.min() < 0 or mi.max() >= x.shape[0] or ni.min() < 0 or ni.max() >= packed.shape[0]):
        raise IndexError("output index out of range")
    b = None if bias is None else _bits16(bias)
    y = np.empty(mi.shape, dtype=np.float64)
    mag = np.empty(mi.shape, dtype=np.float64)
    _check(_load().oracle_linear_at(_ptr(x), k, _ptr(packed), _ptr(scales), _ptr(b),
                                    _ptr(mi), _ptr(ni), mi.size, _ptr(y), _ptr(mag)))
    return y, mag


def geglu(x, packed, scales, bias=None):
    """g = GELU(a) * b with a, b the two row halves.  Returns (g, a, b, mag_a, mag_b)."""
    x = _bits16(x)
    m, k = x.shape
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = _bits16(scales)
    two_f = packed.shape[0]
    if two_f % 2 or packed.shape[1] * 2 != k or scales.shape[0] != two_f:
        raise ValueError("shape mismatch")
    f = two_f // 2
    b = None if bias is None else _bits16(bias)
    outs = [np.empty((m, f), dtype=np.float64) for _ in range(5)]
    _check(_load().oracle_geglu(_ptr(x), m, k, _ptr(packed), _ptr(scales), f, _ptr(b),
                                *[_ptr(o) for o in outs]))
    return tuple(outs)


def geglu_at(x, packed, scales, mi, ni, bias=None):
    """Selected GeGLU outputs g[mi[t], ni[t]].  Returns (g, a, b, mag_a, mag_b)."""
    x = _bits16(x)
    k = x.shape[1]
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = _bits16(scales)
    f = packed.shape[0] // 2
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    if mi.size and (mi.min() < 0 or mi.max() >= x.shape[0] or ni.min() < 0 or ni.max() >= f):
        raise IndexError("output index out of range")
    b = None if bias is None else _bits16(bias)
    outs = [np.empty(mi.shape, dtype=np.float64) for _ in range(5)]
    _check(_load().oracle_geglu_at(_ptr(x), k, _ptr(packed), _ptr(scales), f, _ptr(b),
                                   _ptr(mi), _ptr(ni), mi.size, *[_ptr(o) for o in outs]))
    return tuple(outs)


# ------------------------------------------------------------ INT8 variant

def quantize_rowwise_int8(w):
    """W fp16 [n][k] -> (codes int8 [n][k], scale bits uint16 [n]); s = fp16(a/127)."""
    w = _bits16(w)
    n, k = w.shape
    codes = np.empty((n, k), dtype=np.int8)
    scales = np.empty(n, dtype=np.uint16)
    _check(_load().oracle_quantize_rowwise_int8(_ptr(w), n, k, _ptr(codes), _ptr(scales)))
    return codes, scales


def _codes8(codes, k):
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    if codes.ndim != 2 or codes.shape[1] != k:
        raise ValueError("INT8 codes must be [rows][k]")
    return codes


def linear_int8(x, codes, scales, bias=None):
    """y = x . (s*q)^T (+ bias) over INT8 codes, binary64.  Returns (y, mag)."""
    x = _bits16(x)
    m, k = x.shape
    codes = _codes8(codes, k)
    scales = _bits16(scales)
    n = codes.shape[0]
    if scales.shape[0] != n:
        raise ValueError("shape mismatch")
    b = None if bias is None else _bits16(bias)
    y = np.empty((m, n), dtype=np.float64)
    mag = np.empty((m, n), dtype=np.float64)
    _check(_load().oracle_linear_int8(_ptr(x), m, k, _ptr(codes), _ptr(scales), n,
                                      _ptr(b), _ptr(y), _ptr(mag)))
    return y, mag


def linear_int8_at(x, codes, scales, mi, ni, bias=None):
    """Selected outputs y[mi[t], ni[t]] over INT8 codes.  Returns (y, mag)."""
    x = _bits16(x)
    k = x.shape[1]
    codes = _codes8(codes, k)
    scales = _bits16(scales)
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    if mi.shape != ni.shape:
        raise ValueError("index shape mismatch")
    if mi.size and (mi.min() < 0 or mi.max() >= x.shape[0] or ni.min() < 0 or ni.max() >= codes.shape[0]):
        raise IndexError("output index out of range")
    b = None if bias is None else _bits16(bias)
    y = np.empty(mi.shape, dtype=np.float64)
    mag = np.empty(mi.shape, dtype=np.float64)
    _check(_load().oracle_linear_int8_at(_ptr(x), k, _ptr(codes), _ptr(scales), _ptr(b),
                                         _ptr(mi), _ptr(ni), mi.size, _ptr(y), _ptr(mag)))
    return y, mag


def geglu_int8(x, codes, scales, bias=None):
    """GeGLU over INT8 codes [2f][k].  Returns (g, a, b, mag_a, mag_b)."""
    x = _bits16(x)
    m, k = x.shape
    codes = _codes8(codes, k)
    scales = _bits16(scales)
    two_f = codes.shape[0]
    if two_f % 2 or scales.shape[0] != two_f:
        raise ValueError("shape mismatch")
    f = two_f // 2
    b = None if bias is None else _bits16(bias)
    outs = [np.empty((m, f), dtype=np.float64) for _ in range(5)]
    _check(_load().oracle_geglu_int8(_ptr(x), m, k, _ptr(codes), _ptr(scales), f, _ptr(b),
                                     *[_ptr(o) for o in outs]))
    return tuple(outs)


def geglu_int8_at(x, codes, scales, mi, ni, bias=None):
    """Selected GeGLU outputs over INT8 codes.  Returns (g, a, b, mag_a, mag_b)."""
    x = _bits16(x)
    k = x.shape[1]
    codes = _codes8(codes, k)
    scales = _bits16(scales)
    f = codes.shape[0] // 2
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    if mi.size and (mi.min() < 0 or mi.max() >= x.shape[0] or ni.min() < 0 or ni.max() >= f):
        raise IndexError("output index out of range")
    b = None if bias is None else _bits16(bias)
    outs = [np.empty(mi.shape, dtype=np.float64) for _ in range(5)]
    _check(_load().oracle_geglu_int8_at(_ptr(x), k, _ptr(codes), _ptr(scales), f, _ptr(b),
                                        _ptr(mi), _ptr(ni), mi.size, *[_ptr(o) for o in outs]))
    return tuple(outs)


# ------------------------------------------------------ zero-point INT4

def quantize_codes_zp(w):
    """W fp16 [n][k] -> (codes uint8 [n][k] in [0, 15], scale bits uint16 [n], zero points uint8 [n])."""
    w = _bits16(w)
    n, k = w.shape
    codes = np.empty((n, k), dtype=np.uint8)
    scales = np.empty(n, dtype=np.uint16)
    zeros = np.empty(n, dtype=np.uint8)
    _check(_load().oracle_quantize_codes_zp(_ptr(w), n, k, _ptr(codes), _ptr(scales), _ptr(zeros)))
    return codes, scales, zeros


def quantize_rowwise_int4_zp(w):
    """W fp16 [n][k] -> (packed uint8 [n][k/2], scale bits uint16 [n], zero points uint8 [n])."""
    w = _bits16(w)
    n, k = w.shape
    packed = np.empty((n, k // 2), dtype=np.uint8)
    scales = np.empty(n, dtype=np.uint16)
    zeros = np.empty(n, dtype=np.uint8)
    _check(_load().oracle_quantize_rowwise_int4_zp(_ptr(w), n, k, _ptr(packed), _ptr(scales), _ptr(zeros)))
    return packed, scales, zeros


def linear_zp(x, packed, scales, zeros, bias=None):
    """y = x . (s*(q - z))^T (+ bias) in binary64.  Returns (y, mag)."""
    x = _bits16(x)
    m, k = x.shape
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = _bits16(scales)
    zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
    n = packed.shape[0]
    if packed.shape[1] * 2 != k or scales.shape[0] != n or zeros.shape[0] != n:
        raise ValueError("shape mismatch")
    b = None if bias is None else _bits16(bias)
    y = np.empty((m, n), dtype=np.float64)
    mag = np.empty((m, n), dtype=np.float64)
    _check(_load().oracle_linear_zp(_ptr(x), m, k, _ptr(packed), _ptr(scales), _ptr(zeros), n,
                                    _ptr(b), _ptr(y), _ptr(mag)))
    return y, mag


def geglu_zp(x, packed, scales, zeros, bias=None):
    """GeGLU over zero-point codes [2f][k/2].  Returns (g, a, b, mag_a, mag_b)."""
    x = _bits16(x)
    m, k = x.shape
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = _bits16(scales)
    zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
    two_f = packed.shape[0]
    if two_f % 2 or packed.shape[1] * 2 != k or scales.shape[0] != two_f or zeros.shape[0] != two_f:
        raise ValueError("shape mismatch")
    f = two_f // 2
    b = None if bias is None else _bits16(bias)
    outs = [np.empty((m, f), dtype=np.float64) for _ in range(5)]
    _check(_load().oracle_geglu_zp(_ptr(x), m, k, _ptr(packed), _ptr(scales), _ptr(zeros), f,
                                   _ptr(b), *[_ptr(o) for o in outs]))
    return tuple(outs)


# Acceptance bound for a linear output, as fixed for this method: an error of
# at most 2e-3 of the absolute-value sum of the terms, plus 1e-4.
LINEAR_REL = 2e-3
LINEAR_ABS = 1e-4


def linear_bound(mag):
    return LINEAR_REL * np.asarray(mag) + LINEAR_ABS


def geglu_bound(g_ref, a_ref, b_ref, mag_a, mag_b):
    """Bound for g = GELU(a)*b computed from a and b that each carry at most
    their linear bound eps_a, eps_b of error.

    With a' = a + da, b' = b + db (|da| <= eps_a, |db| <= eps_b):
    GELU(a')b' - GELU(a)b = (GELU(a') - GELU(a))b' + GELU(a)(b' - b), and by
    the mean value theorem |GELU(a') - GELU(a)| <= 1.13 eps_a, since
    |GELU'| = |Phi(t) + t phi(t)| <= 1.13 on the real line.  So
    |g' - g| <= 1.13|b|eps_a + |GELU(a)|eps_b + 1.13 eps_a eps_b, plus the
    final fp16 rounding (2^-11 relative, taken as 2^-10 to cover fp32
    evaluation of GELU itself) and the 1e-4 floor."""
    ea = linear_bound(mag_a)
    eb = linear_bound(mag_b)
    return (1.13 * np.abs(b_ref) * ea + np.abs(gelu_n(a_ref)) * eb + 1.13 * ea * eb
            + 2.0 ** -10 * np.abs(g_ref) + LINEAR_ABS)
