"""MI355X (gfx950) weight-only INT4 row-wise quantization and W4A16 linears.

GLM-130B's inference scheme (paper card on wikillm.com, "Method" and "Paper
vs code"): each FP16 weight matrix [out][in] gets one absmax/7 scale per
output row and integer codes in [-7, 7] packed two per byte; the linear layers
keep FP16 activations.  This package is a thin binding over the C ABI of
``include/w4a16.h`` (libw4a16.so, hand-written HIP kernels): it checks tensor
placement, allocates outputs with torch, and passes raw device pointers and
the current HIP stream.  Every step of the computation runs in the library.

    q, s = quantize_rowwise_int4(w)            # w: cuda fp16 [n][k]
    y = w4a16_linear(x, q, s, bias=None)       # x: cuda fp16 [m][k] -> [m][n]
    g = w4a16_geglu_linear(x, q, s)            # q: [2f][k/2] -> [m][f]

    qp = w4a16_prepack(q)                      # load-time tile layout, same bytes
    y = w4a16_linear_prepacked(x, qp, s)       # identical results, faster reads

The INT8 variant (W8A16, include/w8a16.h; the pages' b-bit scale with
b = 8: s = absmax / 127, one int8 code per weight) has the same calls:

    c, s = quantize_rowwise_int8(w)            # c: cuda int8 [n][k]
    y = w8a16_linear(x, c, s)
    y = w8a16_linear_prepacked(x, w8a16_prepack(c), s)

The zero-point INT4 variant (include/w4a16_zp.h; the scheme the pages compare
absmax with) adds uint8 zero points [n]; w4a16_prepack reorders its codes:

    q, s, z = quantize_rowwise_int4_zp(w)
    y = w4a16_zp_linear(x, q, s, z)
    y = w4a16_zp_linear_prepacked(x, w4a16_prepack(q), s, z)
"""
from __future__ import annotations

from . import _lib
from ._lib import W4A16Error

__all__ = [
    "quantize_rowwise_int4",
    "w4a16_linear",
    "w4a16_geglu_linear",
    "w4a16_prepacked_bytes",
    "w4a16_prepack",
    "w4a16_linear_prepacked",
    "w4a16_geglu_linear_prepacked",
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
    "read_probe",
    "W4A16Error",
    "library",
]


def library():
    """The loaded libw4a16.so (raises if it is not built)."""
    return _lib.load()


_torch_mod = None


def _torch():
    global _torch_mod
    if _torch_mod is None:
        import torch
        _torch_mod = torch
    return _torch_mod


def _require(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU (got {t.device}); there is no CPU path")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(t, dev, name, what):
    if t.get_device() != dev:
        raise ValueError(f"{what}: {name} on {t.device}, expected cuda:{dev}")


_stream_getter = None


def _raw_stream(dev):
    """Handle of the current stream of GPU `dev` (torch's current stream):
    torch's raw-handle query where it has one, else the Stream object's."""
    global _stream_getter
    if _stream_getter is None:
        torch = _torch()
        _stream_getter = getattr(torch._C, "_cuda_getCurrentRawStream", None) or \
            (lambda d: torch.cuda.current_stream(d).cuda_stream)
    return _stream_getter(dev)


def _launch(fn, dev, *args):
    """fn(*args, stream) with GPU `dev` current and its current stream."""
    torch = _torch()
    if torch.cuda.current_device() == dev:
        return fn(*args, _raw_stream(dev))
    with torch.cuda.device(dev):
        return fn(*args, _raw_stream(dev))


_PREPACKED_SIZES: dict = {}


def _prepacked_size(lib, rows, k, cb=4):
    """w4a16_prepacked_bytes (cb = 4) or w8a16_prepacked_bytes (cb = 8) of
    (rows, k), remembered per shape."""
    key = (rows, k, cb)
    size = _PREPACKED_SIZES.get(key)
    if size is None:
        fn = lib.w4a16_prepacked_bytes if cb == 4 else lib.w8a16_prepacked_bytes
        size = int(fn(rows, k))
        _PREPACKED_SIZES[key] = size
    return size


def quantize_rowwise_int4(w, q_out=None, s_out=None):
    """W fp16 [n][k] (k even) -> (packed uint8 [n][k/2], scales fp16 [n])."""
    torch = _torch()
    lib = _lib.load()
    _require(w, torch.float16, "w")
    if w.dim() != 2:
        raise ValueError("w must be 2-D [out_features][in_features]")
    n, k = w.shape
    if q_out is None:
        q_out = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    if s_out is None:
        s_out = torch.empty((n,), dtype=torch.float16, device=w.device)
    _require(q_out, torch.uint8, "q_out")
    _require(s_out, torch.float16, "s_out")
    if tuple(q_out.shape) != (n, k // 2) or tuple(s_out.shape) != (n,):
        raise ValueError("output shape mismatch")
    dev = w.get_device()
    _same_device(q_out, dev, "q_out", "quantize_rowwise_int4")
    _same_device(s_out, dev, "s_out", "quantize_rowwise_int4")
    st = _launch(lib.quantize_rowwise_int4, dev,
                 w.data_ptr(), n, k, q_out.data_ptr(), s_out.data_ptr())
    _lib.check(st, "quantize_rowwise_int4")
    return q_out, s_out


def _linear_common(x, q, s, bias, out_cols, rows, y_out, name, cb=4):
    torch = _torch()
    _require(x, torch.float16, "x")
    _require(q, torch.uint8 if cb == 4 else torch.int8, "q")
    _require(s, torch.float16, "s")
    if x.dim() != 2 or q.dim() != 2 or s.dim() != 1:
        raise ValueError(f"{name}: x [m][k], q [rows][{'k/2' if cb == 4 else 'k'}], s [rows] expected")
    m, k = x.shape
    if q.shape[0] != rows or q.shape[1] * 8 // cb != k or s.shape[0] != rows:
        raise ValueError(f"{name}: shape mismatch x {tuple(x.shape)} q {tuple(q.shape)} s {tuple(s.shape)}")
    dev = x.get_device()
    _same_device(q, dev, "q", name)
    _same_device(s, dev, "s", name)
    if bias is not None:
        _require(bias, torch.float16, "bias")
        if tuple(bias.shape) != (rows,):
            raise ValueError(f"{name}: bias must be fp16 [{rows}]")
        _same_device(bias, dev, "bias", name)
    if y_out is None:
        y_out = torch.empty((m, out_cols), dtype=torch.float16, device=x.device)
    _require(y_out, torch.float16, "y_out")
    if tuple(y_out.shape) != (m, out_cols):
        raise ValueError(f"{name}: y_out must be [{m}][{out_cols}]")
    _same_device(y_out, dev, "y_out", name)
    return m, k, y_out


def w4a16_linear(x, q, s, bias=None, y_out=None):
    """y[m][n] = fp16(s * (x . q^T) + bias): fp16 activations, INT4 weights."""
    lib = _lib.load()
    n = q.shape[0]
    m, k, y_out = _linear_common(x, q, s, bias, n, n, y_out, "w4a16_linear")
    st = _launch(lib.w4a16_linear, x.get_device(),
                 x.data_ptr(), m, k, q.data_ptr(), s.data_ptr(), n,
                 None if bias is None else bias.data_ptr(), y_out.data_ptr())
    _lib.check(st, "w4a16_linear")
    return y_out


def w4a16_geglu_linear(x, q, s, bias=None, y_out=None):
    """y[m][f] = fp16(GELU(a) * b), a / b the linears through rows [0,f) / [f,2f)."""
    lib = _lib.load()
    rows = q.shape[0]
    if rows % 2:
        raise ValueError("w4a16_geglu_linear: q must have an even number of rows (2f)")
    f = rows // 2
    m, k, y_out = _linear_common(x, q, s, bias, f, rows, y_out, "w4a16_geglu_linear")
    st = _launch(lib.w4a16_geglu_linear, x.get_device(),
                 x.data_ptr(), m, k, q.data_ptr(), s.data_ptr(), f,
                 None if bias is None else bias.data_ptr(), y_out.data_ptr())
    _lib.check(st, "w4a16_geglu_linear")
    return y_out


def w4a16_prepacked_bytes(n: int, k: int) -> int:
    """Bytes of the prepacked layout of an [n][k] weight (-1 for bad sizes)."""
    return int(_lib.load().w4a16_prepacked_bytes(int(n), int(k)))


def w4a16_prepack(q, q_out=None):
    """Row-major packed codes [n][k/2] -> prepacked tile layout (uint8, 1-D)."""
    torch = _torch()
    lib = _lib.load()
    _require(q, torch.uint8, "q")
    if q.dim() != 2:
        raise ValueError("q must be 2-D [n][k/2]")
    n, k = q.shape[0], 2 * q.shape[1]
    size = lib.w4a16_prepacked_bytes(n, k)
    if size < 0:
        raise ValueError(f"w4a16_prepack: bad shape n={n} k={k} (k % 32 must be 0)")
    if q_out is None:
        q_out = torch.empty((size,), dtype=torch.uint8, device=q.device)
    _require(q_out, torch.uint8, "q_out")
    if q_out.numel() != size or q_out.device != q.device:
        raise ValueError(f"w4a16_prepack: q_out must hold {size} bytes on {q.device}")
    st = _launch(lib.w4a16_prepack, q.get_device(), q.data_ptr(), n, k, q_out.data_ptr())
    _lib.check(st, "w4a16_prepack")
    return q_out


def _prepacked_common(x, qp, s, bias, out_cols, rows, y_out, name, cb=4):
    torch = _torch()
    lib = _lib.load()
    _require(x, torch.float16, "x")
    _require(qp, torch.uint8, "qp")
    _require(s, torch.float16, "s")
    if x.dim() != 2 or s.dim() != 1 or s.shape[0] != rows:
        raise ValueError(f"{name}: x [m][k] and s [{rows}] expected")
    m, k = x.shape
    size = _prepacked_size(lib, rows, k, cb)
    if size < 0 or qp.numel() != size:
        raise ValueError(f"{name}: prepacked weight must hold {size} bytes for {rows} x {k}")
    dev = x.get_device()
    _same_device(qp, dev, "qp", name)
    _same_device(s, dev, "s", name)
    if bias is not None:
        _require(bias, torch.float16, "bias")
        if tuple(bias.shape) != (rows,):
            raise ValueError(f"{name}: bias must be fp16 [{rows}]")
        _same_device(bias, dev, "bias", name)
    if y_out is None:
        y_out = torch.empty((m, out_cols), dtype=torch.float16, device=x.device)
    _require(y_out, torch.float16, "y_out")
    if tuple(y_out.shape) != (m, out_cols):
        raise ValueError(f"{name}: y_out must be [{m}][{out_cols}]")
    _same_device(y_out, dev, "y_out", name)
    return lib, m, k, y_out


def w4a16_linear_prepacked(x, qp, s, bias=None, y_out=None):
    """w4a16_linear with the weight in the prepacked layout (n = len(s))."""
    n = s.shape[0]
    lib, m, k, y_out = _prepacked_common(x, qp, s, bias, n, n, y_out, "w4a16_linear_prepacked")
    st = _launch(lib.w4a16_linear_prepacked, x.get_device(),
                 x.data_ptr(), m, k, qp.data_ptr(), s.data_ptr(), n,
                 None if bias is None else bias.data_ptr(), y_out.data_ptr())
    _lib.check(st, "w4a16_linear_prepacked")
    return y_out


def w4a16_geglu_linear_prepacked(x, qp, s, bias=None, y_out=None):
    """w4a16_geglu_linear with the weight in the prepacked layout (f = len(s) / 2)."""
    rows = s.shape[0]
    if rows % 2:
        raise ValueError("w4a16_geglu_linear_prepacked: s must have 2f entries")
    f = rows // 2
    lib, m, k, y_out = _prepacked_common(x, qp, s, bias, f, rows, y_out,
                                         "w4a16_geglu_linear_prepacked")
    st = _launch(lib.w4a16_geglu_linear_prepacked, x.get_device(),
                 x.data_ptr(), m, k, qp.data_ptr(), s.data_ptr(), f,
                 None if bias is None else bias.data_ptr(), y_out.data_ptr())
    _lib.check(st, "w4a16_geglu_linear_prepacked")
    return y_out


# --------------------------------------------------------------------------
# INT8 variant (include/w8a16.h)
# --------------------------------------------------------------------------

def quantize_rowwise_int8(w, q_out=None, s_out=None):
    """W fp16 [n][k] (k even) -> (codes int8 [n][k], scales fp16 [n]); s = fp16(absmax / 127)."""
    torch = _torch()
    lib = _lib.load()
    _require(w, torch.float16, "w")
    if w.dim() != 2:
        raise ValueError("w must be 2-D [out_features][in_features]")
    n, k = w.shape
    if q_out is None:
        q_out = torch.empty((n, k), dtype=torch.int8, device=w.device)
    if s_out is None:
        s_out = torch.empty((n,), dtype=torch.float16, device=w.device)
    _require(q_out, torch.int8, "q_out")
    _require(s_out, torch.float16, "s_out")
    if tuple(q_out.shape) != (n, k) or tuple(s_out.shape) != (n,):
        raise ValueError("output shape mismatch")
    dev = w.get_device()
    _same_device(q_out, dev, "q_out", "quantize_rowwise_int8")
    _same_device(s_out, dev, "s_out", "quantize_rowwise_int8")
    st = _launch(lib.quantize_rowwise_int8, dev, w.data_ptr(), n, k, q_out.data_ptr(),
                 s_out.data_ptr())
    _lib.check(st, "quantize_rowwise_int8")
    return q_out, s_out


def w8a16_linear(x, q, s, bias=None, y_out=None):
    """y[m][n] = fp16(s * (x . q^T) + bias) over INT8 codes q [n][k]."""
    lib = _lib.load()
    n = q.shape[0]
    m, k, y_out = _linear_common(x, q, s, bias, n, n, y_out, "w8a16_linear", cb=8)
    st = _launch(lib.w8a16_linear, x.get_device(),
                 x.data_ptr(), m, k, q.data_ptr(), s.data_ptr(), n,
                 None if bias is None else bias.data_ptr(), y_out.data_ptr())
    _lib.check(st, "w8a16_linear")
    return y_out


def w8a16_geglu_linear(x, q, s, bias=None, y_out=None):
    """GeGLU over INT8 codes q [2f][k]: y[m][f] = fp16(GELU(a) * b)."""
    lib = _lib.load()
    rows = q.shape[0]
    if rows % 2:
        raise ValueError("w8a16_geglu_linear: q must have an even number of rows (2f)")
    f = rows // 2
    m, k, y_out = _linear_common(x, q, s, bias, f, rows, y_out, "w8a16_geglu_linear", cb=8)
    st = _launch(lib.w8a16_geglu_linear, x.get_device(),
                 x.data_ptr(), m, k, q.data_ptr(), s.data_ptr(), f,
                 None if bias is None else bias.data_ptr(), y_out.data_ptr())
    _lib.check(st, "w8a16_geglu_linear")
    return y_out


def w8a16_prepacked_bytes(n: int, k: int) -> int:
    """Bytes of the prepacked layout of INT8 codes [n][k] (-1 for bad sizes)."""
    return int(_lib.load().w8a16_prepacked_bytes(int(n), int(k)))


def w8a16_prepack(q, q_out=None):
    """INT8 codes [n][k] -> prepacked tile layout (uint8, 1-D)."""
    torch = _torch()
    lib = _lib.load()
    _require(q, torch.int8, "q")
    if q.dim() != 2:
        raise ValueError("q must be 2-D [n][k]")
    n, k = q.shape
    size = lib.w8a16_prepacked_bytes(n, k)
    if size < 0:
        raise ValueError(f"w8a16_prepack: bad shape n={n} k={k} (k % 32 must be 0)")
    if q_out is None:
        q_out = torch.empty((size,), dtype=torch.uint8, device=q.device)
    _require(q_out, torch.uint8, "q_out")
    if q_out.numel() != size:
        raise ValueError(f"w8a16_prepack: q_out must hold {size} bytes")
    _same_device(q_out, q.get_device(), "q_out", "w8a16_prepack")
    st = _launch(lib.w8a16_prepack, q.get_device(), q.data_ptr(), n, k, q_out.data_ptr())
    _lib.check(st, "w8a16_prepack")
    return q_out


def w8a16_linear_prepacked(x, qp, s, bias=None, y_out=None):
    """w8a16_linear with the codes in the prepacked layout (n = len(s))."""
    n = s.shape[0]
    lib, m, k, y_out = _prepacked_common(x, qp, s, bias, n, n, y_out, "w8a16_linear_prepacked", cb=8)
    st = _launch(lib.w8a16_linear_prepacked, x.get_device(),
                 x.data_ptr(), m, k, qp.data_ptr(), s.data_ptr(), n,
                 None if bias is None else bias.data_ptr(), y_out.data_ptr())
    _lib.check(st, "w8a16_linear_prepacked")
    return y_out


def w8a16_geglu_linear_prepacked(x, qp, s, bias=None, y_out=None):
    """w8a16_geglu_linear with the codes in the prepacked layout (f = len(s) / 2)."""
    rows = s.shape[0]
    if rows % 2:
        raise ValueError("w8a16_geglu_linear_prepacked: s must have 2f entries")
    f = rows // 2
    lib, m, k, y_out = _prepacked_common(x, qp, s, bias, f, rows, y_out,
                                         "w8a16_geglu_linear_prepacked", cb=8)
    st = _launch(lib.w8a16_geglu_linear_prepacked, x.get_device(),
                 x.data_ptr(), m, k, qp.data_ptr(), s.data_ptr(), f,
                 None if bias is None else bias.data_ptr(), y_out.data_ptr())
    _lib.check(st, "w8a16_geglu_linear_prepacked")
    return y_out


# --------------------------------------------------------------------------
# Zero-point INT4 variant (include/w4a16_zp.h)
# --------------------------------------------------------------------------

def quantize_rowwise_int4_zp(w, q_out=None, s_out=None, z_out=None):
    """W fp16 [n][k] (k even) -> (packed uint8 [n][k/2] unsigned codes, scales fp16 [n],
    zero points uint8 [n])."""
    torch = _torch()
    lib = _lib.load()
    _require(w, torch.float16, "w")
    if w.dim() != 2:
        raise ValueError("w must be 2-D [out_features][in_features]")
    n, k = w.shape
    if q_out is None:
        q_out = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    if s_out is None:
        s_out = torch.empty((n,), dtype=torch.float16, device=w.device)
    if z_out is None:
        z_out = torch.empty((n,), dtype=torch.uint8, device=w.device)
    _require(q_out, torch.uint8, "q_out")
    _require(s_out, torch.float16, "s_out")
    _require(z_out, torch.uint8, "z_out")
    if tuple(q_out.shape) != (n, k // 2) or tuple(s_out.shape) != (n,) or tuple(z_out.shape) != (n,):
        raise ValueError("output shape mismatch")
    dev = w.get_device()
    for t, nm in ((q_out, "q_out"), (s_out, "s_out"), (z_out, "z_out")):
        _same_device(t, dev, nm, "quantize_rowwise_int4_zp")
    st = _launch(lib.quantize_rowwise_int4_zp, dev, w.data_ptr(), n, k, q_out.data_ptr(),
                 s_out.data_ptr(), z_out.data_ptr())
    _lib.check(st, "quantize_rowwise_int4_zp")
    return q_out, s_out, z_out


def _zeros_check(z, rows, dev, name):
    torch = _torch()
    _require(z, torch.uint8, "z")
    if z.dim() != 1 or z.shape[0] != rows:
        raise ValueError(f"{name}: zero points must be uint8 [{rows}]")
    _same_device(z, dev, "z", name)


def w4a16_zp_linear(x, q, s, z, bias=None, y_out=None):
    """y[m][n] = fp16(s * (x . (q - z)^T) + bias) over zero-point codes."""
    lib = _lib.load()
    n = q.shape[0]
    m, k, y_out = _linear_common(x, q, s, bias, n, n, y_out, "w4a16_zp_linear")
    _zeros_check(z, n, x.get_device(), "w4a16_zp_linear")
    st = _launch(lib.w4a16_zp_linear, x.get_device(),
                 x.data_ptr(), m, k, q.data_ptr(), s.data_ptr(), z.data_ptr(), n,
                 None if bias is None else bias.data_ptr(), y_out.data_ptr())
    _lib.check(st, "w4a16_zp_linear")
    return y_out


def w4a16_zp_geglu_linear(x, q, s, z, bias=None, y_out=None):
    """GeGLU over zero-point codes [2f][k/2] with zero points [2f]."""
    lib = _lib.load()
    rows = q.shape[0]
    if rows % 2:
        raise ValueError("w4a16_zp_geglu_linear: q must have an even number of rows (2f)")
    f = rows // 2
    m, k, y_out = _linear_common(x, q, s, bias, f, rows, y_out, "w4a16_zp_geglu_linear")
    _zeros_check(z, rows, x.get_device(), "w4a16_zp_geglu_linear")
    st = _launch(lib.w4a16_zp_geglu_linear, x.get_device(),
                 x.data_ptr(), m, k, q.data_ptr(), s.data_ptr(), z.data_ptr(), f,
                 None if bias is None else bias.data_ptr(), y_out.data_ptr())
    _lib.check(st, "w4a16_zp_geglu_linear")
    return y_out


def w4a16_zp_linear_prepacked(x, qp, s, z, bias=None, y_out=None):
    """w4a16_zp_linear with the codes reordered by w4a16_prepack (n = len(s))."""
    n = s.shape[0]
    lib, m, k, y_out = _prepacked_common(x, qp, s, bias, n, n, y_out, "w4a16_zp_linear_prepacked")
    _zeros_check(z, n, x.get_device(), "w4a16_zp_linear_prepacked")
    st = _launch(lib.w4a16_zp_linear_prepacked, x.get_device(),
                 x.data_ptr(), m, k, qp.data_ptr(), s.data_ptr(), z.data_ptr(), n,
                 None if bias is None else bias.data_ptr(), y_out.data_ptr())
    _lib.check(st, "w4a16_zp_linear_prepacked")
    return y_out


def w4a16_zp_geglu_linear_prepacked(x, qp, s, z, bias=None, y_out=None):
    """w4a16_zp_geglu_linear with prepacked codes (f = len(s) / 2)."""
    rows = s.shape[0]
    if rows % 2:
        raise ValueError("w4a16_zp_geglu_linear_prepacked: s must have 2f entries")
    f = rows // 2
    lib, m, k, y_out = _prepacked_common(x, qp, s, bias, f, rows, y_out,
                                         "w4a16_zp_geglu_linear_prepacked")
    _zeros_check(z, rows, x.get_device(), "w4a16_zp_geglu_linear_prepacked")
    st = _launch(lib.w4a16_zp_geglu_linear_prepacked, x.get_device(),
                 x.data_ptr(), m, k, qp.data_ptr(), s.data_ptr(), z.data_ptr(), f,
                 None if bias is None else bias.data_ptr(), y_out.data_ptr())
    _lib.check(st, "w4a16_zp_geglu_linear_prepacked")
    return y_out


def read_probe(buf, nbytes=None, sink=None):
    """Measurement utility (not a step of the method): reads the first
    `nbytes` (default: all; a multiple of 1024) of the device tensor `buf`
    once in the plainest streaming pattern (w4a16_read_probe).  `sink`: an
    int32 device tensor of at least one element, or None to allocate one."""
    torch = _torch()
    lib = _lib.load()
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("read_probe: buf must be a contiguous GPU tensor")
    total = buf.numel() * buf.element_size()
    nbytes = total if nbytes is None else int(nbytes)
    if nbytes < 0 or nbytes > total:
        raise ValueError(f"read_probe: nbytes {nbytes} outside the buffer's {total} bytes")
    if sink is None:
        sink = torch.empty(1, dtype=torch.int32, device=buf.device)
    _require(sink, torch.int32, "sink")
    if sink.device != buf.device or sink.numel() < 1:
        raise ValueError("read_probe: sink must hold one int32 on the buffer's GPU")
    st = _launch(lib.w4a16_read_probe, buf.get_device(), buf.data_ptr(), nbytes, sink.data_ptr())
    _lib.check(st, "w4a16_read_probe")
    return sink
