"""The C-ABI library loads, exports what include/w4a16.h, include/w8a16.h and
include/w4a16_zp.h declare, and rejects bad arguments before touching any device (runs without
a GPU)."""
import ctypes
import os
import re

import pytest

from weight_only_int4_rowwise_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("w4a16.h", "w8a16.h", "w4a16_zp.h")]

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libw4a16.so not built (python -m weight_only_int4_rowwise_amd.build)")


def _declared_functions():
    names = set()
    for header in HEADERS:
        text = open(header).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\([^;{]*\)\s*;", text))
    return names


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_and_binding_agree():
    assert _declared_functions() == set(_lib.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_abi_version_and_status_strings(lib):
    assert lib.w4a16_abi_version() == _lib.ABI_VERSION
    for st in range(6):
        s = lib.w4a16_status_string(st).decode()
        assert s and s != "unknown status"
    assert lib.w4a16_status_string(99).decode() == "unknown status"
    assert lib.w4a16_last_error() is not None


# Fake device addresses: never dereferenced, because every call below is
# rejected (or is empty) before the library makes any HIP call.
A = 0x10000          # 16-byte aligned
B = 0x20000
C = 0x30000
D = 0x40000
MIS = 0x10008        # 8-byte aligned only


def test_quantize_argument_checks(lib):
    q = lib.quantize_rowwise_int4
    assert q(None, 4, 32, B, C, None) == _lib.ERR_NULL
    assert q(A, 4, 32, None, C, None) == _lib.ERR_NULL
    assert q(A, 4, 32, B, None, None) == _lib.ERR_NULL
    assert q(A, -1, 32, B, C, None) == _lib.ERR_SHAPE
    assert q(A, 4, 0, B, C, None) == _lib.ERR_SHAPE
    assert q(A, 4, 33, B, C, None) == _lib.ERR_SHAPE      # two codes per byte needs even k
    assert q(A, 1 << 31, 32, B, C, None) == _lib.ERR_SHAPE
    assert q(MIS, 4, 32, B, C, None) == _lib.ERR_ALIGN
    assert q(A, 4, 32, MIS, C, None) == _lib.ERR_ALIGN
    assert q(A, 0, 32, B, C, None) == _lib.OK            # empty: nothing launched
    assert q(None, 0, 32, None, None, None) == _lib.OK   # empty: pointers not looked at


@pytest.mark.parametrize("fn", ["w4a16_linear", "w4a16_geglu_linear", "w8a16_linear",
                                "w8a16_geglu_linear"])
def test_linear_argument_checks(lib, fn):
    f = getattr(lib, fn)
    assert f(None, 1, 64, B, C, 16, None, D, None) == _lib.ERR_NULL
    assert f(A, 1, 64, None, C, 16, None, D, None) == _lib.ERR_NULL
    assert f(A, 1, 64, B, None, 16, None, D, None) == _lib.ERR_NULL
    assert f(A, 1, 64, B, C, 16, None, None, None) == _lib.ERR_NULL
    assert f(A, -1, 64, B, C, 16, None, D, None) == _lib.ERR_SHAPE
    assert f(A, 1, 0, B, C, 16, None, D, None) == _lib.ERR_SHAPE
    assert f(A, 1, 48, B, C, 16, None, D, None) == _lib.ERR_SHAPE   # k % 32 != 0
    assert f(A, 1, 64, B, C, -2, None, D, None) == _lib.ERR_SHAPE
    assert f(A, 1 << 31, 64, B, C, 16, None, D, None) == _lib.ERR_SHAPE
    assert f(MIS, 1, 64, B, C, 16, None, D, None) == _lib.ERR_ALIGN
    assert f(A, 1, 64, B, C, 16, MIS, D, None) == _lib.ERR_ALIGN     # bias
    assert f(A, 1, 64, B, C, 16, None, MIS, None) == _lib.ERR_ALIGN
    assert f(A, 0, 64, B, C, 16, None, D, None) == _lib.OK           # empty
    assert f(A, 3, 64, B, C, 0, None, D, None) == _lib.OK            # empty
    assert f(None, 0, 64, None, None, 16, None, None, None) == _lib.OK


def test_binding_refuses_cpu_tensors():
    import torch
    import weight_only_int4_rowwise_amd as w4
    w = torch.zeros(4, 32, dtype=torch.float16)
    with pytest.raises(ValueError, match="no CPU path"):
        w4.quantize_rowwise_int4(w)


class _OnGpu:
    """Stand-in for a GPU tensor of a given shape on GPU `index`: only what the
    binding reads before its device checks (never launched)."""

    def __init__(self, shape, index):
        self.shape = tuple(shape)
        self.device = f"cuda:{index}"
        self._index = index

    def dim(self):
        return len(self.shape)

    def get_device(self):
        return self._index


@pytest.mark.parametrize("which", ["int4", "int8", "zp"])
def test_quantizers_refuse_outputs_on_another_gpu(monkeypatch, which):
    """Every quantizer checks that caller-supplied outputs sit on w's GPU
    before it launches (the dtype and layout checks are bypassed here, since
    there is no GPU tensor without a GPU)."""
    import weight_only_int4_rowwise_amd as w4
    monkeypatch.setattr(w4, "_require", lambda *a, **kw: None)
    n, k = 4, 32
    w = _OnGpu((n, k), 0)
    cols = k // 2 if which != "int8" else k
    good_q, bad_q = _OnGpu((n, cols), 0), _OnGpu((n, cols), 1)
    good_s, bad_s = _OnGpu((n,), 0), _OnGpu((n,), 1)
    if which == "int4":
        fn = lambda q, s: w4.quantize_rowwise_int4(w, q_out=q, s_out=s)
    elif which == "int8":
        fn = lambda q, s: w4.quantize_rowwise_int8(w, q_out=q, s_out=s)
    else:
        fn = lambda q, s: w4.quantize_rowwise_int4_zp(w, q_out=q, s_out=s, z_out=_OnGpu((n,), 0))
    with pytest.raises(ValueError, match="q_out on cuda:1"):
        fn(bad_q, good_s)
    with pytest.raises(ValueError, match="s_out on cuda:1"):
        fn(good_q, bad_s)


def test_prepacked_size_and_checks(lib):
    assert lib.w4a16_prepacked_bytes(16, 128) == 1024
    assert lib.w4a16_prepacked_bytes(17, 128) == 2048
    assert lib.w4a16_prepacked_bytes(16, 160) == 2048
    assert lib.w4a16_prepacked_bytes(36864, 12288) == 36864 * 12288 // 2
    assert lib.w4a16_prepacked_bytes(0, 64) == 0
    assert lib.w4a16_prepacked_bytes(-1, 64) == -1
    assert lib.w4a16_prepacked_bytes(16, 48) == -1
    assert lib.w4a16_prepacked_bytes(16, 0) == -1
    p = lib.w4a16_prepack
    assert p(None, 16, 64, B, None) == _lib.ERR_NULL
    assert p(A, 16, 64, None, None) == _lib.ERR_NULL
    assert p(A, 16, 48, B, None) == _lib.ERR_SHAPE
    assert p(MIS, 16, 64, B, None) == _lib.ERR_ALIGN
    assert p(None, 0, 64, None, None) == _lib.OK
    g = lib.w4a16_geglu_linear_prepacked
    assert g(A, 1, 64, B, C, 24, None, D, None) == _lib.ERR_SHAPE     # f % 16 != 0
    assert g(A, 1, 64, B, C, 32, None, MIS, None) == _lib.ERR_ALIGN
    lp = lib.w4a16_linear_prepacked
    assert lp(A, 1, 48, B, C, 16, None, D, None) == _lib.ERR_SHAPE
    assert lp(None, 1, 64, B, C, 16, None, D, None) == _lib.ERR_NULL


@pytest.mark.parametrize("fn,geglu", [("w4a16_linear", False), ("w4a16_geglu_linear", True),
                                      ("w4a16_linear_prepacked", False),
                                      ("w4a16_geglu_linear_prepacked", True)])
def test_buffer_size_limit(lib, fn, geglu):
    """Activations and packed weights must each stay below 2 GiB (32-bit buffer offsets)."""
    f = getattr(lib, fn)
    k = 32768
    m_max = (1 << 31) // (2 * k)                          # 2 m k == 2 GiB exactly
    assert f(A, m_max, k, B, C, 16, None, D, None) == _lib.ERR_SHAPE
    assert f(A, m_max - 1, k, B, C, 16, None, MIS, None) == _lib.ERR_ALIGN
    rows = (1 << 31) // (k // 2)                          # packed weight == 2 GiB exactly
    n = rows // 2 if geglu else rows
    assert f(A, 1, k, B, C, n, None, D, None) == _lib.ERR_SHAPE
    # the GLM-130B FFN up-projection (2 x 32768 rows x 12288) is accepted by the
    # size check (the call then fails on the fake pointers' alignment)
    n = 32768 if geglu else 65536
    assert f(A, 1, 12288, B, C, n, None, MIS, None) == _lib.ERR_ALIGN


def test_int8_quantize_argument_checks(lib):
    q = lib.quantize_rowwise_int8
    assert q(None, 4, 32, B, C, None) == _lib.ERR_NULL
    assert q(A, 4, 32, None, C, None) == _lib.ERR_NULL
    assert q(A, -1, 32, B, C, None) == _lib.ERR_SHAPE
    assert q(A, 4, 33, B, C, None) == _lib.ERR_SHAPE      # pairs of fp16 per load: k even
    assert q(MIS, 4, 32, B, C, None) == _lib.ERR_ALIGN
    assert q(A, 4, 32, MIS, C, None) == _lib.ERR_ALIGN
    assert q(None, 0, 32, None, None, None) == _lib.OK


def test_int8_prepacked_size_and_checks(lib):
    assert lib.w8a16_prepacked_bytes(16, 128) == 2048
    assert lib.w8a16_prepacked_bytes(17, 128) == 4096
    assert lib.w8a16_prepacked_bytes(16, 160) == 4096
    assert lib.w8a16_prepacked_bytes(36864, 12288) == 36864 * 12288
    assert lib.w8a16_prepacked_bytes(16, 48) == -1
    p = lib.w8a16_prepack
    assert p(None, 16, 64, B, None) == _lib.ERR_NULL
    assert p(A, 16, 48, B, None) == _lib.ERR_SHAPE
    assert p(MIS, 16, 64, B, None) == _lib.ERR_ALIGN
    assert p(None, 0, 64, None, None) == _lib.OK
    g = lib.w8a16_geglu_linear_prepacked
    assert g(A, 1, 64, B, C, 24, None, D, None) == _lib.ERR_SHAPE     # f % 16 != 0
    assert lib.w8a16_linear_prepacked(A, 1, 48, B, C, 16, None, D, None) == _lib.ERR_SHAPE


@pytest.mark.parametrize("fn,geglu", [("w8a16_linear", False), ("w8a16_geglu_linear", True),
                                      ("w8a16_linear_prepacked", False),
                                      ("w8a16_geglu_linear_prepacked", True)])
def test_int8_buffer_size_limit(lib, fn, geglu):
    """One byte per code: the INT8 weight reaches 2 GiB at half the rows of INT4."""
    f = getattr(lib, fn)
    k = 32768
    rows = (1 << 31) // k                                 # codes == 2 GiB exactly
    n = rows // 2 if geglu else rows
    assert f(A, 1, k, B, C, n, None, D, None) == _lib.ERR_SHAPE
    assert f(A, 1, k, B, C, n - 16, None, MIS, None) == _lib.ERR_ALIGN
    # the GLM-130B FFN up-projection in INT8 (768 MiB) passes the size check
    n = 32768 if geglu else 65536
    assert f(A, 1, 12288, B, C, n, None, MIS, None) == _lib.ERR_ALIGN


def test_int8_binding_refuses_cpu_tensors():
    import torch
    import weight_only_int4_rowwise_amd as w4
    with pytest.raises(ValueError, match="no CPU path"):
        w4.quantize_rowwise_int8(torch.zeros(4, 32, dtype=torch.float16))


def test_zp_quantize_argument_checks(lib):
    q = lib.quantize_rowwise_int4_zp
    assert q(A, 4, 32, B, C, None, None) == _lib.ERR_NULL          # zero points
    assert q(A, 4, 33, B, C, D, None) == _lib.ERR_SHAPE
    assert q(A, 4, 32, B, C, MIS, None) == _lib.ERR_ALIGN
    assert q(None, 0, 32, None, None, None, None) == _lib.OK


@pytest.mark.parametrize("fn", ["w4a16_zp_linear", "w4a16_zp_geglu_linear",
                                "w4a16_zp_linear_prepacked", "w4a16_zp_geglu_linear_prepacked"])
def test_zp_linear_argument_checks(lib, fn):
    f = getattr(lib, fn)
    E = 0x50000
    assert f(A, 1, 64, B, C, None, 16, None, D, None) == _lib.ERR_NULL     # zero points
    assert f(A, 1, 64, B, C, MIS, 16, None, D, None) == _lib.ERR_ALIGN
    assert f(None, 1, 64, B, C, E, 16, None, D, None) == _lib.ERR_NULL
    assert f(A, 1, 48, B, C, E, 16, None, D, None) == _lib.ERR_SHAPE       # k % 32 != 0
    assert f(None, 0, 64, None, None, None, 16, None, None, None) == _lib.OK


def test_read_probe_argument_checks(lib):
    """The measurement probe rejects sizes that are not whole 1 KB blocks,
    NULL and misaligned pointers; an empty read succeeds without a device."""
    p = lib.w4a16_read_probe
    assert p(A, -1024, B, None) == _lib.ERR_SHAPE
    assert p(A, 1000, B, None) == _lib.ERR_SHAPE
    assert p(A, (1 << 40) + 1024, B, None) == _lib.ERR_SHAPE
    assert p(None, 0, None, None) == _lib.OK
    assert p(None, 1024, B, None) == _lib.ERR_NULL
    assert p(A, 1024, None, None) == _lib.ERR_NULL
    assert p(MIS, 1024, B, None) == _lib.ERR_ALIGN
    assert p(A, 1024, B + 2, None) == _lib.ERR_ALIGN
