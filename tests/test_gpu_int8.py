"""GPU parity of the INT8 row-wise variant (W8A16, include/w8a16.h) against
the CPU oracle, through the C ABI.

Codes and scales must be bit-exact.  Linear outputs must satisfy the same
bound as W4A16, |y - y_ref| <= 2e-3 * sum_k |x_k w_hat_k| (+|bias|) + 1e-4,
GeGLU outputs oracle.geglu_bound; one-hot activations and power-of-two
scales with integer activations are single roundings and must be
bit-exact; the prepacked layout must give bit-identical outputs.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_int4_rowwise_amd as w4
from weight_only_int4_rowwise_amd import synth

from helpers import announce, assert_bits_equal, assert_within, bits, f64, u8

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w4.library()
    oracle._load()
    yield
    torch.cuda.synchronize()


def quantize_both(w_cpu: torch.Tensor, what: str):
    announce("quantize int8", what, tuple(w_cpu.shape))
    q, s = w4.quantize_rowwise_int8(w_cpu.to(DEV))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_rowwise_int8(bits(w_cpu))
    assert_bits_equal(bits(s), s_ref, f"{what}: scales")
    assert_bits_equal(u8(q), q_ref, f"{what}: codes")
    return q, s, q_ref, s_ref


def check_linear(x_cpu, q, s, q_ref, s_ref, what, bias_cpu=None, prepacked=None):
    announce("linear int8", what, tuple(x_cpu.shape), tuple(q.shape))
    xd = x_cpu.to(DEV)
    bd = None if bias_cpu is None else bias_cpu.to(DEV)
    y = w4.w8a16_linear(xd, q, s, bd)
    if prepacked is not None:
        yp = w4.w8a16_linear_prepacked(xd, prepacked, s, bd)
    torch.cuda.synchronize()
    y_ref, mag = oracle.linear_int8(bits(x_cpu), q_ref, s_ref, None if bias_cpu is None else bits(bias_cpu))
    r = assert_within(f64(y), y_ref, oracle.linear_bound(mag), what)
    if prepacked is not None:
        assert_bits_equal(bits(yp), bits(y), f"{what}: prepacked vs row-major")
    return r


def check_geglu(x_cpu, q, s, q_ref, s_ref, what, bias_cpu=None, prepacked=None):
    announce("geglu int8", what, tuple(x_cpu.shape), tuple(q.shape))
    xd = x_cpu.to(DEV)
    bd = None if bias_cpu is None else bias_cpu.to(DEV)
    y = w4.w8a16_geglu_linear(xd, q, s, bd)
    if prepacked is not None:
        yp = w4.w8a16_geglu_linear_prepacked(xd, prepacked, s, bd)
    torch.cuda.synchronize()
    g, a, b, ma, mb = oracle.geglu_int8(bits(x_cpu), q_ref, s_ref, None if bias_cpu is None else bits(bias_cpu))
    r = assert_within(f64(y), g, oracle.geglu_bound(g, a, b, ma, mb), what)
    if prepacked is not None:
        assert_bits_equal(bits(yp), bits(y), f"{what}: prepacked vs row-major")
    return r


# ------------------------------------------------------------------ quantizer

def test_int8_quantize_toy_and_workload_rows_bit_exact():
    w, _ = synth.toy()
    quantize_both(w, "toy 1024x1024")
    g = synth.generator(2)
    quantize_both(synth.weight(300, 12288, g, "t4"), "t4 300x12288")


@pytest.mark.parametrize("k", [12288, 1000, 4096, 2, 30, 65538, 32768])
def test_int8_quantize_paths(k):
    """Register paths (k % 8 == 0, rows up to 32768), and the two-sweep path
    (k % 8 != 0 or longer rows); grid rows hit every tie."""
    g = synth.generator(40 + k)
    quantize_both(synth.exponent_rows(37, k, g, -10, 2, top=127), f"grid k={k}")
    quantize_both(synth.weight(21, k, g), f"normal k={k}")


def test_int8_quantize_every_absmax_and_weight_pair():
    """All 31744 finite non-negative fp16 absmax values a; each row holds
    every fp16 weight of magnitude <= a, in both signs."""
    all_a = torch.arange(0, 0x7C00)
    for start in range(0, all_a.numel(), 4096):
        a = all_a[start:start + 4096]
        k = (2 * int(a[-1]) + 1 + 7) // 8 * 8
        w = synth.enumeration_rows(a, k)
        quantize_both(w, f"int8 enumeration absmax {start}..{start + a.numel() - 1} k={k}")


def test_int8_quantize_zero_tiny_and_subnormal_rows():
    w = torch.zeros(6, 64, dtype=torch.float16)
    w[1, 3] = torch.tensor(63, dtype=torch.int16).view(torch.float16)       # a/127 rounds to 0
    w[2, :] = -0.0
    w[3, 0] = torch.tensor(190, dtype=torch.int16).view(torch.float16)      # s = 2^-24, clamp 127
    w[3, 1] = torch.tensor(101, dtype=torch.int16).view(torch.float16)
    w[4, 5] = 65504.0                                                       # largest finite
    w[4, 6] = -65504.0
    w[5, :] = 1.0
    q, s, q_ref, s_ref = quantize_both(w, "zero/tiny/subnormal")
    assert q_ref[3, 0] == 127 and q_ref[3, 1] == 101 and s_ref[1] == 0 and s_ref[2] == 0


# ------------------------------------------------------------ prepacked layout

def _prepack8_reference(q_ref: np.ndarray, n: int, k: int) -> np.ndarray:
    """The INT8 prepacked layout written out from its definition
    (include/w8a16.h): 2 KB tiles, two 1 KB halves in lane order, codes as
    offset bytes q + 128, padding code 0."""
    ng, kt = -(-n // 16), -(-k // 128)
    padded = np.zeros((ng * 16, kt * 128), dtype=np.int16)
    padded[:n, :k] = q_ref
    out = np.zeros((ng, kt, 2, 64, 16), dtype=np.uint8)
    for lane in range(64):
        r, j = lane % 16, lane // 16
        for t in range(kt):
            for h in range(2):
                c0 = 128 * t + 32 * j + 16 * h
                out[:, t, h, lane, :] = (padded[r::16, c0:c0 + 16] + 128).astype(np.uint8)
    return out.reshape(-1)


@pytest.mark.parametrize("n,k", [(48, 256), (37, 160), (1000, 1120), (16, 128)])
def test_int8_prepack_layout_matches_definition(n, k):
    g = synth.generator(1100 + n)
    q, s, q_ref, s_ref = quantize_both(synth.weight(n, k, g, "t4"), f"prepack {n}x{k}")
    announce("prepack int8", n, k)
    qp = w4.w8a16_prepack(q)
    torch.cuda.synchronize()
    assert qp.numel() == w4.w8a16_prepacked_bytes(n, k)
    assert_bits_equal(u8(qp), _prepack8_reference(q_ref, n, k), f"prepack int8 {n}x{k}")


# ------------------------------------------------------------ decode linear

@pytest.mark.parametrize("m", [1, 2, 5, 8, 13, 16, 17, 31, 32, 33, 48, 49, 64])
def test_int8_decode_ragged_shapes(m):
    """n not a multiple of any tile; k a multiple of 32 but not of 128."""
    g = synth.generator(100 + m)
    w = synth.weight(1000, 1120, g, "t4")
    bias = synth.normal_fp16((1000,), 0.5, g)
    q, s, q_ref, s_ref = quantize_both(w, f"ragged m={m}")
    qp = w4.w8a16_prepack(q)
    x = synth.activations(m, 1120, g)
    check_linear(x, q, s, q_ref, s_ref, f"ragged m={m}", prepacked=qp)
    check_linear(x, q, s, q_ref, s_ref, f"ragged m={m} bias", bias, prepacked=qp)


@pytest.mark.parametrize("k", [32, 64, 96, 160])
def test_int8_decode_short_reduction(k):
    g = synth.generator(7 + k)
    q, s, q_ref, s_ref = quantize_both(synth.weight(77, k, g), f"short k={k}")
    for m in (1, 7, 64):
        check_linear(synth.activations(m, k, g), q, s, q_ref, s_ref, f"short k={k} m={m}")


@pytest.mark.parametrize("m", [1, 16, 37, 64, 100, 300])
def test_int8_one_hot_bit_exact(m):
    """y = fp16(s * q): a single rounding, in every kernel (decode, two
    decode launches, prefill)."""
    g = synth.generator(300 + m)
    n, k = 530, 4096
    q, s, q_ref, s_ref = quantize_both(synth.weight(n, k, g, "t4"), f"one-hot n={n} k={k}")
    cols = torch.randint(0, k, (m,), generator=g).tolist()
    x = synth.one_hot_activations(cols, k)
    announce("one-hot int8", m, n, k)
    y = w4.w8a16_linear(x.to(DEV), q, s)
    torch.cuda.synchronize()
    y_ref, _ = oracle.linear_int8(bits(x), q_ref, s_ref)
    assert_bits_equal(bits(y), oracle.double_to_half(y_ref.ravel()).reshape(y_ref.shape), f"one-hot m={m}")


@pytest.mark.parametrize("m", [1, 9, 16, 50, 64, 130])
def test_int8_pow2_scales_bit_exact(m):
    """Rows with absmax 127 * 2^e have s = 2^e; integer activations make
    every sum an exact integer in fp32, so y is one rounding."""
    g = synth.generator(400 + m)
    n, k = 700, 2048
    w = synth.exponent_rows(n, k, g, -6, 0, top=127)
    q, s, q_ref, s_ref = quantize_both(w, f"pow2 n={n} k={k}")
    x = synth.small_int_activations(m, k, g)
    announce("pow2 int8", m, n, k)
    y = w4.w8a16_linear(x.to(DEV), q, s)
    yp = w4.w8a16_linear_prepacked(x.to(DEV), w4.w8a16_prepack(q), s)
    torch.cuda.synchronize()
    y_ref, _ = oracle.linear_int8(bits(x), q_ref, s_ref)
    exact = oracle.double_to_half(y_ref.ravel()).reshape(y_ref.shape)
    assert_bits_equal(bits(y), exact, f"pow2 m={m}")
    assert_bits_equal(bits(yp), exact, f"pow2 prepacked m={m}")


_CLASS_MS = [1, 3, 8, 12, 17, 32, 45, 64]


@pytest.mark.parametrize("n,k", [(1000, 2048), (8200, 4160), (12280, 1024), (12288, 4096),
                                 (18424, 1024), (36848, 1024), (65520, 512)])
def test_int8_decode_every_launch_class(n, k):
    """Every (token class, height band) pair of the INT8 launch table, both
    sides of the short-reduction threshold, both layouts."""
    g = synth.generator(1800 + n)
    w = synth.weight(n, k, g, "t4")
    bias = synth.normal_fp16((n,), 0.5, g)
    q, s, q_ref, s_ref = quantize_both(w, f"class n={n} k={k}")
    qp = w4.w8a16_prepack(q)
    for m in _CLASS_MS:
        x = synth.activations(m, k, g)
        check_linear(x, q, s, q_ref, s_ref, f"class {m}x{n}x{k} bias", bias, prepacked=qp)


@pytest.mark.parametrize("f,k", [(496, 2048), (6160, 1024), (12304, 1024), (32752, 512)])
def test_int8_decode_geglu_every_launch_class(f, k):
    g = synth.generator(1900 + f)
    w = synth.weight(2 * f, k, g, "t4")
    bias = synth.normal_fp16((2 * f,), 0.5, g)
    q, s, q_ref, s_ref = quantize_both(w, f"geglu class f={f} k={k}")
    qp = w4.w8a16_prepack(q)
    for m in _CLASS_MS:
        x = synth.activations(m, k, g)
        check_geglu(x, q, s, q_ref, s_ref, f"geglu class {m}x{f}x{k} bias", bias, prepacked=qp)


@pytest.mark.parametrize("m", [65, 100, 128])
def test_int8_two_decode_launches(m):
    g = synth.generator(2300 + m)
    for geglu, rows, k in ((False, 1000, 1120), (True, 2 * 496, 1056)):
        w = synth.weight(rows, k, g, "t4")
        bias = synth.normal_fp16((rows,), 0.5, g)
        q, s, q_ref, s_ref = quantize_both(w, f"two launches rows={rows}")
        qp = w4.w8a16_prepack(q)
        x = synth.activations(m, k, g)
        if geglu:
            check_geglu(x, q, s, q_ref, s_ref, f"two launches geglu m={m}", bias, prepacked=qp)
        else:
            check_linear(x, q, s, q_ref, s_ref, f"two launches m={m}", bias, prepacked=qp)


# ------------------------------------------------------------------ prefill

@pytest.mark.parametrize("m,n,k", [(129, 300, 160), (200, 1000, 1120), (300, 257, 96),
                                   (520, 2000, 256), (2000, 12280, 160)])
def test_int8_prefill_shapes(m, n, k):
    """The MFMA GEMM path (m > 128) over INT8 codes: ragged m, n, k, small
    grids (192 x 64 tiles) and large ones (192 x 128), both layouts."""
    g = synth.generator(2500 + m + n)
    w = synth.weight(n, k, g, "t4")
    bias = synth.normal_fp16((n,), 0.5, g)
    q, s, q_ref, s_ref = quantize_both(w, f"prefill {n}x{k}")
    qp = w4.w8a16_prepack(q)
    check_linear(synth.activations(m, k, g), q, s, q_ref, s_ref, f"prefill {m}x{n}x{k} bias", bias,
                 prepacked=qp)


@pytest.mark.parametrize("m,f,k", [(129, 96, 256), (300, 512, 1056), (1000, 4080, 160), (2000, 8192, 160)])
def test_int8_prefill_geglu(m, f, k):
    g = synth.generator(2600 + m + f)
    w = synth.weight(2 * f, k, g, "t4")
    q, s, q_ref, s_ref = quantize_both(w, f"prefill geglu f={f} k={k}")
    qp = w4.w8a16_prepack(q)
    check_geglu(synth.activations(m, k, g), q, s, q_ref, s_ref, f"prefill geglu {m}x{f}x{k}",
                prepacked=qp)
