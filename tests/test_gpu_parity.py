"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Quantized bytes and scales must be bit-exact.  Linear outputs must satisfy
|y - y_ref| <= 2e-3 * sum_k |x_k w_hat_k| (+|bias|) + 1e-4, GeGLU outputs the
propagated bound of oracle.geglu_bound; structural cases whose exact result
is a single rounding (one-hot activations, power-of-two scales with integer
activations) must be bit-exact.
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
    announce("quantize", what, tuple(w_cpu.shape))
    q, s = w4.quantize_rowwise_int4(w_cpu.to(DEV))
    torch.cuda.synchronize()
    p_ref, s_ref = oracle.quantize_rowwise_int4(bits(w_cpu))
    assert_bits_equal(bits(s), s_ref, f"{what}: scales")
    assert_bits_equal(u8(q), p_ref, f"{what}: packed codes")
    return q, s, p_ref, s_ref


def check_linear(x_cpu, q, s, p_ref, s_ref, what, bias_cpu=None):
    announce("linear", what, tuple(x_cpu.shape), tuple(q.shape))
    y = w4.w4a16_linear(x_cpu.to(DEV), q, s, None if bias_cpu is None else bias_cpu.to(DEV))
    torch.cuda.synchronize()
    y_ref, mag = oracle.linear(bits(x_cpu), p_ref, s_ref, None if bias_cpu is None else bits(bias_cpu))
    return assert_within(f64(y), y_ref, oracle.linear_bound(mag), what)


def check_geglu(x_cpu, q, s, p_ref, s_ref, what, bias_cpu=None):
    announce("geglu", what, tuple(x_cpu.shape), tuple(q.shape))
    y = w4.w4a16_geglu_linear(x_cpu.to(DEV), q, s, None if bias_cpu is None else bias_cpu.to(DEV))
    torch.cuda.synchronize()
    g, a, b, ma, mb = oracle.geglu(bits(x_cpu), p_ref, s_ref, None if bias_cpu is None else bits(bias_cpu))
    return assert_within(f64(y), g, oracle.geglu_bound(g, a, b, ma, mb), what)


# ------------------------------------------------------------------ quantizer

def test_quantize_toy_bit_exact():
    w, _ = synth.toy()
    quantize_both(w, "toy 1024x1024")


def test_quantize_every_absmax_and_weight_pair():
    """All 31744 finite non-negative fp16 absmax values a; each row holds
    every fp16 weight of magnitude <= a, in both signs (row length >= 2a+1,
    so the first batch runs the register path, the others the two-sweep
    path)."""
    all_a = torch.arange(0, 0x7C00)
    for start in range(0, all_a.numel(), 4096):
        a = all_a[start:start + 4096]
        k = (2 * int(a[-1]) + 1 + 7) // 8 * 8
        w = synth.enumeration_rows(a, k)
        quantize_both(w, f"enumeration absmax {start}..{start + a.numel() - 1} k={k}")


@pytest.mark.parametrize("k", [12288, 1000, 4096, 2, 30, 65538])
def test_quantize_ties_and_paths(k):
    """Power-of-two grids full of exact ties; k picks the register path
    (k % 8 == 0, k <= 32768) or the two-sweep path."""
    g = synth.generator(21)
    w = synth.exponent_rows(300, k, g)
    quantize_both(w, f"ties k={k}")


def test_quantize_zero_tiny_and_signed_zero_rows():
    w = torch.zeros(6, 256, dtype=torch.float16)
    w[1, 7] = torch.tensor([1], dtype=torch.int16).view(torch.float16)          # 2^-24
    w[2, 9] = -torch.tensor([3], dtype=torch.int16).view(torch.float16)         # -3 * 2^-24
    w[3] = -0.0
    w[4, 100] = torch.tensor([11], dtype=torch.int16).view(torch.float16)       # subnormal scale
    w[5, :] = torch.tensor([17], dtype=torch.int16).view(torch.float16)         # a/s > 7.5 -> clamp
    _, s, _, s_ref = quantize_both(w, "zero/tiny rows")
    assert (bits(s)[:4] == 0).all()


# ------------------------------------------------------------ decode linear

def test_toy_linear_m1_m16_with_and_without_bias():
    w, xs = synth.toy()
    q, s, p_ref, s_ref = quantize_both(w, "toy")
    g = synth.generator(1)
    bias = synth.normal_fp16((1024,), 0.5, g)
    for m, x in xs.items():
        check_linear(x, q, s, p_ref, s_ref, f"toy M={m}")
        check_linear(x, q, s, p_ref, s_ref, f"toy M={m} bias", bias)


@pytest.mark.parametrize("m", [1, 2, 3, 5, 8, 13, 16, 17, 24, 31, 32, 33, 40, 48, 49, 63, 64])
def test_decode_ragged_shapes(m):
    """m across all four 16-token blocks; n not a multiple of any tile; k a
    multiple of 32 but not of 128 (partial last reduction step)."""
    g = synth.generator(100 + m)
    w = synth.weight(1000, 1120, g, "t4")
    x = synth.activations(m, 1120, g)
    bias = synth.normal_fp16((1000,), 0.5, g)
    q, s, p_ref, s_ref = quantize_both(w, f"ragged m={m}")
    check_linear(x, q, s, p_ref, s_ref, f"ragged m={m}")
    check_linear(x, q, s, p_ref, s_ref, f"ragged m={m} bias", bias)


@pytest.mark.parametrize("k", [32, 64, 96, 160])
def test_decode_short_reduction(k):
    g = synth.generator(7 + k)
    w = synth.weight(77, k, g)
    q, s, p_ref, s_ref = quantize_both(w, f"short k={k}")
    for m in (1, 7, 64):
        check_linear(synth.activations(m, k, g), q, s, p_ref, s_ref, f"short k={k} m={m}")


def _one_hot_case(m, n, k, seed):
    g = synth.generator(seed)
    w = synth.weight(n, k, g, "t4")
    q, s, p_ref, s_ref = quantize_both(w, f"one-hot n={n} k={k}")
    cols = torch.randint(0, k, (m,), generator=g).tolist()
    x = synth.one_hot_activations(cols, k)
    announce("one-hot linear", m, n, k)
    y = w4.w4a16_linear(x.to(DEV), q, s)
    torch.cuda.synchronize()
    y_ref, _ = oracle.linear(bits(x), p_ref, s_ref)
    # a single product s * q: its fp16 rounding is the only rounding
    assert_bits_equal(bits(y), oracle.double_to_half(y_ref.ravel()).reshape(y_ref.shape), f"one-hot m={m}")


@pytest.mark.parametrize("m", [1, 16, 37, 64])
def test_decode_one_hot_bit_exact(m):
    _one_hot_case(m, 530, 4096, 300 + m)


def _pow2_case(m, n, k, seed):
    g = synth.generator(seed)
    w = synth.exponent_rows(n, k, g, -6, 0)
    q, s, p_ref, s_ref = quantize_both(w, f"pow2 n={n} k={k}")
    x = synth.small_int_activations(m, k, g)
    announce("pow2 linear", m, n, k)
    y = w4.w4a16_linear(x.to(DEV), q, s)
    torch.cuda.synchronize()
    y_ref, _ = oracle.linear(bits(x), p_ref, s_ref)
    # integer sums are exact in fp32 and s = 2^e: one rounding to fp16
    assert_bits_equal(bits(y), oracle.double_to_half(y_ref.ravel()).reshape(y_ref.shape), f"pow2 m={m}")


@pytest.mark.parametrize("m", [1, 9, 16, 50, 64])
def test_decode_pow2_scales_bit_exact(m):
    _pow2_case(m, 700, 2048, 400 + m)


@pytest.mark.parametrize("m", [1, 5, 16, 33, 64])
def test_decode_geglu_small(m):
    g = synth.generator(500 + m)
    f, k = 500, 1056
    w = synth.weight(2 * f, k, g, "t4")
    q, s, p_ref, s_ref = quantize_both(w, f"geglu f={f}")
    x = synth.activations(m, k, g)
    check_geglu(x, q, s, p_ref, s_ref, f"geglu m={m}")
    bias = synth.normal_fp16((2 * f,), 0.5, g)
    check_geglu(x, q, s, p_ref, s_ref, f"geglu m={m} bias", bias)


def test_geglu_negative_gate_region_distinguishes_erf_from_tanh():
    """Gate pre-activations near -3 where the erf and tanh GELU differ by
    ~10% relative: the fused output must follow the erf form."""
    f, k = 64, 256
    w = torch.zeros(2 * f, k, dtype=torch.float16)
    w[:f, 0] = 7.0 * 2.0 ** -2                   # gate rows: s = 2^-2, code 7 at k=0
    w[f:, 1] = 7.0                               # value rows: s = 1, code 7 at k=1
    q, s, p_ref, s_ref = quantize_both(w, "erf gate")
    x = torch.zeros(3, k, dtype=torch.float16)
    x[:, 0] = torch.tensor([-1.75, -1.5, -2.0], dtype=torch.float16)   # a = 7/4 * x0
    x[:, 1] = 1.0 / 7.0                                                # b ~= 1
    y = w4.w4a16_geglu_linear(x.to(DEV), q, s)
    torch.cuda.synchronize()
    g, a, b, ma, mb = oracle.geglu(bits(x), p_ref, s_ref)
    assert_within(f64(y), g, oracle.geglu_bound(g, a, b, ma, mb), "erf gate")
    assert np.all(np.abs(f64(y) - g) <= 2e-3 * np.abs(g) + 1e-6)


def test_geglu_fused_matches_unfused_halves():
    g = synth.generator(600)
    f, k, m = 384, 2048, 16
    w = synth.weight(2 * f, k, g, "t4")
    x = synth.activations(m, k, g).to(DEV)
    q, s = w4.quantize_rowwise_int4(w.to(DEV))
    fused = w4.w4a16_geglu_linear(x, q, s).double()
    a = w4.w4a16_linear(x, q[:f].contiguous(), s[:f].contiguous()).double()
    b = w4.w4a16_linear(x, q[f:].contiguous(), s[f:].contiguous()).double()
    unfused = torch.nn.functional.gelu(a) * b
    # the unfused path rounds a and b to fp16 first: allow for that
    tol = 2 ** -10 * (a.abs() * 1.13 * b.abs() + a.abs() * b.abs()) + 2 ** -10 * unfused.abs() + 1e-3
    assert torch.all((fused - unfused).abs() <= tol)


# ------------------------------------------------ every decode launch class
# The decode launch shape depends on the token class (m <= 4, 8, 16, 32, 48,
# 64), on the weight height (plain: bands from 8192, 16384, 24576 and 49152
# rows; GeGLU: from 12288, 24576 and 49152 rows of both halves) and, for
# 8192 to 16383 rows, on whether the reduction is short (k below or at
# 4096).  One weight per band (and both sides of the reduction threshold),
# every token class, reduction lengths that are whole and partial rounds of
# the chosen shapes, and both weight layouts.

_CLASS_MS = [1, 3, 8, 12, 17, 32, 45, 64]


@pytest.mark.parametrize("n,k", [(1000, 2048), (8200, 4160), (12280, 1024), (12288, 4096),
                                 (18424, 1024), (36848, 1024), (65520, 1024)])
def test_decode_every_launch_class(n, k):
    g = synth.generator(1800 + n)
    w = synth.weight(n, k, g, "t4")
    bias = synth.normal_fp16((n,), 0.5, g)
    q, s, p_ref, s_ref = quantize_both(w, f"class n={n} k={k}")
    qp = w4.w4a16_prepack(q)
    for m in _CLASS_MS:
        x = synth.activations(m, k, g)
        check_linear(x, q, s, p_ref, s_ref, f"class {m}x{n}x{k} bias", bias)
        announce("class prepacked", m, n, k)
        xd, bd = x.to(DEV), bias.to(DEV)
        y0 = w4.w4a16_linear(xd, q, s, bd)
        y1 = w4.w4a16_linear_prepacked(xd, qp, s, bd)
        torch.cuda.synchronize()
        assert_bits_equal(bits(y1), bits(y0), f"class prepacked vs row-major {m}x{n}x{k}")


@pytest.mark.parametrize("geglu,rows,k,m_gemm", [
    (False, 8192, 3072, 65),    # 8192-16383 rows, k < 4096
    (False, 8192, 4096, 80),    # 8192-16383 rows, 4096 <= k < 8192
    (False, 16384, 1024, 65),   # 16384-24575 rows
    (True, 24576, 1024, 65),    # GeGLU, 24576-49151 rows of both halves
])
def test_gemm_threshold_in_two_launch_range(geglu, rows, k, m_gemm):
    """64 < m <= 128: INT4 calls take one GEMM launch from a threshold m
    set by the weight's rows and, for 8192-16383 rows, its reduction
    length; below it, two decode launches.  At the threshold and one token
    below it (where the result must also equal separate calls on tokens
    0..63 and the rest, bit for bit), every output against the oracle."""
    g = synth.generator(2400 + rows // 1024 + k // 256 + geglu)
    w = synth.weight(rows, k, g, "t4")
    bias = synth.normal_fp16((rows,), 0.5, g)
    q, s, p_ref, s_ref = quantize_both(w, f"GEMM threshold rows={rows} k={k}")
    check = check_geglu if geglu else check_linear
    f = w4.w4a16_geglu_linear if geglu else w4.w4a16_linear
    for m in (m_gemm - 1, m_gemm):
        if m <= 64:
            continue
        x = synth.activations(m, k, g)
        check(x, q, s, p_ref, s_ref, f"threshold geglu={geglu} rows={rows} k={k} m={m}", bias)
        if m < m_gemm:
            announce("below the GEMM threshold: split calls", m, rows, k, geglu)
            xd, bd = x.to(DEV), bias.to(DEV)
            y = f(xd, q, s, bd)
            lo = f(xd[:64].contiguous(), q, s, bd)
            hi = f(xd[64:].contiguous(), q, s, bd)
            torch.cuda.synchronize()
            assert_bits_equal(bits(y), np.concatenate([bits(lo), bits(hi)]), f"two launches vs split calls m={m}")


@pytest.mark.parametrize("m", [65, 100, 128])
def test_two_decode_launches(m):
    """64 < m <= 128 runs the decode kernel on tokens 0..63, then on the
    rest through offset activation and output pointers.  Against the
    oracle (ragged n and k, bias, plain and GeGLU), bit-identical in both
    layouts and to separate calls on the two token ranges."""
    g = synth.generator(2300 + m)
    for geglu, rows, k in ((False, 1000, 1120), (True, 2 * 496, 1056)):
        w = synth.weight(rows, k, g, "t4")
        bias = synth.normal_fp16((rows,), 0.5, g)
        q, s, p_ref, s_ref = quantize_both(w, f"two launches rows={rows}")
        x = synth.activations(m, k, g)
        if geglu:
            check_geglu(x, q, s, p_ref, s_ref, f"two launches geglu m={m}", bias)
            f0, f1 = w4.w4a16_geglu_linear, w4.w4a16_geglu_linear_prepacked
        else:
            check_linear(x, q, s, p_ref, s_ref, f"two launches m={m}", bias)
            f0, f1 = w4.w4a16_linear, w4.w4a16_linear_prepacked
        announce("two launches split", m, rows, k, geglu)
        xd, bd = x.to(DEV), bias.to(DEV)
        y = f0(xd, q, s, bd)
        yp = f1(xd, w4.w4a16_prepack(q), s, bd)
        lo = f0(xd[:64].contiguous(), q, s, bd)
        hi = f0(xd[64:].contiguous(), q, s, bd)
        torch.cuda.synchronize()
        assert_bits_equal(bits(yp), bits(y), f"two launches prepacked vs row-major m={m} geglu={geglu}")
        assert_bits_equal(bits(y), np.concatenate([bits(lo), bits(hi)]), f"two launches vs split calls m={m}")


@pytest.mark.parametrize("n", [1001, 1002, 1003])
def test_decode_rows_not_a_multiple_of_four(n):
    """Output rows of n values lose 8-byte alignment when n % 4 != 0: every
    launch class then stores and reads its scales and biases element-wise."""
    g = synth.generator(2000 + n)
    k = 1056
    w = synth.weight(n, k, g, "t4")
    bias = synth.normal_fp16((n,), 0.5, g)
    q, s, p_ref, s_ref = quantize_both(w, f"n%4 n={n}")
    qp = w4.w4a16_prepack(q)
    for m in _CLASS_MS:
        x = synth.activations(m, k, g)
        check_linear(x, q, s, p_ref, s_ref, f"n%4 {m}x{n}x{k} bias", bias)
        announce("n%4 prepacked", m, n, k)
        xd, bd = x.to(DEV), bias.to(DEV)
        y0 = w4.w4a16_linear(xd, q, s, bd)
        y1 = w4.w4a16_linear_prepacked(xd, qp, s, bd)
        torch.cuda.synchronize()
        assert_bits_equal(bits(y1), bits(y0), f"n%4 prepacked vs row-major {m}x{n}x{k}")


@pytest.mark.parametrize("f", [499, 502])
def test_decode_geglu_halves_not_a_multiple_of_four(f):
    """The value half of the scales and biases starts at entry f: with
    f % 4 != 0 it is not 8-byte aligned."""
    g = synth.generator(2100 + f)
    k = 1056
    w = synth.weight(2 * f, k, g, "t4")
    bias = synth.normal_fp16((2 * f,), 0.5, g)
    q, s, p_ref, s_ref = quantize_both(w, f"geglu f%4 f={f}")
    for m in _CLASS_MS:
        x = synth.activations(m, k, g)
        check_geglu(x, q, s, p_ref, s_ref, f"geglu f%4 {m}x{f}x{k} bias", bias)


@pytest.mark.parametrize("f,k", [(496, 2048), (6160, 1024), (12304, 1024), (32752, 1024)])
def test_decode_geglu_every_launch_class(f, k):
    g = synth.generator(1900 + f)
    w = synth.weight(2 * f, k, g, "t4")
    bias = synth.normal_fp16((2 * f,), 0.5, g)
    q, s, p_ref, s_ref = quantize_both(w, f"geglu class f={f} k={k}")
    qp = w4.w4a16_prepack(q)
    for m in _CLASS_MS:
        x = synth.activations(m, k, g)
        check_geglu(x, q, s, p_ref, s_ref, f"geglu class {m}x{f}x{k} bias", bias)
        announce("geglu class prepacked", m, f, k)
        xd, bd = x.to(DEV), bias.to(DEV)
        y0 = w4.w4a16_geglu_linear(xd, q, s, bd)
        y1 = w4.w4a16_geglu_linear_prepacked(xd, qp, s, bd)
        torch.cuda.synchronize()
        assert_bits_equal(bits(y1), bits(y0), f"geglu class prepacked vs row-major {m}x{f}x{k}")


# ---------------------------------------- tall weights at 32 < m <= 64
# QKV-, FFN-up- and GeGLU-shaped weights (36864 / 65536 rows, 2 x 32768)
# take their own decode launch shapes at 32 < m <= 64 (several row groups
# per wavefront, K split over the workgroup); rows and k are ragged here.

@pytest.mark.parametrize("m,n,k", [(33, 36860, 160), (48, 36864, 256), (49, 36850, 96),
                                   (64, 36864, 160), (40, 65530, 96), (64, 65536, 128)])
def test_tall_decode_shapes(m, n, k):
    g = synth.generator(1400 + m + n)
    w = synth.weight(n, k, g, "t4")
    x = synth.activations(m, k, g)
    bias = synth.normal_fp16((n,), 0.5, g)
    q, s, p_ref, s_ref = quantize_both(w, f"tall {m}x{n}x{k}")
    check_linear(x, q, s, p_ref, s_ref, f"tall {m}x{n}x{k}")
    check_linear(x, q, s, p_ref, s_ref, f"tall {m}x{n}x{k} bias", bias)
    announce("tall prepacked", m, n, k)
    xd, bd = x.to(DEV), bias.to(DEV)
    y0 = w4.w4a16_linear(xd, q, s, bd)
    y1 = w4.w4a16_linear_prepacked(xd, w4.w4a16_prepack(q), s, bd)
    torch.cuda.synchronize()
    assert_bits_equal(bits(y1), bits(y0), f"tall prepacked vs row-major {m}x{n}x{k}")


@pytest.mark.parametrize("m", [37, 64])
def test_tall_decode_one_hot_and_pow2_bit_exact(m):
    _one_hot_case(m, 36864, 256, 1500 + m)
    _pow2_case(m, 36864, 256, 1600 + m)


@pytest.mark.parametrize("m,f,k", [(36, 32768, 160), (64, 32760, 96), (64, 32768, 128)])
def test_tall_decode_geglu(m, f, k):
    g = synth.generator(1700 + m + f)
    w = synth.weight(2 * f, k, g, "t4")
    x = synth.activations(m, k, g)
    q, s, p_ref, s_ref = quantize_both(w, f"tall geglu f={f} k={k}")
    check_geglu(x, q, s, p_ref, s_ref, f"tall geglu {m}x{f}x{k}")
    bias = synth.normal_fp16((2 * f,), 0.5, g)
    check_geglu(x, q, s, p_ref, s_ref, f"tall geglu {m}x{f}x{k} bias", bias)
    if f % 16 == 0:
        announce("tall geglu prepacked", m, f, k)
        xd = x.to(DEV)
        y0 = w4.w4a16_geglu_linear(xd, q, s)
        y1 = w4.w4a16_geglu_linear_prepacked(xd, w4.w4a16_prepack(q), s)
        torch.cuda.synchronize()
        assert_bits_equal(bits(y1), bits(y0), f"tall geglu prepacked vs row-major {m}x{f}x{k}")


# ----------------------------------------------------------- prefill GEMM

@pytest.mark.parametrize("m,n,k", [(65, 300, 160), (128, 128, 128), (129, 257, 96),
                                   (200, 1000, 1120), (256, 64, 32), (511, 33, 64)])
def test_prefill_ragged_shapes(m, n, k):
    g = synth.generator(m * 7 + n)
    w = synth.weight(n, k, g, "t4")
    x = synth.activations(m, k, g)
    bias = synth.normal_fp16((n,), 0.5, g)
    q, s, p_ref, s_ref = quantize_both(w, f"prefill {m}x{n}x{k}")
    check_linear(x, q, s, p_ref, s_ref, f"prefill {m}x{n}x{k}")
    check_linear(x, q, s, p_ref, s_ref, f"prefill {m}x{n}x{k} bias", bias)


@pytest.mark.parametrize("m", [65, 130, 300])
def test_prefill_one_hot_and_pow2_bit_exact(m):
    _one_hot_case(m, 300, 1024, 700 + m)
    _pow2_case(m, 260, 1024, 800 + m)


@pytest.mark.parametrize("geglu", [False, True])
def test_prefill_64_token_tiles(geglu):
    """A small grid (13 output tiles x 4 token tiles of the largest shape)
    takes 64-token tiles (128 rows with the reduction split; GeGLU 64
    outputs); ragged rows, tokens and k."""
    g = synth.generator(1800 + geglu)
    m, k = 500, 160
    n = 3328 - 6 if not geglu else 2 * 1661
    w = synth.weight(n, k, g, "t4")
    x = synth.activations(m, k, g)
    bias = synth.normal_fp16((n,), 0.5, g)
    q, s, p_ref, s_ref = quantize_both(w, f"prefill 64-token tiles n={n}")
    if geglu:
        check_geglu(x, q, s, p_ref, s_ref, f"prefill 64-token tiles geglu {m}x{n // 2}x{k}", bias)
    else:
        check_linear(x, q, s, p_ref, s_ref, f"prefill 64-token tiles {m}x{n}x{k}", bias)


@pytest.mark.parametrize("k", [8320, 8224])
def test_prefill_split_reduction(k):
    """A small grid with a long reduction (3072 rows, m = 300, on a 256-CU
    MI355X) takes 128-row x 64-token tiles with the reduction split over
    two halves of a 512-thread workgroup: an odd number of 128-wide steps
    (k = 8320), and a ragged last step (k = 8224); bias; both layouts
    bit-identical; power-of-two scales with integer activations bit-exact."""
    g = synth.generator(2400 + k)
    m, n = 300, 3072
    w = synth.weight(n, k, g, "t4")
    x = synth.activations(m, k, g)
    bias = synth.normal_fp16((n,), 0.5, g)
    q, s, p_ref, s_ref = quantize_both(w, f"prefill split reduction n={n} k={k}")
    check_linear(x, q, s, p_ref, s_ref, f"prefill split reduction {m}x{n}x{k} bias", bias)
    xd, bd = x.to(DEV), bias.to(DEV)
    y0 = w4.w4a16_linear(xd, q, s, bd)
    y1 = w4.w4a16_linear_prepacked(xd, w4.w4a16_prepack(q), s, bd)
    torch.cuda.synchronize()
    assert_bits_equal(bits(y1), bits(y0), f"prefill split reduction prepacked vs row-major k={k}")
    if k == 8320:
        _pow2_case(m, n, k, 2500)


@pytest.mark.parametrize("m,n", [(199, 32832), (129, 10944), (129, 32832), (325, 32832), (129, 256), (2053, 1024)])
def test_prefill_small_grid_shapes(m, n):
    """Small plain grids take the tile shape of least modelled time; on a
    256-CU MI355X these (m, n) pick 192 x 64, split 192 x 64, 256 x 64,
    256 x 128, split 128 x 64 and split 192 x 64 tiles.  Short ragged k
    (two steps, the second partial), bias, both layouts bit-identical."""
    g = synth.generator(2800 + m + n)
    k = 160
    w = synth.weight(n, k, g, "t4")
    x = synth.activations(m, k, g)
    bias = synth.normal_fp16((n,), 0.5, g)
    q, s, p_ref, s_ref = quantize_both(w, f"prefill small grid n={n}")
    check_linear(x, q, s, p_ref, s_ref, f"prefill small grid {m}x{n}x{k} bias", bias)
    xd, bd = x.to(DEV), bias.to(DEV)
    y0 = w4.w4a16_linear(xd, q, s, bd)
    y1 = w4.w4a16_linear_prepacked(xd, w4.w4a16_prepack(q), s, bd)
    torch.cuda.synchronize()
    assert_bits_equal(bits(y1), bits(y0), f"prefill small grid prepacked vs row-major {m}x{n}")


@pytest.mark.parametrize("geglu,m,n,k", [(False, 2000, 12280, 160), (False, 2000, 16380, 256),
                                         (True, 2000, 2 * 4080, 160)])
def test_prefill_large_grids(geglu, m, n, k):
    """Grids of more than two 256-row x 128-token tiles per CU (on a
    256-CU MI355X) take the 256-row tiles: 12280 rows at m = 2000 with
    64-token tiles (768 large tiles fill 1.5 waves, and k is short), 16380 rows with
    128-token tiles (1024 fill 2 waves), and GeGLU with 128-token tiles
    (f = 4080: ragged against 128-output tiles, a multiple of 16 as the
    prepacked GeGLU layout requires).  Ragged tokens and k; both layouts."""
    g = synth.generator(2200 + n + k)
    w = synth.weight(n, k, g, "t4")
    x = synth.activations(m, k, g)
    bias = synth.normal_fp16((n,), 0.5, g)
    q, s, p_ref, s_ref = quantize_both(w, f"prefill large grid {m}x{n}x{k}")
    if geglu:
        check_geglu(x, q, s, p_ref, s_ref, f"prefill large grid geglu {m}x{n // 2}x{k}", bias)
    else:
        check_linear(x, q, s, p_ref, s_ref, f"prefill large grid {m}x{n}x{k}", bias)
    announce("prefill large grid prepacked", m, n, k)
    xd, bd = x.to(DEV), bias.to(DEV)
    f0, f1 = ((w4.w4a16_geglu_linear, w4.w4a16_geglu_linear_prepacked) if geglu
              else (w4.w4a16_linear, w4.w4a16_linear_prepacked))
    y0 = f0(xd, q, s, bd)
    y1 = f1(xd, w4.w4a16_prepack(q), s, bd)
    torch.cuda.synchronize()
    assert_bits_equal(bits(y1), bits(y0), f"prefill large grid prepacked vs row-major {m}x{n}x{k}")


@pytest.mark.parametrize("m", [1000, 1060])
def test_prefill_geglu_tile_choice(m):
    """f = 4096 on a 256-CU MI355X: at m = 1000 one 128 x 128 tile per CU,
    so 64-output tiles, 128 tokens wide (their grid gives two per CU); at
    m = 1060 the 128-token tiles would pad half a tile more than 64-token
    ones and those fit one wave at three per CU, so 128 outputs x 64
    tokens.  Ragged tokens, short k, bias, both layouts bit-identical."""
    g = synth.generator(2700 + m)
    f, k = 4096, 160
    w = synth.weight(2 * f, k, g, "t4")
    x = synth.activations(m, k, g)
    bias = synth.normal_fp16((2 * f,), 0.5, g)
    q, s, p_ref, s_ref = quantize_both(w, f"prefill geglu tiles f={f}")
    check_geglu(x, q, s, p_ref, s_ref, f"prefill geglu tiles {m}x{f}x{k} bias", bias)
    xd, bd = x.to(DEV), bias.to(DEV)
    y0 = w4.w4a16_geglu_linear(xd, q, s, bd)
    y1 = w4.w4a16_geglu_linear_prepacked(xd, w4.w4a16_prepack(q), s, bd)
    torch.cuda.synchronize()
    assert_bits_equal(bits(y1), bits(y0), f"prefill geglu tiles prepacked vs row-major m={m}")


@pytest.mark.parametrize("m,f,k", [(65, 100, 256), (200, 300, 1024), (257, 64, 64)])
def test_prefill_geglu_small(m, f, k):
    g = synth.generator(900 + m)
    w = synth.weight(2 * f, k, g, "t4")
    x = synth.activations(m, k, g)
    q, s, p_ref, s_ref = quantize_both(w, f"prefill geglu f={f}")
    check_geglu(x, q, s, p_ref, s_ref, f"prefill geglu {m}x{f}x{k}")
    bias = synth.normal_fp16((2 * f,), 0.5, g)
    check_geglu(x, q, s, p_ref, s_ref, f"prefill geglu {m}x{f}x{k} bias", bias)


# ------------------------------------------------------- misc properties

def test_deterministic_reruns():
    g = synth.generator(1000)
    w = synth.weight(2048, 4096, g).to(DEV)
    q, s = w4.quantize_rowwise_int4(w)
    q2, s2 = w4.quantize_rowwise_int4(w)
    assert torch.equal(q, q2) and torch.equal(s, s2)
    for m in (1, 32, 300):
        x = synth.activations(m, 4096, g).to(DEV)
        y1 = w4.w4a16_linear(x, q, s)
        y2 = w4.w4a16_linear(x, q, s)
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), m


def test_read_probe_reads_without_writing():
    """The streaming-read probe the benchmark uses (a measurement utility,
    not a step of the method) reads whole 1 KB blocks, including a tail
    shorter than one round of its wavefronts, and writes neither the buffer
    nor (for data whose xor is not its constant) the sink."""
    nbytes = (256 * 12 * 4 + 3) * 1024
    buf = torch.zeros(nbytes + 4096, dtype=torch.uint8, device=DEV)
    sink = torch.full((1,), 12345, dtype=torch.int32, device=DEV)
    announce("read probe", nbytes)
    w4.read_probe(buf, nbytes, sink)
    w4.read_probe(buf, 1024, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 12345
    assert int(buf.count_nonzero().item()) == 0
    with pytest.raises(w4.W4A16Error):
        w4.read_probe(buf, 1000, sink)


def test_calls_follow_the_current_stream():
    """The binding passes torch's current stream; results on a side stream
    (default priority) equal those on the default stream."""
    g = synth.generator(1100)
    w = synth.weight(700, 2048, g).to(DEV)
    xs = {m: synth.activations(m, 2048, g).to(DEV) for m in (8, 130)}
    q, s = w4.quantize_rowwise_int4(w)
    ref = {m: w4.w4a16_linear(x, q, s) for m, x in xs.items()}
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q2, s2 = w4.quantize_rowwise_int4(w)
        out = {m: w4.w4a16_linear(x, q2, s2) for m, x in xs.items()}
    side.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2)
    for m in xs:
        assert torch.equal(out[m].view(torch.int16), ref[m].view(torch.int16)), m


def test_empty_and_rejected_calls():
    x = torch.zeros(0, 64, dtype=torch.float16, device=DEV)
    q = torch.zeros(16, 32, dtype=torch.uint8, device=DEV)
    s = torch.zeros(16, dtype=torch.float16, device=DEV)
    assert w4.w4a16_linear(x, q, s).shape == (0, 16)
    assert w4.w4a16_geglu_linear(x, q, s).shape == (0, 8)
    with pytest.raises(w4.W4A16Error):
        w4.w4a16_linear(torch.zeros(2, 48, dtype=torch.float16, device=DEV),
                        torch.zeros(4, 24, dtype=torch.uint8, device=DEV),
                        torch.zeros(4, dtype=torch.float16, device=DEV))
    with pytest.raises(w4.W4A16Error):
        w4.quantize_rowwise_int4(torch.zeros(4, 3, dtype=torch.float16, device=DEV))


# ------------------------------------------------------------ prepacked layout

def _prepack_reference(p_ref: np.ndarray, n: int, k: int) -> np.ndarray:
    """The prepacked layout written out from its definition (include/w4a16.h):
    1 KB tiles in lane order, each dword's codes e0..e7 stored as bytes
    e0|e2<<4, e4|e6<<4, e1|e3<<4, e5|e7<<4."""
    ng, kt = -(-n // 16), -(-k // 128)
    out = np.zeros((ng, kt, 64, 16), dtype=np.uint8)
    padded = np.zeros((ng * 16, kt * 64), dtype=np.uint8)
    padded[:n, :k // 2] = p_ref
    for lane in range(64):
        r, j = lane % 16, lane // 16
        for t in range(kt):
            out[:, t, lane, :] = padded[r::16, 64 * t + 16 * j: 64 * t + 16 * j + 16]
    d = out.reshape(-1, 4)
    e = np.empty((d.shape[0], 8), dtype=np.uint8)
    e[:, 0::2] = d & 0xF
    e[:, 1::2] = d >> 4
    nib = np.stack([e[:, 0] | (e[:, 2] << 4), e[:, 4] | (e[:, 6] << 4),
                    e[:, 1] | (e[:, 3] << 4), e[:, 5] | (e[:, 7] << 4)], axis=1)
    return nib.astype(np.uint8).reshape(-1)


@pytest.mark.parametrize("n,k", [(48, 256), (37, 160), (1000, 1120), (16, 128)])
def test_prepack_layout_matches_definition(n, k):
    g = synth.generator(1100 + n)
    w = synth.weight(n, k, g, "t4")
    q, s, p_ref, s_ref = quantize_both(w, f"prepack {n}x{k}")
    announce("prepack", n, k)
    qp = w4.w4a16_prepack(q)
    torch.cuda.synchronize()
    assert qp.numel() == w4.w4a16_prepacked_bytes(n, k)
    assert_bits_equal(u8(qp), _prepack_reference(p_ref, n, k), f"prepack {n}x{k}")


@pytest.mark.parametrize("m", [1, 5, 16, 17, 33, 64, 65, 130, 300])
def test_prepacked_linear_bit_identical_to_row_major(m):
    g = synth.generator(1200 + m)
    n, k = 1000, 1120
    w = synth.weight(n, k, g, "t4")
    x = synth.activations(m, k, g).to(DEV)
    bias = synth.normal_fp16((n,), 0.5, g).to(DEV)
    q, s = w4.quantize_rowwise_int4(w.to(DEV))
    qp = w4.w4a16_prepack(q)
    announce("prepacked linear", m, n, k)
    for b in (None, bias):
        y0 = w4.w4a16_linear(x, q, s, b)
        y1 = w4.w4a16_linear_prepacked(x, qp, s, b)
        torch.cuda.synchronize()
        assert_bits_equal(bits(y1), bits(y0), f"prepacked vs row-major m={m}")


@pytest.mark.parametrize("m", [1, 16, 40, 64, 130])
def test_prepacked_geglu_bit_identical_to_row_major(m):
    g = synth.generator(1300 + m)
    f, k = 512, 1056
    w = synth.weight(2 * f, k, g, "t4")
    x = synth.activations(m, k, g).to(DEV)
    q, s = w4.quantize_rowwise_int4(w.to(DEV))
    qp = w4.w4a16_prepack(q)
    announce("prepacked geglu", m, f, k)
    y0 = w4.w4a16_geglu_linear(x, q, s)
    y1 = w4.w4a16_geglu_linear_prepacked(x, qp, s)
    torch.cuda.synchronize()
    assert_bits_equal(bits(y1), bits(y0), f"prepacked geglu m={m}")
    with pytest.raises(w4.W4A16Error):
        q2, s2 = w4.quantize_rowwise_int4(synth.weight(2 * 24, k, g).to(DEV))
        w4.w4a16_geglu_linear_prepacked(x, w4.w4a16_prepack(q2), s2)
