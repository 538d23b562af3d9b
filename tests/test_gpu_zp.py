"""GPU parity of the zero-point INT4 variant (include/w4a16_zp.h) against the
CPU oracle, through the C ABI.

Codes, scales and zero points must be bit-exact.  Linear outputs must
satisfy |y - y_ref| <= 2e-3 * sum_k |x_k w_hat_k| (+|bias|) + 1e-4 with
w_hat = s (q - z), GeGLU outputs oracle.geglu_bound; one-hot activations and
power-of-two scales with integer activations are single roundings and must
be bit-exact; the prepacked layout must give bit-identical outputs.
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
    announce("quantize zp", what, tuple(w_cpu.shape))
    q, s, z = w4.quantize_rowwise_int4_zp(w_cpu.to(DEV))
    torch.cuda.synchronize()
    p_ref, s_ref, z_ref = oracle.quantize_rowwise_int4_zp(bits(w_cpu))
    assert_bits_equal(bits(s), s_ref, f"{what}: scales")
    assert_bits_equal(u8(z), z_ref, f"{what}: zero points")
    assert_bits_equal(u8(q), p_ref, f"{what}: packed codes")
    return q, s, z, p_ref, s_ref, z_ref


def check_linear(x_cpu, qsz, what, bias_cpu=None, prepacked=True):
    q, s, z, p_ref, s_ref, z_ref = qsz
    announce("linear zp", what, tuple(x_cpu.shape), tuple(q.shape))
    xd = x_cpu.to(DEV)
    bd = None if bias_cpu is None else bias_cpu.to(DEV)
    y = w4.w4a16_zp_linear(xd, q, s, z, bd)
    if prepacked:
        yp = w4.w4a16_zp_linear_prepacked(xd, w4.w4a16_prepack(q), s, z, bd)
    torch.cuda.synchronize()
    y_ref, mag = oracle.linear_zp(bits(x_cpu), p_ref, s_ref, z_ref, None if bias_cpu is None else bits(bias_cpu))
    r = assert_within(f64(y), y_ref, oracle.linear_bound(mag), what)
    if prepacked:
        assert_bits_equal(bits(yp), bits(y), f"{what}: prepacked vs row-major")
    return r


def check_geglu(x_cpu, qsz, what, bias_cpu=None, prepacked=True):
    q, s, z, p_ref, s_ref, z_ref = qsz
    announce("geglu zp", what, tuple(x_cpu.shape), tuple(q.shape))
    xd = x_cpu.to(DEV)
    bd = None if bias_cpu is None else bias_cpu.to(DEV)
    y = w4.w4a16_zp_geglu_linear(xd, q, s, z, bd)
    if prepacked:
        yp = w4.w4a16_zp_geglu_linear_prepacked(xd, w4.w4a16_prepack(q), s, z, bd)
    torch.cuda.synchronize()
    g, a, b, ma, mb = oracle.geglu_zp(bits(x_cpu), p_ref, s_ref, z_ref, None if bias_cpu is None else bits(bias_cpu))
    r = assert_within(f64(y), g, oracle.geglu_bound(g, a, b, ma, mb), what)
    if prepacked:
        assert_bits_equal(bits(yp), bits(y), f"{what}: prepacked vs row-major")
    return r


def _grid_rows(n, k, seed):
    """lo = -L 2^e, hi = (15 - L) 2^e: s = 2^e and z = L exactly; the other
    entries on the half-step grid (ties and exact levels)."""
    rng = np.random.default_rng(seed)
    rows = np.zeros((n, k), dtype=np.float64)
    for r in range(n):
        e = int(rng.integers(-8, 1))
        L = int(rng.integers(0, 16))
        rows[r] = rng.integers(-2 * L, 2 * (15 - L) + 1, size=k) * 0.5 * 2.0 ** e
        rows[r, 0] = -L * 2.0 ** e
        rows[r, 1] = (15 - L) * 2.0 ** e
    return torch.from_numpy(rows.astype(np.float16))


# ------------------------------------------------------------------ quantizer

def test_zp_quantize_toy_and_workload_rows():
    w, _ = synth.toy()
    quantize_both(w, "toy 1024x1024")
    g = synth.generator(2)
    quantize_both(synth.weight(300, 12288, g, "t4"), "t4 300x12288")
    quantize_both(synth.weight(40, 32768, g).abs(), "all-positive rows")
    quantize_both(-synth.weight(40, 32768, g).abs(), "all-negative rows")


@pytest.mark.parametrize("k", [12288, 1000, 2, 30, 65538])
def test_zp_quantize_paths_and_ties(k):
    """16-byte chunks (k % 8 == 0) and fp16 pairs (other even k); grid rows
    hit every tie with odd and even zero points."""
    g = synth.generator(40 + k)
    if k >= 2:
        quantize_both(_grid_rows(37, max(k, 2), 40 + k), f"grid k={k}")
    quantize_both(synth.weight(21, k, g), f"normal k={k}")


def test_zp_quantize_symmetric_enumeration():
    """Rows holding every fp16 value in [-a, a] (lo = -a, hi = a) for every
    third finite absmax a: every code of every such range."""
    all_a = torch.arange(0, 0x7C00, 3)
    for start in range(0, all_a.numel(), 4096):
        a = all_a[start:start + 4096]
        k = (2 * int(a[-1]) + 1 + 7) // 8 * 8
        quantize_both(synth.enumeration_rows(a, k), f"zp enumeration rows {start}.. k={k}")


@pytest.mark.parametrize("k", [8, 10])
def test_zp_quantize_asymmetric_ranges(k):
    """Scales of asymmetric ranges must be one rounding of (hi - lo) / 15:
    rows [1934, -0.0624694824, 0 ...] and [1.888671875, -6.0976e-05, 0 ...]
    and 1.6 M more range pairs (k = 8: the register-resident kernel, k = 10:
    the two-sweep kernel)."""
    hi, lo = synth.asymmetric_range_pairs()
    hi = torch.cat([torch.tensor([1934.0, 1.888671875], dtype=torch.float16), hi])
    lo = torch.cat([torch.tensor([-0.062469482421875, -6.0976e-05], dtype=torch.float16), lo])
    quantize_both(synth.range_end_rows(hi, lo, k), f"asymmetric range ends k={k}")


def test_zp_quantize_zero_and_tiny_rows():
    w = torch.zeros(4, 64, dtype=torch.float16)
    w[1, 3] = torch.tensor(7, dtype=torch.int16).view(torch.float16)      # (hi - lo)/15 rounds to 0
    w[2, :] = -0.0
    w[3, 0] = 65504.0
    w[3, 1] = -65504.0
    quantize_both(w, "zero/tiny/extreme")


# ------------------------------------------------------------------ linears

@pytest.mark.parametrize("m", [1, 5, 16, 17, 33, 64, 100, 300])
def test_zp_linear_ragged_shapes(m):
    g = synth.generator(100 + m)
    w = synth.weight(1000, 1120, g, "t4")
    bias = synth.normal_fp16((1000,), 0.5, g)
    qsz = quantize_both(w, f"ragged m={m}")
    x = synth.activations(m, 1120, g)
    check_linear(x, qsz, f"ragged m={m}")
    check_linear(x, qsz, f"ragged m={m} bias", bias)


@pytest.mark.parametrize("m", [1, 37, 64, 130])
def test_zp_one_hot_bit_exact(m):
    """y = fp16(s (q - z)): one exact product, one rounding."""
    g = synth.generator(300 + m)
    n, k = 530, 4096
    q, s, z, p_ref, s_ref, z_ref = quantize_both(synth.weight(n, k, g, "t4"), f"one-hot n={n}")
    x = synth.one_hot_activations(torch.randint(0, k, (m,), generator=g).tolist(), k)
    announce("one-hot zp", m)
    y = w4.w4a16_zp_linear(x.to(DEV), q, s, z)
    torch.cuda.synchronize()
    y_ref, _ = oracle.linear_zp(bits(x), p_ref, s_ref, z_ref)
    assert_bits_equal(bits(y), oracle.double_to_half(y_ref.ravel()).reshape(y_ref.shape), f"one-hot m={m}")


@pytest.mark.parametrize("m", [1, 16, 50, 64, 130])
def test_zp_pow2_scales_bit_exact(m):
    """Grid rows have s = 2^e; with integer activations every sum is an exact
    integer in fp32, so y is one rounding."""
    g = synth.generator(400 + m)
    n, k = 700, 2048
    q, s, z, p_ref, s_ref, z_ref = quantize_both(_grid_rows(n, k, 400 + m), f"pow2 n={n}")
    x = synth.small_int_activations(m, k, g)
    announce("pow2 zp", m)
    y = w4.w4a16_zp_linear(x.to(DEV), q, s, z)
    yp = w4.w4a16_zp_linear_prepacked(x.to(DEV), w4.w4a16_prepack(q), s, z)
    torch.cuda.synchronize()
    y_ref, _ = oracle.linear_zp(bits(x), p_ref, s_ref, z_ref)
    exact = oracle.double_to_half(y_ref.ravel()).reshape(y_ref.shape)
    assert_bits_equal(bits(y), exact, f"pow2 m={m}")
    assert_bits_equal(bits(yp), exact, f"pow2 prepacked m={m}")


_CLASS_MS = [1, 3, 8, 12, 17, 32, 45, 64]


@pytest.mark.parametrize("n,k", [(1000, 2048), (12288, 4096), (18424, 1024), (36848, 1024), (65520, 512)])
def test_zp_every_launch_class(n, k):
    g = synth.generator(1800 + n)
    w = synth.weight(n, k, g, "t4")
    bias = synth.normal_fp16((n,), 0.5, g)
    qsz = quantize_both(w, f"class n={n} k={k}")
    for m in _CLASS_MS:
        check_linear(synth.activations(m, k, g), qsz, f"class {m}x{n}x{k} bias", bias)


@pytest.mark.parametrize("f,k", [(496, 2048), (6160, 1024), (32752, 512)])
def test_zp_geglu_every_launch_class(f, k):
    g = synth.generator(1900 + f)
    w = synth.weight(2 * f, k, g, "t4")
    bias = synth.normal_fp16((2 * f,), 0.5, g)
    qsz = quantize_both(w, f"geglu class f={f} k={k}")
    for m in _CLASS_MS + [100]:
        check_geglu(synth.activations(m, k, g), qsz, f"geglu class {m}x{f}x{k} bias", bias)


@pytest.mark.parametrize("m,n,k", [(200, 1000, 1120), (520, 2000, 256), (2000, 12280, 160), (300, 3072, 8320)])
def test_zp_prefill_shapes(m, n, k):
    """Prefill tile shapes with zero points; 300 x 3072 x 8320 splits the
    reduction over two halves of a 512-thread workgroup (odd step count)."""
    g = synth.generator(2500 + m + n)
    w = synth.weight(n, k, g, "t4")
    qsz = quantize_both(w, f"prefill {n}x{k}")
    check_linear(synth.activations(m, k, g), qsz, f"prefill {m}x{n}x{k}", synth.normal_fp16((n,), 0.5, g))


@pytest.mark.parametrize("m,f,k", [(300, 512, 1056), (1000, 4080, 160)])
def test_zp_prefill_geglu(m, f, k):
    g = synth.generator(2600 + m + f)
    qsz = quantize_both(synth.weight(2 * f, k, g, "t4"), f"prefill geglu f={f}")
    check_geglu(synth.activations(m, k, g), qsz, f"prefill geglu {m}x{f}x{k}")
