"""GPU parity at the full GLM-130B shapes, in the launch configurations the
benchmark times.

Inputs are drawn on the GPU (seeded ``torch.Generator('cuda')``; the same
tensors are copied to the host for the oracle).  Quantized bytes and scales
are compared in full; decode outputs (m <= 64) in full; two-launch decode
(m = 100) and prefill outputs (m = 512, 2048) on sampled rows and columns
that touch every output tile.
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
    torch.cuda.empty_cache()


def _quantize_checked(w, what):
    announce("quantize", what, tuple(w.shape))
    q, s = w4.quantize_rowwise_int4(w)
    torch.cuda.synchronize()
    p_ref, s_ref = oracle.quantize_rowwise_int4(bits(w))
    assert_bits_equal(bits(s), s_ref, f"{what}: scales")
    assert_bits_equal(u8(q), p_ref, f"{what}: packed")
    return q, s, p_ref, s_ref


@pytest.fixture(scope="module")
def qkv():
    w, xs = synth.qkv_decode(device=DEV)
    q, s, p_ref, s_ref = _quantize_checked(w, "QKV 36864x12288")
    del w
    return q, s, p_ref, s_ref, xs


@pytest.mark.parametrize("m", [1, 8, 32, 64])
def test_qkv_decode_full(qkv, m):
    q, s, p_ref, s_ref, xs = qkv
    x = xs[m]
    announce("QKV decode", m)
    y = w4.w4a16_linear(x, q, s)
    torch.cuda.synchronize()
    y_ref, mag = oracle.linear(bits(x), p_ref, s_ref)
    r = assert_within(f64(y), y_ref, oracle.linear_bound(mag), f"QKV M={m}")
    print(f"QKV M={m}: max err/bound {r:.4f}")


def test_qkv_two_decode_launches_sampled(qkv):
    """64 < m <= 128 runs the decode kernel on tokens 0..63, then on the
    rest: QKV at m = 100, one token in every 16-token block and two
    columns in every 144-row workgroup tile, against the oracle."""
    q, s, p_ref, s_ref, _ = qkv
    m = 100
    x = synth.activations(m, synth.HIDDEN, synth.generator(7, DEV), DEV)
    announce("QKV two decode launches", m)
    y = w4.w4a16_linear(x, q, s)
    torch.cuda.synchronize()
    mi, ni = _sample_indices(m, q.shape[0], 16, 144, 5)
    y_ref, mag = oracle.linear_at(bits(x), p_ref, s_ref, mi, ni)
    r = assert_within(_gather(y, mi, ni), y_ref, oracle.linear_bound(mag), f"QKV M={m}")
    print(f"QKV M={m}: {mi.size} sampled outputs, max err/bound {r:.4f}")


@pytest.fixture(scope="module")
def ffn():
    w_up, w_down, x_up, x_down = synth.geglu_decode(device=DEV)
    up = _quantize_checked(w_up, "FFN up 65536x12288 t4")
    del w_up
    down = _quantize_checked(w_down, "FFN down 12288x32768 t4")
    del w_down
    return up, down, x_up, x_down


@pytest.mark.parametrize("m", [1, 16])
def test_geglu_decode_full(ffn, m):
    (q, s, p_ref, s_ref), _, x_up, _ = ffn
    x = x_up[m]
    announce("GeGLU up decode", m)
    y = w4.w4a16_geglu_linear(x, q, s)
    torch.cuda.synchronize()
    g, a, b, ma, mb = oracle.geglu(bits(x), p_ref, s_ref)
    r = assert_within(f64(y), g, oracle.geglu_bound(g, a, b, ma, mb), f"GeGLU up M={m}")
    print(f"GeGLU up M={m}: max err/bound {r:.4f}")


@pytest.mark.parametrize("m", [1, 16])
def test_down_decode_full(ffn, m):
    _, (q, s, p_ref, s_ref), _, x_down = ffn
    x = x_down[m]
    announce("FFN down decode", m)
    y = w4.w4a16_linear(x, q, s)
    torch.cuda.synchronize()
    y_ref, mag = oracle.linear(bits(x), p_ref, s_ref)
    r = assert_within(f64(y), y_ref, oracle.linear_bound(mag), f"down M={m}")
    print(f"down M={m}: max err/bound {r:.4f}")


# 4-way tensor-parallel shards of the GLM-130B linears, the layout the pages
# serve INT4 with (paper card, "Paper vs code"): QKV and FFN-up split their
# output rows, attention-out and FFN-down their reduction.
_SHARDS = {"qkv/4": (9216, 12288, False, "normal"), "attn_out/4": (12288, 3072, False, "normal"),
           "down/4": (12288, 8192, False, "t4"), "up_geglu/4": (8192, 12288, True, "t4")}


@pytest.mark.parametrize("name", list(_SHARDS))
def test_tensor_parallel_shard_decode(name):
    """Decode on one GPU's shard at m = 1, 8, 32, 48 (prepacked weights),
    every output against the oracle."""
    n, k, geglu, dist = _SHARDS[name]
    rows = 2 * n if geglu else n
    g = synth.generator(3100 + rows + k, DEV)
    w = synth.weight(rows, k, g, dist, device=DEV)
    q, s, p_ref, s_ref = _quantize_checked(w, f"shard {name} {rows}x{k}")
    del w
    qp = w4.w4a16_prepack(q)
    for m in (1, 8, 32, 48):
        x = synth.activations(m, k, g, DEV)
        announce("shard decode", name, m)
        if geglu:
            y = w4.w4a16_geglu_linear_prepacked(x, qp, s)
            torch.cuda.synchronize()
            gr, a, b, ma, mb = oracle.geglu(bits(x), p_ref, s_ref)
            r = assert_within(f64(y), gr, oracle.geglu_bound(gr, a, b, ma, mb), f"shard {name} M={m}")
        else:
            y = w4.w4a16_linear_prepacked(x, qp, s)
            torch.cuda.synchronize()
            y_ref, mag = oracle.linear(bits(x), p_ref, s_ref)
            r = assert_within(f64(y), y_ref, oracle.linear_bound(mag), f"shard {name} M={m}")
        print(f"shard {name} M={m}: max err/bound {r:.4f}")


def _gather(y, mi, ni):
    """y[mi[t], ni[t]] taken on the device (the full output is large)."""
    return y[torch.as_tensor(mi, device=y.device), torch.as_tensor(ni, device=y.device)].double().cpu().numpy()


def _sample_indices(m, n, tile_m, tile_n, seed):
    """One random token row in every token tile and two random columns in
    every output tile; returns (rows, cols) of the sampled outputs."""
    rng = np.random.default_rng(seed)
    rows = np.array([min(m - 1, t + rng.integers(tile_m)) for t in range(0, m, tile_m)])
    cols = np.concatenate([rng.integers(t, min(n, t + tile_n), 2) for t in range(0, n, tile_n)])
    cols = np.unique(cols)
    mi = np.concatenate([np.repeat(rows, n), np.tile(np.arange(m), cols.size)])
    ni = np.concatenate([np.tile(np.arange(n), rows.size), np.repeat(cols, m)])
    return mi, ni


@pytest.fixture(scope="module")
def prefill_data():
    w_attn, w_up, x = synth.prefill(device=DEV)
    attn = _quantize_checked(w_attn, "attn-out 12288x12288")
    del w_attn
    up = _quantize_checked(w_up, "FFN up 65536x12288")
    del w_up
    return attn, up, x


def test_prefill_attn_out_sampled(prefill_data):
    (q, s, p_ref, s_ref), _, x = prefill_data
    announce("prefill attn-out", tuple(x.shape))
    y = w4.w4a16_linear(x, q, s)
    torch.cuda.synchronize()
    mi, ni = _sample_indices(x.shape[0], q.shape[0], 128, 128, 1)
    y_ref, mag = oracle.linear_at(bits(x), p_ref, s_ref, mi, ni)
    yg = _gather(y, mi, ni)
    r = assert_within(yg, y_ref, oracle.linear_bound(mag), "prefill attn-out")
    print(f"prefill attn-out: {mi.size} sampled outputs, max err/bound {r:.4f}")


def test_prefill_attn_out_m512_sampled(prefill_data):
    """m = 512 runs the small-grid tiles (192 rows x 64 tokens) on the
    attention-out weight: one token in every 64-token tile and two columns
    in every 192-row tile."""
    (q, s, p_ref, s_ref), _, x = prefill_data
    x5 = x[:512].contiguous()
    announce("prefill attn-out", tuple(x5.shape))
    y = w4.w4a16_linear(x5, q, s)
    torch.cuda.synchronize()
    mi, ni = _sample_indices(x5.shape[0], q.shape[0], 64, 192, 6)
    y_ref, mag = oracle.linear_at(bits(x5), p_ref, s_ref, mi, ni)
    r = assert_within(_gather(y, mi, ni), y_ref, oracle.linear_bound(mag), "prefill attn-out m=512")
    print(f"prefill attn-out m=512: {mi.size} sampled outputs, max err/bound {r:.4f}")


def test_prefill_ffn_up_geglu_sampled(prefill_data):
    _, (q, s, p_ref, s_ref), x = prefill_data
    announce("prefill FFN-up GeGLU", tuple(x.shape))
    y = w4.w4a16_geglu_linear(x, q, s)
    torch.cuda.synchronize()
    f = q.shape[0] // 2
    mi, ni = _sample_indices(x.shape[0], f, 128, 64, 2)
    g, a, b, ma, mb = oracle.geglu_at(bits(x), p_ref, s_ref, mi, ni)
    yg = _gather(y, mi, ni)
    r = assert_within(yg, g, oracle.geglu_bound(g, a, b, ma, mb), "prefill FFN-up GeGLU")
    print(f"prefill FFN-up GeGLU: {mi.size} sampled outputs, max err/bound {r:.4f}")


def test_prefill_ffn_up_plain_sampled(prefill_data):
    _, (q, s, p_ref, s_ref), x = prefill_data
    announce("prefill FFN-up plain", tuple(x.shape))
    y = w4.w4a16_linear(x, q, s)
    torch.cuda.synchronize()
    mi, ni = _sample_indices(x.shape[0], q.shape[0], 128, 128, 3)
    keep = np.random.default_rng(4).random(mi.size) < 0.25     # a quarter of the sample
    mi, ni = mi[keep], ni[keep]
    y_ref, mag = oracle.linear_at(bits(x), p_ref, s_ref, mi, ni)
    r = assert_within(_gather(y, mi, ni), y_ref, oracle.linear_bound(mag), "prefill FFN-up plain")
    print(f"prefill FFN-up plain: {mi.size} sampled outputs, max err/bound {r:.4f}")


# ----------------------------------------------------- largest accepted size

def test_largest_accepted_weight():
    """A weight whose packed form is just under the 2 GiB buffer limit the
    kernels address (131040 x 32768: 2 146 959 360 bytes, also as prepacked
    tiles).  Quantized bytes and scales compared in full; decode (m = 8),
    fused GeGLU (m = 8, f = 65520) and prefill (m = 80) on sampled outputs
    of every output tile, row-major and prepacked."""
    n, k = 131040, 32768
    assert w4.w4a16_prepacked_bytes(n, k) < 2 ** 31 and n * k // 2 < 2 ** 31
    g = synth.generator(77, DEV)
    w = synth.weight(n, k, g, device=DEV)
    q, s, p_ref, s_ref = _quantize_checked(w, f"largest {n}x{k}")
    del w
    qp = w4.w4a16_prepack(q)
    for m, tile_m in ((8, 16), (80, 128)):
        x = synth.activations(m, k, g, DEV)
        announce("largest linear", m, n, k)
        mi, ni = _sample_indices(m, n, tile_m, 256, 10 + m)
        y_ref, mag = oracle.linear_at(bits(x), p_ref, s_ref, mi, ni)
        for name, y in (("row-major", w4.w4a16_linear(x, q, s)),
                        ("prepacked", w4.w4a16_linear_prepacked(x, qp, s))):
            torch.cuda.synchronize()
            r = assert_within(_gather(y, mi, ni), y_ref, oracle.linear_bound(mag),
                              f"largest m={m} {name}")
            print(f"largest {n}x{k} m={m} {name}: {mi.size} sampled outputs, max err/bound {r:.4f}")
            del y
    x = synth.activations(8, k, g, DEV)
    mi, ni = _sample_indices(8, n // 2, 16, 256, 30)
    gr, a, b, ma, mb = oracle.geglu_at(bits(x), p_ref, s_ref, mi, ni)
    y = w4.w4a16_geglu_linear_prepacked(x, qp, s)
    torch.cuda.synchronize()
    r = assert_within(_gather(y, mi, ni), gr, oracle.geglu_bound(gr, a, b, ma, mb), "largest GeGLU m=8")
    print(f"largest GeGLU m=8: {mi.size} sampled outputs, max err/bound {r:.4f}")
