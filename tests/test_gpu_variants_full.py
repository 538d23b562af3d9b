"""GPU parity of the INT8 row-wise (W8A16) and zero-point INT4 variants at the
full GLM-130B shapes, in the launch configurations the benchmark times them
in (prepacked weights, the same shapes, token counts and weight
distributions):

  * QKV decode 36864 x 12288 at M = 1, 8, 32, 64: every output;
  * the fused GeGLU up-projection 65536 x 12288 at M = 1 and 16 on
    Student-t(4) weights, and (INT8) FFN-down 12288 x 32768 at M = 1 and 16:
    every output;
  * attention-out prefill 12288 x 12288 at M = 2048: one token in every
    128-token tile and two columns in every output tile;
  * the INT8 70-layer decode step at M = 8, built and launched as the
    benchmark does (seeds 1000 layer + matrix id, generator 7 inputs): layers
    0 and 69 in full.

Codes, scales and zero points are compared bit for bit with the oracle's
quantization of the same fp16 weights; outputs must lie within the linear
bound (oracle.linear_bound) or the GeGLU bound (oracle.geglu_bound).
Inputs are drawn on the GPU and copied to the host for the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_int4_rowwise_amd as w4
from weight_only_int4_rowwise_amd import synth

import bench
from helpers import announce, assert_bits_equal, assert_within, bits, f64, u8

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
H, F, N = synth.HIDDEN, synth.FFN, synth.QKV_OUT


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w4.library()
    oracle._load()
    yield
    torch.cuda.empty_cache()


def _gather(y, mi, ni):
    return y[torch.as_tensor(mi, device=y.device), torch.as_tensor(ni, device=y.device)].double().cpu().numpy()


def _sample(m, n, tile_m, tile_n, seed):
    """One random token row in every token tile and two random columns in
    every output tile: (token rows, columns, and the flat (mi, ni) pairs of
    the sampled outputs)."""
    rng = np.random.default_rng(seed)
    rows = np.array([min(m - 1, t + rng.integers(tile_m)) for t in range(0, m, tile_m)])
    cols = np.unique(np.concatenate([rng.integers(t, min(n, t + tile_n), 2) for t in range(0, n, tile_n)]))
    mi = np.concatenate([np.repeat(rows, n), np.tile(np.arange(m), cols.size)])
    ni = np.concatenate([np.tile(np.arange(n), rows.size), np.repeat(cols, m)])
    return rows, cols, mi, ni


# ---------------------------------------------------------------- INT8

def _int8_checked(w, what):
    announce("int8 quantize", what, tuple(w.shape))
    q, s = w4.quantize_rowwise_int8(w)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_rowwise_int8(bits(w))
    assert_bits_equal(bits(s), s_ref, f"{what}: scales")
    assert_bits_equal(u8(q), q_ref, f"{what}: codes")
    qp = w4.w8a16_prepack(q)
    del q
    return qp, s, q_ref, s_ref


@pytest.fixture(scope="module")
def int8_qkv():
    w = synth.weight(N, H, synth.generator(0, DEV), device=DEV)
    out = _int8_checked(w, f"QKV {N}x{H}")
    del w
    return out


@pytest.mark.parametrize("m", [1, 8, 32, 64])
def test_int8_qkv_decode_full(int8_qkv, m):
    qp, s, q_ref, s_ref = int8_qkv
    x = synth.activations(m, H, synth.generator(100 + m, DEV), DEV)
    announce("int8 QKV decode", m)
    y = w4.w8a16_linear_prepacked(x, qp, s)
    torch.cuda.synchronize()
    y_ref, mag = oracle.linear_int8(bits(x), q_ref, s_ref)
    r = assert_within(f64(y), y_ref, oracle.linear_bound(mag), f"int8 QKV M={m}")
    print(f"int8 QKV M={m}: max err/bound {r:.4f}")


@pytest.fixture(scope="module")
def int8_ffn():
    g = synth.generator(1, DEV)
    w = synth.weight(2 * F, H, g, "t4", device=DEV)
    up = _int8_checked(w, f"FFN up {2 * F}x{H} t4")
    del w
    w = synth.weight(H, F, g, "t4", device=DEV)
    down = _int8_checked(w, f"FFN down {H}x{F} t4")
    del w
    return up, down


@pytest.mark.parametrize("m", [1, 16])
def test_int8_geglu_up_decode_full(int8_ffn, m):
    (qp, s, q_ref, s_ref), _ = int8_ffn
    x = synth.activations(m, H, synth.generator(200 + m, DEV), DEV)
    announce("int8 GeGLU up decode", m)
    y = w4.w8a16_geglu_linear_prepacked(x, qp, s)
    torch.cuda.synchronize()
    g, a, b, ma, mb = oracle.geglu_int8(bits(x), q_ref, s_ref)
    r = assert_within(f64(y), g, oracle.geglu_bound(g, a, b, ma, mb), f"int8 GeGLU up M={m}")
    print(f"int8 GeGLU up M={m}: max err/bound {r:.4f}")


@pytest.mark.parametrize("m", [1, 16])
def test_int8_down_decode_full(int8_ffn, m):
    _, (qp, s, q_ref, s_ref) = int8_ffn
    x = synth.activations(m, F, synth.generator(300 + m, DEV), DEV)
    announce("int8 FFN down decode", m)
    y = w4.w8a16_linear_prepacked(x, qp, s)
    torch.cuda.synchronize()
    y_ref, mag = oracle.linear_int8(bits(x), q_ref, s_ref)
    r = assert_within(f64(y), y_ref, oracle.linear_bound(mag), f"int8 down M={m}")
    print(f"int8 down M={m}: max err/bound {r:.4f}")


def test_int8_prefill_attn_out_sampled():
    """INT8 attention-out at M = 2048 runs 192-row x 128-token tiles."""
    g = synth.generator(2, DEV)
    w = synth.weight(H, H, g, device=DEV)
    qp, s, q_ref, s_ref = _int8_checked(w, f"attn-out {H}x{H}")
    del w
    x = synth.activations(synth.SEQ, H, g, DEV)
    announce("int8 prefill attn-out", tuple(x.shape))
    y = w4.w8a16_linear_prepacked(x, qp, s)
    torch.cuda.synchronize()
    _, _, mi, ni = _sample(synth.SEQ, H, 128, 192, 21)
    y_ref, mag = oracle.linear_int8_at(bits(x), q_ref, s_ref, mi, ni)
    r = assert_within(_gather(y, mi, ni), y_ref, oracle.linear_bound(mag), "int8 prefill attn-out")
    print(f"int8 prefill attn-out: {mi.size} sampled outputs, max err/bound {r:.4f}")


def test_int8_full_decode_step_70_layers():
    """The INT8 70-layer decode step as the benchmark runs it (280 matrices,
    127 GB of codes resident, M = 8, one stream); layers 0 and 69: codes and
    scales bit-exact, every output of the four linears within the bound."""
    check = (0, synth.LAYERS - 1)
    announce("INT8 70-layer step: building", synth.LAYER_LINEARS)
    step = bench.FullStep(torch, w4, synth, DEV, synth.LAYER_LINEARS, cb=8, keep=check,
                          label="INT8 70-layer step parity")
    snaps = {}

    def snap(layer):
        if layer in check:
            snaps[layer] = [y.clone() for _, _, y in step.calls]

    announce("INT8 70-layer step: 280 launches", step.bytes)
    step.run(after_layer=snap)
    torch.cuda.synchronize()
    for layer in check:
        for (name, n, k), (_, x, _), (w_bits, q_gpu, s_gpu), y in zip(
                step.linears, step.calls, step.kept[layer], snaps[layer]):
            what = f"INT8 layer {layer} {name} {n}x{k}"
            announce("INT8 70-layer step: oracle", what)
            q_ref, s_ref = oracle.quantize_rowwise_int8(w_bits)
            del w_bits
            assert_bits_equal(s_gpu, s_ref, f"{what}: scales")
            assert_bits_equal(q_gpu, q_ref, f"{what}: codes")
            if name == "ffn_up":
                g, a, b, ma, mb = oracle.geglu_int8(bits(x), q_ref, s_ref)
                r = assert_within(f64(y), g, oracle.geglu_bound(g, a, b, ma, mb), what)
            else:
                y_ref, mag = oracle.linear_int8(bits(x), q_ref, s_ref)
                r = assert_within(f64(y), y_ref, oracle.linear_bound(mag), what)
            print(f"{what}: {y.numel()} outputs, max err/bound {r:.4f}", flush=True)
        step.kept[layer] = None
    del step, snaps
    torch.cuda.empty_cache()


# ---------------------------------------------------------- zero-point INT4

def _zp_checked(w, what):
    announce("zp quantize", what, tuple(w.shape))
    q, s, z = w4.quantize_rowwise_int4_zp(w)
    torch.cuda.synchronize()
    p_ref, s_ref, z_ref = oracle.quantize_rowwise_int4_zp(bits(w))
    assert_bits_equal(bits(s), s_ref, f"{what}: scales")
    assert_bits_equal(u8(z), z_ref, f"{what}: zero points")
    assert_bits_equal(u8(q), p_ref, f"{what}: packed codes")
    qp = w4.w4a16_prepack(q)
    del q
    return qp, s, z, p_ref, s_ref, z_ref


@pytest.fixture(scope="module")
def zp_qkv():
    w = synth.weight(N, H, synth.generator(4, DEV), device=DEV)
    out = _zp_checked(w, f"QKV {N}x{H}")
    del w
    return out


@pytest.mark.parametrize("m", [1, 8, 32, 64])
def test_zp_qkv_decode_full(zp_qkv, m):
    qp, s, z, p_ref, s_ref, z_ref = zp_qkv
    x = synth.activations(m, H, synth.generator(400 + m, DEV), DEV)
    announce("zp QKV decode", m)
    y = w4.w4a16_zp_linear_prepacked(x, qp, s, z)
    torch.cuda.synchronize()
    y_ref, mag = oracle.linear_zp(bits(x), p_ref, s_ref, z_ref)
    r = assert_within(f64(y), y_ref, oracle.linear_bound(mag), f"zp QKV M={m}")
    print(f"zp QKV M={m}: max err/bound {r:.4f}")


@pytest.fixture(scope="module")
def zp_up():
    w = synth.weight(2 * F, H, synth.generator(5, DEV), "t4", device=DEV)
    out = _zp_checked(w, f"FFN up {2 * F}x{H} t4")
    del w
    return out


@pytest.mark.parametrize("m", [1, 16])
def test_zp_geglu_up_decode_full(zp_up, m):
    qp, s, z, p_ref, s_ref, z_ref = zp_up
    x = synth.activations(m, H, synth.generator(500 + m, DEV), DEV)
    announce("zp GeGLU up decode", m)
    y = w4.w4a16_zp_geglu_linear_prepacked(x, qp, s, z)
    torch.cuda.synchronize()
    g, a, b, ma, mb = oracle.geglu_zp(bits(x), p_ref, s_ref, z_ref)
    r = assert_within(f64(y), g, oracle.geglu_bound(g, a, b, ma, mb), f"zp GeGLU up M={m}")
    print(f"zp GeGLU up M={m}: max err/bound {r:.4f}")


def test_zp_prefill_attn_out_sampled():
    """Zero-point attention-out at M = 2048 (256-row x 128-token tiles): the
    sampled token rows against the oracle over every column, and the sampled
    columns over every token."""
    g = synth.generator(6, DEV)
    w = synth.weight(H, H, g, device=DEV)
    qp, s, z, p_ref, s_ref, z_ref = _zp_checked(w, f"attn-out {H}x{H}")
    del w
    x = synth.activations(synth.SEQ, H, g, DEV)
    announce("zp prefill attn-out", tuple(x.shape))
    y = w4.w4a16_zp_linear_prepacked(x, qp, s, z)
    torch.cuda.synchronize()
    rows, cols, _, _ = _sample(synth.SEQ, H, 128, 256, 61)
    xb = bits(x)
    y_rows, mag_rows = oracle.linear_zp(xb[rows], p_ref, s_ref, z_ref)
    r1 = assert_within(f64(y[torch.as_tensor(rows, device=y.device)]), y_rows,
                       oracle.linear_bound(mag_rows), "zp prefill attn-out, sampled tokens")
    y_cols, mag_cols = oracle.linear_zp(xb, p_ref[cols], s_ref[cols], z_ref[cols])
    r2 = assert_within(f64(y[:, torch.as_tensor(cols, device=y.device)]), y_cols,
                       oracle.linear_bound(mag_cols), "zp prefill attn-out, sampled columns")
    print(f"zp prefill attn-out: {rows.size} tokens x {H} + {cols.size} columns x {synth.SEQ}, "
          f"max err/bound {max(r1, r2):.4f}")
