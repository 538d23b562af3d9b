"""GPU parity at the full GLM-130B shapes, in the launch configurations the
benchmark times.

Inputs are drawn on the GPU (seeded ``torch.Generator('cuda')``; the same
tensors are copied to the host for the oracle).  Quantized bytes and scales
are compared in full; decode outputs (m <= 64) in full; two-launch decode
(m = 100) and prefill outputs (m = 512, 2048) on sampled rows and columns
that touch every output tile.  Each of these calls also runs on the
prepacked layout (the one the benchmark times), whose whole output must
equal the row-major call's bit for bit.  The 70-layer decode step runs as the
benchmark builds and launches it, and its first and last layers are
checked in full.
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w4.library()
    oracle._load()
    yield
    torch.cuda.empty_cache()


def _same_bits(y_prepacked, y, what):
    """Whole outputs of the prepacked and row-major calls, bit for bit
    (compared on the device)."""
    torch.cuda.synchronize()
    differ = int((y_prepacked.view(torch.int16) != y.view(torch.int16)).sum().item())
    assert differ == 0, f"{what}: {differ} of {y.numel()} outputs differ between the layouts"


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
    return q, s, p_ref, s_ref, xs, w4.w4a16_prepack(q)


@pytest.mark.parametrize("m", [1, 8, 32, 64])
def test_qkv_decode_full(qkv, m):
    q, s, p_ref, s_ref, xs, qp = qkv
    x = xs[m]
    announce("QKV decode", m)
    y = w4.w4a16_linear(x, q, s)
    _same_bits(w4.w4a16_linear_prepacked(x, qp, s), y, f"QKV M={m}")
    y_ref, mag = oracle.linear(bits(x), p_ref, s_ref)
    r = assert_within(f64(y), y_ref, oracle.linear_bound(mag), f"QKV M={m}")
    print(f"QKV M={m}: max err/bound {r:.4f}")


def test_qkv_two_decode_launches_sampled(qkv):
    """64 < m <= 128 runs the decode kernel on tokens 0..63, then on the
    rest: QKV at m = 100, one token in every 16-token block and two
    columns in every 144-row workgroup tile, against the oracle."""
    q, s, p_ref, s_ref, _, qp = qkv
    m = 100
    x = synth.activations(m, synth.HIDDEN, synth.generator(7, DEV), DEV)
    announce("QKV two decode launches", m)
    y = w4.w4a16_linear(x, q, s)
    _same_bits(w4.w4a16_linear_prepacked(x, qp, s), y, f"QKV M={m}")
    mi, ni = _sample_indices(m, q.shape[0], 16, 144, 5)
    y_ref, mag = oracle.linear_at(bits(x), p_ref, s_ref, mi, ni)
    r = assert_within(_gather(y, mi, ni), y_ref, oracle.linear_bound(mag), f"QKV M={m}")
    print(f"QKV M={m}: {mi.size} sampled outputs, max err/bound {r:.4f}")


def test_qkv_m128_sampled(qkv):
    """QKV at m = 128 runs the GEMM (192-row x 64-token tiles, reduction
    split over two halves of the workgroup) rather than two decode
    launches: one token in every 16-token block and two columns in every
    192-row tile, against the oracle."""
    q, s, p_ref, s_ref, _, qp = qkv
    m = 128
    x = synth.activations(m, synth.HIDDEN, synth.generator(13, DEV), DEV)
    announce("QKV m=128 GEMM", m)
    y = w4.w4a16_linear(x, q, s)
    _same_bits(w4.w4a16_linear_prepacked(x, qp, s), y, f"QKV M={m}")
    mi, ni = _sample_indices(m, q.shape[0], 16, 192, 14)
    y_ref, mag = oracle.linear_at(bits(x), p_ref, s_ref, mi, ni)
    r = assert_within(_gather(y, mi, ni), y_ref, oracle.linear_bound(mag), f"QKV M={m}")
    print(f"QKV M={m}: {mi.size} sampled outputs, max err/bound {r:.4f}")


def test_qkv_prefill_m1024_sampled(qkv):
    """QKV at m = 1024 runs 256-row x 64-token tiles (the 128-token grid
    would leave half the CUs idle in its last wave): one token in every
    64-token tile and two columns in every 256-row tile, a quarter of that
    sample against the oracle."""
    q, s, p_ref, s_ref, _, qp = qkv
    m = 1024
    x = synth.activations(m, synth.HIDDEN, synth.generator(8, DEV), DEV)
    announce("QKV prefill", m)
    y = w4.w4a16_linear(x, q, s)
    _same_bits(w4.w4a16_linear_prepacked(x, qp, s), y, f"QKV prefill M={m}")
    mi, ni = _sample_indices(m, q.shape[0], 64, 256, 9)
    keep = np.random.default_rng(10).random(mi.size) < 0.25
    mi, ni = mi[keep], ni[keep]
    y_ref, mag = oracle.linear_at(bits(x), p_ref, s_ref, mi, ni)
    r = assert_within(_gather(y, mi, ni), y_ref, oracle.linear_bound(mag), f"QKV prefill M={m}")
    print(f"QKV prefill M={m}: {mi.size} sampled outputs, max err/bound {r:.4f}")


@pytest.fixture(scope="module")
def ffn():
    w_up, w_down, x_up, x_down = synth.geglu_decode(device=DEV)
    up = _quantize_checked(w_up, "FFN up 65536x12288 t4")
    del w_up
    down = _quantize_checked(w_down, "FFN down 12288x32768 t4")
    del w_down
    up = (*up, w4.w4a16_prepack(up[0]))
    down = (*down, w4.w4a16_prepack(down[0]))
    return up, down, x_up, x_down


@pytest.mark.parametrize("m", [1, 16])
def test_geglu_decode_full(ffn, m):
    (q, s, p_ref, s_ref, qp), _, x_up, _ = ffn
    x = x_up[m]
    announce("GeGLU up decode", m)
    y = w4.w4a16_geglu_linear(x, q, s)
    _same_bits(w4.w4a16_geglu_linear_prepacked(x, qp, s), y, f"GeGLU up M={m}")
    g, a, b, ma, mb = oracle.geglu(bits(x), p_ref, s_ref)
    r = assert_within(f64(y), g, oracle.geglu_bound(g, a, b, ma, mb), f"GeGLU up M={m}")
    print(f"GeGLU up M={m}: max err/bound {r:.4f}")


def test_down_prefill_m256_sampled(ffn):
    """FFN-down 12288 x 32768 at m = 256 runs 192-row x 64-token tiles with
    the reduction split over two halves of a 512-thread workgroup: one token
    in every 64-token tile and two columns in every 192-row tile."""
    _, (q, s, p_ref, s_ref, qp), _, _ = ffn
    m = 256
    x = synth.activations(m, synth.FFN, synth.generator(11, DEV), DEV)
    announce("FFN-down prefill", m)
    y = w4.w4a16_linear(x, q, s)
    _same_bits(w4.w4a16_linear_prepacked(x, qp, s), y, f"FFN-down prefill M={m}")
    mi, ni = _sample_indices(m, q.shape[0], 64, 192, 12)
    y_ref, mag = oracle.linear_at(bits(x), p_ref, s_ref, mi, ni)
    r = assert_within(_gather(y, mi, ni), y_ref, oracle.linear_bound(mag), f"FFN-down prefill M={m}")
    print(f"FFN-down prefill M={m}: {mi.size} sampled outputs, max err/bound {r:.4f}")


@pytest.mark.parametrize("m", [1, 16])
def test_down_decode_full(ffn, m):
    _, (q, s, p_ref, s_ref, qp), _, x_down = ffn
    x = x_down[m]
    announce("FFN down decode", m)
    y = w4.w4a16_linear(x, q, s)
    _same_bits(w4.w4a16_linear_prepacked(x, qp, s), y, f"down M={m}")
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
    """Decode on one GPU's shard at every token class, m = 1, 8, 16, 32, 48,
    64 (prepacked weights), every output against the oracle."""
    n, k, geglu, dist = _SHARDS[name]
    rows = 2 * n if geglu else n
    g = synth.generator(3100 + rows + k, DEV)
    w = synth.weight(rows, k, g, dist, device=DEV)
    q, s, p_ref, s_ref = _quantize_checked(w, f"shard {name} {rows}x{k}")
    del w
    qp = w4.w4a16_prepack(q)
    for m in (1, 8, 16, 32, 48, 64):
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
    attn = (*attn, w4.w4a16_prepack(attn[0]))
    up = (*up, w4.w4a16_prepack(up[0]))
    return attn, up, x


def test_prefill_attn_out_sampled(prefill_data):
    """Attention-out at m = 2048: 256-row x 128-token tiles (768 of them,
    a last wave of one workgroup per CU)."""
    (q, s, p_ref, s_ref, qp), _, x = prefill_data
    announce("prefill attn-out", tuple(x.shape))
    y = w4.w4a16_linear(x, q, s)
    _same_bits(w4.w4a16_linear_prepacked(x, qp, s), y, "prefill attn-out")
    mi, ni = _sample_indices(x.shape[0], q.shape[0], 128, 128, 1)
    y_ref, mag = oracle.linear_at(bits(x), p_ref, s_ref, mi, ni)
    yg = _gather(y, mi, ni)
    r = assert_within(yg, y_ref, oracle.linear_bound(mag), "prefill attn-out")
    print(f"prefill attn-out: {mi.size} sampled outputs, max err/bound {r:.4f}")


def test_prefill_attn_out_m512_sampled(prefill_data):
    """m = 512 on the attention-out weight runs 192-row x 128-token tiles
    (one per CU) with the reduction split over two halves of a 512-thread
    workgroup: one token in every 64-token block and two columns in every
    192-row tile."""
    (q, s, p_ref, s_ref, qp), _, x = prefill_data
    x5 = x[:512].contiguous()
    announce("prefill attn-out", tuple(x5.shape))
    y = w4.w4a16_linear(x5, q, s)
    _same_bits(w4.w4a16_linear_prepacked(x5, qp, s), y, "prefill attn-out m=512")
    mi, ni = _sample_indices(x5.shape[0], q.shape[0], 64, 192, 6)
    y_ref, mag = oracle.linear_at(bits(x5), p_ref, s_ref, mi, ni)
    r = assert_within(_gather(y, mi, ni), y_ref, oracle.linear_bound(mag), "prefill attn-out m=512")
    print(f"prefill attn-out m=512: {mi.size} sampled outputs, max err/bound {r:.4f}")


def test_attn_out_m96_gemm_sampled(prefill_data):
    """m = 96 on the attention-out weight (12288 x 12288) runs one GEMM
    launch rather than two decode launches (128-row x 64-token tiles, the
    reduction split over two halves of the workgroup): one token in every
    16-token block and two columns in every 128-row tile."""
    (q, s, p_ref, s_ref, qp), _, x = prefill_data
    x96 = x[:96].contiguous()
    announce("attn-out m=96 GEMM", tuple(x96.shape))
    y = w4.w4a16_linear(x96, q, s)
    _same_bits(w4.w4a16_linear_prepacked(x96, qp, s), y, "attn-out m=96")
    mi, ni = _sample_indices(x96.shape[0], q.shape[0], 16, 128, 9)
    y_ref, mag = oracle.linear_at(bits(x96), p_ref, s_ref, mi, ni)
    r = assert_within(_gather(y, mi, ni), y_ref, oracle.linear_bound(mag), "attn-out m=96")
    print(f"attn-out m=96: {mi.size} sampled outputs, max err/bound {r:.4f}")


def test_prefill_ffn_up_geglu_sampled(prefill_data):
    _, (q, s, p_ref, s_ref, qp), x = prefill_data
    announce("prefill FFN-up GeGLU", tuple(x.shape))
    y = w4.w4a16_geglu_linear(x, q, s)
    _same_bits(w4.w4a16_geglu_linear_prepacked(x, qp, s), y, "prefill FFN-up GeGLU")
    f = q.shape[0] // 2
    mi, ni = _sample_indices(x.shape[0], f, 128, 64, 2)
    g, a, b, ma, mb = oracle.geglu_at(bits(x), p_ref, s_ref, mi, ni)
    yg = _gather(y, mi, ni)
    r = assert_within(yg, g, oracle.geglu_bound(g, a, b, ma, mb), "prefill FFN-up GeGLU")
    print(f"prefill FFN-up GeGLU: {mi.size} sampled outputs, max err/bound {r:.4f}")


def test_prefill_ffn_up_geglu_m512_sampled(prefill_data):
    """The fused FFN-up at m = 512 (128-output x 128-token tiles, 1024 of
    them), prepacked as the benchmark times it: one token in every 128-token
    tile and two columns in every 64-output tile."""
    _, (_, s, p_ref, s_ref, qp), x = prefill_data
    x5 = x[:512].contiguous()
    announce("prefill FFN-up GeGLU", tuple(x5.shape))
    y = w4.w4a16_geglu_linear_prepacked(x5, qp, s)
    torch.cuda.synchronize()
    mi, ni = _sample_indices(x5.shape[0], s.shape[0] // 2, 128, 64, 15)
    g, a, b, ma, mb = oracle.geglu_at(bits(x5), p_ref, s_ref, mi, ni)
    r = assert_within(_gather(y, mi, ni), g, oracle.geglu_bound(g, a, b, ma, mb), "prefill FFN-up GeGLU m=512")
    print(f"prefill FFN-up GeGLU m=512: {mi.size} sampled outputs, max err/bound {r:.4f}")


def test_prefill_ffn_up_plain_sampled(prefill_data):
    _, (q, s, p_ref, s_ref, qp), x = prefill_data
    announce("prefill FFN-up plain", tuple(x.shape))
    y = w4.w4a16_linear(x, q, s)
    _same_bits(w4.w4a16_linear_prepacked(x, qp, s), y, "prefill FFN-up plain")
    mi, ni = _sample_indices(x.shape[0], q.shape[0], 128, 128, 3)
    keep = np.random.default_rng(4).random(mi.size) < 0.25     # a quarter of the sample
    mi, ni = mi[keep], ni[keep]
    y_ref, mag = oracle.linear_at(bits(x), p_ref, s_ref, mi, ni)
    r = assert_within(_gather(y, mi, ni), y_ref, oracle.linear_bound(mag), "prefill FFN-up plain")
    print(f"prefill FFN-up plain: {mi.size} sampled outputs, max err/bound {r:.4f}")


@pytest.mark.parametrize("m", [96, 128, 192, 256, 384])
@pytest.mark.parametrize("weight", ["qkv", "attn_out", "ffn_up_geglu"])
def test_intermediate_m_sampled(qkv, prefill_data, weight, m):
    """The benchmark's intermediate token counts on its three weights,
    prepacked: QKV 36864 x 12288 and the fused FFN-up 65536 x 12288 at
    m = 96 run two decode launches, attention-out at m = 96 and every
    weight from m = 128 one GEMM launch with the tile the launch rule
    picks.  One token in every 32-token block and two columns in every
    128-row block, a quarter of that sample against the oracle."""
    if weight == "qkv":
        _, s, p_ref, s_ref, _, qp = qkv
    else:
        _, s, p_ref, s_ref, qp = prefill_data[0 if weight == "attn_out" else 1]
    geglu = weight == "ffn_up_geglu"
    n = s.shape[0] // 2 if geglu else s.shape[0]
    x = synth.activations(m, synth.HIDDEN, synth.generator(40 + m, DEV), DEV)
    announce("intermediate m", weight, m)
    fn = w4.w4a16_geglu_linear_prepacked if geglu else w4.w4a16_linear_prepacked
    y = fn(x, qp, s)
    torch.cuda.synchronize()
    mi, ni = _sample_indices(m, n, 32, 128, 50 + m)
    keep = np.random.default_rng(51 + m).random(mi.size) < 0.25
    mi, ni = mi[keep], ni[keep]
    if geglu:
        gr, a, b, ma, mb = oracle.geglu_at(bits(x), p_ref, s_ref, mi, ni)
        r = assert_within(_gather(y, mi, ni), gr, oracle.geglu_bound(gr, a, b, ma, mb), f"{weight} m={m}")
    else:
        y_ref, mag = oracle.linear_at(bits(x), p_ref, s_ref, mi, ni)
        r = assert_within(_gather(y, mi, ni), y_ref, oracle.linear_bound(mag), f"{weight} m={m}")
    print(f"{weight} m={m}: {mi.size} sampled outputs, max err/bound {r:.4f}")


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


# ------------------------------------------------- 70-layer decode step

@pytest.mark.timeout(900)
def test_full_decode_step_70_layers():
    """The full-model decode step as the benchmark runs it (GLM-130B paper
    card, "Paper vs code": QKV, attention output and both MLP projections
    quantized in every layer; "Hyperparameters": 70 layers): 280 matrices
    drawn on the GPU with seeds 1000 layer + matrix id, quantized, prepacked
    and resident (63.4 GB), M = 8 inputs from generator 7, all 280 launches
    in one stream.  Layers 0 and 69: packed codes and scales bit-exact with
    the oracle's quantization of the same fp16 weights, and every output of
    QKV, attention-out, the fused GeGLU up-projection and down within the
    bound."""
    check = (0, synth.LAYERS - 1)
    announce("70-layer step: building", synth.LAYER_LINEARS)
    step = bench.FullStep(torch, w4, synth, DEV, synth.LAYER_LINEARS, keep=check,
                          label="70-layer step parity")
    snaps = {}

    def snap(layer):
        if layer in check:
            snaps[layer] = [y.clone() for _, _, y in step.calls]

    announce("70-layer step: 280 launches", step.bytes)
    step.run(after_layer=snap)
    torch.cuda.synchronize()
    for layer in check:
        for (name, n, k), (_, x, _), (w_bits, q_gpu, s_gpu), y in zip(
                step.linears, step.calls, step.kept[layer], snaps[layer]):
            what = f"layer {layer} {name} {n}x{k}"
            announce("70-layer step: oracle", what)
            p_ref, s_ref = oracle.quantize_rowwise_int4(w_bits)
            del w_bits
            assert_bits_equal(s_gpu, s_ref, f"{what}: scales")
            assert_bits_equal(q_gpu, p_ref, f"{what}: packed")
            if name == "ffn_up":
                g, a, b, ma, mb = oracle.geglu(bits(x), p_ref, s_ref)
                r = assert_within(f64(y), g, oracle.geglu_bound(g, a, b, ma, mb), what)
            else:
                y_ref, mag = oracle.linear(bits(x), p_ref, s_ref)
                r = assert_within(f64(y), y_ref, oracle.linear_bound(mag), what)
            print(f"{what}: {y.numel()} outputs, max err/bound {r:.4f}", flush=True)
        step.kept[layer] = None
    del step, snaps
    torch.cuda.empty_cache()
