"""Host-side checks of bench.py that need no GPU: argument handling, the
algorithmic byte accounting behind `value`, and the source hash that keys
the committed HBM-traffic counters."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().err


def test_no_gpu_visible_exits_cleanly(capsys):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert bench.main(["--no-cpu-baseline", "--no-extra"]) == 2
    assert "no GPU" in capsys.readouterr().err


@pytest.mark.parametrize("m,expected", [(1, 226_664_448), (8, 227_352_576),
                                        (32, 229_711_872), (64, 232_857_600)])
def test_qkv_decode_bytes(m, expected):
    """Packed weights n k / 2, fp16 scales 2 n, activations 2 m k, outputs
    2 m n for the 36864 x 12288 QKV projection."""
    n, k = 36864, 12288
    assert bench.linear_bytes(m, n, k, n) == n * k // 2 + 2 * n + 2 * m * k + 2 * m * n == expected


def test_geglu_bytes_count_both_halves_of_the_weight():
    """The fused up-projection reads 2 f rows and writes f outputs."""
    f, k, m = 32768, 12288, 1
    assert bench.linear_bytes(m, 2 * f, k, f) == 2 * f * k // 2 + 4 * f + 2 * m * k + 2 * m * f


def test_source_hash_is_stable_and_short():
    h1, h2 = bench.csrc_hash(), bench.csrc_hash()
    assert h1 == h2 and len(h1) == 16 and int(h1, 16) >= 0


@pytest.mark.parametrize("tp", [1, 2, 4, 8])
def test_shard_linears_split_each_layer_evenly(tp):
    """One GPU's shard of a layer: QKV and FFN-up split rows, attention-out
    and down split the reduction; tp shards hold the whole layer."""
    from weight_only_int4_rowwise_amd import synth
    full = {name: (n, k) for name, n, k in synth.LAYER_LINEARS}
    shard = {name: (n, k) for name, n, k in synth.shard_linears(tp)}
    assert shard.keys() == full.keys()
    for name, (n, k) in shard.items():
        fn, fk = full[name]
        assert n * k * tp == fn * fk
        assert (n == fn // tp and k == fk) if name in ("qkv", "ffn_up") else (n == fn and k == fk // tp)
    assert shard["ffn_up"][0] % 2 == 0


def test_int8_bytes_count_one_byte_per_code():
    """INT8 QKV 36864 x 12288 at M = 1: codes n k, scales 2 n, x 2 m k, y 2 m n."""
    n, k, m = 36864, 12288, 1
    assert bench.linear_bytes8(m, n, k, n) == n * k + 2 * n + 2 * m * k + 2 * m * n == 453_156_864
    assert bench.linear_bytes8(m, n, k, n) - bench.linear_bytes(m, n, k, n) == n * k // 2


def test_zero_point_bytes_add_one_byte_per_row():
    n, k, m = 36864, 12288, 8
    assert bench.linear_bytes_zp(m, n, k, n) == bench.linear_bytes(m, n, k, n) + n
