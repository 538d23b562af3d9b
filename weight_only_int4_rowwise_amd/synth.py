"""Seeded synthetic inputs at GLM-130B shapes.

This module only draws and arranges numbers.  It holds none of the
quantization or matmul arithmetic, so both the GPU path and the CPU oracle can
be fed from it without sharing any of the method's code.

Recipe (one ``torch.Generator`` per workload, seed 0 unless stated; weights
are drawn before activations):

* N(0, sigma^2) values: ``randn`` in float32, times sigma, rounded to fp16.
* Student-t(nu=4) * scale: Z0 / sqrt((Z1^2 + Z2^2 + Z3^2 + Z4^2) / 4) * scale
  from five successive ``randn`` draws, rounded to fp16 (heavy tails that
  stress the row absmax).
* Activations: N(0, 1) in fp16.

Shapes are GLM-130B's (GLM-130B paper card, "Method" and "Hyperparameters"):
hidden 12288, 96 heads of 128, FFN width 32768 (GeGLU, so the up-projection
has 2 x 32768 output rows), 70 layers, sequence length 2048.
"""
from __future__ import annotations

import torch

HIDDEN = 12288
FFN = 32768
LAYERS = 70
SEQ = 2048
QKV_OUT = 3 * HIDDEN

# (name, out_features, in_features) of the four quantized linears of a layer
# (QKV projection, attention output, GeGLU up-projection, down-projection).
LAYER_LINEARS = (
    ("qkv", QKV_OUT, HIDDEN),
    ("attn_out", HIDDEN, HIDDEN),
    ("ffn_up", 2 * FFN, HIDDEN),
    ("ffn_down", HIDDEN, FFN),
)


def shard_linears(tp: int):
    """The four linears of a layer as one GPU holds them under tp-way tensor
    parallelism: QKV and the GeGLU up-projection split their output rows
    (each GPU keeps a matching slice of gate and value rows, 2 F / tp rows
    in all), attention-out and down split their reduction."""
    return (
        ("qkv", QKV_OUT // tp, HIDDEN),
        ("attn_out", HIDDEN, HIDDEN // tp),
        ("ffn_up", 2 * FFN // tp, HIDDEN),
        ("ffn_down", HIDDEN, FFN // tp),
    )


def generator(seed: int = 0, device: str = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal_fp16(shape, sigma: float, gen: torch.Generator, device: str = "cpu") -> torch.Tensor:
    t = torch.randn(*shape, generator=gen, dtype=torch.float32, device=device)
    if sigma != 1.0:
        t.mul_(sigma)
    return t.to(torch.float16)


def student_t4_fp16(shape, scale: float, gen: torch.Generator, device: str = "cpu") -> torch.Tensor:
    z0 = torch.randn(*shape, generator=gen, dtype=torch.float32, device=device)
    chi = torch.zeros(*shape, dtype=torch.float32, device=device)
    for _ in range(4):
        z = torch.randn(*shape, generator=gen, dtype=torch.float32, device=device)
        chi.addcmul_(z, z)
    return (z0 / torch.sqrt(chi / 4.0) * scale).to(torch.float16)


def weight(n: int, k: int, gen: torch.Generator, dist: str = "normal", device: str = "cpu") -> torch.Tensor:
    """FP16 weight [n][k] (out x in): 'normal' = N(0, 0.02^2), 't4' = t(4) * 0.02."""
    if dist == "normal":
        return normal_fp16((n, k), 0.02, gen, device)
    if dist == "t4":
        return student_t4_fp16((n, k), 0.02, gen, device)
    raise ValueError(dist)


def activations(m: int, k: int, gen: torch.Generator, device: str = "cpu") -> torch.Tensor:
    return normal_fp16((m, k), 1.0, gen, device)


# ---------------------------------------------------------------------------
# Workloads.  Tensors are drawn on `device` with a generator of that device
# (the CPU and GPU generators give different streams for the same seed; both
# sides of a comparison always receive the very same tensors).
# ---------------------------------------------------------------------------

def toy(seed: int = 0, device: str = "cpu"):
    """Weight 1024 x 1024 ~ N(0, 0.02^2); activations for M = 1 and M = 16."""
    g = generator(seed, device)
    w = weight(1024, 1024, g, device=device)
    x1 = activations(1, 1024, g, device)
    x16 = activations(16, 1024, g, device)
    return w, {1: x1, 16: x16}


def qkv_decode(ms=(1, 8, 32, 64), seed: int = 0, device: str = "cpu"):
    """QKV projection 36864 x 12288 ~ N(0, 0.02^2); activations per M."""
    g = generator(seed, device)
    w = weight(QKV_OUT, HIDDEN, g, device=device)
    return w, {m: activations(m, HIDDEN, g, device) for m in ms}


def geglu_decode(ms=(1, 16), seed: int = 0, device: str = "cpu"):
    """GeGLU up 65536 x 12288 and down 12288 x 32768, t(4) * 0.02 weights."""
    g = generator(seed, device)
    w_up = weight(2 * FFN, HIDDEN, g, "t4", device)
    w_down = weight(HIDDEN, FFN, g, "t4", device)
    x_up = {m: activations(m, HIDDEN, g, device) for m in ms}
    x_down = {m: activations(m, FFN, g, device) for m in ms}
    return w_up, w_down, x_up, x_down


def prefill(seed: int = 0, m: int = SEQ, device: str = "cpu"):
    """Attention-out 12288 x 12288 and FFN-up 65536 x 12288 ~ N(0, 0.02^2); M = 2048."""
    g = generator(seed, device)
    w_attn = weight(HIDDEN, HIDDEN, g, device=device)
    w_up = weight(2 * FFN, HIDDEN, g, device=device)
    x = activations(m, HIDDEN, g, device)
    return w_attn, w_up, x


def layer_weight_seed(layer: int, matrix_id: int) -> int:
    """Seed of one matrix of the full-model decode step (drawn on the device)."""
    return 1000 * layer + matrix_id


# ---------------------------------------------------------------------------
# Structured inputs for exact tests (bit patterns only, no method arithmetic)
# ---------------------------------------------------------------------------

def all_finite_nonneg_fp16() -> torch.Tensor:
    """Every finite non-negative fp16 value, +0 .. 65504 (31744 values)."""
    return torch.arange(0, 0x7C00, dtype=torch.int32).to(torch.int16).view(torch.float16)


def enumeration_rows(absmax_bits, k: int) -> torch.Tensor:
    """One row per absmax bit pattern a: the row holds +a, then every fp16
    value v with 0 < |v| <= a (positive bit patterns 1..a, then the same with
    the sign bit), repeated cyclically to fill k entries.  With k >= 2a + 1
    every weight that can occur in a row with absmax a appears in it."""
    a = torch.as_tensor(absmax_bits, dtype=torch.int64).reshape(-1, 1)
    j = torch.arange(k, dtype=torch.int64).reshape(1, -1)
    idx = j % (2 * a + 1)
    val = torch.where(idx == 0, a, torch.where(idx <= a, idx, (idx - a) | 0x8000))
    val = torch.where(val >= 0x8000, val - 0x10000, val)
    return val.to(torch.int16).view(torch.float16)


def exponent_rows(n: int, k: int, gen: torch.Generator, e_lo: int = -8, e_hi: int = 0,
                  top: int = 7) -> torch.Tensor:
    """Rows whose absmax is top * 2^e (e drawn in [e_lo, e_hi]), with every
    other entry an integer j * 2^e or (j + 1/2) * 2^e, |j| < top: exact
    power-of-two grids that hit every rounding tie (top = 7 for the INT4
    code range, 127 for INT8)."""
    e = torch.randint(e_lo, e_hi + 1, (n, 1), generator=gen)
    half_steps = torch.randint(-(2 * top - 1), 2 * top, (n, k), generator=gen).to(torch.float64)
    vals = half_steps * 0.5 * torch.pow(2.0, e.to(torch.float64))
    col = torch.randint(0, k, (n,), generator=gen)
    sign = torch.where(torch.rand(n, generator=gen) < 0.5, -1.0, 1.0).to(torch.float64)
    vals[torch.arange(n), col] = float(top) * torch.pow(2.0, e[:, 0].to(torch.float64)) * sign
    return vals.to(torch.float16)


def range_end_rows(hi, lo, k: int) -> torch.Tensor:
    """One row per pair (hi[i], lo[i]) of fp16 values: the row holds hi, then
    lo, then zeros to k entries (k >= 2), so its range ends are exactly hi and
    lo (and 0)."""
    hi = torch.as_tensor(hi, dtype=torch.float16).reshape(-1)
    lo = torch.as_tensor(lo, dtype=torch.float16).reshape(-1)
    rows = torch.zeros(hi.numel(), k, dtype=torch.float16)
    rows[:, 0] = hi
    rows[:, 1] = lo
    return rows


def asymmetric_range_pairs():
    """(hi, lo) pairs of range ends for rows [hi, lo, 0, ...]: every finite
    positive fp16 hi against lo values with many significant bits (all-ones
    subnormals -(2^j - 1) 2^-24, full-mantissa normals -2047 2^(e-10), and
    -1365 2^-24), then the mirror images (hi, lo) -> (-lo, -hi).  hi - lo then
    needs up to 40 significant bits, and (hi - lo) / 15 lands next to fp16
    midpoints in ways a symmetric range never does."""
    his = all_finite_nonneg_fp16()[1:].to(torch.float64)
    los = ([-(2 ** j - 1) * 2.0 ** -24 for j in range(1, 12)]
           + [-2047 * 2.0 ** (e - 10) for e in range(-14, 0)] + [-1365 * 2.0 ** -24])
    hi = torch.cat([his] * len(los))
    lo = torch.cat([torch.full_like(his, v) for v in los])
    hi, lo = torch.cat([hi, -lo]), torch.cat([lo, -hi])
    return hi.to(torch.float16), lo.to(torch.float16)


def small_int_activations(m: int, k: int, gen: torch.Generator, lo: int = -3, hi: int = 3) -> torch.Tensor:
    """Integer-valued fp16 activations in [lo, hi]."""
    return torch.randint(lo, hi + 1, (m, k), generator=gen).to(torch.float16)


def one_hot_activations(cols, k: int) -> torch.Tensor:
    """Row t is the unit vector e_{cols[t]} of length k."""
    x = torch.zeros(len(cols), k, dtype=torch.float16)
    x[torch.arange(len(cols)), torch.as_tensor(cols)] = 1.0
    return x
