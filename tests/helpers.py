"""Shared helpers for the parity tests (marshalling and comparisons only)."""
import sys

import numpy as np
import torch


def bits(t: torch.Tensor) -> np.ndarray:
    """fp16 tensor (any device) -> numpy uint16 bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def announce(*parts):
    """Name the case on stdout before a GPU step (survives a lost box)."""
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def assert_within(y_gpu, y_ref, bound, what):
    y = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y - y_ref)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside the bound; first "
            + ", ".join(f"{tuple(i)}: got {y[tuple(i)]!r} ref {y_ref[tuple(i)]!r} "
                        f"bound {np.asarray(bound)[tuple(i)]!r}" for i in idx))
    return float((err / bound).max()) if err.size else 0.0


def assert_bits_equal(a, b, what):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    neq = a != b
    if neq.any():
        idx = np.argwhere(neq)[:5]
        raise AssertionError(f"{what}: {int(neq.sum())} of {neq.size} differ; first "
                             + ", ".join(f"{tuple(i)}: {a[tuple(i)]:#x} vs {b[tuple(i)]:#x}" for i in idx))
