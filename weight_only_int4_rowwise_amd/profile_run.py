"""Fixed launch sequence for hardware-counter runs (rocprofv3 --pmc).

    python -m weight_only_int4_rowwise_amd.profile_run --m 64 --reps 10

Launches the decode QKV linear (36864 x 12288 INT4 row-wise weights, or
INT8 ones with --codes int8, rotating over 5 matrices so every launch
streams from HBM; prepacked or row-major layout) `reps` times at token
count m, then a plain device-to-device copy of exactly 1 GiB (torch
copy_) `reps` times.  The copy has a known HBM traffic (1 GiB read, 1 GiB
written per launch), which calibrates what FETCH_SIZE / WRITE_SIZE report
per byte on this GPU.
"""
from __future__ import annotations

import argparse
import sys


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--m", type=int, default=64)
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--layout", choices=("prepacked", "row-major"), default="prepacked")
    ap.add_argument("--codes", choices=("int4", "int8"), default="int4")
    a = ap.parse_args(argv)

    import torch
    import weight_only_int4_rowwise_amd as w4
    from weight_only_int4_rowwise_amd import synth

    dev = "cuda:0"
    n, k = synth.QKV_OUT, synth.HIDDEN
    qs = []
    int8 = a.codes == "int8"
    for i in range(5):
        w = synth.weight(n, k, synth.generator(10 + i, dev), device=dev)
        q, s = w4.quantize_rowwise_int8(w) if int8 else w4.quantize_rowwise_int4(w)
        del w
        qs.append((q, s, w4.w8a16_prepack(q) if int8 else w4.w4a16_prepack(q)))
    x = synth.activations(a.m, k, synth.generator(0, dev), dev)
    y = torch.empty(a.m, n, dtype=torch.float16, device=dev)
    torch.cuda.synchronize()
    print(f"decode QKV m={a.m} ({a.codes}, {a.layout}): {a.reps} launches", flush=True)
    lin, lin_p = (w4.w8a16_linear, w4.w8a16_linear_prepacked) if int8 else (w4.w4a16_linear, w4.w4a16_linear_prepacked)
    for r in range(a.reps):
        q, s, qp = qs[r % 5]
        if a.layout == "prepacked":
            lin_p(x, qp, s, y_out=y)
        else:
            lin(x, q, s, y_out=y)
    torch.cuda.synchronize()
    src = torch.empty(a.copy_bytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    print(f"copy {a.copy_bytes} bytes: {a.reps} launches", flush=True)
    for _ in range(a.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("done", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
