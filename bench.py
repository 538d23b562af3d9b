#!/usr/bin/env python3
"""Benchmark of the MI355X W4A16 row-wise INT4 path at GLM-130B shapes.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]

Headline workload: the GLM-130B decode QKV projection, weight 36864 x 12288
quantized INT4 row-wise (N(0, 0.02^2) weights), fp16 activations
M in {1, 8, 32, 64}.  One step = one W4A16 linear launch per M (the memory-
bound decode kernel) on the weights in the prepacked tile layout
(w4a16_prepack, applied once at load time like the quantization itself;
same bytes, reordered).  The weights rotate over 5 independently drawn
matrices (1.13 GB of packed weights, over 4x the 256 MB last-level cache),
so every launch streams its weights from HBM.  `value` is the algorithmic
bytes of the step (packed weights + scales + activations + outputs) over
its time: HBM GB/s.  The same step on the row-major packed layout
(w4a16_linear) is reported in `extra`.

The same JSON line also carries, measured in the same run:
  roofline      the dominant decode launch against 8 TB/s HBM
  cpu_baseline  the CPU oracle on a bounded sample of the same workload
  extra         GeGLU decode (fused up-projection, down-projection),
                prefill GEMM TFLOP/s (attention-out and fused FFN-up at
                M = 2048 and 512) against the 2.5 PFLOP/s fp16 MFMA peak, the
                quantizer, and the full 70-layer decode step at M = 8.
Inputs are synthetic, seeded and resident in HBM before timing starts.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_F16_PEAK_TFS = 2516.6     # MI355X dense fp16 MFMA, 2.5 PFLOP/s
METRIC = "W4A16 linear: decode HBM GB/s (% of peak) + prefill TFLOP/s (% MFMA peak)"
DECODE_MS = (1, 8, 32, 64)
ROTATE = 5


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def linear_bytes(m, n_rows, k, n_out):
    """Algorithmic bytes of one W4A16 linear: packed weights, fp16 scales,
    fp16 activations in, fp16 outputs out."""
    return n_rows * k // 2 + 2 * n_rows + 2 * m * k + 2 * m * n_out


def csrc_hash():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "weight_only_int4_rowwise_amd", "csrc")
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def time_launches(torch, fn, reps, warm=2, repeats=5):
    """Duration (s) of one fn() call: the median over `repeats` timings of
    reps back-to-back launches each, timed with events on the current stream
    (the stream the kernels run on)."""
    for _ in range(warm):
        fn()
    times = []
    for _ in range(repeats):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        e.synchronize()
        times.append(s.elapsed_time(e) / 1e3 / reps)
    return sorted(times)[len(times) // 2]


def make_rotating(torch, w4, synth, n, k, dist, count, seed0, dev):
    """count independently drawn weights: (row-major packed, scales, prepacked)."""
    qs = []
    for i in range(count):
        g = synth.generator(seed0 + i, dev)
        w = synth.weight(n, k, g, dist, dev)
        q, s = w4.quantize_rowwise_int4(w)
        del w
        qs.append((q, s, w4.w4a16_prepack(q)))
    torch.cuda.synchronize()
    return qs


def make_rotating8(torch, w4, synth, n, k, dist, count, seed0, dev):
    """count independently drawn weights in INT8: (prepacked codes, scales)."""
    qs = []
    for i in range(count):
        g = synth.generator(seed0 + i, dev)
        w = synth.weight(n, k, g, dist, dev)
        q, s = w4.quantize_rowwise_int8(w)
        del w
        qs.append((w4.w8a16_prepack(q), s))
        del q
    torch.cuda.synchronize()
    return qs


def linear_bytes8(m, n_rows, k, n_out):
    """Algorithmic bytes of one INT8 linear call: codes n k, fp16 scales,
    activations in, outputs out."""
    return n_rows * k + 2 * n_rows + 2 * m * k + 2 * m * n_out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the non-headline workloads")
    ap.add_argument("--no-full-step", action="store_true", help="skip the 70-layer decode step")
    a = ap.parse_args(argv)

    if a.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {a.gpus}); "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import weight_only_int4_rowwise_amd as w4
    from weight_only_int4_rowwise_amd import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    w4.library()      # raises if the HIP library is not built
    dev = "cuda:0"
    torch.cuda.set_device(0)
    N, K = synth.QKV_OUT, synth.HIDDEN

    # ------------------------------------------------------------ headline
    log(f"preparing {ROTATE} QKV weights {N}x{K} on the GPU")
    qkv = make_rotating(torch, w4, synth, N, K, "normal", ROTATE, 10, dev)
    gx = synth.generator(0, dev)
    xs = {m: synth.activations(m, K, gx, dev) for m in DECODE_MS}
    ys = {m: torch.empty(m, N, dtype=torch.float16, device=dev) for m in DECODE_MS}
    step_bytes = sum(linear_bytes(m, N, K, N) for m in DECODE_MS)

    it = [0]

    def step():
        for m in DECODE_MS:
            _, s, qp = qkv[it[0] % ROTATE]
            it[0] += 1
            w4.w4a16_linear_prepacked(xs[m], qp, s, y_out=ys[m])

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(a.steps):
        step()
    t1.record()
    t1.synchronize()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / a.steps
    value = step_bytes / (ms_step / 1e3) / 1e9
    log(f"headline: {ms_step * 1e3:.1f} us/step, {value:.0f} GB/s")

    # per-M launch durations (roofline of the dominant decode launch), both layouts
    per_m, per_m_rm = {}, {}
    for m in DECODE_MS:
        for layout, table in (("prepacked", per_m), ("row-major", per_m_rm)):
            j = [0]

            def one(m=m, j=j, layout=layout):
                q, s, qp = qkv[j[0] % ROTATE]
                j[0] += 1
                if layout == "prepacked":
                    w4.w4a16_linear_prepacked(xs[m], qp, s, y_out=ys[m])
                else:
                    w4.w4a16_linear(xs[m], q, s, y_out=ys[m])

            t = time_launches(torch, one, 40)
            b = linear_bytes(m, N, K, N)
            table[m] = {"us": round(t * 1e6, 2), "bytes": b, "GBs": round(b / t / 1e9, 1),
                        "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 4),
                        "mfma_frac_needed": round(2.0 * m * N * K / t / 1e12 / MFMA_F16_PEAK_TFS, 4)}
            log(f"decode QKV M={m} {layout}: {t * 1e6:.1f} us, {b / t / 1e9:.0f} GB/s")
    dom = max(DECODE_MS, key=lambda m: per_m[m]["us"])
    mb = (dom + 15) // 16
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "decode_qkv_traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as fh:
            tr = json.load(fh)
        if tr.get("csrc_hash") == csrc_hash() and str(dom) in tr.get("bytes_per_launch", {}):
            traffic = tr["bytes_per_launch"][str(dom)]
    roofline = {
        "bound": "hbm",
        "kernel": f"decode_kernel, M={dom} ({mb} token block{'s' if mb > 1 else ''}), prepacked "
                  "QKV 36864x12288",
        "achieved": per_m[dom]["GBs"],
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(per_m[dom]["GBs"] / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "algorithmic_bytes_per_launch": per_m[dom]["bytes"],
        "avg_launch_us": per_m[dom]["us"],
    }

    # ------------------------------------------------------- cpu baseline
    cpu = None
    if not a.no_cpu_baseline:
        import oracle
        rows = 24576          # two thirds of the QKV rows: about 10-20 s of CPU work
        q0, s0, _ = qkv[0]
        p_host = q0[:rows].cpu().numpy()
        s_host = s0[:rows].cpu().view(torch.int16).numpy().view("uint16")
        tot_b, tot_t = 0, 0.0
        for m in DECODE_MS:
            xh = xs[m].cpu().view(torch.int16).numpy().view("uint16")
            c0 = time.perf_counter()
            oracle.linear(xh, p_host, s_host)
            tot_t += time.perf_counter() - c0
            tot_b += linear_bytes(m, rows, K, rows)
        cpu = {"value": round(tot_b / tot_t / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
               "kind": "oracle",
               "sample": f"oracle.linear (fp64, plain loops, OpenMP over outputs) on the first {rows} of "
                         f"{N} QKV rows at M = 1, 8, 32, 64 ({tot_t:.1f} s of CPU time); "
                         "same algorithmic-byte accounting as value"}
        log(f"cpu baseline: {cpu['value']} GB/s on {cpu['cores']} threads")

    # -------------------------------------------------------------- extra
    tot_b = sum(per_m_rm[m]["bytes"] for m in DECODE_MS)
    tot_t = sum(per_m_rm[m]["us"] for m in DECODE_MS) / 1e6
    extra = {"decode_qkv_per_m": {str(m): v for m, v in per_m.items()},
             "decode_qkv_row_major_per_m": {str(m): v for m, v in per_m_rm.items()},
             "decode_qkv_row_major_step_GBs": round(tot_b / tot_t / 1e9, 1)}
    del ys
    if not a.no_extra:
        extra.update(extra_workloads(torch, w4, synth, dev, a))

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": "GLM-130B decode QKV projection: INT4 row-wise weight 36864x12288 "
                        "(N(0,0.02^2)), fp16 activations M in {1,8,32,64}, one launch per M per step, "
                        "weights in the prepacked tile layout",
            "N": N, "K": K, "M": list(DECODE_MS),
            "rotating_weight_buffers": ROTATE,
            "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)
    return 0


def extra_workloads(torch, w4, synth, dev, a):
    res = {}
    H, F = synth.HIDDEN, synth.FFN

    # GeGLU decode: fused up-projection 65536 x 12288 and down 12288 x 32768, t(4) weights
    log("GeGLU decode")
    ups = make_rotating(torch, w4, synth, 2 * F, H, "t4", 3, 100, dev)
    downs = make_rotating(torch, w4, synth, H, F, "t4", 5, 200, dev)
    g = synth.generator(1, dev)
    gd = {}
    for m in (1, 16):
        xu = synth.activations(m, H, g, dev)
        xd = synth.activations(m, F, g, dev)
        yu = torch.empty(m, F, dtype=torch.float16, device=dev)
        yd = torch.empty(m, H, dtype=torch.float16, device=dev)
        c = [0]

        def up(c=c, xu=xu, yu=yu):
            _, s, qp = ups[c[0] % len(ups)]
            c[0] += 1
            w4.w4a16_geglu_linear_prepacked(xu, qp, s, y_out=yu)

        def down(c=c, xd=xd, yd=yd):
            _, s, qp = downs[c[0] % len(downs)]
            c[0] += 1
            w4.w4a16_linear_prepacked(xd, qp, s, y_out=yd)

        tu = time_launches(torch, up, 30)
        td = time_launches(torch, down, 30)
        bu = linear_bytes(m, 2 * F, H, F)
        bd = linear_bytes(m, H, F, H)
        gd[str(m)] = {"up_geglu_us": round(tu * 1e6, 2), "up_geglu_GBs": round(bu / tu / 1e9, 1),
                      "down_us": round(td * 1e6, 2), "down_GBs": round(bd / td / 1e9, 1)}
        log(f"GeGLU decode M={m}: up {bu / tu / 1e9:.0f} GB/s, down {bd / td / 1e9:.0f} GB/s")
    res["decode_geglu_ffn"] = gd
    del downs

    # prefill: attention-out 12288 x 12288 and FFN-up 65536 x 12288 at M = 2048
    log("prefill")
    M = synth.SEQ
    attn = make_rotating(torch, w4, synth, H, H, "normal", 2, 300, dev)
    x = synth.activations(M, H, g, dev)
    pf = {}
    def rec(t, fl):
        return {"us": round(t * 1e6, 1), "TFLOPs": round(fl / t / 1e12, 1),
                "frac_mfma": round(fl / t / 1e12 / MFMA_F16_PEAK_TFS, 4)}

    y1 = torch.empty(M, H, dtype=torch.float16, device=dev)
    fl = 2.0 * M * H * H
    pf["attn_out"] = rec(time_launches(
        torch, lambda: w4.w4a16_linear_prepacked(x, attn[0][2], attn[0][1], y_out=y1), 10), fl)
    pf["attn_out_row_major"] = rec(time_launches(
        torch, lambda: w4.w4a16_linear(x, attn[0][0], attn[0][1], y_out=y1), 10), fl)
    del y1
    y2 = torch.empty(M, F, dtype=torch.float16, device=dev)
    fl = 2.0 * M * 2 * F * H
    pf["ffn_up_geglu"] = rec(time_launches(
        torch, lambda: w4.w4a16_geglu_linear_prepacked(x, ups[0][2], ups[0][1], y_out=y2), 5), fl)
    pf["ffn_up_geglu_row_major"] = rec(time_launches(
        torch, lambda: w4.w4a16_geglu_linear(x, ups[0][0], ups[0][1], y_out=y2), 5), fl)
    del y2
    y3 = torch.empty(M, 2 * F, dtype=torch.float16, device=dev)
    pf["ffn_up_plain"] = rec(time_launches(
        torch, lambda: w4.w4a16_linear_prepacked(x, ups[0][2], ups[0][1], y_out=y3), 5), fl)
    del y3
    # the fp16 GEMM of the same shape through torch, as a context ceiling
    wf = synth.weight(H, H, g, device=dev)
    yt = torch.empty(M, H, dtype=torch.float16, device=dev)
    t = time_launches(torch, lambda: torch.matmul(x, wf.t(), out=yt), 10)
    pf["context_torch_fp16_matmul_attn_out"] = {"us": round(t * 1e6, 1),
                                                "TFLOPs": round(2.0 * M * H * H / t / 1e12, 1)}
    del wf, yt
    res["prefill_m2048"] = pf
    log(f"prefill: {pf}")

    # prefill at M = 512 (the short end of the prefill range): attention-out
    # and the fused FFN-up, prepacked, with torch's fp16 GEMM as context
    M5 = 512
    x5 = synth.activations(M5, H, g, dev)
    pf5 = {}
    y5 = torch.empty(M5, H, dtype=torch.float16, device=dev)
    pf5["attn_out"] = rec(time_launches(
        torch, lambda: w4.w4a16_linear_prepacked(x5, attn[0][2], attn[0][1], y_out=y5), 20),
        2.0 * M5 * H * H)
    wf = synth.weight(H, H, g, device=dev)
    t = time_launches(torch, lambda: torch.matmul(x5, wf.t(), out=y5), 20)
    pf5["context_torch_fp16_matmul_attn_out"] = {"us": round(t * 1e6, 1),
                                                 "TFLOPs": round(2.0 * M5 * H * H / t / 1e12, 1)}
    del wf, y5
    y6 = torch.empty(M5, F, dtype=torch.float16, device=dev)
    pf5["ffn_up_geglu"] = rec(time_launches(
        torch, lambda: w4.w4a16_geglu_linear_prepacked(x5, ups[0][2], ups[0][1], y_out=y6), 10),
        2.0 * M5 * 2 * F * H)
    del y6, x5
    res["prefill_m512"] = pf5
    log(f"prefill M=512: {pf5}")
    del ups, attn

    res["w8a16"] = int8_workloads(torch, w4, synth, dev, g)
    res["w4a16_zp"] = zp_workloads(torch, w4, synth, dev, g)

    # quantizer: QKV-shaped fp16 weight -> packed + scales
    log("quantizer")
    wq = synth.weight(synth.QKV_OUT, H, g, device=dev)
    qo = torch.empty(synth.QKV_OUT, H // 2, dtype=torch.uint8, device=dev)
    so = torch.empty(synth.QKV_OUT, dtype=torch.float16, device=dev)
    t = time_launches(torch, lambda: w4.quantize_rowwise_int4(wq, q_out=qo, s_out=so), 10)
    qb = synth.QKV_OUT * H * 2 + synth.QKV_OUT * H // 2 + 2 * synth.QKV_OUT
    res["quantize_qkv"] = {"us": round(t * 1e6, 1), "GBs": round(qb / t / 1e9, 1),
                           "frac_hbm": round(qb / t / 1e9 / HBM_PEAK_GBS, 4)}
    del qo
    # the variants' quantizers on the same weight: INT8 codes (one byte per
    # code) and the zero-point codes (packed codes, scales, zero points)
    co = torch.empty(synth.QKV_OUT, H, dtype=torch.int8, device=dev)
    t = time_launches(torch, lambda: w4.quantize_rowwise_int8(wq, q_out=co, s_out=so), 10)
    qb8 = synth.QKV_OUT * H * 2 + synth.QKV_OUT * H + 2 * synth.QKV_OUT
    res["quantize_qkv_int8"] = {"us": round(t * 1e6, 1), "GBs": round(qb8 / t / 1e9, 1),
                                "frac_hbm": round(qb8 / t / 1e9 / HBM_PEAK_GBS, 4)}
    del co
    qo = torch.empty(synth.QKV_OUT, H // 2, dtype=torch.uint8, device=dev)
    zo = torch.empty(synth.QKV_OUT, dtype=torch.uint8, device=dev)
    t = time_launches(torch, lambda: w4.quantize_rowwise_int4_zp(wq, q_out=qo, s_out=so, z_out=zo), 10)
    qbz = qb + synth.QKV_OUT
    res["quantize_qkv_zero_point"] = {"us": round(t * 1e6, 1), "GBs": round(qbz / t / 1e9, 1),
                                      "frac_hbm": round(qbz / t / 1e9 / HBM_PEAK_GBS, 4)}
    log(f"quantizers: {res['quantize_qkv']} int8 {res['quantize_qkv_int8']} "
        f"zero-point {res['quantize_qkv_zero_point']}")
    del wq, qo, so, zo

    if not a.no_full_step:
        res["full_decode_step_m8"] = full_step(torch, w4, synth, dev, synth.LAYER_LINEARS,
                                               "full 70-layer decode step")
        # one GPU's share of the model under 4-way tensor parallelism (the
        # layout the pages serve INT4 with): the same step on the shard shapes
        res["full_decode_step_m8_tp4_shard"] = full_step(torch, w4, synth, dev, synth.shard_linears(4),
                                                         "70-layer decode step, 4-way shard")
        res["w8a16"]["full_decode_step_m8"] = full_step(torch, w4, synth, dev, synth.LAYER_LINEARS,
                                                        "INT8 70-layer decode step", cb=8)
    return res


def linear_bytes_zp(m, n_rows, k, n_out):
    """Algorithmic bytes of one zero-point INT4 linear call: packed codes,
    fp16 scales, uint8 zero points, activations in, outputs out."""
    return linear_bytes(m, n_rows, k, n_out) + n_rows


def zp_workloads(torch, w4, synth, dev, g):
    """The zero-point INT4 variant at the GLM-130B shapes: QKV decode per M,
    the fused GeGLU up-projection at M = 1 and 16, and attention-out prefill
    at M = 2048, all prepacked."""
    log("zero-point INT4 workloads")
    H, F, N = synth.HIDDEN, synth.FFN, synth.QKV_OUT

    def rotating(n, k, dist, count, seed0):
        out = []
        for i in range(count):
            w = synth.weight(n, k, synth.generator(seed0 + i, dev), dist, dev)
            q, s, z = w4.quantize_rowwise_int4_zp(w)
            del w
            out.append((w4.w4a16_prepack(q), s, z))
            del q
        torch.cuda.synchronize()
        return out

    r = {}
    qkv = rotating(N, H, "normal", 5, 900)
    per_m = {}
    for m in DECODE_MS:
        x = synth.activations(m, H, g, dev)
        y = torch.empty(m, N, dtype=torch.float16, device=dev)
        c = [0]

        def one(c=c, x=x, y=y):
            qp, s, z = qkv[c[0] % len(qkv)]
            c[0] += 1
            w4.w4a16_zp_linear_prepacked(x, qp, s, z, y_out=y)

        t = time_launches(torch, one, 30)
        b = linear_bytes_zp(m, N, H, N)
        per_m[str(m)] = {"us": round(t * 1e6, 2), "bytes": b, "GBs": round(b / t / 1e9, 1),
                         "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 4)}
    r["decode_qkv_per_m"] = per_m
    log(f"zero-point QKV decode: {per_m}")
    del qkv
    ups = rotating(2 * F, H, "t4", 3, 950)
    gd = {}
    for m in (1, 16):
        xu = synth.activations(m, H, g, dev)
        yu = torch.empty(m, F, dtype=torch.float16, device=dev)
        c = [0]

        def up(c=c, xu=xu, yu=yu):
            qp, s, z = ups[c[0] % len(ups)]
            c[0] += 1
            w4.w4a16_zp_geglu_linear_prepacked(xu, qp, s, z, y_out=yu)

        t = time_launches(torch, up, 20)
        b = linear_bytes_zp(m, 2 * F, H, F)
        gd[str(m)] = {"up_geglu_us": round(t * 1e6, 2), "up_geglu_GBs": round(b / t / 1e9, 1)}
    r["decode_geglu_up"] = gd
    del ups
    attn = rotating(H, H, "normal", 1, 990)
    M = synth.SEQ
    x = synth.activations(M, H, g, dev)
    y = torch.empty(M, H, dtype=torch.float16, device=dev)
    t = time_launches(torch, lambda: w4.w4a16_zp_linear_prepacked(x, attn[0][0], attn[0][1], attn[0][2],
                                                                    y_out=y), 10)
    fl = 2.0 * M * H * H
    r["prefill_m2048_attn_out"] = {"us": round(t * 1e6, 1), "TFLOPs": round(fl / t / 1e12, 1),
                                   "frac_mfma": round(fl / t / 1e12 / MFMA_F16_PEAK_TFS, 4)}
    log(f"zero-point GeGLU and prefill: {gd} {r['prefill_m2048_attn_out']}")
    del attn, x, y
    torch.cuda.empty_cache()
    return r


def int8_workloads(torch, w4, synth, dev, g):
    """The INT8 row-wise variant (W8A16) at the GLM-130B shapes: QKV decode
    per M, the fused GeGLU up-projection and down at M = 1 and 16, and the
    attention-out prefill at M = 2048, all prepacked."""
    log("INT8 (W8A16) workloads")
    H, F, N = synth.HIDDEN, synth.FFN, synth.QKV_OUT
    r = {}
    qkv = make_rotating8(torch, w4, synth, N, H, "normal", 3, 500, dev)
    per_m = {}
    for m in DECODE_MS:
        x = synth.activations(m, H, g, dev)
        y = torch.empty(m, N, dtype=torch.float16, device=dev)
        c = [0]

        def one(c=c, x=x, y=y):
            qp, s = qkv[c[0] % len(qkv)]
            c[0] += 1
            w4.w8a16_linear_prepacked(x, qp, s, y_out=y)

        t = time_launches(torch, one, 30)
        b = linear_bytes8(m, N, H, N)
        per_m[str(m)] = {"us": round(t * 1e6, 2), "bytes": b, "GBs": round(b / t / 1e9, 1),
                         "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 4)}
    r["decode_qkv_per_m"] = per_m
    log(f"INT8 QKV decode: {per_m}")
    del qkv
    ups = make_rotating8(torch, w4, synth, 2 * F, H, "t4", 2, 600, dev)
    downs = make_rotating8(torch, w4, synth, H, F, "t4", 3, 700, dev)
    gd = {}
    for m in (1, 16):
        xu = synth.activations(m, H, g, dev)
        xd = synth.activations(m, F, g, dev)
        yu = torch.empty(m, F, dtype=torch.float16, device=dev)
        yd = torch.empty(m, H, dtype=torch.float16, device=dev)
        c = [0]

        def up(c=c, xu=xu, yu=yu):
            qp, s = ups[c[0] % len(ups)]
            c[0] += 1
            w4.w8a16_geglu_linear_prepacked(xu, qp, s, y_out=yu)

        def down(c=c, xd=xd, yd=yd):
            qp, s = downs[c[0] % len(downs)]
            c[0] += 1
            w4.w8a16_linear_prepacked(xd, qp, s, y_out=yd)

        tu = time_launches(torch, up, 20)
        td = time_launches(torch, down, 20)
        bu = linear_bytes8(m, 2 * F, H, F)
        bd = linear_bytes8(m, H, F, H)
        gd[str(m)] = {"up_geglu_us": round(tu * 1e6, 2), "up_geglu_GBs": round(bu / tu / 1e9, 1),
                      "down_us": round(td * 1e6, 2), "down_GBs": round(bd / td / 1e9, 1)}
    r["decode_geglu_ffn"] = gd
    log(f"INT8 GeGLU decode: {gd}")
    del ups, downs
    attn = make_rotating8(torch, w4, synth, H, H, "normal", 1, 800, dev)
    M = synth.SEQ
    x = synth.activations(M, H, g, dev)
    y = torch.empty(M, H, dtype=torch.float16, device=dev)
    t = time_launches(torch, lambda: w4.w8a16_linear_prepacked(x, attn[0][0], attn[0][1], y_out=y), 10)
    fl = 2.0 * M * H * H
    r["prefill_m2048_attn_out"] = {"us": round(t * 1e6, 1), "TFLOPs": round(fl / t / 1e12, 1),
                                   "frac_mfma": round(fl / t / 1e12 / MFMA_F16_PEAK_TFS, 4)}
    log(f"INT8 prefill: {r['prefill_m2048_attn_out']}")
    del attn, x, y
    torch.cuda.empty_cache()
    return r


def full_step(torch, w4, synth, dev, linears, label, cb=4):
    """70 layers x the four linears of `linears` (name, rows, k) at M = 8,
    all weights resident and prepacked (INT4, or INT8 for cb = 8), launched
    back to back on one stream."""
    log(f"{label}: generating and quantizing {synth.LAYERS * len(linears)} matrices")
    layers = []
    for l in range(synth.LAYERS):
        mats = []
        for mid, (name, n, k) in enumerate(linears):
            g = synth.generator(synth.layer_weight_seed(l, mid), dev)
            w = synth.weight(n, k, g, device=dev)
            if cb == 8:
                q, s = w4.quantize_rowwise_int8(w)
                del w
                mats.append((w4.w8a16_prepack(q), s))
            else:
                q, s = w4.quantize_rowwise_int4(w)
                del w
                mats.append((w4.w4a16_prepack(q), s))
            del q
        layers.append(mats)
    torch.cuda.synchronize()
    g = synth.generator(7, dev)
    M = 8
    xs = {k: synth.activations(M, k, g, dev) for k in sorted({k for _, _, k in linears})}
    calls = []
    total = 0
    for name, n, k in linears:
        geglu = name == "ffn_up"
        out = n // 2 if geglu else n
        if cb == 8:
            fn = w4.w8a16_geglu_linear_prepacked if geglu else w4.w8a16_linear_prepacked
            total += linear_bytes8(M, n, k, out)
        else:
            fn = w4.w4a16_geglu_linear_prepacked if geglu else w4.w4a16_linear_prepacked
            total += linear_bytes(M, n, k, out)
        calls.append((fn, xs[k], torch.empty(M, out, dtype=torch.float16, device=dev)))
    total *= synth.LAYERS

    def run():
        for mats in layers:
            for (fn, x, y), (qp, s) in zip(calls, mats):
                fn(x, qp, s, y_out=y)

    t = time_launches(torch, run, 3, warm=1)
    r = {"ms": round(t * 1e3, 3), "bytes": total, "GBs": round(total / t / 1e9, 1),
         "frac_hbm": round(total / t / 1e9 / HBM_PEAK_GBS, 4),
         "shapes": [[name, n, k] for name, n, k in linears]}
    log(f"{label}: {r}")
    del layers
    torch.cuda.empty_cache()
    return r


if __name__ == "__main__":
    sys.exit(main())
