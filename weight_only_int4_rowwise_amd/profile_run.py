"""Fixed launch sequences for profiler runs (rocprofv3 --pmc / --kernel-trace),
and the summaries made from their output.

    python -m weight_only_int4_rowwise_amd.profile_run decode --m 64 --reps 10
    python -m weight_only_int4_rowwise_amd.profile_run prefill --reps 5
    python -m weight_only_int4_rowwise_amd.profile_run step --reps 20
    python -m weight_only_int4_rowwise_amd.profile_run summarize-pmc DIR...
    python -m weight_only_int4_rowwise_amd.profile_run summarize-trace DIR
    python -m weight_only_int4_rowwise_amd.profile_run step-timeline DIR --after-ms 60

decode   the decode QKV linear (36864 x 12288 INT4 row-wise weights, or INT8
         ones with --codes int8; prepacked or row-major) `reps` times at token
         count m, rotating over 5 matrices so every launch streams from HBM.
prefill  the prefill GEMMs at M = 2048 tokens on prepacked weights:
         attention-out 12288 x 12288, then the fused GeGLU FFN-up
         65536 x 12288 (--which selects one), `reps` times each.
step     the decode step of the benchmark's headline workload: QKV at
         M = 1, 8, 32, 64 (or the --ms list), one launch each, back to
         back, `reps` times.
Each mode ends with a plain device-to-device copy of exactly 1 GiB (torch
copy_) `reps` times, whose HBM traffic is known (1 GiB read and 1 GiB
written per launch): it calibrates what FETCH_SIZE / WRITE_SIZE report per
byte, and its kernel marks the end of the sequence in a trace.

summarize-pmc reads the counter CSVs of one or more rocprofv3 --pmc runs
and prints, per kernel, the mean of every counter per dispatch;
summarize-trace reads a --kernel-trace CSV and prints the per-kernel
durations and, for the step mode, the gaps between consecutive launches;
step-timeline reads the --kernel-trace CSV of a step run and prints, over
the launches that start after --after-ms (past the post-idle clock
transient), each launch's mean duration and the mean gap from the previous
launch's end to its start, and the mean step period.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import sys
from collections import OrderedDict, defaultdict


def _decode(a, torch, w4, synth, dev):
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
    lin, lin_p = ((w4.w8a16_linear, w4.w8a16_linear_prepacked) if int8
                  else (w4.w4a16_linear, w4.w4a16_linear_prepacked))
    for r in range(a.reps):
        q, s, qp = qs[r % 5]
        if a.layout == "prepacked":
            lin_p(x, qp, s, y_out=y)
        else:
            lin(x, q, s, y_out=y)
    torch.cuda.synchronize()


def _prefill(a, torch, w4, synth, dev):
    M, H, F = synth.SEQ, synth.HIDDEN, synth.FFN
    g = synth.generator(300, dev)
    x = synth.activations(M, H, g, dev)
    if a.which in ("all", "attn_out"):
        w = synth.weight(H, H, g, device=dev)
        q, s = w4.quantize_rowwise_int4(w)
        qp = w4.w4a16_prepack(q)
        del w, q
        y = torch.empty(M, H, dtype=torch.float16, device=dev)
        torch.cuda.synchronize()
        print(f"prefill attention-out {H}x{H} M={M}: {a.reps} launches", flush=True)
        for _ in range(a.reps):
            w4.w4a16_linear_prepacked(x, qp, s, y_out=y)
        torch.cuda.synchronize()
        del qp, s, y
    if a.which in ("all", "ffn_up_geglu"):
        w = synth.weight(2 * F, H, g, device=dev)
        q, s = w4.quantize_rowwise_int4(w)
        qp = w4.w4a16_prepack(q)
        del w, q
        y = torch.empty(M, F, dtype=torch.float16, device=dev)
        torch.cuda.synchronize()
        print(f"prefill FFN-up GeGLU {2 * F}x{H} M={M}: {a.reps} launches", flush=True)
        for _ in range(a.reps):
            w4.w4a16_geglu_linear_prepacked(x, qp, s, y_out=y)
        torch.cuda.synchronize()


def _step(a, torch, w4, synth, dev):
    n, k = synth.QKV_OUT, synth.HIDDEN
    qs = []
    for i in range(5):
        w = synth.weight(n, k, synth.generator(10 + i, dev), device=dev)
        q, s = w4.quantize_rowwise_int4(w)
        qs.append((w4.w4a16_prepack(q), s))
        del w, q
    g = synth.generator(0, dev)
    ms = tuple(int(v) for v in a.ms.split(","))
    xs = {m: synth.activations(m, k, g, dev) for m in ms}
    ys = {m: torch.empty(m, n, dtype=torch.float16, device=dev) for m in ms}
    torch.cuda.synchronize()
    print(f"decode step QKV M = {ms}: {a.reps} steps", flush=True)
    i = 0
    for _ in range(a.reps):
        for m in ms:
            qp, s = qs[i % 5]
            i += 1
            w4.w4a16_linear_prepacked(xs[m], qp, s, y_out=ys[m])
    torch.cuda.synchronize()


def _copy(a, torch, dev):
    src = torch.empty(a.copy_bytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    print(f"copy {a.copy_bytes} bytes: {a.reps} launches", flush=True)
    for _ in range(a.reps):
        dst.copy_(src)
    torch.cuda.synchronize()


# ------------------------------------------------------------- summaries

def _csv_rows(pattern_dirs, suffix):
    rows = []
    for d in pattern_dirs:
        for path in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
            with open(path, newline="") as fh:
                rows.extend(csv.DictReader(fh))
    return rows


def summarize_pmc(dirs):
    """Mean of each counter per dispatch, per kernel, over the counter CSVs
    (rocprofv3 writes one row per dispatch and counter); the pseudo-counter
    DURATION_NS is the mean dispatch duration from the rows' timestamps."""
    acc = defaultdict(lambda: defaultdict(list))
    for r in _csv_rows(dirs, "counter_collection.csv"):
        acc[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
        acc[r["Kernel_Name"]]["DURATION_NS"].append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    out = OrderedDict()
    for kern, counters in acc.items():
        out[kern] = {c: (sum(v) / len(v), len(v)) for c, v in counters.items()}
    return out


# gfx950 as a rocprofv3 run sees it: GRBM_GUI_ACTIVE is summed over the 8
# XCDs; SQ_* cycle counters over all compute units or SIMDs as noted
XCDS, CUS, SIMDS = 8, 256, 1024


def derived(counters):
    """Per-dispatch utilisations from the mean counters of one kernel."""
    c = {k: v[0] for k, v in counters.items()}
    cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / XCDS            # kernel cycles (each XCD's clock)
    d = {"duration_us": c.get("DURATION_NS", 0.0) / 1e3, "cycles": cyc}
    if cyc and c.get("DURATION_NS"):
        d["clock_GHz"] = cyc / c["DURATION_NS"]
    if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
        d["mfma_busy"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * SIMDS)
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in c and c["SQ_VALU_MFMA_BUSY_CYCLES"]:
            d["mfma_cycles_with_valu"] = c["SQ_VALU_MFMA_COEXEC_CYCLES"] / c["SQ_VALU_MFMA_BUSY_CYCLES"]
    if cyc and "SQ_INSTS_VALU" in c:
        valu = c["SQ_INSTS_VALU"] - c.get("SQ_INSTS_MFMA", 0.0)    # SQ_INSTS_VALU counts MFMAs too
        d["valu_insts_per_simd"] = valu / SIMDS
        d["valu_busy"] = 4.0 * valu / SIMDS / cyc                   # a wave64 VALU op takes 4 cycles
    if cyc and "SQ_LDS_IDX_ACTIVE" in c:
        d["lds_busy"] = c["SQ_LDS_IDX_ACTIVE"] / (cyc * CUS)
        if c["SQ_LDS_IDX_ACTIVE"]:
            d["lds_bank_conflict_share"] = c.get("SQ_LDS_BANK_CONFLICT", 0.0) / c["SQ_LDS_IDX_ACTIVE"]
    if cyc and "TA_TA_BUSY" in c:
        d["ta_busy"] = c["TA_TA_BUSY"] / (cyc * CUS)
    if "SQ_WAIT_INST_ANY" in c and c.get("SQ_WAVE_CYCLES"):
        d["wave_cycles_waiting"] = c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"]
    return d


def summarize_trace(d):
    """Per-kernel durations of a --kernel-trace run, and the launch order
    with start / end times (ns) for gap analysis."""
    rows = _csv_rows([d], "kernel_trace.csv")
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    seq = [(r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows]
    return seq


def traffic(fetch_dir, write_dir, kernel_part, copy_bytes=1 << 30):
    """HBM bytes per dispatch of the kernel whose name contains kernel_part,
    from a FETCH_SIZE run and a WRITE_SIZE run (KiB per dispatch), each
    scaled by what the counter reads for the 1 GiB device copy of the same
    run (1 GiB read and 1 GiB written per dispatch)."""
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = summarize_pmc([d])
        kern = [v[counter][0] for k, v in per.items() if kernel_part in k and counter in v]
        copy = [v[counter][0] for k, v in per.items() if "copyBuffer" in k and counter in v]
        if len(kern) != 1 or len(copy) != 1:
            raise RuntimeError(f"{counter}: expected one matching kernel and one copy in {d}")
        factor = copy_bytes / (copy[0] * 1024)
        out[counter] = {"kib_per_dispatch": kern[0], "copy_kib_per_dispatch": copy[0],
                        "factor": factor, "bytes": kern[0] * 1024 * factor}
    return out


def _print_pmc(dirs):
    for kern, counters in summarize_pmc(dirs).items():
        print(kern)
        for c, (mean, n) in sorted(counters.items()):
            print(f"    {c:32s} {mean:16.1f}   ({n} dispatches)")


def trace_stats(d, name_part="", by_grid=False):
    """Per-kernel call count, mean, median, min and max duration (us) of a
    --kernel-trace run, for kernels whose name contains name_part; with
    by_grid, per (kernel, workgroups per launch), which tells apart the
    workloads that share one kernel."""
    per = defaultdict(list)
    rows = _csv_rows([d], "kernel_trace.csv")
    for r in rows:
        name = r["Kernel_Name"]
        if name_part in name:
            if by_grid:
                wgs = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
                name = f"{name} [{wgs} workgroups]"
            per[name].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = OrderedDict()
    for name, v in per.items():
        v = sorted(v)
        out[name] = {"calls": len(v), "mean": sum(v) / len(v), "median": v[len(v) // 2],
                     "min": v[0], "max": v[-1]}
    return out


def _print_trace(d, sequence=False, by_grid=False):
    for name, st in trace_stats(d, by_grid=by_grid).items():
        print(f"{st['calls']:6d} calls  mean {st['mean']:9.2f} us  median {st['median']:9.2f}  "
              f"min {st['min']:9.2f}  max {st['max']:9.2f}  {name}")
    if not sequence:
        return
    print("launch sequence (us): kernel, duration, gap after the previous launch's end")
    prev = None
    for name, s, e in summarize_trace(d):
        gap = "" if prev is None else f"{(s - prev) / 1e3:8.2f}"
        print(f"  {(e - s) / 1e3:9.2f} {gap:>8s}  {name[:90]}")
        prev = e


def step_timeline(d, after_ms=60.0, name_part="decode_kernel"):
    """Launch timeline of a step trace: for every kernel whose name contains
    name_part and that starts at least after_ms after the first such
    launch, the mean duration and the mean gap from the previous traced
    launch's end to its start (us), in launch order of one step; and the
    mean step period (us), from consecutive starts of the step's first
    kernel."""
    seq = [t for t in summarize_trace(d) if name_part in t[0]]
    if not seq:
        raise RuntimeError(f"no {name_part} launches in {d}")
    t0 = seq[0][1]
    per = OrderedDict()
    starts = defaultdict(list)
    prev_end = None
    for name, st, en in seq:
        if st - t0 >= after_ms * 1e6 and prev_end is not None:
            r = per.setdefault(name, {"dur": [], "gap": []})
            r["dur"].append((en - st) / 1e3)
            r["gap"].append((st - prev_end) / 1e3)
            starts[name].append(st)
        prev_end = en
    order = []
    for name, _, _ in seq:                       # the step's launch order
        if name not in order:
            order.append(name)
    per = OrderedDict((name, per[name]) for name in order if name in per)
    if not per:
        raise RuntimeError(f"no {name_part} launch starts {after_ms} ms or more into {d}")
    first = next(iter(per))
    st0 = starts[first]
    period = (st0[-1] - st0[0]) / 1e3 / (len(st0) - 1) if len(st0) > 1 else float("nan")
    rows = [(name, len(v["dur"]), sum(v["dur"]) / len(v["dur"]), sorted(v["dur"])[len(v["dur"]) // 2],
             sum(v["gap"]) / len(v["gap"])) for name, v in per.items()]
    return rows, period


def _print_timeline(d, after_ms):
    rows, period = step_timeline(d, after_ms)
    print(f"launches starting {after_ms:g} ms or more after the first traced decode launch")
    print("| kernel | launches | mean us | median us | mean gap before it, us |")
    print("|---|---|---|---|---|")
    for name, n, mean, med, gap in rows:
        print(f"| `{name.split('(')[0]}` | {n} | {mean:.2f} | {med:.2f} | {gap:.2f} |")
    busy = sum(r[2] for r in rows)
    gaps = sum(r[4] for r in rows)
    print(f"step period {period:.2f} us = launches {busy:.2f} us + gaps {gaps:.2f} us "
          f"(+{period - busy - gaps:.2f} us unaccounted)")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="mode", required=True)
    for mode in ("decode", "prefill", "step"):
        p = sub.add_parser(mode)
        p.add_argument("--reps", type=int, default=10)
        p.add_argument("--copy-bytes", type=int, default=1 << 30)
        if mode == "decode":
            p.add_argument("--m", type=int, default=64)
            p.add_argument("--layout", choices=("prepacked", "row-major"), default="prepacked")
            p.add_argument("--codes", choices=("int4", "int8"), default="int4")
        if mode == "prefill":
            p.add_argument("--which", choices=("all", "attn_out", "ffn_up_geglu"), default="all")
        if mode == "step":
            p.add_argument("--ms", default="1,8,32,64", help="token counts of one step, in launch order")
    p = sub.add_parser("summarize-pmc")
    p.add_argument("dirs", nargs="+")
    p = sub.add_parser("summarize-trace")
    p.add_argument("dir")
    p.add_argument("--sequence", action="store_true", help="also list every launch in order")
    p.add_argument("--by-grid", action="store_true", help="one line per kernel and grid size")
    p = sub.add_parser("step-timeline")
    p.add_argument("dir")
    p.add_argument("--after-ms", type=float, default=60.0)
    p = sub.add_parser("derived")
    p.add_argument("kernel_part")
    p.add_argument("dirs", nargs="+")
    p = sub.add_parser("traffic")
    p.add_argument("fetch_dir")
    p.add_argument("write_dir")
    p.add_argument("kernel_part")
    a = ap.parse_args(argv)

    if a.mode == "derived":
        for kern, counters in summarize_pmc(a.dirs).items():
            if a.kernel_part in kern:
                print(kern.split("(")[0])
                for k, v in derived(counters).items():
                    print(f"    {k:24s} {v:12.4f}")
        return 0
    if a.mode == "traffic":
        import json
        print(json.dumps(traffic(a.fetch_dir, a.write_dir, a.kernel_part), indent=1))
        return 0

    if a.mode == "summarize-pmc":
        _print_pmc(a.dirs)
        return 0
    if a.mode == "summarize-trace":
        _print_trace(a.dir, a.sequence, a.by_grid)
        return 0
    if a.mode == "step-timeline":
        _print_timeline(a.dir, a.after_ms)
        return 0

    import torch
    import weight_only_int4_rowwise_amd as w4
    from weight_only_int4_rowwise_amd import synth

    dev = "cuda:0"
    {"decode": _decode, "prefill": _prefill, "step": _step}[a.mode](a, torch, w4, synth, dev)
    _copy(a, torch, dev)
    print("done", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
