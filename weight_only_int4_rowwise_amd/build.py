"""Build libw4a16.so (the gfx950 HIP library) in-tree with hipcc.

    python -m weight_only_int4_rowwise_amd.build [--verbose]

Always recompiles.  The library lands next to this file, where the Python
binding loads it from.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libw4a16.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["api.hip", "quantize.hip", "decode.hip", "decode_w8.hip", "decode_zp.hip", "prefill.hip",
           "prepack.hip", "probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-Wall",
        "-Wno-unused-result",
    ]


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source to an object in parallel (the decode launch tables
    are split over three sources for this), then link the shared library."""
    import tempfile
    with tempfile.TemporaryDirectory(prefix="w4a16_build_") as tmpdir:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmpdir, src.replace(".hip", ".o"))
            cmd = [hipcc(), *compile_flags(), *(extra or []), "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd)))
            objs.append(obj)
        failed = [src for src, p in procs if p.wait() != 0]
        if failed:
            raise subprocess.CalledProcessError(1, f"hipcc {' '.join(failed)}")
        tmp = LIB_PATH + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true",
                    help="print per-kernel register / LDS usage")
    a = ap.parse_args(argv)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if a.resource_usage else None
    print(build(a.verbose, extra))
    return 0


if __name__ == "__main__":
    sys.exit(main())
