"""Build the HIP library librtopk.so for gfx950, in-tree.

Usage: python -m row_wise_top_amd.build [--asm DIR]

Flags: IEEE single precision with no FMA contraction (the capped search's
midpoint must round exactly as specified), subnormals kept (no
flush-to-zero), packed FP32 instructions disabled.

The packed-FP32 switch is a gfx950 target feature. hipcc compiles each unit
for the device and the host in one invocation and offers no way to hand a
cc1 target feature to the device pass alone (-Xarch_device refuses
-Xclang), and a per-function target attribute instead blocks inlining of
the device library. So the feature goes to both passes, and the host (x86)
pass prints one line saying it does not know it; build() drops exactly that
line from the compiler's output and shows everything else.
"""

from __future__ import annotations

import argparse
import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "librtopk.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["rtopk_api.hip", "rtopk_dispatch.hip", "rtopk_rows_a.hip",
           "rtopk_rows_b.hip", "rtopk_rows_c.hip", "rtopk_rows_d.hip",
           "rtopk_rows_e.hip", "rtopk_rows_f.hip", "rtopk_maxk.hip",
           "rtopk_spgemm.hip", "rtopk_bucket.hip", "rtopk_group.hip"]
ARCH = "gfx950"

# The one line the host pass prints for the device-only feature (see above).
HOST_FEATURE_NOTE = ("'-packed-fp32-ops' is not a recognized feature for this "
                     "target (ignoring feature)")

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    # Inputs are required finite: lets min/max skip NaN quieting.
    "-fno-honor-nans",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every unit (in parallel) and link librtopk.so in-tree."""
    jobs = jobs or min(8, os.cpu_count() or 1)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        os.makedirs(BUILD_DIR, exist_ok=True)
        cmd = [hipcc(), *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        while len([p for p, _ in procs if p.poll() is None]) >= jobs:
            time.sleep(0.05)
        log = open(obj + ".log", "w+")
        procs.append((subprocess.Popen(cmd, stderr=log), log))
        objs.append(obj)
    failed = []
    for p, log in procs:
        p.wait()
        log.seek(0)
        for line in log.read().splitlines():
            if line.strip() != HOST_FEATURE_NOTE:
                print(line, file=sys.stderr)
        log.close()
        if p.returncode != 0:
            failed.append(p.args[-3])
    if failed:
        raise RuntimeError(f"hipcc failed for: {failed}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def dump_asm(out_dir: str, only: str | None = None) -> None:
    """Write the gfx950 assembly of the units (for inspection)."""
    os.makedirs(out_dir, exist_ok=True)
    for src in SOURCES:
        if only and only not in src:
            continue
        out = os.path.join(out_dir, src.replace(".hip", f"-{ARCH}.s"))
        cmd = [hipcc(), *HIP_FLAGS, "--cuda-device-only", "-S",
               os.path.join(CSRC, src), "-o", out]
        subprocess.run(cmd, check=True)


if __name__ == "__main__":
    p = argparse.ArgumentParser()
    p.add_argument("--asm", default=None, help="write assembly to this dir")
    p.add_argument("--only", default=None, help="with --asm: units matching")
    p.add_argument("-v", action="store_true")
    args = p.parse_args()
    if args.asm:
        dump_asm(args.asm, args.only)
    else:
        print(build(verbose=args.v))
        sys.exit(0)
