#!/usr/bin/env python3
"""Throughput of row-wise top-k on one MI355X.

Default workload (the headline): 262,144 rows x 256 fp32, exact top-32 with
one-byte column indices (the compressed balanced layout of a MaxK
nonlinearity), rows = N(0,1) x per-row scale U(0.5,2) with 5% exact zeros
(workloads.py). One step = one call of the library over the whole batch.
Inputs rotate over several resident buffers so that the 256 MB last-level
cache cannot serve them; everything is in HBM before timing starts. From
idle, launch times drift by up to 25% over the first ~150 launches while the
GPU's power management settles, so the default run warms up with 300 untimed
launches and then times 300.

Prints one JSON line: rows/s (whole job), the kernel's achieved algorithmic
HBM bandwidth against the 8 TB/s peak (roofline), the HBM traffic measured by
rocprofv3 counters when they match the current kernel sources, and the CPU
oracle's throughput on a bounded sample of the same workload.
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

HBM_PEAK_GBS = 8000.0
METRIC = "rows/sec and achieved HBM GB/s (% of peak), N=262144 M=256 k=32 fp32"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# Sources each kernel family is built from, beside the dispatch code every
# launch goes through: a counter record stays valid while these are unchanged
# (a change to the aggregation kernels leaves the selection's records valid).
_DISPATCH_SOURCES = ["rtopk_api.hip", "rtopk_internal.h", "rtopk_dispatch.hip"]
FAMILY_SOURCES = {
    "rows_in_registers": ["rtopk_rows.hpp"],
    "rows_in_group": ["rtopk_rows.hpp", "rtopk_group.hpp"],
    "bucket_lanes": ["rtopk_bucket.hip"],
    "bucket_quads": ["rtopk_bucket.hip"],
    "scatter_rows": ["rtopk_maxk.hip"],
    "spgemm_rows": ["rtopk_spgemm.hip"],
    "sspmm_rows": ["rtopk_spgemm.hip"],
}
KERNEL_SOURCES = sorted({f for v in FAMILY_SOURCES.values() for f in v} | set(_DISPATCH_SOURCES))
COPY_REF_BYTES = 2**28

# The headline workload (bench.py with no flags).
HEADLINE = {"rows": 262144, "m": 256, "k": 32, "mode": "exact", "max_iter": -1,
            "eps": 0.0, "index": "u8", "inputs": "maxk"}
# Named workloads (workloads.py): shape and first setting of each; sweeps
# (k, eps, max_iter, row length) are chosen with the flags.
CONFIGS = {
    1: {"rows": 1024, "m": 256, "k": 32, "mode": "exact", "index": "i32"},
    2: {"rows": 65536, "m": 256, "k": 32, "mode": "exact", "index": "i32"},
    3: {"rows": 262144, "m": 256, "k": 32, "mode": "exact", "index": "u8"},
    4: {"rows": 16384, "m": 8192, "k": 64, "mode": "exact", "index": "i32"},
    5: {"rows": 1048576, "m": 1024, "k": 64, "mode": "capped", "max_iter": 2,
        "index": "i32"},
}


def kernel_family(kernel: str) -> str:
    """Family of a kernel name fragment from op_kernel(): the register-resident
    row kernels are told apart by their mode argument; a fragment of several
    parts ("a&b") belongs to the family of its first part."""
    first = kernel.split("&")[0]
    return "rows_in_registers" if first.startswith("(rtopk::Mode)") else first


def kernel_matches(kernel: str, name: str) -> bool:
    """Whether a kernel name from a counter file matches an op_kernel()
    fragment (every part of "a&b" must occur in it)."""
    return all(part in name for part in kernel.split("&"))


def kernel_source_hash(kernel: str | None = None) -> str:
    """Hash of the sources of the kernel named by an op_kernel() fragment and
    of the dispatch code (all kernel sources if None)."""
    if kernel is None:
        names = KERNEL_SOURCES
    else:
        names = sorted(set(FAMILY_SOURCES[kernel_family(kernel)]) | set(_DISPATCH_SOURCES))
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "row_wise_top_amd", "csrc")
    for name in names:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current sources of the kernel for this workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_hash") != kernel_source_hash(kernel):
        return None
    return float(rec["bytes_per_launch"])


def _counter_means(csv_path: str, counter: str, kernel: str):
    """Mean per-dispatch value of one counter for the op's kernel and for the
    negation kernel, from a rocprofv3 counter_collection.csv."""
    import csv
    sel, ref = [], []
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            if kernel_matches(kernel, name):
                sel.append(float(r["Counter_Value"]))
            elif "neg" in name.lower():
                ref.append(float(r["Counter_Value"]))
    if not sel or not ref:
        raise SystemExit(f"{csv_path}: no {counter} records for the select "
                         "kernel or the negation reference")
    return sum(sel) / len(sel), sum(ref) / len(ref)


def record_traffic(workload: str, kernel: str, fetch_csv: str, write_csv: str) -> None:
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per
    dispatch) of `bench.py --copy-reference` into HBM bytes per launch. Each
    counter is scaled by the bytes the negation kernel is known to move
    divided by what the same counter reads for it."""
    f_sel, f_ref = _counter_means(fetch_csv, "FETCH_SIZE", kernel)
    w_sel, w_ref = _counter_means(write_csv, "WRITE_SIZE", kernel)
    f_scale = COPY_REF_BYTES / (f_ref * 1024.0)
    w_scale = COPY_REF_BYTES / (w_ref * 1024.0)
    fetched = f_sel * 1024.0 * f_scale
    written = w_sel * 1024.0 * w_scale
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    data[workload] = {"kernel_hash": kernel_source_hash(kernel), "kernel": kernel,
                      "bytes_per_launch": fetched + written,
                      "fetch_bytes": fetched, "write_bytes": written,
                      "fetch_kib_raw": f_sel, "write_kib_raw": w_sel,
                      "fetch_scale": f_scale, "write_scale": w_scale}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(data[workload]))


def workload_name(args) -> str:
    if args.config is not None and args.op == "select":
        return (f"config {args.config} N={args.rows} M={args.m} k={args.k} {args.mode}"
                + ("" if args.mode == "exact" else f" max_iter={args.max_iter} eps={args.eps}")
                + f" idx={args.index}")
    if args.op in ("maxk_backward", "maxk_forward"):
        return f"{args.op} {args.inputs} N={args.rows} M={args.m} k={args.k} idx={args.index}"
    if args.op == "bucketed":
        return (f"bucketed {args.inputs} N={args.rows} M={args.m} k={args.k} "
                f"buckets={args.buckets} idx={args.index}")
    if args.op in ("spgemm", "sspmm"):
        src = "" if getattr(args, "src_rows", None) in (None, args.rows) else \
            f" src_rows={args.src_rows}"
        return (f"{args.op} power-law graph N={args.rows} mean_degree={args.degree:g}{src} "
                f"M={args.m} k={args.k} idx={args.index}")
    return (f"{args.inputs} N={args.rows} M={args.m} k={args.k} {args.mode}"
            + ("" if args.mode == "exact" else f" max_iter={args.max_iter} eps={args.eps}")
            + f" idx={args.index}")


def _short_kernel(width: int, kb: int):
    """Kernel of the library's short rows (or buckets) of `width` columns
    keeping `kb` (inputs 16-byte aligned, as bench.py allocates them), if
    they take one."""
    if width <= 64 and kb <= 8:
        return "bucket_lanes"
    if width <= 128 and kb <= 16 and width % 4 == 0:
        return "bucket_quads"
    return None


def op_kernel(args) -> str:
    """Name fragment of the kernel the op's counters are attributed to, as the
    library routes the workload (specific enough to leave out the exact
    selection the approximate ops run once for their quality figures)."""
    index = getattr(args, "index", "i32")
    if args.op == "maxk_backward":
        return "scatter_rows"
    if args.op in ("spgemm", "sspmm"):
        return f"{args.op}_rows"
    if args.op == "bucketed":
        width, kb = args.m // args.buckets, args.k // args.buckets
        return _short_kernel(width, kb) or "(rtopk::Mode)3"
    if args.op == "maxk_forward":
        if args.m <= 1024:
            return "(rtopk::Mode)2"
        return "rows_in_group&, false, int>" if args.m > 4096 else "(rtopk::Mode)1"
    # Selection: no cap and eps = 0 is the exact selection. Row groups are
    # told apart by their CAPPED argument (the last before the index type):
    # a capped run also launches the exact selection once, for its quality
    # figures.
    exact = args.mode == "exact" or (getattr(args, "max_iter", 0) < 0
                                     and getattr(args, "eps", 1.0) == 0.0)
    if not exact:
        if args.m > 6144 and index != "u8":
            return "rows_in_group&, true, int>"
        return "(rtopk::Mode)0"
    short = _short_kernel(args.m, args.k)
    if short:
        return short
    if args.m > 4096 and index != "u8":
        return "rows_in_group&, false, int>"
    return "(rtopk::Mode)1"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--op", choices=["select", "maxk_forward", "maxk_backward", "bucketed",
                                    "spgemm", "sspmm"],
                   default="select",
                   help="select: row-wise top-k (the headline); maxk_forward: "
                        "the MaxK nonlinearity (dense output plus the compressed "
                        "pair); maxk_backward: the MaxK gradient scatter on the "
                        "indices the selection produces for the same rows")
    p.add_argument("--steps", type=int, default=300)
    p.add_argument("--warmup", type=int, default=300,
                   help="untimed launches first; the GPU's clocks take about "
                        "150 launches (~10 ms) of sustained load to settle")
    p.add_argument("--degree", type=float, default=64.0,
                   help="mean degree of the power-law graph for --op spgemm")
    p.add_argument("--src-rows", type=int, default=None,
                   help="--op spgemm/sspmm: the graph's edges point into the first "
                        "SRC_ROWS rows only (default: all rows). A smaller footprint "
                        "stands for what one XCD would gather from if the edges were "
                        "partitioned by source-row block")
    p.add_argument("--no-torch-topk", action="store_true",
                   help="--op select: skip timing torch.topk on the same inputs")
    p.add_argument("--buckets", type=int, default=8,
                   help="buckets per row for --op bucketed")
    p.add_argument("--config", type=int, choices=sorted(CONFIGS), default=None,
                   help="a named workload (workloads.py): its rows, row length, "
                        "seed, k, mode and index width; flags given explicitly "
                        "override them")
    p.add_argument("--rows", type=int, default=None)
    p.add_argument("--m", type=int, default=None)
    p.add_argument("--k", type=int, default=None)
    p.add_argument("--mode", choices=["exact", "capped"], default=None)
    p.add_argument("--max-iter", type=int, default=None)
    p.add_argument("--eps", type=float, default=None)
    p.add_argument("--index", choices=["u8", "i32"], default=None)
    p.add_argument("--inputs", choices=["maxk", "normal", "grid"], default=None)
    p.add_argument("--buffers", type=int, default=0,
                   help="input buffers to rotate (0: enough to exceed 768 MB)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="approximate CPU time for the oracle baseline (0: skip)")
    p.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="write profiles/traffic.json for this workload from two "
                        "rocprofv3 counter_collection.csv files and exit")
    p.add_argument("--copy-reference", action="store_true",
                   help="after timing, run a plain 256 MiB streaming kernel so that "
                        "a counter run can calibrate FETCH_SIZE / WRITE_SIZE")
    args = p.parse_args()
    # Unset flags: the named workload's value, else the headline's.
    named = CONFIGS.get(args.config, {})
    for key, value in HEADLINE.items():
        if getattr(args, key) is None:
            setattr(args, key, named.get(key, value))
    return args


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not "
              "supported (rows are independent: a multi-GPU run would give each "
              "GPU its own block of rows with no exchange).", file=sys.stderr)
        sys.exit(2)
    if args.record_traffic:
        record_traffic(workload_name(args), op_kernel(args), *args.record_traffic)
        return

    import numpy as np
    import torch

    import row_wise_top_amd as rt
    import workloads

    n, m, k = args.rows, args.m, args.k
    u8 = args.index == "u8"
    if args.config is not None:
        x_np = workloads.config_input(args.config, n, m)
    elif args.inputs == "maxk":
        x_np = workloads.maxk_activation(n, m, workloads.CONFIG_SEEDS[3])
    elif args.inputs == "normal":
        x_np = workloads.normal(n, m, 6)
    else:
        x_np = workloads.grid_ties(n, m, 5)
    in_bytes = x_np.nbytes
    nbuf = args.buffers or max(1, -(-768 * 2**20 // in_bytes))
    dev = torch.device("cuda:0")
    xs = [torch.from_numpy(x_np).to(dev)]
    for b in range(1, nbuf):
        # Same rows, rotated by b rows: a different byte image of the workload.
        xs.append(torch.roll(xs[0], shifts=b, dims=0).contiguous())
    idx_dtype = torch.uint8 if u8 else torch.int32
    out_v = torch.empty((n, k), dtype=torch.float32, device=dev)
    out_i = torch.empty((n, k), dtype=idx_dtype, device=dev)
    stream = torch.cuda.current_stream(dev)

    if args.op == "maxk_backward":
        # Inputs: the survivors' indices of each rotated buffer (from the
        # library's exact selection) and seeded gradients. Outputs rotate too,
        # so that neither side is served by the last-level cache.
        sel = rt.rtopk_select_exact_u8 if u8 else rt.rtopk_select_exact
        rng = np.random.default_rng(7)
        base_idx = [sel(xb, k)[1] for xb in xs]
        del xs
        nbuf = max(1, -(-768 * 2**20 // (n * k * (4 + (1 if u8 else 4)))))
        grads, idxs = [], []
        for b in range(nbuf):
            # Index sets of the selection, rotated by b rows past the first few.
            ib = base_idx[b % len(base_idx)]
            idxs.append(ib if b < len(base_idx) else
                        torch.roll(ib, shifts=b, dims=0).contiguous())
            grads.append(torch.from_numpy(
                rng.standard_normal((n, k), dtype=np.float32)).to(dev))
        nout = max(1, -(-768 * 2**20 // (n * m * 4)))
        outs = [torch.empty((n, m), dtype=torch.float32, device=dev) for _ in range(nout)]

        def step(i):
            rt.rtopk_maxk_backward(grads[i % nbuf], idxs[i % nbuf], m,
                                   grad_x=outs[i % nout])
    elif args.op in ("spgemm", "sspmm"):
        # A power-law graph over the same rows; features: the exact top-k of
        # each rotated buffer (from the library's selection). Outputs rotate;
        # for the backward the rotated inputs are dense gradients dY.
        sel = rt.rtopk_select_exact_u8 if u8 else rt.rtopk_select_exact
        feats = [sel(xb, k) for xb in xs]
        del xs
        n_src = n if args.src_rows is None else args.src_rows
        if not 1 <= n_src <= n:
            raise SystemExit("--src-rows must be between 1 and --rows")
        rp_np, ci_np, va_np = workloads.power_law_graph(n, n_src, args.degree, 4096, seed=48)
        nnz = int(ci_np.shape[0])
        rp_t = torch.from_numpy(rp_np).to(dev)
        ci_t = torch.from_numpy(ci_np).to(dev)
        va_t = torch.from_numpy(va_np).to(dev)
        nout = max(1, -(-768 * 2**20 // (n * m * 4)))
        outs = [torch.empty((n, m), dtype=torch.float32, device=dev) for _ in range(nout)]

        if args.op == "spgemm":
            def step(i):
                fv, fi = feats[i % nbuf]
                rt.rtopk_cbsr_spgemm(rp_t, ci_t, va_t, fv, fi, m, y=outs[i % nout])
        else:
            dys = outs
            for b, t in enumerate(dys):
                t.copy_(torch.from_numpy(workloads.normal(n, m, 90 + b)))
            gs = [torch.empty((n, k), dtype=torch.float32, device=dev) for _ in range(nbuf)]

            def step(i):
                rt.rtopk_cbsr_sspmm(rp_t, ci_t, va_t, dys[i % nout], feats[i % nbuf][1],
                                    grad_sp=gs[i % nbuf])
    elif args.op == "bucketed":
        def step(i):
            rt.rtopk_select_bucketed(xs[i % nbuf], k, args.buckets, out_val=out_v,
                                     out_idx=out_i, index_dtype=idx_dtype)
    elif args.op == "maxk_forward":
        nout = max(1, -(-768 * 2**20 // (n * m * 4)))
        ys = [torch.empty((n, m), dtype=torch.float32, device=dev) for _ in range(nout)]

        def step(i):
            rt.rtopk_maxk_forward(xs[i % nbuf], k, y=ys[i % nout], sp_data=out_v,
                                  sp_index=out_i, index_dtype=idx_dtype)
    elif args.mode == "exact":
        fn = rt.rtopk_select_exact_u8 if u8 else rt.rtopk_select_exact

        def step(i):
            fn(xs[i % nbuf], k, out_val=out_v, out_idx=out_i)
    else:
        fn = rt.rtopk_select_u8 if u8 else rt.rtopk_select

        def step(i):
            fn(xs[i % nbuf], k, args.max_iter, args.eps, out_val=out_v, out_idx=out_i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K back-to-back launches on one stream between one pair of
    # HIP events (per-launch event pairs would add their own stream overhead
    # to every launch). The kernel's average launch duration is that span / K.
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / args.steps
    avg_launch_ms = ms_per_step

    # Spread of single launches (not used for the throughput figure): an event
    # pair around each of up to 100 further launches.
    n_single = min(args.steps, 100)
    pairs = [(torch.cuda.Event(enable_timing=True),
              torch.cuda.Event(enable_timing=True)) for _ in range(n_single)]
    for i, (a, b) in enumerate(pairs):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    single_us = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)

    def pct(q):
        return single_us[min(len(single_us) - 1, int(q * len(single_us)))]

    # Practical streaming ceiling of this GPU: an elementwise negation over
    # 256 MiB (read once, written once), timed the same way.
    src = torch.ones(COPY_REF_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(20):
        torch.neg(src, out=dst)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0.record(stream)
    for _ in range(50):
        torch.neg(src, out=dst)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * COPY_REF_BYTES / (c0.elapsed_time(c1) / 50 * 1e-3) / 1e9
    del src, dst

    if args.copy_reference:
        # Plain streaming kernel of known size for scaling the HBM counters:
        # three more negations, each reading and writing 268,435,456 bytes.
        src = torch.ones(COPY_REF_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()

    idx_bytes = 1 if u8 else 4
    # select and maxk_backward: M floats one way, k entries the other;
    # maxk_forward: M floats in, M floats and k entries out.
    per_row = 4 * m + k * (4 + idx_bytes) + (4 * m if args.op == "maxk_forward" else 0)
    extra = {}
    if args.op in ("spgemm", "sspmm"):
        # Bytes that must cross HBM at least once per launch: the CSR arrays,
        # each compressed row once, each dense row once (forward: output;
        # backward: the input dY, plus the gradient written, k floats per
        # row). The per-edge gathers of neighbour rows (nnz * k * (4 + b);
        # backward: index rows plus atomics) are served mostly by the caches
        # and reported separately.
        n_src = n if args.src_rows is None else args.src_rows
        per_row = 4 * m + k * (4 + idx_bytes) * n_src / n + 8 + (nnz * 8) / n
        if args.op == "sspmm":
            per_row = 4 * m + k * (idx_bytes + 4) + 8 + (nnz * 8) / n
        gather = nnz * k * (4 + idx_bytes)
        extra = {"edges": nnz, "edges_per_s": nnz / (avg_launch_ms * 1e-3),
                 "gather_bytes_per_launch": gather,
                 "gather_gbs": gather / (avg_launch_ms * 1e-3) / 1e9}
        if args.op == "sspmm":
            # Float-atomic reference: torch's index_add_ adding one k-float row
            # per edge into a [n, k] array at the same destination rows (the
            # edges' columns), from one cached source row, timed the same way:
            # as many float atomics as the kernel issues (nnz * k), none of
            # its gathers.
            g_ref = torch.zeros(n, k, dtype=torch.float32, device=dev)
            rows_ref = ci_t.long()
            src_ref = torch.ones(1, k, dtype=torch.float32, device=dev).expand(nnz, k)
            for _ in range(3):
                g_ref.index_add_(0, rows_ref, src_ref)
            a0 = torch.cuda.Event(enable_timing=True)
            a1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a0.record(stream)
            for _ in range(10):
                g_ref.index_add_(0, rows_ref, src_ref)
            a1.record(stream)
            torch.cuda.synchronize()
            ref_ms = a0.elapsed_time(a1) / 10
            extra["atomic_reference"] = {
                "what": "torch index_add_ of one k-float row per edge (nnz * k float atomics)",
                "us": ref_ms * 1e3,
                "float_atomics": nnz * k,
                "kernel_over_reference": avg_launch_ms / ref_ms}
            del g_ref, rows_ref, src_ref
    if args.op == "select" and not args.no_torch_topk:
        # Context, not a target: the pages quote their speedups over PyTorch's
        # topk at M = 256. torch.topk (largest, unsorted, int64 indices) on the
        # same rotating inputs, timed the same way.
        for i in range(20):
            torch.topk(xs[i % nbuf], k, dim=1, largest=True, sorted=False)
        r0 = torch.cuda.Event(enable_timing=True)
        r1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        r0.record(stream)
        for i in range(50):
            torch.topk(xs[i % nbuf], k, dim=1, largest=True, sorted=False)
        r1.record(stream)
        torch.cuda.synchronize()
        ref_ms = r0.elapsed_time(r1) / 50
        extra["torch_topk"] = {"what": "torch.topk(x, k, dim=1, sorted=False), same inputs",
                               "us": ref_ms * 1e3,
                               "speedup": ref_ms / avg_launch_ms}
    algo_bytes = int(n * per_row)
    achieved = algo_bytes / (avg_launch_ms * 1e-3) / 1e9
    workload = workload_name(args)
    traffic = measured_traffic(workload, op_kernel(args))

    # Approximate ops: hit rate and relative errors against the library's exact
    # selection of the same rows (definitions in row_wise_top_amd/quality.py).
    quality = None
    if args.op == "bucketed" or (args.op == "select" and args.mode == "capped"):
        from row_wise_top_amd.quality import topk_quality
        step(0)
        ev, _ = rt.rtopk_select_exact(xs[0], k)
        torch.cuda.synchronize()
        quality = topk_quality(out_v.cpu().numpy(), ev.cpu().numpy())

    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        oracle.exact(x_np[:1024], k)  # load and warm
        if args.op == "maxk_backward":
            g_np = grads[0].cpu().numpy()
            i_np = idxs[0].cpu().numpy().astype(np.int32)
        if args.op in ("spgemm", "sspmm"):
            sp_np = (feats[0][0].cpu().numpy(), feats[0][1].cpu().numpy().astype(np.int32))
        if args.op == "sspmm":
            dy_np = dys[0].cpu().numpy()

        def oracle_pass(r):
            """The op on the first r rows of the batch (r = n: all of it)."""
            if args.op == "maxk_backward":
                oracle.maxk_backward(g_np[:r], i_np[:r], m)
            elif args.op == "maxk_forward":
                oracle.maxk_forward(x_np[:r], k)
            elif args.op == "bucketed":
                oracle.bucketed(x_np[:r], k, args.buckets)
            elif args.op == "spgemm":
                e = int(rp_np[r])
                oracle.spgemm(rp_np[:r + 1], ci_np[:e], va_np[:e], n, sp_np[0], sp_np[1], m)
            elif args.op == "sspmm":
                e = int(rp_np[r])
                oracle.sspmm(rp_np[:r + 1], ci_np[:e], va_np[:e], dy_np[:r], sp_np[1])
            elif args.mode == "exact":
                oracle.exact(x_np[:r], k)
            else:
                # The per-row count numbers of the last pass are kept for the
                # iteration report.
                state["counts"] = oracle.capped(x_np[:r], k, args.max_iter, args.eps,
                                                return_state=True)[2]

        def timed_passes(r, seconds):
            passes, spent = 0, 0.0
            while spent < seconds and passes < 100:
                t = time.perf_counter()
                oracle_pass(r)
                spent += time.perf_counter() - t
                passes += 1
            return passes, spent

        # The oracle's SSpMM scatters into one accumulator on one thread.
        state = {}
        cores = 1 if args.op == "sspmm" else oracle.threads()
        passes, t_cpu = timed_passes(n, args.cpu_seconds)
        iterations = None
        if "counts" in state:
            # Counts the specified search made per row (RTop-K page,
            # "Surprising findings": at eps = 0 it usually ends within 16).
            cnt = state["counts"]
            values, freq = np.unique(cnt, return_counts=True)
            iterations = {"rows": int(cnt.size), "mean": float(cnt.mean()),
                          "max": int(cnt.max()),
                          "within_16": float((cnt <= 16).mean()),
                          "histogram": {str(int(v)): int(f) for v, f in zip(values, freq)}}
        cpu = {"value": passes * n / t_cpu, "unit": "rows/s",
               "gbs": passes * n * per_row / t_cpu / 1e9,
               "cores": cores, "kind": "oracle",
               "method": ("std::nth_element per row" if args.op == "select" and
                          args.mode == "exact" else "the oracle of the op"),
               "sample": f"{passes} full pass(es) over the same {n}-row batch "
                         f"({t_cpu:.1f} s of oracle time)"}
        if iterations is not None:
            cpu["iterations"] = iterations
        # The same oracle on one thread, over the first rows of the batch (a
        # slice that one thread finishes in about two seconds).
        if cores == 1:
            cpu["single_thread"] = dict(cpu, sample="the figure above (one thread)")
            del cpu["single_thread"]["kind"]
        else:
            per_row_1t = t_cpu / (passes * n) * cores
            r1 = int(min(n, max(1024, 2.0 / per_row_1t)))
            oracle.set_threads(1)
            try:
                p1, t1 = timed_passes(r1, max(2.0, args.cpu_seconds / 4))
            finally:
                oracle.set_threads(cores)
            cpu["single_thread"] = {"value": p1 * r1 / t1, "unit": "rows/s",
                                    "gbs": p1 * r1 * per_row / t1 / 1e9, "cores": 1,
                                    "sample": f"{p1} pass(es) over the first {r1} rows "
                                              f"({t1:.1f} s of oracle time)"}

    line = {
        "metric": (METRIC if args.op == "select" else
                   f"rows/sec and achieved HBM GB/s (% of peak), bucketed top-k "
                   f"N={n} M={m} k={k} buckets={args.buckets} fp32" if args.op == "bucketed" else
                   f"rows/sec and achieved HBM GB/s (% of peak), MaxK-GNN aggregation "
                   f"N={n} M={m} k={k} fp32" if args.op == "spgemm" else
                   f"rows/sec and achieved HBM GB/s (% of peak), MaxK-GNN aggregation backward "
                   f"(SSpMM) N={n} M={m} k={k} fp32" if args.op == "sspmm" else
                   f"rows/sec and achieved HBM GB/s (% of peak), MaxK "
                   f"{args.op.split('_')[1]} N={n} M={m} k={k} fp32"),
        "value": n / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": workload, "op": args.op, "rows": n,
                   "row_length": m, "k": k,
                   "mode": args.mode, "index": args.index,
                   "input_buffers": nbuf, "bytes_per_row": per_row},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "kernel_avg_us": avg_launch_ms * 1e3,
        "single_launch_us": {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9),
                             "launches": n_single},
        "stream_copy_gbs": copy_gbs,
    }
    if quality is not None:
        line["quality_vs_exact"] = quality
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
