"""Host logic of bench.py (no GPU): the counter calibration that turns two
rocprofv3 --pmc runs into HBM bytes per launch, which kernel each op's
counters are attributed to, the source-hash gate on stored traffic figures,
and the refusal of multi-GPU runs."""

from __future__ import annotations

import argparse
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def write_counters(path, counter, rows):
    """A counter_collection.csv with (kernel name, value in KiB) records."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


SEL = "void rtopk::rows_detail::rows_in_registers<4, true, (rtopk::Mode)1, 1, unsigned char>(rtopk::SelectArgs)"
EXACT_REF = SEL
CAPPED = "void rtopk::rows_detail::rows_in_registers<4, true, (rtopk::Mode)0, 0, unsigned char>(rtopk::SelectArgs)"
NEG = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)>"


def test_record_traffic_calibrates_both_counters(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    # The negation kernel moves 2^28 bytes each way; FETCH_SIZE reads half of
    # that (as on gfx950), WRITE_SIZE all of it.
    ref_kib = bench.COPY_REF_BYTES / 1024.0
    write_counters(tmp_path / "f.csv", "FETCH_SIZE",
                   [(SEL, 1000.0), (SEL, 1002.0), (NEG, ref_kib / 2)])
    write_counters(tmp_path / "w.csv", "WRITE_SIZE", [(SEL, 160.0), (SEL, 160.0), (NEG, ref_kib)])
    bench.record_traffic("wl", "(rtopk::Mode)1", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    rec = json.load(open(tmp_path / "traffic.json"))["wl"]
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_bytes"] == pytest.approx(1001.0 * 1024 * 2)
    assert rec["write_bytes"] == pytest.approx(160.0 * 1024)
    assert rec["bytes_per_launch"] == pytest.approx(1001.0 * 2048 + 160.0 * 1024)
    assert rec["kernel_hash"] == bench.kernel_source_hash("(rtopk::Mode)1")
    # The stored figure is served back only while the sources are unchanged.
    assert bench.measured_traffic("wl", "(rtopk::Mode)1") == pytest.approx(rec["bytes_per_launch"])
    assert bench.measured_traffic("wl", "bucket_lanes") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda kernel=None: "changed")
    assert bench.measured_traffic("wl", "(rtopk::Mode)1") is None
    assert bench.measured_traffic("other workload", "(rtopk::Mode)1") is None


def test_counters_of_other_kernels_are_left_out(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    ref_kib = bench.COPY_REF_BYTES / 1024.0
    # A capped run also launches the exact selection once (quality figures):
    # its record must not enter the capped kernel's mean.
    write_counters(tmp_path / "f.csv", "FETCH_SIZE",
                   [(CAPPED, 500.0), (CAPPED, 500.0), (EXACT_REF, 9999.0), (NEG, ref_kib / 2)])
    write_counters(tmp_path / "w.csv", "WRITE_SIZE",
                   [(CAPPED, 80.0), (EXACT_REF, 9999.0), (NEG, ref_kib)])
    args = argparse.Namespace(op="select", mode="capped", m=256, k=32, buckets=1)
    bench.record_traffic("capped", bench.op_kernel(args), str(tmp_path / "f.csv"),
                         str(tmp_path / "w.csv"))
    rec = json.load(open(tmp_path / "traffic.json"))["capped"]
    assert rec["fetch_kib_raw"] == pytest.approx(500.0)
    assert rec["write_kib_raw"] == pytest.approx(80.0)


def test_missing_records_are_an_error(tmp_path):
    write_counters(tmp_path / "f.csv", "FETCH_SIZE", [(SEL, 1.0)])
    with pytest.raises(SystemExit):
        bench._counter_means(str(tmp_path / "f.csv"), "FETCH_SIZE", "(rtopk::Mode)1")


@pytest.mark.parametrize("op,mode,m,k,buckets,index,want", [
    ("select", "exact", 256, 32, 1, "u8", "(rtopk::Mode)1"),
    ("select", "capped", 256, 32, 1, "u8", "(rtopk::Mode)0"),
    ("select", "exact", 64, 8, 1, "u8", "bucket_lanes"),
    ("select", "exact", 128, 16, 1, "u8", "bucket_quads"),
    ("select", "exact", 128, 32, 1, "u8", "(rtopk::Mode)1"),
    ("select", "exact", 126, 16, 1, "u8", "(rtopk::Mode)1"),
    ("select", "exact", 8192, 64, 1, "i32", "rows_in_group&, false, int>"),
    ("select", "capped", 8192, 64, 1, "i32", "rows_in_group&, true, int>"),
    ("select", "capped", 6000, 64, 1, "i32", "(rtopk::Mode)0"),
    ("select", "exact", 4096, 64, 1, "i32", "(rtopk::Mode)1"),
    ("maxk_forward", "exact", 256, 32, 1, "u8", "(rtopk::Mode)2"),
    ("maxk_forward", "exact", 8192, 32, 1, "i32", "rows_in_group&, false, int>"),
    ("maxk_backward", "exact", 256, 32, 1, "u8", "scatter_rows"),
    ("bucketed", "exact", 256, 32, 8, "u8", "bucket_lanes"),
    ("bucketed", "exact", 256, 32, 4, "u8", "bucket_lanes"),
    ("bucketed", "exact", 256, 32, 2, "u8", "bucket_quads"),
    ("bucketed", "exact", 256, 64, 2, "u8", "(rtopk::Mode)3"),
    ("bucketed", "exact", 512, 32, 2, "i32", "(rtopk::Mode)3"),
    ("spgemm", "exact", 256, 32, 1, "u8", "spgemm_rows"),
    ("sspmm", "exact", 256, 32, 1, "u8", "sspmm_rows"),
])
def test_op_kernel(op, mode, m, k, buckets, index, want):
    args = argparse.Namespace(op=op, mode=mode, m=m, k=k, buckets=buckets, index=index,
                              max_iter=4, eps=0.0)
    assert bench.op_kernel(args) == want


def test_uncapped_search_is_counted_as_the_exact_kernel():
    # No cap and eps = 0 runs the exact selection.
    args = argparse.Namespace(op="select", mode="capped", m=256, k=32, buckets=1,
                              index="u8", max_iter=-1, eps=0.0)
    assert bench.op_kernel(args) == "(rtopk::Mode)1"
    args.eps = 1e-4
    assert bench.op_kernel(args) == "(rtopk::Mode)0"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_named_configs_and_overrides(monkeypatch):
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert (a.rows, a.m, a.k, a.mode, a.index, a.inputs) == (262144, 256, 32, "exact", "u8", "maxk")
    assert a.config is None and a.max_iter == -1 and a.eps == 0.0
    monkeypatch.setattr(sys, "argv", ["bench.py", "--config", "5"])
    a = bench.parse()
    assert (a.rows, a.m, a.k, a.mode, a.max_iter, a.index) == (1048576, 1024, 64, "capped", 2, "i32")
    assert bench.workload_name(a).startswith("config 5 N=1048576 M=1024 k=64 capped max_iter=2")
    monkeypatch.setattr(sys, "argv", ["bench.py", "--config", "4", "--m", "2048", "--k", "128"])
    a = bench.parse()
    assert (a.rows, a.m, a.k, a.mode) == (16384, 2048, 128, "exact")
    monkeypatch.setattr(sys, "argv", ["bench.py", "--config", "2", "--mode", "capped",
                                      "--max-iter", "4", "--eps", "1e-4"])
    a = bench.parse()
    assert (a.rows, a.k, a.max_iter, a.eps) == (65536, 32, 4, 1e-4)
    monkeypatch.setattr(sys, "argv", ["bench.py", "--op", "spgemm", "--src-rows", "32768"])
    a = bench.parse()
    assert "src_rows=32768" in bench.workload_name(a)
    monkeypatch.setattr(sys, "argv", ["bench.py", "--op", "spgemm"])
    assert "src_rows" not in bench.workload_name(bench.parse())
    # The torch.topk context timing is on by default and can be skipped; the
    # workload name does not depend on it.
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert not a.no_torch_topk
    monkeypatch.setattr(sys, "argv", ["bench.py", "--no-torch-topk"])
    b = bench.parse()
    assert b.no_torch_topk and bench.workload_name(b) == bench.workload_name(a)


def test_group_fragments_tell_exact_from_capped():
    exact = "void rtopk::group_detail::rows_in_group<32, true, 4, false, int>(rtopk::SelectArgs)"
    capped = "void rtopk::group_detail::rows_in_group<32, true, 4, true, int>(rtopk::SelectArgs)"
    assert bench.kernel_matches("rows_in_group&, true, int>", capped)
    assert not bench.kernel_matches("rows_in_group&, true, int>", exact)
    assert bench.kernel_matches("rows_in_group&, false, int>", exact)
    assert bench.kernel_family("rows_in_group&, true, int>") == "rows_in_group"
    assert bench.kernel_source_hash("rows_in_group&, true, int>") == \
        bench.kernel_source_hash("rows_in_group")


def test_source_hash_is_per_kernel():
    # A change to the aggregation kernels leaves the selection's records valid.
    assert set(bench.FAMILY_SOURCES["spgemm_rows"]).isdisjoint(
        bench.FAMILY_SOURCES["rows_in_registers"])
    assert bench.kernel_source_hash("(rtopk::Mode)1") != bench.kernel_source_hash("spgemm_rows")
    assert bench.kernel_source_hash("(rtopk::Mode)1") == bench.kernel_source_hash("(rtopk::Mode)0")
    assert bench.kernel_source_hash("(rtopk::Mode)1") != bench.kernel_source_hash("bucket_lanes")
    for fam in bench.FAMILY_SOURCES:
        assert len(bench.kernel_source_hash(fam)) == 16
        for name in bench.FAMILY_SOURCES[fam]:
            assert os.path.exists(os.path.join(ROOT, "row_wise_top_amd", "csrc", name))
