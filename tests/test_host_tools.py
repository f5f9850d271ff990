"""Host-side tools, on the CPU: bench.py's contract for more than one GPU,
its statistics and the digest that gates the HBM-traffic figure, and the
profiling module that turns rocprofv3 output into the committed summaries."""

import csv
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from collective_reduction_amd import profiling  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode != 0
    assert "one GPU" in proc.stderr
    assert proc.stdout == ""


def test_stats():
    st = bench.stats([4.0, 1.0, 3.0, 2.0, 5.0])
    assert st["median_ms"] == 3.0
    assert st["p95_ms"] == 5.0
    assert st["mean_ms"] == 3.0
    assert st["cv"] == pytest.approx((2.0 ** 0.5) / 3.0)
    assert bench.stats([2.0])["cv"] == 0.0


def test_kernel_digest_ignores_comments_but_not_code(tmp_path):
    src = os.path.join(ROOT, "collective_reduction_amd", "csrc")
    copy = tmp_path / "csrc"
    shutil.copytree(src, copy)
    base = {k: bench.kernel_source_digest(k, str(copy)) for k in bench.KERNEL_FILES}
    assert base == {k: bench.kernel_source_digest(k) for k in bench.KERNEL_FILES}
    ring = copy / "kernels_ring.hip"
    text = ring.read_text()
    ring.write_text("// a new comment line\n/* and a\n   block comment */\n" + text.replace("\n", "\n\n", 3))
    assert {k: bench.kernel_source_digest(k, str(copy)) for k in bench.KERNEL_FILES} == base
    ring.write_text(text.replace("1u << 22", "1u << 21", 1))
    after = {k: bench.kernel_source_digest(k, str(copy)) for k in bench.KERNEL_FILES}
    assert after["ring_step_kernel"] != base["ring_step_kernel"]
    assert after["ag_direct_kernel"] == base["ag_direct_kernel"]  # another file's kernels keep their digest


def test_load_traffic_is_gated_by_the_digest(tmp_path):
    digest = bench.kernel_source_digest("ag_direct_kernel")
    rec = {"ag_direct_kernel:w": {"traffic_bytes": 123.0, "source_digest": digest},
           "rs_direct_kernel:w": {"traffic_bytes": 456.0, "source_digest": "0" * 16}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    assert bench.load_traffic("ag_direct_kernel", "w", str(path)) == 123.0
    assert bench.load_traffic("rs_direct_kernel", "w", str(path)) is None  # stale
    assert bench.load_traffic("ag_direct_kernel", "other", str(path)) is None
    assert bench.load_traffic("ag_direct_kernel", "w", str(tmp_path / "missing.json")) is None


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


AG = "void ccl::(anonymous namespace)::ag_direct_kernel<ccl::F32>(ccl::(anonymous namespace)::ShardArgs)"
RS = ("void ccl::(anonymous namespace)::rs_direct_kernel<ccl::F32, 0, ccl::(anonymous namespace)::Policy<256, 2, "
      "true, 2> >(ccl::(anonymous namespace)::ShardArgs)")
PAD = "void ccl::(anonymous namespace)::pad_kernel<ccl::F32, 0>(ccl::(anonymous namespace)::PadArgs)"


def test_trace_summary_groups_by_kernel_shape_and_grid(tmp_path):
    header = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Grid_Size_X"]
    rows = [["KERNEL_DISPATCH", AG, 0, 1000, 256, 256 * 4096],
            ["KERNEL_DISPATCH", AG, 0, 3000, 256, 256 * 4096],
            ["KERNEL_DISPATCH", AG, 0, 500, 256, 256 * 1024],
            ["KERNEL_DISPATCH", RS, 0, 7000, 256, 256 * 2048]]
    trace = tmp_path / "t.csv"
    _write_csv(trace, header, rows)
    out = tmp_path / "t.md"
    profiling.trace(str(trace), str(out), "the command")
    lines = out.read_text().splitlines()
    assert "the command" in lines
    table = [ln for ln in lines if ln.startswith("| `")]
    assert table[0] == "| `rs_direct_kernel` (256 lanes x 2 vectors) | 2048 | 1 | 7.0 | 7.0 | 7.0 | 0.01 |"
    assert "| `ag_direct_kernel` | 4096 | 2 | 2.0 | 1.0 | 3.0 | 0.00 |" in table
    assert "| `ag_direct_kernel` | 1024 | 1 | 0.5 | 0.5 | 0.5 | 0.00 |" in table


def test_traffic_scales_each_counter_by_the_plain_copy(tmp_path):
    header = ["Kernel_Name", "Counter_Value"]
    # the calibration copy moves 1 MiB each way; FETCH_SIZE reads half of it, WRITE_SIZE all of it
    fetch = [[PAD, 512.0], [AG, 64.0], [RS, 4096.0], [RS, 4096.0]]
    write = [[PAD, 1024.0], [AG, 1024.0], [RS, 128.0], [RS, 128.0]]
    _write_csv(tmp_path / "f.csv", header, fetch)
    _write_csv(tmp_path / "w.csv", header, write)
    info = {"counters_pass": True, "copy_read_bytes": 1 << 20, "copy_write_bytes": 1 << 20,
            "calls": {"ag_direct_kernel": 9 * 128 * 1024, "rs_direct_kernel": 2 * 9 * 128 * 1024},
            "kernel_source_digests": {"ag_direct_kernel": "a" * 16, "rs_direct_kernel": "b" * 16,
                                      "pad_kernel": "c" * 16}}
    (tmp_path / "pass.out").write_text("noise\n" + json.dumps(info) + "\n")
    rec = profiling.traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "pass.out"), "w",
                            str(tmp_path / "t.json"), str(tmp_path / "t.md"), "cmd")
    ag = rec["ag_direct_kernel:w"]
    assert ag["read_bytes"] == 128 * 1024 and ag["write_bytes"] == 1024 * 1024
    assert ag["traffic_over_algorithmic"] == pytest.approx(1.0)
    assert ag["source_digest"] == "a" * 16
    rs = rec["rs_direct_kernel:w"]
    assert rs["dispatches"] == 2
    assert rs["call_traffic_bytes"] == 2 * (8192 * 1024 + 128 * 1024)
    assert rs["traffic_bytes"] == rs["call_traffic_bytes"] / 2
    assert json.loads((tmp_path / "t.json").read_text()) == rec
    assert "`rs_direct_kernel` | 2 |" in (tmp_path / "t.md").read_text()


def test_traffic_calibrates_on_every_padding_dispatch_and_merges_workloads(tmp_path):
    """Above 64 ranks the calibration's one padding call is several
    dispatches: the scale uses their sum.  A second workload's records join
    the first's in the same file instead of replacing them."""
    header = ["Kernel_Name", "Counter_Value"]
    fetch = [[PAD, 128.0], [PAD, 128.0], [PAD, 128.0], [PAD, 128.0], [AG, 64.0]]
    write = [[PAD, 256.0], [PAD, 256.0], [PAD, 256.0], [PAD, 256.0], [AG, 1024.0]]
    _write_csv(tmp_path / "f.csv", header, fetch)
    _write_csv(tmp_path / "w.csv", header, write)
    info = {"counters_pass": True, "copy_read_bytes": 1 << 20, "copy_write_bytes": 1 << 20,
            "calls": {"ag_direct_kernel": 9 * 128 * 1024},
            "kernel_source_digests": {"ag_direct_kernel": "a" * 16, "pad_kernel": "c" * 16}}
    (tmp_path / "pass.out").write_text(json.dumps(info) + "\n")
    out = tmp_path / "t.json"
    out.write_text(json.dumps({"ag_direct_kernel:other": {"traffic_bytes": 1.0}}))
    rec = profiling.traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "pass.out"), "w",
                            str(out), str(tmp_path / "t.md"), "cmd")
    ag = rec["ag_direct_kernel:w"]
    assert ag["fetch_scale"] == pytest.approx(2.0) and ag["write_scale"] == pytest.approx(1.0)
    assert ag["traffic_over_algorithmic"] == pytest.approx(1.0)
    merged = json.loads(out.read_text())
    assert set(merged) == {"ag_direct_kernel:other", "ag_direct_kernel:w"}


def test_latency_ratio_is_stated_only_when_both_cvs_are_small():
    res = {"a": {"median_ms": 3.0, "cv": 0.01}, "b": {"median_ms": 2.5, "cv": 0.02},
           "noisy": {"median_ms": 2.0, "cv": 0.08}, "failed": {"error": "refused"}}
    r = bench.latency_ratio(res, "a", "b", 9 / 8)
    assert r["ratio"] == 3.0 / 2.5 and r["bytes_ratio"] == 9 / 8 and r["of"] == "a / b"
    assert bench.latency_ratio(res, "a", "noisy", 1.0)["ratio"] is None
    assert bench.latency_ratio(res, "a", "failed", 1.0) is None
    assert bench.latency_ratio(res, "a", "missing", 1.0) is None


def test_label_rows_on_every_row_shape():
    """Timed rows get a CV flag and a rate kind; the chained drivers and
    the cache-resident shape are labelled cache-assisted; rows with a list
    of CVs (the latency ratio) or without a rate are left as they are;
    rows covered by counters get their traffic ratio; the persistent-ring
    rows say how their steps were ordered."""
    rows = {
        "allreduce_ring_stepwise": {"gbs": 5000.0, "cv": 0.01},
        "rs_ag_direct": {"gbs": 6000.0, "cv": 0.07},
        "allreduce_ring_chained_256x4194304_fp32": {"gbs": 6900.0, "cv": 0.0},
        "rs_ag_direct_8x1048576_fp32_cache_resident": {"gbs": 3000.0, "calls": 100, "mean_ms": 0.02},
        "ratio_rs_ag_over_allreduce_direct": {"of": "a / b", "ratio": None, "cv": [0.01, 0.09]},
        "launch_floor_allreduce_direct_8x64": {"gbs": None, "calls": 100},
        "rs_ag_ring_chained_m2^24": {"gbs": 7000.0, "cv": 0.02},
        "allreduce_ring_persistent": {"gbs": 5600.0, "cv": 0.01},
        "rs_ag_ring_persistent_m2^24": {"gbs": 6000.0, "cv": 0.01},
        "allreduce_ring_persistent_256x6553600_bf16": {"gbs": 5600.0, "cv": 0.01},
        "broken": {"error": "refused"},
        "ratio_missing": None,
    }
    bench.label_rows(rows, "uniform_8x268435456_fp32")
    assert rows["allreduce_ring_stepwise"]["cv_over_5pct"] is False
    assert rows["allreduce_ring_stepwise"]["rate_kind"] == "hbm"
    assert rows["rs_ag_direct"]["cv_over_5pct"] is True
    assert rows["allreduce_ring_chained_256x4194304_fp32"]["rate_kind"] == "effective_cache_assisted"
    assert rows["rs_ag_ring_chained_m2^24"]["rate_kind"] == "effective_cache_assisted"
    assert rows["rs_ag_direct_8x1048576_fp32_cache_resident"]["rate_kind"] == "effective_cache_assisted"
    assert "cv_over_5pct" not in rows["ratio_rs_ag_over_allreduce_direct"]
    assert rows["broken"] == {"error": "refused"}
    # the persistent rows say how the library ordered their steps
    assert rows["allreduce_ring_persistent"]["ordering"] == "grid"
    assert rows["rs_ag_ring_persistent_m2^24"]["ordering"] == "flags"
    assert rows["allreduce_ring_persistent_256x6553600_bf16"]["ordering"] == "flags"
    assert "ordering" not in rows["allreduce_ring_stepwise"]
    assert "rate_kind" not in rows["launch_floor_allreduce_direct_8x64"]
    assert bench.row_kernels("allreduce_ring_persistent_256x6553600_bf16", "w") == \
        (["ring_persistent_flags_kernel"], "normal_256x6553600_bf16")
    assert bench.row_kernels("allreduce_ring_persistent", "uniform_8x268435456_fp32") == \
        (["ring_persistent_kernel"], "uniform_8x268435456_fp32")
    assert bench.row_kernels("allreduce_ring_persistent", "w") is None
    assert bench.row_kernels("rs_ag_direct", "w") == (["rs_direct_kernel", "ag_direct_kernel"], "w")
    assert bench.row_kernels("rs_ag_ring_chained_m2^24", "w") is None
    assert bench.row_kernels("allreduce_direct_8x268435456_bf16", "w") is None


def test_traffic_merges_passes_over_different_schedules(tmp_path):
    """The persistent ring's counters come from a pass of their own: a
    second pass on the same workload replaces only the kernels it measured,
    keeps the first pass's records, and the summary lists every record of
    the workload with both passes' commands."""
    header = ["Kernel_Name", "Counter_Value"]
    ring = "void ccl::(anonymous namespace)::ring_step_kernel<ccl::F32, 0, Policy<256, 1, true, 2>>(RingArgs)"
    pers = "void ccl::(anonymous namespace)::ring_persistent_kernel<ccl::F32, 0, Policy<256, 4, true, 2>, false>(R)"
    out, md = tmp_path / "t.json", tmp_path / "t.md"

    def one_pass(name, kernel_name, kernel, schedules_arg):
        _write_csv(tmp_path / f"{name}.f.csv", header, [[PAD, 512.0], [AG, 64.0], [kernel_name, 1536.0]])
        _write_csv(tmp_path / f"{name}.w.csv", header, [[PAD, 1024.0], [AG, 1024.0], [kernel_name, 2048.0]])
        info = {"counters_pass": True, "copy_read_bytes": 1 << 20, "copy_write_bytes": 1 << 20,
                "counters_schedules_arg": schedules_arg,
                "calls": {"ag_direct_kernel": 9 * 128 * 1024, kernel: 5 * 1024 * 1024},
                "kernel_source_digests": {"ag_direct_kernel": "a" * 16, kernel: "d" * 16, "pad_kernel": "c" * 16}}
        (tmp_path / f"{name}.out").write_text(json.dumps(info) + "\n")
        return profiling.traffic(str(tmp_path / f"{name}.f.csv"), str(tmp_path / f"{name}.w.csv"),
                                 str(tmp_path / f"{name}.out"), "w", str(out), str(md), f"cmd {name}")

    one_pass("rest", ring, "ring_step_kernel", "direct,ring_stepwise")
    one_pass("pers", pers, "ring_persistent_kernel", "ring_persistent")
    merged = json.loads(out.read_text())
    assert set(merged) == {"ag_direct_kernel:w", "ring_step_kernel:w", "ring_persistent_kernel:w"}
    assert merged["ring_step_kernel:w"]["command"] == "cmd rest"
    assert merged["ring_persistent_kernel:w"]["command"] == "cmd pers"
    assert merged["ring_persistent_kernel:w"]["traffic_over_algorithmic"] == pytest.approx(1.0)
    text = md.read_text()
    assert "`ring_step_kernel`" in text and "`ring_persistent_kernel`" in text and "`ag_direct_kernel`" in text
    assert "--counters-schedules direct,ring_stepwise" in text and "--counters-schedules ring_persistent" in text
    assert text.index("`ag_direct_kernel`") < text.index("`ring_step_kernel`") < text.index("`ring_persistent_kernel`")
