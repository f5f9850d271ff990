"""Turn rocprofv3 output into the short summaries kept under profiles/.

    python -m collective_reduction_amd.profiling stats  <kernel_stats.csv> <out.md> <command...>
    python -m collective_reduction_amd.profiling trace  <kernel_trace.csv> <out.md> <command...>
    python -m collective_reduction_amd.profiling traffic <fetch_counter_collection.csv> \
        <write_counter_collection.csv> <counters_pass_stdout> <workload> <out.json> <out.md>

``stats`` keeps the per-kernel call count and durations of a
``--kernel-trace --stats`` run; ``trace`` computes the same from the
per-dispatch trace, grouped by kernel, launch shape and grid size.  ``traffic`` reads two ``--pmc`` runs of
``bench.py --counters-pass`` (FETCH_SIZE, then WRITE_SIZE; KiB per
dispatch) and scales each counter by what it reads for the plain copy in
the same pass (``ccl_sim_pad_identity`` with nothing to pad, which reads
and writes a known N·M·s bytes).  For each call of the pass it sums the
counters over the call's dispatches of its kernel (one for the direct
kernels, the persistent and chained ring and the chained recursive driver,
2(N-1) for the stepwise ring, 2·log2 N for the stepwise recursive one) and
sets the HBM bytes beside the call's
algorithmic bytes.  It writes ``profiles/traffic.json`` and a Markdown
table of the same figures.  The record carries the digest of the kernel
sources the counters were taken on; bench.py reports the traffic only
while that digest still matches.
"""

import csv
import json
import os
import re
import sys


def _short(name):
    for key in ("rs_direct_kernel", "ag_direct_kernel", "ar_direct_kernel", "ring_step_kernel",
                "ring_persistent_kernel", "ring_persistent_flags_kernel", "ring_chained_kernel",
                "recursive_step_kernel", "recursive_chained_kernel", "pad_kernel", "reset_ctrl_kernel",
                "store_table_kernel"):
        if key in name:
            return key
    # another library's kernel (torch's fill and random kernels): its bare
    # function name, without namespaces, template arguments or parameters
    head = re.split(r"[<(]", name.replace("(anonymous namespace)", ""), maxsplit=1)[0].split()
    return head[-1].split("::")[-1] if head else name


def _shape(name):
    """The launch shape a kernel instance was built with (its Policy's lanes
    per workgroup and vectors per lane), when the name carries one."""
    m = re.search(r"Policy<(\d+), (\d+),", name)
    return f" ({m.group(1)} lanes x {m.group(2)} vectors)" if m else ""


def stats(stats_csv, out_md, command):
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [
        "# rocprofv3 kernel statistics",
        "",
        "Command (run from `/tmp` with `TMPDIR=/tmp`; `<repo>` is the repository root):",
        "",
        "```",
        command,
        "```",
        "",
        "| kernel | calls | average µs | min µs | max µs | total ms |",
        "|---|---:|---:|---:|---:|---:|",
    ]
    for r in rows:
        lines.append("| `{}`{} | {} | {:.1f} | {:.1f} | {:.1f} | {:.2f} |".format(
            _short(r["Name"]), _shape(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e6))
    lines.append("")
    lines.append("Full kernel names: " + "; ".join(sorted({r["Name"] for r in rows})))
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def trace(trace_csv, out_md, command):
    """Per-kernel durations from a --kernel-trace CSV, grouped by kernel,
    launch shape and grid size, so that launches of one kernel at different
    sizes (the bench's own step and its secondary runs) stay apart."""
    groups = {}
    for r in csv.DictReader(open(trace_csv)):
        if r.get("Kind", "KERNEL_DISPATCH") != "KERNEL_DISPATCH":
            continue
        name = r["Kernel_Name"]
        key = (_short(name), _shape(name), int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])))
        ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        groups.setdefault(key, []).append(ns)
    lines = [
        "# rocprofv3 kernel trace, grouped by kernel and grid",
        "",
        "Command (run from `/tmp` with `TMPDIR=/tmp`; `<repo>` is the repository root):",
        "",
        "```",
        command,
        "```",
        "",
        "The rows come from the run's per-dispatch `kernel_trace.csv`. rocprofv3's own `--stats` table averages "
        "every launch of one kernel instance across sizes; here launches are grouped by kernel, launch shape and "
        "grid size, so that the bench step's launches (the largest grids) keep a row of their own.",
        "",
        "| kernel | workgroups | calls | average µs | min µs | max µs | total ms |",
        "|---|---:|---:|---:|---:|---:|---:|",
    ]
    for (kernel, shape, wgs), ns in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{kernel}`{shape} | {wgs} | {len(ns)} | {sum(ns) / len(ns) / 1e3:.1f} | {min(ns) / 1e3:.1f} "
                     f"| {max(ns) / 1e3:.1f} | {sum(ns) / 1e6:.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _counter(path):
    vals = {}
    for r in csv.DictReader(open(path)):
        vals.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return vals


def traffic(fetch_csv, write_csv, pass_out, workload, out_json, out_md, command):
    info = None
    for line in open(pass_out):
        line = line.strip()
        if line.startswith("{") and "counters_pass" in line:
            info = json.loads(line)
    if info is None:
        raise SystemExit("no counters-pass record in " + pass_out)
    fetch, write = _counter(fetch_csv), _counter(write_csv)
    extra = info.get("counters_schedules_arg")
    pass_commands = [f"rocprofv3 --pmc {c} --kernel-trace -d <out> -o pmc --output-format csv -- python "
                     f"<repo>/bench.py --workload {workload} --counters-pass" + (f" --counters-schedules {extra}"
                                                                                  if extra else "")
                     for c in ("FETCH_SIZE", "WRITE_SIZE")]
    # the pass makes one padding call; above 64 ranks it is several
    # dispatches (one per 64-rank group), so the calibration sums them all
    fscale = info["copy_read_bytes"] / (sum(fetch["pad_kernel"]) * 1024)
    wscale = info["copy_write_bytes"] / (sum(write["pad_kernel"]) * 1024)
    rec = {}
    for kernel, algo in info["calls"].items():
        if len(fetch[kernel]) != len(write[kernel]):
            raise SystemExit(f"{kernel}: {len(fetch[kernel])} FETCH_SIZE and {len(write[kernel])} WRITE_SIZE records")
        k = len(fetch[kernel])
        rd = sum(fetch[kernel]) * 1024 * fscale
        wr = sum(write[kernel]) * 1024 * wscale
        rec[f"{kernel}:{workload}"] = {
            "dispatches": k,
            "traffic_bytes": (rd + wr) / k,
            "read_bytes": rd / k,
            "write_bytes": wr / k,
            "algorithmic_bytes": algo / k,
            "call_traffic_bytes": rd + wr,
            "call_algorithmic_bytes": algo,
            "traffic_over_algorithmic": (rd + wr) / algo,
            "fetch_size_kib": sum(fetch[kernel]),
            "write_size_kib": sum(write[kernel]),
            "fetch_scale": fscale,
            "write_scale": wscale,
            "calibration": "ccl_sim_pad_identity with count == padded_count (plain copy of N*M elements)",
            "source_digest": info["kernel_source_digests"][kernel],
            "command": command,
            "pass_commands": pass_commands,
        }
    # one file holds every workload's records: replace the kernels this pass
    # measured on this workload, keep the rest (other workloads, and kernels
    # of this workload that a pass over other schedules measured)
    merged = {}
    if os.path.exists(out_json):
        with open(out_json) as f:
            merged = {k: v for k, v in json.load(f).items() if k not in rec}
    merged.update(rec)
    with open(out_json, "w") as f:
        json.dump(dict(sorted(merged.items())), f, indent=1)
        f.write("\n")
    here = {k: v for k, v in merged.items() if k.endswith(":" + workload)}
    _traffic_md(here, workload, info, out_md)
    return rec


KERNEL_ORDER = ("rs_direct_kernel", "ag_direct_kernel", "ar_direct_kernel", "ring_step_kernel",
                "ring_persistent_kernel", "ring_persistent_flags_kernel", "ring_chained_kernel",
                "recursive_step_kernel", "recursive_chained_kernel")


def _traffic_md(rec, workload, info, out_md):
    """The Markdown summary of every record of one workload, with the
    commands of the passes that produced them and each pass's calibration."""
    what = {"rs_direct_kernel": "ReduceScatter, direct", "ag_direct_kernel": "AllGather, direct",
            "ar_direct_kernel": "AllReduce, direct (one kernel)",
            "ring_step_kernel": "AllReduce, stepwise ring (all steps)",
            "ring_persistent_kernel": "AllReduce, persistent ring, grid barrier (one launch)",
            "ring_persistent_flags_kernel": "AllReduce, persistent ring, step flags (one launch)",
            "ring_chained_kernel": "AllReduce, chained ring (one launch)",
            "recursive_step_kernel": "AllReduce, recursive halving + doubling (all steps)",
            "recursive_chained_kernel": "AllReduce, chained recursive halving + doubling (one launch)"}
    order = {k: i for i, k in enumerate(KERNEL_ORDER)}
    keys = sorted(rec, key=lambda k: order.get(k.split(":")[0], len(order)))
    commands = []
    for k in keys:
        for c in rec[k].get("pass_commands", []) + [rec[k]["command"]]:
            if c not in commands:
                commands.append(c)
    scales = sorted({(round(1 / r["fetch_scale"], 4), round(1 / r["write_scale"], 6)) for r in rec.values()})
    lines = [
        f"# HBM traffic of the library's kernels (rocprofv3 counters), {workload}",
        "",
        "Commands (from `/tmp` with `TMPDIR=/tmp`; `<repo>` is the repository root):",
        "",
        "```",
        *commands,
        "```",
        "",
        f"Calibration: every pass runs `ccl_sim_pad_identity` with nothing to pad, a plain copy that reads and "
        f"writes exactly {info['copy_read_bytes']:,} bytes, and each kernel's counters are multiplied by the factors "
        f"that copy gives in the same pass. FETCH_SIZE / WRITE_SIZE reported "
        + "; ".join(f"{f} / {w}" for f, w in scales) +
        " of the copy's bytes. Figures are per call, summed over the call's dispatches.",
        "",
        "| call | kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read B | HBM write B | traffic B "
        "| algorithmic B | traffic / algorithmic | source digest |",
        "|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---|",
    ]
    for key in keys:
        r = rec[key]
        kernel = key.split(":")[0]
        lines.append(
            f"| {what.get(kernel, kernel)} | `{kernel}` | {r['dispatches']} | {r['fetch_size_kib']:.1f} | "
            f"{r['write_size_kib']:.1f} | {r['read_bytes'] * r['dispatches']:.4e} | "
            f"{r['write_bytes'] * r['dispatches']:.4e} | {r['call_traffic_bytes']:.4e} | "
            f"{r['call_algorithmic_bytes']:.4e} | {r['traffic_over_algorithmic']:.5f} | `{r['source_digest']}` |")
    lines += ["", "Source digest: the kernel's own source file and the shared device headers, without comments, "
              "when the counters were taken; bench.py reports a kernel's `traffic` only while its sources still "
              "hash to it."]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "stats":
        stats(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]))
    elif mode == "trace":
        trace(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]))
    elif mode == "traffic":
        traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6], sys.argv[7],
                "python -m collective_reduction_amd.profiling " + " ".join(sys.argv[1:]))
    else:
        raise SystemExit(__doc__)
