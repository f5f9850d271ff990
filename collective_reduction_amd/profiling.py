"""Turn rocprofv3 output into the short summaries kept under profiles/.

    python -m collective_reduction_amd.profiling stats  <kernel_stats.csv> <out.md> <command...>
    python -m collective_reduction_amd.profiling traffic <fetch_counter_collection.csv> \
        <write_counter_collection.csv> <counters_pass_stdout> <workload> <out.json> <command...>

``stats`` keeps the per-kernel call count and durations of a
``--kernel-trace --stats`` run.  ``traffic`` reads two ``--pmc`` runs of
``bench.py --counters-pass`` (FETCH_SIZE, then WRITE_SIZE; KiB per
dispatch) and scales each counter by what it reads for the plain copy in
the same pass (``ccl_sim_pad_identity`` with nothing to pad, which reads
and writes a known N·M·s bytes), giving HBM bytes per launch of the
ReduceScatter and AllGather kernels.  The record carries the digest of the
kernel sources the counters were taken on; bench.py reports the traffic
only while that digest still matches.
"""

import csv
import json
import os
import sys


def _short(name):
    for key in ("rs_direct_kernel", "ag_direct_kernel", "ar_direct_kernel", "ring_step_kernel",
                "ring_persistent_kernel", "pad_kernel", "reset_ctrl_kernel", "store_table_kernel"):
        if key in name:
            return key
    return name


def stats(stats_csv, out_md, command):
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [
        "# rocprofv3 kernel statistics",
        "",
        "Command (from the repository root on the GPU box, after `cd /tmp && export TMPDIR=/tmp`):",
        "",
        "```",
        command,
        "```",
        "",
        "| kernel | calls | average µs | min µs | max µs | total ms |",
        "|---|---:|---:|---:|---:|---:|",
    ]
    for r in rows:
        lines.append("| `{}` | {} | {:.1f} | {:.1f} | {:.1f} | {:.2f} |".format(
            _short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e6))
    lines.append("")
    lines.append("Full kernel names: " + "; ".join(sorted({r["Name"] for r in rows})))
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _counter(path):
    vals = {}
    for r in csv.DictReader(open(path)):
        vals.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return vals


def traffic(fetch_csv, write_csv, pass_out, workload, out_json, command):
    info = None
    for line in open(pass_out):
        line = line.strip()
        if line.startswith("{") and "counters_pass" in line:
            info = json.loads(line)
    if info is None:
        raise SystemExit("no counters-pass record in " + pass_out)
    fetch, write = _counter(fetch_csv), _counter(write_csv)
    fscale = info["copy_read_bytes"] / (fetch["pad_kernel"][0] * 1024)
    wscale = info["copy_write_bytes"] / (write["pad_kernel"][0] * 1024)
    rec = {}
    if os.path.exists(out_json):
        rec = json.load(open(out_json))
    for kernel, algo in (("rs_direct_kernel", info["rs_bytes"]), ("ag_direct_kernel", info["ag_bytes"])):
        rd = fetch[kernel][0] * 1024 * fscale
        wr = write[kernel][0] * 1024 * wscale
        rec[f"{kernel}:{workload}"] = {
            "traffic_bytes": rd + wr,
            "read_bytes": rd,
            "write_bytes": wr,
            "algorithmic_bytes": algo,
            "traffic_over_algorithmic": (rd + wr) / algo,
            "fetch_size_kib": fetch[kernel][0],
            "write_size_kib": write[kernel][0],
            "fetch_scale": fscale,
            "write_scale": wscale,
            "calibration": "ccl_sim_pad_identity with count == padded_count (plain copy of N*M elements)",
            "source_digest": info["kernel_source_digest"],
            "command": command,
        }
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "stats":
        stats(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]))
    elif mode == "traffic":
        traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6], " ".join(sys.argv[7:]))
    else:
        raise SystemExit(__doc__)
