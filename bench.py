"""Throughput of ReduceScatter + AllGather AllReduce over N virtual ranks on
one MI355X, through the C-ABI library.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is the whole hot path on one batch: ccl_sim_reduce_scatter followed
by ccl_sim_all_gather (direct fused schedule) over N=8 ranks of M=2^28
float32 each, inputs resident in HBM.  W untimed steps, then K timed steps
between device synchronisations.  The value is effective HBM bandwidth:
the schedule's algorithmic bytes 2(N+1)·M·4 divided by the time per step.

Also reported: per-kernel durations from HIP events on the launch stream
(the roofline of the dominant kernel); on the same buffers, the other
schedules (RS+AG under the three ring drivers and both recursive drivers,
every schedule's AllReduce, RS alone, smaller M), timed in interleaved
rounds; the 256-rank float32 and bf16 workloads and the bench's shape in
bf16; the alpha-beta model of the same payload on two networks; the
measured buffer lifetimes; and the CPU oracle timed on a bounded sample of
the workload.  Prints exactly one JSON line on stdout; progress goes to
stderr.
"""

import os

# The CPU baseline times the oracle on one core: pin NumPy's and any BLAS
# thread pools to one thread before NumPy (or torch, which loads it) is
# imported.  Nothing else here uses those pools; the input generator's
# worker threads are Python threads.
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS",
             "NUMEXPR_NUM_THREADS", "VECLIB_MAXIMUM_THREADS"):
    os.environ[_var] = "1"

import argparse  # noqa: E402
import hashlib  # noqa: E402
import json  # noqa: E402
import re  # noqa: E402
import statistics  # noqa: E402
import sys  # noqa: E402
import time  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
# The headline: N=8 virtual ranks of 2^28 float32 elements (1 GiB each).
DEFAULT_WORKLOAD = "uniform_8x268435456_fp32"
METRIC = "effective HBM GB/s (and % of peak) for RS+AG AllReduce, N=8, M=2^28 fp32"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, vendor figure


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--secondary-iters", type=int, default=10)
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle work for cpu_baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--counters-pass", action="store_true",
                   help="run one RS, one AG and one plain copy of known size, for rocprofv3 --pmc")
    p.add_argument("--counters-schedules", default=",".join(AR_KERNEL),
                   help="the AllReduce schedules the counters pass runs (comma-separated)")
    return p.parse_args()


# The source file that holds each kernel; every kernel also depends on the
# shared device headers.
KERNEL_FILES = {
    "rs_direct_kernel": "kernels_direct.hip",
    "ag_direct_kernel": "kernels_direct.hip",
    "ar_direct_kernel": "kernels_direct.hip",
    "ring_step_kernel": "kernels_ring.hip",
    "ring_persistent_kernel": "kernels_ring.hip",
    "ring_persistent_flags_kernel": "kernels_ring.hip",
    "ring_chained_kernel": "kernels_ring.hip",
    "recursive_step_kernel": "kernels_recursive.hip",
    "recursive_chained_kernel": "kernels_recursive.hip",
    "pad_kernel": "kernels_misc.hip",
}


def kernel_source_digest(kernel, csrc=None):
    """Digest of the device code a kernel is built from: its own source file
    and the shared headers, with comments and whitespace dropped first, so
    a comment edit or a change to another kernel's file does not count as a
    change of this kernel."""
    csrc = csrc or os.path.join(HERE, "collective_reduction_amd", "csrc")
    h = hashlib.sha256()
    for name in ("kernel_common.hpp", "device.hpp", "internal.hpp", KERNEL_FILES[kernel]):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload, path=None):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None
    when none were taken for this kernel and workload or the kernel source
    has changed since."""
    entry = load_traffic_entry(kernel, workload, path)
    return entry.get("traffic_bytes") if entry else None


def load_traffic_entry(kernel, workload, path=None):
    """The committed counter record of one kernel on one workload, or None
    when none was taken or the kernel's source has changed since."""
    path = path or os.path.join(HERE, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(f"{kernel}:{workload}")
    if not entry or entry.get("source_digest") != kernel_source_digest(kernel):
        return None
    return entry


AR_KERNEL = {"direct": "ar_direct_kernel", "ring_stepwise": "ring_step_kernel",
             "ring_persistent": "ring_persistent_kernel", "ring_chained": "ring_chained_kernel",
             "recursive": "recursive_step_kernel", "recursive_chained": "recursive_chained_kernel"}
ROW_WORKLOADS = {"256x4194304_fp32": "normal_256x4194304_fp32", "256x6553600_bf16": "normal_256x6553600_bf16"}
PERSISTENT_KERNEL = {"grid": "ring_persistent_kernel", "flags": "ring_persistent_flags_kernel"}


def persistent_ordering(nranks, count):
    """How the library's persistent ring orders the steps of an AllReduce
    of this shape ("grid" or "flags"), as the library itself reports it."""
    from collective_reduction_amd import ccl_sim
    return ccl_sim.ccl_sim_persistent_ordering("allreduce", nranks, count)


def ar_kernel(schedule, nranks, count):
    """The kernel an AllReduce of `schedule` runs on N = nranks, M = count:
    the persistent ring's kernel depends on how it orders the steps."""
    if schedule == "ring_persistent":
        return PERSISTENT_KERNEL[persistent_ordering(nranks, count)]
    return AR_KERNEL[schedule]


def row_shape(name, default_workload):
    """(row name without its workload suffix, workload, N, M) of a bench
    row: the 256-rank rows name their workload, the _m2^k rows run the
    default workload's first 2^k positions, the rest the default workload;
    N and M are None for a workload this module does not know."""
    from collective_reduction_amd import inputs as I
    workload = default_workload
    for suffix, wl in ROW_WORKLOADS.items():
        if name.endswith("_" + suffix):
            name, workload = name[:-len(suffix) - 1], wl
            break
    spec = I.WORKLOADS.get(workload)
    n, m = (spec["nranks"], spec["count"]) if spec else (None, None)
    if "_m2^" in name:
        name, lg = name.rsplit("_m2^", 1)
        m = 1 << int(lg)
    return name, workload, n, m


def row_kernels(name, default_workload):
    """(kernels, workload) whose committed counters cover one bench row, or
    None: the AllReduce rows (one kernel each), the direct ReduceScatter
    alone, and the direct RS+AG pair."""
    if "_m2^" in name or (name.endswith("_bf16") and not any(name.endswith("_" + s) for s in ROW_WORKLOADS)):
        return None
    name, workload, n, m = row_shape(name, default_workload)
    if name.startswith("allreduce_") and name[len("allreduce_"):] in AR_KERNEL:
        schedule = name[len("allreduce_"):]
        if schedule == "ring_persistent" and n is None:
            return None
        return [ar_kernel(schedule, n, m)], workload
    if name == "rs_only_direct":
        return ["rs_direct_kernel"], workload
    if name == "rs_ag_direct":
        return ["rs_direct_kernel", "ag_direct_kernel"], workload
    return None


def label_rows(rows, default_workload):
    """Say what each timed row's rate is.  Every row gets `cv_over_5pct`
    (its median is then not stable enough to compare against another
    row's; [DECOMP] states no ratio past that spread) and `rate_kind`:
    "hbm" where the row's bytes come from HBM, or "effective_cache_assisted"
    for the chained drivers and the cache-resident workload, whose data is
    partly served from the 256 MB Infinity Cache (a chained driver reads
    each partial back soon after writing it), so that their fraction of the
    HBM peak is an effective rate, not an HBM roofline fraction.  Rows
    covered by committed rocprofv3 counters also get
    `traffic_over_algorithmic`: L2-to-fabric bytes (FETCH_SIZE +
    WRITE_SIZE, calibrated on a plain copy) over algorithmic bytes.  Those
    counters see Infinity Cache hits as fetches, so a ratio near 1 does not
    show how much of a row came from HBM itself."""
    for name, row in rows.items():
        if not isinstance(row, dict):
            continue
        if isinstance(row.get("cv"), float):
            row["cv_over_5pct"] = row["cv"] > 0.05
        if row.get("gbs") is not None:
            cached = "chained" in name or "cache_resident" in name
            row["rate_kind"] = "effective_cache_assisted" if cached else "hbm"
        if "ring_persistent" in name:
            _, _, n, m = row_shape(name, default_workload)
            if n is not None:
                row["ordering"] = persistent_ordering(n, m)
        cover = row_kernels(name, default_workload)
        if cover is None:
            continue
        kernels, workload = cover
        entries = [load_traffic_entry(k, workload) for k in kernels]
        if all(entries):
            traffic = sum(e["call_traffic_bytes"] for e in entries)
            alg = sum(e["call_algorithmic_bytes"] for e in entries)
            row["traffic_over_algorithmic"] = traffic / alg
            row["traffic_source"] = [f"{k}:{workload}" for k in kernels]


def stats(ms):
    ms = sorted(ms)
    med = statistics.median(ms)
    p95 = ms[min(len(ms) - 1, int(round(0.95 * (len(ms) - 1))))]
    mean = statistics.fmean(ms)
    cv = statistics.pstdev(ms) / mean if len(ms) > 1 and mean > 0 else 0.0
    return {"median_ms": med, "p95_ms": p95, "mean_ms": mean, "cv": cv}


def cpu_baseline(spec, target_s):
    """The oracle's RS + AG timed on a bounded sample: the first qs positions
    of every shard (so the sample keeps the rank-major structure), qs grown
    until the oracle's own work reaches about target_s seconds.  When the
    whole workload takes less than that, it is run again until the passes
    together reach target_s, and the rate is their total bytes over their
    total time."""
    import numpy as np
    from collective_reduction_amd import inputs as I
    from oracle import collectives as C

    n, m = spec["nranks"], spec["count"]
    q = -(-m // n)
    es = np.dtype(I._STORAGE[spec["dtype"]]).itemsize

    def sample(qs):
        xs = []
        for r in range(n):
            parts = [I.rank_buffer(spec, r, s * q, min(s * q + qs, m), workers=8) for s in range(n)]
            xs.append(np.concatenate(parts))
        return xs

    qs = min(q, 1 << 16)
    while True:
        xs = sample(qs)
        t0 = time.perf_counter()
        shards = C.reduce_scatter(xs, "sum", spec["dtype"], qs)
        C.all_gather(shards)
        dt = time.perf_counter() - t0
        if dt >= target_s or qs >= q:
            break
        qs = min(q, max(qs * 2, int(qs * target_s / max(dt, 1e-3) * 1.1)))
        del xs, shards
    passes, total = 1, dt
    while total < target_s:
        t0 = time.perf_counter()
        shards = C.reduce_scatter(xs, "sum", spec["dtype"], qs)
        C.all_gather(shards)
        total += time.perf_counter() - t0
        passes += 1
    dt = total
    nbytes = 2 * (n + 1) * n * qs * es * passes
    threads = os.environ.get("OMP_NUM_THREADS")
    pools = None
    try:
        from threadpoolctl import threadpool_info
        pools = sorted({p.get("num_threads") for p in threadpool_info()})
    except Exception:  # noqa: BLE001  (the report works without it)
        pass
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {
        "value": nbytes / dt / 1e9,
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"first {qs} positions of each of the {n} shards ({n * qs} of {m} positions per rank, "
                  f"{n} ranks), {passes} pass(es); oracle reduce_scatter + all_gather took {dt:.2f} s in all, "
                  f"single-threaded NumPy",
        "passes": passes,
        "seconds": dt,
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "omp_num_threads": threads,
        "blas_pool_threads": pools,
        "cpu_model": model,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: every rank here is a virtual rank in one GPU's HBM, so "
              f"--gpus {args.gpus} is not supported (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from collective_reduction_amd import ccl_sim as cs
    from collective_reduction_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    spec = I.spec(args.workload)
    n, m, dtype = spec["nranks"], spec["count"], spec["dtype"]
    q = -(-m // n)
    if n * q != m:
        print("the bench workload must divide into N shards", file=sys.stderr)
        sys.exit(2)
    tdt = {"float32": torch.float32, "bfloat16": torch.bfloat16, "int32": torch.int32, "int64": torch.int64}[dtype]
    stream = torch.cuda.current_stream()
    dev_name = torch.cuda.get_device_name(0)
    log(f"device {dev_name}; workload {args.workload}: N={n} M={m} {dtype}")

    # Inputs resident in HBM before timing.
    t0 = time.time()
    send = []
    for r in range(n):
        host = I.rank_buffer(spec, r, workers=16)
        t = torch.empty(m, dtype=tdt, device="cuda")
        if dtype == "bfloat16":
            t.view(torch.int16).copy_(torch.from_numpy(host.view("int16")))
        else:
            t.copy_(torch.from_numpy(host))
        send.append(t)
        del host
        log(f"rank {r} uploaded ({time.time() - t0:.1f} s)")
    shards = [torch.empty(q, dtype=tdt, device="cuda") for _ in range(n)]
    recv = [torch.empty(m, dtype=tdt, device="cuda") for _ in range(n)]
    torch.cuda.synchronize()

    if args.counters_pass:
        counters_pass(cs, torch, stream, send, shards, recv, n, m, q, dtype, args.counters_schedules.split(","))
        del send, shards, recv
        release_device_memory(torch)
        return

    send_elem_size = send[0].element_size()
    bytes_rs = cs.ccl_sim_algorithmic_bytes("reduce_scatter", n, m, dtype, "direct")
    bytes_ag = cs.ccl_sim_algorithmic_bytes("all_gather", n, m, dtype, "direct")
    bytes_step = bytes_rs + bytes_ag

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        cs.ccl_sim_reduce_scatter(send, shards, m, q, op="sum", schedule="direct", stream=stream)
        if ev is not None:
            ev[1].record(stream)
        cs.ccl_sim_all_gather(shards, recv, q, m, schedule="direct", stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"{args.warmup} warmup steps done")

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    log(f"{args.steps} timed steps done in {wall * 1e3:.1f} ms")

    step_ms = [e[0].elapsed_time(e[2]) for e in events]
    rs_ms = [e[0].elapsed_time(e[1]) for e in events]
    ag_ms = [e[1].elapsed_time(e[2]) for e in events]
    ms_per_step = wall * 1e3 / args.steps
    value = bytes_step / (ms_per_step / 1e3) / 1e9

    rs_avg, ag_avg = statistics.fmean(rs_ms), statistics.fmean(ag_ms)
    dominant = ("rs_direct_kernel", rs_avg, bytes_rs) if rs_avg >= ag_avg else ("ag_direct_kernel", ag_avg, bytes_ag)
    achieved = dominant[2] / (dominant[1] / 1e3) / 1e9
    traffic = load_traffic(dominant[0], args.workload)
    roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": traffic, "kernel": dominant[0],
                "avg_launch_ms": dominant[1], "algorithmic_bytes_per_launch": dominant[2]}

    step_collective = collective_context(cs, "all_reduce", n, m * send_elem_size, ms_per_step / 1e3)

    kernels = {
        "rs_direct_kernel": {"avg_ms": rs_avg, "bytes": bytes_rs, "gbs": bytes_rs / (rs_avg / 1e3) / 1e9,
                             **stats(rs_ms)},
        "ag_direct_kernel": {"avg_ms": ag_avg, "bytes": bytes_ag, "gbs": bytes_ag / (ag_avg / 1e3) / 1e9,
                             **stats(ag_ms)},
    }

    secondary = {}
    if not args.no_secondary:
        secondary = run_secondary(cs, torch, stream, send, shards, recv, n, m, q, dtype, args.secondary_iters)
    del send, shards, recv
    release_device_memory(torch)
    if not args.no_secondary:
        secondary.update(run_more_workloads(cs, torch, stream, args.secondary_iters))
        secondary.update(run_small(cs, torch, stream))
        label_rows(secondary, args.workload)

    # Modeled context only (not a measurement, not a target): the pages'
    # α-β model of the same collective between N real ranks on their two
    # example links.
    modeled = {}
    for label, alpha_us, beta_gbps in (("ib_hdr_alpha10us_beta25GBps", 10.0, 25.0),
                                       ("alpha5us_beta300GBps", 5.0, 300.0)):
        for algo in ("ring", "tree"):
            modeled[f"{label}_{algo}"] = cs.ccl_sim_model_estimate("all_reduce", algo, n, m * send_elem_size,
                                                                  alpha_us, beta_gbps)

    lifetimes = lifetimes_big = None
    if not args.no_secondary:
        from collective_reduction_amd import lifetime as LT
        # the pages' example (256 MiB per rank, 4 ranks), then the bench's own scale (1 GiB per rank, 8 ranks)
        lifetimes = {mode: LT.measure(mode, 4, 64 << 20, "float32", "direct") for mode in LT.MODES}
        lifetimes_big = {mode: LT.measure(mode, n, m, dtype, "direct") for mode in LT.MODES}
        for label, lt in (("256 MiB x 4", lifetimes), (f"{m * send_elem_size >> 20} MiB x {n}", lifetimes_big)):
            log(f"lifetimes {label} (MiB per rank, steady/peak): " + ", ".join(
                f"{k} {v['steady'] / 2**20:.0f}/{v['peak'] / 2**20:.0f}" for k, v in lt.items()))

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        cpu = cpu_baseline(spec, args.cpu_seconds)
        log(f"oracle: {cpu['value']:.3f} GB/s over {cpu['seconds']:.1f} s")

    out = {
        "metric": METRIC if args.workload == DEFAULT_WORKLOAD else
                  f"effective HBM GB/s (and % of peak) for RS+AG AllReduce, N={n}, M={m} {dtype}",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"float32": "f32", "bfloat16": "bf16", "int32": "i32", "int64": "i64"}[dtype],
        "data": "synthetic",
        "config": {"workload": args.workload, "nranks": n, "count": m, "op": "sum",
                   "collective": "reduce_scatter + all_gather", "schedule": "direct",
                   "bytes_per_step": bytes_step},
        "frac_of_peak": value / PEAK_HBM_GBS,
        "step_stats": stats(step_ms),
        "collective": step_collective,
        "elements_per_s": n * m / (ms_per_step / 1e3),
        "roofline": roofline,
        "kernels": kernels,
        "secondary": secondary,
        "modeled_context": modeled,
        "lifetimes_256MiB_per_rank_world4": lifetimes,
        "lifetimes_bench_scale": lifetimes_big,
        "cpu_baseline": cpu,
        "device": dev_name,
        "kernel_source_digest": kernel_source_digest(dominant[0]),
    }
    release_device_memory(torch)
    print(json.dumps(out), flush=True)


def release_device_memory(torch):
    """Wait for the device and hand every cached block back to the runtime,
    so that nothing allocated here is still alive when the process exits
    (at exit the HIP runtime, and a profiler's library when one is loaded,
    tear down in an order this program does not control)."""
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def counters_pass(cs, torch, stream, send, shards, recv, n, m, q, dtype, schedules=tuple(AR_KERNEL)):
    """One call of each kernel the bench times, for hardware counters: the
    direct ReduceScatter and AllGather, ccl_sim_pad_identity with nothing to
    pad (a plain copy of N·M elements, reading and writing N·M·s bytes,
    which calibrates FETCH_SIZE / WRITE_SIZE against a known byte count),
    then one AllReduce with each of `schedules` (by default the direct,
    stepwise-ring, persistent-ring, chained-ring and both recursive
    schedules; recursive only for a power-of-two N)."""
    unknown = set(schedules) - set(AR_KERNEL)
    if unknown:
        raise SystemExit(f"unknown schedules {sorted(unknown)}")
    ws = cs.Workspace.largest([("reduce_scatter", n, m, dtype, "direct"), ("all_gather", n, m, dtype, "direct")])
    cs.ccl_sim_reduce_scatter(send, shards, m, q, schedule="direct", workspace=ws, stream=stream)
    cs.ccl_sim_all_gather(shards, recv, q, m, schedule="direct", workspace=ws, stream=stream)
    cs.ccl_sim_pad_identity(send, recv, m, m, "sum", stream=stream)
    calls = {"rs_direct_kernel": cs.ccl_sim_algorithmic_bytes("reduce_scatter", n, m, dtype, "direct"),
             "ag_direct_kernel": cs.ccl_sim_algorithmic_bytes("all_gather", n, m, dtype, "direct")}
    for schedule in AR_KERNEL:
        if schedule not in schedules or (schedule.startswith("recursive") and n & (n - 1)):
            continue
        kernel = ar_kernel(schedule, n, m)
        ws = cs.Workspace("allreduce", n, m, dtype, schedule)
        cs.ccl_sim_allreduce(send, recv, m, schedule=schedule, workspace=ws, stream=stream)
        torch.cuda.synchronize()
        del ws
        calls[kernel] = cs.ccl_sim_algorithmic_bytes("allreduce", n, m, dtype, schedule)
    torch.cuda.synchronize()
    es = send[0].element_size()
    print(json.dumps({"counters_pass": True, "calls": calls,
                      "counters_schedules_arg": None if set(schedules) >= set(AR_KERNEL) else ",".join(schedules),
                      "copy_read_bytes": n * m * es, "copy_write_bytes": n * m * es,
                      "kernel_source_digests": {k: kernel_source_digest(k) for k in list(calls) + ["pad_kernel"]}}),
          flush=True)


def collective_context(cs, coll, nranks, payload_bytes, seconds):
    """nccl-tests style figures for one measured collective of
    `payload_bytes` per rank ([PRIMS] §七): algbw = payload / time and
    busbw = algbw x the collective's bus factor, from the measured time on
    this GPU; and, for context only, the alpha-beta model's time for the same
    collective between N real ranks on an IB HDR-like link (alpha = 10 us,
    beta = 25 GB/s, [PRIMS] §四)."""
    algbw = payload_bytes / seconds / 1e9
    ring = cs.ccl_sim_model_estimate(coll, "ring", nranks, payload_bytes, 10.0, 25.0)
    return {"algbw_gbps": algbw, "busbw_gbps": algbw * cs.ccl_sim_busbw_factor(coll, nranks),
            "modeled_ring_ib_hdr_ms": ring["time_s"] * 1e3}


def pacer_cycles(torch, stream, target_ms=1.0):
    """Argument of torch.cuda._sleep for a GPU spin of about target_ms on
    this device (the spin counts clock ticks whose rate is measured here)."""
    probe = 1_000_000
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    torch.cuda._sleep(probe)
    b.record(stream)
    torch.cuda.synchronize()
    ms = max(a.elapsed_time(b), 1e-3)
    return int(min(max(probe * target_ms / ms, 1e4), 2e9))


def time_interleaved(torch, stream, cases, iters, context=None):
    """Time every case with HIP events on `stream`: one warm-up call each,
    then `iters` rounds that run every case once, in forward order in even
    rounds and reverse order in odd ones, so that no case always follows the
    same neighbour.  Each round starts with a GPU spin of about 1 ms: the
    rounds are separated by a device synchronisation, and without the spin
    the round's first case would start on an idle GPU and count the host's
    work for its call (marshalling 2N tensor addresses: about 190 us at
    N = 256) as GPU time, while every later case's host work overlaps the
    case before it.  A case that raises is reported, not fatal.  `context`
    maps a case name to (coll, nranks, payload bytes) for the nccl-tests
    style figures of collective_context."""
    spin = pacer_cycles(torch, stream)
    res, live = {}, []
    for name, fn, nbytes in cases:
        try:
            fn()
            torch.cuda.synchronize()
            live.append((name, fn, nbytes))
        except Exception as e:  # a schedule this device cannot run
            res[name] = {"error": str(e)}
            log(f"{name}: {e}")
    ms = {name: [] for name, _, _ in live}
    for rnd in range(iters):
        order = live if rnd % 2 == 0 else live[::-1]
        ev = []
        torch.cuda._sleep(spin)
        for name, fn, _ in order:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            ev.append((name, a, b))
        torch.cuda.synchronize()
        for name, a, b in ev:
            ms[name].append(a.elapsed_time(b))
    for name, _, nbytes in live:
        st = stats(ms[name])
        gbs = nbytes / (st["median_ms"] / 1e3) / 1e9
        res[name] = {"bytes": nbytes, "gbs": gbs, "frac_of_peak": gbs / PEAK_HBM_GBS, **st}
        if context and name in context:
            res[name]["collective"] = collective_context(*context[name], st["median_ms"] / 1e3)
        log(f"{name}: {st['median_ms']:.3f} ms, {gbs:.0f} GB/s (cv {100 * st['cv']:.1f} %)")
    return res


RING_AND_RECURSIVE = ("ring_stepwise", "ring_persistent", "ring_chained", "recursive", "recursive_chained")


def run_secondary(cs, torch, stream, send, shards, recv, n, m, q, dtype, iters):
    """Other schedules and collectives on the same buffers (every schedule's
    RS+AG and AllReduce, RS alone, smaller M on prefixes, a plain copy for
    scale), timed together by time_interleaved."""
    ws = cs.Workspace.largest([(c, n, m, dtype, s) for c in ("reduce_scatter", "all_gather", "allreduce")
                               for s in RING_AND_RECURSIVE])
    ab = cs.ccl_sim_algorithmic_bytes
    cases = []
    for sched in RING_AND_RECURSIVE:
        cases.append((f"rs_ag_{sched}", lambda s=sched: (
            cs.ccl_sim_reduce_scatter(send, shards, m, q, schedule=s, workspace=ws, stream=stream),
            cs.ccl_sim_all_gather(shards, recv, q, m, schedule=s, workspace=ws, stream=stream)),
            ab("reduce_scatter", n, m, dtype, sched) + ab("all_gather", n, m, dtype, sched)))
    # the direct pair again, interleaved with the direct AllReduce for the latency ratio below
    cases.append(("rs_ag_direct", lambda: (
        cs.ccl_sim_reduce_scatter(send, shards, m, q, schedule="direct", stream=stream),
        cs.ccl_sim_all_gather(shards, recv, q, m, schedule="direct", stream=stream)),
        ab("reduce_scatter", n, m, dtype, "direct") + ab("all_gather", n, m, dtype, "direct")))
    for sched in ("direct",) + RING_AND_RECURSIVE:
        cases.append((f"allreduce_{sched}", lambda s=sched: cs.ccl_sim_allreduce(
            send, recv, m, schedule=s, workspace=ws, stream=stream), ab("allreduce", n, m, dtype, sched)))
    cases.append(("rs_only_direct", lambda: cs.ccl_sim_reduce_scatter(send, shards, m, q, stream=stream),
                  ab("reduce_scatter", n, m, dtype, "direct")))
    # smaller M on prefixes of the same buffers (N=8, M = 2^24 and 2^26)
    for lg in (24, 26):
        mm = 1 << lg
        if mm >= m or mm % n:
            continue
        qq = mm // n
        sv = [t[:mm] for t in send]
        rv = [t[:mm] for t in recv]
        hv = [t[:qq] for t in shards]
        for sched in ("direct",) + RING_AND_RECURSIVE:
            if sched.startswith("recursive") and n & (n - 1):
                continue
            cases.append((f"rs_ag_{sched}_m2^{lg}", lambda s=sched, sv=sv, rv=rv, hv=hv, mm=mm, qq=qq: (
                cs.ccl_sim_reduce_scatter(sv, hv, mm, qq, schedule=s, workspace=ws, stream=stream),
                cs.ccl_sim_all_gather(hv, rv, qq, mm, schedule=s, workspace=ws, stream=stream)),
                ab("reduce_scatter", n, mm, dtype, sched) + ab("all_gather", n, mm, dtype, sched)))
    # plain copy of the same size as one rank's buffer, for scale
    cases.append(("copy_one_rank_torch", lambda: recv[0].copy_(send[0]), 2 * m * send[0].element_size()))
    es = send[0].element_size()
    context = {}
    for name, _, _ in cases:
        if name.startswith("rs_ag_") or name.startswith("allreduce_"):
            mm = (1 << int(name.rsplit("m2^", 1)[1])) if "_m2^" in name else m
            context[name] = (cs, "all_reduce", n, mm * es)
        elif name == "rs_only_direct":
            context[name] = (cs, "reduce_scatter", n, m * es)
    res = time_interleaved(torch, stream, cases, iters, context)
    res["ratio_rs_ag_over_allreduce_direct"] = latency_ratio(res, "rs_ag_direct", "allreduce_direct", (n + 1) / n)
    return res


def latency_ratio(res, num, den, bytes_ratio):
    """Median latency of `num` over that of `den`, timed interleaved, with
    the ratio of their algorithmic bytes beside it.  Only stated when both
    CVs are at most 5 %; otherwise the ratio is null and the CVs say why."""
    a, b = res.get(num, {}), res.get(den, {})
    if "median_ms" not in a or "median_ms" not in b:
        return None
    ok = a["cv"] <= 0.05 and b["cv"] <= 0.05
    return {"of": f"{num} / {den}", "ratio": a["median_ms"] / b["median_ms"] if ok else None,
            "cv": [a["cv"], b["cv"]], "bytes_ratio": bytes_ratio}


def run_more_workloads(cs, torch, stream, iters):
    """On freshly drawn device buffers, timed together per workload by
    time_interleaved: the 256-rank workloads (M=2^22 float32 and the
    6,553,600-element bf16 bucket, normal(0, 1e-3)) under every schedule's
    AllReduce and the direct RS+AG; and the bench's own shape in bf16 (N=8,
    M=2^28, uniform[-1,1)) under the direct RS+AG and the direct and chained
    AllReduces."""
    res = {}
    ab = cs.ccl_sim_algorithmic_bytes
    for name, n, m, tdt, dtype, scheds in (
            ("256x4194304_fp32", 256, 1 << 22, torch.float32, "float32", ("direct",) + RING_AND_RECURSIVE),
            ("256x6553600_bf16", 256, 6_553_600, torch.bfloat16, "bfloat16", ("direct",) + RING_AND_RECURSIVE),
            ("8x268435456_bf16", 8, 1 << 28, torch.bfloat16, "bfloat16", ("direct", "ring_chained", "recursive_chained"))):
        q = m // n
        if n == 256:
            send = [torch.randn(m, device="cuda").mul_(1e-3).to(tdt) for _ in range(n)]
        else:
            send = [torch.rand(m, device="cuda").mul_(2).sub_(1).to(tdt) for _ in range(n)]
        recv = [torch.empty(m, dtype=tdt, device="cuda") for _ in range(n)]
        shards = [torch.empty(q, dtype=tdt, device="cuda") for _ in range(n)]
        ws = cs.Workspace.largest([(c, n, m, dtype, s) for c in ("reduce_scatter", "allreduce") for s in scheds])
        torch.cuda.synchronize()
        cases = [(f"allreduce_{sched}_{name}", lambda s=sched: cs.ccl_sim_allreduce(
                    send, recv, m, schedule=s, workspace=ws, stream=stream), ab("allreduce", n, m, dtype, sched))
                 for sched in scheds]
        cases.append((f"rs_ag_direct_{name}", lambda: (
            cs.ccl_sim_reduce_scatter(send, shards, m, q, workspace=ws, stream=stream),
            cs.ccl_sim_all_gather(shards, recv, q, m, workspace=ws, stream=stream)),
            ab("reduce_scatter", n, m, dtype, "direct") + ab("all_gather", n, m, dtype, "direct")))
        context = {c[0]: (cs, "all_reduce", n, m * send[0].element_size()) for c in cases}
        res.update(time_interleaved(torch, stream, cases, iters, context))
        del send, recv, shards, ws, cases
        torch.cuda.empty_cache()
    return res


def run_small(cs, torch, stream, calls=100):
    """The cache-resident workload (N=8, M=2^20 uniform float32: 32 MiB of
    inputs, which the 256 MB Infinity Cache holds) and the launch floor.
    Each figure is the mean over `calls` back-to-back calls between two
    events, after one warm-up, so the per-call time includes the launch
    cost: RS+AG with the direct, stepwise-ring and chained-ring schedules,
    and a 64-element direct AllReduce, which moves almost nothing and so
    measures what one call costs in launch alone; the direct RS+AG and the
    64-element AllReduce again through Plans, which marshal their arguments
    once; then the direct and stepwise-ring RS+AG once more, captured into a
    HIP graph and replayed, which leaves out the host's per-call work."""
    from collective_reduction_amd import inputs as I
    s = I.spec("uniform_8x1048576_fp32")
    n, m = s["nranks"], s["count"]
    q = m // n
    send = [torch.from_numpy(I.rank_buffer(s, r)).to("cuda") for r in range(n)]
    shards = [torch.empty(q, device="cuda") for _ in range(n)]
    recv = [torch.empty(m, device="cuda") for _ in range(n)]
    ab = cs.ccl_sim_algorithmic_bytes
    ws = cs.Workspace.largest([(c, n, m, "float32", sc) for c in ("reduce_scatter", "all_gather")
                               for sc in ("ring_stepwise", "ring_chained")])
    res = {}

    def timed(name, fn, nbytes):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(calls):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        per_ms = a.elapsed_time(b) / calls
        res[name] = {"bytes": nbytes, "calls": calls, "mean_ms": per_ms, "us_per_call": per_ms * 1e3,
                     "gbs": nbytes / (per_ms / 1e3) / 1e9 if nbytes else None}
        log(f"{name}: {per_ms * 1e3:.1f} us per call" + (f", {res[name]['gbs']:.0f} GB/s" if nbytes else ""))

    for sched in ("direct", "ring_stepwise", "ring_chained"):
        timed(f"rs_ag_{sched}_8x1048576_fp32_cache_resident", lambda sc=sched: (
            cs.ccl_sim_reduce_scatter(send, shards, m, q, schedule=sc, workspace=ws, stream=stream),
            cs.ccl_sim_all_gather(shards, recv, q, m, schedule=sc, workspace=ws, stream=stream)),
            ab("reduce_scatter", n, m, "float32", sched) + ab("all_gather", n, m, "float32", sched))
    tiny_in, tiny_out = [t[:64] for t in send], [t[:64] for t in recv]
    timed("launch_floor_allreduce_direct_8x64", lambda: cs.ccl_sim_allreduce(tiny_in, tiny_out, 64, stream=stream), 0)
    # the same calls through Plans, which marshal their arguments once
    rs_plan = cs.Plan("reduce_scatter", send, shards, m, q)
    ag_plan = cs.Plan("all_gather", shards, recv, q, m)
    timed("rs_ag_direct_8x1048576_fp32_cache_resident_plan", lambda: (rs_plan.run(stream), ag_plan.run(stream)),
          ab("reduce_scatter", n, m, "float32", "direct") + ab("all_gather", n, m, "float32", "direct"))
    tiny_plan = cs.Plan("allreduce", tiny_in, tiny_out, 64)
    timed("launch_floor_allreduce_direct_8x64_plan", lambda: tiny_plan.run(stream), 0)
    del rs_plan, ag_plan, tiny_plan
    # the same RS+AG steps captured once into a HIP graph and replayed: no
    # per-call host work, so what remains is the GPU's own time
    for sched in ("direct", "ring_stepwise"):
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            cs.ccl_sim_reduce_scatter(send, shards, m, q, schedule=sched, workspace=ws)
            cs.ccl_sim_all_gather(shards, recv, q, m, schedule=sched, workspace=ws)
        torch.cuda.synchronize()
        timed(f"rs_ag_{sched}_8x1048576_fp32_cache_resident_graph", graph.replay,
              ab("reduce_scatter", n, m, "float32", sched) + ab("all_gather", n, m, "float32", sched))
        del graph
    del send, shards, recv, ws
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
