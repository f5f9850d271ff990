"""Buffer-lifetime accounting for AllReduce versus ReduceScatter + AllGather.

[DECOMP] §显存实验必须区分 steady 与 peak compares four buffer lifetimes for
one rank holding a payload of P bytes in a world of N ranks:

* ``allreduce_full``: one full buffer, reduced in place.  Steady P, peak P.
* ``reduce_scatter_only``: the full input and a P/N shard live during the
  ReduceScatter; the input is freed afterwards.  Steady P/N, peak P + P/N.
  (This is the sharded-optimizer state path.)
* ``rs_ag_naive``: input, shard and gathered output all allocated before the
  two collectives and freed at the end.  Steady P, peak 2P + P/N.
* ``rs_ag_optimized``: the input is freed after the ReduceScatter and the
  gathered output is allocated only then.  Steady P, peak P + P/N.

``model`` states those byte counts.  ``measure`` runs the same four
schedules on the GPU through the library's collectives, with every rank
buffer a torch allocation, and reads torch's allocator statistics.  Memory
is reported per rank: the N virtual ranks share one GPU, so the measured
totals are divided by N.  The ring schedules also hold the caller's
workspace, which the report includes.
"""

MODES = ("allreduce_full", "reduce_scatter_only", "rs_ag_naive", "rs_ag_optimized")


def model(payload_bytes, nranks):
    """Steady and peak bytes per rank for each lifetime ([DECOMP], four
    lifetimes); the shard is payload / nranks."""
    p = payload_bytes
    s = payload_bytes // nranks
    return {
        "allreduce_full": {"steady": p, "peak": p},
        "reduce_scatter_only": {"steady": s, "peak": p + s},
        "rs_ag_naive": {"steady": p, "peak": 2 * p + s},
        "rs_ag_optimized": {"steady": p, "peak": p + s},
    }


def measure(mode, nranks, count, dtype="float32", schedule="direct", device="cuda"):
    """Run one lifetime over N virtual ranks of `count` elements and return
    steady and peak allocated bytes per rank (allocator deltas from a clean
    start), plus the workspace bytes per rank that the schedule needed."""
    import torch

    from . import ccl_sim as cs

    tdt = {"float32": torch.float32, "bfloat16": torch.bfloat16, "int32": torch.int32, "int64": torch.int64}[dtype]
    n, m = nranks, count
    q = m // n
    if n * q != m:
        raise ValueError("count must divide into nranks shards")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated(device)
    torch.cuda.reset_peak_memory_stats(device)

    def alloc(k):
        return [torch.empty(k, dtype=tdt, device=device) for _ in range(n)]

    ws = None
    if mode == "allreduce_full":
        full = alloc(m)
        ws = cs.Workspace("allreduce", n, m, dtype, schedule, device=device)
        cs.ccl_sim_allreduce(full, full, m, schedule=schedule, workspace=ws)
        torch.cuda.synchronize()
        keep = [full]
    elif mode == "reduce_scatter_only":
        full = alloc(m)
        shard = alloc(q)
        ws = cs.Workspace("reduce_scatter", n, m, dtype, schedule, device=device)
        cs.ccl_sim_reduce_scatter(full, shard, m, q, schedule=schedule, workspace=ws)
        torch.cuda.synchronize()
        del full
        keep = [shard]
    elif mode == "rs_ag_naive":
        full = alloc(m)
        shard = alloc(q)
        gathered = alloc(m)
        ws = cs.Workspace.largest([("reduce_scatter", n, m, dtype, schedule), ("all_gather", n, m, dtype, schedule)],
                                  device=device)
        cs.ccl_sim_reduce_scatter(full, shard, m, q, schedule=schedule, workspace=ws)
        cs.ccl_sim_all_gather(shard, gathered, q, m, schedule=schedule, workspace=ws)
        torch.cuda.synchronize()
        del full, shard
        keep = [gathered]
    elif mode == "rs_ag_optimized":
        full = alloc(m)
        shard = alloc(q)
        ws = cs.Workspace.largest([("reduce_scatter", n, m, dtype, schedule), ("all_gather", n, m, dtype, schedule)],
                                  device=device)
        cs.ccl_sim_reduce_scatter(full, shard, m, q, schedule=schedule, workspace=ws)
        torch.cuda.synchronize()
        del full
        gathered = alloc(m)
        cs.ccl_sim_all_gather(shard, gathered, q, m, schedule=schedule, workspace=ws)
        torch.cuda.synchronize()
        del shard
        keep = [gathered]
    else:
        raise ValueError(f"unknown lifetime {mode!r}")
    ws_bytes = ws.nbytes if ws is not None else 0
    del ws
    torch.cuda.synchronize()
    steady = torch.cuda.memory_allocated(device) - base
    peak = torch.cuda.max_memory_allocated(device) - base
    del keep
    torch.cuda.empty_cache()
    return {"steady": steady / n, "peak": peak / n, "workspace": ws_bytes / n}
