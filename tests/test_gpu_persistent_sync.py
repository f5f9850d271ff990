"""The persistent ring's two step orderings, forced from the host.

CCL_SIM_PERSISTENT_SYNC=grid puts a grid barrier between steps;
CCL_SIM_PERSISTENT_SYNC=flags lets each workgroup wait only for the
workgroups that hold the upstream tiles of its own, with the partials keyed
by chunk.  By default the library picks by step size, so each form runs
here on shapes where it would not be chosen too.  Both must give the
stepwise ring's result bit for bit (the same transfers and the same
combining order), and the oracle's ring fold where the oracle is cheap:
every collective, in-place forms, ragged chunks, 2 to 256 ranks, steps of
either launch shape.
"""

import os

import numpy as np
import pytest
import torch

import gpu_util as U
from oracle import collectives as C
from oracle import ring as G
from oracle import reduction as R

pytestmark = pytest.mark.gpu

SYNCS = ("grid", "flags")
BITS = {"float32": torch.int32, "bfloat16": torch.int16, "int32": torch.int32, "int64": torch.int64}


@pytest.fixture(scope="module")
def cs():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from collective_reduction_amd import ccl_sim
    return ccl_sim


@pytest.fixture(params=SYNCS)
def sync(request):
    saved = os.environ.get("CCL_SIM_PERSISTENT_SYNC")
    os.environ["CCL_SIM_PERSISTENT_SYNC"] = request.param
    yield request.param
    if saved is None:
        os.environ.pop("CCL_SIM_PERSISTENT_SYNC", None)
    else:
        os.environ["CCL_SIM_PERSISTENT_SYNC"] = saved


def dev_equal(a, b, dtype):
    return torch.equal(a.view(BITS[dtype]), b.view(BITS[dtype]))


def run_pair(cs, coll, xs, dtype, op, in_place, q=None, recvcount=None):
    """One call under the persistent ring and one under the stepwise ring
    on the same device inputs; returns both ranks' outputs (device)."""
    n = len(xs)
    outs = {}
    for schedule in ("ring_persistent", "ring_stepwise"):
        if coll == "allreduce":
            m = len(xs[0])
            send = U.bufs_from(xs, dtype)
            recv = send if in_place else [U.empty(m, dtype) for _ in range(n)]
            ws = cs.Workspace("allreduce", n, m, dtype, schedule)
            cs.ccl_sim_allreduce(send, recv, m, op=op, schedule=schedule, workspace=ws, dtype=dtype)
        elif coll == "reduce_scatter":
            send = U.bufs_from(xs, dtype)
            recv = [send[r][r * q:(r + 1) * q] for r in range(n)] if in_place else [U.empty(q, dtype) for _ in range(n)]
            ws = cs.Workspace("reduce_scatter", n, n * q, dtype, schedule)
            cs.ccl_sim_reduce_scatter(send, recv, n * q, q, op=op, schedule=schedule, workspace=ws, dtype=dtype)
        else:
            shard = len(xs[0])
            if in_place:
                full = [U.empty(n * shard, dtype) for _ in range(n)]
                send = []
                for r in range(n):
                    v = full[r][r * shard:(r + 1) * shard]
                    v.copy_(U.to_dev(xs[r], dtype))
                    send.append(v)
                recv = [b[:recvcount] for b in full]
            else:
                send = U.bufs_from(xs, dtype)
                recv = [U.empty(recvcount, dtype) for _ in range(n)]
            ws = cs.Workspace("all_gather", n, recvcount, dtype, schedule)
            cs.ccl_sim_all_gather(send, recv, shard, recvcount, schedule=schedule, workspace=ws, dtype=dtype)
        torch.cuda.synchronize()
        if schedule == "ring_persistent":
            assert cs.ccl_sim_persistent_aborted(ws) is False
        outs[schedule] = recv
    return outs["ring_persistent"], outs["ring_stepwise"]


CASES = [
    # n, q, dtype, op: short and ragged chunks, every accumulator width
    (2, 1001, "float32", "sum"),
    (3, 5003, "float32", "max"),
    (5, 16384 + 7, "bfloat16", "sum"),
    (8, 4096, "int32", "sum"),
    (8, 3 * 16384 + 5, "int64", "prod"),
    (16, 777, "float32", "avg"),
    (64, 1000, "bfloat16", "min"),
    (100, 31, "int32", "max"),
    (256, 311, "float32", "sum"),
    # line-aligned chunks, where the flag form reads data written by a
    # workgroup on its own XCD from that XCD's L2: one tile per chunk with
    # the ring's neighbours placed on one XCD (N = 256, 64, 16), and eight
    # tiles per chunk, where a tile and its upstream share an XCD anyway
    (256, 1024, "float32", "sum"),
    (64, 4096, "bfloat16", "max"),
    (16, 3 * 16384, "float32", "sum"),
    (8, 8 * 16384, "int32", "sum"),
]


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("n,q,dtype,op", CASES)
def test_allreduce_matches_stepwise_and_oracle(cs, sync, n, q, dtype, op, in_place):
    m = n * q - 3
    xs = U.random_inputs(n, m, dtype, seed=n * 7 + q, op=op)
    got, want = run_pair(cs, "allreduce", xs, dtype, op, in_place)
    for r in range(n):
        assert dev_equal(got[r], want[r], dtype), f"{sync}: rank {r}"
    assert U.same_bits(U.to_host(got[n - 1], dtype), G.ring_allreduce(xs, op, dtype)[0])


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("n,q,dtype,op", CASES)
def test_reduce_scatter_matches_stepwise_and_oracle(cs, sync, n, q, dtype, op, in_place):
    xs = U.random_inputs(n, n * q, dtype, seed=n * 11 + q, op=op)
    got, want = run_pair(cs, "reduce_scatter", xs, dtype, op, in_place, q=q)
    oracle = G.ring_reduce_scatter(xs, op, dtype, q)
    for r in range(n):
        assert dev_equal(got[r], want[r], dtype), f"{sync}: rank {r}"
        assert U.same_bits(U.to_host(got[r], dtype), oracle[r]), f"{sync}: rank {r} against the oracle"


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("n,q,dtype", [(2, 999, "float32"), (3, 5003, "int64"), (8, 16384 + 9, "bfloat16"),
                                       (64, 1000, "int32"), (256, 257, "float32"), (256, 1024, "float32"),
                                       (64, 8192, "bfloat16")])
def test_all_gather_matches_stepwise_and_oracle(cs, sync, n, q, dtype, in_place):
    shards = U.random_inputs(n, q, dtype, seed=n * 13 + q)
    recvcount = n * q - 5
    got, want = run_pair(cs, "all_gather", shards, dtype, "sum", in_place, recvcount=recvcount)
    cat = G.ring_all_gather(shards, recvcount)
    for r in range(n):
        assert dev_equal(got[r], want[r], dtype), f"{sync}: rank {r}"
    assert U.same_bits(U.to_host(got[0], dtype), cat[0])


@pytest.mark.parametrize("n,q,dtype", [(64, 1000, "float32"), (256, 311, "bfloat16"), (256, 16384, "float32"),
                                       (8, 3 * 16384 + 5, "int32"), (64, 25600, "bfloat16")])
def test_repeats_on_the_same_buffers(cs, sync, n, q, dtype):
    """New data on the same workspace and outputs, six calls in a row: the
    flags and counters of one call must not leak into the next."""
    m = n * q - 3
    ws = cs.Workspace.largest([("allreduce", n, m, dtype, s) for s in ("ring_stepwise", "ring_persistent")])
    got = [U.empty(m, dtype) for _ in range(n)]
    want = [U.empty(m, dtype) for _ in range(n)]
    for rep in range(6):
        xs = U.random_inputs(n, m, dtype, seed=700 + rep)
        send = U.bufs_from(xs, dtype)
        cs.ccl_sim_allreduce(send, got, m, schedule="ring_persistent", workspace=ws, dtype=dtype)
        torch.cuda.synchronize()
        assert cs.ccl_sim_persistent_aborted(ws) is False
        cs.ccl_sim_allreduce(send, want, m, schedule="ring_stepwise", workspace=ws, dtype=dtype)
        torch.cuda.synchronize()
        for r in range(n):
            assert dev_equal(got[r], want[r], dtype), f"{sync}: repeat {rep}, rank {r}"


def test_large_steps_every_element(cs, sync):
    """N = 8, M = 2^26 + 12345 float32: steps above 2^26 elements, the
    256-lane launch shape, where the library would pick the grid barrier on
    the fenced path.  Forced flags run it on the agent-coherent path.
    AllReduce and RS + AG, every element against the oracle's ring fold."""
    n, m = 8, (1 << 26) + 12345
    q = -(-m // n)
    xs = U.random_inputs(n, n * q, "float32", seed=41)
    send = [U.to_dev(x, "float32") for x in xs]
    ws = cs.Workspace.largest([("allreduce", n, m, "float32", "ring_persistent"),
                               ("reduce_scatter", n, n * q, "float32", "ring_persistent")])
    ar = [torch.empty(m, dtype=torch.float32, device="cuda") for _ in range(n)]
    cs.ccl_sim_allreduce([x[:m] for x in send], ar, m, schedule="ring_persistent", workspace=ws)
    torch.cuda.synchronize()
    assert cs.ccl_sim_persistent_aborted(ws) is False
    shards = [torch.empty(q, dtype=torch.float32, device="cuda") for _ in range(n)]
    cs.ccl_sim_reduce_scatter(send, shards, n * q, q, schedule="ring_persistent", workspace=ws)
    gathered = [torch.empty(m, dtype=torch.float32, device="cuda") for _ in range(n)]
    cs.ccl_sim_all_gather(shards, gathered, q, m, schedule="ring_persistent", workspace=ws)
    torch.cuda.synchronize()
    assert cs.ccl_sim_persistent_aborted(ws) is False
    del send
    for c in range(n):
        cols = [x[c * q:(c + 1) * q] for x in xs]
        want = R.narrow(C.fold(cols, "sum", "float32", G.chunk_order(n, c)), "float32")
        assert U.same_bits(U.to_host(shards[c], "float32"), want), f"{sync}: shard {c}"
        hi = min((c + 1) * q, m)
        want_dev = torch.from_numpy(np.ascontiguousarray(want[:hi - c * q])).cuda().view(torch.int32)
        for r in range(n):
            assert torch.equal(ar[r][c * q:hi].view(torch.int32), want_dev), f"{sync}: allreduce rank {r}, chunk {c}"
            assert torch.equal(gathered[r][c * q:hi].view(torch.int32), want_dev), f"{sync}: gathered rank {r}, chunk {c}"
    del ar, shards, gathered
    torch.cuda.empty_cache()


LARGE_ALIGNED = [
    # n, q, dtype, op.  256-lane tiles (4,096 float32 or 8,192 bf16 elements)
    # at steps above 2^26 elements, 64 to 82 tiles per workgroup of the
    # 256-workgroup grid, whose upstream tiles sit on two other workgroups.
    (8, 4096 * 2100, "float32", "sum"),
    (3, 4096 * 7000, "float32", "max"),
    (8, 8192 * 2100, "bfloat16", "sum"),
]


@pytest.mark.parametrize("n,q,dtype,op", LARGE_ALIGNED)
def test_large_line_aligned_steps_match_stepwise(cs, n, q, dtype, op):
    """Forced step flags on large line-aligned steps, where each workgroup
    holds many tiles per step and reads same-XCD data from the L2:
    AllReduce and ReduceScatter, every element of every rank against the
    stepwise ring."""
    saved = os.environ.get("CCL_SIM_PERSISTENT_SYNC")
    os.environ["CCL_SIM_PERSISTENT_SYNC"] = "flags"
    try:
        xs = U.random_inputs(n, n * q, dtype, seed=n * 7 + len(dtype), op=op)
        for coll in ("allreduce", "reduce_scatter"):
            got, want = run_pair(cs, coll, xs, dtype, op, False, q=q)
            for r in range(n):
                assert dev_equal(got[r], want[r], dtype), f"{coll} n={n} q={q} {dtype} rank {r}"
            del got, want
            torch.cuda.empty_cache()
    finally:
        if saved is None:
            os.environ.pop("CCL_SIM_PERSISTENT_SYNC", None)
        else:
            os.environ["CCL_SIM_PERSISTENT_SYNC"] = saved


def test_debug_plan_names_the_same_xcd_reads(cs, capfd):
    """The launch plan that CCL_SIM_DEBUG=1 prints names the step ordering
    that ccl_sim_persistent_ordering predicts, and says whether a
    flag-ordered call reads same-XCD data from the L2: on when every chunk
    and rank buffer is made of whole 128-byte lines, off when a chunk ends
    inside a line (and always off under the grid barrier)."""
    saved = {k: os.environ.get(k) for k in ("CCL_SIM_DEBUG", "CCL_SIM_PERSISTENT_SYNC")}
    os.environ["CCL_SIM_DEBUG"] = "1"
    os.environ.pop("CCL_SIM_PERSISTENT_SYNC", None)
    try:
        n = 8
        # separate torch allocations start on 512-byte boundaries, so the
        # rank buffers are line-aligned and q alone decides
        # (q, ordering, same-XCD reads); q = 2^24 makes a step of 2^27
        # elements, above the flags' default range
        for q, sync, want in ((1024, "flags", 1), (1001, "flags", 0), (1 << 24, "grid", 0)):
            m = n * q
            assert cs.ccl_sim_persistent_ordering("allreduce", n, m) == sync
            send = [torch.rand(m, device="cuda") for _ in range(n)]
            recv = [torch.empty(m, device="cuda") for _ in range(n)]
            ws = cs.Workspace("allreduce", n, m, "float32", "ring_persistent")
            capfd.readouterr()
            cs.ccl_sim_allreduce(send, recv, m, schedule="ring_persistent", workspace=ws)
            torch.cuda.synchronize()
            lines = [ln for ln in capfd.readouterr().err.splitlines() if ln.startswith("[ccl_sim] persistent")]
            assert lines, "no launch plan printed"
            assert f"sync={sync}" in lines[-1] and f"same_xcd_reads={want}" in lines[-1], lines[-1]
            assert torch.allclose(recv[0], torch.stack(send).sum(0), rtol=0, atol=1e-5 * n)
            del send, recv, ws
        torch.cuda.empty_cache()
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def test_unknown_value_is_refused_before_any_launch(cs):
    saved = os.environ.get("CCL_SIM_PERSISTENT_SYNC")
    os.environ["CCL_SIM_PERSISTENT_SYNC"] = "barrier"
    try:
        n, m = 4, 1000
        send = [torch.ones(m, device="cuda") for _ in range(n)]
        recv = [torch.full((m,), -7.0, device="cuda") for _ in range(n)]
        ws = cs.Workspace("allreduce", n, m, "float32", "ring_persistent")
        with pytest.raises(cs.CclSimError, match="CCL_SIM_PERSISTENT_SYNC"):
            cs.ccl_sim_allreduce(send, recv, m, schedule="ring_persistent", workspace=ws)
        torch.cuda.synchronize()
        assert all(bool((r == -7.0).all()) for r in recv)
        # other schedules do not read the knob
        cs.ccl_sim_allreduce(send, recv, m, schedule="direct")
        torch.cuda.synchronize()
        assert bool((recv[0] == n).all())
    finally:
        if saved is None:
            os.environ.pop("CCL_SIM_PERSISTENT_SYNC", None)
        else:
            os.environ["CCL_SIM_PERSISTENT_SYNC"] = saved


RANDOM_ALIGNED = int(os.environ.get("CCL_SIM_TEST_ALIGNED_CASES", "60"))


def test_random_line_aligned_shapes_match_stepwise(cs):
    """Seeded random calls whose rank buffers and chunks are whole 128-byte
    lines, with the step flags forced, so that the flag form reads
    same-XCD data from the L2 wherever the placement allows: 2 to 256
    ranks, every collective, dtype and op, in place and out of place,
    against the stepwise ring bit for bit (CCL_SIM_TEST_ALIGNED_CASES
    scales the count)."""
    rng = np.random.default_rng(20261203)
    saved = os.environ.get("CCL_SIM_PERSISTENT_SYNC")
    os.environ["CCL_SIM_PERSISTENT_SYNC"] = "flags"
    try:
        for case in range(RANDOM_ALIGNED):
            n = int(rng.choice([2, 3, 4, 8, 12, 16, 24, 32, 64, 100, 128, 256]))
            dtype = str(rng.choice(["float32", "bfloat16", "int32", "int64"]))
            op = str(rng.choice(["sum", "max", "min", "prod", "avg"]))
            line_elems = 128 // {"float32": 4, "bfloat16": 2, "int32": 4, "int64": 8}[dtype]
            line_elems = max(line_elems, 32)  # bf16 accumulates in float32: 32 floats per line
            q = line_elems * int(rng.integers(1, max(2, (1 << 24) // (n * n * line_elems))))  # ~16M elements at most
            coll = str(rng.choice(["allreduce", "reduce_scatter", "all_gather"]))
            in_place = bool(rng.integers(0, 2))
            if coll == "all_gather":
                xs = U.random_inputs(n, q, dtype, seed=case)
                got, want = run_pair(cs, coll, xs, dtype, "sum", in_place, recvcount=n * q)
            elif coll == "reduce_scatter":
                xs = U.random_inputs(n, n * q, dtype, seed=case, op=op)
                got, want = run_pair(cs, coll, xs, dtype, op, in_place, q=q)
            else:
                xs = U.random_inputs(n, n * q, dtype, seed=case, op=op)
                got, want = run_pair(cs, coll, xs, dtype, op, in_place)
            for r in range(n):
                assert dev_equal(got[r], want[r], dtype), f"case {case}: {coll} n={n} q={q} {dtype} {op} " \
                                                            f"in_place={in_place} rank {r}"
        print(f"{RANDOM_ALIGNED} line-aligned random calls matched the stepwise ring", flush=True)
    finally:
        if saved is None:
            os.environ.pop("CCL_SIM_PERSISTENT_SYNC", None)
        else:
            os.environ["CCL_SIM_PERSISTENT_SYNC"] = saved
