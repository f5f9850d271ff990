"""ccl_sim_allreduce_noalloc (the library's own scratch, no workspace) against
ccl_sim_allreduce with a caller-owned workspace, bit for bit, through the C
ABI: two calls in a row on the same scratch, the second smaller than the
first, for every schedule the entry point offers, with and without pointer
tables, in float32, bf16 and int32; and the call captured into a HIP graph
and replayed, with other calls reusing the scratch between replays."""

import numpy as np
import pytest
import torch

import gpu_util as U

pytestmark = pytest.mark.gpu

BITS = {"float32": torch.int32, "bfloat16": torch.int16, "int32": torch.int32}


@pytest.fixture(scope="module")
def cs():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from collective_reduction_amd import ccl_sim
    return ccl_sim


def _pair(cs, n, m, dtype, op, schedule, seed):
    """The same AllReduce through both entry points; returns the two sets of
    outputs (device tensors)."""
    xs = U.random_inputs(n, m, dtype, seed=seed, op=op)
    send = U.bufs_from(xs, dtype)
    want = [U.empty(m, dtype) for _ in range(n)]
    got = [U.empty(m, dtype) for _ in range(n)]
    ws = cs.Workspace("allreduce", n, m, dtype, schedule)
    cs.ccl_sim_allreduce(send, want, m, op=op, schedule=schedule, workspace=ws, dtype=dtype)
    cs.ccl_sim_allreduce_noalloc(send, got, m, op=op, schedule=schedule, dtype=dtype)
    torch.cuda.synchronize()
    return got, want


def _same(got, want, dtype, what):
    for r, (g, w) in enumerate(zip(got, want)):
        assert torch.equal(g.view(BITS[dtype]), w.view(BITS[dtype])), f"{what}: rank {r}"


SHAPES = {  # (first call, second and smaller call)
    "direct": [(8, 3001 * 8 + 5), (8, 1000)],
    "ring_stepwise": [(8, 3001 * 8 + 5), (5, 1003)],
    "ring_chained": [(8, 3001 * 8 + 5), (5, 1003)],
    "recursive": [(8, 3001 * 8 + 5), (4, 1003)],
    "recursive_chained": [(8, 3001 * 8 + 5), (4, 1003)],
}
MANY = {  # more than 64 ranks: the pointer tables live in the scratch too
    "direct": [(100, 3689), (65, 7)],
    "ring_stepwise": [(100, 3689), (65, 7)],
    "ring_chained": [(100, 3689), (65, 7)],
    "recursive": [(128, 3689), (128, 7)],
    "recursive_chained": [(128, 3689), (128, 7)],
}


@pytest.mark.parametrize("dtype,op", [("float32", "sum"), ("bfloat16", "sum"), ("int32", "max")])
@pytest.mark.parametrize("schedule", list(SHAPES))
def test_noalloc_matches_the_workspace_entry_point(cs, schedule, dtype, op):
    for k, (n, m) in enumerate(SHAPES[schedule]):
        print(f"[noalloc] {schedule} {dtype} {op} n={n} m={m}", flush=True)
        got, want = _pair(cs, n, m, dtype, op, schedule, seed=100 + k)
        _same(got, want, dtype, f"{schedule} call {k + 1} n={n} m={m}")


@pytest.mark.parametrize("schedule", list(MANY))
def test_noalloc_with_pointer_tables(cs, schedule):
    for k, (n, m) in enumerate(MANY[schedule]):
        print(f"[noalloc] {schedule} float32 n={n} m={m}", flush=True)
        got, want = _pair(cs, n, m, "float32", "sum", schedule, seed=200 + k)
        _same(got, want, "float32", f"{schedule} call {k + 1} n={n} m={m}")


def test_noalloc_at_the_scratch_limit_then_small(cs):
    """The largest float32 ring AllReduce whose partials fill the scratch
    (N = 8, M = 2^23), then a small one on the same scratch."""
    n = 8
    m = cs.NOALLOC_SCRATCH_BYTES // 8
    assert cs.ccl_sim_workspace_size("allreduce", n, m, "float32", "ring_stepwise") <= cs.NOALLOC_SCRATCH_BYTES
    for k, (nn, mm) in enumerate([(n, m), (3, 17)]):
        print(f"[noalloc] ring_stepwise float32 n={nn} m={mm}", flush=True)
        got, want = _pair(cs, nn, mm, "float32", "sum", "ring_stepwise", seed=300 + k)
        _same(got, want, "float32", f"limit call {k + 1}")
        del got, want
        torch.cuda.empty_cache()


def test_noalloc_refusals_enqueue_nothing(cs):
    """Refused calls leave the outputs untouched."""
    n, m = 8, 4096
    send = U.bufs_from(U.random_inputs(n, m, "float32", seed=7), "float32")
    out = [torch.full((m,), 3.0, device="cuda") for _ in range(n)]
    with pytest.raises(cs.CclSimError, match="persistent"):
        cs.ccl_sim_allreduce_noalloc(send, out, m, schedule="ring_persistent")
    torch.cuda.synchronize()
    assert all(bool((o == 3.0).all()) for o in out)
    got = np.stack([U.to_host(o, "float32") for o in out])
    assert np.all(got == 3.0)


@pytest.mark.parametrize("schedule", ["direct", "ring_stepwise", "ring_chained", "recursive", "recursive_chained"])
@pytest.mark.parametrize("n,m", [(8, 3 * 8 * 1024 + 5), (128, 128 * 37 - 11)])
def test_noalloc_graph_replays_match_eager(cs, schedule, n, m):
    """The call allocates nothing, so it can be captured once its first call
    on the device has read the scratch's address.  Between replays, eager
    noalloc calls of another shape reuse the same scratch; every replay must
    still equal an eager call with a caller-owned workspace, bit for bit."""
    send = [torch.empty(m, device="cuda") for _ in range(n)]
    recv = [torch.empty(m, device="cuda") for _ in range(n)]
    want = [torch.empty(m, device="cuda") for _ in range(n)]
    other_in = [torch.rand(m // 2 + 1, device="cuda") for _ in range(n)]
    other_out = [torch.empty(m // 2 + 1, device="cuda") for _ in range(n)]
    ws = cs.Workspace("allreduce", n, m, "float32", schedule)
    gen = torch.Generator(device="cuda").manual_seed(n + m)

    def refill():
        for t in send:
            t.uniform_(-1, 1, generator=gen)

    refill()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        cs.ccl_sim_allreduce_noalloc(send, recv, m, schedule=schedule)  # first call outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        cs.ccl_sim_allreduce_noalloc(send, recv, m, schedule=schedule)
    torch.cuda.synchronize()
    for replay in range(4):
        refill()
        for t in recv:
            t.fill_(float("nan"))
        cs.ccl_sim_allreduce_noalloc(other_in, other_out, m // 2 + 1, schedule=schedule)  # the scratch reused
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        cs.ccl_sim_allreduce(send, want, m, schedule=schedule, workspace=ws)
        torch.cuda.synchronize()
        for r in range(n):
            assert torch.equal(recv[r].view(torch.int32), want[r].view(torch.int32)), (schedule, replay, r)
