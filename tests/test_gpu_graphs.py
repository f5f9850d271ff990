"""HIP graph capture of the library's calls.

Every launch the library enqueues is a kernel (the control block and the
pointer tables are written by small kernels, never by a memset or a host
copy), so a call can be captured into a HIP graph and replayed.  Each test
captures one call, then replays the graph several times with new inputs
written by eager work between the replays, and checks every replay bit for
bit against an eager call of the same collective on the same inputs."""

import pytest
import torch

import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cs():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from collective_reduction_amd import ccl_sim
    return ccl_sim


@pytest.mark.parametrize("schedule", U.SCHEDULES)
@pytest.mark.parametrize("n,m", [(8, 3 * 8 * 1024 + 5), (100, 100 * 37 - 11)])
def test_allreduce_graph_replays_match_eager(cs, schedule, n, m):
    if U.is_recursive(schedule) and not U.pow2(n):
        pytest.skip("recursive halving needs a power-of-two N")
    if schedule == "ring_persistent":
        pytest.skip("the persistent ring is a cooperative launch, which HIP does not document as capturable")
    send = [torch.empty(m, device="cuda") for _ in range(n)]
    recv = [torch.empty(m, device="cuda") for _ in range(n)]
    want = [torch.empty(m, device="cuda") for _ in range(n)]
    ws = cs.Workspace("allreduce", n, m, "float32", schedule)
    gen = torch.Generator(device="cuda").manual_seed(n + m)

    def refill():
        for t in send:
            t.uniform_(-1, 1, generator=gen)

    refill()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        cs.ccl_sim_allreduce(send, recv, m, schedule=schedule, workspace=ws)  # warm-up outside capture
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        cs.ccl_sim_allreduce(send, recv, m, schedule=schedule, workspace=ws)
    torch.cuda.synchronize()
    for replay in range(4):
        refill()
        for t in recv:
            t.fill_(float("nan"))  # eager work between replays, and proof the replay rewrites every element
        graph.replay()
        torch.cuda.synchronize()
        cs.ccl_sim_allreduce(send, want, m, schedule=schedule, workspace=ws)
        torch.cuda.synchronize()
        for r in range(n):
            assert torch.equal(recv[r].view(torch.int32), want[r].view(torch.int32)), (schedule, replay, r)
