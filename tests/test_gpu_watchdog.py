"""The persistent ring's watchdog, seen from the host.

A clean persistent-ring call leaves the abort word clear, and
ccl_sim_persistent_aborted says so.  The failure path is forced from the
host, never by breaking the kernel: CCL_SIM_SPIN_LIMIT=1 (read on every
call) sets the poll limit to one, so the first wait a workgroup reaches
before the data it waits for is ready gives up almost at once: a grid
barrier reached before the rest of the grid, or, in the flag-ordered form
(CCL_SIM_PERSISTENT_SYNC=flags), a step whose upstream workgroup is still
busy.  Every workgroup then stops and the kernel exits normally; the query
must report the abort, CCL_SIM_DEBUG=1 must turn it into an error of the
call itself, and the next calls must run normally.  Everything runs in this
process: ROCm can refuse a cooperative launch from a second process on the
same GPU.
"""

import os

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cs():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from collective_reduction_amd import ccl_sim
    return ccl_sim


@pytest.fixture
def knobs():
    """Set library environment knobs for one test and restore them after."""
    saved = {k: os.environ.get(k) for k in ("CCL_SIM_SPIN_LIMIT", "CCL_SIM_DEBUG", "CCL_SIM_PERSISTENT_SYNC")}
    yield os.environ
    for k, v in saved.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v


def allreduce_case(n, m):
    send = [torch.rand(m, device="cuda") for _ in range(n)]
    recv = [torch.zeros(m, device="cuda") for _ in range(n)]
    return send, recv


@pytest.mark.parametrize("sync", ["grid", "flags"])
@pytest.mark.parametrize("n,m", [(8, 1 << 20), (256, 256 * 1000 + 3)])
def test_clean_persistent_calls_report_no_abort(cs, knobs, sync, n, m):
    knobs["CCL_SIM_PERSISTENT_SYNC"] = sync
    send, recv = allreduce_case(n, m)
    ws = cs.Workspace("allreduce", n, m, "float32", "ring_persistent")
    for _ in range(2):
        cs.ccl_sim_allreduce(send, recv, m, schedule="ring_persistent", workspace=ws)
        torch.cuda.synchronize()
        assert cs.ccl_sim_persistent_aborted(ws) is False
    want = torch.stack(send).sum(0)  # float32 in another order: a tolerance check only
    assert torch.allclose(recv[n - 1], want, rtol=0, atol=1e-5 * n)


def check_recovery(cs, send, ws, n, m):
    """The next persistent call (default poll limit) and a direct call both
    run to the end."""
    out = [torch.zeros(m, device="cuda") for _ in range(n)]
    cs.ccl_sim_allreduce(send, out, m, schedule="ring_persistent", workspace=ws)
    torch.cuda.synchronize()
    assert cs.ccl_sim_persistent_aborted(ws) is False
    direct = [torch.zeros(m, device="cuda") for _ in range(n)]
    cs.ccl_sim_allreduce(send, direct, m)
    torch.cuda.synchronize()
    want = torch.stack(send).sum(0)
    assert torch.allclose(out[0], want, rtol=0, atol=1e-4) and torch.allclose(direct[0], want, rtol=0, atol=1e-4)


# Grid barrier: N = 8, M = 2^26 has 16 tiles per workgroup per step, so
# arrivals spread far beyond two polls.  Flags: 100 tiles of 16,384 per
# chunk on 256 workgroups, so a workgroup's upstream tiles sit on other
# workgroups (with 2^26 they would all be its own), and workgroups with 3
# tiles per step wait on ones with 4.
ABORT_CASES = [("grid", 8, 1 << 26), ("flags", 8, 8 * 100 * 16384)]


@pytest.mark.parametrize("sync,n,m", ABORT_CASES)
def test_forced_abort_is_reported_and_the_next_calls_run(cs, knobs, sync, n, m):
    send, recv = allreduce_case(n, m)
    ws = cs.Workspace("allreduce", n, m, "float32", "ring_persistent")
    knobs["CCL_SIM_PERSISTENT_SYNC"] = sync
    knobs["CCL_SIM_SPIN_LIMIT"] = "1"
    cs.ccl_sim_allreduce(send, recv, m, schedule="ring_persistent", workspace=ws)  # returns before the kernel runs
    torch.cuda.synchronize()
    del knobs["CCL_SIM_SPIN_LIMIT"]
    assert cs.ccl_sim_persistent_aborted(ws) is True
    check_recovery(cs, send, ws, n, m)


@pytest.mark.parametrize("sync,n,m", ABORT_CASES)
def test_forced_abort_is_an_error_in_debug_mode(cs, knobs, sync, n, m):
    send, recv = allreduce_case(n, m)
    ws = cs.Workspace("allreduce", n, m, "float32", "ring_persistent")
    knobs["CCL_SIM_PERSISTENT_SYNC"] = sync
    knobs["CCL_SIM_SPIN_LIMIT"] = "1"
    knobs["CCL_SIM_DEBUG"] = "1"
    with pytest.raises(cs.CclSimError, match="poll limit"):
        cs.ccl_sim_allreduce(send, recv, m, schedule="ring_persistent", workspace=ws)
    torch.cuda.synchronize()
    del knobs["CCL_SIM_SPIN_LIMIT"]
    del knobs["CCL_SIM_DEBUG"]
    assert cs.ccl_sim_persistent_aborted(ws) is True
    check_recovery(cs, send, ws, n, m)
