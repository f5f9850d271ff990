"""GPU parity at full size, every element of every rank.

The 256-rank workloads (M = 2^22 float32 normal(0, 1e-3), 510 ring steps,
and the 6,553,600-element bf16 bucket with float32 accumulation) and the
bf16 shape above every small-launch threshold (N = 8, M = 2^27), under all
six schedules: ReduceScatter, AllGather of the ReduceScatter's shards, and
AllReduce.  Each is compared bit for bit, at every position of every rank,
with the oracle's fold of the same inputs in the schedule's combining order:
ascending ranks (direct), chunk c from its origin rank c round the ring
(the three ring drivers), or the halving butterfly (both recursive
drivers).  The expected values are folded on the host, one 2^20-position
column block of all N ranks at a time, uploaded once, and compared on the
device as integer bit patterns.  The float64 tolerance bound of the
workload is checked for each of the three orders on every block.

Reference for the method of checking: the correctness rule of "NCCL 专家课程
07：AllReduce 等价分解、显存生命周期与 Kernel 证据" (its performance-experiment
section: every element, scanned in chunks), and the element-by-element
checks over N = 2 ... 256 of "Ring AllReduce 核心流程" (pseudocode and
measured-data section).
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import gpu_util as U
from collective_reduction_amd import inputs as I
from oracle import collectives as C
from oracle import recursive as H
from oracle import reduction as R
from oracle import ring as G

pytestmark = pytest.mark.gpu

FAMILY = {"direct": "ascending", "ring_stepwise": "ring", "ring_persistent": "ring", "ring_chained": "ring",
          "recursive": "butterfly", "recursive_chained": "butterfly"}
BITS = {"float32": torch.int32, "bfloat16": torch.int16, "int32": torch.int32, "int64": torch.int64}


@pytest.fixture(scope="module")
def cs():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from collective_reduction_amd import ccl_sim
    return ccl_sim


class FullWorkload:
    """Device copies of a workload's N rank buffers and, on the host, the
    oracle's result of each combining order at every position."""

    def __init__(self, s, op="sum"):
        self.s, self.op = s, op
        self.n, self.m, self.dtype = s["nranks"], s["count"], s["dtype"]
        n, m, dtype = self.n, self.m, self.dtype
        self.q = C.shard_count(m, n)
        assert n * self.q == m, "full-scan workloads divide into N shards"
        print(f"[full-scan] preparing {n}x{m} {dtype} {op}", flush=True)
        self.send = [U.empty(m, dtype) for _ in range(n)]
        self.want = {f: np.empty(m, dtype=U.NP[dtype]) for f in ("ascending", "ring", "butterfly")}
        self.errors = {f: 0.0 for f in self.want}
        block = I.CHUNK
        with ThreadPoolExecutor(16) as pool:
            for lo in range(0, m, block):
                hi = min(m, lo + block)
                rows = list(pool.map(lambda r: I.rank_buffer(self.s, r, lo, hi), range(n)))
                for r in range(n):
                    self.send[r][lo:hi].copy_(U.to_dev(rows[r], dtype))
                self._fold_block(rows, lo, hi)
        torch.cuda.synchronize()
        self.want_dev = {f: U.to_dev(w, dtype).view(BITS[dtype]) for f, w in self.want.items()}
        print(f"[full-scan] ready: normalised errors {self.errors}", flush=True)

    def _finish(self, acc):
        return R.narrow(R.finalize(self.op, acc, self.n), self.dtype)

    def _fold_block(self, rows, lo, hi):
        n, q, op, dtype = self.n, self.q, self.op, self.dtype
        self.want["ascending"][lo:hi] = self._finish(C.fold(rows, op, dtype, list(range(n))))
        self.want["butterfly"][lo:hi] = self._finish(H.butterfly_fold(rows, op, dtype))
        for c in range(lo // q, (hi - 1) // q + 1):
            a, b = max(lo, c * q), min(hi, (c + 1) * q)
            cols = [x[a - lo:b - lo] for x in rows]
            self.want["ring"][a:b] = self._finish(C.fold(cols, op, dtype, G.chunk_order(n, c)))
        if op == "sum" and dtype in ("float32", "bfloat16"):
            ref = R.fp64_reference(rows, dtype)
            scale = np.maximum(R.abs_sum64(rows, dtype), np.finfo(np.float64).tiny)
            for f, w in self.want.items():
                err = float(np.max(np.abs(R.widen(w[lo:hi], dtype).astype(np.float64) - ref) / scale))
                self.errors[f] = max(self.errors[f], err)

    def check_tolerance(self):
        if self.op != "sum" or self.dtype not in ("float32", "bfloat16"):
            return
        bound = 1e-5 * self.n if self.dtype == "float32" else 1e-2
        for f, err in self.errors.items():
            assert err <= bound, (f, err, bound)

    def run_and_compare(self, cs, schedule):
        n, m, q, dtype = self.n, self.m, self.q, self.dtype
        print(f"[full-scan] {n}x{m} {dtype} {schedule}", flush=True)
        ws = cs.Workspace.largest([(c, n, m, dtype, schedule) for c in ("reduce_scatter", "all_gather", "allreduce")])
        shards = [U.empty(q, dtype) for _ in range(n)]
        gathered = [U.empty(m, dtype) for _ in range(n)]
        ar = [U.empty(m, dtype) for _ in range(n)]
        cs.ccl_sim_reduce_scatter(self.send, shards, m, q, op=self.op, schedule=schedule, workspace=ws, dtype=dtype)
        if schedule == "ring_persistent":
            torch.cuda.synchronize()
            assert cs.ccl_sim_persistent_aborted(ws) is False
        cs.ccl_sim_all_gather(shards, gathered, q, m, schedule=schedule, workspace=ws, dtype=dtype)
        if schedule == "ring_persistent":
            torch.cuda.synchronize()
            assert cs.ccl_sim_persistent_aborted(ws) is False
        cs.ccl_sim_allreduce(self.send, ar, m, op=self.op, schedule=schedule, workspace=ws, dtype=dtype)
        torch.cuda.synchronize()
        if schedule == "ring_persistent":
            assert cs.ccl_sim_persistent_aborted(ws) is False
        want = self.want_dev[FAMILY[schedule]]
        bad = []
        for r in range(n):
            for what, got, exp in (("shard", shards[r], want[r * q:(r + 1) * q]),
                                   ("gathered", gathered[r], want), ("allreduce", ar[r], want)):
                g = got.view(BITS[dtype])
                if not torch.equal(g, exp):
                    idx = torch.nonzero(g != exp)[:4].flatten().tolist()
                    bad.append(f"{what} of rank {r}: first differing positions {idx}")
        del shards, gathered, ar, ws
        torch.cuda.empty_cache()
        assert not bad, f"{schedule}: " + "; ".join(bad[:8]) + (f" (and {len(bad) - 8} more)" if len(bad) > 8 else "")


_CACHE = {}


def workload(name, **overrides):
    key = (name, tuple(sorted(overrides.items())))
    if key not in _CACHE:
        _CACHE.clear()  # one workload resident at a time
        torch.cuda.empty_cache()
        _CACHE[key] = FullWorkload(I.spec(name, **overrides))
    return _CACHE[key]


@pytest.fixture(scope="module", autouse=True)
def _release():
    yield
    _CACHE.clear()
    if torch.cuda.is_available():
        torch.cuda.empty_cache()


@pytest.mark.parametrize("schedule", U.SCHEDULES)
def test_gradient_256x4194304_fp32_every_element(cs, schedule):
    """N=256, M=2^22 normal(0, 1e-3) float32 SUM (the ring runs 510 steps)."""
    w = workload("normal_256x4194304_fp32")
    w.check_tolerance()
    w.run_and_compare(cs, schedule)


@pytest.mark.parametrize("schedule", U.SCHEDULES)
def test_gradient_256x6553600_bf16_every_element(cs, schedule):
    """The 6,553,600-element bf16 bucket over 256 ranks, float32 accumulation."""
    w = workload("normal_256x6553600_bf16")
    w.check_tolerance()
    w.run_and_compare(cs, schedule)


@pytest.mark.parametrize("schedule", U.SCHEDULES)
def test_uniform_8x134217728_bf16_every_element(cs, schedule):
    """bf16 above every small-launch threshold (N=8, M=2^27): each schedule
    runs its large-step launch shape, and the ring its 32-byte float32
    accumulator vectors, on bf16 data."""
    w = workload("uniform_8x268435456_fp32", count=1 << 27, dtype="bfloat16")
    w.check_tolerance()
    w.run_and_compare(cs, schedule)


@pytest.mark.parametrize("schedule", U.SCHEDULES)
def test_max_ranks_1024_fp32_every_element(cs, schedule):
    """The largest rank count the library accepts, 1,024 ranks of 320
    float32 elements (whole 128-byte lines, so the persistent ring's step
    flags read same-XCD data from the L2, with the XCD placement of its
    workgroups): 2,046 ring steps, pointer tables in the workspace, ten
    halving levels, every tile ragged."""
    w = workload("normal_256x4194304_fp32", nranks=1024, count=1024 * 320)
    w.check_tolerance()
    w.run_and_compare(cs, schedule)


@pytest.mark.parametrize("schedule", U.SCHEDULES)
def test_max_ranks_1024_int32_every_element(cs, schedule):
    """1,024 ranks of 301 int32 elements (chunks off the line grid):
    integer SUM is exact in any order, so every schedule must reproduce the
    same values at every position."""
    w = workload("intuniform_8x1000003_int32", nranks=1024, count=1024 * 301)
    w.run_and_compare(cs, schedule)
