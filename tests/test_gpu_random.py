"""GPU parity over seeded random call shapes.

Each case draws a rank count (1 to 256, powers of two and not), a length
(empty, shorter than the rank count, a few tiles with a ragged tail), a
dtype, an op, a schedule, a collective, the in-place form or not, and a
base-address offset; the library's result must equal the oracle's in the
schedule's combining order, bit for bit.  The draws come from one fixed
seed, so a failure names a case that can be rerun exactly.

CCL_SIM_TEST_RANDOM_SEED and CCL_SIM_TEST_RANDOM_BLOCKS (default 20261202
and 8 blocks of 60 cases) widen the sweep: another seed draws other shapes,
and its inputs are seeded apart from the default's (from 500000 on).
"""

import os

import numpy as np
import pytest
import torch

import gpu_util as U
from oracle import collectives as C
from oracle import recursive as H
from oracle import ring as G

pytestmark = pytest.mark.gpu

RANKS = (1, 2, 3, 4, 5, 7, 8, 13, 16, 31, 64, 65, 100, 128, 256)
DTYPES = ("int32", "int64", "float32", "bfloat16")
OPS = ("sum", "prod", "max", "min", "avg")
DEFAULT_SEED = 20261202
SEED = int(os.environ.get("CCL_SIM_TEST_RANDOM_SEED", DEFAULT_SEED))
BLOCKS = int(os.environ.get("CCL_SIM_TEST_RANDOM_BLOCKS", 8))
INPUT_BASE = 0 if SEED == DEFAULT_SEED else 500000


@pytest.fixture(scope="module")
def cs():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from collective_reduction_amd import ccl_sim
    return ccl_sim


def draw(rng):
    n = int(rng.choice(RANKS))
    schedules = [s for s in U.SCHEDULES if not U.is_recursive(s) or U.pow2(n)]
    case = {
        "n": n,
        "dtype": str(rng.choice(DTYPES)),
        "op": str(rng.choice(OPS)),
        "schedule": str(rng.choice(schedules)),
        "coll": str(rng.choice(("reduce_scatter", "all_gather", "allreduce"))),
        "in_place": bool(rng.random() < 0.25),
        "offset": int(rng.choice((0, 0, 1, 3))),
    }
    kind = rng.random()
    if kind < 0.1:
        q = 0
    elif kind < 0.3:
        q = int(rng.integers(1, 8))
    else:
        q = int(rng.integers(8, max(9, 24_000 // n)))
    case["q"] = q
    # AllReduce and the AllGather's trim take any length up to N·q
    case["m"] = max(n * q - int(rng.integers(0, n)), 0) if rng.random() < 0.5 else n * q
    return case


def oracle_rs(xs, op, dtype, q, schedule):
    if schedule == "direct":
        return C.reduce_scatter(xs, op, dtype, q)
    if U.is_recursive(schedule):
        return H.reduce_scatter(xs, op, dtype, q)
    return G.ring_reduce_scatter(xs, op, dtype, q)


def oracle_ar(xs, op, dtype, schedule):
    if schedule == "direct":
        return C.direct_allreduce(xs, op, dtype)
    if U.is_recursive(schedule):
        return H.allreduce(xs, op, dtype)
    return G.ring_allreduce(xs, op, dtype)


def run_case(cs, c, seed):
    n, q, m, dtype, op, schedule = c["n"], c["q"], c["m"], c["dtype"], c["op"], c["schedule"]
    kw = {"offset": c["offset"], "in_place": c["in_place"]}
    if c["coll"] == "reduce_scatter":
        xs = U.random_inputs(n, n * q, dtype, seed=seed, op=op)
        got = U.run_rs(cs, xs, q, op, dtype, schedule, **kw)
        want = oracle_rs(xs, op, dtype, q, schedule)
        return all(U.same_bits(got[r], want[r]) for r in range(n))
    if c["coll"] == "all_gather":
        shards = U.random_inputs(n, q, dtype, seed=seed)
        got = U.run_ag(cs, shards, m, dtype, schedule, **kw)
        want = C.all_gather(shards, m)[0]
        return all(U.same_bits(y, want) for y in got)
    if m == 0:
        return True
    xs = U.random_inputs(n, m, dtype, seed=seed, op=op)
    got = U.run_ar(cs, xs, op, dtype, schedule, **kw)
    want = oracle_ar(xs, op, dtype, schedule)[0]
    return all(U.same_bits(y, want) for y in got)


@pytest.mark.parametrize("block", range(BLOCKS))
def test_random_call_shapes(cs, block):
    """60 seeded cases per block; every failing case is listed."""
    rng = np.random.default_rng([SEED, block])
    failed = []
    for i in range(60):
        c = draw(rng)
        if not run_case(cs, c, seed=INPUT_BASE + 1000 * block + i):
            failed.append((i, c))
    assert not failed, f"cases that differ from the oracle: {failed}"
