"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: every expected value is a
number the pages print (``tests/golden/*.json``, each with its citation), a
closed form, a brute-force count with Python integers, or an invariant of
the definitions.  ``test_oracle_mutants.py`` plants plausible mistakes in
the oracle and checks that these pins catch them.
"""

import math

import numpy as np
import pytest

from oracle import collectives as C
from oracle import reduction as R
from oracle import ring as G
from oracle import scalar as S

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def affine(nranks, count, a, dtype):
    return [np.array([a * r + i for i in range(count)], dtype=R.STORAGE[dtype]) for r in range(nranks)]


# --------------------------------------------------------------------------
# The four-rank, 20-element int64 worked example.
# --------------------------------------------------------------------------

def test_worked_example_all_routes(golden):
    g = golden("worked_example_4x20_int64.json")
    n, m = g["nranks"], g["count"]
    xs = affine(n, m, 100, "int64")
    expect = np.array(g["allreduce"], dtype=np.int64)
    q = C.shard_count(m, n)
    assert q == g["shard_len"]

    for y in C.direct_allreduce(xs, "sum", "int64"):
        assert np.array_equal(y, expect)
    shards = C.reduce_scatter(xs, "sum", "int64", q)
    assert [s.tolist() for s in shards] == g["shards"]
    for y in C.all_gather(shards):
        assert np.array_equal(y, expect)
    for y in C.allreduce_via_rs_ag(xs, "sum", "int64"):
        assert np.array_equal(y, expect)
    for y in G.ring_allreduce(xs, "sum", "int64"):
        assert np.array_equal(y, expect)
    rshards = G.ring_reduce_scatter(xs, "sum", "int64", q)
    assert [s.tolist() for s in rshards] == g["shards"]
    for y in G.ring_all_gather(rshards):
        assert np.array_equal(y, expect)
    lists = [x.tolist() for x in xs]
    for fn in (S.allreduce_direct, S.allreduce_rs_ag, S.allreduce_ring):
        for y in fn(lists, "sum", "int64"):
            assert y == g["allreduce"]
    # the page's independent formula, 600 + 4i
    assert expect.tolist() == [600 + 4 * i for i in range(m)]
    # AVG divides the same sums by the world size: 150 + i
    for route in (C.direct_allreduce, C.allreduce_via_rs_ag, G.ring_allreduce):
        assert route(xs, "avg", "int64")[0].tolist() == [150 + i for i in range(m)]


def test_worked_example_negatives_differ_everywhere(golden):
    """RS(MAX)+AG and a gathered result rolled by ±1 shard must differ from
    the SUM AllReduce at every element, not just somewhere."""
    g = golden("worked_example_4x20_int64.json")
    n, m = g["nranks"], g["count"]
    xs = affine(n, m, 100, "int64")
    direct = C.direct_allreduce(xs, "sum", "int64")[0]
    q = C.shard_count(m, n)
    max_gathered = C.all_gather(C.reduce_scatter(xs, "max", "int64", q))[0]
    assert max_gathered.tolist() == [300 + i for i in range(m)]
    assert np.all(max_gathered != direct)
    for shifts in (1, -1):
        wrong = C.roll_shards(direct, n, shifts)
        assert np.all(wrong != direct)
    # roll +1 puts shard 3 where shard 0 belongs: 600 + 4(i + 15)
    assert C.roll_shards(direct, n, 1)[:5].tolist() == [600 + 4 * (i + 15) for i in range(5)]


# --------------------------------------------------------------------------
# Padding.
# --------------------------------------------------------------------------

def test_padding_arithmetic(golden):
    g = golden("padding_1003_over_4.json")
    q = C.shard_count(g["logical_count"], g["nranks"])
    assert q == g["shard_len"] == g["nccl_info"]["reduce_scatter_recvcount"]
    assert q * g["nranks"] == g["padded_count"]
    assert C.shard_count(1_000_003, 8) == 125_001
    assert 8 * 125_001 - 1_000_003 == 5
    assert C.shard_count(0, 8) == 0
    assert C.shard_count(1, 8) == 1


def test_padding_and_trim_equivalence_1003(golden):
    g = golden("padding_1003_over_4.json")
    n, m = g["nranks"], g["logical_count"]
    rng = np.random.default_rng(7)
    xs = [rng.integers(-1000, 1000, m).astype(np.int64) for _ in range(n)]
    exact = [sum(int(x[i]) for x in xs) for i in range(m)]
    y = C.allreduce_via_rs_ag(xs, "sum", "int64")[0]
    assert y.tolist() == exact
    assert y.size == m


def test_nondivisible_without_padding_rejected(golden):
    g = golden("padding_1003_over_4.json")
    n, m = g["nranks"], g["logical_count"]
    xs = [np.zeros(m, dtype=np.int64) for _ in range(n)]
    assert g["rejection_exception"] == "TypeError"
    with pytest.raises(TypeError, match="sendcount"):
        C.reduce_scatter(xs, "sum", "int64", g["unpadded_floor_shard"])
    with pytest.raises(TypeError):
        G.ring_reduce_scatter(xs, "sum", "int64", g["unpadded_floor_shard"])


@pytest.mark.parametrize("dtype,op,ident_bits", [
    ("float32", "max", 0xFF800000),
    ("float32", "min", 0x7F800000),
    ("float32", "sum", 0x00000000),
    ("float32", "prod", 0x3F800000),
    ("bfloat16", "max", 0xFF80),
    ("bfloat16", "prod", 0x3F80),
])
def test_padded_tail_is_identity_bits(dtype, op, ident_bits):
    """The padded positions of the last shard carry the identity bit for bit
    (the place where the pad value is observable after a ReduceScatter)."""
    n, m = 8, 1003
    q = C.shard_count(m, n)
    rng = np.random.default_rng(3)
    f = rng.standard_normal((n, m)).astype(np.float32)
    xs = [(r.view(np.uint32) >> 16).astype(np.uint16) if dtype == "bfloat16" else r for r in f]
    shards = C.reduce_scatter(C.pad_identity(xs, op, dtype, n * q), op, dtype, q)
    tail = shards[-1][m - (n - 1) * q:]
    assert tail.size == n * q - m == 5
    view = np.uint16 if dtype == "bfloat16" else np.uint32
    assert np.all(tail.view(view) == ident_bits)


@pytest.mark.parametrize("dtype,op,ident", [("int32", "sum", 0), ("int32", "max", -2**31),
                                            ("int32", "min", 2**31 - 1), ("int64", "prod", 1),
                                            ("int64", "max", -2**63)])
def test_padded_tail_is_identity_int(dtype, op, ident):
    n, m = 8, 1003
    q = C.shard_count(m, n)
    xs = [np.arange(m, dtype=R.STORAGE[dtype]) - 500 for _ in range(n)]
    shards = C.reduce_scatter(C.pad_identity(xs, op, dtype, n * q), op, dtype, q)
    assert shards[-1][m - (n - 1) * q:].tolist() == [ident] * 5


def test_max_padding_must_not_be_zero():
    """On all-negative data a downstream max over all shards sees the pad:
    the identity keeps the true maximum, a mechanical zero would not."""
    n, m = 8, 1003
    q = C.shard_count(m, n)
    rng = np.random.default_rng(11)
    xs = [-(np.abs(rng.standard_normal(m)) + 0.5).astype(np.float32) for _ in range(n)]
    true_max = max(float(x.max()) for x in xs)
    shards = C.reduce_scatter(C.pad_identity(xs, "max", "float32", n * q), "max", "float32", q)
    assert max(float(z.max()) for z in shards) == true_max
    zero_padded = [np.concatenate([x, np.zeros(n * q - m, np.float32)]) for x in xs]
    bad = C.reduce_scatter(zero_padded, "max", "float32", q)
    assert max(float(z.max()) for z in bad) == 0.0 != true_max


# --------------------------------------------------------------------------
# Ring routing, ownership, per-step state.
# --------------------------------------------------------------------------

def test_ring_routing_table_n4(golden):
    g = golden("ring_n4_routing.json")
    n = g["nranks"]
    for t, row in enumerate(g["reduce_scatter_send"]):
        assert [G.reduce_scatter_route(n, t, r)[0] for r in range(n)] == row
        # what rank r+1 receives is what rank r sent
        assert [G.reduce_scatter_route(n, t, (r + 1) % n)[1] for r in range(n)] == row
    assert [G.ring_owner(n, r) for r in range(n)] == g["owner_after_reduce_scatter"]
    for t, row in enumerate(g["all_gather_send"]):
        assert [G.all_gather_route(n, t, r)[0] for r in range(n)] == row
        assert [G.all_gather_route(n, t, (r + 1) % n)[1] for r in range(n)] == row


def _token_bufs(n, letters=None):
    """Per-rank buffers of symbolic tokens: rank g's chunk k is 'Lk+' where L
    is the rank's letter; SUM over object arrays concatenates, so a partial
    spells out the addends in the order they were combined."""
    letters = letters or [str(r) for r in range(n)]
    return [np.array([f"{letters[g]}{k}+" for k in range(n)], dtype=object) for g in range(n)]


def _tokens(cell):
    return [t for t in cell.split("+") if t]


def test_ring_round_sums_in_order(golden):
    """Round-by-round partial sums of the four-GPU ring, addends in order."""
    g = golden("ring_n4_round_sums.json")
    n = g["nranks"]
    bufs = _token_bufs(n, list("abcd"))
    states = G._rs_phase(bufs, "sum", 1, record=True)
    for t, expect in enumerate(g["rounds"]):
        for gpu, (chunk, addends) in expect.items():
            got = _tokens(states[t][int(gpu)][chunk])
            if t == len(g["rounds"]) - 1:
                assert sorted(got) == sorted(addends)  # the page writes S_k in letter order
            else:
                assert got == addends
    for gpu, chunk in g["owner_after_reduce_scatter"].items():
        assert len(_tokens(states[-1][int(gpu)][chunk])) == n


def test_ring_staircase_n4(golden):
    g = golden("ring_n4_staircase.json")
    n = g["nranks"]
    states = G._rs_phase(_token_bufs(n), "sum", 1, record=True)
    for t, changes in enumerate(g["changes_per_step"]):
        for rank, (chunk, contributors) in changes.items():
            assert [int(tok[0]) for tok in _tokens(states[t][int(rank)][chunk])] == contributors
    final = states[-1]
    for r in range(n):
        for c in range(n):
            assert [int(tok[0]) for tok in _tokens(final[r][c])] == g["state_after_reduce_scatter"][r][c]


def test_ring_onehot_bitmasks():
    """x^(r) = 2^r under int64 SUM: after RS step t, rank r's chunk
    (r-1-t) holds exactly ranks {r-1-t, ..., r}; afterwards rank r holds
    all ones in chunk r+1 (N up to 12)."""
    for n in range(2, 13):
        xs = [np.full(n, 1 << r, dtype=np.int64) for r in range(n)]
        bufs = [R.widen(x, "int64") for x in xs]
        states = G._rs_phase(bufs, "sum", 1, record=True)
        assert len(states) == n - 1
        for t, st in enumerate(states):
            for r in range(n):
                c = (r - 1 - t) % n
                want = sum(1 << ((r - k) % n) for k in range(t + 2))
                assert int(st[r][c]) == want
        for r in range(n):
            assert int(states[-1][r][G.ring_owner(n, r)]) == (1 << n) - 1


def test_ring_allgather_grid_n4(golden):
    g = golden("ring_n4_allgather_grid.json")
    n = g["nranks"]
    xs = [np.full(n, 1 << r, dtype=np.int64) for r in range(n)]
    _, states = G.ring_allreduce(xs, "sum", "int64", record=True)
    full = (1 << n) - 1
    for k, key in enumerate(["after_step_3", "after_step_4", "after_step_5", "after_step_6"]):
        st = states[2 + k]
        grid = ["".join("#" if int(st[r][c]) == full else "." for c in range(n)) for r in range(n)]
        assert grid == g["grids"][key]


def test_step_counts(golden):
    g = golden("step_counts.json")
    for n, steps in g["allreduce_steps"].items():
        assert G.step_counts(int(n))["allreduce"] == steps
    xs = [np.arange(8, dtype=np.int64) for _ in range(8)]
    _, states = G.ring_allreduce(xs, "sum", "int64", record=True)
    assert len(states) == g["allreduce_steps"]["8"]
    xs4 = [np.arange(4, dtype=np.int64) for _ in range(4)]
    _, rs = G.ring_reduce_scatter(xs4, "sum", "int64", 1, record=True)
    assert len(rs) == g["phase_steps_n4"]
    _, ag = G.ring_all_gather([np.arange(1, dtype=np.int64)] * 4, record=True)
    assert len(ag) == g["phase_steps_n4"]


# --------------------------------------------------------------------------
# Closed forms and brute force.
# --------------------------------------------------------------------------

def _wrap(v, bits):
    v &= (1 << bits) - 1
    return v - (1 << bits) if v >> (bits - 1) else v


def _trunc_div(v, n):
    """Integer division rounding toward zero (the AVG post-operation)."""
    q = abs(v) // n
    return q if v >= 0 else -q


ROUTES = {
    "direct": lambda xs, op, dt: C.direct_allreduce(xs, op, dt),
    "rs_ag": lambda xs, op, dt: C.allreduce_via_rs_ag(xs, op, dt),
    "ring": lambda xs, op, dt: G.ring_allreduce(xs, op, dt),
    "ring_rs_ag": lambda xs, op, dt: _ring_rs_ag(xs, op, dt),
}


def _ring_rs_ag(xs, op, dt):
    n, m = len(xs), xs[0].size
    q = C.shard_count(m, n)
    padded = C.pad_identity(xs, op, dt, n * q)
    return G.ring_all_gather(G.ring_reduce_scatter(padded, op, dt, q), m)


@pytest.mark.parametrize("dtype", ["int32", "int64"])
@pytest.mark.parametrize("n,m,a", [(1, 5, 7), (2, 7, 3), (3, 10, 100), (5, 17, 1000), (8, 29, 12345)])
def test_closed_forms(dtype, n, m, a):
    bits = 32 if dtype == "int32" else 64
    xs = affine(n, m, a, dtype)
    want = {
        "sum": [_wrap(a * n * (n - 1) // 2 + n * i, bits) for i in range(m)],
        "avg": [_trunc_div(_wrap(a * n * (n - 1) // 2 + n * i, bits), n) for i in range(m)],
        "max": [a * (n - 1) + i for i in range(m)],
        "min": list(range(m)),
        "prod": [_wrap(math.prod(a * r + i for r in range(n)), bits) for i in range(m)],
    }
    for op, expect in want.items():
        for name, route in ROUTES.items():
            outs = route(xs, op, dtype)
            assert len(outs) == n
            for y in outs:
                assert y.tolist() == expect, (name, op)


def test_brute_force_integer_routes_agree_with_exact():
    rng = np.random.default_rng(2024)
    for n in range(1, 10):
        for m in range(0, 3 * n + 3):
            for dtype, bits in (("int32", 32), ("int64", 64)):
                lim = 1 << (bits - 2)
                xs = [rng.integers(-lim, lim, m).astype(R.STORAGE[dtype]) for _ in range(n)]
                for op in R.OPS:
                    if op == "sum":
                        exact = [_wrap(sum(int(x[i]) for x in xs), bits) for i in range(m)]
                    elif op == "avg":
                        exact = [_trunc_div(_wrap(sum(int(x[i]) for x in xs), bits), n) for i in range(m)]
                    elif op == "prod":
                        exact = [_wrap(math.prod(int(x[i]) for x in xs), bits) for i in range(m)]
                    elif op == "max":
                        exact = [max(int(x[i]) for x in xs) for i in range(m)]
                    else:
                        exact = [min(int(x[i]) for x in xs) for i in range(m)]
                    for name, route in ROUTES.items():
                        for y in route(xs, op, dtype):
                            assert y.tolist() == exact, (n, m, dtype, op, name)
                    lists = [x.tolist() for x in xs]
                    for fn in (S.allreduce_direct, S.allreduce_rs_ag, S.allreduce_ring):
                        assert fn(lists, op, dtype)[0] == exact


def test_ring_sweep_up_to_256_ranks_matches_exact_sum():
    """The ring is correct for N = 2..256 against an exact sum."""
    for n in (2, 3, 4, 7, 16, 63, 256):
        rng = np.random.default_rng(n)
        m = n + 3
        xs = [rng.integers(-10**6, 10**6, m).astype(np.int64) for _ in range(n)]
        exact = [sum(int(x[i]) for x in xs) for i in range(m)]
        outs = G.ring_allreduce(xs, "sum", "int64")
        for y in outs:
            assert y.tolist() == exact


# --------------------------------------------------------------------------
# Floating point: order emulation and error bounds.
# --------------------------------------------------------------------------

def _f32_inputs(n, m, seed, dist="uniform"):
    rng = np.random.default_rng(seed)
    if dist == "uniform":
        return [rng.uniform(-1, 1, m).astype(np.float32) for _ in range(n)]
    return [(rng.standard_normal(m) * 1e-3).astype(np.float32) for _ in range(n)]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 13])
def test_fp32_orders_match_scalar_twin_bitwise(n):
    m = 3 * n + 2
    xs = _f32_inputs(n, m, 100 + n)
    lists = [x.astype(np.float64).tolist() for x in xs]
    for op in R.OPS:
        d = C.direct_allreduce(xs, op, "float32")[0]
        sd = np.array(S.allreduce_direct(lists, op, "float32")[0], dtype=np.float32)
        assert np.array_equal(d.view(np.uint32), sd.view(np.uint32))
        rg = G.ring_allreduce(xs, op, "float32")[0]
        sr = np.array(S.allreduce_ring(lists, op, "float32")[0], dtype=np.float32)
        assert np.array_equal(rg.view(np.uint32), sr.view(np.uint32))
        ra = C.allreduce_via_rs_ag(xs, op, "float32")[0]
        assert np.array_equal(ra.view(np.uint32), d.view(np.uint32))


def test_fp32_ring_fold_matches_chunk_order():
    """The stepped ring equals, chunk by chunk, a left fold over the ranks
    x^(c), x^(c+1), ..., x^(c-1)."""
    for n in (3, 5, 8):
        q = 7
        xs = _f32_inputs(n, n * q, 9 + n)
        ring = G.ring_allreduce(xs, "sum", "float32")[0]
        for c in range(n):
            sl = slice(c * q, (c + 1) * q)
            want = C.fold([x[sl] for x in xs], "sum", "float32", G.chunk_order(n, c))
            assert np.array_equal(ring[sl].view(np.uint32), want.view(np.uint32))


def test_fp32_ring_vs_ascending_order():
    """N <= 2: every order gives the same bits (IEEE ⊕ is commutative).
    N >= 3: the ring order and the ascending order differ somewhere, and
    both stay within (N-1)·2^-24 of the exact sum, normalised by Σ|x|."""
    for n in (1, 2):
        xs = _f32_inputs(n, 4096, 5 + n)
        a = C.direct_allreduce(xs, "sum", "float32")[0]
        b = G.ring_allreduce(xs, "sum", "float32")[0]
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    for n in (3, 4, 8, 17):
        xs = _f32_inputs(n, 4096, 5 + n)
        a = C.direct_allreduce(xs, "sum", "float32")[0]
        b = G.ring_allreduce(xs, "sum", "float32")[0]
        assert not np.array_equal(a.view(np.uint32), b.view(np.uint32))
        bound = (n - 1) * 2.0 ** -24 * 1.01
        ea = R.normalized_sum_error(a, xs, "float32")
        eb = R.normalized_sum_error(b, xs, "float32")
        assert 0 < ea <= bound and 0 < eb <= bound
        assert ea <= 1e-5 * n and eb <= 1e-5 * n


def test_normalized_sum_error_by_hand():
    """The tolerance measure on values worked out by hand: the error is
    |y - Σx| over Σ|x| (not over |Σx|, which a cancelling sum would make
    tiny), computed in float64, maximised over positions."""
    xs = [np.array([1.0, 1.0, 0.5], dtype=np.float32), np.array([2.0, -1.0, 0.25], dtype=np.float32)]
    y = np.array([3.0, 2.0 ** -20, 0.75], dtype=np.float32)
    # position 0: exact -> 0; position 1: sum 0, |x| sum 2 -> 2^-20 / 2; position 2: exact
    assert R.normalized_sum_error(y, xs, "float32") == 2.0 ** -21
    y2 = np.array([3.0 + 2.0 ** -22, 0.0, 0.75], dtype=np.float32)
    assert R.normalized_sum_error(y2, xs, "float32") == 2.0 ** -22 / 3.0
    bf = [(x.view(np.uint32) >> 16).astype(np.uint16) for x in xs]
    yb = (np.array([3.0, 0.0, 0.75], dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert R.normalized_sum_error(yb, bf, "bfloat16") == 0.0


def test_avg_is_the_sum_divided_once():
    """AVG = one correctly rounded division of the schedule's float32 sum by
    N (checked against Python's own division of the exact binary32 sum), and
    integer AVG truncates toward zero (-7 / 2 -> -3, not -4)."""
    for n in (2, 3, 8):
        xs = _f32_inputs(n, 333, 50 + n)
        for route in (C.direct_allreduce, G.ring_allreduce):
            s = route(xs, "sum", "float32")[0]
            a = route(xs, "avg", "float32")[0]
            want = np.array([np.float32(float(v) / n) for v in s], dtype=np.float32)
            assert np.array_equal(a.view(np.uint32), want.view(np.uint32))
    xs = [np.array([-3, 5], dtype=np.int32), np.array([-4, 2], dtype=np.int32)]
    assert C.direct_allreduce(xs, "avg", "int32")[0].tolist() == [-3, 3]
    xs64 = [np.array([-(2**62), 2**62], dtype=np.int64) for _ in range(3)]
    assert C.direct_allreduce(xs64, "avg", "int64")[0].tolist() == [_trunc_div(_wrap(-3 * 2**62, 64), 3),
                                                                     _trunc_div(_wrap(3 * 2**62, 64), 3)]


def test_fp32_sum_matches_fsum_within_bound():
    """Scalar check against math.fsum (the exactly rounded sum)."""
    n = 16
    xs = _f32_inputs(n, 200, 77)
    y = C.direct_allreduce(xs, "sum", "float32")[0]
    for i in range(200):
        vals = [float(x[i]) for x in xs]
        exact = math.fsum(vals)
        scale = math.fsum(abs(v) for v in vals)
        assert abs(float(y[i]) - exact) <= (n - 1) * 2.0 ** -24 * scale * 1.01


def test_gradient_like_256_ranks_tolerance():
    n = 256
    xs = _f32_inputs(n, 2048, 31, dist="normal")
    for route in (C.direct_allreduce, G.ring_allreduce):
        y = route(xs, "sum", "float32")[0]
        assert R.normalized_sum_error(y, xs, "float32") <= 1e-5 * n
    bf = [(x.view(np.uint32) >> 16).astype(np.uint16) for x in xs]
    for route in (C.direct_allreduce, G.ring_allreduce):
        y = route(bf, "sum", "bfloat16")[0]
        err = R.normalized_sum_error(y, bf, "bfloat16")
        assert err <= 1e-2
        # one final rounding: within half a bf16 ulp plus the fp32 sum error
        assert err <= 2.0 ** -8 + n * 2.0 ** -24


# --------------------------------------------------------------------------
# bf16 rounding from its definition.
# --------------------------------------------------------------------------

BF16_CASES = [
    (0x3F800000, 0x3F80),   # 1.0 exact
    (0x3F808000, 0x3F80),   # halfway, lower pattern even -> stays
    (0x3F818000, 0x3F82),   # halfway, lower pattern odd -> up to even
    (0x3F808001, 0x3F81),   # above half -> up
    (0x3F807FFF, 0x3F80),   # below half -> down
    (0xBFC00000, 0xBFC0),   # -1.5 exact
    (0xBF808001, 0xBF81),   # negative, above half -> away from zero
    (0x7F7FFFFF, 0x7F80),   # largest float rounds to +inf
    (0x7F7F7FFF, 0x7F7F),   # just below the rounding point stays finite
    (0xFF7FFFFF, 0xFF80),   # to -inf
    (0x7F800000, 0x7F80),   # +inf
    (0xFF800000, 0xFF80),   # -inf
    (0x00008000, 0x0000),   # subnormal tie at zero -> even (zero)
    (0x00018000, 0x0002),   # subnormal tie, odd -> up
    (0x80000000, 0x8000),   # -0
    (0x7FC00001, 0x7FC0),   # quiet NaN stays quiet
    (0x7F800001, 0x7FC0),   # signalling NaN made quiet
]


def test_bf16_rounding_cases():
    bits = np.array([c[0] for c in BF16_CASES], dtype=np.uint32)
    want = [c[1] for c in BF16_CASES]
    assert R.bf16_round_bits(bits.view(np.float32)).tolist() == want
    for u, w in BF16_CASES:
        assert S.f32_to_bf16(S.bits_f32(u)) == w, hex(u)


def test_bf16_rounding_exhaustive_upper_patterns_against_twin():
    """Every upper pattern with low halves around the rounding point."""
    rng = np.random.default_rng(1)
    uppers = np.arange(0, 1 << 16, 37, dtype=np.uint32)
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    bits = ((uppers[:, None] << 16) | lows[None, :]).ravel()
    bits = np.concatenate([bits, rng.integers(0, 1 << 32, 2000, dtype=np.uint64).astype(np.uint32)])
    got = R.bf16_round_bits(bits.view(np.float32))
    for u, gv in zip(bits.tolist(), got.tolist()):
        assert S.f32_to_bf16(S.bits_f32(u)) == gv, hex(u)


def test_identities():
    assert R.identity("sum", "int32") == 0
    assert R.identity("prod", "float32") == 1.0
    assert R.identity("max", "float32") == -np.inf
    assert R.identity("min", "bfloat16") == np.inf
    assert R.identity("max", "int32") == -2**31
    assert R.identity("min", "int64") == 2**63 - 1
    for op in R.OPS:
        for dt in R.DTYPES:
            e = R.identity(op, dt)
            x = R.widen(np.array([3, -5, 0], dtype=R.STORAGE[dt]) if dt != "bfloat16"
                        else np.array([0x4040, 0xC0A0, 0x0000], dtype=np.uint16), dt)
            ident = np.full(3, e, dtype=R.ACCUM[dt])
            assert np.array_equal(R.combine(op, ident, x), x)
            assert np.array_equal(R.combine(op, x, ident), x)
