"""Pins of the recursive-halving / recursive-doubling oracle: the pair
table and exchange volumes the page prints, rank-major ownership, exact
integer results by brute force, and the butterfly combining order checked
against an explicitly bracketed float32 expression."""

import math

import numpy as np
import pytest

from oracle import collectives as C
from oracle import recursive as H
from oracle import reduction as R
from oracle import scalar as S


def test_pair_table_and_volumes(golden):
    g = golden("recursive_halving_n8.json")
    n = g["nranks"]
    assert [[list(p) for p in step] for step in H.halving_pairs(n)] == g["pairs"]
    q = 5
    for j, frac in enumerate(g["data_per_node_after"], start=1):
        for i in range(n):
            lo, hi = H.kept_range(n, q, j, i)
            assert hi - lo == frac * n * q
    # every rank ends with its own block: the result is rank-major
    for i in range(n):
        assert H.kept_range(n, q, len(g["pairs"]), i) == (i * q, (i + 1) * q)
    xs = [np.arange(n * q, dtype=np.int64) for _ in range(n)]
    _, states = H.reduce_scatter(xs, "sum", "int64", q, record=True)
    assert len(states) == int(math.log2(n))


def test_onehot_partials_cover_the_pair_groups():
    """x^(r) = 2^r under int64 SUM: after step j, rank i's kept range holds
    the bitmask of the 2^j ranks reachable from i by XOR with the distances
    used so far (N/2, N/4, ...); after the last step, all N ranks."""
    n, q = 16, 3
    xs = [np.full(n * q, 1 << r, dtype=np.int64) for r in range(n)]
    _, states = H.reduce_scatter(xs, "sum", "int64", q, record=True)
    for j, st in enumerate(states, start=1):
        dists = [n >> jj for jj in range(1, j + 1)]
        for i in range(n):
            group = {i}
            for d in dists:
                group |= {g ^ d for g in group}
            lo, hi = H.kept_range(n, q, j, i)
            assert np.all(st[i][lo:hi] == sum(1 << g for g in group))
    shards = H.reduce_scatter(xs, "sum", "int64", q)
    assert all(np.all(z == (1 << n) - 1) for z in shards)


def _wrap(v, bits):
    v &= (1 << bits) - 1
    return v - (1 << bits) if v >> (bits - 1) else v


def test_brute_force_integers():
    rng = np.random.default_rng(99)
    for n in (1, 2, 4, 8, 16):
        for m in range(0, 2 * n + 3):
            for dtype, bits in (("int32", 32), ("int64", 64)):
                xs = [rng.integers(-(1 << (bits - 2)), 1 << (bits - 2), m).astype(R.STORAGE[dtype])
                      for _ in range(n)]
                for op in R.OPS:
                    vals = [[int(x[i]) for x in xs] for i in range(m)]
                    if op == "sum":
                        exact = [_wrap(sum(v), bits) for v in vals]
                    elif op == "avg":
                        exact = [S.finalize("avg", _wrap(sum(v), bits), n, dtype) for v in vals]
                    elif op == "prod":
                        exact = [_wrap(math.prod(v), bits) for v in vals]
                    elif op == "max":
                        exact = [max(v) for v in vals]
                    else:
                        exact = [min(v) for v in vals]
                    for y in H.allreduce(xs, op, dtype):
                        assert y.tolist() == exact, (n, m, dtype, op)


def test_butterfly_order_float32():
    """Block b of N = 8 is ((x0+x4)+(x2+x6))+((x1+x5)+(x3+x7)), bracketed as
    the halving steps pair the ranks, computed here one binary32 addition at
    a time."""
    n, q = 8, 64
    rng = np.random.default_rng(4)
    xs = [rng.uniform(-1, 1, n * q).astype(np.float32) for _ in range(n)]
    shards = H.reduce_scatter(xs, "sum", "float32", q)
    got = np.concatenate(shards)
    for i in range(n * q):
        v = [float(x[i]) for x in xs]
        f = S.f32
        want = f(f(f(v[0] + v[4]) + f(v[2] + v[6])) + f(f(v[1] + v[5]) + f(v[3] + v[7])))
        assert np.float32(want).view(np.uint32) == got[i].view(np.uint32)
    # and it is a third order, distinct from the ascending fold somewhere
    direct = np.concatenate(C.reduce_scatter(xs, "sum", "float32", q))
    assert not np.array_equal(direct.view(np.uint32), got.view(np.uint32))
    assert R.normalized_sum_error(got, xs, "float32") <= (n - 1) * 2.0 ** -24


def test_max_ties_keep_the_lower_ranks_partial():
    """Operand order inside each pair: under MAX a tie keeps the left operand
    (max(a, b) = b > a ? b : a), and +0 and -0 tie.  With every input a
    signed zero, the butterfly keeps the lower rank's partial at every
    step, so every result carries the sign of rank 0's input."""
    n, q = 8, 16
    rng = np.random.default_rng(7)
    xs = [np.where(rng.random(n * q) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
          for _ in range(n)]
    got = np.concatenate(H.reduce_scatter(xs, "max", "float32", q))
    assert np.array_equal(np.signbit(got), np.signbit(xs[0]))
    assert not np.array_equal(np.signbit(xs[0]), np.signbit(xs[n - 1]))


def test_doubling_all_gather_and_trim():
    n, q = 8, 7
    rng = np.random.default_rng(1)
    shards = [rng.integers(0, 1000, q).astype(np.int32) for _ in range(n)]
    for rc in (n * q, n * q - 3, q + 1):
        got = H.all_gather(shards, rc)
        want = C.all_gather(shards, rc)
        for y in got:
            assert np.array_equal(y, want[0])


def test_non_power_of_two_rejected():
    with pytest.raises(ValueError):
        H.halving_pairs(6)


def test_butterfly_fold_is_the_bracketed_tree():
    """butterfly_fold at N = 8 is ((x0+x4)+(x2+x6))+((x1+x5)+(x3+x7)), one
    binary32 addition at a time, at every position."""
    n, m = 8, 257
    rng = np.random.default_rng(14)
    xs = [rng.uniform(-1, 1, m).astype(np.float32) for _ in range(n)]
    got = H.butterfly_fold(xs, "sum", "float32")
    f = S.f32
    for i in range(m):
        v = [float(x[i]) for x in xs]
        want = f(f(f(v[0] + v[4]) + f(v[2] + v[6])) + f(f(v[1] + v[5]) + f(v[3] + v[7])))
        assert np.float32(want).view(np.uint32) == got[i].view(np.uint32)


@pytest.mark.parametrize("dtype", R.DTYPES)
@pytest.mark.parametrize("op", R.OPS)
def test_butterfly_fold_matches_the_stepped_ranks(dtype, op):
    """The fold written as one tree over whole arrays gives, at every
    position, what stepping the halving and doubling phases rank by rank
    gives (a different route through the same pairs), for every op and
    dtype, N = 1 .. 32, lengths with and without padding; signed zeros make
    MAX / MIN ties visible."""
    for n in (1, 2, 4, 8, 16, 32):
        for m in (n * 3, n * 3 + 1, 1):
            rng = np.random.default_rng([n, m, len(op), len(dtype)])
            if dtype in ("int32", "int64"):
                lo, hi = (-4, 5) if op == "prod" else (-1000, 1000)
                xs = [rng.integers(lo, hi, m).astype(R.STORAGE[dtype]) for _ in range(n)]
            else:
                f = rng.uniform(-1, 1, m).astype(np.float32)
                xs = []
                for _ in range(n):
                    f = rng.uniform(0.5, 1.5, m).astype(np.float32) if op == "prod" else \
                        rng.uniform(-1, 1, m).astype(np.float32)
                    f = np.where(rng.random(m) < 0.2, np.float32(0.0) * np.sign(f), f).astype(np.float32)
                    xs.append((f.view(np.uint32) >> np.uint32(16)).astype(np.uint16) if dtype == "bfloat16" else f)
            want = H.allreduce(xs, op, dtype)[0]
            got = R.narrow(R.finalize(op, H.butterfly_fold(xs, op, dtype), n), dtype)
            assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), (n, m)


def test_butterfly_fold_is_neither_ascending_nor_ring_order():
    """At N = 16 the tree differs from the ascending fold and from every
    ring chunk order somewhere (float32 SUM), and stays within the
    summation bound."""
    from oracle import ring as G
    n, m = 16, 4096
    rng = np.random.default_rng(15)
    xs = [rng.uniform(-1, 1, m).astype(np.float32) for _ in range(n)]
    got = H.butterfly_fold(xs, "sum", "float32")
    for order in [list(range(n))] + [G.chunk_order(n, c) for c in range(n)]:
        assert not np.array_equal(C.fold(xs, "sum", "float32", order).view(np.uint32), got.view(np.uint32))
    assert R.normalized_sum_error(got, xs, "float32") <= (n - 1) * 2.0 ** -24


def test_butterfly_fold_rejects_non_powers_of_two():
    with pytest.raises(ValueError):
        H.butterfly_fold([np.zeros(3, np.float32)] * 6, "sum", "float32")
