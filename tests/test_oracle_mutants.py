"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
in ``test_oracle_pins.py`` catch every one of them.

Each mutant replaces one oracle function with a subtly wrong version (a
dropped term, a wrong index, a swapped operand, a zero pad, a truncating
rounding) and re-runs a set of pins; the mutant must make at least one pin
fail.  This shows the pins are sensitive to the mistakes they are meant to
exclude, rather than passing for any implementation.
"""

import json
import os

import numpy as np
import pytest

import test_oracle_pins as P
import test_oracle_recursive as Q
from oracle import collectives as C
from oracle import recursive as H
from oracle import reduction as R
from oracle import ring as G

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


PINS = [
    lambda: P.test_worked_example_all_routes(_golden),
    lambda: P.test_worked_example_negatives_differ_everywhere(_golden),
    lambda: P.test_padding_and_trim_equivalence_1003(_golden),
    lambda: P.test_padded_tail_is_identity_bits("float32", "max", 0xFF800000),
    lambda: P.test_padded_tail_is_identity_int("int32", "max", -2**31),
    lambda: P.test_max_padding_must_not_be_zero(),
    lambda: P.test_ring_routing_table_n4(_golden),
    lambda: P.test_ring_round_sums_in_order(_golden),
    lambda: P.test_ring_staircase_n4(_golden),
    lambda: P.test_ring_onehot_bitmasks(),
    lambda: P.test_ring_allgather_grid_n4(_golden),
    lambda: P.test_closed_forms("int32", 5, 17, 1000),
    lambda: P.test_closed_forms("int64", 8, 29, 12345),
    lambda: P.test_fp32_orders_match_scalar_twin_bitwise(8),
    lambda: P.test_fp32_ring_fold_matches_chunk_order(),
    lambda: P.test_bf16_rounding_cases(),
    lambda: P.test_gradient_like_256_ranks_tolerance(),
    lambda: P.test_avg_is_the_sum_divided_once(),
    lambda: P.test_normalized_sum_error_by_hand(),
    lambda: Q.test_pair_table_and_volumes(_golden),
    lambda: Q.test_onehot_partials_cover_the_pair_groups(),
    lambda: Q.test_brute_force_integers(),
    lambda: Q.test_butterfly_order_float32(),
    lambda: Q.test_max_ties_keep_the_lower_ranks_partial(),
    lambda: Q.test_doubling_all_gather_and_trim(),
    lambda: Q.test_butterfly_fold_is_the_bracketed_tree(),
    lambda: Q.test_butterfly_fold_matches_the_stepped_ranks("float32", "max"),
]


def _caught():
    for pin in PINS:
        try:
            pin()
        except (AssertionError, TypeError, ValueError, IndexError):
            return True
    return False


def test_unmutated_oracle_passes_every_pin():
    assert not _caught()


def _fold_descending(xs, op, dtype, order):
    return _ORIG_FOLD(xs, op, dtype, list(reversed(order)))


def _fold_drop_last(xs, op, dtype, order):
    return _ORIG_FOLD(xs, op, dtype, order[:-1] if len(order) > 1 else order)


def _rs_route_off_by_one(nranks, step, rank):
    return (rank - step) % nranks, (rank - step) % nranks


def _ag_route_wrong(nranks, step, rank, owner_offset=1):
    return (rank + owner_offset - step) % nranks, (rank + owner_offset - step) % nranks


def _gather_reversed(shards, recvcount=None):
    return _ORIG_GATHER(list(reversed(shards)), recvcount)


def _identity_zero(op, dtype):
    return R.ACCUM[dtype].type(0)


def _combine_swapped_max(op, a, b):
    if op == "max":
        return np.where(b < a, b, a)
    return _ORIG_COMBINE(op, a, b)


def _combine_right_operand(op, a, b):
    return _ORIG_COMBINE(op, b, a)


def _round_truncate(f):
    return (np.asarray(f, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _owner_same_rank(nranks, rank):
    return rank


def _finalize_floor(op, acc, nranks):
    if op == "avg" and np.asarray(acc).dtype.kind == "i":
        return (np.asarray(acc) // nranks).astype(np.asarray(acc).dtype)
    return _ORIG_FINALIZE(op, acc, nranks)


def _finalize_by_n_minus_1(op, acc, nranks):
    return _ORIG_FINALIZE(op, acc, nranks - 1 if nranks > 1 else 1)


def _halving_pairs_doubling_distance(nranks):
    k = nranks.bit_length() - 1
    return [[(i, i ^ (1 << (j - 1))) for i in range(nranks) if i < (i ^ (1 << (j - 1)))] for j in range(1, k + 1)]


def _kept_range_swapped(nranks, q, step, rank):
    lo, length = 0, nranks * q
    for j in range(1, step + 1):
        length //= 2
        if not rank & (nranks >> j):
            lo += length
    return lo, lo + length


def _rh_phase_upper_left(bufs, op, q, record):
    n = len(bufs)
    states = []
    for j in range(1, n.bit_length()):
        d = n >> j
        new = [b.copy() for b in bufs]
        for i in range(n):
            p = i ^ d
            lo, hi = H.kept_range(n, q, j, i)
            low, up = (i, p) if i < p else (p, i)
            new[i][lo:hi] = R.combine(op, bufs[up][lo:hi], bufs[low][lo:hi])
        bufs[:] = new
        if record:
            states.append([b.copy() for b in bufs])
    return states


def _rd_phase_own_block(bufs, q, record):
    n = len(bufs)
    states = []
    for t in range(n.bit_length() - 1):
        new = [b.copy() for b in bufs]
        for i in range(n):
            p = i ^ (1 << t)
            lo = ((i >> t) << t) * q
            hi = (((i >> t) + 1) << t) * q
            new[i][lo:hi] = bufs[p][lo:hi]
        bufs[:] = new
        if record:
            states.append([b.copy() for b in bufs])
    return states


def _error_over_abs_of_sum(y, xs, dtype):
    ref = R.fp64_reference(xs, dtype)
    got = R.widen(y, dtype).astype(np.float64)
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), np.finfo(np.float64).tiny)))


def _butterfly_adjacent_pairs(xs, op, dtype):
    acc = [R.widen(x, dtype) for x in xs]
    while len(acc) > 1:
        acc = [R.combine(op, acc[2 * i], acc[2 * i + 1]) for i in range(len(acc) // 2)]
    return acc[0]


def _butterfly_upper_left(xs, op, dtype):
    acc = [R.widen(x, dtype) for x in xs]
    d = len(acc) // 2
    while d >= 1:
        acc = [R.combine(op, acc[i + d], acc[i]) for i in range(d)]
        d //= 2
    return acc[0]


_ORIG_FOLD = C.fold
_ORIG_GATHER = C.all_gather
_ORIG_COMBINE = R.combine
_ORIG_FINALIZE = R.finalize

MUTANTS = {
    "fold in descending rank order": (C, "fold", _fold_descending),
    "fold drops the last rank": (C, "fold", _fold_drop_last),
    "ring RS receives the chunk it sends": (G, "reduce_scatter_route", _rs_route_off_by_one),
    "ring AG receives the chunk it sends": (G, "all_gather_route", _ag_route_wrong),
    "AllGather concatenates in reverse rank order": (C, "all_gather", _gather_reversed),
    "identity is a mechanical zero": (R, "identity", _identity_zero),
    "MAX computes MIN": (R, "combine", _combine_swapped_max),
    "incoming partial is the right operand": (R, "combine", _combine_right_operand),
    "bf16 rounding truncates": (R, "bf16_round_bits", _round_truncate),
    "ring owner is the rank itself": (G, "ring_owner", _owner_same_rank),
    "integer AVG rounds toward minus infinity": (R, "finalize", _finalize_floor),
    "AVG divides by N-1": (R, "finalize", _finalize_by_n_minus_1),
    "halving pairs at the doubling distances": (H, "halving_pairs", _halving_pairs_doubling_distance),
    "halving keeps the other half": (H, "kept_range", _kept_range_swapped),
    "halving combines upper rank on the left": (H, "_rh_phase", _rh_phase_upper_left),
    "doubling copies the receiver's own block": (H, "_rd_phase", _rd_phase_own_block),
    "tolerance measure divides by |sum| instead of sum of |x|": (R, "normalized_sum_error", _error_over_abs_of_sum),
    "butterfly fold pairs neighbouring ranks first": (H, "butterfly_fold", _butterfly_adjacent_pairs),
    "butterfly fold puts the upper rank on the left": (H, "butterfly_fold", _butterfly_upper_left),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    module, attr, fn = MUTANTS[name]
    monkeypatch.setattr(module, attr, fn)
    # modules that imported the name directly see the mutant too
    if module is C and attr in ("fold", "all_gather"):
        monkeypatch.setattr(P.C, attr, fn)
    assert _caught(), f"no pin caught the mutant: {name}"
