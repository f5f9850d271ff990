"""Recursive-halving ReduceScatter and recursive-doubling AllGather (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

[RS-PAGE] §Recursive Halving ReduceScatter: for N = 2^k ranks the
ReduceScatter takes log2 N steps.  At step j (1-based) rank i pairs with
rank i XOR N/2^j and the pair exchanges M/2^j elements: for N = 8 the pairs
are (0,4)(1,5)(2,6)(3,7), then (0,2)(1,3)(4,6)(5,7), then (0,1)(2,3)(4,5)(6,7),
and each rank ends with M/N fully reduced elements.  The page calls it the
dual of recursive-doubling AllGather, which undoes the halving in reverse.

Readings where the page is silent:

* Which half a rank keeps: the rank whose bit N/2^j is clear keeps the lower
  half of the range the pair shares, the other the upper half.  Rank i then
  ends holding block i, so the result is rank-major with no relabelling.
* Combining order: the pair combines as (lower rank's partial) ⊕ (upper
  rank's partial), so block b is reduced as a butterfly tree; for N = 8:
  ((x0⊕x4)⊕(x2⊕x6))⊕((x1⊕x5)⊕(x3⊕x7)).
* Partials travel in the accumulator type (float32 for bf16) and the AVG
  division and the bf16 rounding happen once, at the final store.
* N must be a power of two; M is padded to N·q with the identity and the
  padding is trimmed, as in the other schedules.
"""

import numpy as np

from . import reduction as R
from .collectives import check_capacity, shard_count, pad_identity


def _check_pow2(n):
    if n < 1 or (n & (n - 1)) != 0:
        raise ValueError("recursive halving needs a power-of-two number of ranks")
    return n.bit_length() - 1


def halving_pairs(nranks):
    """Pairs of each step: [[(i, i ^ d) for i < i ^ d] for d = N/2, N/4, ..., 1]."""
    k = _check_pow2(nranks)
    steps = []
    for j in range(1, k + 1):
        d = nranks >> j
        steps.append([(i, i ^ d) for i in range(nranks) if i < (i ^ d)])
    return steps


def kept_range(nranks, q, step, rank):
    """Element range [lo, hi) rank ``rank`` holds after halving step ``step``
    (step 0 = the whole padded buffer)."""
    lo, length = 0, nranks * q
    for j in range(1, step + 1):
        d = nranks >> j
        length //= 2
        if rank & d:
            lo += length
    return lo, lo + length


def _rh_phase(bufs, op, q, record):
    """The log2 N halving steps, rank by rank, on full-length accumulator
    buffers; after the last step rank i's block i is complete."""
    n = len(bufs)
    k = _check_pow2(n)
    states = []
    for j in range(1, k + 1):
        d = n >> j
        new = [b.copy() for b in bufs]
        for i in range(n):
            p = i ^ d
            lo, hi = kept_range(n, q, j, i)
            low, up = (i, p) if i < p else (p, i)
            new[i][lo:hi] = R.combine(op, bufs[low][lo:hi], bufs[up][lo:hi])
        bufs[:] = new
        if record:
            states.append([b.copy() for b in bufs])
    return states


def _rd_phase(bufs, q, record):
    """The log2 N doubling steps: rank i receives its partner's gathered
    blocks and copies them into place."""
    n = len(bufs)
    k = _check_pow2(n)
    states = []
    for t in range(k):
        d = 1 << t
        new = [b.copy() for b in bufs]
        for i in range(n):
            p = i ^ d
            lo = ((p >> t) << t) * q
            hi = (((p >> t) + 1) << t) * q
            new[i][lo:hi] = bufs[p][lo:hi]
        bufs[:] = new
        if record:
            states.append([b.copy() for b in bufs])
    return states


def butterfly_fold(xs, op, dtype):
    """The combining tree of the halving phase, applied to whole arrays.

    Every block is reduced by the same tree (see the module docstring): the
    first step pairs rank i with rank i + N/2, the next pairs those partials
    at distance N/4, and so on down to distance 1, the partial of the lower
    rank always on the left.  Returns the accumulator of that tree at every
    position (before AVG's division and bf16 rounding), so that a result
    can be checked at any length without stepping the ranks.
    """
    n = len(xs)
    _check_pow2(n)
    acc = [R.widen(x, dtype) for x in xs]
    d = n // 2
    while d >= 1:
        acc = [R.combine(op, acc[i], acc[i + d]) for i in range(d)]
        d //= 2
    return acc[0]


def reduce_scatter(xs, op, dtype, recvcount, record=False):
    """Recursive-halving ReduceScatter with sendcount = N·recvcount."""
    n = len(xs)
    for x in xs:
        check_capacity(np.asarray(x).size, n, recvcount)
    q = recvcount
    bufs = [R.widen(x, dtype) for x in xs]
    states = _rh_phase(bufs, op, q, record)
    shards = [R.narrow(R.finalize(op, bufs[i][i * q:(i + 1) * q], n), dtype) for i in range(n)]
    return (shards, states) if record else shards


def all_gather(shards, recvcount=None, record=False):
    """Recursive-doubling AllGather: rank r starts with shard r."""
    n = len(shards)
    q = np.asarray(shards[0]).size
    total = n * q
    recvcount = total if recvcount is None else recvcount
    if recvcount > total:
        raise TypeError("recvcount exceeds nranks * sendcount")
    bufs = []
    for r in range(n):
        b = np.zeros(total, dtype=np.asarray(shards[r]).dtype)
        b[r * q:(r + 1) * q] = shards[r]
        bufs.append(b)
    states = _rd_phase(bufs, q, record)
    outs = [b[:recvcount].copy() for b in bufs]
    return (outs, states) if record else outs


def allreduce(xs, op, dtype, record=False):
    """Pad, recursive-halving ReduceScatter, recursive-doubling AllGather, trim."""
    n = len(xs)
    m = np.asarray(xs[0]).size
    q = shard_count(m, n)
    padded = pad_identity(xs, op, dtype, n * q)
    bufs = [R.widen(x, dtype) for x in padded]
    rs_states = _rh_phase(bufs, op, q, record)
    stored = []
    for i, b in enumerate(bufs):
        b = b.copy()
        b[i * q:(i + 1) * q] = R.finalize(op, b[i * q:(i + 1) * q], n)
        stored.append(R.narrow(b, dtype))
    ag_states = _rd_phase(stored, q, record)
    outs = [b[:m].copy() for b in stored]
    return (outs, rs_states + ag_states) if record else outs
