"""Direct AllReduce, ReduceScatter, AllGather, padding and trim (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

Definitions followed ([DECOMP] §数学证明; [RS-PAGE] §语义定义, equation
rs-semantic-output; [PRIMS] §二.1):

* Direct AllReduce: y^(r)_i = ⊕_{s=0}^{N-1} x^(s)_i, the same for every r.
* ReduceScatter, rank-major: with M = N·q, z^(r)_j = ⊕_s x^(s)_{rq+j},
  0 <= j < q.
* AllGather in source-rank order: ŷ^(r)_{sq+j} = z^(s)_j.
* Non-divisible M ([DECOMP] §等价成立的条件, condition three): q = ceil(M/N),
  pad every input to N·q with the op's identity, run RS then AG, trim the
  gathered result back to M.

Combining order.  The pages define ⊕ over the rank set; float ⊕ is not
associative ([DECOMP] condition five), so each schedule has its own order.
Here ``order`` is the explicit sequence of ranks folded left to right:
acc = x^(order[0]); acc = acc ⊕ x^(order[k]) for k = 1..N-1.  The direct
fused schedule folds ranks in ascending order 0, 1, ..., N-1.  The fold never
calls a library reduction along the rank axis (NumPy's pairwise summation
would change the order).

Arrays: each rank's buffer is a 1-D NumPy array of the stored dtype
(bf16 as uint16 bits).  Functions take and return Python lists of such
arrays, one per rank.
"""

import numpy as np

from . import reduction as R


def shard_count(count, nranks):
    """q = ceil(M / N) ([DECOMP] condition three); 0 for an empty buffer."""
    if nranks < 1:
        raise ValueError("nranks must be >= 1")
    if count < 0:
        raise ValueError("count must be >= 0")
    return -(-count // nranks)


def check_capacity(sendcount, nranks, recvcount):
    """The ReduceScatter capacity rule ([DECOMP] §Contract 实验四): a rank's
    input holds exactly one recvcount-element shard per rank, else TypeError."""
    if sendcount != nranks * recvcount:
        raise TypeError(f"sendcount ({sendcount}) != nranks ({nranks}) x recvcount ({recvcount})")


def pad_identity(xs, op, dtype, padded_count):
    """Copy each rank's M elements and fill up to ``padded_count`` with the
    identity of ``op`` ([DECOMP] condition three: the pad value is the
    reduction identity, not a mechanical zero)."""
    out = []
    ident = R.identity_storage(op, dtype)
    for x in xs:
        x = np.asarray(x, dtype=R.STORAGE[dtype])
        if padded_count < x.size:
            raise ValueError("padded_count smaller than count")
        p = np.full(padded_count, ident, dtype=R.STORAGE[dtype])
        p[: x.size] = x
        out.append(p)
    return out


def fold(xs, op, dtype, order):
    """Left fold of ⊕ over the ranks listed in ``order``, in accumulator type."""
    if len(order) == 0:
        raise ValueError("empty rank order")
    acc = R.widen(xs[order[0]], dtype)
    for s in order[1:]:
        acc = R.combine(op, acc, R.widen(xs[s], dtype))
    return acc


def direct_allreduce(xs, op, dtype):
    """Direct AllReduce, ascending rank order; returns N identical outputs."""
    n = len(xs)
    y = R.narrow(R.finalize(op, fold(xs, op, dtype, list(range(n))), n), dtype)
    return [y.copy() for _ in range(n)]


def reduce_scatter(xs, op, dtype, recvcount):
    """Rank-major ReduceScatter with sendcount = N·recvcount (ascending order).

    Raises TypeError, the exception the capacity check in [DECOMP]
    §Contract 实验四 raises, when an input's length is not exactly
    N·recvcount.
    """
    n = len(xs)
    for x in xs:
        check_capacity(np.asarray(x).size, n, recvcount)
    full = R.narrow(R.finalize(op, fold(xs, op, dtype, list(range(n))), n), dtype)
    return [full[r * recvcount:(r + 1) * recvcount].copy() for r in range(n)]


def all_gather(shards, recvcount=None):
    """AllGather in source-rank order, optionally trimmed to ``recvcount``.

    ŷ^(r)_{sq+j} = z^(s)_j for every r; all shards must have the same q.
    A ``recvcount`` below N·q keeps the first ``recvcount`` elements (the
    trim of [DECOMP] §Contract 实验四).
    """
    n = len(shards)
    q = np.asarray(shards[0]).size
    for z in shards:
        if np.asarray(z).size != q:
            raise TypeError("all shards must have the same length")
    total = n * q
    if recvcount is None:
        recvcount = total
    if recvcount > total:
        raise TypeError("recvcount exceeds nranks * sendcount")
    out = np.empty(total, dtype=np.asarray(shards[0]).dtype)
    for s in range(n):
        out[s * q:(s + 1) * q] = shards[s]
    out = out[:recvcount]
    return [out.copy() for _ in range(n)]


def allreduce_via_rs_ag(xs, op, dtype):
    """Pad to N·q with the identity, ReduceScatter, AllGather, trim to M."""
    n = len(xs)
    m = np.asarray(xs[0]).size
    q = shard_count(m, n)
    padded = pad_identity(xs, op, dtype, n * q)
    shards = reduce_scatter(padded, op, dtype, q)
    return all_gather(shards, m)


def roll_shards(y, nranks, shifts):
    """The wrong-order transform of [DECOMP] §等价成立的条件, condition one:
    view the gathered result as N shards and rotate the shard order."""
    y = np.asarray(y)
    return np.roll(y.reshape(nranks, -1), shifts, axis=0).reshape(-1)
