"""The ring schedule, stepped literally rank by rank (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

Routing ([RING] §1 流程, the N=4 table of §2 and the pseudocode under
"展开：伪代码 + 实测数据"; [PRIMS] §五.2 and §五.3; [WHY-EQ] §5 and §6):

* Ranks form a ring; rank r sends only to r+1 and receives only from r-1
  (indices mod N).  Each rank's buffer is cut into N chunks of q elements;
  chunk c covers global indices [c·q, (c+1)·q).
* ReduceScatter phase, steps t = 0..N-2: rank r sends its current partial of
  chunk (r - t) and receives chunk (r - 1 - t), which it combines into its
  own copy of that chunk.  After N-1 steps rank r holds the complete
  reduction of chunk (r + 1) mod N.
* AllGather phase, steps t = 0..N-2: rank r sends chunk (r + 1 - t) and
  receives chunk (r - t), overwriting its copy (no reduction).

[RS-PAGE] §Ring ReduceScatter has node i send chunk i+1 (mod N) at step 1,
which contradicts the ownership the same section states (node 0 ends with
chunk 1); the routing above is the one the other four pages agree on.

All sends of a step are taken before any receive of that step is applied,
which is what non-blocking send/recv followed by a wait means ([RING]: a
blocking send-then-receive ring would deadlock).

Combining order.  The incoming partial is the left operand:
b_r[c] <- incoming ⊕ b_r[c].  Chunk c is therefore folded as
x^(c), x^(c+1), ..., x^(c-1) (ranks mod N), starting at its origin rank c and
ending at rank c-1, which owns it ([WHY-EQ] §5 shows chunk 0 built up as
a0+b0, then +c0, then +d0, ending on the last GPU).  For SUM and PROD the
operand order within one ⊕ does not change a binary32 result; it only
decides which of +0 / -0 a MAX / MIN tie keeps.

Rank-major result.  The ring leaves chunk (n+1) on ring rank n; the
ReduceScatter contract puts shard r on rank r.  The reading taken: one ring
(the routing above) serves ring AllReduce, ring ReduceScatter and ring
AllGather, and ring rank n's completed chunk (n+1) mod N is delivered as
output shard (n+1) mod N.  [PRIMS] §五.2 notes the ownership is rotated
without affecting what follows.

bf16: partials travel in float32 and are rounded to bf16 once, when the
completed chunk is stored.
"""

import numpy as np

from . import reduction as R
from .collectives import check_capacity, shard_count, pad_identity


def reduce_scatter_route(nranks, step, rank):
    """(send_chunk, recv_chunk) of ``rank`` at ReduceScatter step ``step``."""
    return (rank - step) % nranks, (rank - 1 - step) % nranks


def all_gather_route(nranks, step, rank, owner_offset=1):
    """(send_chunk, recv_chunk) at AllGather step ``step``.

    ``owner_offset`` is the chunk a rank holds complete before the phase,
    relative to its own index: 1 after the ring ReduceScatter phase (rank r
    owns chunk r+1), 0 for a stand-alone AllGather whose rank r starts with
    shard r.
    """
    return (rank + owner_offset - step) % nranks, (rank + owner_offset - 1 - step) % nranks


def ring_owner(nranks, rank):
    """Chunk a ring rank holds complete after the ReduceScatter phase."""
    return (rank + 1) % nranks


def chunk_order(nranks, chunk):
    """Ranks in the order the ring folds chunk ``chunk``: c, c+1, ..., c-1."""
    return [(chunk + k) % nranks for k in range(nranks)]


def _chunk(q, c):
    return slice(c * q, (c + 1) * q)


def _rs_phase(bufs, op, q, record):
    """Run the N-1 ReduceScatter steps in place on accumulator buffers."""
    n = len(bufs)
    states = []
    for t in range(n - 1):
        sent = []
        for r in range(n):
            send_c, _ = reduce_scatter_route(n, t, r)
            sent.append(bufs[r][_chunk(q, send_c)].copy())
        for r in range(n):
            _, recv_c = reduce_scatter_route(n, t, r)
            incoming = sent[(r - 1) % n]
            sl = _chunk(q, recv_c)
            bufs[r][sl] = R.combine(op, incoming, bufs[r][sl])
        if record:
            states.append([b.copy() for b in bufs])
    return states


def _ag_phase(bufs, q, owner_offset, record):
    """Run the N-1 AllGather steps in place (copy, no reduction)."""
    n = len(bufs)
    states = []
    for t in range(n - 1):
        sent = []
        for r in range(n):
            send_c, _ = all_gather_route(n, t, r, owner_offset)
            sent.append(bufs[r][_chunk(q, send_c)].copy())
        for r in range(n):
            _, recv_c = all_gather_route(n, t, r, owner_offset)
            bufs[r][_chunk(q, recv_c)] = sent[(r - 1) % n]
        if record:
            states.append([b.copy() for b in bufs])
    return states


def ring_allreduce(xs, op, dtype, record=False):
    """Ring AllReduce: pad to N·q with the identity, 2(N-1) steps, trim.

    Returns the N outputs (each M elements).  With ``record`` it also returns
    the per-step state: a list of 2(N-1) snapshots, each the N padded
    buffers (ReduceScatter snapshots in accumulator type, AllGather snapshots
    in stored type).
    """
    n = len(xs)
    m = np.asarray(xs[0]).size
    q = shard_count(m, n)
    padded = pad_identity(xs, op, dtype, n * q)
    bufs = [R.widen(x, dtype) for x in padded]
    rs_states = _rs_phase(bufs, op, q, record)
    stored = []
    for owner, b in enumerate(bufs):
        b = b.copy()
        sl = _chunk(q, ring_owner(n, owner))
        b[sl] = R.finalize(op, b[sl], n)   # the completed chunk gets the post-operation
        stored.append(R.narrow(b, dtype))
    ag_states = _ag_phase(stored, q, 1, record)
    outs = [b[:m].copy() for b in stored]
    if record:
        return outs, rs_states + ag_states
    return outs


def ring_reduce_scatter(xs, op, dtype, recvcount, record=False):
    """Ring ReduceScatter with sendcount = N·recvcount.

    Output shard c is the complete chunk c, which ring rank (c-1) mod N
    holds after the N-1 steps.
    """
    n = len(xs)
    for x in xs:
        check_capacity(np.asarray(x).size, n, recvcount)
    q = recvcount
    bufs = [R.widen(x, dtype) for x in xs]
    states = _rs_phase(bufs, op, q, record)
    shards = [None] * n
    for owner in range(n):
        c = ring_owner(n, owner)
        shards[c] = R.narrow(R.finalize(op, bufs[owner][_chunk(q, c)], n), dtype)
    if record:
        return shards, states
    return shards


def ring_all_gather(shards, recvcount=None, record=False):
    """Ring AllGather: rank r starts with shard r, N-1 copy steps, trim."""
    n = len(shards)
    q = np.asarray(shards[0]).size
    total = n * q
    if recvcount is None:
        recvcount = total
    if recvcount > total:
        raise TypeError("recvcount exceeds nranks * sendcount")
    bufs = []
    for r in range(n):
        b = np.zeros(total, dtype=np.asarray(shards[r]).dtype)
        b[_chunk(q, r)] = shards[r]
        bufs.append(b)
    states = _ag_phase(bufs, q, 0, record)
    outs = [b[:recvcount].copy() for b in bufs]
    if record:
        return outs, states
    return outs


def step_counts(nranks):
    """Steps per collective: RS N-1, AG N-1, AR 2(N-1)."""
    return {"reduce_scatter": nranks - 1, "all_gather": nranks - 1, "allreduce": 2 * (nranks - 1)}
