"""CPU model of the chained recursive driver's walk order.

The chained recursive kernel visits the halving tree of block b depth first
(step-1 nodes in bit-reversed order of their low bits, each parent as soon
as its second child is done) and fills the ranks of the doubling tree in
the order b XOR bitrev(c), c = 1 .. N-1, each from the rank that differs in
the top bit of bitrev(c).  These tests restate that order in Python and
check, for every power-of-two N up to 256 and every block, that it visits
each node exactly once after both of its operands, that it reproduces the
step-by-step butterfly of the oracle bit for bit, and that every doubling
copy reads a rank that already holds the block.
"""

import numpy as np
import pytest

from oracle import recursive as H


def bitrev(v, bits):
    return 0 if bits == 0 else int(format(v, f"0{bits}b")[::-1], 2)


def halving_walk(n, b):
    """(step j, rank i, partner p) in the order the kernel combines them."""
    k = n.bit_length() - 1
    out = []
    for c in range(n >> 1):
        j, v = 1, c
        while True:
            d = n >> j
            i = (b & ~(d - 1)) | bitrev(v, k - j)
            out.append((j, i, i ^ d))
            if not v & 1:
                break
            v >>= 1
            j += 1
    return out


def doubling_walk(n, b):
    """(receiver, source) in the order the kernel copies block b."""
    k = n.bit_length() - 1
    out = []
    for c in range(1, n):
        x = bitrev(c, k)
        i = b ^ x
        out.append((i, i ^ (1 << (x.bit_length() - 1))))
    return out


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32, 64, 128, 256])
def test_walks_respect_every_dependency(n):
    k = n.bit_length() - 1
    for b in range(n):
        done = {(0, r) for r in range(n)}  # step 0: every rank's own input
        nodes = halving_walk(n, b)
        assert len(nodes) == n - 1
        for j, i, p in nodes:
            # rank i holds block b after step j iff its top j bits equal b's
            assert (i >> (k - j)) == (b >> (k - j))
            assert (j - 1, i) in done and (j - 1, p) in done, (n, b, j, i)
            assert (j, i) not in done
            done.add((j, i))
        assert nodes[-1][:2] == (k, b)  # the root, stored to rank b's output, comes last
        filled = {b}
        for i, src in doubling_walk(n, b):
            assert src in filled and i not in filled, (n, b, i, src)
            # a doubling step t copies between ranks that differ in bit t only
            t = (i ^ src).bit_length() - 1
            assert i ^ src == 1 << t and (i >> (t + 1)) == (b >> (t + 1))
            filled.add(i)
        assert filled == set(range(n))


@pytest.mark.parametrize("n", [2, 4, 8, 16, 64])
def test_depth_first_walk_reproduces_the_butterfly(n):
    """Folding each block in the walk's order, (lower rank) + (upper rank) at
    every node in float32, gives the oracle's step-by-step result bit for
    bit: the walk changes when a node is combined, not its operands."""
    q = 7
    rng = np.random.default_rng(n)
    xs = [rng.uniform(-1, 1, n * q).astype(np.float32) for _ in range(n)]
    want = H.allreduce(xs, "sum", "float32")[0]
    got = np.empty(n * q, np.float32)
    for b in range(n):
        part = {r: xs[r][b * q:(b + 1) * q] for r in range(n)}
        for j, i, p in halving_walk(n, b):
            lo, up = min(i, p), max(i, p)
            part[i] = (part[lo] + part[up]).astype(np.float32)
        got[b * q:(b + 1) * q] = part[b]
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
