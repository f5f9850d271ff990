"""Pure-Python scalar twin of the oracle, for tiny inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

The same definitions as ``collectives`` and ``ring`` ([DECOMP] §数学证明;
[RING] §1 and its pseudocode; [PRIMS] §五), written a second way: one
element at a time, with Python integers and floats instead of NumPy arrays.
It exists so that a slip in the vectorised oracle (a broadcast, a view that
aliases, a dtype that silently widens) shows up as a disagreement on small
brute-force cases.

Values
------
* int32 / int64: Python ints kept in two's-complement range after every ⊕.
* float32: Python floats that are exactly binary32 values.  Each ⊕ is done
  in binary64 and rounded once to binary32; for one addition or
  multiplication of two binary32 operands that double rounding is
  innocuous (53 >= 2·24 + 2), so it equals the correctly rounded binary32
  result.
* bfloat16: Python ints holding the 16-bit pattern; combined as float32 as
  above and rounded back to bf16 by comparing the two neighbouring bf16
  values' distances exactly (ties to the even pattern).
"""

import math
import struct

_BITS = {"int32": 32, "int64": 64}


def _wrap(v, bits):
    v &= (1 << bits) - 1
    return v - (1 << bits) if v >> (bits - 1) else v


def f32(x):
    """Round a Python float to the nearest binary32 value (ties to even)."""
    if math.isnan(x) or math.isinf(x):
        return x
    try:
        return struct.unpack("<f", struct.pack("<f", x))[0]
    except OverflowError:
        return math.copysign(math.inf, x)


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def bits_f32(u):
    return struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]


def bf16_to_f32(h):
    return bits_f32((h & 0xFFFF) << 16)


def _bf16_value(h):
    """Exact value of a bf16 pattern, reading a carried-over exponent of 255
    with zero mantissa as 2^128 (the value rounding compares against)."""
    sign = -1.0 if h & 0x8000 else 1.0
    mag = h & 0x7FFF
    if mag == 0x7F80:
        return sign * 2.0 ** 128
    return bf16_to_f32(h)


def f32_to_bf16(x):
    """binary32 value -> bf16 pattern, nearest, ties to even."""
    if math.isnan(x):
        return ((f32_bits(x) >> 16) | 0x0040) & 0xFFFF
    u = f32_bits(x)
    lo = (u >> 16) & 0xFFFF          # truncated toward zero
    if math.isinf(x) or (u & 0xFFFF) == 0:
        return lo
    hi = (lo + 1) & 0xFFFF           # next pattern away from zero
    d_lo = abs(x - _bf16_value(lo))
    d_hi = abs(_bf16_value(hi) - x)
    if d_lo < d_hi:
        return lo
    if d_hi < d_lo:
        return hi
    return lo if lo % 2 == 0 else hi


def identity(op, dtype):
    if op in ("sum", "avg"):
        return 0.0 if dtype in ("float32", "bfloat16") else 0
    if op == "prod":
        return 1.0 if dtype in ("float32", "bfloat16") else 1
    if dtype in ("float32", "bfloat16"):
        return -math.inf if op == "max" else math.inf
    bits = _BITS[dtype]
    return -(1 << (bits - 1)) if op == "max" else (1 << (bits - 1)) - 1


def widen(v, dtype):
    return bf16_to_f32(v) if dtype == "bfloat16" else v


def narrow(v, dtype):
    return f32_to_bf16(v) if dtype == "bfloat16" else v


def combine(op, a, b, dtype):
    """a ⊕ b for one element; ``a`` is the running partial."""
    if op == "max":
        return b if b > a else a
    if op == "min":
        return b if b < a else a
    if dtype in ("int32", "int64"):
        v = a * b if op == "prod" else a + b
        return _wrap(v, _BITS[dtype])
    v = a * b if op == "prod" else a + b
    return f32(v)


def finalize(op, v, n, dtype):
    """AVG: divide the completed sum by N once (binary32 division, or integer
    division truncating toward zero); other ops unchanged."""
    if op != "avg":
        return v
    if dtype in ("int32", "int64"):
        q = abs(v) // n
        return q if v >= 0 else -q
    return f32(v / n)


def allreduce_direct(xs, op, dtype):
    """xs: N lists of M stored values -> N lists (ascending rank order)."""
    n, m = len(xs), len(xs[0])
    y = []
    for i in range(m):
        acc = widen(xs[0][i], dtype)
        for s in range(1, n):
            acc = combine(op, acc, widen(xs[s][i], dtype), dtype)
        y.append(narrow(finalize(op, acc, n, dtype), dtype))
    return [list(y) for _ in range(n)]


def allreduce_rs_ag(xs, op, dtype):
    """Pad with the identity, ReduceScatter, AllGather, trim."""
    n, m = len(xs), len(xs[0])
    q = -(-m // n)
    ident = narrow(identity(op, dtype), dtype)
    padded = [list(x) + [ident] * (n * q - m) for x in xs]
    shards = []
    for r in range(n):
        z = []
        for j in range(q):
            acc = widen(padded[0][r * q + j], dtype)
            for s in range(1, n):
                acc = combine(op, acc, widen(padded[s][r * q + j], dtype), dtype)
            z.append(narrow(finalize(op, acc, n, dtype), dtype))
        shards.append(z)
    gathered = [v for z in shards for v in z][:m]
    return [list(gathered) for _ in range(n)]


def allreduce_ring(xs, op, dtype):
    """Ring AllReduce, element by element: chunk c folds x^(c), ..., x^(c-1)."""
    n, m = len(xs), len(xs[0])
    q = -(-m // n)
    y = []
    for i in range(m):
        c = i // q
        acc = widen(xs[c][i], dtype)
        for k in range(1, n):
            acc = combine(op, acc, widen(xs[(c + k) % n][i], dtype), dtype)
        y.append(narrow(finalize(op, acc, n, dtype), dtype))
    return [list(y) for _ in range(n)]
