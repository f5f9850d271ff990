"""The reduction operator ⊕, its identities, and bf16 rounding (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

[PRIMS] §二.1 lists the reduction operators sum, max, min, prod and avg.
[DECOMP] §等价成立的条件, condition three, fixes two identities: 0 for SUM
and "negative infinity or the dtype's minimum" for MAX, never a mechanical 0.
The identities of PROD (1) and MIN (+inf / dtype maximum) are not printed on
the pages; they are the plain readings of "identity of the reduction".

AVG is a SUM fold followed by one division by N when the final result is
stored (the postOp flag on the last reduce of [DECOMP] §源码三 / §源码四).
Reading taken for its details: float32 and bf16 divide the float32 sum by
N with one correctly rounded binary32 division; integers divide the
(wrapped) sum by N truncating toward zero, as C's integer division does.
Its padding identity is SUM's, 0.

Representation
--------------
* int32 / int64: NumPy ints.  SUM and PROD wrap modulo 2^32 / 2^64
  (two's complement); [DECOMP] condition five only promises exactness
  "without overflow", wraparound is the reading taken for the overflow case.
* float32: NumPy float32; every ⊕ is one IEEE-754 binary32 operation rounded
  to nearest even.
* bfloat16: stored as uint16 bit patterns.  Values are widened exactly to
  float32 (bits << 16), combined in float32, and rounded back to bf16 once,
  when a final result is stored (fp32 accumulation).

MAX / MIN tie rule: max(a, b) = b if b > a else a (the first operand wins a
tie, which only matters for +0 / -0).  NaN inputs are out of scope.
"""

import numpy as np

DTYPES = ("int32", "int64", "float32", "bfloat16")
OPS = ("sum", "prod", "max", "min", "avg")

# NumPy dtype that holds one stored element.
STORAGE = {
    "int32": np.dtype(np.int32),
    "int64": np.dtype(np.int64),
    "float32": np.dtype(np.float32),
    "bfloat16": np.dtype(np.uint16),
}
# NumPy dtype the combine runs in.
ACCUM = {
    "int32": np.dtype(np.int32),
    "int64": np.dtype(np.int64),
    "float32": np.dtype(np.float32),
    "bfloat16": np.dtype(np.float32),
}


def _check(op, dtype):
    if op not in OPS:
        raise ValueError(f"unknown op {op!r}")
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")


def identity(op, dtype):
    """Identity of ⊕ in the accumulator type ([DECOMP] condition three)."""
    _check(op, dtype)
    acc = ACCUM[dtype]
    if op in ("sum", "avg"):
        return acc.type(0)
    if op == "prod":
        return acc.type(1)
    if acc.kind == "f":
        return acc.type(-np.inf) if op == "max" else acc.type(np.inf)
    info = np.iinfo(acc)
    return acc.type(info.min) if op == "max" else acc.type(info.max)


def identity_storage(op, dtype):
    """Identity as one stored element (bf16: its bit pattern)."""
    v = np.array([identity(op, dtype)], dtype=ACCUM[dtype])
    return narrow(v, dtype)[0]


def widen(x, dtype):
    """Stored elements -> accumulator values.  bf16 widening is exact."""
    x = np.asarray(x, dtype=STORAGE[dtype])
    if dtype == "bfloat16":
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return x.copy()


def bf16_round_bits(f):
    """float32 values -> bf16 bit patterns, round to nearest, ties to even.

    The upper 16 bits are kept; the discarded lower 16 bits decide: above
    half (0x8000) rounds up, below half truncates, exactly half rounds to the
    even upper pattern.  A carry out of the mantissa moves into the exponent,
    which turns the largest finite values into infinity as IEEE rounding
    requires.  NaNs keep their sign and upper payload and are made quiet.
    """
    bits = np.asarray(f, dtype=np.float32).view(np.uint32)
    upper = (bits >> np.uint32(16)).astype(np.uint32)
    lower = bits & np.uint32(0xFFFF)
    round_up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    out = upper + round_up.astype(np.uint32)
    is_nan = ((bits & np.uint32(0x7F800000)) == 0x7F800000) & ((bits & np.uint32(0x7FFFFF)) != 0)
    out = np.where(is_nan, upper | np.uint32(0x0040), out)
    return out.astype(np.uint16)


def narrow(acc, dtype):
    """Accumulator values -> stored elements (bf16: one RNE rounding)."""
    if dtype == "bfloat16":
        return bf16_round_bits(acc)
    return np.asarray(acc, dtype=STORAGE[dtype]).copy()


def combine(op, a, b):
    """One application of ⊕ elementwise: a ⊕ b, a the running partial.

    Both operands are accumulator arrays of one dtype.  Integer SUM / PROD
    wrap (NumPy array arithmetic is modular); float32 SUM / PROD are single
    IEEE binary32 operations.
    """
    if op in ("sum", "avg"):
        return np.add(a, b, dtype=a.dtype)
    if op == "prod":
        return np.multiply(a, b, dtype=a.dtype)
    if op == "max":
        return np.where(b > a, b, a)
    if op == "min":
        return np.where(b < a, b, a)
    raise ValueError(f"unknown op {op!r}")


def finalize(op, acc, nranks):
    """The post-operation applied once to a completed reduction: AVG divides
    by N (float: one binary32 division; integer: truncation toward zero);
    every other op leaves the value as it is."""
    if op != "avg":
        return acc
    acc = np.asarray(acc)
    if acc.dtype.kind == "f":
        return np.divide(acc, acc.dtype.type(nranks), dtype=acc.dtype)
    q = acc // nranks                      # floor division ...
    rem = acc - q * nranks
    return np.where((rem != 0) & (acc < 0), q + 1, q).astype(acc.dtype)  # ... turned toward zero


def fp64_reference(xs, dtype):
    """Σ_s x^(s)_i in float64 for floating inputs (the tolerance reference).

    ``xs`` is a sequence of N stored arrays.  Values are widened exactly and
    summed in float64, rank by rank; with N <= 1024 and |x| <= 1 the float64
    rounding error is below 2^-42 relative, far under any tolerance used.
    """
    acc = np.zeros(np.asarray(xs[0]).shape, dtype=np.float64)
    for x in xs:
        acc += widen(x, dtype).astype(np.float64)
    return acc


def abs_sum64(xs, dtype):
    """Σ_s |x^(s)_i| in float64: the scale of the summation error bound."""
    acc = np.zeros(np.asarray(xs[0]).shape, dtype=np.float64)
    for x in xs:
        acc += np.abs(widen(x, dtype).astype(np.float64))
    return acc


def normalized_sum_error(y, xs, dtype):
    """max_i |y_i - Σ_s x^(s)_i| / max(Σ_s |x^(s)_i|, tiny).

    The forward-error normalisation of recursive summation: any order of N
    binary32 additions stays within about (N-1)·2^-24 of this bound, so the
    measure does not blow up where the sum cancels to nearly zero.
    """
    ref = fp64_reference(xs, dtype)
    scale = np.maximum(abs_sum64(xs, dtype), np.finfo(np.float64).tiny)
    got = widen(y, dtype).astype(np.float64)
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) / scale))
