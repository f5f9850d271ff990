"""Seeded synthetic rank buffers, shared by the tests, the bench and the oracle.

This module draws numbers and nothing else: it holds none of the
collectives' arithmetic (no ⊕, no padding, no rounding of results).  The
same call returns the same values on any machine, so the oracle and the HIP
path see identical inputs.

Every workload names N virtual ranks, M elements per rank, a dtype and a
value distribution.  Values are produced per (rank, chunk of 2^20 elements)
from ``numpy.random.default_rng([1234, workload_id, stream, rank, chunk])``,
so any slice of any rank can be regenerated on its own and host memory stays
bounded for the 1 GiB-per-rank buffers.

Distributions
-------------
* ``affine``: x^(r)_i = a·r + i exactly (the four-rank, 20-element int64
  worked example uses a = 100).
* ``uniform``: float64 uniform on [lo, hi), cast to float32 (NumPy's cast
  rounds to nearest even).
* ``normal``: float64 normal(0, sigma), cast to float32.
* ``int_uniform``: integers uniform on [lo, hi], both ends included.
* bf16 buffers are float32 draws with the low 16 bits cleared, so every
  value is exactly representable; they are returned as uint16 bit patterns.
"""

import numpy as np

CHUNK = 1 << 20

# name -> parameters.  ``wid`` separates the seed spaces of the workloads.
WORKLOADS = {
    "worked_example_4x20_int64": dict(wid=0, nranks=4, count=20, dtype="int64", dist="affine", a=100),
    "uniform_8x1048576_fp32": dict(wid=1, nranks=8, count=1 << 20, dtype="float32", dist="uniform", lo=-1.0, hi=1.0),
    "normal_8x1000003_fp32": dict(wid=2, nranks=8, count=1_000_003, dtype="float32", dist="normal", sigma=1.0),
    "intuniform_8x1000003_int32": dict(wid=2, stream=1, nranks=8, count=1_000_003, dtype="int32",
                                       dist="int_uniform", lo=-(1 << 20), hi=1 << 20),
    "normal_256x4194304_fp32": dict(wid=3, nranks=256, count=1 << 22, dtype="float32", dist="normal", sigma=1e-3),
    "normal_256x6553600_bf16": dict(wid=3, stream=1, nranks=256, count=6_553_600, dtype="bfloat16",
                                    dist="normal", sigma=1e-3),
    "uniform_8x268435456_fp32": dict(wid=4, nranks=8, count=1 << 28, dtype="float32", dist="uniform",
                                     lo=-1.0, hi=1.0),
}

_STORAGE = {"int32": np.int32, "int64": np.int64, "float32": np.float32, "bfloat16": np.uint16}


def spec(name, **overrides):
    """Parameters of a named workload, optionally with fields replaced
    (e.g. a smaller ``count`` or ``nranks`` of the same distribution)."""
    s = dict(WORKLOADS[name])
    s.update(overrides)
    s.setdefault("stream", 0)
    return s


def _draw_chunk(s, rank, chunk, dtype_override=None):
    dtype = dtype_override or s["dtype"]
    lo_i = chunk * CHUNK
    hi_i = min(lo_i + CHUNK, s["count"])
    n = hi_i - lo_i
    dist = s["dist"]
    if dist == "affine":
        vals = s["a"] * rank + np.arange(lo_i, hi_i, dtype=np.int64)
        return vals.astype(_STORAGE[dtype])
    rng = np.random.default_rng([1234, s["wid"], s["stream"], rank, chunk])
    if dist == "uniform":
        f = rng.uniform(s["lo"], s["hi"], n).astype(np.float32)
    elif dist == "normal":
        f = (rng.standard_normal(n) * s["sigma"]).astype(np.float32)
    elif dist == "int_uniform":
        return rng.integers(s["lo"], s["hi"], size=n, endpoint=True, dtype=np.int64).astype(_STORAGE[dtype])
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    if dtype == "bfloat16":
        return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    if dtype == "float32":
        return f
    raise ValueError(f"distribution {dist!r} does not produce {dtype}")


def rank_buffer(s, rank, start=0, stop=None, workers=1):
    """Elements [start, stop) of rank ``rank``'s buffer for workload spec ``s``.

    ``workers`` > 1 draws the chunks on that many threads (NumPy's generators
    release the GIL while filling); the values do not depend on it.
    """
    count = s["count"]
    stop = count if stop is None else min(stop, count)
    out = np.empty(max(stop - start, 0), dtype=_STORAGE[s["dtype"]])
    if start >= stop:
        return out
    chunks = list(range(start // CHUNK, (stop - 1) // CHUNK + 1))

    def fill(c):
        block = _draw_chunk(s, rank, c)
        base = c * CHUNK
        lo, hi = max(start, base), min(stop, base + block.size)
        out[lo - start:hi - start] = block[lo - base:hi - base]

    if workers > 1 and len(chunks) > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(min(workers, len(chunks))) as ex:
            list(ex.map(fill, chunks))
    else:
        for c in chunks:
            fill(c)
    return out


def all_buffers(s):
    """All N rank buffers as one (N, M) array (small workloads only)."""
    return np.stack([rank_buffer(s, r) for r in range(s["nranks"])])


def gather_positions(s, positions):
    """x^(r)_i for every rank r at the given global positions: an (N, k)
    array built by regenerating only the chunks those positions fall in."""
    positions = np.asarray(positions, dtype=np.int64)
    out = np.empty((s["nranks"], positions.size), dtype=_STORAGE[s["dtype"]])
    chunks = positions // CHUNK
    for c in np.unique(chunks):
        sel = np.nonzero(chunks == c)[0]
        local = positions[sel] - c * CHUNK
        for r in range(s["nranks"]):
            out[r, sel] = _draw_chunk(s, r, int(c))[local]
    return out
