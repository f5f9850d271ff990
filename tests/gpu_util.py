"""Helpers for the GPU parity tests: move NumPy rank buffers to the device,
run the library's collectives through the C-ABI binding, and bring results
back as NumPy arrays in the oracle's representation (bf16 as uint16 bits)."""

import numpy as np
import torch

TORCH = {"int32": torch.int32, "int64": torch.int64, "float32": torch.float32, "bfloat16": torch.bfloat16}
NP = {"int32": np.int32, "int64": np.int64, "float32": np.float32, "bfloat16": np.uint16}
SCHEDULES = ("direct", "ring_stepwise", "ring_persistent", "recursive", "ring_chained", "recursive_chained")


def is_recursive(schedule):
    """Both drivers of recursive halving / doubling (power-of-two N only)."""
    return schedule.startswith("recursive")


def pow2(n):
    return n > 0 and (n & (n - 1)) == 0


def to_dev(x, dtype, device="cuda"):
    x = np.ascontiguousarray(x)
    if dtype == "bfloat16":
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(x).to(device)


def to_host(t, dtype):
    if dtype == "bfloat16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def empty(n, dtype, device="cuda", offset=0):
    """A device buffer of n elements; ``offset`` elements into a larger
    allocation, to test base addresses off a 16-byte boundary."""
    big = torch.empty(n + offset + 8, dtype=TORCH[dtype], device=device)
    return big[offset:offset + n]


def bufs_from(xs, dtype, offset=0):
    out = []
    for x in xs:
        b = empty(len(x), dtype, offset=offset)
        if len(x):
            b.copy_(to_dev(x, dtype))
        out.append(b)
    return out


def workspace(cs, coll, n, m, dtype, schedule):
    return cs.Workspace(coll, n, m, dtype, schedule)


def run_rs(cs, xs, q, op, dtype, schedule, offset=0, in_place=False):
    n = len(xs)
    send = bufs_from(xs, dtype, offset)
    if in_place:
        recv = [send[r][r * q:(r + 1) * q] for r in range(n)]
    else:
        recv = [empty(q, dtype, offset=offset) for _ in range(n)]
    ws = workspace(cs, "reduce_scatter", n, n * q, dtype, schedule)
    cs.ccl_sim_reduce_scatter(send, recv, n * q, q, op=op, schedule=schedule, workspace=ws, dtype=dtype)
    torch.cuda.synchronize()
    return [to_host(r, dtype) for r in recv]


def run_ag(cs, shards, recvcount, dtype, schedule, offset=0, in_place=False):
    n = len(shards)
    q = len(shards[0])
    if in_place:
        recv = [empty(n * q, dtype, offset=offset) for _ in range(n)]
        send = []
        for r in range(n):
            v = recv[r][r * q:(r + 1) * q]
            if q:
                v.copy_(to_dev(shards[r], dtype))
            send.append(v)
        recv = [b[:recvcount] for b in recv]
    else:
        send = bufs_from(shards, dtype, offset)
        recv = [empty(recvcount, dtype, offset=offset) for _ in range(n)]
    ws = workspace(cs, "all_gather", n, recvcount, dtype, schedule)
    cs.ccl_sim_all_gather(send, recv, q, recvcount, schedule=schedule, workspace=ws, dtype=dtype)
    torch.cuda.synchronize()
    return [to_host(r, dtype) for r in recv]


def run_ar(cs, xs, op, dtype, schedule, offset=0, in_place=False):
    n, m = len(xs), len(xs[0])
    send = bufs_from(xs, dtype, offset)
    recv = send if in_place else [empty(m, dtype, offset=offset) for _ in range(n)]
    ws = workspace(cs, "allreduce", n, m, dtype, schedule)
    cs.ccl_sim_allreduce(send, recv, m, op=op, schedule=schedule, workspace=ws, dtype=dtype)
    torch.cuda.synchronize()
    return [to_host(r, dtype) for r in recv]


def random_inputs(n, m, dtype, seed, op="sum"):
    """Small random rank buffers.  PROD draws values near 1 so long products
    stay finite and exercise rounding rather than overflow."""
    rng = np.random.default_rng(seed)
    if dtype in ("int32", "int64"):
        info = np.iinfo(NP[dtype])
        if op == "prod":
            return [rng.integers(-5, 6, m).astype(NP[dtype]) for _ in range(n)]
        return [rng.integers(info.min // 2, info.max // 2, m, dtype=np.int64).astype(NP[dtype]) for _ in range(n)]
    if op == "prod":
        f = [rng.uniform(0.5, 1.5, m).astype(np.float32) * np.where(rng.random(m) < 0.5, -1, 1).astype(np.float32)
             for _ in range(n)]
    else:
        f = [rng.uniform(-1, 1, m).astype(np.float32) for _ in range(n)]
    if dtype == "bfloat16":
        return [(x.view(np.uint32) >> np.uint32(16)).astype(np.uint16) for x in f]
    return f


def same_bits(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    if a.shape != b.shape:
        return False
    if a.dtype == np.float32:
        return np.array_equal(a.view(np.uint32), b.view(np.uint32))
    return np.array_equal(a, b)
