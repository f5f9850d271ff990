"""ctypes binding of libccl_sim.so (declared in include/ccl_sim.h).

Argument marshalling only: rank buffers given as torch tensors (or raw
device addresses) become arrays of device pointers, torch dtypes become the
library's dtype codes, and the current torch stream becomes the HIP stream.
Every collective runs in the library's HIP kernels; there is no CPU path.
A missing library raises ImportError at import.

torch is imported before the library is loaded: torch ships its own HIP
runtime under the same soname, and loading torch first makes the library
bind to that one runtime instead of a second copy.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# CCL_SIM_LIBRARY may name another build of the same library (a debug or
# tuning variant); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("CCL_SIM_LIBRARY") or os.path.join(_HERE, "libccl_sim.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -m collective_reduction_amd._build` "
        "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes_mapped():
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


if len(_hip_runtimes_mapped()) > 1:
    raise ImportError(f"two HIP runtimes are loaded: {sorted(_hip_runtimes_mapped())}")

# enums (include/ccl_sim.h)
SUCCESS, INVALID_ARGUMENT, UNSUPPORTED, INSUFFICIENT_WORKSPACE, HIP_ERROR, CAPACITY_MISMATCH = range(6)
DTYPES = {"int32": 0, "int64": 1, "float32": 2, "bfloat16": 3}
OPS = {"sum": 0, "prod": 1, "max": 2, "min": 3, "avg": 4}
SCHEDULES = {"direct": 0, "ring_stepwise": 1, "ring_persistent": 2, "recursive": 3, "ring_chained": 4,
             "recursive_chained": 5}
COLLS = {"reduce_scatter": 0, "all_gather": 1, "allreduce": 2}
INLINE_RANKS = 64
MAX_RANKS = 1024

_TORCH_DTYPES = {torch.int32: "int32", torch.int64: "int64", torch.float32: "float32", torch.bfloat16: "bfloat16"}

_c_size = ctypes.c_size_t
_vpp = ctypes.POINTER(ctypes.c_void_p)


def _sig(name, restype, argtypes):
    fn = getattr(_lib, name)
    fn.restype = restype
    fn.argtypes = argtypes
    return fn


_reduce_scatter = _sig("ccl_sim_reduce_scatter", ctypes.c_int,
                       [_vpp, _vpp, ctypes.c_int, _c_size, _c_size, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                        ctypes.c_void_p, _c_size, ctypes.c_void_p])
_all_gather = _sig("ccl_sim_all_gather", ctypes.c_int,
                   [_vpp, _vpp, ctypes.c_int, _c_size, _c_size, ctypes.c_int, ctypes.c_int,
                    ctypes.c_void_p, _c_size, ctypes.c_void_p])
_allreduce = _sig("ccl_sim_allreduce", ctypes.c_int,
                  [_vpp, _vpp, ctypes.c_int, _c_size, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p, _c_size, ctypes.c_void_p])
_allreduce_noalloc = _sig("ccl_sim_allreduce_noalloc", ctypes.c_int,
                          [_vpp, _vpp, ctypes.c_int, _c_size, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                           ctypes.c_void_p])
_pad_identity = _sig("ccl_sim_pad_identity", ctypes.c_int,
                     [_vpp, _vpp, ctypes.c_int, _c_size, _c_size, ctypes.c_int, ctypes.c_int, ctypes.c_void_p])
_workspace_size = _sig("ccl_sim_workspace_size", _c_size,
                       [ctypes.c_int, ctypes.c_int, _c_size, ctypes.c_int, ctypes.c_int])
_algorithmic_bytes = _sig("ccl_sim_algorithmic_bytes", ctypes.c_uint64,
                          [ctypes.c_int, ctypes.c_int, _c_size, ctypes.c_int, ctypes.c_int])
_launch_count = _sig("ccl_sim_launch_count", ctypes.c_int,
                     [ctypes.c_int, ctypes.c_int, _c_size, ctypes.c_int, ctypes.c_int])
_ring_owner = _sig("ccl_sim_ring_owner", ctypes.c_int, [ctypes.c_int, ctypes.c_int])
_ring_route = _sig("ccl_sim_ring_route", ctypes.c_int,
                   [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                    ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)])
_recursive_route = _sig("ccl_sim_recursive_route", ctypes.c_int,
                        [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                         ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)])
_result_string = _sig("ccl_sim_result_string", ctypes.c_char_p, [ctypes.c_int])
_persistent_aborted = _sig("ccl_sim_persistent_aborted", ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int)])
_persistent_ordering = _sig("ccl_sim_persistent_ordering", ctypes.c_int, [ctypes.c_int, ctypes.c_int, _c_size])
_last_error = _sig("ccl_sim_last_error", ctypes.c_char_p, [])
_version = _sig("ccl_sim_version", ctypes.c_int, [])


class _LinkParams(ctypes.Structure):
    _fields_ = [("alpha_s", ctypes.c_double), ("beta_bytes_per_s", ctypes.c_double), ("ranks_per_node", ctypes.c_int),
                ("alpha_intra_s", ctypes.c_double), ("beta_intra_bytes_per_s", ctypes.c_double)]


class _Estimate(ctypes.Structure):
    _fields_ = [("time_s", ctypes.c_double), ("latency_s", ctypes.c_double), ("bandwidth_s", ctypes.c_double),
                ("latency_fraction", ctypes.c_double), ("algbw_gbps", ctypes.c_double),
                ("busbw_gbps", ctypes.c_double), ("steps", ctypes.c_double)]


_model_estimate = _sig("ccl_sim_model_estimate", ctypes.c_int,
                       [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.POINTER(_LinkParams),
                        ctypes.POINTER(_Estimate)])
_busbw_factor = _sig("ccl_sim_busbw_factor", ctypes.c_double, [ctypes.c_int, ctypes.c_int])
MODEL_COLLS = {"all_reduce": 0, "all_gather": 1, "reduce_scatter": 2, "all_to_all": 3, "broadcast": 4, "reduce": 5}
MODEL_ALGOS = {"ring": 0, "tree": 1, "2level": 2}

EXPORTED = ("ccl_sim_reduce_scatter", "ccl_sim_all_gather", "ccl_sim_allreduce", "ccl_sim_pad_identity",
            "ccl_sim_workspace_size", "ccl_sim_algorithmic_bytes", "ccl_sim_launch_count", "ccl_sim_ring_owner",
            "ccl_sim_ring_route", "ccl_sim_result_string", "ccl_sim_last_error", "ccl_sim_version",
            "ccl_sim_model_estimate", "ccl_sim_busbw_factor", "ccl_sim_recursive_route",
            "ccl_sim_persistent_aborted", "ccl_sim_allreduce_noalloc", "ccl_sim_persistent_ordering")
NOALLOC_SCRATCH_BYTES = 64 << 20  # CCL_SIM_NOALLOC_SCRATCH_BYTES


class CclSimError(RuntimeError):
    """A non-capacity failure reported by the library."""

    def __init__(self, code, message):
        super().__init__(message)
        self.code = code


def _check(code):
    if code == SUCCESS:
        return
    detail = _last_error().decode()
    what = _result_string(code).decode()
    msg = f"{what}: {detail}" if detail else what
    if code == CAPACITY_MISMATCH:
        # the same exception type the PyTorch capacity check raises
        raise TypeError(msg)
    raise CclSimError(code, msg)


def _enum(table, value, what):
    if isinstance(value, int):
        return value
    try:
        return table[value]
    except KeyError:
        raise ValueError(f"unknown {what} {value!r}; expected one of {sorted(table)}") from None


def _dtype_code(dtype):
    if isinstance(dtype, torch.dtype):
        if dtype not in _TORCH_DTYPES:
            raise ValueError(f"unsupported dtype {dtype}")
        dtype = _TORCH_DTYPES[dtype]
    return _enum(DTYPES, dtype, "dtype")


_HAVE_GPU = None
# torch's accessor of the current stream's raw handle; it skips building a
# Stream object, which costs more than the rest of a small call
_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, dev=None):
    global _HAVE_GPU
    if stream is None:
        if _HAVE_GPU is None:
            _HAVE_GPU = torch.cuda.is_available()
        if not _HAVE_GPU:
            # without a GPU the library rejects or fails the call itself; the
            # null stream keeps argument validation reachable on a host
            return None
        if _RAW_STREAM is not None:
            return _RAW_STREAM(torch.cuda.current_device() if dev is None else dev)
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _infer_dtype(bufs, dtype):
    if dtype is not None:
        return _dtype_code(dtype)
    for b in bufs:
        if isinstance(b, torch.Tensor):
            return _dtype_code(b.dtype)
    raise ValueError("dtype must be given when buffers are raw addresses")


_CODE_NAMES = {v: k for k, v in DTYPES.items()}
_CODE_TORCH = {DTYPES[name]: dt for dt, name in _TORCH_DTYPES.items()}


def _refuse(b, r, need, code, what, dev):
    if b.device.type != "cuda":
        raise ValueError(f"{what}[{r}] is a {b.device.type} tensor; the library takes device buffers")
    if b.get_device() != dev:
        raise ValueError(f"{what}[{r}] is on {b.device}, not on the current device cuda:{dev}")
    if b.dtype is not _CODE_TORCH.get(code):
        raise ValueError(f"{what}[{r}] has dtype {b.dtype}; the call is {_CODE_NAMES.get(code, code)}")
    if not b.is_contiguous():
        raise ValueError(f"{what}[{r}] is not contiguous")
    raise ValueError(f"{what}[{r}] holds {b.numel()} elements; the call needs {need}")


def _marshal(bufs, need, code, what, dev=None):
    """The host array of device addresses the C ABI takes, one per rank.
    Rank buffers given as tensors must be contiguous device tensors of the
    call's dtype, on the current device, holding at least `need` elements:
    the library sees only addresses, and a host address or a short buffer
    would reach the kernels.  Raw addresses are the caller's
    responsibility.  Also returns the current device once it has been read,
    so a call reads it at most once (the checks run on every call, so they
    keep to a few cheap tensor attributes)."""
    want = _CODE_TORCH.get(code)
    ptrs = [0] * len(bufs)
    for r, b in enumerate(bufs):
        if isinstance(b, torch.Tensor):
            d = b.get_device()
            if d < 0:
                _refuse(b, r, need, code, what, dev)
            if dev is None:
                dev = torch.cuda.current_device()
            if d != dev or b.dtype is not want or b.numel() < need or not b.is_contiguous():
                _refuse(b, r, need, code, what, dev)
            ptrs[r] = b.data_ptr()
        else:
            ptrs[r] = int(b)
    return (ctypes.c_void_p * len(ptrs))(*ptrs), dev


def _ws(workspace, dev=None):
    """(address, bytes) of the workspace.  A tensor must be a contiguous
    device tensor on the call's device (`dev`, when the call has read it)."""
    if workspace is None:
        return ctypes.c_void_p(0), 0
    if isinstance(workspace, Workspace):
        if workspace.tensor is None:
            return ctypes.c_void_p(0), 0
        workspace = workspace.tensor
    if isinstance(workspace, torch.Tensor):
        if workspace.device.type != "cuda" or not workspace.is_contiguous():
            raise ValueError("the workspace must be a contiguous device tensor")
        if dev is not None and workspace.get_device() != dev:
            raise ValueError(f"the workspace is on {workspace.device}, not on the current device cuda:{dev}")
        return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()
    addr, nbytes = workspace
    return ctypes.c_void_p(int(addr)), int(nbytes)


def ccl_sim_reduce_scatter(sendbufs, recvbufs, sendcount, recvcount, op="sum", schedule="direct",
                           workspace=None, stream=None, dtype=None):
    """ReduceScatter over len(sendbufs) virtual ranks (rank-major shards)."""
    n = len(sendbufs)
    if len(recvbufs) != n:
        raise ValueError("sendbufs and recvbufs must list the same ranks")
    code = _infer_dtype(sendbufs, dtype)
    s, dev = _marshal(sendbufs, sendcount, code, "sendbufs")
    r, dev = _marshal(recvbufs, recvcount, code, "recvbufs", dev)
    wp, wb = _ws(workspace, dev)
    _check(_reduce_scatter(s, r, n, sendcount, recvcount, code, _enum(OPS, op, "op"),
                           _enum(SCHEDULES, schedule, "schedule"), wp, wb, _stream(stream, dev)))


def ccl_sim_all_gather(sendbufs, recvbufs, sendcount, recvcount, schedule="direct", workspace=None, stream=None,
                       dtype=None):
    """AllGather in source-rank order, trimmed to recvcount."""
    n = len(sendbufs)
    if len(recvbufs) != n:
        raise ValueError("sendbufs and recvbufs must list the same ranks")
    code = _infer_dtype(sendbufs, dtype)
    s, dev = _marshal(sendbufs, sendcount, code, "sendbufs")
    r, dev = _marshal(recvbufs, recvcount, code, "recvbufs", dev)
    wp, wb = _ws(workspace, dev)
    _check(_all_gather(s, r, n, sendcount, recvcount, code, _enum(SCHEDULES, schedule, "schedule"), wp, wb,
                       _stream(stream, dev)))


def ccl_sim_allreduce(sendbufs, recvbufs, count, op="sum", schedule="direct", workspace=None, stream=None,
                      dtype=None):
    """AllReduce of count elements per rank (any count)."""
    n = len(sendbufs)
    if len(recvbufs) != n:
        raise ValueError("sendbufs and recvbufs must list the same ranks")
    code = _infer_dtype(sendbufs, dtype)
    s, dev = _marshal(sendbufs, count, code, "sendbufs")
    r, dev = _marshal(recvbufs, count, code, "recvbufs", dev)
    wp, wb = _ws(workspace, dev)
    _check(_allreduce(s, r, n, count, code, _enum(OPS, op, "op"), _enum(SCHEDULES, schedule, "schedule"), wp, wb,
                      _stream(stream, dev)))


def ccl_sim_allreduce_noalloc(sendbufs, recvbufs, count, op="sum", schedule="direct", stream=None, dtype=None):
    """AllReduce with the library's own device scratch instead of a
    workspace: the call allocates nothing (for graph capture and loops that
    must not allocate).  Calls that overlap in time on one GPU race on its
    scratch; see ccl_sim.h for the size limit."""
    n = len(sendbufs)
    if len(recvbufs) != n:
        raise ValueError("sendbufs and recvbufs must list the same ranks")
    code = _infer_dtype(sendbufs, dtype)
    s, dev = _marshal(sendbufs, count, code, "sendbufs")
    r, dev = _marshal(recvbufs, count, code, "recvbufs", dev)
    _check(_allreduce_noalloc(s, r, n, count, code, _enum(OPS, op, "op"), _enum(SCHEDULES, schedule, "schedule"),
                              _stream(stream, dev)))


def ccl_sim_pad_identity(srcs, dsts, count, padded_count, op, stream=None, dtype=None):
    """dsts[r] = srcs[r] followed by the identity of op up to padded_count."""
    n = len(dsts)
    if len(srcs) != n:
        raise ValueError("srcs and dsts must list the same ranks")
    code = _infer_dtype(dsts, dtype)
    s, dev = _marshal(srcs, count, code, "srcs")
    d, dev = _marshal(dsts, padded_count, code, "dsts", dev)
    _check(_pad_identity(s, d, n, count, padded_count, code, _enum(OPS, op, "op"), _stream(stream, dev)))


class Plan:
    """One collective call with its arguments marshalled once, for loops that
    repeat the same call on the same buffers (a training step's gradient
    buckets, a serving loop).  The binding's tensor checks and the arrays of
    device addresses are done here, at creation; run() only issues the C
    call, which still validates every argument before it enqueues anything.
    The plan keeps references to its tensors and workspace, so their memory
    stays valid; their contents may change between runs, but the tensors
    must not be replaced or resized.

        plan = Plan("allreduce", send, recv, count, op="sum", schedule="ring_chained", workspace=ws)
        plan.run()              # on torch's current stream
        plan.run(stream=s)      # or on a given stream

    For "reduce_scatter" and "all_gather" give sendcount and recvcount as for
    the functions of the same names; for "allreduce" and "pad_identity" the
    counts are count (and padded_count)."""

    def __init__(self, coll, sendbufs, recvbufs, sendcount, recvcount=None, op="sum", schedule="direct",
                 workspace=None, dtype=None):
        n = len(sendbufs)
        if len(recvbufs) != n:
            raise ValueError("sendbufs and recvbufs must list the same ranks")
        self.coll = coll
        code = _infer_dtype(recvbufs if coll == "pad_identity" else sendbufs, dtype)
        if coll in ("allreduce",):
            recvcount = sendcount
        elif recvcount is None:
            raise ValueError(f"{coll} needs both counts")
        s, dev = _marshal(sendbufs, sendcount, code, "sendbufs")
        r, dev = _marshal(recvbufs, recvcount, code, "recvbufs", dev)
        wp, wb = _ws(workspace, dev)
        self._dev = dev
        self._keep = (sendbufs, recvbufs, workspace, s, r)
        sched = _enum(SCHEDULES, schedule, "schedule")
        if coll == "reduce_scatter":
            self._fn, self._args = _reduce_scatter, (s, r, n, sendcount, recvcount, code, _enum(OPS, op, "op"),
                                                     sched, wp, wb)
        elif coll == "all_gather":
            self._fn, self._args = _all_gather, (s, r, n, sendcount, recvcount, code, sched, wp, wb)
        elif coll == "allreduce":
            self._fn, self._args = _allreduce, (s, r, n, sendcount, code, _enum(OPS, op, "op"), sched, wp, wb)
        elif coll == "pad_identity":
            self._fn, self._args = _pad_identity, (s, r, n, sendcount, recvcount, code, _enum(OPS, op, "op"))
        else:
            raise ValueError(f"unknown collective {coll!r}")

    def run(self, stream=None):
        _check(self._fn(*self._args, _stream(stream, self._dev)))


def ccl_sim_workspace_size(coll, nranks, count, dtype, schedule):
    return _workspace_size(_enum(COLLS, coll, "coll"), nranks, count, _dtype_code(dtype),
                           _enum(SCHEDULES, schedule, "schedule"))


def ccl_sim_algorithmic_bytes(coll, nranks, count, dtype, schedule):
    return _algorithmic_bytes(_enum(COLLS, coll, "coll"), nranks, count, _dtype_code(dtype),
                              _enum(SCHEDULES, schedule, "schedule"))


def ccl_sim_launch_count(coll, nranks, count, schedule, in_place=False):
    return _launch_count(_enum(COLLS, coll, "coll"), nranks, count, _enum(SCHEDULES, schedule, "schedule"),
                         int(bool(in_place)))


def ccl_sim_ring_owner(nranks, rank):
    return _ring_owner(nranks, rank)


def ccl_sim_ring_route(nranks, phase, step, rank):
    """(send_chunk, recv_chunk); phase 0 RS, 1 AG after RS, 2 stand-alone AG."""
    s, r = ctypes.c_int(), ctypes.c_int()
    _check(_ring_route(nranks, phase, step, rank, ctypes.byref(s), ctypes.byref(r)))
    return s.value, r.value


def ccl_sim_recursive_route(nranks, phase, step, rank):
    """(partner, first_block, nblocks); phase 0 halving step (1-based),
    phase 1 doubling step (0-based)."""
    p, f, nb = ctypes.c_int(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(_recursive_route(nranks, phase, step, rank, ctypes.byref(p), ctypes.byref(f), ctypes.byref(nb)))
    return p.value, f.value, nb.value


def ccl_sim_persistent_aborted(workspace):
    """True if the last persistent-ring call that used `workspace` stopped
    at a wait's poll limit (its outputs are then incomplete).  Call it
    once that call's stream work has completed, and before another call
    reuses the workspace (the other schedules keep their partials where the
    persistent ring's control block was)."""
    wp, _ = _ws(workspace)
    flag = ctypes.c_int()
    _check(_persistent_aborted(wp, ctypes.byref(flag)))
    return bool(flag.value)


def ccl_sim_persistent_ordering(coll, nranks, count):
    """How a persistent-ring call of these arguments orders its steps under
    the current environment: "grid" (a grid barrier between steps) or
    "flags" (per-workgroup step flags); None when the call runs no ring
    (nranks 1, count 0).  `count` is M, as for ccl_sim_workspace_size."""
    v = _persistent_ordering(_enum(COLLS, coll, "coll"), nranks, count)
    if v < 0:
        raise CclSimError(INVALID_ARGUMENT, "invalid arguments or CCL_SIM_PERSISTENT_SYNC value")
    return {0: None, 1: "grid", 2: "flags"}[v]


def ccl_sim_result_string(code):
    return _result_string(code).decode()


def ccl_sim_last_error():
    return _last_error().decode()


def ccl_sim_version():
    return _version()


def ccl_sim_model_estimate(coll, algo, nranks, size_bytes, alpha_us=10.0, beta_gbps=25.0, ranks_per_node=8,
                           alpha_intra_us=3.0, beta_intra_gbps=200.0):
    """α-β model of a collective on a network (see ccl_sim.h); returns a dict
    with time_s, latency_s, bandwidth_s, latency_fraction, algbw_gbps,
    busbw_gbps and steps.  Bandwidths are 10^9 bytes per second."""
    link = _LinkParams(alpha_us * 1e-6, beta_gbps * 1e9, ranks_per_node, alpha_intra_us * 1e-6,
                       beta_intra_gbps * 1e9)
    est = _Estimate()
    _check(_model_estimate(_enum(MODEL_COLLS, coll, "coll"), _enum(MODEL_ALGOS, algo, "algo"), nranks,
                           float(size_bytes), ctypes.byref(link), ctypes.byref(est)))
    return {name: getattr(est, name) for name, _ in _Estimate._fields_}


def ccl_sim_busbw_factor(coll, nranks):
    return _busbw_factor(_enum(MODEL_COLLS, coll, "coll"), nranks)


class Workspace:
    """Caller-owned device workspace sized by ccl_sim_workspace_size (a
    torch uint8 tensor; torch allocations are at least 256-byte aligned)."""

    def __init__(self, coll, nranks, count, dtype, schedule, device="cuda"):
        nbytes = ccl_sim_workspace_size(coll, nranks, count, dtype, schedule)
        if nbytes == ctypes.c_size_t(-1).value:
            raise ValueError("invalid arguments for the workspace size")
        self.nbytes = nbytes
        self.tensor = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device) if nbytes else None

    @staticmethod
    def largest(requests, device="cuda"):
        """One workspace big enough for every (coll, nranks, count, dtype, schedule) request."""
        sizes = [ccl_sim_workspace_size(*r) for r in requests]
        if not sizes or ctypes.c_size_t(-1).value in sizes:
            raise ValueError("invalid or empty workspace requests")
        w = Workspace.__new__(Workspace)
        w.nbytes = max(sizes)
        w.tensor = torch.empty(max(w.nbytes, 1), dtype=torch.uint8, device=device) if w.nbytes else None
        return w
