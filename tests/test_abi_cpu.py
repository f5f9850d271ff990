"""Host-side checks of the C-ABI library: it loads, exports every declared
symbol, and rejects bad arguments before any HIP call (so these run without
a GPU).  Device addresses here are fake integers: a rejected call never
dereferences them."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def cs():
    from collective_reduction_amd import ccl_sim
    return ccl_sim


def declared_functions():
    text = open(os.path.join(ROOT, "include", "ccl_sim.h"), encoding="utf-8").read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(ccl_sim_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol(cs):
    names = declared_functions()
    assert len(names) >= 12
    lib = ctypes.CDLL(cs.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(cs.EXPORTED)
    assert cs.ccl_sim_version() == 100


BASE = 1 << 32


def fake(n, count, es, stride=None, base=BASE):
    stride = stride or ((count * es + 4095) // 4096 + 1) * 4096
    return [base + r * stride for r in range(n)]


def code_of(fn, *a, **k):
    try:
        fn(*a, **k)
    except TypeError:
        return "capacity"
    except Exception as e:  # noqa: BLE001
        return getattr(e, "code", str(e))
    return 0


def test_capacity_check_rejects_nondivisible_reduce_scatter(cs):
    """1003 elements over 4 ranks with recvcount 250 is rejected with the
    capacity-check message before anything runs."""
    n = 4
    with pytest.raises(TypeError, match=r"sendcount \(1003\) != nranks \(4\) x recvcount \(250\)"):
        cs.ccl_sim_reduce_scatter(fake(n, 1003, 8), fake(n, 250, 8, base=BASE * 3), 1003, 250, dtype="int64")
    with pytest.raises(TypeError):
        cs.ccl_sim_all_gather(fake(n, 10, 4), fake(n, 41, 4, base=BASE * 3), 10, 41, dtype="float32")


def test_argument_validation(cs):
    n, m = 4, 1000
    s, r = fake(n, m, 4), fake(n, m, 4, base=BASE * 3)
    ar = cs.ccl_sim_allreduce
    assert code_of(ar, s, r, m, dtype="float32", op=9) == cs.INVALID_ARGUMENT
    assert code_of(ar, s, r, m, dtype="float32", op=5) == cs.INVALID_ARGUMENT
    assert code_of(ar, s, r, m, dtype=7) == cs.INVALID_ARGUMENT
    assert code_of(ar, s, r, m, dtype="float32", schedule=6) == cs.INVALID_ARGUMENT
    assert code_of(ar, [], [], m, dtype="float32") == cs.INVALID_ARGUMENT
    big = fake(1025, 1, 4)
    assert code_of(ar, big, fake(1025, 1, 4, base=BASE * 9), 1, dtype="float32") == cs.INVALID_ARGUMENT
    # null and misaligned pointers
    assert code_of(ar, [s[0], 0, s[2], s[3]], r, m, dtype="float32") == cs.INVALID_ARGUMENT
    assert code_of(ar, [s[0] + 2, s[1], s[2], s[3]], r, m, dtype="float32") == cs.INVALID_ARGUMENT
    assert "aligned" in cs.ccl_sim_last_error()
    # overlapping outputs
    r_bad = [r[0], r[0] + 400, r[2], r[3]]
    assert code_of(ar, s, r_bad, m, dtype="float32") == cs.INVALID_ARGUMENT
    assert "overlap" in cs.ccl_sim_last_error()
    # input of one rank overlapping another rank's output
    s_bad = [r[1], s[1], s[2], s[3]]
    assert code_of(ar, s_bad, r, m, dtype="float32") == cs.INVALID_ARGUMENT
    # ring without a workspace
    assert code_of(ar, s, r, m, dtype="float32", schedule="ring_stepwise") == cs.INSUFFICIENT_WORKSPACE
    need = cs.ccl_sim_workspace_size("allreduce", n, m, "float32", "ring_stepwise")
    ws = (BASE * 7, need - 1)
    assert code_of(ar, s, r, m, dtype="float32", schedule="ring_stepwise", workspace=ws) == \
        cs.INSUFFICIENT_WORKSPACE
    # workspace overlapping a buffer
    ws_bad = (r[2], need)
    assert code_of(ar, s, r, m, dtype="float32", schedule="ring_stepwise", workspace=ws_bad) == \
        cs.INVALID_ARGUMENT
    # misaligned workspace
    assert code_of(ar, s, r, m, dtype="float32", schedule="ring_stepwise", workspace=(BASE * 7 + 64, need)) == \
        cs.INVALID_ARGUMENT
    # pad: padded smaller than count
    assert code_of(cs.ccl_sim_pad_identity, s, r, 10, 9, "max", dtype="float32") == cs.INVALID_ARGUMENT


def test_count_zero_is_a_noop_even_with_null_pointers(cs):
    cs.ccl_sim_allreduce([0] * 4, [0] * 4, 0, dtype="float32")
    cs.ccl_sim_reduce_scatter([0] * 4, [0] * 4, 0, 0, dtype="int32")
    cs.ccl_sim_all_gather([0] * 4, [0] * 4, 5, 0, dtype="int32")
    cs.ccl_sim_pad_identity([0] * 4, [0] * 4, 0, 0, "sum", dtype="int32")


def test_binding_rejects_host_tensors(cs):
    """A host tensor's address would reach the kernels as a device pointer:
    the binding refuses it before calling the library."""
    import torch
    t = [torch.zeros(8) for _ in range(2)]
    for call in (lambda: cs.ccl_sim_allreduce(t, t, 8),
                 lambda: cs.ccl_sim_reduce_scatter(t, t, 8, 4),
                 lambda: cs.ccl_sim_all_gather(t, t, 4, 8),
                 lambda: cs.ccl_sim_pad_identity(t, t, 4, 8, "max")):
        with pytest.raises(ValueError, match="device buffers"):
            call()


def test_plan_checks_at_creation_and_validates_at_run(cs):
    """A Plan refuses host tensors when it is made; counts are validated by
    the library on every run, before anything is enqueued."""
    import torch
    with pytest.raises(ValueError, match="device buffers"):
        cs.Plan("allreduce", [torch.zeros(8)] * 2, [torch.zeros(8)] * 2, 8)
    with pytest.raises(ValueError, match="both counts"):
        cs.Plan("reduce_scatter", fake(4, 100, 4), fake(4, 25, 4, base=BASE * 3), 100, dtype="float32")
    with pytest.raises(ValueError, match="unknown collective"):
        cs.Plan("broadcast", fake(4, 100, 4), fake(4, 100, 4, base=BASE * 3), 100, 100, dtype="float32")
    plan = cs.Plan("reduce_scatter", fake(4, 1003, 8), fake(4, 250, 8, base=BASE * 3), 1003, 250, dtype="int64")
    for _ in range(2):
        with pytest.raises(TypeError, match="sendcount"):
            plan.run()


def test_in_place_forms_pass_validation_overlap(cs):
    """The in-place forms are accepted by the overlap check (the call then
    fails only at the first HIP call when no GPU is present)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only check")
    n, q, es = 4, 256, 4
    s = fake(n, n * q, es)
    ok_codes = (0, cs.HIP_ERROR)
    assert code_of(cs.ccl_sim_allreduce, s, s, n * q, dtype="float32") in ok_codes
    r = [s[i] + i * q * es for i in range(n)]
    assert code_of(cs.ccl_sim_reduce_scatter, s, r, n * q, q, dtype="float32") in ok_codes
    out = fake(n, n * q, es, base=BASE * 5)
    ins = [out[i] + i * q * es for i in range(n)]
    assert code_of(cs.ccl_sim_all_gather, ins, out, q, n * q, dtype="float32") in ok_codes
    # shifted by one shard is not an in-place form
    r_bad = [s[i] + ((i + 1) % n) * q * es for i in range(n)]
    assert code_of(cs.ccl_sim_reduce_scatter, s, r_bad, n * q, q, dtype="float32") == cs.INVALID_ARGUMENT


def test_workspace_sizes(cs):
    ws = cs.ccl_sim_workspace_size
    assert ws("allreduce", 8, 1 << 20, "float32", "direct") == 0
    assert ws("reduce_scatter", 8, 1 << 20, "float32", "direct") == 0
    # ring partials: 2 generations x N x q accumulators
    assert ws("allreduce", 8, 1 << 20, "float32", "ring_stepwise") == 2 * 8 * (1 << 17) * 4
    assert ws("allreduce", 8, 1 << 20, "bfloat16", "ring_stepwise") == 2 * 8 * (1 << 17) * 4
    assert ws("allreduce", 2, 1000, "float32", "ring_stepwise") == 0
    assert ws("all_gather", 8, 1000, "float32", "ring_stepwise") == 0
    # persistent ring: control block of 160 barrier words + 4096 step flags, rounded to 256 bytes
    ctrl = (4256 * 4 + 255) // 256 * 256
    assert ctrl == 17152
    assert ws("all_gather", 8, 1000, "float32", "ring_persistent") == ctrl
    # more than 64 ranks: two pointer tables
    assert ws("allreduce", 256, 1 << 22, "float32", "direct") == 2 * 2048
    assert ws("allreduce", 256, 1 << 22, "float32", "ring_persistent") == ctrl + 4096 + 2 * (1 << 22) * 4
    assert ws("allreduce", 1, 100, "float32", "ring_persistent") == 0
    # chained ring: one partial per chunk, N x q accumulators
    assert ws("allreduce", 8, 1 << 20, "float32", "ring_chained") == 8 * (1 << 17) * 4
    assert ws("reduce_scatter", 8, 1 << 20, "bfloat16", "ring_chained") == 8 * (1 << 17) * 4
    assert ws("all_gather", 8, 1 << 20, "float32", "ring_chained") == 0
    assert ws("allreduce", 2, 1000, "float32", "ring_chained") == 0
    assert ws("allreduce", 0, 100, "float32", "direct") == ctypes.c_size_t(-1).value


def test_workspace_objects_refuse_invalid_requests(cs):
    """No allocation is attempted for a request the library calls invalid."""
    with pytest.raises(ValueError, match="invalid"):
        cs.Workspace("allreduce", 0, 100, "float32", "direct", device="cpu")
    with pytest.raises(ValueError, match="invalid"):
        cs.Workspace.largest([("allreduce", 8, 100, "float32", "direct"),
                              ("allreduce", 2000, 100, "float32", "direct")], device="cpu")
    with pytest.raises(ValueError, match="empty"):
        cs.Workspace.largest([], device="cpu")
    # sizes of zero need no tensor at all
    w = cs.Workspace.largest([("allreduce", 8, 100, "float32", "direct")], device="cpu")
    assert w.nbytes == 0 and w.tensor is None


def test_algorithmic_bytes(cs):
    ab = cs.ccl_sim_algorithmic_bytes
    n, m = 8, 1 << 28
    assert ab("reduce_scatter", n, m, "float32", "direct") == (n + 1) * m * 4
    assert ab("all_gather", n, m, "float32", "direct") == (n + 1) * m * 4
    assert ab("allreduce", n, m, "float32", "direct") == 2 * n * m * 4
    assert ab("reduce_scatter", n, m, "float32", "ring_stepwise") == 3 * (n - 1) * m * 4
    assert ab("all_gather", n, m, "float32", "ring_persistent") == 2 * n * m * 4
    for coll in ("reduce_scatter", "all_gather", "allreduce"):
        assert ab(coll, n, m, "float32", "ring_chained") == ab(coll, n, m, "float32", "ring_stepwise")
    assert ab("allreduce", n, m, "float32", "ring_stepwise") == 5 * (n - 1) * m * 4
    assert ab("allreduce", 256, 1 << 22, "float32", "ring_stepwise") == 21_390_950_400
    # bf16 with fp32 partials: first step 2+2+4, middle 4+2+4, last 4+2+2 bytes per position
    n2, m2 = 256, 6_553_600
    assert ab("reduce_scatter", n2, m2, "bfloat16", "ring_stepwise") == (8 + 10 * (n2 - 3) + 8) * m2
    assert ab("allreduce", 1, 10, "int64", "ring_stepwise") == 2 * 10 * 8


def test_launch_counts_follow_the_step_counts(cs, golden):
    g = golden("step_counts.json")
    lc = cs.ccl_sim_launch_count
    for n, steps in g["allreduce_steps"].items():
        assert lc("allreduce", int(n), 100, "ring_stepwise") == steps
    assert lc("reduce_scatter", 4, 100, "ring_stepwise") == g["phase_steps_n4"]
    assert lc("all_gather", 4, 100, "ring_stepwise", in_place=True) == g["phase_steps_n4"]
    assert lc("all_gather", 4, 100, "ring_stepwise") == 4
    assert lc("allreduce", 8, 100, "direct") == 1
    assert lc("allreduce", 8, 100, "ring_persistent") == 1
    assert lc("allreduce", 8, 100, "ring_chained") == 1
    assert lc("all_gather", 8, 100, "ring_chained") == 1
    assert lc("allreduce", 8, 0, "ring_stepwise") == 0


def test_ring_routing_matches_the_n4_table(cs, golden):
    g = golden("ring_n4_routing.json")
    n = g["nranks"]
    for t, row in enumerate(g["reduce_scatter_send"]):
        assert [cs.ccl_sim_ring_route(n, 0, t, r)[0] for r in range(n)] == row
        assert [cs.ccl_sim_ring_route(n, 0, t, (r + 1) % n)[1] for r in range(n)] == row
    assert [cs.ccl_sim_ring_owner(n, r) for r in range(n)] == g["owner_after_reduce_scatter"]
    for t, row in enumerate(g["all_gather_send"]):
        assert [cs.ccl_sim_ring_route(n, 1, t, r)[0] for r in range(n)] == row
    # stand-alone AllGather: rank r starts with shard r and first receives r-1
    assert [cs.ccl_sim_ring_route(n, 2, 0, r)[1] for r in range(n)] == [3, 0, 1, 2]
    assert cs.ccl_sim_ring_owner(4, 4) == -1
    with pytest.raises(Exception):
        cs.ccl_sim_ring_route(4, 0, 3, 0)


def test_recursive_routing_matches_the_pair_table(cs, golden):
    g = golden("recursive_halving_n8.json")
    n = g["nranks"]
    for j, pairs in enumerate(g["pairs"], start=1):
        for a, b in pairs:
            pa, fa, na = cs.ccl_sim_recursive_route(n, 0, j, a)
            pb, fb, nb = cs.ccl_sim_recursive_route(n, 0, j, b)
            assert (pa, pb) == (b, a)
            assert na == nb == g["data_per_node_after"][j - 1] * n
            assert fa + na == fb  # the lower rank keeps the lower half
    for i in range(n):
        assert cs.ccl_sim_recursive_route(n, 0, 3, i)[1:] == (i, 1)
    # doubling: rank 5 gets block 4 from rank 4, then blocks 6-7, then 0-3
    assert [cs.ccl_sim_recursive_route(n, 1, t, 5) for t in range(3)] == [(4, 4, 1), (7, 6, 2), (1, 0, 4)]
    with pytest.raises(Exception):
        cs.ccl_sim_recursive_route(6, 0, 1, 0)


def test_recursive_planning(cs):
    ws, ab, lc = cs.ccl_sim_workspace_size, cs.ccl_sim_algorithmic_bytes, cs.ccl_sim_launch_count
    n, m = 8, 1 << 28
    assert ws("allreduce", n, m, "float32", "recursive") == n * (n // 2) * (m // n) * 4
    assert ws("allreduce", 2, 1000, "float32", "recursive") == 0
    assert ws("all_gather", 8, 1000, "float32", "recursive") == 0
    assert ab("reduce_scatter", n, m, "float32", "recursive") == 3 * (n - 1) * m * 4
    assert ab("allreduce", n, m, "float32", "recursive") == 5 * (n - 1) * m * 4
    assert ab("all_gather", n, m, "float32", "recursive") == 2 * n * m * 4
    assert lc("allreduce", 8, 100, "recursive") == 6
    assert lc("reduce_scatter", 256, 100, "recursive") == 8
    assert lc("all_gather", 16, 100, "recursive") == 5
    assert lc("allreduce", 6, 100, "recursive") == -1
    s, r = fake(6, 60, 4), fake(6, 60, 4, base=BASE * 3)
    assert code_of(cs.ccl_sim_allreduce, s, r, 60, dtype="float32", schedule="recursive") == cs.UNSUPPORTED
    # the chained driver: same workspace and bytes, one launch, same power-of-two rule
    for coll in ("reduce_scatter", "all_gather", "allreduce"):
        for nn, mm, dt in ((8, m, "float32"), (256, 1 << 22, "bfloat16"), (2, 1000, "int64"), (4, 1003, "int32")):
            assert ws(coll, nn, mm, dt, "recursive_chained") == ws(coll, nn, mm, dt, "recursive")
            assert ab(coll, nn, mm, dt, "recursive_chained") == ab(coll, nn, mm, dt, "recursive")
            assert lc(coll, nn, mm, "recursive_chained") == 1
        assert lc(coll, 6, 100, "recursive_chained") == -1
    assert lc("allreduce", 1, 100, "recursive_chained") == 1
    assert code_of(cs.ccl_sim_allreduce, s, r, 60, dtype="float32", schedule="recursive_chained") == cs.UNSUPPORTED
    assert code_of(cs.ccl_sim_allreduce, s, r, 60, dtype="float32", schedule=6) == cs.INVALID_ARGUMENT


def test_result_strings(cs):
    assert cs.ccl_sim_result_string(0) == "success"
    assert cs.ccl_sim_result_string(5) == "capacity mismatch"


def test_c_abi_from_plain_c(tmp_path, cs):
    """include/ccl_sim.h compiles as C11 (with -Wall -Wextra -Werror) and a
    plain C program linked against the library gets the planning, model and
    validation results the header states (tests/c/abi_check.c; no GPU)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    libdir = os.path.dirname(cs.LIB_PATH)
    exe = tmp_path / "abi_check"
    build = subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                            os.path.join(ROOT, "tests", "c", "abi_check.c"), "-L", libdir, "-l:" + os.path.basename(cs.LIB_PATH),
                            "-lm", f"-Wl,-rpath,{libdir}", "-o", str(exe)], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = {k: v for k, v in os.environ.items() if k != "CCL_SIM_PERSISTENT_SYNC"}  # the library's own choice
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60, env=env)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr


def test_persistent_grid_request_is_capped(cs, monkeypatch):
    """CCL_SIM_PERSISTENT_BLOCKS_PER_CU above 4 (the largest grid seen to run
    to completion) or below 0 is refused with CCL_SIM_UNSUPPORTED before any
    HIP call, for the persistent ring only; accepted values pass validation
    and reach the device query, which fails here without a GPU."""
    n, m = 4, 1000
    s, r = fake(n, m, 4), fake(n, m, 4, base=BASE * 3)
    need = cs.ccl_sim_workspace_size("allreduce", n, m, "float32", "ring_persistent")
    ws = (BASE * 7, need)
    ar = cs.ccl_sim_allreduce
    for bad in ("5", "7", "-1"):
        monkeypatch.setenv("CCL_SIM_PERSISTENT_BLOCKS_PER_CU", bad)
        assert code_of(ar, s, r, m, dtype="float32", schedule="ring_persistent", workspace=ws) == cs.UNSUPPORTED
        assert "CCL_SIM_PERSISTENT_BLOCKS_PER_CU" in cs.ccl_sim_last_error()
        # the knob belongs to the persistent ring: other schedules ignore it
        got = code_of(ar, s, r, m, dtype="float32", schedule="ring_stepwise", workspace=ws)
        assert got != cs.UNSUPPORTED
    for good in ("0", "1", "4"):
        monkeypatch.setenv("CCL_SIM_PERSISTENT_BLOCKS_PER_CU", good)
        got = code_of(ar, s, r, m, dtype="float32", schedule="ring_persistent", workspace=ws)
        assert got != cs.UNSUPPORTED
        assert "CCL_SIM_PERSISTENT_BLOCKS_PER_CU" not in cs.ccl_sim_last_error()
    # a single rank has nothing to exchange and runs the direct copy: no grid to cap
    monkeypatch.setenv("CCL_SIM_PERSISTENT_BLOCKS_PER_CU", "9")
    got = code_of(ar, s[:1], r[:1], m, dtype="float32", schedule="ring_persistent")
    assert got != cs.UNSUPPORTED


def test_unknown_step_ordering_is_refused_before_any_hip_call(cs, monkeypatch):
    """CCL_SIM_PERSISTENT_SYNC other than grid, flags, auto or empty makes a
    persistent-ring call fail with CCL_SIM_INVALID_ARGUMENT before anything
    is enqueued; the other schedules do not read it."""
    n, m = 4, 1000
    s, r = fake(n, m, 4), fake(n, m, 4, base=BASE * 3)
    need = cs.ccl_sim_workspace_size("allreduce", n, m, "float32", "ring_persistent")
    ws = (BASE * 7, need)
    ar = cs.ccl_sim_allreduce
    for bad in ("barrier", "GRID", "1"):
        monkeypatch.setenv("CCL_SIM_PERSISTENT_SYNC", bad)
        assert code_of(ar, s, r, m, dtype="float32", schedule="ring_persistent", workspace=ws) == cs.INVALID_ARGUMENT
        assert "CCL_SIM_PERSISTENT_SYNC" in cs.ccl_sim_last_error()
        got = code_of(ar, s, r, m, dtype="float32", schedule="ring_stepwise", workspace=ws)
        assert got != cs.INVALID_ARGUMENT or "CCL_SIM_PERSISTENT_SYNC" not in cs.ccl_sim_last_error()
    for good in ("grid", "flags", "auto", ""):
        monkeypatch.setenv("CCL_SIM_PERSISTENT_SYNC", good)
        code_of(ar, s, r, m, dtype="float32", schedule="ring_persistent", workspace=ws)
        assert "CCL_SIM_PERSISTENT_SYNC" not in cs.ccl_sim_last_error()


def test_persistent_ordering_query(cs, monkeypatch):
    """The persistent ring takes per-workgroup step flags for steps (N chunks
    of ceil(M/N)) of up to 2^26 elements and the grid barrier above, unless
    CCL_SIM_PERSISTENT_SYNC says otherwise; the query answers without a GPU."""
    monkeypatch.delenv("CCL_SIM_PERSISTENT_SYNC", raising=False)
    po = cs.ccl_sim_persistent_ordering
    assert po("allreduce", 256, 1 << 22) == "flags"
    assert po("allreduce", 256, 6_553_600) == "flags"
    assert po("reduce_scatter", 8, 1 << 24) == "flags"
    assert po("allreduce", 8, 1 << 25) == "flags"
    assert po("allreduce", 8, 1 << 26) == "flags"            # a step of exactly 2^26
    assert po("allreduce", 8, (1 << 26) + 1) == "grid"       # q rounds up: a step of 2^26 + 8
    assert po("allreduce", 3, 1 << 26) == "grid"             # 3 x 22,369,622 = 2^26 + 2
    assert po("allreduce", 3, (1 << 26) - 1) == "flags"      # 3 x 22,369,621 = 2^26 - 1
    assert po("all_gather", 16, 1 << 27) == "grid"
    assert po("allreduce", 8, 1 << 28) == "grid"
    assert po("allreduce", 1, 1 << 20) is None               # one rank: the direct copy
    assert po("allreduce", 8, 0) is None
    monkeypatch.setenv("CCL_SIM_PERSISTENT_SYNC", "grid")
    assert po("allreduce", 256, 1 << 22) == "grid"
    monkeypatch.setenv("CCL_SIM_PERSISTENT_SYNC", "flags")
    assert po("allreduce", 8, 1 << 28) == "flags"
    monkeypatch.setenv("CCL_SIM_PERSISTENT_SYNC", "auto")
    assert po("allreduce", 8, 1 << 28) == "grid"
    monkeypatch.setenv("CCL_SIM_PERSISTENT_SYNC", "sometimes")
    with pytest.raises(cs.CclSimError):
        po("allreduce", 8, 1 << 20)
    monkeypatch.delenv("CCL_SIM_PERSISTENT_SYNC")
    lib = cs._lib
    lib.ccl_sim_persistent_ordering.restype = ctypes.c_int
    lib.ccl_sim_persistent_ordering.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_size_t]
    assert lib.ccl_sim_persistent_ordering(7, 8, 1000) == -1   # not a collective
    assert lib.ccl_sim_persistent_ordering(2, 0, 1000) == -1
    assert lib.ccl_sim_persistent_ordering(2, 1025, 1000) == -1  # above CCL_SIM_MAX_RANKS
    assert lib.ccl_sim_persistent_ordering(2, 256, 1 << 22) == 2  # CCL_SIM_ORDER_FLAGS


def test_noalloc_allreduce_limits_are_checked_before_any_hip_call(cs):
    """ccl_sim_allreduce_noalloc refuses the persistent ring and any call
    whose workspace would not fit the library's scratch before touching the
    device; count 0 is a no-op; invalid arguments are reported as by
    ccl_sim_allreduce."""
    n, m = 8, 1000
    s, r = fake(n, m, 4), fake(n, m, 4, base=BASE * 3)
    noalloc = cs.ccl_sim_allreduce_noalloc
    assert code_of(noalloc, s, r, m, dtype="float32", schedule="ring_persistent") == cs.UNSUPPORTED
    assert "persistent" in cs.ccl_sim_last_error()
    # ring partials 2·N·q·4 bytes: the largest M that fits, and the next size up
    cap = cs.NOALLOC_SCRATCH_BYTES
    fits = cap // 8
    assert cs.ccl_sim_workspace_size("allreduce", n, fits, "float32", "ring_stepwise") <= cap
    too_big = fits + 8 * 64
    assert cs.ccl_sim_workspace_size("allreduce", n, too_big, "float32", "ring_stepwise") > cap
    big_s, big_r = fake(n, too_big, 4), fake(n, too_big, 4, base=BASE * 40)
    assert code_of(noalloc, big_s, big_r, too_big, dtype="float32", schedule="ring_stepwise") == \
        cs.INSUFFICIENT_WORKSPACE
    assert "scratch" in cs.ccl_sim_last_error()
    # the recursive halves N·(N/2)·q·a reach the limit sooner
    assert code_of(noalloc, big_s, big_r, too_big, dtype="float32", schedule="recursive") == \
        cs.INSUFFICIENT_WORKSPACE
    cs.ccl_sim_allreduce_noalloc([0] * 4, [0] * 4, 0, dtype="float32", schedule="ring_stepwise")
    assert code_of(noalloc, s, r, m, dtype="float32", op=9) == cs.INVALID_ARGUMENT
    assert code_of(noalloc, s[:6], r[:6], m, dtype="float32", schedule="recursive") == cs.UNSUPPORTED
    assert code_of(noalloc, [], [], m, dtype="float32") == cs.INVALID_ARGUMENT
