// C-ABI front end of libccl_sim: argument validation, planning (shard
// length, workspace layout, in-place detection) and
// dispatch to the kernels.  Every check runs before the first HIP call, so
// a rejected call enqueues nothing.
//
// Pages cited:
//   [DECOMP] "NCCL 专家课程 07：AllReduce 等价分解、显存生命周期与 Kernel 证据"
//   [RING]   "Ring AllReduce 核心流程：梯度是怎么聚合的"
//   [PRIMS]  "通信与互联（01）：集合通信原语与代价模型——α-β 模型与 ring all-reduce"

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "ccl_sim.h"
#include "internal.hpp"

namespace {

using namespace ccl;

// The last failure's message, per thread.  The validation path keeps to
// fixed buffers (this one, and the rank spans on the stack), so that no
// call allocates memory of any kind on the host either.
constexpr int kMessageBytes = 512;
thread_local char g_last_error[kMessageBytes];

void clear_error() { g_last_error[0] = '\0'; }

// Records the message for ccl_sim_last_error() and returns `code`.  A HIP
// failure is reported through the returned code, so HIP's own last-error
// slot is cleared as well: left set, it would resurface in the caller's
// next, unrelated HIP call.
ccl_sim_result_t fail(ccl_sim_result_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  if (code == CCL_SIM_HIP_ERROR) (void)hipGetLastError();
  return code;
}

bool valid_dtype(int d) { return d >= CCL_SIM_INT32 && d <= CCL_SIM_BFLOAT16; }
bool valid_op(int o) { return o >= CCL_SIM_SUM && o <= CCL_SIM_AVG; }
bool valid_sched(int s) { return s >= CCL_SIM_DIRECT && s <= CCL_SIM_RECURSIVE_CHAINED; }
bool recursive(int s) { return s == CCL_SIM_RECURSIVE || s == CCL_SIM_RECURSIVE_CHAINED; }
bool pow2(int n) { return n > 0 && (n & (n - 1)) == 0; }
int log2i(int n) {
  int k = 0;
  while ((1 << k) < n) ++k;
  return k;
}
bool valid_coll(int c) { return c >= CCL_SIM_COLL_REDUCE_SCATTER && c <= CCL_SIM_COLL_ALLREDUCE; }

constexpr size_t kAlign = 256;
constexpr uint64_t kLine = 128;  // bytes in a cache line

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// A single rank has nothing to exchange: every schedule is the direct copy.
int effective_schedule(int nranks, int schedule) { return nranks == 1 ? CCL_SIM_DIRECT : schedule; }

uint64_t shard_len(uint64_t m, int n) { return m / uint64_t(n) + (m % uint64_t(n) != 0); }

// Workspace layout.  `m` is the logical per-rank length (see ccl_sim.h).
struct Layout {
  size_t ctrl = SIZE_MAX, send_tab = SIZE_MAX, recv_tab = SIZE_MAX, partial = SIZE_MAX;
  size_t total = 0;
  bool ok = true;
};

Layout layout(int coll, int nranks, uint64_t m, int dtype, int schedule) {
  Layout l;
  const int sched = effective_schedule(nranks, schedule);
  size_t off = 0;
  if (sched == CCL_SIM_RING_PERSISTENT) {
    l.ctrl = off;
    off += round_up(kCtrlWords * sizeof(unsigned));
  }
  if (nranks > kInlineRanks) {
    const size_t tab = round_up(size_t(nranks) * sizeof(void*));
    l.send_tab = off;
    l.recv_tab = off + tab;
    off += 2 * tab;
  }
  const bool ring = sched == CCL_SIM_RING_STEPWISE || sched == CCL_SIM_RING_PERSISTENT || sched == CCL_SIM_RING_CHAINED;
  const bool halving = recursive(sched);
  if ((ring && nranks >= 3) || (halving && nranks >= 4)) {
    if (coll == CCL_SIM_COLL_ALL_GATHER) {
      l.total = off;
      return l;
    }
    const uint64_t q = shard_len(m, nranks);
    // ring: [2][N][q] partials (chained ring: [N][q], one per chunk);
    // recursive halving: [N][(N/2)·q] per-rank halves
    const uint64_t per_q = sched == CCL_SIM_RING_CHAINED ? uint64_t(nranks)
                           : ring                          ? uint64_t(2) * uint64_t(nranks)
                                                           : uint64_t(nranks) * uint64_t(nranks / 2);
    uint64_t bytes = 0;
    if (__builtin_mul_overflow(q, per_q * accum_size(dtype), &bytes) ||
        bytes > SIZE_MAX - off - kAlign) {
      l.ok = false;
      return l;
    }
    l.partial = off;
    off += round_up(size_t(bytes));
  }
  l.total = off;
  return l;
}

std::atomic<int> g_cus[64];

// Largest persistent-ring grid, in workgroups per CU, that a call may ask
// for.  Grids of 1 to 4 per CU have run to completion on MI355X in every
// measurement; a grid at the occupancy calculator's figure (7 per CU) once
// ran its first grid barrier into the poll limit, and why is not known, so
// nothing above the largest grid seen to work is launched.
constexpr int kMaxPersistentPerCu = 4;

// Environment knobs (read on every call; see env()).
//   CCL_SIM_DEBUG=1                      log each launch plan to stderr; fill the
//                                        partials' scratch with all-ones bits before
//                                        a ring or recursive call, so a read of a
//                                        partial before its write shows in the
//                                        result; after a persistent ring, wait for
//                                        it and report a barrier or flag wait that
//                                        hit its poll limit
//   CCL_SIM_PERSISTENT_BLOCKS_PER_CU=k   persistent ring workgroups per CU, 1..4
//                                        (anything else is refused before a launch)
//   CCL_SIM_PERSISTENT_SYNC=grid|flags   persistent ring step ordering: a grid
//                                        barrier, or per-workgroup step flags;
//                                        unset, empty or "auto": by step size
//                                        (anything else is refused before a launch)
//   CCL_SIM_SPIN_LIMIT=n                 persistent ring poll limit
struct Env {
  bool debug = false;
  int per_cu = 0;
  int sync = kSyncAuto;  // -1: not a known value
  const char* sync_text = "";
  unsigned spin_limit = 0;
  Env() {
    if (const char* v = std::getenv("CCL_SIM_DEBUG")) debug = std::atoi(v) != 0;
    if (const char* v = std::getenv("CCL_SIM_PERSISTENT_BLOCKS_PER_CU")) per_cu = std::atoi(v);
    if (const char* v = std::getenv("CCL_SIM_PERSISTENT_SYNC")) {
      sync_text = v;
      sync = (v[0] == '\0' || std::strcmp(v, "auto") == 0) ? kSyncAuto
             : std::strcmp(v, "grid") == 0                   ? kSyncGrid
             : std::strcmp(v, "flags") == 0                  ? kSyncFlags
                                                             : -1;
    }
    if (const char* v = std::getenv("CCL_SIM_SPIN_LIMIT")) spin_limit = static_cast<unsigned>(std::strtoul(v, nullptr, 10));
  }
};

// Four getenv lookups per call, so that a process can change a knob
// between calls.
Env env() { return Env(); }

hipError_t device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    const int cached = g_cus[dev].load(std::memory_order_relaxed);
    if (cached > 0) {
      *cus = cached;
      return hipSuccess;
    }
  }
  int v = 0;
  e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) g_cus[dev].store(v, std::memory_order_relaxed);
  *cus = v;
  return hipSuccess;
}

struct Span {
  uintptr_t lo, hi;
  int rank;
};

// Outputs must be pairwise disjoint; an input may overlap an output only
// when they belong to the same rank and `allowed(rank)` says the pair is the
// in-place form.  Sorts `outs` (n_outs spans) in place; on failure the
// reason is recorded with fail().  O(N log N).
template <class Allowed>
bool overlap_ok(Span* outs, int n_outs, const Span* ins, int n_ins, Allowed allowed) {
  Span* end = std::remove_if(outs, outs + n_outs, [](const Span& s) { return s.hi == s.lo; });
  std::sort(outs, end, [](const Span& a, const Span& b) { return a.lo < b.lo; });
  for (Span* o = outs + 1; o < end; ++o)
    if (o[-1].hi > o->lo) {
      fail(CCL_SIM_INVALID_ARGUMENT, "output buffers of ranks %d and %d overlap", o[-1].rank, o->rank);
      return false;
    }
  for (int i = 0; i < n_ins; ++i) {
    const Span& in = ins[i];
    if (in.hi == in.lo) continue;
    const Span* it = std::upper_bound(outs, end, in.lo, [](uintptr_t v, const Span& s) { return v < s.hi; });
    for (; it != end && it->lo < in.hi; ++it) {
      if (it->rank != in.rank || !allowed(in.rank)) {
        fail(CCL_SIM_INVALID_ARGUMENT, "input of rank %d overlaps the output of rank %d outside the in-place form",
             in.rank, it->rank);
        return false;
      }
    }
  }
  return true;
}

bool spans_clear_of(const Span* spans, int n, uintptr_t lo, uintptr_t hi) {
  for (int i = 0; i < n; ++i)
    if (spans[i].hi > spans[i].lo && spans[i].lo < hi && lo < spans[i].hi) return false;
  return true;
}

ccl_sim_result_t check_ptrs(const void* const* ptrs, int nranks, const char* what, size_t es) {
  if (ptrs == nullptr) return fail(CCL_SIM_INVALID_ARGUMENT, "%s array is NULL", what);
  for (int r = 0; r < nranks; ++r) {
    if (ptrs[r] == nullptr) return fail(CCL_SIM_INVALID_ARGUMENT, "%s[%d] is NULL", what, r);
    if (reinterpret_cast<uintptr_t>(ptrs[r]) % es != 0)
      return fail(CCL_SIM_INVALID_ARGUMENT, "%s[%d] is not aligned to the element size (%zu bytes)", what, r, es);
  }
  return CCL_SIM_SUCCESS;
}

// Shared path of the three collectives.
ccl_sim_result_t run_collective(int coll, const void* const* sendbufs, void* const* recvbufs, int nranks,
                                size_t sendcount, size_t recvcount, int dtype, int op, int schedule, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  if (nranks < 1 || nranks > CCL_SIM_MAX_RANKS)
    return fail(CCL_SIM_INVALID_ARGUMENT, "nranks=%d outside [1, %d]", nranks, CCL_SIM_MAX_RANKS);
  if (!valid_dtype(dtype)) return fail(CCL_SIM_INVALID_ARGUMENT, "invalid dtype %d", dtype);
  if (coll != CCL_SIM_COLL_ALL_GATHER && !valid_op(op)) return fail(CCL_SIM_INVALID_ARGUMENT, "invalid op %d", op);
  if (!valid_sched(schedule)) return fail(CCL_SIM_INVALID_ARGUMENT, "invalid schedule %d", schedule);
  if (recursive(schedule) && !pow2(nranks))
    return fail(CCL_SIM_UNSUPPORTED, "the recursive halving schedule needs a power-of-two nranks (got %d)", nranks);
  const Env knobs = env();
  if (effective_schedule(nranks, schedule) == CCL_SIM_RING_PERSISTENT &&
      (knobs.per_cu < 0 || knobs.per_cu > kMaxPersistentPerCu))
    return fail(CCL_SIM_UNSUPPORTED,
                "CCL_SIM_PERSISTENT_BLOCKS_PER_CU=%d: the persistent ring runs 1 to %d workgroups per CU (0 = the "
                "default); larger grids are not known to be co-resident",
                knobs.per_cu, kMaxPersistentPerCu);
  if (effective_schedule(nranks, schedule) == CCL_SIM_RING_PERSISTENT && knobs.sync < 0)
    return fail(CCL_SIM_INVALID_ARGUMENT, "CCL_SIM_PERSISTENT_SYNC=\"%.64s\": expected grid, flags or auto",
                knobs.sync_text);
  const size_t es = elem_size(dtype);

  // Counts ([DECOMP] §源码一 count rules; §Contract 实验四 capacity check).
  uint64_t m = 0, q = 0, in_len = 0, out_len = 0;
  if (coll == CCL_SIM_COLL_REDUCE_SCATTER) {
    uint64_t need = 0;
    // The capacity check of [DECOMP] §Contract 实验四: every rank's input
    // must hold exactly one recvcount-element shard per rank.
    if (__builtin_mul_overflow(uint64_t(recvcount), uint64_t(nranks), &need) || need != sendcount)
      return fail(CCL_SIM_CAPACITY_MISMATCH, "sendcount (%zu) != nranks (%d) x recvcount (%zu)", sendcount, nranks,
                  recvcount);
    m = sendcount;
    q = recvcount;
    in_len = sendcount;
    out_len = recvcount;
  } else if (coll == CCL_SIM_COLL_ALL_GATHER) {
    uint64_t have = 0;
    if (!__builtin_mul_overflow(uint64_t(sendcount), uint64_t(nranks), &have) && recvcount > have)
      return fail(CCL_SIM_CAPACITY_MISMATCH,
                  "output tensor larger than input size times world size (sendcount=%zu, nranks=%d, recvcount=%zu)",
                  sendcount, nranks, recvcount);
    m = recvcount;
    q = sendcount;
    in_len = sendcount;
    out_len = recvcount;
  } else {
    m = sendcount;
    q = shard_len(m, nranks);
    in_len = out_len = sendcount;
  }
  uint64_t bytes_tmp = 0;
  if (__builtin_mul_overflow(in_len, uint64_t(es), &bytes_tmp) || __builtin_mul_overflow(out_len, uint64_t(es), &bytes_tmp))
    return fail(CCL_SIM_INVALID_ARGUMENT, "buffer size in bytes overflows");
  if (out_len == 0) return CCL_SIM_SUCCESS;  // nothing to compute or store

  ccl_sim_result_t rc = check_ptrs(sendbufs, nranks, "sendbufs", es);
  if (rc != CCL_SIM_SUCCESS) return rc;
  rc = check_ptrs(const_cast<const void* const*>(recvbufs), nranks, "recvbufs", es);
  if (rc != CCL_SIM_SUCCESS) return rc;

  Span ins[CCL_SIM_MAX_RANKS], outs[CCL_SIM_MAX_RANKS];
  for (int r = 0; r < nranks; ++r) {
    const uintptr_t s = reinterpret_cast<uintptr_t>(sendbufs[r]);
    const uintptr_t d = reinterpret_cast<uintptr_t>(recvbufs[r]);
    ins[r] = Span{s, s + in_len * es, r};
    outs[r] = Span{d, d + out_len * es, r};
  }
  auto in_place = [&](int r) -> bool {
    const uintptr_t s = ins[r].lo, d = outs[r].lo;
    if (coll == CCL_SIM_COLL_ALLREDUCE) return s == d;
    if (coll == CCL_SIM_COLL_REDUCE_SCATTER) return d == s + uint64_t(r) * q * es;
    return s == d + uint64_t(r) * q * es;
  };
  // in_place() reads the spans' original order: sort a copy of the outputs
  Span sorted_outs[CCL_SIM_MAX_RANKS];
  std::copy(outs, outs + nranks, sorted_outs);
  if (!overlap_ok(sorted_outs, nranks, ins, nranks, in_place)) return CCL_SIM_INVALID_ARGUMENT;

  const int sched = effective_schedule(nranks, schedule);
  const Layout lay = layout(coll, nranks, m, dtype, schedule);
  if (!lay.ok) return fail(CCL_SIM_INVALID_ARGUMENT, "workspace size overflows");
  if (lay.total > 0) {
    if (workspace == nullptr || workspace_bytes < lay.total)
      return fail(CCL_SIM_INSUFFICIENT_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", lay.total,
                  workspace == nullptr ? size_t(0) : workspace_bytes, workspace == nullptr ? " (NULL)" : "");
    const uintptr_t w = reinterpret_cast<uintptr_t>(workspace);
    if (w % kAlign != 0) return fail(CCL_SIM_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    if (!spans_clear_of(ins, nranks, w, w + lay.total) || !spans_clear_of(outs, nranks, w, w + lay.total))
      return fail(CCL_SIM_INVALID_ARGUMENT, "workspace overlaps a rank buffer");
  }

  // Plan.
  Call c;
  c.coll = coll;
  c.dtype = dtype;
  c.op = op;
  c.schedule = sched;
  c.nranks = nranks;
  c.q = q;
  c.limit = (coll == CCL_SIM_COLL_REDUCE_SCATTER) ? uint64_t(nranks) * q : m;
  c.in_place = true;
  for (int r = 0; r < nranks && c.in_place; ++r) c.in_place = in_place(r);
  char* ws = static_cast<char*>(workspace);
  if (lay.partial != SIZE_MAX) c.partial = ws + lay.partial;
  if (lay.ctrl != SIZE_MAX) c.ctrl = reinterpret_cast<unsigned*>(ws + lay.ctrl);
  c.stream = stream;
  c.persistent_per_cu = knobs.per_cu;
  c.persistent_sync = knobs.sync;
  c.line_aligned = (q * es) % kLine == 0 && (q * accum_size(dtype)) % kLine == 0;
  for (int r = 0; r < nranks && c.line_aligned; ++r)
    c.line_aligned = ins[r].lo % kLine == 0 && outs[r].lo % kLine == 0;
  c.spin_limit = knobs.spin_limit;
  c.log_plan = knobs.debug;

  hipError_t e = device_cus(&c.num_cus);
  if (e != hipSuccess) return fail(CCL_SIM_HIP_ERROR, "device query failed: %s", hipGetErrorString(e));

  if (nranks <= kInlineRanks) {
    for (int r = 0; r < nranks; ++r) {
      c.send.p[r] = sendbufs[r];
      c.recv.p[r] = recvbufs[r];
    }
  } else {
    const void** st = reinterpret_cast<const void**>(ws + lay.send_tab);
    const void** rt = reinterpret_cast<const void**>(ws + lay.recv_tab);
    e = upload_table(st, sendbufs, nranks, stream);
    if (e == hipSuccess) e = upload_table(rt, const_cast<const void* const*>(recvbufs), nranks, stream);
    if (e != hipSuccess) return fail(CCL_SIM_HIP_ERROR, "pointer table upload failed: %s", hipGetErrorString(e));
    c.send.table = reinterpret_cast<const uint64_t*>(st);
    c.recv.table = reinterpret_cast<const uint64_t*>(rt);
  }

  if (c.log_plan && c.partial != nullptr) {
    e = poison_fill(c.partial, lay.total - lay.partial, stream);
    if (e != hipSuccess) return fail(CCL_SIM_HIP_ERROR, "scratch poison fill failed: %s", hipGetErrorString(e));
  }

  if (sched == CCL_SIM_DIRECT) {
    e = run_direct(c);
  } else if (sched == CCL_SIM_RING_STEPWISE) {
    e = run_ring_stepwise(c);
  } else if (sched == CCL_SIM_RECURSIVE) {
    e = run_recursive(c);
  } else if (sched == CCL_SIM_RING_CHAINED) {
    e = run_ring_chained(c);
  } else if (sched == CCL_SIM_RECURSIVE_CHAINED) {
    e = run_recursive_chained(c);
  } else {
    bool unsupported = false;
    PersistentPlan plan;
    e = run_ring_persistent(c, &unsupported, &plan);
    if (e == hipSuccess && unsupported)
      return plan.refused != hipSuccess
                 ? fail(CCL_SIM_UNSUPPORTED,
                        "the runtime refused the persistent ring's cooperative launch (%s); another process on "
                        "this GPU may hold the device's cooperative launch resources",
                        hipGetErrorString(plan.refused))
                 : fail(CCL_SIM_UNSUPPORTED, "no co-resident grid for the persistent ring kernel on this device");
    if (c.log_plan)
      std::fprintf(stderr,
                   "[ccl_sim] persistent coll=%d N=%d q=%llu cus=%d occupancy/cu=%d used/cu=%d grid=%llu lanes=%d "
                   "tiles/step=%llu coherent=%d sync=%s same_xcd_reads=%d\n",
                   coll, nranks, static_cast<unsigned long long>(q), c.num_cus, plan.occupancy_per_cu, plan.per_cu,
                   static_cast<unsigned long long>(plan.grid), plan.lanes,
                   static_cast<unsigned long long>(plan.tiles_per_step), plan.coherent ? 1 : 0,
                   plan.flags ? "flags" : "grid", plan.flags && c.line_aligned ? 1 : 0);
    if (e == hipSuccess && c.log_plan) {
      // Debug check of the watchdog: wait for the kernel and read the abort
      // word it raises when a barrier or flag wait runs into the poll limit.
      unsigned abort_word = 0;
      e = hipStreamSynchronize(stream);
      if (e == hipSuccess)
        e = hipMemcpy(&abort_word, c.ctrl + kCtrlAbort, sizeof(abort_word), hipMemcpyDeviceToHost);
      if (e == hipSuccess && abort_word != 0)
        return fail(CCL_SIM_HIP_ERROR, "persistent ring wait reached its poll limit; the results are incomplete");
    }
  }
  if (e != hipSuccess) return fail(CCL_SIM_HIP_ERROR, "kernel launch failed: %s", hipGetErrorString(e));
  if (c.log_plan)
    std::fprintf(stderr, "[ccl_sim] coll=%d sched=%d N=%d M=%llu q=%llu dtype=%d op=%d in_place=%d tables=%d\n", coll,
                 sched, nranks, static_cast<unsigned long long>(m), static_cast<unsigned long long>(q), dtype, op,
                 int(c.in_place), int(nranks > kInlineRanks));
  return CCL_SIM_SUCCESS;
}

}  // namespace

extern "C" {

ccl_sim_result_t ccl_sim_reduce_scatter(const void* const* sendbufs, void* const* recvbufs, int nranks,
                                        size_t sendcount, size_t recvcount, ccl_sim_dtype_t dtype, ccl_sim_op_t op,
                                        ccl_sim_schedule_t schedule, void* workspace, size_t workspace_bytes,
                                        ccl_sim_stream_t stream) {
  return run_collective(CCL_SIM_COLL_REDUCE_SCATTER, sendbufs, recvbufs, nranks, sendcount, recvcount, dtype, op,
                        schedule, workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream));
}

ccl_sim_result_t ccl_sim_all_gather(const void* const* sendbufs, void* const* recvbufs, int nranks, size_t sendcount,
                                    size_t recvcount, ccl_sim_dtype_t dtype, ccl_sim_schedule_t schedule,
                                    void* workspace, size_t workspace_bytes, ccl_sim_stream_t stream) {
  return run_collective(CCL_SIM_COLL_ALL_GATHER, sendbufs, recvbufs, nranks, sendcount, recvcount, dtype, CCL_SIM_SUM,
                        schedule, workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream));
}

ccl_sim_result_t ccl_sim_allreduce(const void* const* sendbufs, void* const* recvbufs, int nranks, size_t count,
                                   ccl_sim_dtype_t dtype, ccl_sim_op_t op, ccl_sim_schedule_t schedule,
                                   void* workspace, size_t workspace_bytes, ccl_sim_stream_t stream) {
  return run_collective(CCL_SIM_COLL_ALLREDUCE, sendbufs, recvbufs, nranks, count, count, dtype, op, schedule,
                        workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream));
}

ccl_sim_result_t ccl_sim_allreduce_noalloc(const void* const* sendbufs, void* const* recvbufs, int nranks,
                                           size_t count, ccl_sim_dtype_t dtype, ccl_sim_op_t op,
                                           ccl_sim_schedule_t schedule, ccl_sim_stream_t stream) {
  clear_error();
  if (count == 0) return CCL_SIM_SUCCESS;  // nothing to compute, scratch untouched
  if (nranks >= 1 && nranks <= CCL_SIM_MAX_RANKS && valid_dtype(dtype) && valid_sched(schedule) &&
      !(recursive(schedule) && !pow2(nranks))) {
    if (effective_schedule(nranks, schedule) == CCL_SIM_RING_PERSISTENT)
      return fail(CCL_SIM_UNSUPPORTED,
                  "the persistent ring is not offered without a workspace: its abort word could not be queried");
    const Layout lay = layout(CCL_SIM_COLL_ALLREDUCE, nranks, count, dtype, schedule);
    if (!lay.ok || lay.total > CCL_SIM_NOALLOC_SCRATCH_BYTES)
      return fail(CCL_SIM_INSUFFICIENT_WORKSPACE,
                  "this call needs a workspace of %zu bytes; the library's scratch holds %zu",
                  lay.ok ? lay.total : SIZE_MAX, CCL_SIM_NOALLOC_SCRATCH_BYTES);
    if (lay.total > 0) {
      void* scratch = nullptr;
      size_t bytes = 0;
      const hipError_t e = noalloc_scratch(&scratch, &bytes);
      if (e != hipSuccess)
        return fail(CCL_SIM_HIP_ERROR, "reading the scratch's device address failed: %s", hipGetErrorString(e));
      return run_collective(CCL_SIM_COLL_ALLREDUCE, sendbufs, recvbufs, nranks, count, count, dtype, op, schedule,
                            scratch, bytes, reinterpret_cast<hipStream_t>(stream));
    }
  }
  // no scratch needed, or invalid arguments (which run_collective reports)
  return run_collective(CCL_SIM_COLL_ALLREDUCE, sendbufs, recvbufs, nranks, count, count, dtype, op, schedule, nullptr,
                        0, reinterpret_cast<hipStream_t>(stream));
}

ccl_sim_result_t ccl_sim_pad_identity(const void* const* srcs, void* const* dsts, int nranks, size_t count,
                                      size_t padded_count, ccl_sim_dtype_t dtype, ccl_sim_op_t op,
                                      ccl_sim_stream_t stream) {
  clear_error();
  if (nranks < 1 || nranks > CCL_SIM_MAX_RANKS)
    return fail(CCL_SIM_INVALID_ARGUMENT, "nranks=%d outside [1, %d]", nranks, CCL_SIM_MAX_RANKS);
  if (!valid_dtype(dtype)) return fail(CCL_SIM_INVALID_ARGUMENT, "invalid dtype %d", int(dtype));
  if (!valid_op(op)) return fail(CCL_SIM_INVALID_ARGUMENT, "invalid op %d", int(op));
  if (padded_count < count)
    return fail(CCL_SIM_INVALID_ARGUMENT, "padded_count=%zu is smaller than count=%zu", padded_count, count);
  const size_t es = elem_size(dtype);
  uint64_t tmp = 0;
  if (__builtin_mul_overflow(uint64_t(padded_count), uint64_t(es), &tmp))
    return fail(CCL_SIM_INVALID_ARGUMENT, "buffer size in bytes overflows");
  if (padded_count == 0) return CCL_SIM_SUCCESS;
  ccl_sim_result_t rc = CCL_SIM_SUCCESS;
  if (count > 0) {
    rc = check_ptrs(srcs, nranks, "srcs", es);
    if (rc != CCL_SIM_SUCCESS) return rc;
  }
  rc = check_ptrs(const_cast<const void* const*>(dsts), nranks, "dsts", es);
  if (rc != CCL_SIM_SUCCESS) return rc;
  Span ins[CCL_SIM_MAX_RANKS], outs[CCL_SIM_MAX_RANKS];
  int n_ins = 0;
  for (int r = 0; r < nranks; ++r) {
    const uintptr_t d = reinterpret_cast<uintptr_t>(dsts[r]);
    outs[r] = Span{d, d + padded_count * es, r};
    if (count > 0) {
      const uintptr_t s = reinterpret_cast<uintptr_t>(srcs[r]);
      ins[n_ins++] = Span{s, s + count * es, r};
    }
  }
  auto same = [&](int r) { return count == 0 || srcs[r] == dsts[r]; };
  if (!overlap_ok(outs, nranks, ins, n_ins, same)) return CCL_SIM_INVALID_ARGUMENT;

  Call c;
  c.dtype = dtype;
  c.op = op;
  c.stream = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = device_cus(&c.num_cus);
  if (e != hipSuccess) return fail(CCL_SIM_HIP_ERROR, "device query failed: %s", hipGetErrorString(e));
  for (int base = 0; base < nranks; base += kInlineRanks) {
    const int n = std::min(kInlineRanks, nranks - base);
    c.nranks = n;
    for (int i = 0; i < n; ++i) {
      c.send.p[i] = count > 0 ? srcs[base + i] : dsts[base + i];
      c.recv.p[i] = dsts[base + i];
    }
    e = run_pad(c, count, padded_count);
    if (e != hipSuccess) return fail(CCL_SIM_HIP_ERROR, "kernel launch failed: %s", hipGetErrorString(e));
  }
  return CCL_SIM_SUCCESS;
}

size_t ccl_sim_workspace_size(ccl_sim_coll_t coll, int nranks, size_t count, ccl_sim_dtype_t dtype,
                              ccl_sim_schedule_t schedule) {
  if (!valid_coll(coll) || nranks < 1 || nranks > CCL_SIM_MAX_RANKS || !valid_dtype(dtype) || !valid_sched(schedule))
    return SIZE_MAX;
  const Layout l = layout(coll, nranks, count, dtype, schedule);
  return l.ok ? l.total : SIZE_MAX;
}

uint64_t ccl_sim_algorithmic_bytes(ccl_sim_coll_t coll, int nranks, size_t count, ccl_sim_dtype_t dtype,
                                   ccl_sim_schedule_t schedule) {
  if (!valid_coll(coll) || nranks < 1 || nranks > CCL_SIM_MAX_RANKS || !valid_dtype(dtype) || !valid_sched(schedule))
    return 0;
  const uint64_t n = uint64_t(nranks), m = count, s = elem_size(dtype), a = accum_size(dtype);
  const int sched = effective_schedule(nranks, schedule);
  if (sched == CCL_SIM_DIRECT) {
    if (coll == CCL_SIM_COLL_ALLREDUCE) return 2 * n * m * s;
    return (n + 1) * m * s;
  }
  if (coll == CCL_SIM_COLL_ALL_GATHER) return 2 * n * m * s;
  if (recursive(sched)) {
    if (!pow2(nranks)) return 0;
    // halving step j: every position is reduced by N/2^j ranks, each reading
    // two partials (the inputs at step 1) and writing one (the output at the
    // last step)
    const int k = log2i(nranks);
    uint64_t bytes = 0;
    for (int j = 1; j <= k; ++j) {
      const uint64_t in = (j == 1) ? 2 * s : 2 * a;
      const uint64_t out = (j == k) ? s : a;
      bytes += (n >> j) * m * (in + out);
    }
    if (coll == CCL_SIM_COLL_ALLREDUCE) bytes += 2 * (n - 1) * m * s;
    return bytes;
  }
  // ReduceScatter phase: per step every position reads the incoming partial
  // (stored type at the first step) and the own element, and writes the new
  // partial (stored type at the last step).
  uint64_t per_pos = 0;
  for (int t = 0; t + 1 < nranks; ++t) {
    const uint64_t in = (t == 0) ? s : a;
    const uint64_t out = (t == nranks - 2) ? s : a;
    per_pos += in + s + out;
  }
  uint64_t bytes = per_pos * m;
  if (coll == CCL_SIM_COLL_ALLREDUCE) bytes += 2 * (n - 1) * m * s;
  return bytes;
}

int ccl_sim_launch_count(ccl_sim_coll_t coll, int nranks, size_t count, ccl_sim_schedule_t schedule, int in_place) {
  if (!valid_coll(coll) || nranks < 1 || nranks > CCL_SIM_MAX_RANKS || !valid_sched(schedule)) return -1;
  if (count == 0) return 0;
  const int sched = effective_schedule(nranks, schedule);
  if (sched == CCL_SIM_RECURSIVE_CHAINED) return pow2(nranks) ? 1 : -1;
  if (sched == CCL_SIM_DIRECT || sched == CCL_SIM_RING_PERSISTENT || sched == CCL_SIM_RING_CHAINED) return 1;
  if (sched == CCL_SIM_RECURSIVE) {
    if (!pow2(nranks)) return -1;
    const int k = log2i(nranks);
    if (coll == CCL_SIM_COLL_ALLREDUCE) return 2 * k;
    if (coll == CCL_SIM_COLL_REDUCE_SCATTER) return k;
    return in_place ? k : k + 1;
  }
  if (coll == CCL_SIM_COLL_ALLREDUCE) return 2 * (nranks - 1);
  if (coll == CCL_SIM_COLL_REDUCE_SCATTER) return nranks - 1;
  return in_place ? nranks - 1 : nranks;
}

int ccl_sim_ring_owner(int nranks, int rank) {
  if (nranks < 1 || nranks > CCL_SIM_MAX_RANKS || rank < 0 || rank >= nranks) return -1;
  return (rank + 1) % nranks;
}

ccl_sim_result_t ccl_sim_ring_route(int nranks, int phase, int step, int rank, int* send_chunk, int* recv_chunk) {
  if (nranks < 1 || nranks > CCL_SIM_MAX_RANKS || rank < 0 || rank >= nranks || step < 0 || step > nranks - 2 ||
      phase < 0 || phase > 2 || send_chunk == nullptr || recv_chunk == nullptr)
    return CCL_SIM_INVALID_ARGUMENT;
  const int owner = (phase == 1) ? 1 : 0;  // phase 0 and 2 share the (r - t, r - 1 - t) form
  auto mod = [nranks](int x) { return ((x % nranks) + nranks) % nranks; };
  *send_chunk = mod(rank + owner - step);
  *recv_chunk = mod(rank + owner - 1 - step);
  return CCL_SIM_SUCCESS;
}

ccl_sim_result_t ccl_sim_recursive_route(int nranks, int phase, int step, int rank, int* partner,
                                         size_t* first_block, size_t* nblocks) {
  if (!pow2(nranks) || rank < 0 || rank >= nranks || partner == nullptr || first_block == nullptr ||
      nblocks == nullptr)
    return CCL_SIM_INVALID_ARGUMENT;
  const int k = log2i(nranks);
  if (phase == 0 && step >= 1 && step <= k) {
    const int d = nranks >> step;
    *partner = rank ^ d;
    *first_block = size_t(rank & ((nranks - 1) & ~(d - 1)));
    *nblocks = size_t(d);
    return CCL_SIM_SUCCESS;
  }
  if (phase == 1 && step >= 0 && step < k) {
    const int p = rank ^ (1 << step);
    *partner = p;
    *first_block = size_t((p >> step) << step);
    *nblocks = size_t(1) << step;
    return CCL_SIM_SUCCESS;
  }
  return CCL_SIM_INVALID_ARGUMENT;
}

const char* ccl_sim_result_string(ccl_sim_result_t result) {
  switch (result) {
    case CCL_SIM_SUCCESS: return "success";
    case CCL_SIM_INVALID_ARGUMENT: return "invalid argument";
    case CCL_SIM_UNSUPPORTED: return "unsupported on this device";
    case CCL_SIM_INSUFFICIENT_WORKSPACE: return "insufficient workspace";
    case CCL_SIM_HIP_ERROR: return "HIP runtime error";
    case CCL_SIM_CAPACITY_MISMATCH: return "capacity mismatch";
    default: return "unknown result code";
  }
}

const char* ccl_sim_last_error(void) { return g_last_error; }

int ccl_sim_persistent_ordering(ccl_sim_coll_t coll, int nranks, size_t count) {
  if (!valid_coll(coll) || nranks < 1 || nranks > CCL_SIM_MAX_RANKS) return -1;
  const Env knobs = env();
  if (knobs.sync < 0) return -1;
  if (count == 0 || effective_schedule(nranks, CCL_SIM_RING_PERSISTENT) != CCL_SIM_RING_PERSISTENT) return 0;
  return persistent_uses_flags(nranks, shard_len(count, nranks), knobs.sync) ? CCL_SIM_ORDER_FLAGS
                                                                             : CCL_SIM_ORDER_GRID;
}

ccl_sim_result_t ccl_sim_persistent_aborted(const void* workspace, int* aborted) {
  clear_error();
  if (workspace == nullptr || aborted == nullptr)
    return fail(CCL_SIM_INVALID_ARGUMENT, "workspace and aborted must not be NULL");
  // The control block opens the persistent ring's workspace (layout()).
  unsigned word = 0;
  const hipError_t e = hipMemcpy(&word, static_cast<const unsigned*>(workspace) + kCtrlAbort, sizeof(word),
                                 hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(CCL_SIM_HIP_ERROR, "reading the abort word failed: %s", hipGetErrorString(e));
  *aborted = word != 0 ? 1 : 0;
  return CCL_SIM_SUCCESS;
}

int ccl_sim_version(void) { return CCL_SIM_VERSION; }

}  // extern "C"
