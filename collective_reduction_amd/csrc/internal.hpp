// Internal interface between the C-ABI front end (api.cpp: validation and
// planning) and the kernels (kernels_*.hip: launches).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace ccl {

enum Coll : int { kReduceScatter = 0, kAllGather = 1, kAllReduce = 2 };
enum DT : int { kInt32 = 0, kInt64 = 1, kFloat32 = 2, kBFloat16 = 3 };
enum Sched : int { kDirect = 0, kRingStepwise = 1, kRingPersistent = 2, kRecursive = 3, kRingChained = 4, kRecursiveChained = 5 };

// Everything a launch needs, already validated.
struct Call {
  int coll = 0, dtype = 0, op = 0, schedule = 0;
  int nranks = 0;
  uint64_t q = 0;          // shard (= ring chunk) length in elements
  uint64_t limit = 0;      // positions >= limit are padding (AllReduce) or trimmed (AllGather)
  bool in_place = false;   // AllGather: sendbufs[r] == recvbufs[r] + r·sendcount for every r
  RankPtrs send{}, recv{};
  void* partial = nullptr; // ring partials [2][nranks][q], or recursive-halving scratch [nranks][nranks/2·q]
  unsigned* ctrl = nullptr;// persistent ring: barrier counters, abort word and step flags
  hipStream_t stream = nullptr;
  int num_cus = 0;
  // Persistent ring: workgroups per compute unit (0 = the default), how
  // its steps are ordered (PersistSync), the poll limit of its waits, and
  // whether to log the launch plan to stderr.
  int persistent_per_cu = 0;
  int persistent_sync = 0;
  // Every rank buffer starts on a 128-byte line and a chunk (q elements,
  // and q accumulators) is a whole number of lines, so no line holds data
  // of two chunks (the flag-ordered persistent ring reads from an L2 only
  // then).
  bool line_aligned = false;
  unsigned spin_limit = 0;
  bool log_plan = false;
};

// Grid actually launched by run_ring_persistent (for diagnostics).
struct PersistentPlan {
  int occupancy_per_cu = 0;
  int per_cu = 0;
  uint64_t grid = 0;
  uint64_t tiles_per_step = 0;
  int lanes = 0;  // threads per workgroup
  hipError_t refused = hipSuccess;  // the cooperative launch's error when the runtime refused it
  bool coherent = false;            // agent-coherent data path, waits without cache maintenance
  bool flags = false;               // steps ordered by per-workgroup flags, not a grid barrier
};

// How the persistent ring orders its steps: by the library's choice from
// the step size, by a grid barrier between steps, or by per-workgroup step
// flags (each workgroup waits only for the workgroups whose data its next
// step reads).
enum PersistSync : int { kSyncAuto = 0, kSyncGrid = 1, kSyncFlags = 2 };

// Barrier groups of the persistent ring's two-level arrival.  Measured
// side by side at N = 256 (256 workgroups): 4 groups 1-1.5 % faster than 8
// in float32 and bf16, 2 and 3 within 1 % of 8, 1 group 8 % slower, 16 and
// 32 groups 5-19 % slower; no difference at N = 8.
#ifndef CCL_SIM_CTRL_GROUPS
#define CCL_SIM_CTRL_GROUPS 4
#endif

// Control block of the persistent ring (unsigned words): line 0 holds the
// global arrival counter and the abort word, line 1 + g the arrival counter
// of barrier group g (a line is 128 bytes), and from kCtrlFlags on one step
// flag per workgroup of the flag-ordered form, which launches at most
// kCtrlMaxFlags workgroups (4 per CU on a 1024-CU device).
enum CtrlWord : int {
  kCtrlBarrier = 0,
  kCtrlAbort = 1,
  kCtrlLine = 32,
  kCtrlGroups = CCL_SIM_CTRL_GROUPS,
  kCtrlGroup = kCtrlLine,
  kCtrlFlags = kCtrlLine * (1 + kCtrlGroups),
  kCtrlMaxFlags = 4096,
  kCtrlWords = kCtrlFlags + kCtrlMaxFlags,
};

hipError_t run_direct(const Call& c);
hipError_t run_ring_stepwise(const Call& c);
// Sets *unsupported when no co-resident grid can be formed.
hipError_t run_ring_persistent(const Call& c, bool* unsupported, PersistentPlan* plan);
// Whether the persistent ring orders a call's steps by flags (else by the
// grid barrier): `sync` is the caller's PersistSync, q the chunk length.
bool persistent_uses_flags(int nranks, uint64_t q, int sync);
hipError_t run_recursive(const Call& c);
hipError_t run_ring_chained(const Call& c);
hipError_t run_recursive_chained(const Call& c);
hipError_t run_pad(const Call& c, uint64_t count, uint64_t padded);
// Copy `n` host-side pointers into a device table on the stream (kernel
// arguments carry them; no host-to-device memcpy).
hipError_t upload_table(const void** dev_table, const void* const* host_ptrs, int n, hipStream_t stream);

// Debug check of the scratch (CCL_SIM_DEBUG): all-ones bits over `bytes`
// (a multiple of 4) on the stream, before a schedule that keeps partials
// there runs.
hipError_t poison_fill(void* p, size_t bytes, hipStream_t stream);

// Device address and size of the current device's library-owned scratch
// (scratch.hip), read once per device.
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

size_t elem_size(int dtype);
size_t accum_size(int dtype);

}  // namespace ccl
