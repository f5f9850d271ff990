// Ring schedule: one launch per step, one persistent cooperative kernel
// whose steps are ordered by a grid barrier or by per-workgroup step flags,
// or each chunk's steps chained in one launch.

#include "kernel_common.hpp"

namespace ccl {
namespace {

// ---------------------------------------------------------------------------
// Ring schedule ([RING] §1 and pseudocode; [PRIMS] §五.2-五.3).
//
// Global step numbering of one call:
//   AllReduce      steps 0..N-2 ReduceScatter phase (t = step),
//                  steps N-1..2N-3 AllGather phase (t = step - (N-1));
//   ReduceScatter  steps 0..N-2;
//   AllGather      step 0 places each rank's own shard, steps 1..N-1 copy.
// Each step is N independent transfers, one per rank; a tile belongs to one
// rank's transfer.  "Send" and "receive" are HBM reads of the upstream
// rank's data; the ReduceScatter phase's in-flight partials live in a
// double buffer P[2][N][q] of accumulators (rank r's slot of step t is read
// by rank r+1 at step t+1, so two generations are live at once), or, for
// the chained ring, in P[N][q] keyed by chunk (chunk c's partial moves
// from rank to rank in place; only chunk c's own chain touches it).
// ---------------------------------------------------------------------------
struct RingArgs {
  RankPtrs send, recv;
  int nranks;
  int coll;
  int step;                  // the step a stepwise launch runs
  int first_step;            // persistent: 1 skips an in-place AllGather's placement
  uint64_t q;                // chunk length
  uint64_t limit;            // positions at or past it are padding / trimmed
  uint64_t tiles_per_chunk;
  uint64_t ntiles;           // nranks · tiles_per_chunk
  void* partial;
  int chunk_keyed;           // partials keyed by chunk (chained ring) instead of [step parity][rank]
  unsigned* ctrl;
  unsigned spin_limit;
  int xcd_map;               // flag-ordered persistent ring: ring neighbours placed on one XCD
  int xcd_loads;             // flag-ordered persistent ring: L2 reads allowed (no line spans two chunks)
  // Flag-ordered persistent ring, modulo the grid size G: G - T mod G
  // (T = tiles_per_chunk), (ntiles - T) mod G and ntiles mod G.
  unsigned up_back, up_wrap, ntiles_mod;
};

__device__ inline int mod_n(int x, int n) {
  x %= n;
  return x < 0 ? x + n : x;
}

__device__ inline uint64_t chunk_len(const RingArgs& a, int c) {
  const uint64_t base = uint64_t(c) * a.q;
  if (base >= a.limit) return 0;
  return a.limit - base < a.q ? a.limit - base : a.q;
}

// ReduceScatter step t for rank r: receive chunk c = (r-1-t) from rank r-1
// and combine the rank's own x^(r) chunk into it (incoming partial on the
// left, so chunk c folds x^(c), x^(c+1), ...).  At t = 0 the incoming
// partial is rank r-1's own input; at the last step t = N-2 the completed
// chunk is stored as output instead of a partial: AllReduce into
// out_r[chunk c] (the AllGather phase's source: the phase boundary fused
// in one state machine as in [DECOMP] §源码三), ReduceScatter into
// recvbufs[c], c = r+1.
template <class T, int OP, class P, bool FULL, bool CO, bool XCD = false>
__device__ inline void ring_rs_tile(const RingArgs& a, int t, int r, uint64_t seg, int c, uint64_t len,
                                    const typename Lane<T, P, FULL, CO, XCD>::SV* own_ahead = nullptr) {
  using A = typename T::A;
  using L = Lane<T, P, FULL, CO, XCD>;
  constexpr int V = vec_elems<T>();
  const int n = a.nranks;
  const int up = mod_n(r - 1, n);
  const uint64_t cbase = uint64_t(c) * a.q;
  const bool last = (t == n - 2);
  A* part = static_cast<A*>(a.partial);
  const uint64_t slot = uint64_t(n) * a.q;  // elements per generation
  const L ln(seg, len);
  typename L::AV in[P::U];
  typename L::SV own[P::U];
  const typename T::S* mine = in_ptr<T>(a.send, r) + cbase;
  if (t == 0) {
    const typename T::S* theirs = in_ptr<T>(a.send, up) + cbase;
#pragma unroll
    for (int u = 0; u < P::U; ++u)
      if (ln.on(u)) {
        const typename L::SV x = ln.load(theirs, u);
#pragma unroll
        for (int k = 0; k < V; ++k) in[u][k] = T::widen(x[k]);
      }
  } else {
    const A* theirs = part + (a.chunk_keyed ? cbase : uint64_t((t - 1) & 1) * slot + uint64_t(up) * a.q);
#pragma unroll
    for (int u = 0; u < P::U; ++u)
      if (ln.on(u)) in[u] = ln.load_part(theirs, u);
  }
#pragma unroll
  for (int u = 0; u < P::U; ++u)
    if (ln.on(u)) own[u] = own_ahead ? own_ahead[u] : ln.load(mine, u);
  if (!last) {
    A* dst = part + (a.chunk_keyed ? cbase : uint64_t(t & 1) * slot + uint64_t(r) * a.q);
#pragma unroll
    for (int u = 0; u < P::U; ++u) {
      if (!ln.on(u)) continue;
      typename L::AV v;
#pragma unroll
      for (int k = 0; k < V; ++k) v[k] = combine<T, OP>(in[u][k], T::widen(own[u][k]));
      ln.store_part(dst, u, v);
    }
  } else {
    typename T::S* dst = (a.coll == kAllReduce) ? out_ptr<T>(a.recv, r) + cbase : out_ptr<T>(a.recv, c);
#pragma unroll
    for (int u = 0; u < P::U; ++u) {
      if (!ln.on(u)) continue;
      typename L::SV v;
#pragma unroll
      for (int k = 0; k < V; ++k) v[k] = T::narrow(finalize<T, OP>(combine<T, OP>(in[u][k], T::widen(own[u][k])), n));
      ln.store(dst, u, v);
    }
  }
}

// CO: agent-coherent data accesses (the persistent ring, whose waits then
// need no cache maintenance; see load_vec_coherent).
//
// AT: the tile is given as (rank r_at, tile seg_at of the chunk), which the
// flag-ordered persistent kernel computes once per call for a workgroup's
// first tile; otherwise it is found from `tile`.  (One body for both: a
// separate function for the (rank, segment) form measured 3 % slower in
// the fenced persistent kernel at N = 8, M = 2^28, where the compiler then
// waited for every store of a tile before starting the next.)
template <class T, int OP, class P, bool CO = false, bool AT = false, bool XCD = false>
__device__ inline void ring_body(const RingArgs& a, int step, uint64_t tile, int r_at = 0, uint64_t seg_at = 0) {
  constexpr uint64_t kTile = tile_of<P>(vec_elems<T>());
  const int n = a.nranks;
  const int r = AT ? r_at : rank_of_tile(tile, a.tiles_per_chunk);
  const uint64_t seg = AT ? seg_at : tile - uint64_t(r) * a.tiles_per_chunk;
  int c;
  bool reduce = false;
  const typename T::S* src;
  if (a.coll != kAllGather && step < n - 1) {
    // ReduceScatter phase ([PRIMS] §五.2): receive chunk r-1-t.
    reduce = true;
    c = mod_n(r - 1 - step, n);
    src = nullptr;
  } else if (a.coll == kAllGather && step == 0) {
    // Stand-alone AllGather: rank r's own shard into its chunk r
    // (the directCopySend of [DECOMP] §源码四).
    c = r;
    src = in_ptr<T>(a.send, r);
  } else {
    // AllGather phase ([PRIMS] §五.3): receive chunk c from rank r-1 and
    // overwrite the local copy.  After the ring ReduceScatter phase rank r
    // owns chunk r+1, so it receives chunk r-t; a stand-alone AllGather's
    // rank r owns chunk r and receives chunk r-1-t.
    const int t = (a.coll == kAllGather) ? step - 1 : step - (n - 1);
    const int owner = (a.coll == kAllGather) ? 0 : 1;
    c = mod_n(r + owner - 1 - t, n);
    src = in_ptr<T>(a.recv, mod_n(r - 1, n)) + uint64_t(c) * a.q;
  }
  const uint64_t len = chunk_len(a, c);
  const bool full = (seg + 1) * kTile <= len;
  if (reduce) {
    if (full)
      ring_rs_tile<T, OP, P, true, CO, XCD>(a, step, r, seg, c, len);
    else
      ring_rs_tile<T, OP, P, false, CO, XCD>(a, step, r, seg, c, len);
  } else {
    typename T::S* dst = out_ptr<T>(a.recv, r) + uint64_t(c) * a.q;
    if (full)
      copy_tile<T, P, true, CO, XCD>(src, dst, seg, len);
    else
      copy_tile<T, P, false, CO, XCD>(src, dst, seg, len);
  }
}

template <class T, int OP, class P>
__global__ __launch_bounds__(P::TB) void ring_step_kernel(RingArgs a) {
  for (uint64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) ring_body<T, OP, P>(a, a.step, tile);
}

// The rank that handles chunk c at a global step: the inverse of the chunk
// a rank handles in ring_body.
__device__ inline int ring_rank_at(const RingArgs& a, int step, int c) {
  const int n = a.nranks;
  if (a.coll != kAllGather && step < n - 1) return mod_n(c + 1 + step, n);  // ReduceScatter phase
  if (a.coll == kAllGather && step == 0) return c;                          // own-shard placement
  const int t = (a.coll == kAllGather) ? step - 1 : step - (n - 1);
  const int owner = (a.coll == kAllGather) ? 0 : 1;
  return mod_n(c - owner + 1 + t, n);
}

// Chained ring: work item = (chunk c, tile seg of the chunk).  Each step of
// the ring moves chunk c from one rank to the next and reads only what the
// step before wrote for the same chunk and the same positions, so the
// workgroup that owns an item runs all of its steps in order, each step on
// the rank ring_body would give it, with the same lane-to-element mapping:
// every value a step reads was written by the same lane earlier in program
// order, and a lane's own load after its own store to one address sees the
// store (the single-thread coherence all GPU code relies on; no fence is
// involved).  No other item touches chunk c's positions, so items need no
// synchronisation at all.
template <class T, int OP, class P>
__global__ __launch_bounds__(P::TB) void ring_chained_kernel(RingArgs a) {
  const int nsteps = (a.coll == kAllReduce) ? 2 * (a.nranks - 1) : (a.coll == kReduceScatter ? a.nranks - 1 : a.nranks);
  for (uint64_t item = blockIdx.x; item < a.ntiles; item += gridDim.x) {
    const int c = rank_of_tile(item, a.tiles_per_chunk);
    const uint64_t seg = item - uint64_t(c) * a.tiles_per_chunk;
    for (int step = a.first_step; step < nsteps; ++step)
      ring_body<T, OP, P>(a, step, uint64_t(ring_rank_at(a, step, c)) * a.tiles_per_chunk + seg);
  }
}

// Grid-wide barrier for the persistent ring, in two halves: grid_arrive
// counts the workgroup in, grid_wait waits for the whole grid, and the
// workgroup may issue loads that depend on no other workgroup in between.
// Every workgroup of the grid is co-resident (cooperative launch) and
// arrives once per barrier.
//
// Arrival is two-level: workgroup b counts itself on the counter of group
// b mod kCtrlGroups (each counter on its own cache line), and the group's
// last arriver of this barrier adds one arrival to the global counter, so
// no counter takes more than about gridDim.x / kCtrlGroups atomics per
// barrier instead of gridDim.x on one address.  Every workgroup then polls
// the global counter until all groups are in.  Counters only grow, so
// barrier number `epoch` (from 1) is complete when group g's counter
// reaches epoch·members(g) and the global counter epoch·groups.
//
// Ordering: each wave waits until its own stores have reached its XCD's L2
// (vmcnt 0) before the workgroup barrier; one lane then issues a release
// fence at agent scope, which writes that L2's dirty lines back to memory,
// before arriving.  A group leader fences acquire-release between the
// group counter and the global counter, which carries its members'
// releases on; after the wait, an acquire fence drops stale L1 / L2 lines.
// A workgroup's stores of one step are therefore seen by every other
// workgroup's loads of the next, across all eight XCDs and their separate
// L2 caches.  Release and acquire are separate one-way fences: a full
// fence on each side would write back and invalidate the caches twice.
//
// The wait is bounded: after spin_limit polls a workgroup raises the abort
// word, and every workgroup that sees the word stops, so the grid always
// drains.
template <bool CO>
__device__ inline void grid_arrive(unsigned* ctrl, unsigned epoch) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned grid = gridDim.x;
    const unsigned g = blockIdx.x % unsigned(kCtrlGroups);
    const unsigned members = (grid - g + kCtrlGroups - 1) / kCtrlGroups;
    if constexpr (!CO) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const unsigned before = __hip_atomic_fetch_add(ctrl + kCtrlGroup + g * kCtrlLine, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
    if (before + 1u == epoch * members) {
      if constexpr (!CO) __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
      __hip_atomic_fetch_add(ctrl + kCtrlBarrier, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <bool CO>
__device__ inline bool grid_wait(unsigned* ctrl, unsigned epoch, unsigned spin_limit) {
  __shared__ int s_ok;
  if (threadIdx.x == 0) {
    int ok = 1;
    unsigned spins = 0;
    const unsigned grid = gridDim.x;
    const unsigned groups = grid < unsigned(kCtrlGroups) ? grid : unsigned(kCtrlGroups);
    while (__hip_atomic_load(ctrl + kCtrlBarrier, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < epoch * groups) {
      if (++spins > spin_limit ||
          ((spins & 63u) == 0u &&
           __hip_atomic_load(ctrl + kCtrlAbort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)) {
        __hip_atomic_store(ctrl + kCtrlAbort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if constexpr (!CO) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_ok = ok;
  }
  __syncthreads();
  return s_ok != 0;
}

// The ReduceScatter-phase tile (rank r, tile seg of the chunk) at a step:
// the chunk it receives, and whether it is a whole tile.
struct RsTileAt {
  int r = 0, c = 0;
  uint64_t seg = 0, len = 0;
  bool full = false;
};
template <class P, class T>
__device__ inline RsTileAt rs_tile_at(const RingArgs& a, int step, int r, uint64_t seg) {
  constexpr uint64_t kTile = tile_of<P>(vec_elems<T>());
  RsTileAt x;
  x.r = r;
  x.seg = seg;
  x.c = mod_n(x.r - 1 - step, a.nranks);
  x.len = chunk_len(a, x.c);
  x.full = (x.seg + 1) * kTile <= x.len;
  return x;
}

#ifndef CCL_SIM_PERSIST_AHEAD
#define CCL_SIM_PERSIST_AHEAD 1
#endif

// CO: the data path is agent-coherent and the barrier does no cache
// maintenance (for small steps, where the barrier dominates, when the
// caller asks for the barrier there; by default small steps take the step
// flags below; see run_ring_persistent).
//
// The barrier is split into its arrival and its wait.  In between, a
// workgroup whose next step is a ReduceScatter step loads the rank's own
// input vectors of its first tile of that step: x^(r) is never written
// during the call at a position the ReduceScatter phase still reads (the
// in-place forms overwrite only chunks their rank has already folded, or
// chunk r of rank r, which that rank never reads), so the loads need no
// ordering against the other workgroups' stores, and their latency
// overlaps the wait.  Measured at N = 256, M = 2^22 float32: 4.63 against
// 4.81 ms.  Not for bf16, whose float32 partials already fill the register
// budget of a 1024-lane workgroup (128 VGPRs): there the held vectors made
// the call slower (5.78 against 5.41 ms at the 6,553,600-element bucket).
template <class T, int OP, class P, bool CO>
__global__ __launch_bounds__(P::TB) void ring_persistent_kernel(RingArgs a) {
  using LF = Lane<T, P, true, CO>;
  constexpr bool kAhead = CCL_SIM_PERSIST_AHEAD && sizeof(typename T::A) == sizeof(typename T::S);
  const int n = a.nranks;
  const int nsteps = (a.coll == kAllReduce) ? 2 * (n - 1) : (a.coll == kReduceScatter ? n - 1 : n);
  unsigned epoch = 0;
  typename LF::SV ahead[P::U];
  for (int step = a.first_step; step < nsteps; ++step) {
    bool have_ahead = false;
    RsTileAt first;
    if (step > a.first_step) {
      grid_arrive<CO>(a.ctrl, epoch + 1);
      if (kAhead && a.coll != kAllGather && step < n - 1 && uint64_t(blockIdx.x) < a.ntiles) {
        const int r = rank_of_tile(blockIdx.x, a.tiles_per_chunk);
        first = rs_tile_at<P, T>(a, step, r, blockIdx.x - uint64_t(r) * a.tiles_per_chunk);
        if (first.full) {
          const LF ln(first.seg, first.len);
          const typename T::S* mine = in_ptr<T>(a.send, first.r) + uint64_t(first.c) * a.q;
#pragma unroll
          for (int u = 0; u < P::U; ++u) ahead[u] = ln.load(mine, u);
          have_ahead = true;
        }
      }
      if (!grid_wait<CO>(a.ctrl, ++epoch, a.spin_limit)) return;
    }
    for (uint64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
      if (have_ahead && tile == blockIdx.x)
        ring_rs_tile<T, OP, P, true, CO>(a, step, first.r, first.seg, first.c, first.len, ahead);
      else
        ring_body<T, OP, P, CO>(a, step, tile);
    }
  }
}

// Flag-ordered form of the persistent ring.  Under the grid barrier every
// workgroup waits for every other one at each step, although the data of a
// step comes from one place only: tile (r, seg) reads what tile (r-1, seg)
// wrote at the step before (the chunk received from rank r-1), and every
// position (rank, chunk c) is read and written only by chunk c's own chain
// of steps, which the partials keyed by chunk keep (as in the chained
// ring).  So each workgroup counts its completed steps in a flag of its
// own, and before a step waits only until the workgroups holding the
// upstream tiles of its own tiles have completed the step before.  The
// ring's order, transfers and bytes are unchanged; only waits that no data
// depends on are gone.
//
// Progress: take the workgroup whose next step s is the lowest.  The
// workgroups it waits for have completed all their steps below s, so it can
// go on; every workgroup is co-resident (cooperative launch), so the grid
// always completes.  The poll is bounded like the grid barrier's.
//
// Ordering, on the agent-coherent data path only: a workgroup's waves wait
// for their stores (write-through) to complete before lane 0 publishes the
// flag, and the loads of data written by other workgroups are issued after
// the wait, as agent-scope (sc1) loads, or, where the writer runs on the
// same XCD, as ordinary loads from that XCD's L2 once the CU's L1 has been
// dropped (below).  No other cache maintenance is needed.
//
// Placement.  Workgroup b holds the tiles f(b), f(b) + G, f(b) + 2G, ...
// (G = gridDim.x), where f is the identity, or, with xcd_map, the
// permutation f(b) = (b mod 8)·G/8 + b/8 of [0, G).  Workgroups are spread
// over the eight XCDs in turn (workgroup b on XCD b mod 8), so with xcd_map
// the tiles of one eighth of [0, G) share an XCD, and a tile and its
// upstream tile (r-1, seg), tiles_per_chunk before it, share one unless
// they straddle an eighth.  The host sets xcd_map where that places more
// neighbours together than the identity does.  Only speed depends on it: the
// kernel compares XCDs at run time (below) before it reads from an L2.
__device__ inline uint64_t first_tile(const RingArgs& a, uint64_t b) {
  const uint64_t g = gridDim.x;
  return a.xcd_map ? (b % 8) * (g / 8) + b / 8 : b;
}

// The workgroups a workgroup waits on.  Workgroup b takes tiles f, f + G,
// f + 2G, ... (f = first_tile(b), G workgroups).  The upstream tile of tile
// t, (r-1, seg), is t - T (T tiles per chunk), or t - T + ntiles for rank
// 0's tiles (t < T), and which workgroup holds a tile depends only on its
// index modulo G.  So b's tiles from T on all have their upstream tiles on
// one workgroup, the holder of f - T (mod G), and its tiles below T (its
// first ones) on one other, the holder of f - T + ntiles (mod G): at most
// two workgroups, whatever the number of tiles per step.  Lane 0 of wave 0
// waits on the first, lane 1 on the second.
//
// The lane's flag: a workgroup index, or -1 for none (no such tiles, or
// tiles whose upstream tiles are the workgroup's own, whose steps before
// are done).
__device__ inline int flags_upstream(const RingArgs& a) {
  // Everything below is 32-bit arithmetic on offsets the host reduced
  // modulo G: f < G, and every offset is below G.
  const unsigned g = gridDim.x, f = static_cast<unsigned>(first_tile(a, blockIdx.x));
  const auto slot_holder = [&](unsigned m) -> unsigned {  // the holder of tiles m (mod G), for m < 2G
    m = m >= g ? m - g : m;
    return a.xcd_map ? (m % (g / 8)) * 8 + m / (g / 8) : m;
  };
  const unsigned last_off = a.ntiles_mod + g - 1 - f;  // (ntiles - 1 - f) mod G, before the reduction
  const uint64_t last = a.ntiles - 1 - (last_off >= g ? last_off - g : last_off);  // b's last tile
  // The two candidates are the same in every lane.  Said so explicitly
  // (readfirstlane), the compiler keeps them in scalar registers; left to
  // its own analysis it held more of the kernel in vector registers and the
  // 1024-lane float32 and bf16 forms spilled.
  const unsigned back = __builtin_amdgcn_readfirstlane(last >= a.tiles_per_chunk  // some tile is not rank 0's
                                                           ? slot_holder(f + a.up_back)
                                                           : ~0u);
  const unsigned wrap = __builtin_amdgcn_readfirstlane(f < a.tiles_per_chunk  // some tile is rank 0's
                                                           ? slot_holder(f + a.up_wrap)
                                                           : ~0u);
  const int w = threadIdx.x == 0 ? int(back) : threadIdx.x == 1 ? int(wrap) : -1;
  return w == int(blockIdx.x) ? -1 : w;
}

// A flag word holds the steps its workgroup has completed in its low 24
// bits and the workgroup's XCD in its top 8.
constexpr unsigned kFlagSteps = 0xFFFFFFu;
__device__ inline unsigned xcd_id() { return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)); }

// Waits until the flag of the lane's workgroup `w` reaches `step`; false
// once the poll limit is reached or another workgroup has raised the abort
// word.  `bad` is workgroup-shared, 0 until a wait fails; the workgroup then
// stops.  `near` (workgroup-shared) gets bit 0 set when the workgroup
// holding the upstream tiles of the tiles from T on runs on this
// workgroup's XCD (or is this workgroup), and bit 1 for the tiles below T,
// read from the XCD field of the flag waited on.
__device__ inline bool flags_wait(const RingArgs& a, int step, int w, unsigned xcd, int* bad, unsigned* near) {
  if (threadIdx.x < 64) {
    bool ok = true, same = true;
    if (w >= 0) {
      unsigned spins = 0;
      const unsigned* flag = a.ctrl + kCtrlFlags + w;
      unsigned v;
      while (((v = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) & kFlagSteps) <
             unsigned(step)) {
        if (++spins > a.spin_limit ||
            ((spins & 63u) == 0u &&
             __hip_atomic_load(a.ctrl + kCtrlAbort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)) {
          __hip_atomic_store(a.ctrl + kCtrlAbort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      same = (v >> 24) == xcd;
    }
    const uint64_t mask = __ballot(same);
    if (!ok) *bad = 1;
    if (threadIdx.x == 0) *near = unsigned(mask & 3u);
  }
  __syncthreads();
  return *bad == 0;
}

__device__ inline void flags_publish(const RingArgs& a, int step, unsigned xcd) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(a.ctrl + kCtrlFlags + blockIdx.x, unsigned(step + 1) | (xcd << 24), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Loads.  Data that another workgroup wrote earlier in the kernel (the
// incoming partial, the forwarded chunk) is read with agent scope (sc1),
// or, when the writer runs on the same XCD, with ordinary loads from that
// XCD's L2, after this CU's L1 is dropped (buffer_inv sc0): the writer's
// write-through stores completed (vmcnt 0) before it published the flag
// this workgroup waited on, and they passed through that same L2, which
// they update.  A tile's other reads, the rank's own input and the first
// step's sources, hold data written before the kernel, or by this
// workgroup (the in-place forms); they take the L2 form too.  The first
// step waits on nothing and reads only such data.  Side by side at N = 256,
// M = 2^22 float32: 3.25 against 3.66 ms with agent scope throughout.
//
// The L2 form is used only where no cache line holds data of two chunks
// (xcd_loads: line-aligned rank buffers and chunks).  Otherwise a line at a
// chunk boundary can be filled into the reader's L2 for the neighbouring
// chunk while the writer of this chunk's end is storing into it, and the
// fill can carry the old bytes: measured at N = 16, q = 777 float32, where
// the last elements of chunks came out stale.  Misaligned calls keep agent
// scope for every load.
//
// The rank's own input for the first tile of a ReduceScatter step is
// loaded before the wait, as in the grid-barrier form: x^(r) at a position
// that step reads is written, in the in-place forms, only by later steps of
// the same chunk's chain.
#ifndef CCL_SIM_FLAGS_AHEAD
#define CCL_SIM_FLAGS_AHEAD 1
#endif
template <class T, int OP, class P>
__global__ __launch_bounds__(P::TB) void ring_persistent_flags_kernel(RingArgs a) {
  using LX = Lane<T, P, true, true, true>;  // the prefetch of own input, from the L2 or with agent scope
  using LA = Lane<T, P, true, true, false>;
  constexpr bool kAhead = CCL_SIM_FLAGS_AHEAD && sizeof(typename T::A) == sizeof(typename T::S);
  __shared__ int s_bad;
  __shared__ unsigned s_near;
  const int n = a.nranks;
  const int nsteps = (a.coll == kAllReduce) ? 2 * (n - 1) : (a.coll == kReduceScatter ? n - 1 : n);
  const unsigned xcd = xcd_id();
  const int up = flags_upstream(a);
  const uint64_t t0 = first_tile(a, blockIdx.x);  // < ntiles: the grid is at most ntiles
  const int r0 = rank_of_tile(t0, a.tiles_per_chunk);
  const uint64_t seg0 = t0 - uint64_t(r0) * a.tiles_per_chunk;
  if (threadIdx.x == 0) s_bad = 0;  // seen by every wave after the first step's flags_publish
  typename LX::SV ahead[P::U];
  for (int step = a.first_step; step < nsteps; ++step) {
    bool have_ahead = false;
    RsTileAt first;
    // Bit 0: the tiles from T on read from the L2; bit 1: the tiles below T.
    unsigned local = a.xcd_loads ? 3u : 0u;
    if (step > a.first_step) {
      if (kAhead && a.coll != kAllGather && step < n - 1) {
        first = rs_tile_at<P, T>(a, step, r0, seg0);
        if (first.full) {
          const typename T::S* mine = in_ptr<T>(a.send, first.r) + uint64_t(first.c) * a.q;
          if (a.xcd_loads) {
            const LX ln(first.seg, first.len);
#pragma unroll
            for (int u = 0; u < P::U; ++u) ahead[u] = ln.load(mine, u);
          } else {
            const LA ln(first.seg, first.len);
#pragma unroll
            for (int u = 0; u < P::U; ++u) ahead[u] = ln.load(mine, u);
          }
          have_ahead = true;
        }
      }
      if (!flags_wait(a, step, up, xcd, &s_bad, &s_near)) return;
      local = a.xcd_loads ? __builtin_amdgcn_readfirstlane(s_near) : 0u;
      // Ordinary loads may hit this CU's L1, which can hold a line read at
      // an earlier step (in the in-place forms a step can read again what
      // the first step read).  Drop the L1 (this CU's own cache only)
      // before reading what the wait released from the L2.
      if (local != 0) asm volatile("buffer_inv sc0" ::: "memory");
    }
    if ((local >> (t0 < a.tiles_per_chunk ? 1 : 0)) & 1u) {
      if (have_ahead)
        ring_rs_tile<T, OP, P, true, true, true>(a, step, first.r, first.seg, first.c, first.len, ahead);
      else
        ring_body<T, OP, P, true, true, true>(a, step, 0, r0, seg0);
    } else {
      if (have_ahead)
        ring_rs_tile<T, OP, P, true, true, false>(a, step, first.r, first.seg, first.c, first.len, ahead);
      else
        ring_body<T, OP, P, true, true, false>(a, step, 0, r0, seg0);
    }
    for (uint64_t tile = t0 + gridDim.x; tile < a.ntiles; tile += gridDim.x) {
      if ((local >> (tile < a.tiles_per_chunk ? 1 : 0)) & 1u)
        ring_body<T, OP, P, true, false, true>(a, step, tile);
      else
        ring_body<T, OP, P, true>(a, step, tile);
    }
    flags_publish(a, step, xcd);
  }
}

__global__ void reset_ctrl_kernel(unsigned* ctrl) {
  for (int i = threadIdx.x; i < kCtrlWords; i += blockDim.x) ctrl[i] = 0u;
}

RingArgs make_ring_args(const Call& c, uint64_t tile) {
  RingArgs a{};
  a.send = c.send;
  a.recv = c.recv;
  a.nranks = c.nranks;
  a.coll = c.coll;
  a.q = c.q;
  a.limit = c.limit;
  a.tiles_per_chunk = ceil_div(c.q, tile);
  a.ntiles = uint64_t(c.nranks) * a.tiles_per_chunk;
  a.partial = c.partial;
  a.ctrl = c.ctrl;
  a.spin_limit = 1u << 22;
  return a;
}

}  // namespace

// Launch shape of the ring step kernels by step size.  A step that moves
// few elements is over before a one-vector-per-lane grid has ramped up, and
// two vectors per lane (half the workgroups) measured faster there; large
// steps are faster with one.  The crossover, measured on float32 with N = 8
// to 256: a ring step (N chunks of q) of up to 2^26 elements.
#ifndef CCL_SIM_RING_SMALL_STEP
#define CCL_SIM_RING_SMALL_STEP (uint64_t(1) << 26)
#endif

template <class T, int OP, class P>
hipError_t launch_ring_steps(const Call& c) {
  RingArgs a = make_ring_args(c, tile_elems<T, P>());
  const unsigned grid = grid_for(a.ntiles, c.num_cus);
  const int n = c.nranks;
  const int nsteps = (c.coll == kAllReduce) ? 2 * (n - 1) : (c.coll == kReduceScatter ? n - 1 : n);
  const int first = (c.coll == kAllGather && c.in_place) ? 1 : 0;
  for (int step = first; step < nsteps; ++step) {
    a.step = step;
    hipLaunchKernelGGL((ring_step_kernel<T, OP, P>), dim3(grid), dim3(P::TB), 0, c.stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t run_ring_stepwise(const Call& c) {
  return by_type(c.dtype, [&]<class T>() -> hipError_t {
    const int op = (c.coll == kAllGather) ? int(kSum) : c.op;
    const bool small = uint64_t(c.nranks) * c.q <= CCL_SIM_RING_SMALL_STEP;
    return by_op<T>(op, [&]<class U, int OP>() -> hipError_t {
      return small ? launch_ring_steps<U, OP, RingSmallPolicy>(c) : launch_ring_steps<U, OP, RingPolicy>(c);
    });
  });
}

template <class T, int OP, class P>
hipError_t launch_ring_chained(const Call& c) {
  RingArgs a = make_ring_args(c, tile_elems<T, P>());
  a.first_step = (c.coll == kAllGather && c.in_place) ? 1 : 0;
  a.chunk_keyed = 1;
  hipLaunchKernelGGL((ring_chained_kernel<T, OP, P>), dim3(grid_for(a.ntiles, c.num_cus)), dim3(P::TB), 0, c.stream,
                     a);
  return hipGetLastError();
}

// Launch shape of the chained ring.  Every item runs 2(N-1) dependent
// steps, so each lane should keep several loads in flight: two vectors per
// lane measured best in general (2-6 % over one).  When the chunks are
// short and few items run long chains (N = 256 chunks of 2^14 float32:
// 1024 items of 510 steps), four vectors per lane were faster still
// (3.09 against 3.52 ms), provided the chunk is a whole number of those
// tiles; a ragged last tile took that gain away on bf16 chunks of 25,600.
#ifndef CCL_SIM_CHAIN_POLICY
#define CCL_SIM_CHAIN_POLICY 256, 2, true, kStoreWriteThrough
#endif
#ifndef CCL_SIM_CHAIN_LONG_POLICY
#define CCL_SIM_CHAIN_LONG_POLICY 256, 4, true, kStoreWriteThrough
#endif
using ChainPolicy = Policy<CCL_SIM_CHAIN_POLICY>;
using ChainLongPolicy = Policy<CCL_SIM_CHAIN_LONG_POLICY>;

hipError_t run_ring_chained(const Call& c) {
  return by_type(c.dtype, [&]<class T>() -> hipError_t {
    const int op = (c.coll == kAllGather) ? int(kSum) : c.op;
    const uint64_t long_tile = tile_elems<T, ChainLongPolicy>();
    const uint64_t long_items = uint64_t(c.nranks) * ceil_div(c.q, long_tile);
    const bool long_chains = c.q % long_tile == 0 && long_items <= uint64_t(c.num_cus) * 4;
    return by_op<T>(op, [&]<class U, int OP>() -> hipError_t {
      return long_chains ? launch_ring_chained<U, OP, ChainLongPolicy>(c) : launch_ring_chained<U, OP, ChainPolicy>(c);
    });
  });
}

#ifndef CCL_SIM_PERSISTENT_PER_CU
#define CCL_SIM_PERSISTENT_PER_CU 1
#endif

// The persistent grid holds one workgroup per CU (see below), so its lanes
// alone must keep enough loads in flight.  For steps of up to 2^26
// elements a 1024-lane workgroup (a step of N = 256 chunks of 2^14 float32
// is then one tile per workgroup) measured 9-17 % faster than 256 lanes;
// for larger steps 256 lanes were faster.
//
// A second threshold picks the data path.  Small steps are dominated by
// the barrier, and there the agent-coherent path, whose barrier does no
// cache write-back or invalidation, measured 8-25 % faster (N = 256, M =
// 2^22 float32: 4.87 against 6.51 ms; N = 8, M = 2^24, steps of 2^24
// elements: 0.457 against 0.529 ms for RS + AG).  Larger steps are
// dominated by streaming, and there the plain nontemporal loads of the
// fenced path were faster: with the 1024-lane shape at N = 8, M = 2^26
// (steps of 2^26 elements) 1.648 against 1.820 ms for RS + AG in float32
// and 1.097 against 1.209 ms in bf16; with 256 lanes at M = 2^28, 6.52
// against 7.04 ms.  Both paths gave results bit-identical to the stepwise
// ring in every one of about a hundred calls over eight shapes and three
// dtypes.
#ifndef CCL_SIM_PERSIST_SMALL_STEP
#define CCL_SIM_PERSIST_SMALL_STEP (uint64_t(1) << 26)
#endif
#ifndef CCL_SIM_PERSIST_COHERENT_STEP
#define CCL_SIM_PERSIST_COHERENT_STEP (uint64_t(1) << 25)
#endif

// FLAGS: the flag-ordered form (agent-coherent data path only; CO must be
// set), else the grid barrier.
template <class T, int OP, class P, bool CO, bool FLAGS = false>
hipError_t launch_persistent(const Call& c, bool* unsupported, PersistentPlan* plan) {
  static_assert(CO || !FLAGS, "the flag-ordered ring needs the agent-coherent data path");
  RingArgs a = make_ring_args(c, tile_elems<T, P>());
  a.first_step = (c.coll == kAllGather && c.in_place) ? 1 : 0;
  a.chunk_keyed = FLAGS ? 1 : 0;
  if (c.spin_limit) a.spin_limit = c.spin_limit;
  auto kernel = FLAGS ? ring_persistent_flags_kernel<T, OP, P> : ring_persistent_kernel<T, OP, P, CO>;
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, P::TB, 0);
  if (e != hipSuccess) return e;
  if (per_cu <= 0 || c.num_cus <= 0) {
    *unsupported = true;
    return hipSuccess;
  }
  // Workgroups per CU: the caller's request (the front end refuses more than
  // four, the largest grid seen to complete), at most what the occupancy
  // calculation allows, and by default CCL_SIM_PERSISTENT_PER_CU.  A grid
  // at the full occupancy figure (7 per CU) once ran its first barrier into
  // the poll limit, for a reason not established.  Of the grids that
  // complete, one workgroup per CU measured fastest at every step size: the
  // barrier's cost grows with the number of workgroups that arrive.
  // Never more than 1024 lanes (16 waves) per CU: the largest grids seen to
  // complete held four 256-lane or one 1024-lane workgroup per CU.
  const int lanes_cap = 1024 / P::TB > 0 ? 1024 / P::TB : 1;
  int want = c.persistent_per_cu > 0 ? c.persistent_per_cu : CCL_SIM_PERSISTENT_PER_CU;
  want = want < lanes_cap ? want : lanes_cap;
  const int use = want < per_cu ? want : per_cu;
  uint64_t grid = uint64_t(use) * uint64_t(c.num_cus);
  if (grid > a.ntiles) grid = a.ntiles;
  if (FLAGS && grid > uint64_t(kCtrlMaxFlags)) grid = kCtrlMaxFlags;  // one flag word per workgroup
  if (grid == 0) grid = 1;
  // Placement of the flag-ordered form (first_tile): with tiles_per_chunk a
  // multiple of 8 the identity already puts a tile and its upstream tile on
  // one XCD; otherwise the permutation does for most tiles when the two are
  // less than an eighth of the grid apart.
  a.xcd_map = FLAGS && grid % 8 == 0 && a.tiles_per_chunk % 8 != 0 && a.tiles_per_chunk < grid / 8 ? 1 : 0;
  a.xcd_loads = FLAGS && c.line_aligned ? 1 : 0;
  a.up_back = static_cast<unsigned>((grid - a.tiles_per_chunk % grid) % grid);
  a.up_wrap = static_cast<unsigned>((a.ntiles - a.tiles_per_chunk) % grid);
  a.ntiles_mod = static_cast<unsigned>(a.ntiles % grid);
  if (plan) {
    plan->occupancy_per_cu = per_cu;
    plan->per_cu = use;
    plan->grid = grid;
    plan->tiles_per_step = a.ntiles;
    plan->lanes = P::TB;
    plan->coherent = CO;
    plan->flags = FLAGS;
  }
  hipLaunchKernelGGL(reset_ctrl_kernel, dim3(1), dim3(256), 0, c.stream, c.ctrl);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  void* args[] = {&a};
  e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kernel), dim3(static_cast<unsigned>(grid)), dim3(P::TB),
                                 args, 0, c.stream);
  if (e == hipSuccess) return hipSuccess;
  // The call reports the failure; clear HIP's last-error slot so that it
  // does not resurface in the caller's next, unrelated HIP call.
  (void)hipGetLastError();
  if (e == hipErrorCooperativeLaunchTooLarge || e == hipErrorIllegalState) {
    // Too large: no co-resident grid.  Illegal state: the runtime refused the
    // cooperative launch itself, as it does here when another process on
    // the GPU has made cooperative launches.  Either way the request is
    // valid but cannot run now.
    *unsupported = true;
    if (plan && e == hipErrorIllegalState) plan->refused = e;
    return hipSuccess;
  }
  return e;
}

// A third threshold picks how steps are ordered when the caller leaves it
// to the library: per-workgroup flags on the agent-coherent path for steps
// of up to this many elements, the grid barrier above.  Measured on
// line-aligned calls (same-XCD reads on), flags against barrier: N = 8,
// M = 2^25 AllReduce 0.681 against 0.850 ms; M = 2^26 RS + AG 1.448
// against 1.666 ms and AllReduce 1.336 against 1.567 ms in float32, 0.900
// against 1.039 ms in bf16.  Above 2^26 the barrier won in float32 (N = 16,
// M = 2^27: 7.18 against 7.40 ms; N = 8, M = 2^28: 6.53 against 7.00 ms),
// once a step no longer fits the 256 MB last-level cache.
#ifndef CCL_SIM_PERSIST_FLAGS_STEP
#define CCL_SIM_PERSIST_FLAGS_STEP CCL_SIM_PERSIST_SMALL_STEP
#endif

bool persistent_uses_flags(int nranks, uint64_t q, int sync) {
  return sync == kSyncFlags || (sync == kSyncAuto && uint64_t(nranks) * q <= CCL_SIM_PERSIST_FLAGS_STEP);
}

hipError_t run_ring_persistent(const Call& c, bool* unsupported, PersistentPlan* plan) {
  *unsupported = false;
  return by_type(c.dtype, [&]<class T>() -> hipError_t {
    const int op = (c.coll == kAllGather) ? int(kSum) : c.op;
    const uint64_t step = uint64_t(c.nranks) * c.q;
    const bool small = step <= CCL_SIM_PERSIST_SMALL_STEP;
    const bool coherent = step <= CCL_SIM_PERSIST_COHERENT_STEP;
    const bool flags = persistent_uses_flags(c.nranks, c.q, c.persistent_sync);
    return by_op<T>(op, [&]<class U, int OP>() -> hipError_t {
      if (flags)
        return small ? launch_persistent<U, OP, PersistSmallPolicy, true, true>(c, unsupported, plan)
                     : launch_persistent<U, OP, PersistPolicy, true, true>(c, unsupported, plan);
      if (small)
        return coherent ? launch_persistent<U, OP, PersistSmallPolicy, true>(c, unsupported, plan)
                        : launch_persistent<U, OP, PersistSmallPolicy, false>(c, unsupported, plan);
      return launch_persistent<U, OP, PersistPolicy, false>(c, unsupported, plan);
    });
  });
}

}  // namespace ccl
