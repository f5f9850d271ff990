// Recursive halving ReduceScatter and recursive doubling AllGather.

#include "kernel_common.hpp"

namespace ccl {
namespace {

// ---------------------------------------------------------------------------
// Recursive halving ReduceScatter / recursive doubling AllGather ([RS-PAGE]
// §Recursive Halving ReduceScatter), N = 2^k.
//
// Halving step j = 1..k: rank i pairs with p = i XOR N/2^j; the pair shares
// the range it held before the step, rank i keeps the lower half when bit
// N/2^j of i is clear and the upper half otherwise, and reduces the pair's
// two partials over its half as (lower rank's) ⊕ (upper rank's).  The range
// rank i holds after step j starts at q·(i AND top-j-bits mask) and spans
// N/2^j blocks, so after k steps it is exactly block i: rank-major, with no
// relabelling.  Step 1 reads the two inputs; later steps read the pair's
// partials from the per-rank scratch W_i, which covers the half rank i kept
// at step 1 (W holds N·(N/2)·q accumulators); the last step stores the
// completed block to the output.  Within a step a rank writes only its own
// kept half, which its partner does not read, so W is updated in place.
//
// Doubling step t = 0..k-1: rank i receives from p = i XOR 2^t the 2^t
// blocks p has gathered, starting at block (p >> t) << t, and copies them
// into its output (the stand-alone AllGather first places each rank's own
// shard).
// ---------------------------------------------------------------------------
struct RecArgs {
  RankPtrs send, recv;
  int nranks;
  int coll;
  int phase;                 // 0 halving, 1 doubling, 2 placement
  int step;                  // halving: j (1-based); doubling: t
  int last;                  // halving: this is step k
  uint64_t q;
  uint64_t limit;            // positions at or past it are padding / trimmed
  uint64_t len;              // elements each rank moves in this step
  uint64_t tiles_per_rank;
  uint64_t ntiles;
  void* scratch;
};

template <class T, int OP, class P, bool FULL>
__device__ inline void halving_tile(const RecArgs& a, int i, uint64_t seg, uint64_t base, uint64_t cnt) {
  using A = typename T::A;
  using L = Lane<T, P, FULL>;
  constexpr int V = vec_elems<T>();
  const int n = a.nranks;
  const int d = n >> a.step;
  const int p = i ^ d;
  const int lo = i < p ? i : p, up = i < p ? p : i;
  const uint64_t half = uint64_t(n / 2) * a.q;           // W_i length
  const uint64_t base1 = uint64_t(i & (n / 2)) * a.q;     // start of the half kept at step 1
  A* w = static_cast<A*>(a.scratch);
  const L ln(seg, cnt);
  typename L::AV vl[P::U], vu[P::U];
  if (a.step == 1) {
    const typename T::S* xl = in_ptr<T>(a.send, lo) + base;
    const typename T::S* xu = in_ptr<T>(a.send, up) + base;
#pragma unroll
    for (int u = 0; u < P::U; ++u)
      if (ln.on(u)) {
        const typename L::SV sl = ln.load(xl, u), su = ln.load(xu, u);
#pragma unroll
        for (int k = 0; k < V; ++k) {
          vl[u][k] = T::widen(sl[k]);
          vu[u][k] = T::widen(su[k]);
        }
      }
  } else {
    const A* wl = w + uint64_t(lo) * half + (base - base1);
    const A* wu = w + uint64_t(up) * half + (base - base1);
#pragma unroll
    for (int u = 0; u < P::U; ++u)
      if (ln.on(u)) {
        vl[u] = ln.load_acc(wl, u);
        vu[u] = ln.load_acc(wu, u);
      }
  }
  if (!a.last) {
    A* dst = w + uint64_t(i) * half + (base - base1);
#pragma unroll
    for (int u = 0; u < P::U; ++u) {
      if (!ln.on(u)) continue;
      typename L::AV v;
#pragma unroll
      for (int k = 0; k < V; ++k) v[k] = combine<T, OP>(vl[u][k], vu[u][k]);
      ln.store_acc(dst, u, v);
    }
  } else {
    typename T::S* dst = (a.coll == kAllReduce) ? out_ptr<T>(a.recv, i) + base : out_ptr<T>(a.recv, i);
#pragma unroll
    for (int u = 0; u < P::U; ++u) {
      if (!ln.on(u)) continue;
      typename L::SV v;
#pragma unroll
      for (int k = 0; k < V; ++k) v[k] = T::narrow(finalize<T, OP>(combine<T, OP>(vl[u][k], vu[u][k]), n));
      ln.store(dst, u, v);
    }
  }
}

template <class T, int OP, class P>
__global__ __launch_bounds__(P::TB) void recursive_step_kernel(RecArgs a) {
  constexpr uint64_t kTile = tile_of<P>(vec_elems<T>());
  for (uint64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const int i = rank_of_tile(tile, a.tiles_per_rank);
    const uint64_t seg = tile - uint64_t(i) * a.tiles_per_rank;
    uint64_t base;
    const typename T::S* src = nullptr;
    if (a.phase == 0) {
      const int mask = (a.nranks - 1) & ~((a.nranks >> a.step) - 1);  // top `step` bits of a rank index
      base = uint64_t(i & mask) * a.q;
    } else if (a.phase == 1) {
      const int p = i ^ (1 << a.step);
      base = uint64_t((p >> a.step) << a.step) * a.q;
      src = in_ptr<T>(a.recv, p) + base;
    } else {
      base = uint64_t(i) * a.q;
      src = in_ptr<T>(a.send, i);
    }
    const uint64_t cnt = base >= a.limit ? 0 : (a.limit - base < a.len ? a.limit - base : a.len);
    const bool full = (seg + 1) * kTile <= cnt;
    if (a.phase == 0) {
      if (full)
        halving_tile<T, OP, P, true>(a, i, seg, base, cnt);
      else
        halving_tile<T, OP, P, false>(a, i, seg, base, cnt);
    } else {
      typename T::S* dst = out_ptr<T>(a.recv, i) + base;
      if (full)
        copy_tile<T, P, true>(src, dst, seg, cnt);
      else
        copy_tile<T, P, false>(src, dst, seg, cnt);
    }
  }
}

}  // namespace

// Launch shape of the recursive step kernels by step size, as for the ring
// steps: two vectors per lane for a halving or doubling step of up to 2^24
// elements (the measured crossover on float32, N = 8 to 256), one above.
#ifndef CCL_SIM_RECURSIVE_SMALL_STEP
#define CCL_SIM_RECURSIVE_SMALL_STEP (uint64_t(1) << 24)
#endif

template <class T, int OP, class P>
hipError_t launch_recursive_step(const Call& c, RecArgs& a, int phase, int step, int k, uint64_t len) {
  const uint64_t tile = tile_elems<T, P>();
  a.phase = phase;
  a.step = step;
  a.last = (phase == 0 && step == k) ? 1 : 0;
  a.len = len;
  a.tiles_per_rank = ceil_div(len, tile);
  a.ntiles = uint64_t(c.nranks) * a.tiles_per_rank;
  if (a.ntiles == 0) return hipSuccess;
  const unsigned grid = grid_for(a.ntiles, c.num_cus);
  hipLaunchKernelGGL((recursive_step_kernel<T, OP, P>), dim3(grid), dim3(P::TB), 0, c.stream, a);
  return hipGetLastError();
}

hipError_t run_recursive(const Call& c) {
  return by_type(c.dtype, [&]<class T>() -> hipError_t {
    const int op = (c.coll == kAllGather) ? int(kSum) : c.op;
    return by_op<T>(op, [&]<class U, int OP>() -> hipError_t {
      const int n = c.nranks;
      int k = 0;
      while ((1 << k) < n) ++k;
      RecArgs a{};
      a.send = c.send;
      a.recv = c.recv;
      a.nranks = n;
      a.coll = c.coll;
      a.q = c.q;
      a.limit = c.limit;
      a.scratch = c.partial;
      auto launch = [&](int phase, int step, uint64_t len) -> hipError_t {
        if (uint64_t(n) * len <= CCL_SIM_RECURSIVE_SMALL_STEP)
          return launch_recursive_step<U, OP, RingSmallPolicy>(c, a, phase, step, k, len);
        return launch_recursive_step<U, OP, RingPolicy>(c, a, phase, step, k, len);
      };
      hipError_t e = hipSuccess;
      if (c.coll != kAllGather)
        for (int j = 1; j <= k && e == hipSuccess; ++j) e = launch(0, j, uint64_t(n >> j) * c.q);
      if (c.coll == kAllGather && !c.in_place && e == hipSuccess) e = launch(2, 0, c.q);
      if (c.coll != kReduceScatter)
        for (int t = 0; t < k && e == hipSuccess; ++t) e = launch(1, t, (uint64_t(1) << t) * c.q);
      return e;
    });
  });
}

}  // namespace ccl
