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
  int placed;                // chained AllGather: the own shards are in place already
  uint64_t q;
  uint64_t limit;            // positions at or past it are padding / trimmed
  uint64_t len;              // elements each rank moves in this step
  uint64_t tiles_per_rank;
  uint64_t ntiles;
  void* scratch;
};

// bf16 partials (eight float32 accumulators, 32 bytes, per lane) in the
// stepwise driver's natural layout.  Moved lane by lane, each of a wave's
// two 16-byte accesses covers every other 16 bytes of 2 KB, half of every
// line it touches.  Whole tiles instead move a wave's 2 KB as two
// contiguous 1 KB halves, lane i taking bytes [16i, 16i + 16) of each, and
// the lanes trade values through the cross-lane permute (ds_bpermute,
// which reads another lane's register without touching LDS memory), so
// that each lane still folds its own eight positions.  The layout in
// memory stays the natural one, which the stepwise driver needs: it tiles
// each halving step afresh.  Every lane of the wave takes part, which whole
// tiles guarantee.
#ifndef CCL_SIM_RECURSIVE_WAVE_ACC
#define CCL_SIM_RECURSIVE_WAVE_ACC 1
#endif
__device__ inline float lane_value(int src_lane, float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src_lane << 2, __builtin_bit_cast(int, x)));
}

// The wave's 512 positions from `wave_base` (its first lane's first
// position); returns this lane's eight accumulators.
template <class P, class AV>
__device__ inline AV wave_load_acc8(const float* wave_base) {
  static_assert(sizeof(AV) == 32, "eight float32 accumulators");
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const auto a = vload<float, 4, P::NTL>(wave_base + 4 * lane);        // positions [4i, 4i + 4)
  const auto b = vload<float, 4, P::NTL>(wave_base + 256 + 4 * lane);  // positions [256 + 4i, 256 + 4i + 4)
  // lane j holds positions [8j, 8j + 8): the first half in lane 2j's and the
  // second in lane 2j + 1's access (of a for j < 32, of b above)
  const int s0 = 2 * (lane & 31), s1 = s0 + 1;
  const bool upper = lane >= 32;
  AV v;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a0 = lane_value(s0, a[k]), b0 = lane_value(s0, b[k]);
    const float a1 = lane_value(s1, a[k]), b1 = lane_value(s1, b[k]);
    v[k] = upper ? b0 : a0;
    v[4 + k] = upper ? b1 : a1;
  }
  return v;
}

// Stores this lane's eight accumulators as the wave's 2 KB from the byte
// offset `wave_off` of the tile that starts at `tile_base` (`tile_bytes`
// long), with write-through stores of whole lines.
template <class AV>
__device__ inline void wave_store_acc8(float* tile_base, uint32_t tile_bytes, uint32_t wave_off, AV v) {
  static_assert(sizeof(AV) == 32, "eight float32 accumulators");
  using F4 = typename VecOf<float, 4>::type;
  const int lane = static_cast<int>(threadIdx.x) & 63;
  // access a, lane i: positions [4i, 4i + 4), the first or second half of
  // lane i/2's eight; access b: the same of lane 32 + i/2
  const int src = lane >> 1;
  const bool second = lane & 1;
  F4 a, b;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float x0 = lane_value(src, v[k]), x1 = lane_value(src, v[4 + k]);
    const float y0 = lane_value(32 + src, v[k]), y1 = lane_value(32 + src, v[4 + k]);
    a[k] = second ? x1 : x0;
    b[k] = second ? y1 : y0;
  }
  store_through(tile_base, tile_bytes, wave_off + uint32_t(16 * lane), a);
  store_through(tile_base, tile_bytes, wave_off + 1024u + uint32_t(16 * lane), b);
}

// Halving step `step` for rank i over the tile `seg` of the range that
// starts at position `base` (cnt valid positions from base).  SAME_TILING:
// every step that touches these partials uses this same tile geometry (the
// chained driver), so they may take the Lane's split partial order; the
// stepwise driver re-tiles each step and keeps the natural order.
template <class T, int OP, class P, bool FULL, bool SAME_TILING>
__device__ inline void halving_tile(const RecArgs& a, int step, bool last, int i, uint64_t seg, uint64_t base,
                                    uint64_t cnt) {
  using A = typename T::A;
  using L = Lane<T, P, FULL>;
  constexpr int V = vec_elems<T>();
  // the wave-wide accesses above: natural-layout bf16 partials of a whole tile
  constexpr bool kWave = CCL_SIM_RECURSIVE_WAVE_ACC && !SAME_TILING && FULL && sizeof(typename L::AV) == 32 &&
                         P::ST == kStoreWriteThrough && P::TB % 64 == 0;
  const int n = a.nranks;
  const int d = n >> step;
  const int p = i ^ d;
  const int lo = i < p ? i : p, up = i < p ? p : i;
  const uint64_t half = uint64_t(n / 2) * a.q;           // W_i length
  const uint64_t base1 = uint64_t(i & (n / 2)) * a.q;     // start of the half kept at step 1
  A* w = static_cast<A*>(a.scratch);
  const L ln(seg, cnt);
  typename L::AV vl[P::U], vu[P::U];
  if (step == 1) {
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
        if constexpr (SAME_TILING) {
          vl[u] = ln.load_part(wl, u);
          vu[u] = ln.load_part(wu, u);
        } else if constexpr (kWave) {
          const uint64_t first = ln.j[u] - uint64_t(static_cast<int>(threadIdx.x) & 63) * V;  // the wave's first position
          vl[u] = wave_load_acc8<P, typename L::AV>(wl + first);
          vu[u] = wave_load_acc8<P, typename L::AV>(wu + first);
        } else {
          vl[u] = ln.load_acc(wl, u);
          vu[u] = ln.load_acc(wu, u);
        }
      }
  }
  if (!last) {
    A* dst = w + uint64_t(i) * half + (base - base1);
#pragma unroll
    for (int u = 0; u < P::U; ++u) {
      if (!ln.on(u)) continue;
      typename L::AV v;
#pragma unroll
      for (int k = 0; k < V; ++k) v[k] = combine<T, OP>(vl[u][k], vu[u][k]);
      if constexpr (SAME_TILING) {
        ln.store_part(dst, u, v);
      } else if constexpr (kWave) {
        const uint32_t wave_off =
            uint32_t((u * P::TB + (static_cast<int>(threadIdx.x) & ~63)) * V * int(sizeof(A)));
        wave_store_acc8(dst + ln.t0, uint32_t(tile_of<P>(V) * sizeof(A)), wave_off, v);
      } else {
        ln.store_acc(dst, u, v);
      }
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
        halving_tile<T, OP, P, true, false>(a, a.step, a.last != 0, i, seg, base, cnt);
      else
        halving_tile<T, OP, P, false, false>(a, a.step, a.last != 0, i, seg, base, cnt);
    } else {
      typename T::S* dst = out_ptr<T>(a.recv, i) + base;
      if (full)
        copy_tile<T, P, true>(src, dst, seg, cnt);
      else
        copy_tile<T, P, false>(src, dst, seg, cnt);
    }
  }
}

// Chained driver: work item = (block b, tile seg of the block).  Each
// position's reduction is its own butterfly over the ranks: at halving step
// j the ranks that hold block b are those whose top j bits equal b's, and
// each pairs with the rank that differs in bit N/2^j; at doubling step t
// block b moves from each rank p with p >> t == b >> t to p XOR 2^t.  A
// step of block b reads only what earlier steps of block b wrote, at the
// same positions, so one workgroup runs all of its item's combines and
// copies, with the same lane-to-element mapping throughout; each value it
// reads it wrote itself earlier in program order (single-thread coherence;
// no fence).  Items touch disjoint positions and need no synchronisation.
// Same pairs, same combining order and same bytes as the stepwise driver.
//
// Order inside an item: the halving steps of block b form a binary tree
// (the node of rank i at step j combines the nodes of ranks i and
// i XOR N/2^j at step j-1), and the doubling steps a broadcast tree from
// rank b.  Both are walked depth first rather than step by step, so a
// partial is read back soon after it was written, while it is still in the
// caches; with N/2 combines per step at N = 256 a step-by-step walk would
// leave each item megabytes of partials between write and read.  A node's
// operands are the same in either order, so the results are too.
//   Halving: the step-1 nodes are taken in bit-reversed order of their low
//   bits, which makes the two children of every node consecutive, and a
//   node is combined as soon as its second child is (a binary counter).
//   Doubling: rank b XOR bitrev(c) for c = 1 .. N-1 receives from the rank
//   that differs from it in the top bit of bitrev(c), which c with its
//   lowest set bit cleared has already filled.
__device__ inline int bit_reverse(int v, int bits) {
  return bits == 0 ? 0 : static_cast<int>(__builtin_bitreverse32(static_cast<unsigned>(v)) >> (32 - bits));
}

template <class T, int OP, class P, bool FULL>
__device__ inline void recursive_item(const RecArgs& a, int b, uint64_t seg, uint64_t cnt) {
  const int n = a.nranks;
  int k = 0;
  while ((1 << k) < n) ++k;
  const uint64_t base = uint64_t(b) * a.q;
  if (a.coll != kAllGather) {
    for (int c = 0; c < (n >> 1); ++c) {
      int j = 1, v = c;
      for (;;) {
        const int d = n >> j;  // ranks holding block b after step j: top j bits of b, any low bits
        halving_tile<T, OP, P, FULL, true>(a, j, j == k, (b & ~(d - 1)) | bit_reverse(v, k - j), seg, base, cnt);
        if (!(v & 1)) break;   // the parent's other child is still to come
        v >>= 1;
        ++j;
      }
    }
  } else if (!a.placed) {
    // stand-alone AllGather, out of place: rank b places its own shard
    copy_tile<T, P, FULL>(in_ptr<T>(a.send, b), out_ptr<T>(a.recv, b) + base, seg, cnt);
  }
  if (a.coll != kReduceScatter) {
    for (int c = 1; c < n; ++c) {
      const int x = bit_reverse(c, k);
      const int i = b ^ x;
      const int from = i ^ (1 << (31 - __builtin_clz(static_cast<unsigned>(x))));  // doubling step t = top bit of x
      copy_tile<T, P, FULL>(out_ptr<T>(a.recv, from) + base, out_ptr<T>(a.recv, i) + base, seg, cnt);
    }
  }
}

template <class T, int OP, class P>
__global__ __launch_bounds__(P::TB) void recursive_chained_kernel(RecArgs a) {
  constexpr uint64_t kTile = tile_of<P>(vec_elems<T>());
  for (uint64_t item = blockIdx.x; item < a.ntiles; item += gridDim.x) {
    const int b = rank_of_tile(item, a.tiles_per_rank);
    const uint64_t seg = item - uint64_t(b) * a.tiles_per_rank;
    const uint64_t base = uint64_t(b) * a.q;
    const uint64_t cnt = base >= a.limit ? 0 : (a.limit - base < a.q ? a.limit - base : a.q);
    if (seg * kTile >= cnt) continue;
    if ((seg + 1) * kTile <= cnt)
      recursive_item<T, OP, P, true>(a, b, seg, cnt);
    else
      recursive_item<T, OP, P, false>(a, b, seg, cnt);
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

// Launch shape of the chained recursive driver.  Measured on float32
// AllReduce against 1 and 2 vectors per lane and 512 lanes: four vectors
// per lane were 1-3 % faster at N = 8 (M = 2^24, 2^26), 64 and 256, and
// 0.5 % slower at N = 8, M = 2^28; one vector per lane was 4-7 % slower.
#ifndef CCL_SIM_RECURSIVE_CHAIN_POLICY
#define CCL_SIM_RECURSIVE_CHAIN_POLICY 256, 4, true, kStoreWriteThrough
#endif
using RecursiveChainPolicy = Policy<CCL_SIM_RECURSIVE_CHAIN_POLICY>;

template <class T, int OP, class P>
hipError_t launch_recursive_chained(const Call& c) {
  RecArgs a{};
  a.send = c.send;
  a.recv = c.recv;
  a.nranks = c.nranks;
  a.coll = c.coll;
  a.q = c.q;
  a.limit = c.limit;
  a.scratch = c.partial;
  a.placed = (c.coll == kAllGather && c.in_place) ? 1 : 0;
  a.tiles_per_rank = ceil_div(c.q, tile_elems<T, P>());
  a.ntiles = uint64_t(c.nranks) * a.tiles_per_rank;
  if (a.ntiles == 0) return hipSuccess;
  hipLaunchKernelGGL((recursive_chained_kernel<T, OP, P>), dim3(grid_for(a.ntiles, c.num_cus)), dim3(P::TB), 0,
                     c.stream, a);
  return hipGetLastError();
}

hipError_t run_recursive_chained(const Call& c) {
  return by_type(c.dtype, [&]<class T>() -> hipError_t {
    const int op = (c.coll == kAllGather) ? int(kSum) : c.op;
    return by_op<T>(op, [&]<class U, int OP>() -> hipError_t {
      return launch_recursive_chained<U, OP, RecursiveChainPolicy>(c);
    });
  });
}

}  // namespace ccl
