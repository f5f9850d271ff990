// HIP kernels for gfx950: fused N-way reduce (ReduceScatter), broadcast-copy
// (AllGather), fused AllReduce, ring steps (one launch per step, or one
// persistent cooperative kernel with a grid barrier), recursive halving and
// doubling steps, identity padding.
//
// Pages cited:
//   [DECOMP]  "NCCL 专家课程 07：AllReduce 等价分解、显存生命周期与 Kernel 证据"
//   [RING]    "Ring AllReduce 核心流程：梯度是怎么聚合的"
//   [PRIMS]   "通信与互联（01）：集合通信原语与代价模型——α-β 模型与 ring all-reduce"
//   [WHY-EQ]  "为什么说 AllReduce = ReduceScatter + AllGather？——结合 NCCL Ring AllReduce"
//   [RS-PAGE] "ReduceScatter" (集合通信)
//
// Work decomposition.  Every kernel is a grid-stride loop over tiles of
// TB·V·U elements (V = 16 / sizeof(element): one 128-bit access per lane
// per vector, U vectors per lane, TB lanes; TB and U are part of each
// kernel's Policy).  A tile never crosses a shard (or ring chunk)
// boundary, so the shard a tile belongs to is one scalar division per tile
// and the shard-local side of every access keeps the buffer's alignment;
// the other side (the input of ReduceScatter at r·q + j, the output of
// AllGather at s·q + j) is off a 16-byte boundary when q·sizeof(element)
// is not a multiple of 16, which the unaligned 128-bit accesses absorb.  A
// tile that lies wholly inside the valid range runs without per-lane
// checks; in the last tile of a shard, lanes past the end of the shard, of
// the logical length (padding) or of a trimmed output move fewer elements,
// one at a time.
//
// Nothing here is a contraction: the kernels stream HBM at roughly one
// combine per element loaded, so the only roofline that matters is HBM
// bandwidth and MFMA plays no part.

#include "internal.hpp"

namespace ccl {
namespace {

#define CCL_GLOBAL __attribute__((address_space(1)))

template <class T>
constexpr int vec_elems() {
  return 16 / static_cast<int>(sizeof(typename T::S));
}

// Per-kernel shape and memory policy: TB threads per workgroup, U 128-bit
// vectors per lane per tile, whether rank-buffer loads carry the
// nontemporal hint, and how whole vectors are stored (StoreMode).  Every
// rank buffer is streamed once per call, so keeping it out of the caches
// pays.  Write-through stores measured as fast as or faster than plain and
// nontemporal ones for every collective kernel: the AllGather by about 3 %
// at N = 8, the ring and recursive steps by 1-12 %, the persistent ring by
// a quarter at N = 256, whose barriers then find little dirty data left to
// write back.  The identity pad keeps plain stores: it doubles as the
// plain copy that calibrates the traffic counters.  Each default can be
// replaced at build time.
enum StoreMode : int {
  kStorePlain = 0,         // global store, default cache policy
  kStoreNontemporal = 1,   // global store with the nontemporal hint
  kStoreWriteThrough = 2,  // 128-bit vectors: buffer store with system-scope
                           // bits (sc0 sc1); wider vectors (the float32
                           // accumulators of bf16 data, two 128-bit halves
                           // per lane): as kStoreNontemporal, since a
                           // write-through half covers only every other
                           // 16 bytes of a line and measured slower
};
template <int TB_, int U_, bool NTL_, int ST_>
struct Policy {
  static constexpr int TB = TB_;  // threads per workgroup
  static constexpr int U = U_;
  static constexpr bool NTL = NTL_;
  static constexpr int ST = ST_;
};
#ifndef CCL_SIM_RS_POLICY
#define CCL_SIM_RS_POLICY 256, 1, true, kStoreWriteThrough
#endif
#ifndef CCL_SIM_AG_POLICY
#define CCL_SIM_AG_POLICY 256, 1, true, kStoreWriteThrough
#endif
#ifndef CCL_SIM_AR_POLICY
#define CCL_SIM_AR_POLICY 256, 1, true, kStoreWriteThrough
#endif
#ifndef CCL_SIM_DIRECT_SMALL_POLICY
#define CCL_SIM_DIRECT_SMALL_POLICY 256, 2, true, kStoreWriteThrough
#endif
#ifndef CCL_SIM_RING_POLICY
#define CCL_SIM_RING_POLICY 256, 1, true, kStoreWriteThrough
#endif
#ifndef CCL_SIM_RING_SMALL_POLICY
#define CCL_SIM_RING_SMALL_POLICY 256, 2, true, kStoreWriteThrough
#endif
#ifndef CCL_SIM_PERSIST_POLICY
#define CCL_SIM_PERSIST_POLICY 256, 4, true, kStoreWriteThrough
#endif
#ifndef CCL_SIM_PERSIST_SMALL_POLICY
#define CCL_SIM_PERSIST_SMALL_POLICY 1024, 4, true, kStoreWriteThrough
#endif
#ifndef CCL_SIM_PAD_POLICY
#define CCL_SIM_PAD_POLICY 256, 4, false, kStorePlain
#endif
using RsPolicy = Policy<CCL_SIM_RS_POLICY>;
using AgPolicy = Policy<CCL_SIM_AG_POLICY>;
using ArPolicy = Policy<CCL_SIM_AR_POLICY>;
using DirectSmallPolicy = Policy<CCL_SIM_DIRECT_SMALL_POLICY>;
using RingPolicy = Policy<CCL_SIM_RING_POLICY>;
using RingSmallPolicy = Policy<CCL_SIM_RING_SMALL_POLICY>;
using PersistPolicy = Policy<CCL_SIM_PERSIST_POLICY>;
using PersistSmallPolicy = Policy<CCL_SIM_PERSIST_SMALL_POLICY>;
using PadPolicy = Policy<CCL_SIM_PAD_POLICY>;

template <class P>
constexpr uint64_t tile_of(int v) {
  return uint64_t(P::TB) * uint64_t(v) * P::U;
}

// K elements of E as one vector value, promising only element alignment.
// gfx950 under the HSA runtime accepts unaligned global accesses, so the
// compiler still emits whole 128-bit global loads and stores for these; a
// shard that starts off a 16-byte boundary (q·sizeof(E) not a multiple of
// 16) costs at most one extra cache line per wave, not a slower path.
template <class E, int K>
struct VecOf {
  typedef E __attribute__((ext_vector_type(K), aligned(sizeof(E)))) type;
};

// Accesses go through global-address-space pointers so they compile to
// global_load / global_store rather than flat accesses.
template <class E, int K, bool NT>
__device__ inline typename VecOf<E, K>::type vload(const E* p) {
  using V = typename VecOf<E, K>::type;
  if constexpr (NT)
    return __builtin_nontemporal_load((const CCL_GLOBAL V*)(p));
  else
    return *(const CCL_GLOBAL V*)(p);
}
template <class E, int K, bool NT>
__device__ inline void vstore(E* p, typename VecOf<E, K>::type v) {
  using V = typename VecOf<E, K>::type;
  if constexpr (NT)
    __builtin_nontemporal_store(v, (CCL_GLOBAL V*)(p));
  else
    *(CCL_GLOBAL V*)(p) = v;
}
template <class E>
__device__ inline E get1(const E* p) {
  return *(const CCL_GLOBAL E*)(p);
}
template <class E>
__device__ inline void put1(E* p, E v) {
  *(CCL_GLOBAL E*)(p) = v;
}

// A 128-bit store with the system-scope cache bits (sc0 sc1), which make
// the L2 pass the line on to memory instead of keeping it dirty.  Only
// buffer instructions take explicit cache bits, so the store goes through
// a buffer resource whose base is the start of the workgroup's tile (a
// 32-bit byte range covers the tile) and the lane's byte offset inside it.
// The tile base is the same in every lane of the wave; reading it from the
// first lane lets the compiler keep the resource in scalar registers.
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer, gfx9 family
constexpr int kSystemScope = 1 | 16;    // sc0 | sc1
template <class EV>
__device__ inline void store_through(void* tile_base, uint32_t tile_bytes, uint32_t byte_offset, EV v) {
  using W4 = unsigned __attribute__((ext_vector_type(4)));
  static_assert(sizeof(EV) == sizeof(W4), "one 128-bit vector");
  const uint64_t addr = reinterpret_cast<uint64_t>(tile_base);
  const uint64_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(addr))));
  const uint64_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(addr >> 32))));
  void* base = reinterpret_cast<void*>((hi << 32) | lo);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(base, 0, int(tile_bytes), kRsrcWord3);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(W4, v), rs, int(byte_offset), 0, kSystemScope);
}

__device__ inline int rank_of_tile(uint64_t tile, uint64_t per) { return static_cast<int>(tile / per); }

__device__ inline int lane_count(uint64_t j, uint64_t len, int v) {
  return j < len ? static_cast<int>(len - j < static_cast<uint64_t>(v) ? len - j : static_cast<uint64_t>(v)) : 0;
}

// One lane's P::U vectors inside a tile.  FULL: the whole tile lies inside
// the valid range, so every vector is complete and no lane checks a count;
// otherwise each vector carries its count of valid elements (0..V) and
// incomplete ones move element by element.
template <class T, class P, bool FULL>
struct Lane {
  using S = typename T::S;
  using A = typename T::A;
  static constexpr int U = P::U;
  static constexpr int V = vec_elems<T>();
  using SV = typename VecOf<S, V>::type;
  using AV = typename VecOf<A, V>::type;
  uint64_t t0;  // first element of the tile (the same for every lane)
  uint64_t j[U];
  int cnt[U];

  __device__ Lane(uint64_t seg, uint64_t len) : t0(seg * tile_of<P>(V)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      j[u] = seg * tile_of<P>(V) + uint64_t(u * P::TB + static_cast<int>(threadIdx.x)) * V;
      cnt[u] = FULL ? V : lane_count(j[u], len, V);
    }
  }
  __device__ bool on(int u) const { return FULL || cnt[u] > 0; }
  __device__ bool whole(int u) const { return FULL || cnt[u] == V; }

  template <class E, class EV>
  __device__ EV load_any(const E* base, int u) const {
    if (whole(u)) return vload<E, V, P::NTL>(base + j[u]);
    EV v = {};
#pragma unroll
    for (int k = 0; k < V; ++k)
      if (k < cnt[u]) v[k] = get1(base + j[u] + k);
    return v;
  }
  template <class E, class EV>
  __device__ void store_any(E* base, int u, EV v) const {
    if constexpr (FULL && P::ST == kStoreWriteThrough && sizeof(EV) == 16) {
      store_through(base + t0, uint32_t(tile_of<P>(V) * sizeof(E)),
                    uint32_t((u * P::TB + static_cast<int>(threadIdx.x)) * int(sizeof(EV))), v);
      return;
    }
    if (whole(u)) {
      vstore<E, V, P::ST != kStorePlain>(base + j[u], v);
      return;
    }
#pragma unroll
    for (int k = 0; k < V; ++k)
      if (k < cnt[u]) put1(base + j[u] + k, static_cast<E>(v[k]));
  }
  __device__ SV load(const S* base, int u) const { return load_any<S, SV>(base, u); }
  __device__ void store(S* base, int u, SV v) const { store_any<S, SV>(base, u, v); }
  __device__ AV load_acc(const A* base, int u) const { return load_any<A, AV>(base, u); }
  __device__ void store_acc(A* base, int u, AV v) const { store_any<A, AV>(base, u, v); }
};

template <class T>
__device__ inline typename T::S* out_ptr(const RankPtrs& p, int r) {
  return static_cast<typename T::S*>(const_cast<void*>(p.get(r)));
}

template <class T>
__device__ inline const typename T::S* in_ptr(const RankPtrs& p, int r) {
  return static_cast<const typename T::S*>(p.get(r));
}

// acc[u][k] = x^(0) ⊕ x^(1) ⊕ ... ⊕ x^(N-1) at offset off + j[u] + k, folded
// strictly in ascending rank order.  Loads of kRankBatch ranks are issued
// before any of them is combined, so each lane keeps up to kRankBatch·U
// 128-bit loads in flight; the order of the combines is still x^(0),
// x^(1), ... regardless.
template <class T, int OP, class P, bool FULL>
__device__ inline void fold_ranks(const RankPtrs& src, int nranks, uint64_t off, const Lane<T, P, FULL>& ln,
                                  typename T::A (&acc)[P::U][vec_elems<T>()]) {
  constexpr int V = vec_elems<T>();
  constexpr int U = P::U;
  using SV = typename Lane<T, P, FULL>::SV;
  for (int s0 = 0; s0 < nranks; s0 += kRankBatch) {
    SV buf[kRankBatch][U];
#pragma unroll
    for (int b = 0; b < kRankBatch; ++b) {
      if (s0 + b < nranks) {
        const typename T::S* p = in_ptr<T>(src, s0 + b) + off;
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (ln.on(u)) buf[b][u] = ln.load(p, u);
      }
    }
#pragma unroll
    for (int b = 0; b < kRankBatch; ++b) {
      if (s0 + b < nranks) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int k = 0; k < V; ++k) {
            const typename T::A x = T::widen(buf[b][u][k]);
            acc[u][k] = (s0 + b == 0) ? x : combine<T, OP>(acc[u][k], x);
          }
      }
    }
  }
}

// Completed reductions to stored elements: the op's post-operation, then
// the narrowing (bf16 rounding).
template <class T, int OP, class SV>
__device__ inline SV finish_vec(const typename T::A (&acc)[vec_elems<T>()], int nranks) {
  SV v;
#pragma unroll
  for (int k = 0; k < vec_elems<T>(); ++k) v[k] = T::narrow(finalize<T, OP>(acc[k], nranks));
  return v;
}

// ---------------------------------------------------------------------------
// Direct schedule.
// ---------------------------------------------------------------------------
struct ShardArgs {
  RankPtrs send, recv;
  int nranks;
  uint64_t q;                // shard length
  uint64_t tiles_per_shard;  // ceil(q / tile)
  uint64_t ntiles;           // nranks · tiles_per_shard
  uint64_t limit;            // AllGather: recvcount (positions at or past it are trimmed)
};

// ReduceScatter: recv[r][j] = ⊕_s send[s][r·q + j] ([DECOMP] §数学证明;
// [RS-PAGE] equation rs-semantic-output).  One pass over the N inputs, one
// write of the shards: (N+1)·M elements of HBM traffic.
template <class T, int OP, class P, bool FULL>
__device__ inline void rs_tile(const ShardArgs& a, int r, uint64_t seg) {
  using L = Lane<T, P, FULL>;
  constexpr int V = vec_elems<T>();
  const L ln(seg, a.q);
  typename T::A acc[P::U][V];
  fold_ranks<T, OP, P, FULL>(a.send, a.nranks, uint64_t(r) * a.q, ln, acc);
  typename T::S* out = out_ptr<T>(a.recv, r);
#pragma unroll
  for (int u = 0; u < P::U; ++u)
    if (ln.on(u)) ln.store(out, u, finish_vec<T, OP, typename L::SV>(acc[u], a.nranks));
}

template <class T, int OP, class P>
__global__ __launch_bounds__(P::TB) void rs_direct_kernel(ShardArgs a) {
  constexpr uint64_t kTile = tile_of<P>(vec_elems<T>());
  for (uint64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const int r = rank_of_tile(tile, a.tiles_per_shard);
    const uint64_t seg = tile - uint64_t(r) * a.tiles_per_shard;
    if ((seg + 1) * kTile <= a.q)
      rs_tile<T, OP, P, true>(a, r, seg);
    else
      rs_tile<T, OP, P, false>(a, r, seg);
  }
}

// Output fan-out order of the kernels that store one vector into each of
// the N outputs (the AllGather and the direct AllReduce).  With many ranks
// the workgroup starting on tile t begins at output t mod N and wraps
// around, so the workgroups in flight at one moment write into different
// output buffers instead of all into output 0, then all into output 1.
// Measured on float32: the AllGather went from 4.3 to 5.3 TB/s at N = 256,
// 4.6 to 5.35 at N = 128 and 4.7 to 5.0 at N = 64, the direct AllReduce from
// 4.5 to 5.0 TB/s at N = 256; at N = 8 it made no difference, and the plain
// order is kept below the threshold.
#ifndef CCL_SIM_ROTATE_FROM
#define CCL_SIM_ROTATE_FROM 64
#endif
__device__ inline int first_output(uint64_t tile, int nranks) {
  return nranks >= CCL_SIM_ROTATE_FROM ? int(tile % uint64_t(nranks)) : 0;
}

// AllGather: recv[r][s·q + j] = send[s][j] for every r, positions below
// `limit` only ([DECOMP] §数学证明 AllGather, trim of §Contract 实验四).
// Each shard vector is read once into registers and stored N times.
template <class T, bool FULL>
__device__ inline void ag_tile(const ShardArgs& a, int s, uint64_t seg, uint64_t len, int r0) {
  using P = AgPolicy;
  using L = Lane<T, P, FULL>;
  const L ln(seg, len);
  const uint64_t base = uint64_t(s) * a.q;
  const typename T::S* src = in_ptr<T>(a.send, s);
  typename L::SV v[P::U];
#pragma unroll
  for (int u = 0; u < P::U; ++u)
    if (ln.on(u)) v[u] = ln.load(src, u);
  for (int k = 0, r = r0; k < a.nranks; ++k, r = (r + 1 == a.nranks) ? 0 : r + 1) {
    typename T::S* dst = out_ptr<T>(a.recv, r) + base;
#pragma unroll
    for (int u = 0; u < P::U; ++u)
      if (ln.on(u)) ln.store(dst, u, v[u]);
  }
}

template <class T>
__global__ __launch_bounds__(AgPolicy::TB) void ag_direct_kernel(ShardArgs a) {
  constexpr uint64_t kTile = tile_of<AgPolicy>(vec_elems<T>());
  for (uint64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const int s = rank_of_tile(tile, a.tiles_per_shard);
    const uint64_t seg = tile - uint64_t(s) * a.tiles_per_shard;
    const uint64_t base = uint64_t(s) * a.q;
    const uint64_t len = base >= a.limit ? 0 : (a.limit - base < a.q ? a.limit - base : a.q);
    if ((seg + 1) * kTile <= len)
      ag_tile<T, true>(a, s, seg, len, first_output(tile, a.nranks));
    else
      ag_tile<T, false>(a, s, seg, len, first_output(tile, a.nranks));
  }
}

struct FlatArgs {
  RankPtrs send, recv;
  int nranks;
  uint64_t count;
  uint64_t ntiles;
};

// Direct AllReduce in one kernel: y^(r)_i = ⊕_s x^(s)_i stored to all N
// outputs ([DECOMP] §数学证明 Direct AllReduce): 2N·M elements of traffic.
template <class T, int OP, class P, bool FULL>
__device__ inline void ar_tile(const FlatArgs& a, uint64_t tile) {
  using L = Lane<T, P, FULL>;
  constexpr int V = vec_elems<T>();
  const L ln(tile, a.count);
  typename T::A acc[P::U][V];
  fold_ranks<T, OP, P, FULL>(a.send, a.nranks, 0, ln, acc);
  typename L::SV o[P::U];
#pragma unroll
  for (int u = 0; u < P::U; ++u) o[u] = finish_vec<T, OP, typename L::SV>(acc[u], a.nranks);
  const int r0 = first_output(tile, a.nranks);
  for (int k = 0, r = r0; k < a.nranks; ++k, r = (r + 1 == a.nranks) ? 0 : r + 1) {
    typename T::S* dst = out_ptr<T>(a.recv, r);
#pragma unroll
    for (int u = 0; u < P::U; ++u)
      if (ln.on(u)) ln.store(dst, u, o[u]);
  }
}

template <class T, int OP, class P>
__global__ __launch_bounds__(P::TB) void ar_direct_kernel(FlatArgs a) {
  constexpr uint64_t kTile = tile_of<P>(vec_elems<T>());
  for (uint64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    if ((tile + 1) * kTile <= a.count)
      ar_tile<T, OP, P, true>(a, tile);
    else
      ar_tile<T, OP, P, false>(a, tile);
  }
}

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
// by rank r+1 at step t+1, so two generations are live at once).
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
  unsigned* ctrl;
  unsigned spin_limit;
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
template <class T, int OP, class P, bool FULL>
__device__ inline void ring_rs_tile(const RingArgs& a, int t, int r, uint64_t seg, int c, uint64_t len) {
  using A = typename T::A;
  using L = Lane<T, P, FULL>;
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
    const A* theirs = part + uint64_t((t - 1) & 1) * slot + uint64_t(up) * a.q;
#pragma unroll
    for (int u = 0; u < P::U; ++u)
      if (ln.on(u)) in[u] = ln.load_acc(theirs, u);
  }
#pragma unroll
  for (int u = 0; u < P::U; ++u)
    if (ln.on(u)) own[u] = ln.load(mine, u);
  if (!last) {
    A* dst = part + uint64_t(t & 1) * slot + uint64_t(r) * a.q;
#pragma unroll
    for (int u = 0; u < P::U; ++u) {
      if (!ln.on(u)) continue;
      typename L::AV v;
#pragma unroll
      for (int k = 0; k < V; ++k) v[k] = combine<T, OP>(in[u][k], T::widen(own[u][k]));
      ln.store_acc(dst, u, v);
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

// Copy of `len` elements from src to dst for one tile (AllGather steps and
// the stand-alone AllGather's own-shard placement).
template <class T, class P, bool FULL>
__device__ inline void copy_tile(const typename T::S* src, typename T::S* dst, uint64_t seg, uint64_t len) {
  using L = Lane<T, P, FULL>;
  const L ln(seg, len);
  typename L::SV v[P::U];
#pragma unroll
  for (int u = 0; u < P::U; ++u)
    if (ln.on(u)) v[u] = ln.load(src, u);
#pragma unroll
  for (int u = 0; u < P::U; ++u)
    if (ln.on(u)) ln.store(dst, u, v[u]);
}

template <class T, int OP, class P>
__device__ inline void ring_body(const RingArgs& a, int step, uint64_t tile) {
  constexpr uint64_t kTile = tile_of<P>(vec_elems<T>());
  const int n = a.nranks;
  const int r = rank_of_tile(tile, a.tiles_per_chunk);
  const uint64_t seg = tile - uint64_t(r) * a.tiles_per_chunk;
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
      ring_rs_tile<T, OP, P, true>(a, step, r, seg, c, len);
    else
      ring_rs_tile<T, OP, P, false>(a, step, r, seg, c, len);
  } else {
    typename T::S* dst = out_ptr<T>(a.recv, r) + uint64_t(c) * a.q;
    if (full)
      copy_tile<T, P, true>(src, dst, seg, len);
    else
      copy_tile<T, P, false>(src, dst, seg, len);
  }
}

template <class T, int OP, class P>
__global__ __launch_bounds__(P::TB) void ring_step_kernel(RingArgs a) {
  for (uint64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) ring_body<T, OP, P>(a, a.step, tile);
}

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

// Grid-wide barrier for the persistent ring.  Every workgroup of the grid
// is co-resident (cooperative launch) and arrives once per barrier.
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
__device__ inline bool grid_barrier(unsigned* ctrl, unsigned epoch, unsigned spin_limit) {
  __shared__ int s_ok;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned grid = gridDim.x;
    const unsigned groups = grid < unsigned(kCtrlGroups) ? grid : unsigned(kCtrlGroups);
    const unsigned g = blockIdx.x % unsigned(kCtrlGroups);
    const unsigned members = (grid - g + kCtrlGroups - 1) / kCtrlGroups;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const unsigned before = __hip_atomic_fetch_add(ctrl + kCtrlGroup + g * kCtrlLine, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
    if (before + 1u == epoch * members) {
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
      __hip_atomic_fetch_add(ctrl + kCtrlBarrier, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    int ok = 1;
    unsigned spins = 0;
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
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_ok = ok;
  }
  __syncthreads();
  return s_ok != 0;
}

template <class T, int OP, class P>
__global__ __launch_bounds__(P::TB) void ring_persistent_kernel(RingArgs a) {
  const int n = a.nranks;
  const int nsteps = (a.coll == kAllReduce) ? 2 * (n - 1) : (a.coll == kReduceScatter ? n - 1 : n);
  unsigned epoch = 0;
  for (int step = a.first_step; step < nsteps; ++step) {
    if (step > a.first_step && !grid_barrier(a.ctrl, ++epoch, a.spin_limit)) return;
    for (uint64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) ring_body<T, OP, P>(a, step, tile);
  }
}

__global__ void reset_ctrl_kernel(unsigned* ctrl) {
  for (int i = threadIdx.x; i < kCtrlWords; i += blockDim.x) ctrl[i] = 0u;
}

// ---------------------------------------------------------------------------
// Identity padding ([DECOMP] condition three): dst = src for i < count,
// identity(op) for count <= i < padded.
// ---------------------------------------------------------------------------
struct PadArgs {
  RankPtrs src, dst;
  int nranks;
  uint64_t count, padded, tiles_per_rank, ntiles;
};

template <class T, int OP>
__global__ __launch_bounds__(PadPolicy::TB) void pad_kernel(PadArgs a) {
  using S = typename T::S;
  using P = PadPolicy;
  constexpr int V = vec_elems<T>();
  constexpr uint64_t kTile = tile_of<P>(V);
  const S ident = T::narrow(identity<T, OP>());
  for (uint64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const int r = rank_of_tile(tile, a.tiles_per_rank);
    const uint64_t seg = tile - uint64_t(r) * a.tiles_per_rank;
    const S* src = in_ptr<T>(a.src, r);
    S* dst = out_ptr<T>(a.dst, r);
    const uint64_t lo = seg * kTile, hi = lo + kTile;
    if (hi <= a.count) {
      // wholly inside the copied range: a plain vector copy (nothing to do in place)
      if (src != dst) {
        const Lane<T, P, true> ln(seg, a.count);
        typename Lane<T, P, true>::SV v[P::U];
#pragma unroll
        for (int u = 0; u < P::U; ++u) v[u] = ln.load(src, u);
#pragma unroll
        for (int u = 0; u < P::U; ++u) ln.store(dst, u, v[u]);
      }
    } else if (lo >= a.count && hi <= a.padded) {
      // wholly inside the pad: vector stores of the identity
      const Lane<T, P, true> ln(seg, a.padded);
      typename Lane<T, P, true>::SV v;
#pragma unroll
      for (int k = 0; k < V; ++k) v[k] = ident;
#pragma unroll
      for (int u = 0; u < P::U; ++u) ln.store(dst, u, v);
    } else {
      // the tile holding the boundary (or the end): element by element
      const Lane<T, P, false> ln(seg, a.padded);
#pragma unroll
      for (int u = 0; u < P::U; ++u)
        for (int k = 0; k < ln.cnt[u]; ++k) {
          const uint64_t i = ln.j[u] + k;
          if (i < a.count) {
            if (src != dst) put1(dst + i, get1(src + i));
          } else {
            put1(dst + i, ident);
          }
        }
    }
  }
}

struct TableArgs {
  const void* p[kInlineRanks];
  const void** dst;
  int n;
};

__global__ void store_table_kernel(TableArgs a) {
  if (static_cast<int>(threadIdx.x) < a.n) a.dst[threadIdx.x] = a.p[threadIdx.x];
}

// ---------------------------------------------------------------------------
// Host-side dispatch.
// ---------------------------------------------------------------------------
template <class F>
hipError_t by_type(int dtype, F&& f) {
  switch (dtype) {
    case kInt32: return f.template operator()<I32>();
    case kInt64: return f.template operator()<I64>();
    case kFloat32: return f.template operator()<F32>();
    case kBFloat16: return f.template operator()<BF16>();
    default: return hipErrorInvalidValue;
  }
}

template <class T, class F>
hipError_t by_op(int op, F&& f) {
  switch (op) {
    case kSum: return f.template operator()<T, kSum>();
    case kProd: return f.template operator()<T, kProd>();
    case kMax: return f.template operator()<T, kMax>();
    case kMin: return f.template operator()<T, kMin>();
    case kAvg: return f.template operator()<T, kAvg>();
    default: return hipErrorInvalidValue;
  }
}

// Grid cap in workgroups per CU.  The default is high enough that every
// workload here gets one workgroup per tile (measured faster than a capped
// grid-stride loop for all kernels); the loop only matters past it.
#ifndef CCL_SIM_BLOCKS_PER_CU
#define CCL_SIM_BLOCKS_PER_CU 1024
#endif

unsigned grid_for(uint64_t ntiles, int num_cus) {
  const uint64_t cap = uint64_t(num_cus > 0 ? num_cus : 256) * CCL_SIM_BLOCKS_PER_CU;
  const uint64_t g = ntiles < cap ? ntiles : cap;
  return static_cast<unsigned>(g > 0 ? g : 1);
}

template <class T, class P>
uint64_t tile_elems() {
  return tile_of<P>(vec_elems<T>());
}

uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

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

size_t elem_size(int dtype) {
  switch (dtype) {
    case kInt32: return 4;
    case kInt64: return 8;
    case kFloat32: return 4;
    case kBFloat16: return 2;
    default: return 0;
  }
}

size_t accum_size(int dtype) { return dtype == kBFloat16 ? 4 : elem_size(dtype); }

// The fused reductions (ReduceScatter and AllReduce) take two vectors per
// lane when a call produces at most 2^24 elements per output set (M for
// the AllReduce, N·q for the ReduceScatter): each lane then keeps twice as
// many rank loads in flight, which measured 7-9 % faster there (N = 8 at
// M = 2^24, N = 256 at M = 2^22) and 3 % slower at M = 2^28.  The
// AllGather keeps one vector per lane at every size.
#ifndef CCL_SIM_DIRECT_SMALL_CALL
#define CCL_SIM_DIRECT_SMALL_CALL (uint64_t(1) << 24)
#endif

template <class T, int OP, class P>
hipError_t launch_ar_direct(const Call& c) {
  FlatArgs a{};
  a.send = c.send;
  a.recv = c.recv;
  a.nranks = c.nranks;
  a.count = c.limit;
  a.ntiles = ceil_div(c.limit, tile_elems<T, P>());
  hipLaunchKernelGGL((ar_direct_kernel<T, OP, P>), dim3(grid_for(a.ntiles, c.num_cus)), dim3(P::TB), 0, c.stream, a);
  return hipGetLastError();
}

template <class P, class T>
ShardArgs shard_args(const Call& c) {
  ShardArgs a{};
  a.send = c.send;
  a.recv = c.recv;
  a.nranks = c.nranks;
  a.q = c.q;
  a.tiles_per_shard = ceil_div(c.q, tile_elems<T, P>());
  a.ntiles = uint64_t(c.nranks) * a.tiles_per_shard;
  a.limit = c.limit;
  return a;
}

template <class T, int OP, class P>
hipError_t launch_rs_direct(const Call& c) {
  const ShardArgs a = shard_args<P, T>(c);
  hipLaunchKernelGGL((rs_direct_kernel<T, OP, P>), dim3(grid_for(a.ntiles, c.num_cus)), dim3(P::TB), 0, c.stream, a);
  return hipGetLastError();
}

hipError_t run_direct(const Call& c) {
  return by_type(c.dtype, [&]<class T>() -> hipError_t {
    if (c.coll == kAllGather) {
      const ShardArgs a = shard_args<AgPolicy, T>(c);
      hipLaunchKernelGGL((ag_direct_kernel<T>), dim3(grid_for(a.ntiles, c.num_cus)), dim3(AgPolicy::TB), 0, c.stream,
                         a);
      return hipGetLastError();
    }
    const uint64_t produced = (c.coll == kAllReduce) ? c.limit : uint64_t(c.nranks) * c.q;
    const bool small = produced <= CCL_SIM_DIRECT_SMALL_CALL;
    return by_op<T>(c.op, [&]<class U, int OP>() -> hipError_t {
      if (c.coll == kAllReduce)
        return small ? launch_ar_direct<U, OP, DirectSmallPolicy>(c) : launch_ar_direct<U, OP, ArPolicy>(c);
      return small ? launch_rs_direct<U, OP, DirectSmallPolicy>(c) : launch_rs_direct<U, OP, RsPolicy>(c);
    });
  });
}

// Launch shape of the step kernels by step size.  A step that moves few
// elements is over before a one-vector-per-lane grid has ramped up, and two
// vectors per lane (half the workgroups) measured faster there; large steps
// are faster with one.  The crossovers, measured on float32 with N = 8 to
// 256: a ring step (N chunks of q) up to 2^26 elements, a recursive
// halving or doubling step up to 2^24.
#ifndef CCL_SIM_RING_SMALL_STEP
#define CCL_SIM_RING_SMALL_STEP (uint64_t(1) << 26)
#endif
#ifndef CCL_SIM_RECURSIVE_SMALL_STEP
#define CCL_SIM_RECURSIVE_SMALL_STEP (uint64_t(1) << 24)
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

#ifndef CCL_SIM_PERSISTENT_PER_CU
#define CCL_SIM_PERSISTENT_PER_CU 1
#endif

// The persistent grid holds one workgroup per CU (see below), so its lanes
// alone must keep enough loads in flight.  For steps of up to 2^26
// elements a 1024-lane workgroup (a step of N = 256 chunks of 2^14 float32
// is then one tile per workgroup) measured 9-17 % faster than 256 lanes;
// for larger steps 256 lanes were faster.
#ifndef CCL_SIM_PERSIST_SMALL_STEP
#define CCL_SIM_PERSIST_SMALL_STEP (uint64_t(1) << 26)
#endif

template <class T, int OP, class P>
hipError_t launch_persistent(const Call& c, bool* unsupported, PersistentPlan* plan) {
  RingArgs a = make_ring_args(c, tile_elems<T, P>());
  a.first_step = (c.coll == kAllGather && c.in_place) ? 1 : 0;
  if (c.spin_limit) a.spin_limit = c.spin_limit;
  auto kernel = ring_persistent_kernel<T, OP, P>;
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, P::TB, 0);
  if (e != hipSuccess) return e;
  if (per_cu <= 0 || c.num_cus <= 0) {
    *unsupported = true;
    return hipSuccess;
  }
  // Workgroups per CU: at most what the occupancy calculation allows, and
  // by default only CCL_SIM_PERSISTENT_PER_CU of them.  A grid at the full
  // occupancy figure was found not to be co-resident on MI355X (its first
  // barrier ran into the poll limit); of the grids that are, one workgroup
  // per CU measured fastest, at every step size: the barrier's cost grows
  // with the number of workgroups that arrive.
  const int want = c.persistent_per_cu > 0 ? c.persistent_per_cu : CCL_SIM_PERSISTENT_PER_CU;
  const int use = want < per_cu ? want : per_cu;
  uint64_t grid = uint64_t(use) * uint64_t(c.num_cus);
  if (grid > a.ntiles) grid = a.ntiles;
  if (grid == 0) grid = 1;
  if (plan) {
    plan->occupancy_per_cu = per_cu;
    plan->per_cu = use;
    plan->grid = grid;
    plan->tiles_per_step = a.ntiles;
    plan->lanes = P::TB;
  }
  hipLaunchKernelGGL(reset_ctrl_kernel, dim3(1), dim3(kCtrlWords), 0, c.stream, c.ctrl);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  void* args[] = {&a};
  e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kernel), dim3(static_cast<unsigned>(grid)), dim3(P::TB),
                                 args, 0, c.stream);
  if (e == hipErrorCooperativeLaunchTooLarge) {
    (void)hipGetLastError();
    *unsupported = true;
    return hipSuccess;
  }
  return e;
}

hipError_t run_ring_persistent(const Call& c, bool* unsupported, PersistentPlan* plan) {
  *unsupported = false;
  return by_type(c.dtype, [&]<class T>() -> hipError_t {
    const int op = (c.coll == kAllGather) ? int(kSum) : c.op;
    const bool small = uint64_t(c.nranks) * c.q <= CCL_SIM_PERSIST_SMALL_STEP;
    return by_op<T>(op, [&]<class U, int OP>() -> hipError_t {
      return small ? launch_persistent<U, OP, PersistSmallPolicy>(c, unsupported, plan)
                   : launch_persistent<U, OP, PersistPolicy>(c, unsupported, plan);
    });
  });
}

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

hipError_t run_pad(const Call& c, uint64_t count, uint64_t padded) {
  return by_type(c.dtype, [&]<class T>() -> hipError_t {
    const uint64_t tile = tile_elems<T, PadPolicy>();
    PadArgs a{};
    a.src = c.send;
    a.dst = c.recv;
    a.nranks = c.nranks;
    a.count = count;
    a.padded = padded;
    a.tiles_per_rank = ceil_div(padded, tile);
    a.ntiles = uint64_t(c.nranks) * a.tiles_per_rank;
    const unsigned grid = grid_for(a.ntiles, c.num_cus);
    auto go = [&](auto kernel) -> hipError_t {
      hipLaunchKernelGGL(kernel, dim3(grid), dim3(PadPolicy::TB), 0, c.stream, a);
      return hipGetLastError();
    };
    switch (c.op) {
      case kSum: return go(pad_kernel<T, kSum>);
      case kProd: return go(pad_kernel<T, kProd>);
      case kMax: return go(pad_kernel<T, kMax>);
      case kMin: return go(pad_kernel<T, kMin>);
      case kAvg: return go(pad_kernel<T, kAvg>);
      default: return hipErrorInvalidValue;
    }
  });
}

hipError_t upload_table(const void** dev_table, const void* const* host_ptrs, int n, hipStream_t stream) {
  for (int base = 0; base < n; base += kInlineRanks) {
    TableArgs a{};
    a.n = (n - base < kInlineRanks) ? n - base : kInlineRanks;
    a.dst = dev_table + base;
    for (int i = 0; i < a.n; ++i) a.p[i] = host_ptrs[base + i];
    hipLaunchKernelGGL(store_table_kernel, dim3(1), dim3(kInlineRanks), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ccl
