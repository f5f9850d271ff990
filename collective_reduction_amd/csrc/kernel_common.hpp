// Device helpers shared by the library's kernels (included by each
// kernels_*.hip file): per-kernel policies, 128-bit memory access helpers,
// the per-lane tile view, the ascending rank fold, and host-side dispatch
// over dtype and op.  Everything here has internal linkage, so each
// translation unit instantiates only what it uses.
//
// The kernels, for gfx950: fused N-way reduce (ReduceScatter), broadcast-copy
// (AllGather), fused AllReduce, ring steps (one launch per step, one
// persistent cooperative kernel with a grid barrier, or one launch in which
// each workgroup chains one chunk slice's steps), recursive halving and
// doubling (one launch per step, or one launch in which each workgroup
// walks one block slice's trees), identity padding.
//
// Pages cited:
//   [DECOMP]  "NCCL 专家课程 07：AllReduce 等价分解、显存生命周期与 Kernel 证据"
//   [RING]    "Ring AllReduce 核心流程：梯度是怎么聚合的"
//   [PRIMS]   "通信与互联（01）：集合通信原语与代价模型——α-β 模型与 ring all-reduce"
//   [WHY-EQ]  "为什么说 AllReduce = ReduceScatter + AllGather？——结合 NCCL Ring AllReduce"
//   [RS-PAGE] "ReduceScatter" (集合通信)
//
// Work decomposition.  Every kernel is a grid-stride loop over tiles (the
// chained drivers: over work items of one tile each) of TB·V·U elements (V = 16 / sizeof(element): one 128-bit access per lane
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

#ifndef CCL_SIM_KERNEL_COMMON_HPP
#define CCL_SIM_KERNEL_COMMON_HPP

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
                           // 16 bytes of a line and measured slower, except
                           // for partials a kernel reads back with its own
                           // tiling, which Lane::store_part lays out so
                           // that they can write through
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

// Agent-coherent accesses, for data that other workgroups, on any of the
// eight XCDs, wrote earlier in the same kernel (the persistent ring's
// partials and forwarded chunks).  Each XCD has its own L2, and a plain load
// may hit a line that another XCD has since rewritten.  A load with sc1
// (agent scope) is coherent across the device, and a store with sc0 sc1
// writes through to memory; once a wave's such stores have completed
// (vmcnt 0), any later agent-scope load on the device sees them.  A grid
// barrier between such accesses then needs no cache write-back or
// invalidation, only the arrival counters.  The accesses go through a
// buffer resource over the workgroup's tile (only buffer instructions take
// explicit cache bits); element accesses cover the ragged ends.
//
// Data written earlier in the kernel by a workgroup on the same XCD can
// instead be read with ordinary loads from that XCD's L2, which every CU of
// the XCD shares and which the writer's write-through stores updated on
// their way to memory, provided the reader's CU first drops its own L1
// (buffer_inv sc0).  Whether a load may do so is the caller's to decide
// (the flag-ordered persistent ring compares the writer's XCD with its own
// at run time).  Side by side, loads with sc0 instead of ordinary ones ran
// as slowly as agent-scope loads.
constexpr int kAgentScope = 16;  // sc1
constexpr int kStreamLoad = 2;   // nt: an ordinary load with the nontemporal hint
using W4 = unsigned __attribute__((ext_vector_type(4)));
__device__ inline __amdgpu_buffer_rsrc_t tile_rsrc(const void* tile_base, uint32_t tile_bytes) {
  const uint64_t addr = reinterpret_cast<uint64_t>(tile_base);
  const uint64_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(addr))));
  const uint64_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(addr >> 32))));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((hi << 32) | lo), 0, int(tile_bytes), kRsrcWord3);
}
template <class EV, int BITS = kAgentScope>
__device__ inline EV load_vec_coherent(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  if constexpr (sizeof(EV) == 16) {
    return __builtin_bit_cast(EV, __builtin_amdgcn_raw_buffer_load_b128(rs, int(off), 0, BITS));
  } else {
    static_assert(sizeof(EV) == 32, "one or two 128-bit vectors");
    struct Pair {
      W4 lo, hi;
    };
    const Pair p{__builtin_amdgcn_raw_buffer_load_b128(rs, int(off), 0, BITS),
                 __builtin_amdgcn_raw_buffer_load_b128(rs, int(off) + 16, 0, BITS)};
    return __builtin_bit_cast(EV, p);
  }
}
template <class EV>
__device__ inline void store_vec_coherent(__amdgpu_buffer_rsrc_t rs, uint32_t off, EV v) {
  if constexpr (sizeof(EV) == 16) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(W4, v), rs, int(off), 0, kSystemScope);
  } else {
    static_assert(sizeof(EV) == 32, "one or two 128-bit vectors");
    struct Pair {
      W4 lo, hi;
    };
    const Pair p = __builtin_bit_cast(Pair, v);
    __builtin_amdgcn_raw_buffer_store_b128(p.lo, rs, int(off), 0, kSystemScope);
    __builtin_amdgcn_raw_buffer_store_b128(p.hi, rs, int(off) + 16, 0, kSystemScope);
  }
}
template <class E, int BITS = kAgentScope>
__device__ inline E load1_coherent(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  if constexpr (sizeof(E) == 2)
    return __builtin_bit_cast(E, __builtin_amdgcn_raw_buffer_load_b16(rs, int(off), 0, BITS));
  else if constexpr (sizeof(E) == 4)
    return __builtin_bit_cast(E, __builtin_amdgcn_raw_buffer_load_b32(rs, int(off), 0, BITS));
  else
    return __builtin_bit_cast(E, __builtin_amdgcn_raw_buffer_load_b64(rs, int(off), 0, BITS));
}
template <class E>
__device__ inline void store1_coherent(__amdgpu_buffer_rsrc_t rs, uint32_t off, E v) {
  if constexpr (sizeof(E) == 2)
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), rs, int(off), 0, kSystemScope);
  else if constexpr (sizeof(E) == 4)
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), rs, int(off), 0, kSystemScope);
  else
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(unsigned __attribute__((ext_vector_type(2))), v), rs,
                                          int(off), 0, kSystemScope);
}

__device__ inline int rank_of_tile(uint64_t tile, uint64_t per) { return static_cast<int>(tile / per); }

__device__ inline int lane_count(uint64_t j, uint64_t len, int v) {
  return j < len ? static_cast<int>(len - j < static_cast<uint64_t>(v) ? len - j : static_cast<uint64_t>(v)) : 0;
}

// One lane's P::U vectors inside a tile.  FULL: the whole tile lies inside
// the valid range, so every vector is complete and no lane checks a count;
// otherwise each vector carries its count of valid elements (0..V) and
// incomplete ones move element by element.
//
// XCD (with CO): loads are ordinary ones with the nontemporal hint, through
// the L1 and the XCD's L2, for data that the caller knows to be fresh there;
// they keep the buffer form, whose base sits in scalar registers; stores
// are the same.
template <class T, class P, bool FULL, bool CO = false, bool XCD = false>
struct Lane {
  static constexpr int kLoadBits = XCD ? kStreamLoad : kAgentScope;
  using S = typename T::S;
  using A = typename T::A;
  static constexpr int U = P::U;
  static constexpr int V = vec_elems<T>();
  using SV = typename VecOf<S, V>::type;
  using AV = typename VecOf<A, V>::type;
  uint64_t t0;  // first element of the tile (the same for every lane)
  uint64_t tv;  // valid elements of the tile from t0 (the tile's size when FULL)
  uint64_t j[U];
  int cnt[U];

  __device__ Lane(uint64_t seg, uint64_t len)
      : t0(seg * tile_of<P>(V)),
        tv(FULL ? tile_of<P>(V) : (len > t0 ? (len - t0 < tile_of<P>(V) ? len - t0 : tile_of<P>(V)) : 0)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      j[u] = seg * tile_of<P>(V) + uint64_t(u * P::TB + static_cast<int>(threadIdx.x)) * V;
      cnt[u] = FULL ? V : lane_count(j[u], len, V);
    }
  }
  __device__ bool on(int u) const { return FULL || cnt[u] > 0; }
  __device__ bool whole(int u) const { return FULL || cnt[u] == V; }

  // CO: every access agent-coherent (see load_vec_coherent).  The
  // resource spans the full tile from t0; a lane's vector u starts at
  // element (u·TB + lane)·V of it.
  template <class E>
  __device__ __amdgpu_buffer_rsrc_t rsrc(const E* base) const {
    return tile_rsrc(base + t0, uint32_t(tile_of<P>(V) * sizeof(E)));
  }
  template <class E>
  __device__ uint32_t offset(int u) const {
    return uint32_t((u * P::TB + static_cast<int>(threadIdx.x)) * V * int(sizeof(E)));
  }

  template <class E, class EV>
  __device__ EV load_any(const E* base, int u) const {
    if constexpr (CO) {
      const auto rs = rsrc(base);
      const uint32_t off = offset<E>(u);
      if (whole(u)) return load_vec_coherent<EV, kLoadBits>(rs, off);
      EV v = {};
#pragma unroll
      for (int k = 0; k < V; ++k)
        if (k < cnt[u]) v[k] = load1_coherent<E, kLoadBits>(rs, off + uint32_t(k * int(sizeof(E))));
      return v;
    }
    if (whole(u)) return vload<E, V, P::NTL>(base + j[u]);
    EV v = {};
#pragma unroll
    for (int k = 0; k < V; ++k)
      if (k < cnt[u]) v[k] = get1(base + j[u] + k);
    return v;
  }
  template <class E, class EV>
  __device__ void store_any(E* base, int u, EV v) const {
    if constexpr (CO) {
      static_assert(P::ST == kStoreWriteThrough, "coherent stores write through");
      const auto rs = rsrc(base);
      const uint32_t off = offset<E>(u);
      if (whole(u)) {
        store_vec_coherent<EV>(rs, off, v);
        return;
      }
#pragma unroll
      for (int k = 0; k < V; ++k)
        if (k < cnt[u]) store1_coherent<E>(rs, off + uint32_t(k * int(sizeof(E))), static_cast<E>(v[k]));
      return;
    }
    if (whole(u)) {
      // a whole vector, also in the last, ragged tile of a shard: the
      // resource spans the full tile, but only valid vectors are stored
      if constexpr (P::ST == kStoreWriteThrough && sizeof(EV) == 16)
        store_through(base + t0, uint32_t(tile_of<P>(V) * sizeof(E)),
                      uint32_t((u * P::TB + static_cast<int>(threadIdx.x)) * int(sizeof(EV))), v);
      else
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

  // Accumulators in a scratch buffer that only this kernel's own tiling
  // reads back (the ring's partials, written at one step and read at the
  // next with the same chunk geometry and policy).  A 32-byte accumulator
  // vector (eight float32 of bf16 data) is stored as two 16-byte halves,
  // the first halves of the tile's valid vectors side by side, then the
  // second halves, so that one store instruction covers whole lines and
  // can write through; the tile keeps its place in the buffer, only the
  // order inside it changes.  This holds for every tile whose valid part
  // is whole vectors (a ragged last tile of a chunk too: its halves then
  // split its valid part, not the full tile).  Other vectors, and tiles
  // that end in a partial vector, use the natural order.
  static constexpr bool kSplitAcc = P::ST == kStoreWriteThrough && sizeof(AV) == 32;
  __device__ bool split() const { return FULL || tv % V == 0; }
  __device__ AV load_part(const A* base, int u) const {
    if constexpr (kSplitAcc) {
      if (split()) {
        using H = typename VecOf<A, V / 2>::type;
        H lo, hi;
        if constexpr (CO) {
          const auto rs = tile_rsrc(base + t0, uint32_t(tv * sizeof(A)));
          const uint32_t off = uint32_t((u * P::TB + static_cast<int>(threadIdx.x)) * int(sizeof(H)));
          lo = load_vec_coherent<H, kLoadBits>(rs, off);
          hi = load_vec_coherent<H, kLoadBits>(rs, off + uint32_t(tv / 2 * sizeof(A)));
        } else {
          const A* half0 = base + t0 + uint64_t(u * P::TB + static_cast<int>(threadIdx.x)) * (V / 2);
          lo = vload<A, V / 2, P::NTL>(half0);
          hi = vload<A, V / 2, P::NTL>(half0 + tv / 2);
        }
        AV v;
#pragma unroll
        for (int k = 0; k < V / 2; ++k) {
          v[k] = lo[k];
          v[k + V / 2] = hi[k];
        }
        return v;
      }
    }
    return load_acc(base, u);
  }
  __device__ void store_part(A* base, int u, AV v) const {
    if constexpr (kSplitAcc) {
      if (split()) {
        using H = typename VecOf<A, V / 2>::type;
        H lo, hi;
#pragma unroll
        for (int k = 0; k < V / 2; ++k) {
          lo[k] = v[k];
          hi[k] = v[k + V / 2];
        }
        const uint32_t half_bytes = uint32_t(tv / 2 * sizeof(A));
        const uint32_t off = uint32_t((u * P::TB + static_cast<int>(threadIdx.x)) * int(sizeof(H)));
        store_through(base + t0, half_bytes, off, lo);
        store_through(base + t0 + tv / 2, half_bytes, off, hi);
        return;
      }
    }
    store_acc(base, u, v);
  }
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

// Copy of `len` elements from src to dst for one tile (AllGather steps and
// the stand-alone AllGather's own-shard placement).
template <class T, class P, bool FULL, bool CO = false, bool XCD = false>
__device__ inline void copy_tile(const typename T::S* src, typename T::S* dst, uint64_t seg, uint64_t len) {
  using L = Lane<T, P, FULL, CO, XCD>;
  const L ln(seg, len);
  typename L::SV v[P::U];
#pragma unroll
  for (int u = 0; u < P::U; ++u)
    if (ln.on(u)) v[u] = ln.load(src, u);
#pragma unroll
  for (int u = 0; u < P::U; ++u)
    if (ln.on(u)) ln.store(dst, u, v[u]);
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

}  // namespace
}  // namespace ccl

#endif  // CCL_SIM_KERNEL_COMMON_HPP
