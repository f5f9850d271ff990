// Direct schedule: fused N-way reduce (ReduceScatter), broadcast-copy
// (AllGather) and fused AllReduce, each reading every input once.

#include "kernel_common.hpp"

namespace ccl {
namespace {

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

// The same copy with the fan-out split between H parts of a 256·H-lane
// workgroup: every part loads the tile (the later loads are served by the
// caches), and part h stores outputs h·N/H .. (h+1)·N/H - 1, so each wave
// issues 1/H of the stores per tile.  With H = 2, measured at N = 8 on the
// same buffers against one 256-lane workgroup storing all eight copies:
// 5.8 -> 6.15 TB/s at M = 2^28 float32, 7 % faster in bf16, 5-8 % at
// M = 2^24 and 2^26, 3 % at N = 16, even at N = 4, and 18 % slower at
// N = 2, where each half stores a single copy; with H = 4 it fell to
// 4.7 TB/s at N = 8.  A part is 256 lanes of one vector each by default
// (CCL_SIM_AG_PART_LANES, CCL_SIM_AG_PART_VECS); 512-lane parts measured
// within 1 % at N = 8 to 32 except +6 % in bf16 at N = 8, two vectors per
// lane 6-11 % slower.
#ifndef CCL_SIM_AG_PART_LANES
#define CCL_SIM_AG_PART_LANES 256
#endif
#ifndef CCL_SIM_AG_PART_VECS
#define CCL_SIM_AG_PART_VECS 1
#endif
#ifndef CCL_SIM_AG_PART_ROTATE_MAX
#define CCL_SIM_AG_PART_ROTATE_MAX 6
#endif
using AgPartPolicy = Policy<CCL_SIM_AG_PART_LANES, CCL_SIM_AG_PART_VECS, true, kStoreWriteThrough>;

// The i-th output part h of H stores.  Part h stores outputs h·N/H ..
// (h+1)·N/H - 1.  When a part has at most CCL_SIM_AG_PART_ROTATE_MAX of
// them, the part on tile `seg` of its shard starts at output seg mod count
// and wraps, so that the parts in flight at one moment store into
// different outputs.  Measured with two parts, side by side against the
// unrotated order on the same buffers (float32 unless noted): N = 4 +7 %,
// N = 6 +9 %, N = 8 +3.5 % (AllGather 1.605 against 1.661 ms at M = 2^28;
// the bench step's RS + AG 3.152 against 3.234 ms; bf16 +6 %; M = 2^24
// +10 %, M = 2^26 +5.5 %), N = 12 +2 %; at N = 16 and 24 within 1 %, and
// at N = 32 4 % slower and bf16 at N = 16 3.5 % slower, so larger parts
// keep the plain order.  Two other orders were measured and not kept:
// outputs interleaved between the parts (h, h + H, ...: -2 to +9 %) and the
// odd parts walking theirs backwards (+3.5 % at N = 8 float32, -1 % bf16).
__device__ inline int part_output(int h, int H, int i, int nranks, int* count, uint64_t seg) {
  const int k0 = h * nranks / H, k1 = (h + 1) * nranks / H;
  *count = k1 - k0;
  if (*count > 0 && *count <= CCL_SIM_AG_PART_ROTATE_MAX) return k0 + int((uint64_t(i) + seg) % uint64_t(*count));
  return k0 + i;
}

template <class T, int H>
__device__ inline void ag_tile_parts(const ShardArgs& a, int s, uint64_t seg, uint64_t len) {
  using P = AgPartPolicy;
  constexpr int V = vec_elems<T>();
  constexpr uint64_t kTile = tile_of<P>(V);
  using S = typename T::S;
  using SV = typename VecOf<S, V>::type;
  const int h = static_cast<int>(threadIdx.x) / P::TB, l = static_cast<int>(threadIdx.x) % P::TB;
  const uint64_t base = uint64_t(s) * a.q;
  const uint64_t t0 = seg * kTile;
  const S* src = in_ptr<T>(a.send, s) + t0;
  if (t0 + kTile <= len) {
    SV v[P::U];
#pragma unroll
    for (int u = 0; u < P::U; ++u) v[u] = vload<S, V, P::NTL>(src + uint64_t(u * P::TB + l) * V);
    int count = 0;
    part_output(h, H, 0, a.nranks, &count, seg);
    for (int i = 0; i < count; ++i) {
      const int k = part_output(h, H, i, a.nranks, &count, seg);
#pragma unroll
      for (int u = 0; u < P::U; ++u)
        store_through(out_ptr<T>(a.recv, k) + base + t0, uint32_t(kTile * sizeof(S)),
                      uint32_t((u * P::TB + l) * V * static_cast<int>(sizeof(S))), v[u]);
    }
    return;
  }
  // the ragged last tile of a shard: part 0 copies its valid elements
  if (h != 0) return;
  for (uint64_t j = t0 + uint64_t(l); j < len && j < t0 + kTile; j += P::TB) {
    const S x = get1(src - t0 + j);
    for (int k = 0; k < a.nranks; ++k) put1(out_ptr<T>(a.recv, k) + base + j, x);
  }
}

// Parts per AllGather workgroup for CCL_SIM_AG_PARTS_FROM <= N < 64 (each
// part a 256-lane tile copy).
#ifndef CCL_SIM_AG_PARTS
#define CCL_SIM_AG_PARTS 2
#endif
#ifndef CCL_SIM_AG_PARTS_FROM
#define CCL_SIM_AG_PARTS_FROM 4
#endif

// H = 1: 256-lane workgroups, each storing all N copies of its tile (below
// CCL_SIM_AG_PARTS_FROM ranks, and from 64 up, where the rotated fan-out
// order matters); H > 1: 256·H-lane workgroups split into H parts.
template <class T, int H>
__global__ __launch_bounds__((H > 1 ? AgPartPolicy::TB : AgPolicy::TB) * H) void ag_direct_kernel(ShardArgs a) {
  constexpr uint64_t kTile = tile_of<AgPolicy>(vec_elems<T>());
  for (uint64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const int s = rank_of_tile(tile, a.tiles_per_shard);
    const uint64_t seg = tile - uint64_t(s) * a.tiles_per_shard;
    const uint64_t base = uint64_t(s) * a.q;
    const uint64_t len = base >= a.limit ? 0 : (a.limit - base < a.q ? a.limit - base : a.q);
    if constexpr (H > 1) {
      ag_tile_parts<T, H>(a, s, seg, len);
    } else if ((seg + 1) * kTile <= len) {
      ag_tile<T, true>(a, s, seg, len, first_output(tile, a.nranks));
    } else {
      ag_tile<T, false>(a, s, seg, len, first_output(tile, a.nranks));
    }
  }
}

// The AllGather with its tile staged in LDS: the 256·H lanes of a workgroup
// load a tile of 256·H vectors once, one vector per lane, and park it in
// LDS; after a workgroup barrier, part h (256 lanes) stores the whole tile
// into outputs h·N/H .. (h+1)·N/H - 1, H vectors per lane per output.  No
// part reloads the tile, and each output receives 4·H KiB of contiguous
// stores from one part.  The last, ragged tile of a shard is copied
// element by element by all lanes.
#ifndef CCL_SIM_AG_LDS_PARTS
#define CCL_SIM_AG_LDS_PARTS 0
#endif
template <class T, int H>
__global__ __launch_bounds__(256 * H) void ag_lds_kernel(ShardArgs a) {
  using S = typename T::S;
  constexpr int V = vec_elems<T>();
  using SV = typename VecOf<S, V>::type;
  constexpr int TB = 256 * H;
  constexpr uint64_t kTile = uint64_t(TB) * V;
  __shared__ SV stage[TB];
  const int lane = static_cast<int>(threadIdx.x);
  const int h = lane / 256, l = lane % 256;
  for (uint64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const int s = rank_of_tile(tile, a.tiles_per_shard);
    const uint64_t seg = tile - uint64_t(s) * a.tiles_per_shard;
    const uint64_t base = uint64_t(s) * a.q;
    const uint64_t len = base >= a.limit ? 0 : (a.limit - base < a.q ? a.limit - base : a.q);
    const uint64_t t0 = seg * kTile;
    const S* src = in_ptr<T>(a.send, s) + t0;
    if (t0 + kTile <= len) {
      stage[lane] = vload<S, V, AgPolicy::NTL>(src + uint64_t(lane) * V);
      __syncthreads();
      const int k0 = h * a.nranks / H, k1 = (h + 1) * a.nranks / H;
      for (int k = k0; k < k1; ++k) {
        S* dst = out_ptr<T>(a.recv, k) + base + t0;
#pragma unroll
        for (int i = 0; i < H; ++i)
          store_through(dst, uint32_t(kTile * sizeof(S)), uint32_t((i * 256 + l) * int(sizeof(SV))), stage[i * 256 + l]);
      }
      __syncthreads();  // the next tile reuses the stage
    } else {
      const uint64_t end = len < t0 + kTile ? len : t0 + kTile;
      for (uint64_t j = t0 + uint64_t(lane); j < end; j += TB) {
        const S x = get1(src - t0 + j);
        for (int k = 0; k < a.nranks; ++k) put1(out_ptr<T>(a.recv, k) + base + j, x);
      }
    }
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

// The direct AllReduce with the folded tile shared through LDS: each of
// the 256·H lanes folds its own vector over the N inputs (ascending ranks,
// as ar_tile does) and parks the result in LDS; after a workgroup barrier,
// part h (256 lanes) stores the whole tile into outputs h·N/H ..
// (h+1)·N/H - 1.  The barrier also orders the in-place form: every load of
// the tile's positions, from every input, precedes the first store into
// them.  The ragged last tile takes ar_tile's path (each lane stores its
// own vector to every output).
#ifndef CCL_SIM_AR_LDS_PARTS
#define CCL_SIM_AR_LDS_PARTS 0
#endif
template <class T, int OP, int H>
__global__ __launch_bounds__(256 * H) void ar_lds_kernel(FlatArgs a) {
  using P = Policy<256 * H, 1, true, kStoreWriteThrough>;
  using S = typename T::S;
  constexpr int V = vec_elems<T>();
  using SV = typename VecOf<S, V>::type;
  constexpr uint64_t kTile = tile_of<P>(V);
  __shared__ SV stage[P::TB];
  const int lane = static_cast<int>(threadIdx.x);
  const int h = lane / 256, l = lane % 256;
  for (uint64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    if ((tile + 1) * kTile > a.count) {
      ar_tile<T, OP, P, false>(a, tile);
      continue;
    }
    using L = Lane<T, P, true>;
    const L ln(tile, a.count);
    typename T::A acc[1][V];
    fold_ranks<T, OP, P, true>(a.send, a.nranks, 0, ln, acc);
    stage[lane] = finish_vec<T, OP, SV>(acc[0], a.nranks);
    __syncthreads();
    const uint64_t t0 = tile * kTile;
    const int k0 = h * a.nranks / H, k1 = (h + 1) * a.nranks / H;
    for (int k = k0; k < k1; ++k) {
      S* dst = out_ptr<T>(a.recv, k) + t0;
#pragma unroll
      for (int i = 0; i < H; ++i)
        store_through(dst, uint32_t(kTile * sizeof(S)), uint32_t((i * 256 + l) * int(sizeof(SV))), stage[i * 256 + l]);
    }
    __syncthreads();  // the next tile reuses the stage
  }
}

}  // namespace

// The fused reductions (ReduceScatter and AllReduce) take two vectors per
// lane when a call produces at most 2^24 elements per output set (M for
// the AllReduce, N·q for the ReduceScatter): each lane then keeps twice as
// many rank loads in flight, which measured 7-9 % faster there (N = 8 at
// M = 2^24, N = 256 at M = 2^22) and 3 % slower at M = 2^28.  The
// AllGather keeps one vector per lane at every size.
#ifndef CCL_SIM_DIRECT_SMALL_CALL
#define CCL_SIM_DIRECT_SMALL_CALL (uint64_t(1) << 24)
#endif

template <class T, int OP, int H>
hipError_t launch_ar_lds(const Call& c) {
  FlatArgs a{};
  a.send = c.send;
  a.recv = c.recv;
  a.nranks = c.nranks;
  a.count = c.limit;
  a.ntiles = ceil_div(c.limit, uint64_t(256 * H) * vec_elems<T>());
  hipLaunchKernelGGL((ar_lds_kernel<T, OP, H>), dim3(grid_for(a.ntiles, c.num_cus)), dim3(256 * H), 0, c.stream, a);
  return hipGetLastError();
}

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

// The direct AllReduce on 2-byte types takes 128-lane workgroups, so that
// a tile covers the same 1,024 positions as a float32 tile of ArPolicy.
// Side by side at N = 8, M = 2^28 bf16 in three runs: 1.466-1.500 against
// 1.519-1.554 ms; at M = 2^27 0.698 against 0.724 ms; within 0.5 % at
// N = 256.  (Shapes of one wave of 64 lanes were faster still at some
// sizes and slower at others, in float32 and bf16 alike.)
#ifndef CCL_SIM_AR_HALF_POLICY
#define CCL_SIM_AR_HALF_POLICY 128, 1, true, kStoreWriteThrough
#endif
using ArHalfPolicy = Policy<CCL_SIM_AR_HALF_POLICY>;

hipError_t run_direct(const Call& c) {
  return by_type(c.dtype, [&]<class T>() -> hipError_t {
    if (c.coll == kAllGather) {
      if constexpr (CCL_SIM_AG_LDS_PARTS > 1) {
        if (c.nranks >= CCL_SIM_AG_PARTS_FROM && c.nranks < CCL_SIM_ROTATE_FROM) {
          using LP = Policy<256 * CCL_SIM_AG_LDS_PARTS, 1, true, kStoreWriteThrough>;
          const ShardArgs a = shard_args<LP, T>(c);
          hipLaunchKernelGGL((ag_lds_kernel<T, CCL_SIM_AG_LDS_PARTS>), dim3(grid_for(a.ntiles, c.num_cus)),
                             dim3(LP::TB), 0, c.stream, a);
          return hipGetLastError();
        }
      }
      if (c.nranks >= CCL_SIM_AG_PARTS_FROM && c.nranks < CCL_SIM_ROTATE_FROM) {
        const ShardArgs a = shard_args<AgPartPolicy, T>(c);
        hipLaunchKernelGGL((ag_direct_kernel<T, CCL_SIM_AG_PARTS>), dim3(grid_for(a.ntiles, c.num_cus)),
                           dim3(CCL_SIM_AG_PARTS * AgPartPolicy::TB), 0, c.stream, a);
      } else {
        const ShardArgs a = shard_args<AgPolicy, T>(c);
        hipLaunchKernelGGL((ag_direct_kernel<T, 1>), dim3(grid_for(a.ntiles, c.num_cus)), dim3(AgPolicy::TB), 0,
                           c.stream, a);
      }
      return hipGetLastError();
    }
    const uint64_t produced = (c.coll == kAllReduce) ? c.limit : uint64_t(c.nranks) * c.q;
    const bool small = produced <= CCL_SIM_DIRECT_SMALL_CALL;
    return by_op<T>(c.op, [&]<class U, int OP>() -> hipError_t {
      if (c.coll == kAllReduce) {
        if constexpr (CCL_SIM_AR_LDS_PARTS > 1)
          if (!small && c.nranks >= CCL_SIM_AR_LDS_PARTS) return launch_ar_lds<U, OP, CCL_SIM_AR_LDS_PARTS>(c);
        if (small) return launch_ar_direct<U, OP, DirectSmallPolicy>(c);
        if constexpr (sizeof(typename U::S) == 2) return launch_ar_direct<U, OP, ArHalfPolicy>(c);
        return launch_ar_direct<U, OP, ArPolicy>(c);
      }
      return small ? launch_rs_direct<U, OP, DirectSmallPolicy>(c) : launch_rs_direct<U, OP, RsPolicy>(c);
    });
  });
}

}  // namespace ccl
