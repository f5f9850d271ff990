// Identity padding, pointer-table upload and element sizes.

#include "kernel_common.hpp"

namespace ccl {
namespace {

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

namespace {

// Fills `words` 32-bit words with all-ones bits, one 128-bit store per lane
// per step plus a word-wise tail.  As a float32 the pattern is a NaN, as a
// float32 partial of bf16 data too, and as an integer it is -1, so a result
// that folded any word of it is visibly wrong.
__global__ __launch_bounds__(256) void poison_kernel(unsigned* p, uint64_t words) {
  using W4 = unsigned __attribute__((ext_vector_type(4)));
  const uint64_t vecs = words / 4;
  const uint64_t stride = uint64_t(gridDim.x) * blockDim.x;
  W4 ones = {~0u, ~0u, ~0u, ~0u};
  for (uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < vecs; i += stride)
    *(CCL_GLOBAL W4*)(p + 4 * i) = ones;
  for (uint64_t i = vecs * 4 + uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < words; i += stride)
    *(CCL_GLOBAL unsigned*)(p + i) = ~0u;
}

}  // namespace

hipError_t poison_fill(void* p, size_t bytes, hipStream_t stream) {
  const uint64_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  const uint64_t vecs = (words + 3) / 4;
  const uint64_t blocks = (vecs + 255) / 256;
  const unsigned grid = static_cast<unsigned>(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(poison_kernel, dim3(grid), dim3(256), 0, stream, static_cast<unsigned*>(p), words);
  return hipGetLastError();
}

}  // namespace ccl
