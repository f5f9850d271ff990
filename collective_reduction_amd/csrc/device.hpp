// Device-side building blocks for the ccl_sim kernels (gfx950 / CDNA4).
//
// Element types, the reduction operator ⊕ with its identities, bf16
// rounding, and 16-byte vector memory access.  Pages cited:
//   [DECOMP] "NCCL 专家课程 07：AllReduce 等价分解、显存生命周期与 Kernel 证据"
//   [PRIMS]  "通信与互联（01）：集合通信原语与代价模型——α-β 模型与 ring all-reduce"
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ccl {

constexpr int kInlineRanks = 64;  // rank pointers passed in the kernel arguments

#ifndef CCL_SIM_RANK_BATCH
#define CCL_SIM_RANK_BATCH 8      // rank loads issued before they are combined
#endif
constexpr int kRankBatch = CCL_SIM_RANK_BATCH;

// The reduction operators of [PRIMS] §二.1.  AVG combines as SUM and divides
// the completed result by N once, when it is stored (the postOp of the last
// reduce in [DECOMP] §源码三 / §源码四).
enum Op : int { kSum = 0, kProd = 1, kMax = 2, kMin = 3, kAvg = 4 };

// ---------------------------------------------------------------------------
// Element types.  S = stored element, A = accumulator.  Integer SUM / PROD
// run on the unsigned type so overflow wraps modulo 2^bits instead of being
// undefined ([DECOMP] §等价成立的条件, condition five, promises exactness only
// without overflow; wraparound is the defined behaviour chosen for overflow).
// ---------------------------------------------------------------------------
struct I32 {
  using S = int32_t;
  using A = int32_t;
  using U = uint32_t;
  static constexpr bool kFloat = false;
  __device__ static A widen(S v) { return v; }
  __device__ static S narrow(A v) { return v; }
  __device__ static A lowest() { return INT32_MIN; }
  __device__ static A highest() { return INT32_MAX; }
};

struct I64 {
  using S = int64_t;
  using A = int64_t;
  using U = uint64_t;
  static constexpr bool kFloat = false;
  __device__ static A widen(S v) { return v; }
  __device__ static S narrow(A v) { return v; }
  __device__ static A lowest() { return INT64_MIN; }
  __device__ static A highest() { return INT64_MAX; }
};

struct F32 {
  using S = float;
  using A = float;
  using U = uint32_t;
  static constexpr bool kFloat = true;
  __device__ static A widen(S v) { return v; }
  __device__ static S narrow(A v) { return v; }
  __device__ static A lowest() { return -__builtin_huge_valf(); }
  __device__ static A highest() { return __builtin_huge_valf(); }
};

// bf16 is carried as its 16-bit pattern.  Widening to float32 is exact (the
// pattern becomes the upper half of a binary32).  Narrowing rounds to the
// nearest bf16, ties to the even pattern: adding 0x7FFF plus the lowest kept
// bit to the binary32 pattern carries into the kept half exactly when the
// discarded half exceeds one half-ulp, or equals it with an odd kept half;
// a carry out of the mantissa moves into the exponent, so values past the
// largest finite bf16 become infinity.  NaNs are passed on made quiet.
struct BF16 {
  using S = uint16_t;
  using A = float;
  using U = uint32_t;
  static constexpr bool kFloat = true;
  __device__ static A widen(S v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
  __device__ static S narrow(A v) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u)
      return static_cast<S>((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<S>(u >> 16);
  }
  __device__ static A lowest() { return -__builtin_huge_valf(); }
  __device__ static A highest() { return __builtin_huge_valf(); }
};

// Identity of ⊕ ([DECOMP] condition three: 0 for SUM, -inf / the dtype's
// minimum for MAX; 1 for PROD and +inf / maximum for MIN by the same rule).
template <class T, int OP>
__device__ inline typename T::A identity() {
  using A = typename T::A;
  if constexpr (OP == kSum || OP == kAvg) return A(0);
  else if constexpr (OP == kProd) return A(1);
  else if constexpr (OP == kMax) return T::lowest();
  else return T::highest();
}

// a ⊕ b with `a` the running partial.  MAX / MIN keep `a` on a tie; written
// as a compare-and-select so the result never depends on how a hardware
// max instruction orders +0 / -0.
template <class T, int OP>
__device__ inline typename T::A combine(typename T::A a, typename T::A b) {
  using A = typename T::A;
  if constexpr (OP == kSum || OP == kAvg) {
    if constexpr (T::kFloat) return a + b;
    else return static_cast<A>(static_cast<typename T::U>(a) + static_cast<typename T::U>(b));
  } else if constexpr (OP == kProd) {
    if constexpr (T::kFloat) return a * b;
    else return static_cast<A>(static_cast<typename T::U>(a) * static_cast<typename T::U>(b));
  } else if constexpr (OP == kMax) {
    return (b > a) ? b : a;
  } else {
    return (b < a) ? b : a;
  }
}

// The post-operation on a completed reduction: AVG divides by N (one
// correctly rounded float32 division, or integer division truncating toward
// zero); every other op returns the value unchanged.
template <class T, int OP>
__device__ inline typename T::A finalize(typename T::A v, int nranks) {
  using A = typename T::A;
  if constexpr (OP == kAvg) {
    if constexpr (T::kFloat) return v / static_cast<A>(nranks);
    else return v / static_cast<A>(nranks);
  } else {
    return v;
  }
}

// Rank pointers: up to kInlineRanks travel in the kernel arguments; above
// that they are read from a device table in the workspace.
struct RankPtrs {
  const void* p[kInlineRanks];
  const uint64_t* table;  // device addresses, one per rank
  __device__ inline const void* get(int r) const {
    if (table == nullptr) return p[r];
    const uint64_t a = *(const __attribute__((address_space(1))) uint64_t*)(table + r);
    return reinterpret_cast<const void*>(a);
  }
};

}  // namespace ccl
