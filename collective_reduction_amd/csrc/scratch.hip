// Library-owned device scratch for ccl_sim_allreduce_noalloc, the entry
// point for callers that cannot allocate device memory (code under HIP
// graph capture, serving loops, harnesses that forbid hipMalloc).
//
// The scratch is one statically sized device array.  Each GPU the library
// runs on holds its own copy, at its own address, from the moment this
// file's code object is loaded there until the process ends.  In host code
// the array's name is only a host-side stand-in: the device address is read
// once per device with hipGetSymbolAddress, and only that address is ever
// handed to kernels or copies.  Calls on one GPU share its copy, so calls
// that overlap in time on one GPU race on it.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "ccl_sim.h"

namespace ccl {
namespace {

static_assert(CCL_SIM_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte lines");

static __device__ __align__(256) unsigned char scratch[CCL_SIM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

}  // namespace

// Device address of the current device's scratch (*bytes: its size).  The
// first call on a device reads the address with that device current and
// keeps it; later calls return the kept address.
hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  *bytes = CCL_SIM_NOALLOC_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace ccl
