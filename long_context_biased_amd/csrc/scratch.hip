// Library-owned device scratch for callers that cannot allocate.
//
// The key-range form of the attention (kv_splits > 1) keeps float32 partial
// numerators and denominators between its two kernels.  The plain entry
// points take that buffer from the caller; abg_biased_mqa_fwd_ex_noalloc
// takes it from this file-scope array instead, so that it needs no
// allocation at all (graph capture, serving loops, harnesses that forbid
// hipMalloc).  Each GPU the library runs on holds its own copy of the array
// from the first launch on that GPU until the process ends.
//
// In host code the array's name is a host-side stand-in, not a device
// address: the device address comes from hipGetSymbolAddress, once per
// device with that device current, and only that address is ever passed to a
// kernel.

#include <hip/hip_runtime.h>

#include <mutex>

#include "abg_internal.h"

namespace {

__device__ __align__(256) unsigned char scratch[abg::kScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace abg {

hipError_t scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace abg
