// scratch.hip -- the library's static device scratch, for the entry point that
// allocates nothing (sscan_ssd_fwd_noalloc).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, until the process ends. In host code the
// array's name is only a host-side stand-in, never a device address, so the
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and kept; kernels receive that pointer as they would a
// caller's workspace. Every call on one GPU shares that GPU's array: calls that
// overlap in time on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"
#include "sscan.h"

namespace sscan {

static_assert(kScratchBytes == SSCAN_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");

namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` per device, once resolved

}  // namespace

hipError_t scratch_ptr(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // the current device's copy
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace sscan
