// qkn_mla_decode_attend_noalloc: qkn_mla_decode_attend with its split partials
// in a file-scope device array instead of a caller workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// The array lives in the library's code object: each device the library runs
// on holds its own copy, at its own address, from the module's load until the
// process ends.  Host code never passes the array's name to a kernel or a copy
// (in host code that name is a stand-in, not a device address); it asks the
// runtime for the current device's address once per device and uses that.
#include <mutex>

#include "qkn_internal.h"

namespace qkn {
namespace {

static __device__ __align__(256) uint8_t scratch[QKN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up on the first
// call on each device with that device current; nullptr and the error on failure.
void* scratch_on_current_device(hipError_t* err) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  *err = hipSuccess;
  return addr[dev];
}

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  hipError_t e;
  *ptr = scratch_on_current_device(&e);
  return e;
}

}  // namespace qkn
