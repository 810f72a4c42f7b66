// v4a_csa_decode_step_noalloc: the decode step of v4a_csa_decode_step with its
// workspace in a fixed device array instead of a caller buffer, for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops that
// forbid allocation).  It allocates nothing: no hipMalloc, no hipFree, no
// allocating library call.
//
// The array `scratch` exists once per GPU (each device that loads the library
// holds its own copy until the process ends).  Host code never passes its name to a
// kernel: the name is a host-side stand-in, so the device address of each GPU's
// copy is looked up once per device with hipGetSymbolAddress (on the first call
// made with that device current) and that address is what the kernels receive.
// Every call on one GPU shares that GPU's copy and it keeps the last call's
// contents; the decode kernels clear every counter they use themselves, so no
// clearing is needed between calls.  Calls that overlap in time on one GPU (two
// streams, two threads) race on the array.
#include "../../include/v4a.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>

#include "internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)V4A_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

// device address of each GPU's copy of `scratch` (null until looked up)
std::atomic<void*> g_scratch[kMaxDevices];

int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    char msg[256];
    snprintf(msg, sizeof(msg), "v4a_csa_decode_step_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    return v4a::report_error(V4A_EIO, msg);
  }
  if (dev < 0 || dev >= kMaxDevices)
    return v4a::report_error(V4A_ENOTSUP, "v4a_csa_decode_step_noalloc: device index beyond 63");
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[256];
      snprintf(msg, sizeof(msg), "v4a_csa_decode_step_noalloc: hipGetSymbolAddress: %s",
               hipGetErrorString(e));
      return v4a::report_error(V4A_EIO, msg);
    }
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return V4A_OK;
}

}  // namespace

extern "C" {

int v4a_csa_decode_step_noalloc(const v4a_decode_step* d, void* stream) {
  if (!d) return v4a::report_error(V4A_EINVAL, "v4a_csa_decode_step_noalloc: null step description");
  const size_t need = v4a_csa_decode_step_workspace(d);
  if (need == 0)
    return v4a::report_error(V4A_EINVAL, "v4a_csa_decode_step_noalloc: invalid step description");
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof(msg),
             "v4a_csa_decode_step_noalloc: the step needs %zu bytes of scratch, the fixed array "
             "holds %zu (use v4a_csa_decode_step with a workspace)",
             need, kScratchBytes);
    return v4a::report_error(V4A_ENOSPC, msg);
  }
  void* ws = nullptr;
  const int rc = scratch_ptr(&ws);
  if (rc != V4A_OK) return rc;
  return v4a::decode_step_run(d, ws, kScratchBytes, stream);
}

}  // extern "C"
