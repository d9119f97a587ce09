// ssm_noalloc.hip -- the forward scan for callers that cannot allocate device
// memory (code under HIP graph capture, serving loops, harnesses that forbid
// hipMalloc): ssm_scan_fwd_noalloc runs the plan ssm_scan_fwd_from runs, with
// the chunked form's workspace in a fixed device array of this library
// instead of the stream-ordered pool.
//
// The array lives in the code object (one copy per GPU the library runs on,
// held until the process ends).  Host code never passes its name to a kernel:
// the name is a host-side stand-in, not a device address.  The address of each
// GPU's copy is taken once per device, with that device current, through
// hipGetSymbolAddress, and kept per device.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "ssm_internal.h"

namespace ssm {
namespace {

// The chunked form's workspace: chunk aggregates, chunk step sums and float
// copies of bf16 B / C rows.  No part of it is read before the same call
// writes it, so nothing has to start at zero.
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace ssm
