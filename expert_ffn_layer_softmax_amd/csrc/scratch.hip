// Library-owned scratch memory for moe_layer_forward_noalloc, the entry
// point for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The scratch is one file-scope device array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  Host code
// never uses the array's name as an address (on the host it names a
// host-side stand-in): the first call on a device, with that device current,
// looks the device copy up with hipGetSymbolAddress and keeps the pointer;
// kernels receive that pointer like any workspace.  All calls on one GPU share
// its copy, so calls that overlap on one GPU race.  No part of it needs
// clearing: every kernel of the layer writes what it later reads.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

static __device__ __align__(256) unsigned char scratch[moe::kScratchBytes];

namespace moe {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

}  // namespace

hipError_t scratch_for_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace moe
