// Fixed device scratch for the allocation-free verify entry point.
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc) call
// paged_attn_verify_noalloc, which runs the same two verify kernels with their
// partial rows, lse values and merge plan in this file-scope array instead of
// a caller-owned workspace.  Each device the library runs on holds its own
// copy of the array, at its own address, until the process ends.
//
// In host code `scratch` names a host-side stand-in, not the device array:
// the device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and kept; only that address is ever handed to a
// kernel.
#include <mutex>

#include "pga_args.h"

namespace pga {

static __device__ __align__(256) unsigned char scratch[kVerifyScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_ptr[kMaxDevices] = {};
}  // namespace

// Device address of `scratch` on the current device, looked up on the first
// call per device.  Returns hipSuccess and the address, or the HIP error of
// the lookup (the address is then left null and the lookup retried next time).
hipError_t verify_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace pga
