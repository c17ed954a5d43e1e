// scratch.hip - the decode forward's per-call scratch in a static device
// array, for callers that cannot allocate (moe_forward_static_scratch in
// include/moe_offload.h). Each device the library runs on holds its own copy
// of the array from its first use until the process ends.
//
// In host code the name `scratch` is a host-side stand-in, not a device
// address: its device address comes from hipGetSymbolAddress, taken once per
// device with that device current (moe_create calls static_scratch_init),
// and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <vector>

#include "kernels.h"

namespace moe {

namespace {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

std::mutex g_mu;
std::vector<uint8_t*> g_addr;  // per device ordinal: the array's device address, or null

}  // namespace

hipError_t static_scratch_init(int device) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (device < 0) return hipErrorInvalidDevice;
  if ((size_t)device < g_addr.size() && g_addr[device]) return hipSuccess;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != device) return hipErrorInvalidDevice;  // the caller makes the device current
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!p || ((uintptr_t)p & 255)) return hipErrorInvalidSymbol;
  if ((size_t)device >= g_addr.size()) g_addr.resize(device + 1, nullptr);
  g_addr[device] = static_cast<uint8_t*>(p);
  return hipSuccess;
}

uint8_t* static_scratch(int device) {
  std::lock_guard<std::mutex> lock(g_mu);
  return device >= 0 && (size_t)device < g_addr.size() ? g_addr[device] : nullptr;
}

}  // namespace moe
