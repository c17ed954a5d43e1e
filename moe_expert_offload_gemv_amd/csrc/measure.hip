// measure.hip - achievable read bandwidth of a plain streaming kernel on
// gfx950: the ceiling the GEMV kernels are compared with beside the spec
// figures (HBM from device memory, PCIe from pinned host memory read
// zero-copy). Not part of the MoE path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_offload.h"

namespace moe {
namespace {

// every thread reads four 16-byte words per round, grid-stride; the loads
// stay because their XOR decides a store the compiler cannot rule out
__global__ __launch_bounds__(256) void read_stream_kernel(const uint4* __restrict__ p, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace
}  // namespace moe

extern "C" int moe_measure_read_bandwidth(const void* ptr, int64_t bytes, int32_t reps, int32_t host_coherent,
                                          void* stream, double* gbps) {
  if (bytes <= 0 || bytes % 16 || reps < 1 || !gbps) return MOE_E_INVAL;
  hipStream_t s = (hipStream_t)stream;
  void* host = nullptr;
  const void* src = ptr;
  uint32_t* sink = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = MOE_OK;
  if (!ptr) {
    const unsigned flags = hipHostMallocMapped | (host_coherent ? hipHostMallocCoherent : hipHostMallocNonCoherent);
    if (hipHostMalloc(&host, (size_t)bytes, flags) != hipSuccess) return MOE_E_NOMEM;
    void* dev = nullptr;
    if (hipHostGetDevicePointer(&dev, host, 0) != hipSuccess) {
      hipHostFree(host);
      return MOE_E_HIP;
    }
    src = dev;
  }
  const int64_t n16 = bytes / 16;
  int dev_id = 0, cus = 256;
  if (hipGetDevice(&dev_id) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev_id);
  const int64_t want = (n16 + 4 * 256 - 1) / (4 * 256);
  const int blocks = (int)(want < 8LL * cus ? (want > 0 ? want : 1) : 8LL * cus);
  float ms = 0.f;
  if (hipMalloc(&sink, 4) != hipSuccess) {
    rc = MOE_E_NOMEM;
  } else if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    rc = MOE_E_HIP;
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(src);
    hipLaunchKernelGGL(moe::read_stream_kernel, dim3(blocks), dim3(256), 0, s, p, n16, sink);  // warm-up
    hipEventRecord(e0, s);
    for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(moe::read_stream_kernel, dim3(blocks), dim3(256), 0, s, p, n16, sink);
    hipEventRecord(e1, s);
    if (hipGetLastError() != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
        hipEventElapsedTime(&ms, e0, e1) != hipSuccess || ms <= 0.f)
      rc = MOE_E_HIP;
    else
      *gbps = (double)bytes * reps / ((double)ms * 1e6);
  }
  if (e0) hipEventDestroy(e0);
  if (e1) hipEventDestroy(e1);
  if (sink) hipFree(sink);
  if (host) hipHostFree(host);
  return rc;
}
