// step_copy.hip - the cache step's device-side copies in one launch: the
// promotions (capture block or pinned weights -> pool slot) and the uploads
// of the table, stamps, last-miss copy and control words from pinned,
// device-mapped staging. One launch instead of a copy call per transfer,
// each of which cost a few microseconds of a ~100 us step boundary.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace moe {
namespace {

// Bytes per work-group: 64 per lane, all loaded before any is stored, so a
// chunk read from pinned host memory costs one PCIe round trip, not one per
// 4 KiB (the uploads are host reads of up to ~100 KB each).
constexpr int64_t kCopyChunk = 256 * 64;

// grid = (chunks of the longest transfer, transfers); a work-group moves one
// chunk of one transfer, in 16-byte words when the transfer allows it, else
// in 4-byte words
__global__ __launch_bounds__(256) void copy_list_kernel(CopyList l) {
  const int o = blockIdx.y;
  if (o >= l.n) return;
  const CopyOp op = l.op[o];
  const int64_t b0 = (int64_t)blockIdx.x * kCopyChunk;
  if (b0 >= op.bytes) return;
  const int64_t b1 = op.bytes - b0 < kCopyChunk ? op.bytes : b0 + kCopyChunk;
  if ((((uintptr_t)op.src | (uintptr_t)op.dst | (uint64_t)op.bytes) & 15) == 0) {
    const uint4* s = reinterpret_cast<const uint4*>(op.src);
    uint4* d = reinterpret_cast<uint4*>(op.dst);
    const int64_t i0 = b0 / 16 + threadIdx.x, n = b1 / 16;
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + 256 * u < n) v[u] = s[i0 + 256 * u];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + 256 * u < n) d[i0 + 256 * u] = v[u];
  } else {
    const uint32_t* s = reinterpret_cast<const uint32_t*>(op.src);
    uint32_t* d = reinterpret_cast<uint32_t*>(op.dst);
    const int64_t i0 = b0 / 4 + threadIdx.x, n = b1 / 4;
    uint32_t v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (i0 + 256 * u < n) v[u] = s[i0 + 256 * u];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (i0 + 256 * u < n) d[i0 + 256 * u] = v[u];
  }
}

}  // namespace

hipError_t launch_copy_list(const CopyList& l, hipStream_t s) {
  if (l.n < 0 || l.n > kMaxCopyOps) return hipErrorInvalidValue;
  if (l.n == 0) return hipSuccess;
  int64_t longest = 0;
  for (int i = 0; i < l.n; ++i) {
    const CopyOp& op = l.op[i];
    if (!op.src || !op.dst || op.bytes <= 0 || (op.bytes & 3) || (((uintptr_t)op.src | (uintptr_t)op.dst) & 3))
      return hipErrorInvalidValue;
    longest = op.bytes > longest ? op.bytes : longest;
  }
  const int64_t chunks = (longest + kCopyChunk - 1) / kCopyChunk;
  if (chunks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_list_kernel, dim3((unsigned)chunks, l.n), dim3(256), 0, s, l);
  return hipGetLastError();
}

}  // namespace moe
