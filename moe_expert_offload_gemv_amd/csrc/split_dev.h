// split_dev.h - device helpers shared by the routing kernel and the grouped
// matrix-core decode (internal): a row of fp32 values split into two fp16
// operand terms hi + lo after a power-of-two scale.
//
// The row is scaled by 2^s so its largest magnitude lies in [2^13, 2^14)
// (exact), then each value v becomes hi = fp16(v), lo = fp16(v - hi): 22
// significant bits. Stored per quant block of 32 values as 128 bytes: the
// hi chunks 0..3, then the lo chunks 0..3, chunk c holding the elements
// 4c + {0, 2, 1, 3, 16, 18, 17, 19} of the block (the order in which the
// decode MFMA's weight operand comes out of a block's dword c).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {
namespace split_dev {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr int kTop = 14;  // the scaled row's largest magnitude lies in [2^(kTop-1), 2^kTop)

// exponent s of the row scale: m = f 2^e with f in [0.5, 1) gives s = 14 - e;
// a zero or non-finite m keeps 0 (a NaN is kept visible as m = +inf)
__device__ __forceinline__ int scale_exp(float m) {
  if (!(m > 0.f) || !(m <= 3.4028235e38f)) return 0;
  int e;
  (void)frexpf(m, &e);
  return kTop - e;
}

__device__ __forceinline__ float abs_max4(float4 v, float m) {
  m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  return (v.x != v.x || v.y != v.y || v.z != v.z || v.w != v.w) ? __builtin_inff() : m;
}

__device__ __forceinline__ uint32_t pack(_Float16 a, _Float16 b) {
  const f16x2_t v = {a, b};
  uint32_t u;
  __builtin_memcpy(&u, &v, 4);
  return u;
}

// chunk c of block `blk` (32 values) at scale 2^s: hi and lo, 16 bytes each
__device__ __forceinline__ void chunk(const float* blk, int c, int s, uint4& hi, uint4& lo) {
  const float* q = blk + 4 * c;
  const float v[8] = {q[0], q[2], q[1], q[3], q[16], q[18], q[17], q[19]};
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float s0 = ldexpf(v[2 * i], s), s1 = ldexpf(v[2 * i + 1], s);
    const _Float16 h0 = (_Float16)s0, h1 = (_Float16)s1;
    h[i] = pack(h0, h1);
    l[i] = pack((_Float16)(s0 - (float)h0), (_Float16)(s1 - (float)h1));
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

}  // namespace split_dev
}  // namespace moe
