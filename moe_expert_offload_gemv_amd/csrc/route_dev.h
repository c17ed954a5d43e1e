// route_dev.h - device helpers of top-k routing shared by the routing
// kernel and the fused routing + gate/up GEMV (internal to the library).
//
// The argmax of each round is a wave-wide max of one 64-bit key per lane
// (order-preserving float bits, then 0xFFFFFFFF - id) reduced with DPP
// butterflies inside 16-lane rows and four lane reads across rows.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {
namespace route_dev {

// GFX9 DPP controls
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  return ((uint64_t)dpp32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp32<CTRL>((uint32_t)v);
}
__device__ __forceinline__ uint64_t max64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// all 64 lanes must be active
__device__ __forceinline__ uint64_t wave_max64(uint64_t v) {
  v = max64(v, dpp64<kDppQuadXor1>(v));
  v = max64(v, dpp64<kDppQuadXor2>(v));
  v = max64(v, dpp64<kDppRowHalfMirror>(v));
  v = max64(v, dpp64<kDppRowMirror>(v));  // every lane of a 16-lane row holds the row max
  return max64(max64(readlane64(v, 0), readlane64(v, 16)), max64(readlane64(v, 32), readlane64(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += __uint_as_float(dpp32<kDppQuadXor1>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<kDppQuadXor2>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<kDppRowHalfMirror>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<kDppRowMirror>(__float_as_uint(v)));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// order-preserving key: larger logit first, then lower expert id; 0 = none
__device__ __forceinline__ uint64_t route_key(float v, int e) {
  if (v == 0.0f) v = 0.0f;  // -0 and +0 compare equal
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}
__device__ __forceinline__ float key_logit(uint64_t key) {
  const uint32_t u = (uint32_t)(key >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}


// top-k of one token by one wave (all 64 lanes active): key[j] is the key of
// expert lane + 64 j (0 when past E). Lane i < k ends with pick i's expert
// and key; picks are in descending logit order, equal logits lower id first.
template <int NJ>
__device__ __forceinline__ void wave_topk(const uint64_t (&key)[NJ], int E, int k, int lane, int& my_e,
                                          uint64_t& my_key) {
  uint64_t taken = 0;  // bit j: expert lane + 64 j already picked
  my_e = 0;
  my_key = 0;
  for (int i = 0; i < k; ++i) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) best = ((taken >> j) & 1) ? best : max64(best, key[j]);
    best = wave_max64(best);
    int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    e = (e >= 0 && e < E) ? e : 0;  // always an expert of the layer, so every address stays in bounds
    if ((e & 63) == lane) taken |= 1ull << (e >> 6);
    if (lane == i) my_e = e, my_key = best;
  }
}

// softmax over the k chosen logits (lane i < k holds pick i's key; pick 0
// holds the largest): the weight of this lane's pick, 0 on lanes >= k
__device__ __forceinline__ float wave_pick_weight(uint64_t my_key, int k, int lane) {
  const float my_z = key_logit(my_key);
  const float z0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_z), 0));
  const float ex = lane < k ? expf(my_z - z0) : 0.f;
  return ex / wave_sum(ex);
}

}  // namespace route_dev
}  // namespace moe
