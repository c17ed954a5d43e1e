// route.hip - routing and slot-table lookup of one MoE layer on gfx950, one
// wave per token.
//
// Routing is top-k softmax: the k largest logits (equal logits: lower expert
// id first), listed in that order, weighted by the softmax over the k chosen
// logits. Each pick then looks its expert up in the layer's slot table, the
// per-tensor pointer table of the "a6000-custom-kernels" README (diagram of
// the moe_cache_gemv kernel): a resident expert is read from its HBM slot and
// the slot's use-stamp is raised to the token clock; any other expert is read
// zero-copy from its pinned host copy and the pick is recorded as a miss
// (the README's miss recorder). Every (token, pick) owns a fixed record slot
// (clock << 32 | hit << 31 | layer << 12 | expert), so no returned atomic
// sits on the wave's critical path; the between-step cache step keeps the
// records whose clock lies in the step and sorts the misses.
//
// The argmax of each round is a wave-wide max of one 64-bit key per lane
// (order-preserving float bits, then 0xFFFFFFFF - id) reduced with DPP
// butterflies inside 16-lane rows and four lane reads across rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace moe {

namespace {

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

}  // namespace

template <int NJ>
__global__ __launch_bounds__(64) void route_kernel(RouteArgs a) {
  __shared__ int32_t s_tbl[4096];
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const int E = a.E;

  // issue every load first: logits (or the router chain), the table row, the clock
  float z[NJ];
  if (a.logits) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      z[j] = e < E ? a.logits[(int64_t)t * E + e] : 0.f;
    }
  } else {
    // z_e = fmaf chain over i = 0..H-1 of x_i * W[e][i], starting from 0
    const float* xt = a.x + (int64_t)t * a.H;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      float acc = 0.f;
      if (e < E) {
        const float* we = a.wr + (int64_t)e * a.H;
        for (int i = 0; i < a.H; ++i) acc = fmaf(xt[i], we[i], acc);
      }
      z[j] = acc;
    }
  }
  uint32_t clock0 = 0;
  if (a.policy) {
    clock0 = a.ctrl->clock;
    for (int e = lane; e < E; e += 64) s_tbl[e] = a.tbl[e];
  }

  uint64_t key[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) key[j] = (lane + 64 * j < E) ? route_key(z[j], lane + 64 * j) : 0;

  // k rounds; lane i keeps pick i
  uint64_t taken = 0;  // bit j: expert lane + 64 j already picked
  int my_e = 0;
  uint64_t my_key = 0;
  for (int i = 0; i < a.k; ++i) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) best = ((taken >> j) & 1) ? best : max64(best, key[j]);
    best = wave_max64(best);
    int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    e = (e >= 0 && e < E) ? e : 0;  // always an expert of the layer, so every address stays in bounds
    if ((e & 63) == lane) taken |= 1ull << (e >> 6);
    if (lane == i) my_e = e, my_key = best;
  }

  // softmax over the chosen logits; pick 0 holds the largest
  const float my_z = key_logit(my_key);
  const float z0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_z), 0));
  const float ex = lane < a.k ? expf(my_z - z0) : 0.f;
  const float w = ex / wave_sum(ex);
  __syncthreads();  // the table row in LDS

  if (a.policy && t == 0 && lane == 0) atomicMax(&a.ctrl->step_tokens, (uint32_t)a.T);
  if (lane < a.k) {
    const int e = my_e;
    const int64_t p = (int64_t)t * a.k + lane;
    const uint8_t* addr;
    uint8_t kind;
    if (a.policy) {
      const uint32_t clk = clock0 + (uint32_t)t;
      const int slot = s_tbl[e];
      uint64_t rec = ((uint64_t)clk << 32) | ((uint64_t)a.layer << 12) | (uint64_t)e;
      if (slot >= 0) {
        addr = a.pool + (int64_t)slot * a.expert_bytes;
        kind = kHot;
        rec |= kRecordHit;
        atomicMax(&a.stamps[slot], clk);
      } else {
        addr = a.host + (int64_t)e * a.expert_bytes;
        kind = kCold;
      }
      a.records[p] = rec;
      atomicAdd(&a.counts[e], 1u);
    } else {
      addr = nullptr;  // a prompt pass addresses experts after sorting
      kind = kHot;
    }
    a.ids[p] = e;
    a.w[p] = w;
    if (a.addr) a.addr[p] = addr, a.kind[p] = kind;
    if (a.ids_user) a.ids_user[p] = e;
    if (a.w_user) a.w_user[p] = w;
  }
}

hipError_t launch_route(const RouteArgs& a, const Launch& l) {
  if (a.E < 1 || a.E > 4096 || a.k < 1 || a.k > 32 || a.k > a.E || a.T < 1) return hipErrorInvalidValue;
  const dim3 grid(a.T), block(64);
  if (a.E <= 64) return launch(route_kernel<1>, grid, block, l, a);
  if (a.E <= 128) return launch(route_kernel<2>, grid, block, l, a);
  if (a.E <= 256) return launch(route_kernel<4>, grid, block, l, a);
  if (a.E <= 512) return launch(route_kernel<8>, grid, block, l, a);
  if (a.E <= 1024) return launch(route_kernel<16>, grid, block, l, a);
  if (a.E <= 2048) return launch(route_kernel<32>, grid, block, l, a);
  return launch(route_kernel<64>, grid, block, l, a);
}

}  // namespace moe
