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
// The top-k itself (route_dev.h) is shared with the fused routing + gate/up
// GEMV of the decode path, which routes inside the GEMV when logits are given.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "route_dev.h"
#include "split_dev.h"

namespace moe {

using namespace route_dev;

// One work-group per token: wave 0 routes (64 threads, or 256 when the
// work-group also splits the token's activations for the grouped
// matrix-core decode, which all four waves then do).
template <int NJ>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  __shared__ int32_t s_tbl[4096];
  __shared__ float s_max[4];
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const bool router = tid < 64;  // wave 0
  const int E = a.E;

  // issue every load first: logits (or the router chain), the table row, the clock
  float z[NJ];
  if (router) {
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
  }
  uint32_t clock0 = 0;
  if (a.policy) {
    clock0 = a.ctrl->clock;
    for (int e = tid; e < E; e += blockDim.x) s_tbl[e] = a.tbl[e];
  }

  // k rounds; lane i keeps pick i, then its softmax weight
  int my_e = 0;
  uint32_t my_bits = 0;
  float w = 0.f;
  if (router) {
    wave_topk<NJ>(z, E, a.k, lane, my_e, my_bits);
    w = wave_pick_weight(my_bits, a.k, lane);
  }
  __syncthreads();  // the table row in LDS

  if (router && a.policy && t == 0 && lane == 0) atomicMax(&a.ctrl->step_tokens, (uint32_t)a.T);
  if (router && lane < a.k) {
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
  if (a.xs) {
    // the token's activations as split fp16 operands for the grouped matrix-core decode
    const float* xr = a.x + (int64_t)t * a.H;
    float m = 0.f;
    for (int q = tid; q < a.H / 4; q += blockDim.x) m = split_dev::abs_max4(reinterpret_cast<const float4*>(xr)[q], m);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (lane == 0) s_max[tid >> 6] = m;
    __syncthreads();
    for (int i = 0; i < (int)blockDim.x / 64; ++i) m = fmaxf(m, s_max[i]);
    const int s = split_dev::scale_exp(m);
    if (tid == 0) a.xsig[t] = s;
    const int KB = a.H / 32;
    uint4* out = reinterpret_cast<uint4*>(a.xs) + (int64_t)t * KB * 8;
    for (int q = tid; q < KB * 4; q += blockDim.x) {
      const int b = q >> 2, c = q & 3;
      split_dev::chunk(xr + 32 * b, c, s, out[8 * b + c], out[8 * b + 4 + c]);
    }
  }
}

hipError_t launch_route(const RouteArgs& a, const Launch& l) {
  if (a.E < 1 || a.E > 4096 || a.k < 1 || a.k > 32 || a.k > a.E || a.T < 1) return hipErrorInvalidValue;
  const dim3 grid(a.T), block(a.xs ? 256 : 64);
  if (a.E <= 64) return launch(route_kernel<1>, grid, block, l, a);
  if (a.E <= 128) return launch(route_kernel<2>, grid, block, l, a);
  if (a.E <= 256) return launch(route_kernel<4>, grid, block, l, a);
  if (a.E <= 512) return launch(route_kernel<8>, grid, block, l, a);
  if (a.E <= 1024) return launch(route_kernel<16>, grid, block, l, a);
  if (a.E <= 2048) return launch(route_kernel<32>, grid, block, l, a);
  return launch(route_kernel<64>, grid, block, l, a);
}

}  // namespace moe
