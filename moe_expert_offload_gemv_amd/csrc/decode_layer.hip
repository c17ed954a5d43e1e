// decode_layer.hip - one launch per MoE layer for decode batches of a few
// tokens (1 .. kLayerMaxTokens, top-k <= 8, router logits given, E <= 512).
//
// What is computed is the decode path of decode.hip (routing, slot-table
// lookup, gate/up GEMV + SwiGLU, down GEMV, weighted combine in pick order);
// this file only changes how it is scheduled. The pages put the decode floor
// of a memory-bound MoE step in the per-layer GEMV kernel time and the launch
// overhead (a6000-custom-kernels README, the decode-floor paragraph); the
// down matrix's weights do not depend on h, so they need not wait for a
// second launch.
//
// The 1-D grid holds two kinds of work-groups:
//   [0, T k n_gu)          gate/up work-groups (token, pick, chunk of F rows):
//                          wave 0 routes the token and looks the pick up
//                          while the work-group stages x in LDS, then the
//                          GEMV as gemv_route_gateup_kernel. Their h rows go
//                          out through the device-coherent path (stores
//                          written through to memory); once every wave's
//                          stores are acknowledged, the work-group adds 1 to
//                          its token's counter.
//   [T k n_gu, + T n_dn)   down work-groups (token, chunk of H rows): wave 0
//                          routes the token, each wave issues the loads of
//                          its picks' down-matrix rows (picks wave and wave +
//                          4) straight away, then the work-group waits until
//                          the token's counter shows every gate/up work-group
//                          of its picks done, reads those h rows through the
//                          device-coherent path (they were written on other
//                          XCDs, whose L2s this XCD's does not see), and
//                          finishes the down products and the combine.
// No work-group waits on one with a higher index, and work-groups are
// dispatched in index order, so every awaited gate/up work-group is running
// or done before a down work-group waits for it. The wait is bounded anyway:
// past `max_polls` polls the down work-group sets ctrl->sync_fault (the cache
// step turns it into an error) and goes on with what h holds.
//
// Counter life cycle: 0 when a launch starts; every gate/up work-group of a
// wanted pick adds 1 (n_gu per pick); every down work-group of the token adds
// 1 once its wait is over, and the one that brings the count to its final
// value (all gate/up work-groups plus all n_dn down work-groups) stores 0, so
// the next launch on the stream starts from 0 again. No host memset: the
// launch can be captured in a graph and replayed.
//
// Timing split (kernel timing on): kOnlyHot computes the hot picks' gate/up
// and down (y_pick rows, no combine); kOnlyCold the cold picks', then the
// combine of every pick, the hot ones' from y_pick.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemv_dev.h"
#include "kernels.h"
#include "route_dev.h"

namespace moe {

using namespace gemv_dev;

namespace {

constexpr int kNitGateUp = 4;  // row groups per wave of a gate/up work-group

struct Routed {
  int32_t e[8];     // expert of pick i
  int32_t slot[8];  // its slot in the layer's pool, -1: cold
  uint32_t prev[8]; // its last-miss clock as the step began (0 when not read)
  float w[8];       // routing weight (softmax over the k chosen logits)
};

// Wave 0 (all lanes active) routes token t: the first k picks' expert, slot,
// last-miss clock and weight land in s. Picks in descending logit order,
// equal logits lower expert id first (route_dev's order). When the 8 largest
// order bits are distinct and the 8th occurs once among the E experts, each
// pick has exactly one owner lane, which writes it; otherwise the picks are
// resolved one by one by ballots (route_dev::top8_expert).
__device__ __forceinline__ void route_token(const RouteArgs& r, int t, int k, int lane, bool want_prev,
                                            Routed& s) {
  constexpr int NJ = 8;
  const int E = r.E;
  float z[NJ];
  int32_t tb[NJ];
  uint32_t lm[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    z[j] = e < E ? r.logits[(int64_t)t * E + e] : 0.f;
    tb[j] = e < E ? r.tbl[e] : -1;
    lm[j] = (want_prev && e < E) ? r.last_miss[e] : 0u;
  }
  uint32_t v[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) v[j] = lane + 64 * j < E ? route_dev::order_bits(z[j]) : 0u;
  uint32_t top[8];
  route_dev::wave_top8(v, top);  // every lane ends with the same 8 largest, descending
  bool distinct = top[7] != 0u;
#pragma unroll
  for (int i = 0; i < 7; ++i) distinct = distinct && top[i] != top[i + 1];
  int n_last = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) n_last += __builtin_popcountll(__ballot(v[j] == top[7]));
  if (distinct && n_last == 1) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < k && v[j] == top[i]) s.e[i] = 64 * j + lane, s.slot[i] = tb[j], s.prev[i] = lm[j];
  } else {
    for (int i = 0; i < k; ++i) {
      uint32_t bits;
      const int e = route_dev::top8_expert(v, top, i, E, bits);
      int slot_l = -1;
      uint32_t lm_l = 0;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        slot_l = j == (e >> 6) ? tb[j] : slot_l;
        lm_l = j == (e >> 6) ? lm[j] : lm_l;
      }
      const int slot = __builtin_amdgcn_readlane(slot_l, e & 63);
      const uint32_t prev = (uint32_t)__builtin_amdgcn_readlane((int)lm_l, e & 63);
      if (lane == 0) s.e[i] = e, s.slot[i] = slot, s.prev[i] = prev;
    }
  }
  uint32_t my_bits = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) my_bits = lane == i ? top[i] : my_bits;
  const float wl = route_dev::wave_pick_weight(my_bits, k, lane);
  if (lane < k) s.w[lane] = wl;
}

// the cache step admits a cold pick on its first miss, or on a repeat inside
// the window; such a pick p < capture_picks writes what it reads into the
// layer's capture block p (decode.hip's rule)
__device__ __forceinline__ bool captures(const RouteArgs& r, int p, bool hot, uint32_t prev, uint32_t clk) {
  return !hot && p < r.capture_picks && r.S > 0 &&
         (r.admit_misses == 1 || (prev != 0 && clk - prev < (uint32_t)r.window));
}

template <int LPR_H, int BPL_H, int LPR_F, int BPL_F, int NIT_DN, int MODE>
__global__ __launch_bounds__(256) void decode_layer_kernel(GemvArgs a, RouteArgs r, LayerArgs l) {
  constexpr int KB_H = LPR_H * BPL_H;  // H / 32
  constexpr int KB_F = LPR_F * BPL_F;  // F / 32
  constexpr int H = 32 * KB_H, F = 32 * KB_F;
  constexpr int RPW_H = 64 / LPR_H, RPW_F = 64 / LPR_F;
  constexpr int ROWS_GU = 4 * kNitGateUp * RPW_H;
  constexpr int ROWS_DN = NIT_DN * RPW_F;
  constexpr int N_GU = (F + ROWS_GU - 1) / ROWS_GU;  // gate/up work-groups per pick
  constexpr int N_DN = (H + ROWS_DN - 1) / ROWS_DN;  // down work-groups per token
  static_assert(NIT_DN % 4 == 0, "reduce4_rows sums 4 rows per lane");
  using V = SharedVec<LPR_F, BPL_F>;
  constexpr int XV = KB_H * 8;  // float4s of an x row
  constexpr int BUF = XV > 8 * V::KV ? XV : 8 * V::KV;
  // gate/up: x row, float4 c of block b at 8 b + (c ^ (b & 7)) (the staging
  // writes and the slice reads both hit distinct banks); down: the picks' h rows
  __shared__ float4 s_buf[BUF];
  __shared__ float s_part[8][ROWS_DN];
  __shared__ Routed s_r;
  __shared__ int32_t s_flag;

  const int k = a.k;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_gu_all = a.T * k * N_GU;
  const int bid = blockIdx.x;
  const uint32_t clk0 = r.ctrl->clock;

  if (bid < n_gu_all) {
    // ---------------------------------------------------------------- gate/up
    constexpr int LPR = LPR_H, BPL = BPL_H, NIT = kNitGateUp, RPW = RPW_H;
    const int p = bid / N_GU, xc = bid - p * N_GU;
    const int t = p / k, pick = p - t * k;
    const int lb = lane % LPR, rg = lane / LPR;
    const uint32_t clk = clk0 + (uint32_t)t;
    {
      const float4* src = reinterpret_cast<const float4*>(a.x + (int64_t)t * H);
      for (int q = threadIdx.x; q < XV; q += 256) {
        const int b = q >> 3, c = q & 7;
        s_buf[b * 8 + (c ^ (b & 7))] = src[q];
      }
    }
    const bool policy_wave = r.policy && xc == 0 && wave == 0;
    if (wave == 0) {
      route_token(r, t, k, lane, p < r.capture_picks, s_r);
      if (policy_wave && lane == 0) {
        // the pick's side effects (route_kernel's): record, stamp, count, the
        // pick tables, the capture directory entry, the step's token count
        const int e = s_r.e[pick], slot = s_r.slot[pick];
        const bool hot = slot >= 0;
        const bool capture = captures(r, p, hot, s_r.prev[pick], clk);
        const float w = s_r.w[pick];
        uint64_t rec = ((uint64_t)clk << 32) | ((uint64_t)r.layer << 12) | (uint64_t)e;
        if (hot) {
          rec |= kRecordHit;
          atomicMax(&r.stamps[slot], clk);
        }
        r.records[p] = rec;
        atomicAdd(&r.counts[e], 1u);
        r.ids[p] = e;
        r.w[p] = w;
        r.addr[p] = hot ? r.pool + (int64_t)slot * r.expert_bytes : r.host + (int64_t)e * r.expert_bytes;
        r.kind[p] = hot ? kHot : (capture ? (uint8_t)(kCold | kCaptured) : kCold);
        if (capture) r.cap_dir[p] = ((uint64_t)clk << 32) | (uint64_t)e;
        if (r.ids_user) r.ids_user[p] = e;
        if (r.w_user) r.w_user[p] = w;
        if (p == 0) atomicMax(&r.ctrl->step_tokens, (uint32_t)r.T);
      }
    }
    __syncthreads();
    const int e = __builtin_amdgcn_readfirstlane(s_r.e[pick]);
    const int slot = __builtin_amdgcn_readfirstlane(s_r.slot[pick]);
    const uint32_t prev = (uint32_t)__builtin_amdgcn_readfirstlane((int)s_r.prev[pick]);
    const bool hot = slot >= 0;
    if (!wanted<MODE>(hot ? kHot : kCold)) return;
    const bool capture = captures(r, p, hot, prev, clk);
    const uint8_t* base = hot ? r.pool + (int64_t)slot * r.expert_bytes : r.host + (int64_t)e * r.expert_bytes;
    const int row0 = xc * ROWS_GU + wave * NIT * RPW + rg;
    RowTile<LPR, BPL, NIT> g, u;
    load_gateup(g, u, base, a.lay, row0, F, lb, !hot);
    float xs[BPL][32], sx[BPL];
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const int b = lb + LPR * j;
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float4 q = s_buf[b * 8 + (c ^ (b & 7))];
        xs[j][4 * c + 0] = q.x, xs[j][4 * c + 1] = q.y, xs[j][4 * c + 2] = q.z, xs[j][4 * c + 3] = q.w;
        s += (q.x + q.y) + (q.z + q.w);
      }
      sx[j] = s;
    }
    {
      float pv[2][4], sv[2];
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        pv[0][it] = g.partial(it, xs, sx);
        __builtin_amdgcn_sched_barrier(0);
        pv[1][it] = u.partial(it, xs, sx);
        __builtin_amdgcn_sched_barrier(0);
      }
      reduce4_rows<LPR, 2>(pv, sv);
      const int row = row0 + lb * RPW;
      if (lb < NIT && row < F)
        __hip_atomic_store(l.h + (int64_t)p * F + row, silu(sv[0]) * sv[1], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    // every wave's h stores acknowledged, then the work-group counts itself done
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if (threadIdx.x == 0) atomicAdd(&l.sync[t], 1u);
    if (capture) {  // after the signal: nothing waits for these
      uint8_t* cap = a.capture + (int64_t)p * a.lay.bytes;
      g.store(reinterpret_cast<uint4*>(cap + a.lay.gate_nib), reinterpret_cast<uint16_t*>(cap + a.lay.gate_scl),
              row0, F, lb);
      u.store(reinterpret_cast<uint4*>(cap + a.lay.up_nib), reinterpret_cast<uint16_t*>(cap + a.lay.up_scl), row0, F,
              lb);
    }
    return;
  }

  // ------------------------------------------------------------------ down
  constexpr int LPR = LPR_F, BPL = BPL_F, RPW = RPW_F;
  const int b = bid - n_gu_all;
  const int t = b / N_DN, c = b - t * N_DN;
  const int lb = lane % LPR, rg = lane / LPR;
  const int rows0 = c * ROWS_DN;
  const uint32_t clk = clk0 + (uint32_t)t;
  if (wave == 0) route_token(r, t, k, lane, r.capture_picks > 0, s_r);
  __syncthreads();
  // this wave's picks, wave and wave + 4: their down-matrix rows are loaded
  // now, before h exists
  RowTile<LPR, BPL, NIT_DN> d[2];
  bool want[2] = {false, false}, cap[2] = {false, false};
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int i = wave + 4 * s;
    if (i < k) {
      const int e = __builtin_amdgcn_readfirstlane(s_r.e[i]);
      const int slot = __builtin_amdgcn_readfirstlane(s_r.slot[i]);
      const uint32_t prev = (uint32_t)__builtin_amdgcn_readfirstlane((int)s_r.prev[i]);
      const bool hot = slot >= 0;
      want[s] = wanted<MODE>(hot ? kHot : kCold);
      cap[s] = captures(r, t * k + i, hot, prev, clk);
      if (want[s]) {
        const uint8_t* base = hot ? r.pool + (int64_t)slot * r.expert_bytes : r.host + (int64_t)e * r.expert_bytes;
        d[s].load(reinterpret_cast<const uint4*>(base + a.lay.down_nib),
                  reinterpret_cast<const uint16_t*>(base + a.lay.down_scl), rows0 + rg, H, lb, !hot);
      }
    }
  }
  uint32_t target = 0, depart = 0;
  if (threadIdx.x == 0) {
    int nw = 0;
    for (int i = 0; i < k; ++i) nw += wanted<MODE>(s_r.slot[i] >= 0 ? kHot : kCold) ? 1 : 0;
    target = (uint32_t)(N_GU * nw);
    uint32_t n = 0;
    if (target > 0) {
      for (; n < l.max_polls; ++n) {
        if (__hip_atomic_load(&l.sync[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) break;
        __builtin_amdgcn_s_sleep(1);
      }
      if (n >= l.max_polls) atomicOr(&r.ctrl->sync_fault, 1u);
    }
    depart = atomicAdd(&l.sync[t], 1u);  // the result is needed at the end only
  }
  __syncthreads();
  float4* s_h = s_buf;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int i = wave + 4 * s;
    if (want[s]) V::template issue<kReadCoherent>(l.h + (int64_t)(t * k + i) * F, s_h + i * V::KV, 0, 1, lane);
  }
  V::wait_wave();
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int i = wave + 4 * s;
    if (!want[s]) continue;
    float hs[BPL][32], sh[BPL];
    V::slice(s_h + i * V::KV, lb, hs, sh);
    constexpr int W = NIT_DN / 4;
    float pv[W][4], sv[W];
#pragma unroll
    for (int it = 0; it < NIT_DN; ++it) {
      pv[it / 4][it % 4] = d[s].partial(it, hs, sh);
      __builtin_amdgcn_sched_barrier(0);
    }
    reduce4_rows<LPR, W>(pv, sv);
    if (lb < 4) {
#pragma unroll
      for (int ww = 0; ww < W; ++ww) s_part[i][(4 * ww + lb) * RPW + rg] = sv[ww];
    }
    if (cap[s]) {  // after the arithmetic, as in the gate/up work-groups
      uint8_t* cp = a.capture + (int64_t)(t * k + i) * a.lay.bytes;
      d[s].store(reinterpret_cast<uint4*>(cp + a.lay.down_nib), reinterpret_cast<uint16_t*>(cp + a.lay.down_scl),
                 rows0 + rg, H, lb);
    }
  }
  __syncthreads();
  for (int rr = threadIdx.x; rr < ROWS_DN; rr += 256) {
    const int row = rows0 + rr;
    if (row >= H) continue;
    if (MODE == kOnlyHot) {
      for (int i = 0; i < k; ++i)
        if (s_r.slot[i] >= 0) a.ypick[(int64_t)(t * k + i) * H + row] = s_part[i][rr];
    } else {
      float acc = 0.f;
      for (int i = 0; i < k; ++i) {
        const bool mine = wanted<MODE>(s_r.slot[i] >= 0 ? kHot : kCold);
        const float v = mine ? s_part[i][rr] : a.ypick[(int64_t)(t * k + i) * H + row];
        acc = fmaf(s_r.w[i], v, acc);
      }
      float* yp = l.y + (int64_t)t * H + row;
      *yp = l.accumulate ? *yp + acc : acc;
    }
  }
  if (threadIdx.x == 0 && depart == target + (uint32_t)N_DN - 1u)
    __hip_atomic_store(&l.sync[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int LPR_H, int BPL_H, int LPR_F, int BPL_F, int NIT_DN>
hipError_t layer_t(const GemvArgs& a, const RouteArgs& r, const LayerArgs& l, const Launch& ln, int mode) {
  constexpr int ROWS_GU = 4 * kNitGateUp * (64 / LPR_H);
  constexpr int ROWS_DN = NIT_DN * (64 / LPR_F);
  constexpr int H = 32 * LPR_H * BPL_H, F = 32 * LPR_F * BPL_F;
  constexpr int N_GU = (F + ROWS_GU - 1) / ROWS_GU, N_DN = (H + ROWS_DN - 1) / ROWS_DN;
  if (a.H != H || a.F != F) return hipErrorInvalidValue;
  const dim3 grid(a.T * a.k * N_GU + a.T * N_DN);
  if (mode == kOnlyHot)
    return launch(decode_layer_kernel<LPR_H, BPL_H, LPR_F, BPL_F, NIT_DN, kOnlyHot>, grid, dim3(256), ln, a, r, l);
  if (mode == kOnlyCold)
    return launch(decode_layer_kernel<LPR_H, BPL_H, LPR_F, BPL_F, NIT_DN, kOnlyCold>, grid, dim3(256), ln, a, r, l);
  return launch(decode_layer_kernel<LPR_H, BPL_H, LPR_F, BPL_F, NIT_DN, kAll>, grid, dim3(256), ln, a, r, l);
}

// rows of H per down work-group: NIT_DN row groups of 64 / LPR_F rows
constexpr int kNitDown = 4;

}  // namespace

bool layer_shape_ok(int H, int F, int k, int T, int E) {
  if (T < 1 || T > kLayerMaxTokens || k < 1 || k > 8 || k > E || E > kFusedRouteMaxExperts) return false;
  return (H == 2048 && F == 1024) || (H == 4096 && F == 1536) || (H == 256 && F == 512);
}

hipError_t launch_decode_layer(const GemvArgs& a, const RouteArgs& r, const LayerArgs& l, const Launch& ln, int mode) {
  if (!layer_shape_ok(a.H, a.F, a.k, a.T, r.E) || !r.logits || !r.ctrl || !l.h || !l.y || !l.sync || l.max_polls < 1 ||
      r.pub_seq || (mode != kAll && mode != kOnlyHot && mode != kOnlyCold))
    return hipErrorInvalidValue;
  if (a.H == 2048) return layer_t<64, 1, 32, 1, kNitDown>(a, r, l, ln, mode);
  if (a.H == 4096) return layer_t<64, 2, 16, 3, kNitDown>(a, r, l, ln, mode);
  return layer_t<8, 1, 16, 1, kNitDown>(a, r, l, ln, mode);
}

}  // namespace moe
