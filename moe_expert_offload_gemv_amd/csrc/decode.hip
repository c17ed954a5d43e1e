// decode.hip - gfx950 kernels of the decode path of one MoE layer:
//   route_kernel        top-k softmax routing + slot-table lookup, use-stamps
//                       and the miss recorder (one workgroup per token);
//   gemv_gateup_kernel  h = silu(W_gate x) * (W_up x) per pick, weights read
//                       through the per-pick expert address (HBM slot or
//                       pinned host memory, zero-copy over PCIe);
//   gemv_down_kernel    y = sum_i w_i * W_down,i h_i per token, picks combined
//                       in pick order inside the kernel.
//
// What is computed follows the pointer-table GEMV described in the
// "a6000-custom-kernels" README (diagram of the moe_cache_gemv kernel and the
// paragraph under it): each routed expert is found through a table, hot ones
// in a VRAM pool, cold ones in pinned host RAM read zero-copy, cold reads
// logged for a later promotion pass, use-stamps kept for eviction. The
// fused gate/up GEMV follows the narrow-batch mat-vec of the mx-llama.cpp
// FEATURES page (gate and up lanes fused, one mat-vec per expert assignment).
//
// GEMV mapping (MI355X, wave64): a weight row is a run of 16-byte nibble
// blocks; `LPR` consecutive lanes share a row and each lane owns `BPL` blocks
// of it, so one wave-wide 128-bit load covers 64 consecutive blocks (1 KiB)
// and the activation slice a lane needs stays in its registers for every row
// the wave visits. Per block the lane forms sum_j q_j x_j with q in 0..15
// (byte -> float conversions of masked nibbles), then adds
// d * (that - 8 * sum_j x_j), which is sum_j d (q_j - 8) x_j in fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace moe {

namespace {

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
  _Float16 h;
  uint16_t b = (uint16_t)bits;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}

// sum over the 32 elements of a block of q_j * x_j, q_j in 0..15 as stored:
// element j (< 16) is the low nibble of byte j, element j+16 its high nibble.
__device__ __forceinline__ float block_qdot(uint4 q, const float* __restrict__ x) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = w[i] & 0x0F0F0F0Fu;
    const uint32_t hi = (w[i] >> 4) & 0x0F0F0F0Fu;
    a0 = fmaf((float)(lo & 0xffu), x[4 * i + 0], a0);
    a1 = fmaf((float)((lo >> 8) & 0xffu), x[4 * i + 1], a1);
    a0 = fmaf((float)((lo >> 16) & 0xffu), x[4 * i + 2], a0);
    a1 = fmaf((float)(lo >> 24), x[4 * i + 3], a1);
    a0 = fmaf((float)(hi & 0xffu), x[16 + 4 * i + 0], a0);
    a1 = fmaf((float)((hi >> 8) & 0xffu), x[16 + 4 * i + 1], a1);
    a0 = fmaf((float)((hi >> 16) & 0xffu), x[16 + 4 * i + 2], a0);
    a1 = fmaf((float)(hi >> 24), x[16 + 4 * i + 3], a1);
  }
  return a0 + a1;
}

template <int LPR>
__device__ __forceinline__ float row_reduce(float v) {
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// Load the activation slice of a lane: blocks b_j = lb + LPR*j of a row of
// length 32*KB, plus the per-block sums used for the -8 offset.
template <int LPR, int BPL>
__device__ __forceinline__ void load_slice(const float* __restrict__ v, int lb, float (&xs)[BPL][32],
                                           float (&sx)[BPL]) {
#pragma unroll
  for (int j = 0; j < BPL; ++j) {
    const float4* p = reinterpret_cast<const float4*>(v + 32 * (lb + LPR * j));
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float4 q = p[c];
      xs[j][4 * c + 0] = q.x, xs[j][4 * c + 1] = q.y, xs[j][4 * c + 2] = q.z, xs[j][4 * c + 3] = q.w;
      s += (q.x + q.y) + (q.z + q.w);
    }
    sx[j] = s;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// routing + lookup: one workgroup (256 threads) per token.
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  __shared__ float s_z[4096];
  __shared__ uint8_t s_taken[4096];
  __shared__ float s_bv[4];
  __shared__ int s_bi[4];
  __shared__ int s_ids[32];
  __shared__ float s_w[32];

  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int E = a.E;
  if (a.logits) {
    for (int e = tid; e < E; e += 256) s_z[e] = a.logits[(int64_t)t * E + e];
  } else {
    // z_e = fmaf chain over j = 0..H-1 of x_j * W[e][j], starting from 0
    const float* xt = a.x + (int64_t)t * a.H;
    for (int e = tid; e < E; e += 256) {
      const float* we = a.wr + (int64_t)e * a.H;
      float acc = 0.f;
      for (int j = 0; j < a.H; ++j) acc = fmaf(xt[j], we[j], acc);
      s_z[e] = acc;
    }
  }
  for (int e = tid; e < E; e += 256) s_taken[e] = 0;
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6;
  for (int i = 0; i < a.k; ++i) {
    // best = largest logit, ties to the lower id; -1 = none
    float bv = 0.f;
    int bi = -1;
    for (int e = tid; e < E; e += 256) {
      if (s_taken[e]) continue;
      const float v = s_z[e];
      if (bi < 0 || v > bv) bv = v, bi = e;  // ascending e: ties keep the first
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) bv = ov, bi = oi;
    }
    if (lane == 0) s_bv[wave] = bv, s_bi[wave] = bi;
    __syncthreads();
    if (tid == 0) {
      float v = s_bv[0];
      int id = s_bi[0];
      for (int q = 1; q < 4; ++q) {
        const float ov = s_bv[q];
        const int oi = s_bi[q];
        if (oi >= 0 && (id < 0 || ov > v || (ov == v && oi < id))) v = ov, id = oi;
      }
      s_ids[i] = id;
      s_taken[id] = 1;
    }
    __syncthreads();
  }

  if (tid == 0) {
    // softmax over the chosen logits (the first is the largest)
    const float zmax = s_z[s_ids[0]];
    float s = 0.f;
    for (int i = 0; i < a.k; ++i) {
      const float ei = expf(s_z[s_ids[i]] - zmax);
      s_w[i] = ei;
      s += ei;
    }
    const float inv = 1.0f / s;
    for (int i = 0; i < a.k; ++i) s_w[i] = s_w[i] * inv;
    if (a.policy && t == 0) atomicMax(&a.ctrl->step_tokens, (uint32_t)a.T);
  }
  __syncthreads();

  if (tid < a.k) {
    const int i = tid;
    const int e = s_ids[i];
    const int64_t p = (int64_t)t * a.k + i;
    const uint8_t* addr;
    if (a.policy) {
      const uint32_t clk = a.ctrl->clock + (uint32_t)t;
      const int slot = a.tbl[e];
      if (slot >= 0) {
        addr = a.pool + (int64_t)slot * a.expert_bytes;
        atomicMax(&a.stamps[slot], clk);
        atomicAdd(&a.ctrl->hits, 1u);
      } else {
        addr = a.host + (int64_t)e * a.expert_bytes;
        const uint32_t idx = atomicAdd(&a.ctrl->log_count, 1u);
        if (idx < a.log_cap) a.log[idx] = ((uint64_t)clk << 32) | ((uint64_t)a.layer << 12) | (uint64_t)e;
      }
      atomicAdd(&a.counts[e], 1u);
    } else {
      addr = a.pass_addr[e];
    }
    a.ids[p] = e;
    a.w[p] = s_w[i];
    a.addr[p] = addr;
    if (a.ids_user) a.ids_user[p] = e;
    if (a.w_user) a.w_user[p] = s_w[i];
  }
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(route_kernel, dim3(a.T), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// gate/up GEMV + SwiGLU. grid = (row chunks of F, picks); 4 waves per group,
// each wave NIT row groups of 64/LPR rows.
template <int LPR, int BPL, int NIT>
__global__ __launch_bounds__(256) void gemv_gateup_kernel(GemvArgs a) {
  constexpr int RPW = 64 / LPR;
  constexpr int ROWS_WG = 4 * NIT * RPW;
  const int p = blockIdx.y;
  const int t = p / a.k;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lb = lane % LPR, rg = lane / LPR;
  const int KB = LPR * BPL;
  const int F = a.F;
  const uint8_t* base = a.addr[p];
  const uint4* gn = reinterpret_cast<const uint4*>(base + a.lay.gate_nib);
  const uint16_t* gsc = reinterpret_cast<const uint16_t*>(base + a.lay.gate_scl);
  const uint4* un = reinterpret_cast<const uint4*>(base + a.lay.up_nib);
  const uint16_t* usc = reinterpret_cast<const uint16_t*>(base + a.lay.up_scl);

  const int row0 = blockIdx.x * ROWS_WG + wave * NIT * RPW + rg;
  uint4 qg[NIT][BPL], qu[NIT][BPL];
  uint32_t dg[NIT][BPL], du[NIT][BPL];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int r = row0 + it * RPW;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      if (r < F) {
        const int64_t idx = (int64_t)r * KB + lb + LPR * j;
        qg[it][j] = gn[idx];
        qu[it][j] = un[idx];
        dg[it][j] = gsc[idx];
        du[it][j] = usc[idx];
      } else {
        qg[it][j] = qu[it][j] = make_uint4(0, 0, 0, 0);
        dg[it][j] = du[it][j] = 0;
      }
    }
  }
  float xs[BPL][32], sx[BPL];
  load_slice<LPR, BPL>(a.x + (int64_t)t * a.H, lb, xs, sx);

#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      g = fmaf(half_bits_to_float(dg[it][j]), fmaf(-8.0f, sx[j], block_qdot(qg[it][j], xs[j])), g);
      u = fmaf(half_bits_to_float(du[it][j]), fmaf(-8.0f, sx[j], block_qdot(qu[it][j], xs[j])), u);
    }
    g = row_reduce<LPR>(g);
    u = row_reduce<LPR>(u);
    const int r = row0 + it * RPW;
    if (lb == 0 && r < F) a.out[(int64_t)p * F + r] = silu(g) * u;
  }
}

// ---------------------------------------------------------------------------
// down GEMV + weighted combine. grid = (row chunks of H, tokens); the 4 waves
// of a group take picks wave, wave+4, ... of the token over the same rows and
// the group sums them in pick order.
template <int LPR, int BPL, int NIT>
__global__ __launch_bounds__(256) void gemv_down_kernel(GemvArgs a) {
  constexpr int RPW = 64 / LPR;
  constexpr int ROWS = NIT * RPW;
  __shared__ float part[32][ROWS];
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lb = lane % LPR, rg = lane / LPR;
  const int KB = LPR * BPL;
  const int H = a.H, F = a.F;
  const int row0 = blockIdx.x * ROWS;

  for (int i = wave; i < a.k; i += 4) {
    const int64_t p = (int64_t)t * a.k + i;
    const uint8_t* base = a.addr[p];
    const uint4* dn = reinterpret_cast<const uint4*>(base + a.lay.down_nib);
    const uint16_t* dsc = reinterpret_cast<const uint16_t*>(base + a.lay.down_scl);
    uint4 q[NIT][BPL];
    uint32_t d[NIT][BPL];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int r = row0 + it * RPW + rg;
#pragma unroll
      for (int j = 0; j < BPL; ++j) {
        if (r < H) {
          const int64_t idx = (int64_t)r * KB + lb + LPR * j;
          q[it][j] = dn[idx];
          d[it][j] = dsc[idx];
        } else {
          q[it][j] = make_uint4(0, 0, 0, 0);
          d[it][j] = 0;
        }
      }
    }
    float hs[BPL][32], sh[BPL];
    load_slice<LPR, BPL>(a.x + p * F, lb, hs, sh);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < BPL; ++j)
        acc = fmaf(half_bits_to_float(d[it][j]), fmaf(-8.0f, sh[j], block_qdot(q[it][j], hs[j])), acc);
      acc = row_reduce<LPR>(acc);
      if (lb == 0) part[i][it * RPW + rg] = acc;
    }
  }
  __syncthreads();
  for (int rr = threadIdx.x; rr < ROWS; rr += 256) {
    const int r = row0 + rr;
    if (r >= H) continue;
    float acc = 0.f;
    for (int i = 0; i < a.k; ++i) acc = fmaf(a.w[(int64_t)t * a.k + i], part[i][rr], acc);
    float* yp = a.out + (int64_t)t * H + r;
    *yp = a.accumulate ? *yp + acc : acc;
  }
}

bool gemv_shape(int kb, GemvShape* out) {
  if (kb <= 0) return false;
  int lpr = 1;
  while (lpr < 64 && (kb % (lpr * 2)) == 0) lpr *= 2;
  const int bpl = kb / lpr;
  if (lpr < 8 || bpl > 4) return false;
  out->lpr = lpr;
  out->bpl = bpl;
  return true;
}

namespace {
constexpr int kNitGateUp = 4;
constexpr int kNitDown = 4;

template <int LPR, int BPL>
hipError_t launch_gateup_t(const GemvArgs& a, hipStream_t s) {
  constexpr int ROWS_WG = 4 * kNitGateUp * (64 / LPR);
  dim3 grid((a.F + ROWS_WG - 1) / ROWS_WG, a.T * a.k);
  hipLaunchKernelGGL((gemv_gateup_kernel<LPR, BPL, kNitGateUp>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}
template <int LPR, int BPL>
hipError_t launch_down_t(const GemvArgs& a, hipStream_t s) {
  constexpr int ROWS = kNitDown * (64 / LPR);
  dim3 grid((a.H + ROWS - 1) / ROWS, a.T);
  hipLaunchKernelGGL((gemv_down_kernel<LPR, BPL, kNitDown>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

#define MOE_DISPATCH_GEMV(FN, KB, ARGS, STREAM)                       \
  do {                                                                \
    GemvShape sh;                                                     \
    if (!gemv_shape((KB), &sh)) return hipErrorInvalidValue;          \
    switch (sh.lpr * 8 + sh.bpl) {                                    \
      case 8 * 8 + 1: return FN<8, 1>(ARGS, STREAM);                  \
      case 8 * 8 + 2: return FN<8, 2>(ARGS, STREAM);                  \
      case 8 * 8 + 3: return FN<8, 3>(ARGS, STREAM);                  \
      case 8 * 8 + 4: return FN<8, 4>(ARGS, STREAM);                  \
      case 16 * 8 + 1: return FN<16, 1>(ARGS, STREAM);                \
      case 16 * 8 + 2: return FN<16, 2>(ARGS, STREAM);                \
      case 16 * 8 + 3: return FN<16, 3>(ARGS, STREAM);                \
      case 16 * 8 + 4: return FN<16, 4>(ARGS, STREAM);                \
      case 32 * 8 + 1: return FN<32, 1>(ARGS, STREAM);                \
      case 32 * 8 + 2: return FN<32, 2>(ARGS, STREAM);                \
      case 32 * 8 + 3: return FN<32, 3>(ARGS, STREAM);                \
      case 32 * 8 + 4: return FN<32, 4>(ARGS, STREAM);                \
      case 64 * 8 + 1: return FN<64, 1>(ARGS, STREAM);                \
      case 64 * 8 + 2: return FN<64, 2>(ARGS, STREAM);                \
      case 64 * 8 + 3: return FN<64, 3>(ARGS, STREAM);                \
      case 64 * 8 + 4: return FN<64, 4>(ARGS, STREAM);                \
      default: return hipErrorInvalidValue;                           \
    }                                                                 \
  } while (0)
}  // namespace

hipError_t launch_gemv_gateup(const GemvArgs& a, hipStream_t s) { MOE_DISPATCH_GEMV(launch_gateup_t, a.H / 32, a, s); }

hipError_t launch_gemv_down_combine(const GemvArgs& a, hipStream_t s) {
  if (a.k > 32) return hipErrorInvalidValue;
  MOE_DISPATCH_GEMV(launch_down_t, a.F / 32, a, s);
}

}  // namespace moe
