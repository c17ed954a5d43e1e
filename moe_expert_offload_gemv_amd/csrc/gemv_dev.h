// gemv_dev.h - device helpers of the decode GEMVs (internal): per-block
// dequantising dot products, the lane mapping of a weight row tile, the row
// reductions, and the LDS staging of a K-vector. Shared by the per-pick and
// grouped GEMVs (decode.hip) and the one-launch layer kernel
// (decode_layer.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "route_dev.h"

namespace moe {
namespace gemv_dev {
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
    // the masks go through v_bitop3 (truth table 0xC0: S0 & S1), whose
    // result the compiler does not see through: with a plain AND it folds
    // each mask into a 4-bit extract per element (extract, convert and FMA
    // per weight) instead of converting the bytes in place (ubyte0..3)
    const uint32_t lo = __builtin_amdgcn_bitop3_b32(w[i], 0x0F0F0F0Fu, 0u, 0xC0);
    const uint32_t hi = __builtin_amdgcn_bitop3_b32(w[i] >> 4, 0x0F0F0F0Fu, 0u, 0xC0);
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

// Sums the per-lane partials of a wave's 4 rows (W values per row) over the
// LPR lanes of each row group at once: two butterfly steps (xor 1, xor 2, by
// DPP) in which each lane keeps half of its rows and adds its partner's
// copies of them, then xor shuffles over the rest of the group. Row i ends
// in the lanes with (lb & 3) == i. Against one full butterfly per row (24
// shuffles through the LDS crossbar per value pair), 2 (LPR = 8) to 8
// (LPR = 64) shuffles per wave.
template <int LPR, int W>
__device__ __forceinline__ void reduce4_rows(const float (&v)[W][4], float (&out)[W]) {
  static_assert(LPR >= 8 && LPR <= 64, "row groups of 8 to 64 lanes");
  const int lane = threadIdx.x & 63;
  const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
  float k[W][2];
#pragma unroll
  for (int w = 0; w < W; ++w)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float keep = b0 ? v[w][2 * i + 1] : v[w][2 * i];
      const float send = b0 ? v[w][2 * i] : v[w][2 * i + 1];
      k[w][i] = keep + __uint_as_float(route_dev::dpp32<route_dev::kDppQuadXor1>(__float_as_uint(send)));
    }
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const float keep = b1 ? k[w][1] : k[w][0];
    const float send = b1 ? k[w][0] : k[w][1];
    out[w] = keep + __uint_as_float(route_dev::dpp32<route_dev::kDppQuadXor2>(__float_as_uint(send)));
  }
#pragma unroll
  for (int m = 4; m < LPR; m <<= 1)
#pragma unroll
    for (int w = 0; w < W; ++w) out[w] += __shfl_xor(out[w], m, 64);
}

// Full butterfly of one value over the LPR lanes of its row group. The
// grouped kernels reduce row by row with it: they run one pick after another
// at two work-groups per CU, where the shuffles of row i overlap the
// arithmetic of row i + 1; a 4-row reduce4_rows chain at the end of every
// pick measured slower there (gate/up 436 -> 470 us, down 205 -> 242 us per
// layer at batch 32 on the 256-expert model).
template <int LPR>
__device__ __forceinline__ float row_reduce(float v) {
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// Loads a cold pick's wave keeps in flight after issuing each row of a
// RowTile (a row is one nibble and one scale load per block). Hot picks
// issue every row at once (HBM wants depth); cold picks pace their
// zero-copy reads row by row. The deeper the pacing the slower the PCIe
// reads: on the 48-layer decode workload, cold gate/up per layer 41.3 us at
// 2, 42.2 at 4, 44.0 at 6, 45.5 at 8, 48.0 at 12; with about 8 cold picks
// per launch (18.9 MB), gate/up 364 us at 2, 326 us (58 GB/s) at 1 and at
// 0, down + combine 171 us at 2, 164 at 1 and 0. Unpaced reads also slowed
// the hot picks sharing the launch.
constexpr int kColdLoadsInFlight = 1;
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// The activation slice of a lane: blocks b_j = lb + LPR*j of a vector of
// 32*KB values, plus the per-block sums used for the -8 offset.
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

// Rows [row0 + it*RPW] (it < NIT) of one Q4 matrix (nibble plane `nib`,
// scale plane `scl`, KB blocks per row) dotted with the lane's slice.
template <int LPR, int BPL, int NIT>
struct RowTile {
  uint4 q[NIT][BPL];
  uint32_t d[NIT][BPL];
  // Row it of the tile. Rows past the matrix load its last row instead
  // (their results are never stored): no branch around a load, so the
  // compiler can count the loads in flight and let each row's arithmetic
  // start as soon as that row is in, instead of waiting for the whole tile.
  // The weights are device memory (the HBM pool, a capture block or mapped
  // pinned host memory): loaded as global, not flat, accesses, which an
  // address read from a table would otherwise get (flat loads also count
  // against the LDS counter, so every LDS read would wait for them).
  __device__ __forceinline__ void load_row(const uint4* __restrict__ nib, const uint16_t* __restrict__ scl, int it,
                                           int row0, int nrows, int lb) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(1))) const u32x4 g_u32x4;
    typedef __attribute__((address_space(1))) const uint16_t g_u16;
    constexpr int RPW = 64 / LPR;
    const int r = min(row0 + it * RPW, nrows - 1);
    const g_u32x4* gn = (const g_u32x4*)nib;
    const g_u16* gs = (const g_u16*)scl;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const int64_t idx = (int64_t)r * (LPR * BPL) + lb + LPR * j;
      const u32x4 w = gn[idx];
      q[it][j] = make_uint4(w.x, w.y, w.z, w.w);
      d[it][j] = gs[idx];
    }
  }
  // pace (wave-uniform): wait after each row until at most
  // kColdLoadsInFlight loads are outstanding
  __device__ __forceinline__ void load(const uint4* __restrict__ nib, const uint16_t* __restrict__ scl, int row0,
                                       int nrows, int lb, bool pace = false) {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      load_row(nib, scl, it, row0, nrows, lb);
      if (pace) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kColdLoadsInFlight));
    }
  }
  // the same bytes, written at the same place of another copy of the matrix
  __device__ __forceinline__ void store(uint4* __restrict__ nib, uint16_t* __restrict__ scl, int row0, int nrows,
                                        int lb) const {
    constexpr int RPW = 64 / LPR;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int r = row0 + it * RPW;
#pragma unroll
      for (int j = 0; j < BPL; ++j) {
        if (r < nrows) {
          const int64_t idx = (int64_t)r * (LPR * BPL) + lb + LPR * j;
          nib[idx] = q[it][j];
          scl[idx] = (uint16_t)d[it][j];
        }
      }
    }
  }
  // Loop-carried use (several activations against the same rows): stops the
  // compiler from hoisting the nibble-to-float conversions out of the loop,
  // which would keep 32 floats per block live instead of 4 packed words.
  __device__ __forceinline__ void keep_packed() {
#pragma unroll
    for (int it = 0; it < NIT; ++it)
#pragma unroll
      for (int j = 0; j < BPL; ++j)
        __asm__ volatile("" : "+v"(q[it][j].x), "+v"(q[it][j].y), "+v"(q[it][j].z), "+v"(q[it][j].w), "+v"(d[it][j]));
  }
  // this lane's share of row group it's dot product (reduce4_rows sums it)
  __device__ __forceinline__ float partial(int it, const float (&xs)[BPL][32], const float (&sx)[BPL]) const {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < BPL; ++j)
      acc = fmaf(half_bits_to_float(d[it][j]), fmaf(-8.0f, sx[j], block_qdot(q[it][j], xs[j])), acc);
    return acc;
  }
};

// The gate and up tiles of the same rows, issued row by row alternately (the
// order gateup_store consumes them), paced as RowTile::load.
template <int LPR, int BPL, int NIT>
__device__ __forceinline__ void load_gateup(RowTile<LPR, BPL, NIT>& g, RowTile<LPR, BPL, NIT>& u, const uint8_t* base,
                                            const ExpertLayout& lay, int row0, int nrows, int lb, bool pace) {
  const uint4* gn = reinterpret_cast<const uint4*>(base + lay.gate_nib);
  const uint16_t* gs = reinterpret_cast<const uint16_t*>(base + lay.gate_scl);
  const uint4* un = reinterpret_cast<const uint4*>(base + lay.up_nib);
  const uint16_t* us = reinterpret_cast<const uint16_t*>(base + lay.up_scl);
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    g.load_row(gn, gs, it, row0, nrows, lb);
    if (pace) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kColdLoadsInFlight));
    u.load_row(un, us, it, row0, nrows, lb);
    if (pace) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kColdLoadsInFlight));
  }
}

// which picks a launch computes: every pick, or only the hot / cold ones
template <int MODE>
__device__ __forceinline__ bool wanted(uint8_t kind) {
  return MODE == kAll || (MODE == kOnlyHot && (kind & kCold) == 0) || (MODE == kOnlyCold && (kind & kCold) != 0);
}

// h rows of one pick: lane lb < 4 of each row group stores row row0 + lb RPW
template <int LPR, int BPL, int NIT>
__device__ __forceinline__ void gateup_store(const RowTile<LPR, BPL, NIT>& g, const RowTile<LPR, BPL, NIT>& u,
                                             const float (&xs)[BPL][32], const float (&sx)[BPL], int row0, int lb,
                                             int nrows, float* __restrict__ out) {
  static_assert(NIT == 4, "reduce4_rows sums 4 rows per lane");
  float pv[2][4], sv[2];
  // row by row in load order (load_gateup): each row waits for its own loads only
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    pv[0][it] = g.partial(it, xs, sx);
    __builtin_amdgcn_sched_barrier(0);
    pv[1][it] = u.partial(it, xs, sx);
    __builtin_amdgcn_sched_barrier(0);
  }
  reduce4_rows<LPR, 2>(pv, sv);
  const int r = row0 + lb * (64 / LPR);
  if (lb < NIT && r < nrows) out[r] = silu(sv[0]) * sv[1];
}
template <int LPR, int BPL, int NIT>
__device__ __forceinline__ void down_store(const RowTile<LPR, BPL, NIT>& d, const float (&hs)[BPL][32],
                                           const float (&sh)[BPL], int row0, int lb, int nrows,
                                           float* __restrict__ out) {
  static_assert(NIT == 4, "reduce4_rows sums 4 rows per lane");
  float pv[1][4], sv[1];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    pv[0][it] = d.partial(it, hs, sh);
    __builtin_amdgcn_sched_barrier(0);
  }
  reduce4_rows<LPR, 1>(pv, sv);
  const int r = row0 + lb * (64 / LPR);
  if (lb < NIT && r < nrows) out[r] = sv[0];
}


// A K-vector (activation row or h row) staged in LDS for every wave of the
// work-group (or for one wave): float4 chunk c of block lb + LPR j sits at
// [(8 j + c) LPR + lb], so a wave's 16-byte reads of one chunk are
// consecutive. KV = K / 4 float4s, a multiple of 64. The copy goes global ->
// LDS by the LDS-DMA form of the global load (lane l writes 16 bytes at
// M0 + 16 l): instruction q fills LDS chunks 64 q .. 64 q + 63, each lane
// fetching the source chunk that belongs there; the waves that share the
// copy take the instructions in turn.
typedef __attribute__((address_space(3))) void lds_void_t;
// cache-policy bit SC1 of a gfx950 memory instruction: device (agent) scope,
// the form an agent-scope atomic load takes
constexpr int kReadCoherent = 16;
typedef __attribute__((address_space(1))) void glb_void_t;

template <int LPR, int BPL>
struct SharedVec {
  static constexpr int KV = 8 * LPR * BPL;
  static_assert(KV % 64 == 0, "whole DMA instructions");
  // instructions first, first + step, ... of the copy. AUX: the loads'
  // cache-policy bits (kReadCoherent: device-coherent reads of data another
  // work-group of the same launch wrote, on any XCD)
  template <int AUX = 0>
  __device__ __forceinline__ static void issue(const float* src, float4* dst, int first, int step, int lane) {
    for (int q = first; q < KV / 64; q += step) {
      const int d = 64 * q + lane;
      const int j = d / (8 * LPR), ch = (d / LPR) % 8, lb = d % LPR;
      __builtin_amdgcn_global_load_lds((glb_void_t*)(src + 4 * (8 * (lb + LPR * j) + ch)),
                                       (lds_void_t*)(dst + 64 * q), 16, 0, AUX);
    }
  }
  // the lane's slice (blocks lb + LPR j) and its block sums, from LDS
  __device__ __forceinline__ static void slice(const float4* src, int lb, float (&xs)[BPL][32], float (&sx)[BPL]) {
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float4 q = src[(j * 8 + c) * LPR + lb];
        xs[j][4 * c + 0] = q.x, xs[j][4 * c + 1] = q.y, xs[j][4 * c + 2] = q.z, xs[j][4 * c + 3] = q.w;
        acc += (q.x + q.y) + (q.z + q.w);
      }
      sx[j] = acc;
    }
  }
  // this wave's copies (and every other memory access it issued) are done,
  // then every wave's: the buffer is complete
  __device__ __forceinline__ static void wait() {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
  }
  // a copy this wave made alone is complete
  __device__ __forceinline__ static void wait_wave() { __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); }
};

// A K-vector in LDS in its own order with an XOR swizzle: float4 c of block
// b at 8 b + (c ^ (b & 7)). Copied by one wave through registers: coalesced
// 16-byte global loads (lane l takes float4s 64 q + l), LDS writes that hit
// distinct banks, and slice reads (a lane's blocks lb + LPR j) that do too.
// Plain loads, unlike the LDS-DMA form, are tracked one by one by the
// compiler's wait counting: issued before the weight loads, they let each
// weight row's arithmetic wait for that row only.
// THREADS: the threads sharing the copy (a wave, or a work-group), thread t
// taking float4s t, t + THREADS, ... (the last index repeats past the end, so
// no load sits behind a branch; the repeats are not stored).
template <int LPR, int BPL, int THREADS = 64>
struct SwizVec {
  static constexpr int KV = 8 * LPR * BPL;                  // float4s of the vector
  static constexpr int NQ = (KV + THREADS - 1) / THREADS;  // per thread
  float4 v[NQ];
  __device__ __forceinline__ void load(const float* __restrict__ src, int t) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(1))) const f32x4 g_f32x4;
    const g_f32x4* s4 = (const g_f32x4*)src;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const f32x4 x = s4[min(THREADS * q + t, KV - 1)];
      v[q] = make_float4(x.x, x.y, x.z, x.w);
    }
  }
  __device__ __forceinline__ void store(float4* dst, int t) const {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int s = THREADS * q + t, b = s >> 3, c = s & 7;
      if (KV % THREADS == 0 || s < KV) dst[b * 8 + (c ^ (b & 7))] = v[q];
    }
  }
  // the lane's slice and its block sums (the -8 offset), summed in load_slice's order
  __device__ __forceinline__ static void slice(const float4* src, int lb, float (&xs)[BPL][32], float (&sx)[BPL]) {
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const int b = lb + LPR * j;
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float4 q = src[b * 8 + (c ^ (b & 7))];
        xs[j][4 * c + 0] = q.x, xs[j][4 * c + 1] = q.y, xs[j][4 * c + 2] = q.z, xs[j][4 * c + 3] = q.w;
        acc += (q.x + q.y) + (q.z + q.w);
      }
      sx[j] = acc;
    }
  }
};

}  // namespace
}  // namespace gemv_dev
}  // namespace moe
