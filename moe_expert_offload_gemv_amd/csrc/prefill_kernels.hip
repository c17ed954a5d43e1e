// prefill_kernels.hip - gfx950 kernels of the prompt pass of one MoE layer:
// the (token, pick) pairs are sorted by expert and every expert runs as one
// GEMM over its own rows only, the way the "llama.cpp - very large MoE models
// on a 64 GB Mac" README ("Metal kernels": MUL_MAT_ID over used tiles only)
// launches only (expert, tile) pairs that hold tokens.
//
//   expert_histogram_kernel  pair counts per expert
//   expert_scatter_kernel    stable counting sort: perm[pos] = pair, inv[pair] = pos
//   split_rows_kernel        fp32 rows -> bf16 hi and lo planes (x = hi + lo + O(2^-16 x))
//   grouped_gemm_kernel      per tile of one expert: gate/up -> h = silu(g) * u as
//                            bf16 hi/lo planes, or down -> y_pair (fp32)
//   combine_pairs_kernel     y[t] = sum_i w_i y_pair[inv[t, i]] in pick order
//
// MFMA form (v_mfma_f32_16x16x32_bf16, one 32-weight quant block per
// instruction): the weight operand holds 128 + q exactly (bf16 bits 0x4300 | q,
// built from two nibbles per v_and_or), the accumulator enters each block
// holding -136 * sum_k x_k, so the block result is sum_k (q_k - 8) x_k; the
// block's fp16 scale multiplies it in fp32. The activations enter twice, as
// the bf16 hi and lo parts, so the product carries ~16 bits of x while the
// weight codes stay exact. Within every group of four k the operand order is
// (0, 2, 1, 3), which is how two nibbles per dword land in the weight
// operand; the activation planes are stored in that order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 64;   // pair rows per tile
constexpr int BN = 64;   // output features per workgroup (16 per wave)
constexpr int KB = 32;   // one quant block per MFMA step
constexpr int LDS_ROW = KB + 8;  // padded bf16 row in LDS

__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even (finite inputs)
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_float(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// position of logical element k inside its 32-block of an activation plane
__device__ __forceinline__ int plane_pos(int k) { return (k & ~3) | ((k & 1) << 1) | ((k >> 1) & 1); }

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
  _Float16 h;
  uint16_t b = (uint16_t)bits;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}

// eight nibbles (low halves when shift == 0, high halves when shift == 4) of
// the 8 bytes w0,w1 as bf16(128 + q) in operand order (0,2,1,3),(4,6,5,7)
__device__ __forceinline__ bf16x8_t weight_operand(uint32_t w0, uint32_t w1, int shift) {
  w0 >>= shift;
  w1 >>= shift;
  uint32_t p[4];
  p[0] = (w0 & 0x000F000Fu) | 0x43004300u;
  p[1] = ((w0 >> 8) & 0x000F000Fu) | 0x43004300u;
  p[2] = (w1 & 0x000F000Fu) | 0x43004300u;
  p[3] = ((w1 >> 8) & 0x000F000Fu) | 0x43004300u;
  bf16x8_t r;
  __builtin_memcpy(&r, p, 16);
  return r;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

}  // namespace

// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void expert_histogram_kernel(const int32_t* ids, int32_t n_pairs, int32_t E,
                                                               int32_t* counts) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n_pairs) {
    const int e = ids[i];
    if (e >= 0 && e < E) atomicAdd(&counts[e], 1);
  }
}

// one workgroup per expert walks every pair in order (stable)
__global__ __launch_bounds__(256) void expert_scatter_kernel(const int32_t* ids, int32_t n_pairs,
                                                             const int32_t* offsets, int32_t* perm, int32_t* inv) {
  __shared__ int s_wave[4];
  const int e = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int base = offsets[e];
  for (int c = 0; c < n_pairs; c += 256) {
    const int i = c + threadIdx.x;
    const bool hit = i < n_pairs && ids[i] == e;
    const uint64_t m = __ballot(hit);
    const int before_in_wave = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) s_wave[wave] = __popcll(m);
    __syncthreads();
    int before = before_in_wave;
    for (int w = 0; w < wave; ++w) before += s_wave[w];
    const int total = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
    if (hit) {
      perm[base + before] = i;
      inv[i] = base + before;
    }
    base += total;
    __syncthreads();
  }
}

// rows of fp32 [R][K] -> bf16 hi and lo planes [R][K] in operand order, and
// per (row, 32-block) -136 * sum of (hi + lo): one thread per block
__global__ __launch_bounds__(256) void split_rows_kernel(const float* src, int64_t nblocks, int32_t K, uint16_t* hi,
                                                         uint16_t* lo, float* bsum) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const float4* s4 = reinterpret_cast<const float4*>(src + b * 32);
  uint16_t h[32], l[32];
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float4 q = s4[c];
    const float v[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = 4 * c + j;
      const uint16_t hh = bf16_bits_rne(v[j]);
      const uint16_t ll = bf16_bits_rne(v[j] - bf16_to_float(hh));
      h[plane_pos(k)] = hh;
      l[plane_pos(k)] = ll;
      sum += bf16_to_float(hh) + bf16_to_float(ll);
    }
  }
  uint4* ph = reinterpret_cast<uint4*>(hi + b * 32);
  uint4* pl = reinterpret_cast<uint4*>(lo + b * 32);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t wh[4], wl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wh[j] = (uint32_t)h[8 * c + 2 * j] | ((uint32_t)h[8 * c + 2 * j + 1] << 16);
      wl[j] = (uint32_t)l[8 * c + 2 * j] | ((uint32_t)l[8 * c + 2 * j + 1] << 16);
    }
    ph[c] = make_uint4(wh[0], wh[1], wh[2], wh[3]);
    pl[c] = make_uint4(wl[0], wl[1], wl[2], wl[3]);
  }
  bsum[b] = -136.0f * sum;
  (void)K;
}

namespace {
// GFX9 DPP controls (butterflies inside a 16-lane row)
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
// sum over the 16 lanes of a DPP row; every lane of the row gets it
__device__ __forceinline__ float row16_sum(float v) {
  v += dppf<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dppf<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dppf<0x141>(v);  // row_half_mirror
  v += dppf<0x140>(v);  // row_mirror
  return v;
}
constexpr int kDepth = 1;  // blocks of A and B in flight ahead of the one computed
}  // namespace

// One workgroup computes a 64-row tile of one expert's pairs against
// 4 waves x NSUB x 16 output features.
// MODE 0: gate/up (two weight matrices, SwiGLU, writes h planes and their
//         per-block -136 * sums); NSUB = 2, so each wave owns one 32-feature
//         block of h.
// MODE 1: down (one matrix, writes y_pair); NSUB = 4.
// Work items are numbered so that each XCD (work item id mod 8 of the launch
// order) gets a contiguous range: the n-tiles of one row tile, then the next
// row tile of the same expert, share an L2.
template <int MODE>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmArgs a) {
  constexpr int NMAT = MODE == 0 ? 2 : 1;
  constexpr int NSUB = MODE == 0 ? 2 : 4;
  constexpr int WN = 16 * NSUB;  // features per wave
  constexpr int BNW = 4 * WN;    // features per workgroup
  __shared__ uint16_t sA[2][2][BM][LDS_ROW];  // [stage][hi/lo][row][k]
  __shared__ float sC[2][BM];                 // -136 * sum_k x_k per row and stage

  // XCD-contiguous work numbering
  const int L = blockIdx.x;
  const int per = a.work_padded / 8;
  const int W = (L & 7) * per + (L >> 3);
  if (W >= a.work) return;
  const int n_tiles_n = (a.N + BNW - 1) / BNW;
  const int4 tile = a.tiles[W / n_tiles_n];
  const int e = tile.x, pos0 = tile.y, rows = tile.z;
  const int n0 = (W % n_tiles_n) * BNW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, N = a.N, nkb = K / KB;
  const uint8_t* base = a.eaddr[e];

  // A staging: thread -> (row ar, quarter aq of the block): 8 elements of each plane
  const int ar = tid >> 2, aq = tid & 3;
  const bool arow_ok = ar < rows;
  int64_t src_row = 0;
  if (arow_ok) src_row = a.arow ? (int64_t)(a.arow[pos0 + ar] / a.arow_div) : (int64_t)(pos0 + ar);
  const uint16_t* pah = a.ah + src_row * K + aq * 8;
  const uint16_t* pal = a.al + src_row * K + aq * 8;
  const float* psum = a.asum + src_row * nkb;

  // B: lane -> (feature lane % 16 of each of the wave's NSUB subtiles, k-quarter kq)
  const int kq = lane >> 4;
  const int shift = (kq >> 1) * 4;
  // per-matrix planes (uniform) and per-subtile block index of this lane's row (32-bit)
  const uint8_t* nibm[NMAT];
  const uint16_t* sclm[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    nibm[m] = base + (MODE == 1 ? a.lay.down_nib : (m == 0 ? a.lay.gate_nib : a.lay.up_nib)) + (kq & 1) * 8;
    sclm[m] = reinterpret_cast<const uint16_t*>(base + (MODE == 1 ? a.lay.down_scl : (m == 0 ? a.lay.gate_scl
                                                                                              : a.lay.up_scl)));
  }
  uint32_t brow[NSUB];  // block index of (row, k-block 0); every expert matrix is < 4 GiB
  bool bok[NSUB];
#pragma unroll
  for (int ns = 0; ns < NSUB; ++ns) {
    const int bn = n0 + wave * WN + ns * 16 + (lane & 15);
    bok[ns] = bn < N;
    brow[ns] = bok[ns] ? (uint32_t)bn * (uint32_t)nkb : 0u;
  }

  f32x4_t acc[NMAT][NSUB][4];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int ns = 0; ns < NSUB; ++ns)
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[m][ns][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // register ring: block kb lives in set kb % kDepth
  uint4 ra_hi[kDepth], ra_lo[kDepth];
  float ra_sum[kDepth];
  uint2 rb[kDepth][NMAT][NSUB];
  uint32_t rd[kDepth][NMAT][NSUB];

  auto issue = [&](int set, int kb) __attribute__((always_inline)) {
    if (kb < nkb) {
      if (arow_ok) {
        ra_hi[set] = *reinterpret_cast<const uint4*>(pah + (int64_t)kb * KB);
        ra_lo[set] = *reinterpret_cast<const uint4*>(pal + (int64_t)kb * KB);
        ra_sum[set] = aq == 0 ? psum[kb] : 0.f;
      } else {
        ra_hi[set] = ra_lo[set] = make_uint4(0, 0, 0, 0);
        ra_sum[set] = 0.f;
      }
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int ns = 0; ns < NSUB; ++ns) {
          if (bok[ns]) {
            const uint32_t blk = brow[ns] + (uint32_t)kb;
            rb[set][m][ns] = *reinterpret_cast<const uint2*>(nibm[m] + blk * 16u);
            rd[set][m][ns] = sclm[m][blk];
          } else {
            rb[set][m][ns] = make_uint2(0, 0);
            rd[set][m][ns] = 0;
          }
        }
    }
  };

#pragma unroll
  for (int j = 0; j < kDepth; ++j) issue(j, j);

  for (int kb0 = 0; kb0 < nkb; kb0 += kDepth) {
#pragma unroll
    for (int j = 0; j < kDepth; ++j) {
      const int kb = kb0 + j;
      if (kb >= nkb) break;
      const int stage = kb & 1;
      *reinterpret_cast<uint4*>(&sA[stage][0][ar][aq * 8]) = ra_hi[j];
      *reinterpret_cast<uint4*>(&sA[stage][1][ar][aq * 8]) = ra_lo[j];
      if (aq == 0) sC[stage][ar] = ra_sum[j];
      bf16x8_t bop[NMAT][NSUB];
      float dsc[NMAT][NSUB];
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int ns = 0; ns < NSUB; ++ns) {
          bop[m][ns] = weight_operand(rb[j][m][ns].x, rb[j][m][ns].y, shift);
          dsc[m][ns] = half_bits_to_float(rd[j][m][ns]);
        }
      issue(j, kb + kDepth);  // refill this set while the block computes
      __syncthreads();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int r = s * 16 + (lane & 15);
        const bf16x8_t ahi = *reinterpret_cast<const bf16x8_t*>(&sA[stage][0][r][kq * 8]);
        const bf16x8_t alo = *reinterpret_cast<const bf16x8_t*>(&sA[stage][1][r][kq * 8]);
        const f32x4_t cinit = *reinterpret_cast<const f32x4_t*>(&sC[stage][s * 16 + kq * 4]);
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int ns = 0; ns < NSUB; ++ns) {
            f32x4_t t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bop[m][ns], cinit, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bop[m][ns], t, 0, 0, 0);
            acc[m][ns][s] += dsc[m][ns] * t;
          }
      }
    }
  }

  // epilogue: lane holds rows s*16 + kq*4 + i of feature n0 + wave*WN + ns*16 + lane%16
  if (MODE == 0) {
    float bs[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = s * 16 + kq * 4 + i;
        const int64_t pos = pos0 + r;
        float part = 0.f;
#pragma unroll
        for (int ns = 0; ns < NSUB; ++ns) {
          const int bn = n0 + wave * WN + ns * 16 + (lane & 15);
          const float h = silu(acc[0][ns][s][i]) * acc[1][ns][s][i];
          const uint16_t hh = bf16_bits_rne(h);
          const uint16_t hl = bf16_bits_rne(h - bf16_to_float(hh));
          if (r < rows && bok[ns]) {
            const int64_t o = pos * N + (bn & ~31) + plane_pos(bn & 31);
            a.hh[o] = hh;
            a.hl[o] = hl;
            part += bf16_to_float(hh) + bf16_to_float(hl);
          }
        }
        bs[s][i] = row16_sum(part);  // every feature of this wave's 32-block
      }
    // the wave's 32 features form h block (n0 + wave*WN) / 32 of each row
    const int blk = (n0 + wave * WN) >> 5;
    const int nkb_out = N >> 5;
    if ((lane & 15) == 0 && n0 + wave * WN < N) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = s * 16 + kq * 4 + i;
          if (r < rows) a.hsum[(int64_t)(pos0 + r) * nkb_out + blk] = -136.0f * bs[s][i];
        }
    }
  } else {
#pragma unroll
    for (int ns = 0; ns < NSUB; ++ns) {
      const int bn = n0 + wave * WN + ns * 16 + (lane & 15);
      if (!bok[ns]) continue;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = s * 16 + kq * 4 + i;
          if (r < rows) a.y[(int64_t)(pos0 + r) * N + bn] = acc[0][ns][s][i];
        }
    }
  }
}

__global__ __launch_bounds__(256) void combine_pairs_kernel(const float* ypair, const int32_t* inv, const float* w,
                                                            int32_t k, int32_t H, float* y, int32_t accumulate) {
  const int t = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= H) return;
  float acc = 0.f;
  for (int i = 0; i < k; ++i) {
    const int64_t p = (int64_t)t * k + i;
    acc = fmaf(w[p], ypair[(int64_t)inv[p] * H + j], acc);
  }
  float* yp = y + (int64_t)t * H + j;
  *yp = accumulate ? *yp + acc : acc;
}

// ---------------------------------------------------------------------------

hipError_t launch_expert_histogram(const int32_t* ids, int32_t n_pairs, int32_t E, int32_t* counts,
                                   hipStream_t s) {
  hipLaunchKernelGGL(expert_histogram_kernel, dim3((n_pairs + 255) / 256), dim3(256), 0, s, ids, n_pairs, E, counts);
  return hipGetLastError();
}
hipError_t launch_expert_scatter(const int32_t* ids, int32_t n_pairs, int32_t E, const int32_t* offsets,
                                 int32_t* perm, int32_t* inv, hipStream_t s) {
  hipLaunchKernelGGL(expert_scatter_kernel, dim3(E), dim3(256), 0, s, ids, n_pairs, offsets, perm, inv);
  return hipGetLastError();
}
hipError_t launch_split_rows(const float* src, int64_t rows, int32_t K, uint16_t* hi, uint16_t* lo, float* bsum,
                             hipStream_t s) {
  if (K % 32) return hipErrorInvalidValue;
  const int64_t nb = rows * (K / 32);
  hipLaunchKernelGGL(split_rows_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, src, nb, K, hi, lo, bsum);
  return hipGetLastError();
}
hipError_t launch_grouped_gemm(GemmArgs a, int mode, int n_tiles, const Launch& l) {
  if (a.K % 32 || a.N % 32 || n_tiles <= 0) return hipErrorInvalidValue;
  const int bnw = mode == 0 ? 128 : 256;
  a.work = n_tiles * ((a.N + bnw - 1) / bnw);
  a.work_padded = (a.work + 7) / 8 * 8;
  if (mode == 0) return launch(grouped_gemm_kernel<0>, dim3(a.work_padded), dim3(256), l, a);
  return launch(grouped_gemm_kernel<1>, dim3(a.work_padded), dim3(256), l, a);
}
hipError_t launch_combine_pairs(const float* ypair, const int32_t* inv, const float* w, int32_t T, int32_t k,
                                int32_t H, float* y, int32_t accumulate, hipStream_t s) {
  hipLaunchKernelGGL(combine_pairs_kernel, dim3((H + 255) / 256, T), dim3(256), 0, s, ypair, inv, w, k, H, y,
                     accumulate);
  return hipGetLastError();
}

}  // namespace moe
