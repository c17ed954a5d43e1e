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

// rows of fp32 [R][K] -> bf16 hi and lo planes [R][K] in operand order
__global__ __launch_bounds__(256) void split_rows_kernel(const float* src, int64_t n, int32_t K, uint16_t* hi,
                                                         uint16_t* lo) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float v = src[i];
  const uint16_t h = bf16_bits_rne(v);
  const uint16_t l = bf16_bits_rne(v - bf16_to_float(h));
  const int64_t row = i / K;
  const int k = (int)(i - row * K);
  const int64_t o = row * K + (k & ~31) + plane_pos(k & 31);
  hi[o] = h;
  lo[o] = l;
}

// MODE 0: gate/up (two weight matrices, SwiGLU, writes h planes)
// MODE 1: down (one matrix, writes y_pair)
template <int MODE>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmArgs a) {
  constexpr int NMAT = MODE == 0 ? 2 : 1;
  __shared__ uint16_t sA[2][2][BM][LDS_ROW];  // [stage][hi/lo][row][k]
  __shared__ float sC[2][BM];                 // -136 * sum_k x_k per row and stage

  const int4 tile = a.tiles[blockIdx.y];
  const int e = tile.x, pos0 = tile.y, rows = tile.z;
  const int n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, N = a.N, nkb = K / KB;
  const uint8_t* base = a.eaddr[e];

  // A staging: thread -> (row ar, eighth-of-block aq): 8 elements of each plane
  const int ar = tid >> 2, aq = tid & 3;
  const bool arow_ok = ar < rows;
  const uint16_t* pah = a.ah;
  const uint16_t* pal = a.al;
  if (arow_ok) {
    const int64_t src_row = a.arow ? (int64_t)(a.arow[pos0 + ar] / a.arow_div) : (int64_t)(pos0 + ar);
    pah += src_row * K + aq * 8;
    pal += src_row * K + aq * 8;
  }

  // B: lane -> (feature bn = lane % 16 of the wave's 16, k-quarter kq = lane / 16)
  const int bn = n0 + wave * 16 + (lane & 15);
  const int kq = lane >> 4;
  const bool bn_ok = bn < N;
  const int shift = (kq >> 1) * 4;
  const int64_t brow = bn_ok ? (int64_t)bn * nkb : 0;
  const uint8_t* nib0 = base + (MODE == 0 ? a.lay.gate_nib : a.lay.down_nib) + brow * 16 + (kq & 1) * 8;
  const uint16_t* scl0 = reinterpret_cast<const uint16_t*>(base + (MODE == 0 ? a.lay.gate_scl : a.lay.down_scl)) + brow;
  const uint8_t* nib1 = base + a.lay.up_nib + brow * 16 + (kq & 1) * 8;
  const uint16_t* scl1 = reinterpret_cast<const uint16_t*>(base + a.lay.up_scl) + brow;

  f32x4_t acc0[4], acc1[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) acc0[s] = acc1[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 ra_hi = make_uint4(0, 0, 0, 0), ra_lo = make_uint4(0, 0, 0, 0);
  uint2 rb0 = make_uint2(0, 0), rb1 = make_uint2(0, 0);
  uint32_t rd0 = 0, rd1 = 0;

#define MOE_LOAD_A(KBI)                                                                  \
  if (arow_ok) {                                                                         \
    ra_hi = *reinterpret_cast<const uint4*>(pah + (int64_t)(KBI) * KB);                  \
    ra_lo = *reinterpret_cast<const uint4*>(pal + (int64_t)(KBI) * KB);                  \
  }
#define MOE_LOAD_B(KBI)                                                                  \
  if (bn_ok) {                                                                           \
    rb0 = *reinterpret_cast<const uint2*>(nib0 + (int64_t)(KBI) * 16);                   \
    rd0 = scl0[KBI];                                                                     \
    if (NMAT == 2) {                                                                     \
      rb1 = *reinterpret_cast<const uint2*>(nib1 + (int64_t)(KBI) * 16);                 \
      rd1 = scl1[KBI];                                                                   \
    }                                                                                    \
  }

  MOE_LOAD_A(0)
  MOE_LOAD_B(0)
  for (int kb = 0; kb < nkb; ++kb) {
    const int stage = kb & 1;
    {
      // stage this block's A rows and their sums
      *reinterpret_cast<uint4*>(&sA[stage][0][ar][aq * 8]) = ra_hi;
      *reinterpret_cast<uint4*>(&sA[stage][1][ar][aq * 8]) = ra_lo;
      const uint32_t h[4] = {ra_hi.x, ra_hi.y, ra_hi.z, ra_hi.w};
      const uint32_t l[4] = {ra_lo.x, ra_lo.y, ra_lo.z, ra_lo.w};
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sum += __uint_as_float(h[i] << 16) + __uint_as_float(h[i] & 0xFFFF0000u);
        sum += __uint_as_float(l[i] << 16) + __uint_as_float(l[i] & 0xFFFF0000u);
      }
      sum += __shfl_xor(sum, 1, 64);
      sum += __shfl_xor(sum, 2, 64);
      if (aq == 0) sC[stage][ar] = -136.0f * sum;
    }
    const bf16x8_t b0 = weight_operand(rb0.x, rb0.y, shift);
    const float d0 = half_bits_to_float(rd0);
    bf16x8_t b1 = b0;
    float d1 = 0.f;
    if (NMAT == 2) {
      b1 = weight_operand(rb1.x, rb1.y, shift);
      d1 = half_bits_to_float(rd1);
    }
    __syncthreads();
    if (kb + 1 < nkb) {  // prefetch the next block while this one computes
      MOE_LOAD_A(kb + 1)
      MOE_LOAD_B(kb + 1)
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = s * 16 + (lane & 15);
      const bf16x8_t ahi = *reinterpret_cast<const bf16x8_t*>(&sA[stage][0][r][kq * 8]);
      const bf16x8_t alo = *reinterpret_cast<const bf16x8_t*>(&sA[stage][1][r][kq * 8]);
      const int rc = s * 16 + kq * 4;  // accumulator rows of this lane
      const f32x4_t cinit = {sC[stage][rc + 0], sC[stage][rc + 1], sC[stage][rc + 2], sC[stage][rc + 3]};
      f32x4_t t0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b0, cinit, 0, 0, 0);
      t0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, b0, t0, 0, 0, 0);
      acc0[s] += d0 * t0;
      if (NMAT == 2) {
        f32x4_t t1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b1, cinit, 0, 0, 0);
        t1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, b1, t1, 0, 0, 0);
        acc1[s] += d1 * t1;
      }
    }
  }
#undef MOE_LOAD_A
#undef MOE_LOAD_B

  // epilogue: lane holds rows s*16 + kq*4 + i of feature bn
  if (!bn_ok) return;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = s * 16 + kq * 4 + i;
      if (r >= rows) continue;
      const int64_t pos = pos0 + r;
      if (MODE == 0) {
        const float h = silu(acc0[s][i]) * acc1[s][i];
        const uint16_t hh = bf16_bits_rne(h);
        const uint16_t hl = bf16_bits_rne(h - bf16_to_float(hh));
        const int64_t o = pos * N + (bn & ~31) + plane_pos(bn & 31);
        a.hh[o] = hh;
        a.hl[o] = hl;
      } else {
        a.y[pos * N + bn] = acc0[s][i];
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
hipError_t launch_split_rows(const float* src, int64_t rows, int32_t K, uint16_t* hi, uint16_t* lo, hipStream_t s) {
  const int64_t n = rows * K;
  hipLaunchKernelGGL(split_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, n, K, hi, lo);
  return hipGetLastError();
}
hipError_t launch_grouped_gemm(const GemmArgs& a, int mode, int n_tiles, const Launch& l) {
  if (a.K % 32 || n_tiles <= 0) return hipErrorInvalidValue;
  const dim3 grid((a.N + BN - 1) / BN, n_tiles);
  if (mode == 0) return launch(grouped_gemm_kernel<0>, grid, dim3(256), l, a);
  return launch(grouped_gemm_kernel<1>, grid, dim3(256), l, a);
}
hipError_t launch_combine_pairs(const float* ypair, const int32_t* inv, const float* w, int32_t T, int32_t k,
                                int32_t H, float* y, int32_t accumulate, hipStream_t s) {
  hipLaunchKernelGGL(combine_pairs_kernel, dim3((H + 255) / 256, T), dim3(256), 0, s, ypair, inv, w, k, H, y,
                     accumulate);
  return hipGetLastError();
}

}  // namespace moe
