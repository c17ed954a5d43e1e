// route_dev.h - device helpers of top-k routing shared by the routing
// kernel and the fused routing + gate/up GEMV (internal to the library).
//
// Each round of the top-k is a wave-wide max of order-preserving logit bits
// (DPP butterflies inside 16-lane rows, four lane reads across rows); the
// lowest expert id holding the max comes from ballots.
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

// order-preserving bits of a logit: a larger logit gives a larger value, -0
// counts as +0; 0 stands for "no expert" (past E, or picked already)
__device__ __forceinline__ uint32_t order_bits(float v) {
  // v + 0 is +0 for -0 (round to nearest) and v for every other number, so
  // -0 and +0 get the same bits
  const uint32_t u = __float_as_uint(v + 0.0f);
  // negative: every bit flipped; otherwise the sign bit set
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float order_logit(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// all 64 lanes must be active
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp32<kDppQuadXor1>(v));
  v = max(v, dpp32<kDppQuadXor2>(v));
  v = max(v, dpp32<kDppRowHalfMirror>(v));
  v = max(v, dpp32<kDppRowMirror>(v));  // every lane of a 16-lane row holds the row max
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Top-k of one token by one wave (all 64 lanes active), one pick per round:
// the largest remaining logit, and among equal ones the lowest expert id.
// Lane l holds the order bits of experts l + 64 j. A round is a 32-bit
// wave max; the lowest id holding it comes from the ballots of the equal
// entries (expert 64 j + lane: the first slot j with a match, then its
// lowest lane), so no 64-bit (value, id) key is reduced.
template <int NJ>
struct WaveTopK {
  uint32_t v[NJ];
  __device__ __forceinline__ void init(const float (&z)[NJ], int E, int lane) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) v[j] = lane + 64 * j < E ? order_bits(z[j]) : 0u;
  }
  __device__ __forceinline__ void init_bits(const uint32_t (&bits)[NJ]) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) v[j] = bits[j];
  }
  // the next pick's expert (wave-uniform; always an expert of the layer, so
  // every address stays in bounds) and its order bits
  __device__ __forceinline__ int next(int E, int lane, uint32_t& bits) {
    uint32_t m = v[0];
#pragma unroll
    for (int j = 1; j < NJ; ++j) m = max(m, v[j]);
    m = wave_max_u32(m);
    int e = 0;
    if (m != 0) {
#pragma unroll
      for (int j = NJ - 1; j >= 0; --j) {
        const uint64_t b = __ballot(v[j] == m);
        if (b) e = 64 * j + (int)__builtin_ctzll(b);
      }
    }
    e = e < E ? e : 0;
    const bool mine = lane == (e & 63);
#pragma unroll
    for (int j = 0; j < NJ; ++j) v[j] = (mine && j == (e >> 6)) ? 0u : v[j];
    bits = m;
    return e;
  }
};

// The first `rounds` picks: lane i < rounds ends with pick i's expert and
// order bits; picks are in descending logit order, equal logits lower id first.
template <int NJ>
__device__ __forceinline__ void wave_topk_rounds(WaveTopK<NJ>& tk, int E, int rounds, int lane, int& my_e,
                                                 uint32_t& my_bits) {
  my_e = 0;
  my_bits = 0;
  for (int i = 0; i < rounds; ++i) {
    uint32_t bits;
    const int e = tk.next(E, lane, bits);
    if (lane == i) my_e = e, my_bits = bits;
  }
}
template <int NJ>
__device__ __forceinline__ void wave_topk(const float (&z)[NJ], int E, int rounds, int lane, int& my_e,
                                          uint32_t& my_bits) {
  WaveTopK<NJ> tk;
  tk.init(z, E, lane);
  wave_topk_rounds(tk, E, rounds, lane, my_e, my_bits);
}

// ---------------------------------------------------------------------------
// Top-8 by sorting networks (k <= 8, E <= 512), for the latency-bound decode
// path: the rounds above are a chain of dependent steps each, this is a few
// dozen steps with eight independent operations apiece. Lane l sorts its 8
// order bits (Batcher's odd-even merge sort, 19 compare-exchanges), then six
// butterfly steps each merge a lane's list with a partner's from the other
// half of a group twice the size (lane ^ 1, ^ 2, the mirror within 8 and
// within 16 lanes, ^ 16, ^ 32; the last two by half-swap instructions): the elementwise max of one sorted list and
// the other reversed holds the 8 largest of both as a bitonic sequence,
// which three half-cleaner stages sort. Every lane ends with the 8 largest
// order bits of the wave, descending, ties repeated.

__device__ __forceinline__ void cas_desc(uint32_t& a, uint32_t& b) {
  const uint32_t hi = max(a, b), lo = min(a, b);
  a = hi, b = lo;
}
__device__ __forceinline__ void sort8_desc(uint32_t (&a)[8]) {
  cas_desc(a[0], a[1]), cas_desc(a[2], a[3]), cas_desc(a[4], a[5]), cas_desc(a[6], a[7]);
  cas_desc(a[0], a[2]), cas_desc(a[1], a[3]), cas_desc(a[4], a[6]), cas_desc(a[5], a[7]);
  cas_desc(a[1], a[2]), cas_desc(a[5], a[6]);
  cas_desc(a[0], a[4]), cas_desc(a[1], a[5]), cas_desc(a[2], a[6]), cas_desc(a[3], a[7]);
  cas_desc(a[2], a[4]), cas_desc(a[3], a[5]);
  cas_desc(a[1], a[2]), cas_desc(a[3], a[4]), cas_desc(a[5], a[6]);
}
__device__ __forceinline__ void clean8_desc(uint32_t (&c)[8]) {
  cas_desc(c[0], c[4]), cas_desc(c[1], c[5]), cas_desc(c[2], c[6]), cas_desc(c[3], c[7]);
  cas_desc(c[0], c[2]), cas_desc(c[1], c[3]), cas_desc(c[4], c[6]), cas_desc(c[5], c[7]);
  cas_desc(c[0], c[1]), cas_desc(c[2], c[3]), cas_desc(c[4], c[5]), cas_desc(c[6], c[7]);
}
// the partner value through a DPP move whose lanes all read (full row and
// bank masks), with 0 (the identity of unsigned max) as the "old" operand, so
// the compiler can fold the move into the max as its DPP source
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32_max_src(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ void merge8_dpp(uint32_t (&t)[8]) {
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = max(t[i], dpp32_max_src<CTRL>(t[7 - i]));
  clean8_desc(c);
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = c[i];
}
// partner lane ^ 16 or ^ 32 through one half-swap instruction
// (v_permlane16_swap / v_permlane32_swap: swap the odd 16-lane rows of the
// first operand with the even rows of the second, or the upper 32 lanes of
// the first with the lower 32 of the second). With both operands x the first
// result holds the even rows (lower half) twice and the second the odd rows
// (upper half) twice, so a lane in an even row (lower half) takes its
// partner's value from the second result, the others from the first.
template <int MASK>
__device__ __forceinline__ void merge8_swap(uint32_t (&t)[8]) {
  static_assert(MASK == 16 || MASK == 32, "half-swap partners");
  const bool upper = (__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) & MASK) != 0;
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const auto s = MASK == 32 ? __builtin_amdgcn_permlane32_swap(t[7 - i], t[7 - i], false, false)
                              : __builtin_amdgcn_permlane16_swap(t[7 - i], t[7 - i], false, false);
    c[i] = max(t[i], (uint32_t)(upper ? s[0] : s[1]));
  }
  clean8_desc(c);
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = c[i];
}
// all 64 lanes must be active; v[j]: order bits of expert lane + 64 j
__device__ __forceinline__ void wave_top8(const uint32_t (&v)[8], uint32_t (&t)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) t[j] = v[j];
  sort8_desc(t);
  merge8_dpp<kDppQuadXor1>(t);
  merge8_dpp<kDppQuadXor2>(t);
  merge8_dpp<kDppRowHalfMirror>(t);
  merge8_dpp<kDppRowMirror>(t);
  merge8_swap<16>(t);
  merge8_swap<32>(t);
}
// The expert of pick `rank` (wave-uniform, < 8) and its order bits, from the
// lane's order bits v and their wave_top8 t. With m = t[rank] and r the
// number of earlier picks of the same value, the pick is the r-th lowest
// expert id holding m (ids 64 j + lane: slots j in order, then lanes).
__device__ __forceinline__ int top8_expert(const uint32_t (&v)[8], const uint32_t (&t)[8], int rank, int E,
                                           uint32_t& bits) {
  uint32_t mv = t[0];
  int rv = 0;
#pragma unroll
  for (int i = 1; i < 8; ++i) mv = rank == i ? t[i] : mv;
#pragma unroll
  for (int i = 0; i < 7; ++i) rv += (i < rank && t[i] == mv) ? 1 : 0;
  const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)mv);
  int r = __builtin_amdgcn_readfirstlane(rv);
  int e = 0;
  if (m != 0 && r == 0) {
    // no equal value ranks ahead of this pick (the usual case): the lowest id
    // holding m, slots from the highest down so the lowest nonempty slot
    // decides last (no branches)
#pragma unroll
    for (int j = 7; j >= 0; --j) {
      const uint64_t b = __ballot(v[j] == m);
      e = b ? 64 * j + (int)__builtin_ctzll(b) : e;
    }
  } else if (m != 0) {
    bool found = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint64_t b = __ballot(v[j] == m);
      const int c = __builtin_popcountll(b);
      if (!found) {
        if (r < c) {
          for (int q = 0; q < r; ++q) b &= b - 1;
          e = 64 * j + (int)__builtin_ctzll(b);
          found = true;
        } else {
          r -= c;
        }
      }
    }
  }
  bits = m;
  return e < E ? e : 0;  // always an expert of the layer, so every address stays in bounds
}

// softmax over the k chosen logits (lane i < k holds pick i's order bits;
// pick 0 holds the largest): the weight of this lane's pick, 0 on lanes >= k
__device__ __forceinline__ float wave_pick_weight(uint32_t my_bits, int k, int lane) {
  const float my_z = order_logit(my_bits);
  const float z0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_z), 0));
  const float ex = lane < k ? expf(my_z - z0) : 0.f;
  return ex / wave_sum(ex);
}

}  // namespace route_dev
}  // namespace moe
