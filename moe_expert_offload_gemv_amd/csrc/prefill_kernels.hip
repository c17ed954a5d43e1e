// prefill_kernels.hip - gfx950 kernels of the prompt pass of one MoE layer:
// the (token, pick) pairs are sorted by expert and every expert runs as one
// GEMM over its own rows only, the way the "llama.cpp - very large MoE models
// on a 64 GB Mac" README ("Metal kernels": MUL_MAT_ID over used tiles only)
// launches only (expert, tile) pairs that hold tokens.
//
//   chunk_rank_kernel        per chunk of 256 pairs: each pair's rank among the
//                            chunk's earlier pairs of its expert, and the chunk's
//                            count per expert
//   chunk_scan_kernel        per expert: where each chunk's pairs start among the
//                            expert's pairs, and the expert's pair count
//   expert_scatter_kernel    stable counting sort: perm[pos] = pair, inv[pair] = pos
//   scale_rows_kernel        fp32 rows -> fp16 rows in operand order, each row
//                            scaled by a power of two (its exponent kept)
//   grouped_gemm_kernel      per tile of one expert: gate/up -> h = silu(g) * u
//                            (fp16 rows in operand order), or down -> y_pair (fp32)
//   combine_pairs_kernel     y[t] = sum_i w_i y_pair[inv[t, i]] in pick order
//   stage_experts_kernel     the pass's non-resident experts, read zero-copy
//                            from pinned host memory into HBM staging blocks
//
// Range: fp16 holds 6.1e-5 .. 65504 at full precision, while the API takes
// any fp32 activations. Each token's row is therefore scaled by 2^s (exact)
// so that its largest magnitude lies in [4, 8) before the cast; the gate/up
// epilogue undoes 2^s on the accumulators (exact) and stores h scaled by
// 2^(2s), since silu(g) * u grows like the square of the token's scale in
// both of its regimes (silu(g) ~ g for large positive g, ~ g / 2 near 0);
// the down epilogue multiplies by 2^(-2s). A scaled h that is not finite or
// exceeds 65504 sets a flag that fails the pass (weights far larger than the
// blocks' fp16 scales admit in practice).
//
// MFMA form: v_mfma_f32_16x16x32_f16 with fp32 accumulation straight through
// K. The weight operand is built in registers from the quant blocks as
// fp16(d * (q - 8)): each nibble pair becomes 1024 + q by one v_and_or into
// the fp16 mantissa, 1032 is subtracted exactly and the block scale d
// multiplies, so every weight is rounded once. The activations enter as fp16.
// One K step is 64 (two quant blocks); within a step lane group g of the
// wave reads 8 bytes (16 nibbles) of block g/2 and feeds the low nibbles to
// the first MFMA and the high nibbles to the second. The activation rows are
// stored in the matching order (step_pos), so LDS reads are 16-byte vectors.
//
// Block scales: a scale line of the expert blob holds 32 K steps of one
// column, so a K step reading 4 B of it leaves the line to be fetched again
// for each step once other traffic has evicted it, and costs one memory
// request per column. A pass therefore first transposes the scale planes of
// its experts (transpose_scales_kernel) into [K/32][columns]: a K step's
// scales of a column tile are then one contiguous run, every fetched line
// used at once.
//
// Staging: every operand byte of a K step (the A rows, the weight nibbles,
// the block scales) travels global -> LDS by the LDS-DMA form of the global
// load (global_load_lds_dwordx4 / _dword: lane l of a wave writes 16 or 4
// bytes at M0 + 16 l or + 4 l), into a ring of three stages, issued two steps
// ahead of its use; no VGPR holds data in flight. A rows sit in LDS with their
// 16-byte chunks XOR-swizzled by (row & 7), so the 16-row fragment reads are
// free of bank conflicts without padding.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace moe {

namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int KS = 64;             // k per step: two quant blocks
constexpr int LDS_ROW = KS + 8;    // padded fp16 row in LDS: 144 B, rows 4 banks apart

// (0,2,1,3,4,6,5,7): order of eight consecutive weights in an operand (an involution)
__device__ __forceinline__ int ord8(int i) { return (i & 4) | ((i & 1) << 1) | ((i >> 1) & 1); }

// position of element e (0..63) of a K step inside the stored row: operand
// half h = low/high nibble, lane group g = 2 * block + byte half, slot i
__device__ __forceinline__ int step_pos(int e) {
  const int bl = e >> 5, eb = e & 31, h = eb >> 4, r = eb & 15;
  return 32 * h + 8 * (2 * bl + (r >> 3)) + ord8(r & 7);
}

__device__ __forceinline__ f16x2_t as_h2(uint32_t u) {
  f16x2_t v;
  __builtin_memcpy(&v, &u, 4);
  return v;
}

// 16 weights of one column from 8 bytes of a quant block: bytes jb..jb+7
// hold elements jb..jb+7 (low nibbles) and jb+16..jb+23 (high nibbles).
// lo gets jb + (0,2,1,3,4,6,5,7), hi the same + 16; value fp16(d * (q - 8)).
// One 3-input bit operation (v_bitop3, (S0 & S1) | S2) places two nibbles in
// the mantissas of two fp16 halves of exponent 1024: a low nibble gives
// 1024 + q, a high nibble where it stands 1024 + 16 q, so the odd bytes need
// the only shift. 1024 + q - 1032 and (1024 + 16 q) / 16 - 72 are q - 8
// exactly; the multiplication by d rounds once.
__device__ __forceinline__ void weight_operands(u32x2_t w, f16x2_t d2, f16x8_t& lo, f16x8_t& hi) {
  constexpr uint32_t ML = 0x000F000Fu, MH = 0x00F000F0u, MAGIC = 0x64006400u;  // MAGIC: fp16 1024 in both halves
  constexpr int OR_AND = 0xEA;  // truth table of (S0 & S1) | S2
  const f16x2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const f16x2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f}, off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t x8 = w.x >> 8, y8 = w.y >> 8;
  uint32_t p[8];
  p[0] = __builtin_amdgcn_bitop3_b32(w.x, ML, MAGIC, OR_AND);
  p[1] = __builtin_amdgcn_bitop3_b32(x8, ML, MAGIC, OR_AND);
  p[2] = __builtin_amdgcn_bitop3_b32(w.y, ML, MAGIC, OR_AND);
  p[3] = __builtin_amdgcn_bitop3_b32(y8, ML, MAGIC, OR_AND);
  p[4] = __builtin_amdgcn_bitop3_b32(w.x, MH, MAGIC, OR_AND);
  p[5] = __builtin_amdgcn_bitop3_b32(x8, MH, MAGIC, OR_AND);
  p[6] = __builtin_amdgcn_bitop3_b32(w.y, MH, MAGIC, OR_AND);
  p[7] = __builtin_amdgcn_bitop3_b32(y8, MH, MAGIC, OR_AND);
  f16x2_t v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = (as_h2(p[j]) - off) * d2;
#pragma unroll
  for (int j = 4; j < 8; ++j) v[j] = __builtin_elementwise_fma(as_h2(p[j]), sixteenth, off16) * d2;
  __builtin_memcpy(&lo, &v[0], 16);
  __builtin_memcpy(&hi, &v[4], 16);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// LDS-DMA loads: lane l writes its bytes at lds + 16 l (or + 4 l); lds must
// be wave-uniform (it goes to M0)
__device__ __forceinline__ void dma16(const void* src, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)lds, 4, 0, 0);
}

// s_waitcnt immediate (GFX9 encoding) waiting for vmcnt <= n only
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// workgroup barrier over LDS: this wave's LDS reads are complete, then
// s_barrier. The DMA completions are waited for with vmcnt before it; a
// fence here would make the compiler drain every DMA in flight (vmcnt(0)).
// The memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

constexpr int kStages = 3;       // LDS ring: loads run two K steps ahead
constexpr int kSortChunk = 256;  // pairs per chunk of the counting sort

// Shape of a workgroup tile: BM rows x 4 waves x NSUB x 16 features of NMAT
// matrices, and the LDS stage holding one K step of its operands:
//   [A: BM rows x 128 B][nibbles: NMAT x BNW features x 32 B][scales: NMAT x 2 blocks x BNW x 2 B]
// DA, DB, DS: LDS-DMA instructions per wave and step for each part.
template <int BM, int MODE>
struct GemmTile {
  static constexpr int NMAT = MODE == 0 ? 2 : 1;
  static constexpr int RB = BM / 16;
  // at most 128 accumulators per wave; the 64-row gate/up tile takes half
  // that (128 features of each matrix), so that its registers and LDS allow
  // three work-groups per CU: its gate/up GEMM of the 4096-token decode-shape
  // pass took 0.68 ms at 256 features and two per CU, 0.62 ms now
  static constexpr int NSUB = (BM == 64 && MODE == 0) ? 2 : (32 / (RB * NMAT) < 4 ? 32 / (RB * NMAT) : 4);
  static constexpr int WGS_PER_CU = BM == 64 ? 3 : 2;
  static constexpr int WN = 16 * NSUB;
  static constexpr int BNW = 4 * WN;
  static constexpr int A_BYTES = BM * 2 * KS;
  static constexpr int BN_BYTES = BNW * 32;
  static constexpr int BS_BYTES = BNW * 4;
  static constexpr int OFF_BN = A_BYTES;
  static constexpr int OFF_BS = A_BYTES + NMAT * BN_BYTES;
  static constexpr int STAGE = OFF_BS + NMAT * BS_BYTES;
  static constexpr int DA = A_BYTES / 1024 / 4;
  static constexpr int DB = NMAT * BN_BYTES / 1024 / 4;
  static constexpr int DS = NMAT * BS_BYTES / 256 / 4;
  static constexpr int D = DA + DB + DS;
  static_assert(DA * 4096 == A_BYTES && DB * 4096 == NMAT * BN_BYTES && DS * 1024 == NMAT * BS_BYTES,
                "every wave issues whole DMA instructions");
  static_assert(WGS_PER_CU * kStages * STAGE <= 160 * 1024, "the work-groups per CU fit in LDS");
};

}  // namespace

// ---------------------------------------------------------------------------

// Counting sort of the pairs by expert, stable, in three passes over chunks
// of kSortChunk consecutive pairs (no atomics, no pass over all pairs per
// expert). ccount is [E][n_chunks]: counts per chunk, then (in place) where
// each chunk's pairs start among the expert's. Pair ids outside 0..E-1 are
// left out of every count, so the host's total check catches them.
//
// One wave per chunk, 64 pairs per round in order. Within a round, each
// distinct expert in turn (the lowest pending lane's) takes a ballot of its
// lanes: their ranks are the count so far plus the lanes below them, so the
// order of the pairs is kept.
__global__ __launch_bounds__(64) void chunk_rank_kernel(const int32_t* ids, int32_t n_pairs, int32_t E,
                                                        int32_t n_chunks, int32_t* rank, int32_t* ccount) {
  extern __shared__ int32_t s_cnt[];  // [E]
  const int c = blockIdx.x, lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) s_cnt[e] = 0;
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
  for (int r = 0; r < kSortChunk / 64; ++r) {
    const int i = c * kSortChunk + r * 64 + lane;
    int e = i < n_pairs ? ids[i] : -1;
    e = e >= 0 && e < E ? e : -1;
    uint64_t todo = __ballot(e >= 0);
    while (todo) {
      const int leader = (int)__builtin_ctzll(todo);
      const int le = __builtin_amdgcn_readlane(e, leader);
      const uint64_t m = __ballot(e == le);
      const int base = s_cnt[le];
      if (e == le) rank[i] = base + __popcll(m & below);
      __syncthreads();  // every lane has read the count before it moves on
      if (lane == leader) s_cnt[le] = base + __popcll(m);
      __syncthreads();
      todo &= ~m;
    }
  }
  for (int e = lane; e < E; e += 64) ccount[(int64_t)e * n_chunks + c] = s_cnt[e];
}

// one wave per expert: exclusive prefix of its chunk counts, and its total
__global__ __launch_bounds__(64) void chunk_scan_kernel(int32_t* ccount, int32_t n_chunks, int32_t* counts) {
  const int e = blockIdx.x, lane = threadIdx.x;
  int32_t* row = ccount + (int64_t)e * n_chunks;
  int run = 0;
  for (int c0 = 0; c0 < n_chunks; c0 += 64) {
    const int c = c0 + lane;
    const int v = c < n_chunks ? row[c] : 0;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d, 64);
      x += lane >= d ? y : 0;
    }
    if (c < n_chunks) row[c] = run + x - v;
    run += __shfl(x, 63, 64);
  }
  if (lane == 0) counts[e] = run;
}

__global__ __launch_bounds__(256) void expert_scatter_kernel(const int32_t* ids, int32_t n_pairs, int32_t E,
                                                             int32_t n_chunks, const int32_t* offsets,
                                                             const int32_t* cbase, const int32_t* rank,
                                                             int32_t* perm, int32_t* inv) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n_pairs) return;
  const int e = ids[i];
  if (e < 0 || e >= E) return;
  const int pos = offsets[e] + cbase[(int64_t)e * n_chunks + i / kSortChunk] + rank[i];
  perm[pos] = i;
  inv[i] = pos;
}

// Exponent s of a row's scale 2^s: its largest magnitude m times 2^s lies in
// [4, 8) (m = f * 2^e with f in [0.5, 1): s = 3 - e). A zero or non-finite m
// keeps the row as it is.
__device__ __forceinline__ int row_scale_exp(float m) {
  if (!(m > 0.f) || !(m <= 3.4028235e38f)) return 0;
  int e;
  (void)frexpf(m, &e);
  return 3 - e;
}

// fp32 rows [R][K] -> fp16 rows [R][K] in operand order, row r scaled by
// 2^sig[r] (sig[r] written here). One work-group per row: the row's largest
// magnitude first, then each thread converts 8 stored halves at a time,
// which come from 8 consecutive elements (in ord8 order).
__global__ __launch_bounds__(256) void scale_rows_kernel(const float* src, int32_t K, uint4* dst, int32_t* sig) {
  __shared__ float s_max[4];
  const int64_t r = blockIdx.x;
  const float* row = src + r * K;
  const int n_oct = K / 8;
  float m = 0.f;
  for (int o = threadIdx.x; o < n_oct; o += 256) {
    const float4 a = reinterpret_cast<const float4*>(row)[2 * o], b = reinterpret_cast<const float4*>(row)[2 * o + 1];
    m = fmaxf(m, fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                       fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w)))));
    // a NaN compares false everywhere: keep it visible as +inf
    if (a.x != a.x || a.y != a.y || a.z != a.z || a.w != a.w || b.x != b.x || b.y != b.y || b.z != b.z || b.w != b.w)
      m = __builtin_inff();
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
  __syncthreads();
  const int e = row_scale_exp(fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3])));
  if (threadIdx.x == 0) sig[r] = e;
  for (int o = threadIdx.x; o < n_oct; o += 256) {
    const int step = o >> 3;      // K % 64 == 0: steps never straddle rows
    const int oq = o & 7;         // stored positions 8*oq .. 8*oq+7
    const int h = oq >> 2, g = oq & 3;
    const int e0 = 32 * (g >> 1) + 16 * h + 8 * (g & 1);
    const float4* s4 = reinterpret_cast<const float4*>(row + step * KS + e0);
    const float4 a = s4[0], b = s4[1];
    const float v[8] = {a.x, a.z, a.y, a.w, b.x, b.z, b.y, b.w};  // ord8
    uint32_t u[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f16x2_t t = {(_Float16)ldexpf(v[2 * j], e), (_Float16)ldexpf(v[2 * j + 1], e)};
      __builtin_memcpy(&u[j], &t, 4);
    }
    dst[r * n_oct + o] = make_uint4(u[0], u[1], u[2], u[3]);
  }
}

// One workgroup computes a BM-row tile of one expert's pairs against
// 4 waves x NSUB x 16 output features of NMAT weight matrices; every wave
// covers all BM rows, so each weight is converted once per workgroup.
// MODE 0: gate/up (two matrices, SwiGLU epilogue, writes h as fp16 rows in
//         operand order); MODE 1: down (one matrix, writes y_pair).
// NSUB: every wave holds at most 128 accumulators (64 in the 64-row gate/up
// tile, see GemmTile).
// NRB (1..RB): the tile's 16-row blocks that hold rows. Blocks past them are
// left out at compile time (their A rows are still fetched: the DMA count per
// step is the same for every tile), so the product loop of a step is one
// straight run in which the A fragments of the next block are read while the
// current block's MFMAs execute.
template <int BM, int MODE, int NRB>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, uint8_t* smem, int e, int pos0, int rows, int n0) {
  using C = GemmTile<BM, MODE>;
  constexpr int NMAT = C::NMAT, NSUB = C::NSUB, WN = C::WN, BNW = C::BNW;
  static_assert(NRB >= 1 && NRB <= C::RB, "active row blocks");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4;
  const int K = a.K, N = a.N, nks = K / KS, nkb = K / 32;
  const uint8_t* base = a.eaddr[e];

  // DMA sources of this lane at step 0 (step j adds 128 B, 32 B, 4 B).
  // A: instruction i of the wave fills rows 8 (wave DA + i) .. +7; lane l
  // lands in row + l / 8, physical chunk l % 8 = logical chunk ^ (row & 7).
  // Rows past the tile fetch the tile's first row: they only feed
  // accumulator rows that are never stored.
  const uint8_t* asrc[C::DA];
#pragma unroll
  for (int i = 0; i < C::DA; ++i) {
    int r = 8 * (wave * C::DA + i) + (lane >> 3);
    r = r < rows ? r : 0;
    const int64_t src_row = a.arow ? (int64_t)(a.arow[pos0 + r] / a.arow_div) : (int64_t)(pos0 + r);
    asrc[i] = reinterpret_cast<const uint8_t*>(a.a16 + src_row * K) + 16 * ((lane & 7) ^ (lane >> 3));
  }
  // nibbles: instruction q covers features 32 (q % (BNW/32)) .. +31 of matrix
  // q / (BNW/32); lane l fetches block half l / 32 of feature l % 32 (slot l).
  // Features past N fetch feature 0 and are never stored.
  const int64_t nib_plane[2] = {MODE == 1 ? a.lay.down_nib : a.lay.gate_nib, a.lay.up_nib};
  uint32_t bsrc[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) {
    const int q = wave * C::DB + i, m = q / (BNW / 32);
    int col = n0 + 32 * (q % (BNW / 32)) + (lane & 31);
    col = col < N ? col : 0;
    bsrc[i] = (uint32_t)(nib_plane[m] + ((int64_t)col * nkb + (lane >> 5)) * 16);
  }
  // scales, from the pass's transposed planes ([K/32][N] per matrix):
  // instruction q covers features 128 c .. +127 of block b of the step for
  // matrix m, with q = (2 m + b) * (BNW / 128) + c; lane l fetches features
  // 2 l, 2 l + 1; the LDS part is [matrix][block][feature]. Features past N
  // fetch feature 0 and are never stored.
  const uint8_t* sbase = reinterpret_cast<const uint8_t*>(a.sclT + (int64_t)e * a.sclT_per_expert);
  const uint32_t sstep = 4u * (uint32_t)N;  // bytes per K step
  const int64_t sclT_plane[2] = {MODE == 1 ? 2 * (int64_t)a.lay.F * (a.lay.H / 32) : 0,
                                 (int64_t)a.lay.F * (a.lay.H / 32)};
  uint32_t ssrc[C::DS];
#pragma unroll
  for (int i = 0; i < C::DS; ++i) {
    const int q = wave * C::DS + i;
    const int m = q / (2 * (BNW / 128)), bq = (q / (BNW / 128)) % 2;
    int col = n0 + 128 * (q % (BNW / 128)) + 2 * lane;
    col = col < N ? col : 0;
    ssrc[i] = (uint32_t)((sclT_plane[m] + (int64_t)bq * N + col) * 2);
  }

  auto issue = [&](int j) __attribute__((always_inline)) {
    uint8_t* S = smem + (j % kStages) * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::DA; ++i) dma16(asrc[i] + (int64_t)j * (2 * KS), S + (wave * C::DA + i) * 1024);
#pragma unroll
    for (int i = 0; i < C::DB; ++i) dma16(base + bsrc[i] + 32u * (uint32_t)j, S + C::OFF_BN + (wave * C::DB + i) * 1024);
#pragma unroll
    for (int i = 0; i < C::DS; ++i)
      dma4(sbase + ssrc[i] + sstep * (uint32_t)j, S + C::OFF_BS + (wave * C::DS + i) * 256);
  };

  f32x4_t acc[NMAT][NSUB][NRB];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int ns = 0; ns < NSUB; ++ns)
#pragma unroll
      for (int s = 0; s < NRB; ++s) acc[m][ns][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // this lane's A fragment of row block s, half h: row s*16 + lane%16 (row & 7
  // == lane & 7), logical chunk 4h + g
  const int a_off = (lane & 15) * (2 * KS);
  const int a_chunk[2] = {16 * (g ^ (lane & 7)), 16 * ((4 + g) ^ (lane & 7))};

  issue(0);
  if (nks > 1) issue(1);
  for (int j = 0; j < nks; ++j) {
    // this wave's DMAs of step j are done when at most step j+1's are pending
    if (j + 1 < nks)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(C::D));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    lds_barrier();  // every wave's step j landed; step j-1's stage is free
    if (j + 2 < nks) issue(j + 2);
    const uint8_t* S = smem + (j % kStages) * C::STAGE;

    f16x8_t av[2][2];
    av[0][0] = *reinterpret_cast<const f16x8_t*>(S + a_off + a_chunk[0]);
    av[0][1] = *reinterpret_cast<const f16x8_t*>(S + a_off + a_chunk[1]);
    f16x8_t bop[NMAT][NSUB][2];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int ns = 0; ns < NSUB; ++ns) {
        const int wn = wave * WN + ns * 16 + (lane & 15);
        const u32x2_t w = *reinterpret_cast<const u32x2_t*>(S + C::OFF_BN + m * C::BN_BYTES + (wn >> 5) * 1024 +
                                                            ((wn & 31) + 32 * (g >> 1)) * 16 + 8 * (g & 1));
        const uint32_t d = *reinterpret_cast<const uint16_t*>(
            S + C::OFF_BS + m * C::BS_BYTES + (g >> 1) * BNW * 2 + wn * 2);
        weight_operands(w, as_h2(d | (d << 16)), bop[m][ns][0], bop[m][ns][1]);
      }
#pragma unroll
    for (int s = 0; s < NRB; ++s) {
      if (s + 1 < NRB) {  // next block's fragments, read while this block's MFMAs run
        const uint8_t* An = S + (s + 1) * 16 * (2 * KS) + a_off;
        av[(s + 1) & 1][0] = *reinterpret_cast<const f16x8_t*>(An + a_chunk[0]);
        av[(s + 1) & 1][1] = *reinterpret_cast<const f16x8_t*>(An + a_chunk[1]);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int ns = 0; ns < NSUB; ++ns)
            acc[m][ns][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[s & 1][h], bop[m][ns][h], acc[m][ns][s], 0, 0, 0);
    }
  }

  // epilogue: lane holds rows s*16 + g*4 + i of feature n0 + wave*WN + ns*16 + lane%16.
  // Row scale: the token's activations entered as x * 2^sx
  int sx[NRB][4];
#pragma unroll
  for (int s = 0; s < NRB; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = s * 16 + g * 4 + i;
      sx[s][i] = r < rows ? a.sig[a.perm[pos0 + r] / a.perm_div] : 0;
    }
  bool bad = false;
#pragma unroll
  for (int ns = 0; ns < NSUB; ++ns) {
    const int bn = n0 + wave * WN + ns * 16 + (lane & 15);
    if (bn >= N) continue;
    if (MODE == 0) {
      const int64_t col = (bn & ~(KS - 1)) + step_pos(bn & (KS - 1));
#pragma unroll
      for (int s = 0; s < NRB; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = s * 16 + g * 4 + i;
          if (r < rows) {
            // g and u at the token's own scale, h stored at 2^(2 sx)
            const float gv = ldexpf(acc[0][ns][s][i], -sx[s][i]), uv = ldexpf(acc[NMAT - 1][ns][s][i], -sx[s][i]);
            const float hv = ldexpf(silu(gv) * uv, 2 * sx[s][i]);
            bad |= !(fabsf(hv) <= 65504.f);
            a.h16[(int64_t)(pos0 + r) * N + col] = (_Float16)hv;
          }
        }
    } else {
#pragma unroll
      for (int s = 0; s < NRB; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = s * 16 + g * 4 + i;
          if (r < rows) a.y[(int64_t)(pos0 + r) * N + bn] = ldexpf(acc[0][ns][s][i], -2 * sx[s][i]);
        }
    }
  }
  if (MODE == 0 && __ballot(bad) != 0 && lane == 0) atomicOr(a.range_flag, 1u);
}

// the tile body for the tile's count of active 16-row blocks, nrb in 1..N
template <int BM, int MODE, int N>
__device__ __forceinline__ void gemm_tile_rows(int nrb, const GemmArgs& a, uint8_t* smem, int e, int pos0, int rows,
                                               int n0) {
  if constexpr (N > 1) {
    if (nrb < N) {
      gemm_tile_rows<BM, MODE, N - 1>(nrb, a, smem, e, pos0, rows, n0);
      return;
    }
  }
  gemm_tile<BM, MODE, N>(a, smem, e, pos0, rows, n0);
}

// Work items (row tile, first feature) come from a list the host orders per
// expert by feature tile, then row tile: the row tiles that read the same
// weight columns are neighbours, start together and keep in step, so each
// weight line is fetched from HBM once. Each XCD (work group id mod 8 of the
// launch order) gets a contiguous range of the list, so neighbours share an L2.
template <int BM, int MODE>
__global__ __launch_bounds__(256, (GemmTile<BM, MODE>::WGS_PER_CU)) void grouped_gemm_kernel(GemmArgs a) {
  using C = GemmTile<BM, MODE>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * C::STAGE];
  // XCD-contiguous work numbering over the host's work list
  const int L = blockIdx.x;
  const int per = a.work_padded / 8;
  const int W = (L & 7) * per + (L >> 3);
  if (W >= a.work) return;
  const int2 item = a.items[W];
  const int4 tile = a.tiles[item.x];
  const int rows = tile.z;
  gemm_tile_rows<BM, MODE, C::RB>((rows + 15) / 16, a, smem, tile.x, tile.y, rows, item.y);
}

// Scale planes [rows][K/32] (fp16) of the experts with eaddr[e] set ->
// [K/32][rows] at out + e * per. A work-group moves 64 rows, 128 blocks of K
// at a time: it reads them (one contiguous run per row), writes them
// transposed into LDS, then writes 128-byte pieces of the transposed plane.
// When the rows are whole multiples of 16 bytes (K a multiple of 256) both
// global sides move 16 bytes per lane; otherwise 2. grid = (row chunks of the
// largest matrix, 3 matrices, E).
__global__ __launch_bounds__(256) void transpose_scales_kernel(const uint8_t* const* eaddr, const int32_t* experts,
                                                               ExpertLayout lay, uint16_t* out, int64_t per) {
  constexpr int TS = 64 + 8;  // LDS row of the transposed tile (u16): 144 bytes, 16-byte aligned
  __shared__ __attribute__((aligned(16))) uint16_t tile[128 * TS];  // [block][row]
  const int e = experts[blockIdx.z];
  const uint8_t* base = eaddr[e];
  if (!base) return;
  const int m = blockIdx.y;  // 0 gate, 1 up, 2 down
  const int R = m < 2 ? lay.F : lay.H, KB = (m < 2 ? lay.H : lay.F) / 32;
  const int r0 = blockIdx.x * 64;
  if (r0 >= R) return;
  const int nr = R - r0 < 64 ? R - r0 : 64;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(base + (m == 0 ? lay.gate_scl : m == 1 ? lay.up_scl
                                                                                            : lay.down_scl)) +
                        (int64_t)r0 * KB;
  uint16_t* dst = out + (int64_t)e * per + (int64_t)m * lay.F * (lay.H / 32) + r0;
  const bool vec = KB % 8 == 0 && nr == 64 && ((uintptr_t)src & 15) == 0 && ((uintptr_t)dst & 15) == 0 && R % 8 == 0;
  for (int k0 = 0; k0 < KB; k0 += 128) {
    const int nk = KB - k0 < 128 ? KB - k0 : 128;
    if (vec) {
      const int cpr = nk / 8;  // 16-byte pieces per row
      for (int c = threadIdx.x; c < 64 * cpr; c += 256) {
        const int r = c / cpr, kb = 8 * (c - r * cpr);
        const uint4 v = *reinterpret_cast<const uint4*>(src + (int64_t)r * KB + k0 + kb);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          tile[(kb + 2 * i) * TS + r] = (uint16_t)(w[i] & 0xffffu);
          tile[(kb + 2 * i + 1) * TS + r] = (uint16_t)(w[i] >> 16);
        }
      }
      __syncthreads();
      for (int c = threadIdx.x; c < nk * 8; c += 256) {
        const int kb = c >> 3, rc = c & 7;
        *reinterpret_cast<uint4*>(dst + (int64_t)(k0 + kb) * R + 8 * rc) =
            *reinterpret_cast<const uint4*>(tile + kb * TS + 8 * rc);
      }
    } else {
      for (int i = threadIdx.x; i < nr * nk; i += 256) {
        const int r = i / nk, kb = i - r * nk;
        tile[kb * TS + r] = src[(int64_t)r * KB + k0 + kb];
      }
      __syncthreads();
      for (int i = threadIdx.x; i < nk * 64; i += 256) {
        const int kb = i >> 6, r = i & 63;
        if (r < nr) dst[(int64_t)(k0 + kb) * R + r] = tile[kb * TS + r];
      }
    }
    __syncthreads();
  }
}

// Staging of the pass's non-resident experts: expert experts[i] of a layer's
// pinned weights (read zero-copy over PCIe) goes to staging block i. One
// launch for all of them, four 16-byte reads in flight per thread; this runs
// at the PCIe ceiling (57.5 GB/s measured with 128 work-groups for 256
// experts of 3.5 MB), where one DMA copy per expert reached 49 GB/s, the gaps
// between copies costing 2.6 ms of a 16 ms transfer.
__global__ __launch_bounds__(256) void stage_experts_kernel(const uint4* __restrict__ host,
                                                            const int32_t* __restrict__ experts, int64_t n16,
                                                            int64_t b16, uint4* __restrict__ staging) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = i + u * stride, blk = j / b16;
      v[u] = host[(int64_t)experts[blk] * b16 + (j - blk * b16)];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) staging[i + u * stride] = v[u];
  }
  for (; i < n16; i += stride) {
    const int64_t blk = i / b16;
    staging[i] = host[(int64_t)experts[blk] * b16 + (i - blk * b16)];
  }
}

// y[t] = sum_i w_i y_pair[inv[t, i]] in pick order (one fmaf chain from 0),
// four columns per thread. Up to KMAX picks, every row's load is issued
// before the sum, so a thread has all of them in flight at once.
template <int KMAX>
__global__ __launch_bounds__(256) void combine_pairs_kernel(const float* ypair, const int32_t* inv, const float* w,
                                                            int32_t k, int32_t H, float* y, int32_t accumulate) {
  const int t = blockIdx.y;
  const int j = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (j >= H) return;
  const int64_t p0 = (int64_t)t * k;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (k <= KMAX) {
    float4 v[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
      if (i < k) v[i] = *reinterpret_cast<const float4*>(ypair + (int64_t)inv[p0 + i] * H + j);
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
      if (i < k) {
        const float wi = w[p0 + i];
        acc.x = fmaf(wi, v[i].x, acc.x), acc.y = fmaf(wi, v[i].y, acc.y);
        acc.z = fmaf(wi, v[i].z, acc.z), acc.w = fmaf(wi, v[i].w, acc.w);
      }
  } else {
    for (int i = 0; i < k; ++i) {
      const float wi = w[p0 + i];
      const float4 v = *reinterpret_cast<const float4*>(ypair + (int64_t)inv[p0 + i] * H + j);
      acc.x = fmaf(wi, v.x, acc.x), acc.y = fmaf(wi, v.y, acc.y);
      acc.z = fmaf(wi, v.z, acc.z), acc.w = fmaf(wi, v.w, acc.w);
    }
  }
  float4* yp = reinterpret_cast<float4*>(y + (int64_t)t * H + j);
  if (accumulate) {
    const float4 o = *yp;
    acc.x += o.x, acc.y += o.y, acc.z += o.z, acc.w += o.w;
  }
  *yp = acc;
}

// ---------------------------------------------------------------------------

int32_t sort_chunks(int32_t n_pairs) { return (n_pairs + kSortChunk - 1) / kSortChunk; }
hipError_t launch_expert_counts(const int32_t* ids, int32_t n_pairs, int32_t E, int32_t* rank, int32_t* ccount,
                                int32_t* counts, hipStream_t s) {
  if (n_pairs <= 0 || E <= 0 || E > 4096) return hipErrorInvalidValue;
  const int32_t nc = sort_chunks(n_pairs);
  hipLaunchKernelGGL(chunk_rank_kernel, dim3(nc), dim3(64), sizeof(int32_t) * E, s, ids, n_pairs, E, nc, rank,
                     ccount);
  hipLaunchKernelGGL(chunk_scan_kernel, dim3(E), dim3(64), 0, s, ccount, nc, counts);
  return hipGetLastError();
}
hipError_t launch_expert_scatter(const int32_t* ids, int32_t n_pairs, int32_t E, const int32_t* offsets,
                                 const int32_t* ccount, const int32_t* rank, int32_t* perm, int32_t* inv,
                                 hipStream_t s) {
  if (n_pairs <= 0 || E <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(expert_scatter_kernel, dim3((n_pairs + 255) / 256), dim3(256), 0, s, ids, n_pairs, E,
                     sort_chunks(n_pairs), offsets, ccount, rank, perm, inv);
  return hipGetLastError();
}
hipError_t launch_scale_rows(const float* src, int64_t rows, int32_t K, _Float16* dst, int32_t* sig, hipStream_t s) {
  if (K % KS || rows <= 0 || rows > 0x7fffffff || ((uintptr_t)src & 15)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(scale_rows_kernel, dim3((unsigned)rows), dim3(256), 0, s, src, K, reinterpret_cast<uint4*>(dst),
                     sig);
  return hipGetLastError();
}
int64_t sclT_elements(const ExpertLayout& lay) {
  return 2 * (int64_t)lay.F * (lay.H / 32) + (int64_t)lay.H * (lay.F / 32);
}
hipError_t launch_transpose_scales(const uint8_t* const* eaddr, const int32_t* experts, int32_t n,
                                   const ExpertLayout& lay, uint16_t* out, const Launch& l) {
  if (n <= 0 || !experts || lay.H % 32 || lay.F % 32) return hipErrorInvalidValue;
  const int rmax = lay.F > lay.H ? lay.F : lay.H;
  return launch(transpose_scales_kernel, dim3((rmax + 63) / 64, 3, n), dim3(256), l, eaddr, experts, lay, out,
                sclT_elements(lay));
}
int gemm_features_per_tile(int mode, int bm) {
  if (mode == 0) return bm == 64 ? GemmTile<64, 0>::BNW : GemmTile<128, 0>::BNW;
  return bm == 64 ? GemmTile<64, 1>::BNW : GemmTile<128, 1>::BNW;
}
hipError_t launch_grouped_gemm(GemmArgs a, int mode, int bm, int n_items, const Launch& l) {
  if (a.K % KS || a.N % KS || n_items <= 0 || !a.items || (bm != 64 && bm != 128) || (mode != 0 && mode != 1) ||
      !a.sclT)
    return hipErrorInvalidValue;
  a.work = n_items;
  a.work_padded = (a.work + 7) / 8 * 8;
  const dim3 grid(a.work_padded), block(256);
  if (mode == 0) return bm == 64 ? launch(grouped_gemm_kernel<64, 0>, grid, block, l, a)
                                 : launch(grouped_gemm_kernel<128, 0>, grid, block, l, a);
  return bm == 64 ? launch(grouped_gemm_kernel<64, 1>, grid, block, l, a)
                  : launch(grouped_gemm_kernel<128, 1>, grid, block, l, a);
}
hipError_t launch_stage_experts(const uint8_t* host_layer, const int32_t* experts, int32_t n, int64_t bytes,
                               uint8_t* staging, hipStream_t s) {
  if (n <= 0 || bytes <= 0 || bytes % 16 || ((uintptr_t)host_layer & 15) || ((uintptr_t)staging & 15))
    return hipErrorInvalidValue;
  const int64_t b16 = bytes / 16;
  hipLaunchKernelGGL(stage_experts_kernel, dim3(128), dim3(256), 0, s, reinterpret_cast<const uint4*>(host_layer),
                     experts, (int64_t)n * b16, b16, reinterpret_cast<uint4*>(staging));
  return hipGetLastError();
}
hipError_t launch_combine_pairs(const float* ypair, const int32_t* inv, const float* w, int32_t T, int32_t k,
                                int32_t H, float* y, int32_t accumulate, hipStream_t s) {
  if (H % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_pairs_kernel<8>, dim3((H / 4 + 255) / 256, T), dim3(256), 0, s, ypair, inv, w, k, H, y,
                     accumulate);
  return hipGetLastError();
}

}  // namespace moe
