// grouped_mfma.hip - decode batches grouped by expert, on the matrix cores.
//
// At a batch of many tokens several tokens pick the same expert (about 2.4
// picks per distinct expert at 32 tokens, top-8 of 256). The per-pick GEMV
// dequantises every weight again for each of them; here each expert's
// weights are read and dequantised once per step for all of its picks, and
// the products run as v_mfma_f32_16x16x32_f16 with the picks as the 16 rows
// of the A operand (padding is free: the work is bound by the weight reads).
// This is the narrow-batch MoE mat-mul of the mx-llama.cpp FEATURES page
// (one pass per expert over the tokens that picked it) on MFMA.
//
// Exactness: the weight operand is q - 8 exactly (an fp16 integer); the
// block scale d is applied in fp32 to each quant block's product, so a
// block's dot product is one MFMA pair followed by one fp32 FMA. The
// activations enter as two fp16 terms hi + lo of the row scaled by a power
// of two (its largest magnitude in [2^13, 2^14)): hi = fp16(v), lo = fp16(v -
// hi), 22 significant bits, the scale undone exactly in fp32 afterwards. The
// result matches the fp32 GEMV to about 1e-7 relative.
//
//   split_rows_kernel   fp32 rows -> scaled fp16 hi/lo in operand order (the
//                       activations are split by the routing kernel itself)
//   mfma_grouped_kernel per (expert group, feature tile): gate/up -> h =
//                       silu(g) * u, or down -> y_pick = W_down h
//
// Operand order. A quant block (32 weights, 16 bytes) is one MFMA K step.
// Lane l of a wave covers row/column l % 16 and the K chunk c = l / 16,
// which holds the eight elements 4c + {0, 2, 1, 3, 16, 18, 17, 19} of the
// block: byte 4c + i of the block carries elements 4c + i (low nibble) and
// 4c + i + 16 (high nibble), so chunk c is the block's dword c, and its four
// masked pairs (w, w >> 8, w >> 4, w >> 12) & 0x000F000F, or-ed into the
// fp16 mantissa of 1024, give those elements in that order. The split
// activations are stored in the same order: block b of a row is 128 bytes,
// hi chunks 0..3 then lo chunks 0..3.
//
// Weight loads: one 16-byte load per lane covers four blocks of 16 rows
// (lane l: row l % 16, block 4j + l / 16), 1 KiB per wave and instruction,
// each row's 64 bytes contiguous. After the load lane (row, c) holds block
// 4j + c whole, but the MFMA of block 4j + i wants dword c of that block in
// lane group c: a 4 x 4 transpose of (lane group, dword), done by two rounds
// of v_permlane32_swap / v_permlane16_swap (swap the upper 32 lanes of one
// register with the lower 32 of another; swap odd 16-lane rows of one with
// the even rows of another).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "split_dev.h"

namespace moe {

namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;


__device__ __forceinline__ f16x2_t as_h2(uint32_t u) {
  f16x2_t v;
  __builtin_memcpy(&v, &u, 4);
  return v;
}
__device__ __forceinline__ uint32_t as_u32(f16x2_t v) {
  uint32_t u;
  __builtin_memcpy(&u, &v, 4);
  return u;
}

// (x & m) | c in one v_bitop3 (truth table of S0 & S1 | S2)
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(x, m, c, 0xEA);
}

// 8 weights q - 8 (exact fp16) of chunk c of a block from its dword w
__device__ __forceinline__ f16x8_t dequant_chunk(uint32_t w) {
  constexpr uint32_t M = 0x000F000Fu, MAGIC = 0x64006400u;  // fp16 1024 in both halves
  const f16x2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const f16x2_t p0 = as_h2(and_or(w, M, MAGIC)) - off;        // elements 0, 2
  const f16x2_t p1 = as_h2(and_or(w >> 8, M, MAGIC)) - off;   // 1, 3
  const f16x2_t p2 = as_h2(and_or(w >> 4, M, MAGIC)) - off;   // 16, 18
  const f16x2_t p3 = as_h2(and_or(w >> 12, M, MAGIC)) - off;  // 17, 19
  f16x8_t r;
  r[0] = p0[0], r[1] = p0[1], r[2] = p1[0], r[3] = p1[1];
  r[4] = p2[0], r[5] = p2[1], r[6] = p3[0], r[7] = p3[1];
  return r;
}

// (lane group g, dword d) -> (lane group d, dword g) within each 16-lane
// column of the wave: afterwards dword i of lane group c is the old dword c
// of lane group i
__device__ __forceinline__ void transpose4(uint4& v) {
  auto a = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
  auto b = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  v.x = c[0], v.y = c[1], v.z = d[0], v.w = d[1];
}

__device__ __forceinline__ float half_lo(uint32_t u) { return (float)as_h2(u)[0]; }
__device__ __forceinline__ float half_hi(uint32_t u) { return (float)as_h2(u)[1]; }

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }


// One block of the wave's weight tiles: the MFMA pair on hi and lo, then the
// block scale d in fp32 into the accumulator (4 rows x 1 column per lane).
__device__ __forceinline__ void block_fma(f32x4_t& acc, const f16x8_t& ahi, const f16x8_t& alo, uint32_t wchunk,
                                          float d) {
  const f16x8_t b = dequant_chunk(wchunk);
  f32x4_t c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, b, c, 0, 0, 0);
  acc[0] = fmaf(d, c[0], acc[0]);
  acc[1] = fmaf(d, c[1], acc[1]);
  acc[2] = fmaf(d, c[2], acc[2]);
  acc[3] = fmaf(d, c[3], acc[3]);
}

// The weight loads of one step (four blocks) of NW tiles.
template <int NW>
struct WStep {
  uint4 w[NW];   // nibbles: lane (row, c) holds block 4j + c of its tile's row
};
struct AStep {
  u32x4_t a[2];  // the two 16-byte pieces of a step's A rows this lane stages
};

// Copies bytes [off, off + n) of src to dst, cooperatively in one
// work-group: 16-byte pieces, one in flight per thread (n and off multiples
// of 16). Fewer reads in flight cross PCIe faster here: with about one cold
// expert per layer (its 24 work-groups copying at once) the large model's
// batch-32 step took 22.3 ms at 8 pieces per thread in flight, 21.7 at 4,
// 21.4 at 2 and 21.2 at 1; 128 or 64 copying threads per work-group instead
// of 256 took 23.1 and 31.3 ms.
__device__ __forceinline__ void stage_run(const uint8_t* src, uint8_t* dst, int64_t off, int64_t n) {
  const uint4* s = reinterpret_cast<const uint4*>(src + off);
  uint4* d = reinterpret_cast<uint4*>(dst + off);
  const int64_t n16 = n / 16;
  for (int64_t i = threadIdx.x; i < n16; i += 256) d[i] = s[i];
}

// Each lane group's value of x in every lane of its 16-lane column: out[g]
// holds group g's. Two swap rounds: [x0 x1 x2 x3] -> [x0 x1 x0 x1] and
// [x2 x3 x2 x3] -> [x0 x0 x0 x0], [x1 ...], [x2 ...], [x3 ...].
__device__ __forceinline__ void broadcast4(uint32_t x, uint32_t (&out)[4]) {
  const auto h = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  const auto lo = __builtin_amdgcn_permlane16_swap(h[0], h[0], false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap(h[1], h[1], false, false);
  out[0] = lo[0], out[1] = lo[1], out[2] = hi[0], out[3] = hi[1];
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// s_waitcnt immediate (GFX9 encoding) waiting for vmcnt <= n only
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// The A rows of a step in LDS: 16 rows x 512 bytes (four split blocks); the
// 16-byte chunk g of row r sits at position g ^ ((r & 3) << 2), so that the
// fragment reads of 16 rows x 4 chunks spread over all banks.
constexpr int kRowBytes = 512;
constexpr int kStageBytes = 16 * kRowBytes;
constexpr int kRing = 4;  // steps in the ring: three are in flight while one is computed
__device__ __forceinline__ int a_pos(int r, int g) { return g ^ ((r & 3) << 2); }

}  // namespace

// ---------------------------------------------------------------------------

// fp32 rows [R][K] -> split rows [R][K/32][128 B] (split_dev.h) and their
// exponents; one work-group per row, each thread one chunk of a block at a
// time.
__global__ __launch_bounds__(256) void split_rows_kernel(const float* __restrict__ src, int32_t K,
                                                         uint4* __restrict__ dst, int32_t* __restrict__ sig) {
  __shared__ float s_max[4];
  const int64_t r = blockIdx.x;
  const float4* row = reinterpret_cast<const float4*>(src + r * K);
  float m = 0.f;
  for (int q = threadIdx.x; q < K / 4; q += 256) m = split_dev::abs_max4(row[q], m);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
  __syncthreads();
  const int e = split_dev::scale_exp(fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3])));
  if (threadIdx.x == 0) sig[r] = e;
  const float* rf = src + r * K;
  const int KB = K / 32;
  uint4* out = dst + r * (int64_t)KB * 8;
  for (int q = threadIdx.x; q < KB * 4; q += 256) {
    const int b = q >> 2, c = q & 3;
    split_dev::chunk(rf + 32 * b, c, e, out[8 * b + c], out[8 * b + 4 + c]);
  }
}

// One expert group's products on the matrix cores: grid = (feature tiles of
// 64 NT, groups). MODE 0 (gate/up): wave w covers features f0 + 16 NT w +
// [0, 16 NT) of gate and of up (2 NT weight tiles), the A rows are the split
// activations of the picks' tokens, and h[p][f] = silu(g) * u (fp32).
// MODE 1 (down): NT tiles of W_down, the A rows are the split h rows of the
// picks, and y_pick[p][f]. The group's picks go 16 at a time through the
// A rows.
//
// Per step (four blocks) each wave loads the weights of step j + 3 into a
// ring of kRing register sets, and, if its rows 4w .. 4w + 3 hold picks, that
// step's A rows; it writes step j + 1's A rows (loaded two steps earlier)
// into their LDS stage and computes step j; a barrier per step publishes the
// stage. The block scales of four steps come in one load per tile: lane group
// g fetches the scales of step 4 q + g of its row, and each step broadcasts
// its group's four scales to the whole column. The number of steps is a
// multiple of 4; the loads past the last step re-read it (never used), so the
// compiler's waits count exactly the loads still in flight.
template <int NT, int MODE>
__global__ __launch_bounds__(256) void mfma_grouped_kernel(GemvArgs a, GroupArgs gr, SplitArgs sp) {
  constexpr int NW = MODE == 0 ? 2 * NT : NT;
  __shared__ __attribute__((aligned(1024))) uint8_t s_a[kRing * kStageBytes];
  if ((int)blockIdx.y >= *gr.n_groups) return;
  const int4 grp = gr.groups[blockIdx.y];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, c = lane >> 4;
  const int K = MODE == 0 ? a.H : a.F, N = MODE == 0 ? a.F : a.H;
  const int KB = K / 32, nsteps = KB / 4;
  const int p0 = gr.order[grp.y];
  const uint8_t* base = a.addr[p0];
  const int f0 = blockIdx.x * 64 * NT + wave * 16 * NT;
  if ((a.kind[p0] & kCold) && a.capture && (int)blockIdx.y < a.capture_picks) {
    // a cold expert (groups with a cold expert come first): this work-group's
    // weight rows cross PCIe once, as long contiguous runs, into capture block
    // g of the layer, and the products read them from there (zero-copy reads
    // in the 64-byte pieces of the weight tiles ran at a third of the PCIe
    // rate). The gate/up and down launches together fill the whole block, so
    // the cache step can promote the expert from it.
    uint8_t* cap = a.capture + (int64_t)blockIdx.y * a.lay.bytes;
    const int64_t r0 = (int64_t)blockIdx.x * 64 * NT, rc = N - r0 < 64 * NT ? N - r0 : 64 * NT;
    if (MODE == 0) {
      stage_run(base, cap, a.lay.gate_nib + r0 * KB * 16, rc * KB * 16);
      stage_run(base, cap, a.lay.gate_scl + r0 * KB * 2, rc * KB * 2);
      stage_run(base, cap, a.lay.up_nib + r0 * KB * 16, rc * KB * 16);
      stage_run(base, cap, a.lay.up_scl + r0 * KB * 2, rc * KB * 2);
      if (blockIdx.x == 0 && threadIdx.x == 0)
        a.cap_dir[blockIdx.y] = ((uint64_t)a.ctrl->clock << 32) | (uint32_t)grp.x;
    } else {
      stage_run(base, cap, a.lay.down_nib + r0 * KB * 16, rc * KB * 16);
      stage_run(base, cap, a.lay.down_scl + r0 * KB * 2, rc * KB * 2);
    }
    __syncthreads();  // every wave's copies are visible to the work-group
    base = cap;
  }
  // this lane's weight row of each tile (past N: row N - 1, never stored)
  const uint4* nib[NW];
  const uint2* scl[NW];
#pragma unroll
  for (int t = 0; t < NW; ++t) {
    int f = f0 + 16 * (t % NT) + col;
    f = f < N ? f : N - 1;
    const bool up = MODE == 0 && t >= NT;
    nib[t] = reinterpret_cast<const uint4*>(base + (MODE == 1 ? a.lay.down_nib : up ? a.lay.up_nib : a.lay.gate_nib)) +
             (int64_t)f * KB + c;
    // scales of step 4 q + c of the row: uint2 index 4 q + c
    scl[t] = reinterpret_cast<const uint2*>(base + (MODE == 1 ? a.lay.down_scl : up ? a.lay.up_scl : a.lay.gate_scl)) +
             (int64_t)f * KB / 4 + c;
  }
  const uint8_t* split = MODE == 0 ? sp.x : sp.h;

  for (int r0 = 0; r0 < grp.z; r0 += 16) {
    const int rows = grp.z - r0 < 16 ? grp.z - r0 : 16;
    const bool arows = 4 * wave < rows;  // this wave's A rows hold picks (wave-uniform)
    // A rows this lane moves: r = 4w + 2i + lane / 32, 16-byte chunk lane % 32
    const u32x4_t* asrc[2];
    int adst[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 4 * wave + 2 * i + (lane >> 5);
      const int p = gr.order[grp.y + r0 + (r < rows ? r : 0)];  // past the group: row 0 (never stored)
      const int64_t row = MODE == 0 ? p / a.k : p;
      asrc[i] = reinterpret_cast<const u32x4_t*>(split + row * KB * 128) + (lane & 31);
      adst[i] = r * kRowBytes + 16 * a_pos(r, lane & 31);
    }
    WStep<NW> wb[kRing];
    AStep ab[2];
    auto issue = [&](int j, WStep<NW>& w) __attribute__((always_inline)) {
      j = j < nsteps ? j : nsteps - 1;  // past the end: re-read the last step (never used)
#pragma unroll
      for (int t = 0; t < NW; ++t) w.w[t] = nib[t][4 * j];
    };
    auto issue_a = [&](int j, AStep& av) __attribute__((always_inline)) {
      j = j < nsteps ? j : nsteps - 1;
      if (arows) {
#pragma unroll
        for (int i = 0; i < 2; ++i) av.a[i] = asrc[i][32 * j];
      }
    };
    auto stage = [&](int j, const AStep& av) __attribute__((always_inline)) {
      if (arows) {
        const int st = (j % kRing) * kStageBytes;
#pragma unroll
        for (int i = 0; i < 2; ++i)
          *(lds_u32x4_t*)(s_a + st + adst[i]) = av.a[i];  // an LDS store: aliases no register array
      }
    };
    // scales of steps 4 q .. 4 q + 3 (lane group g: step 4 q + g)
    auto issue_scales = [&](int q, uint2 (&sv)[NW]) __attribute__((always_inline)) {
      q = 4 * q < nsteps ? q : nsteps / 4 - 1;
#pragma unroll
      for (int t = 0; t < NW; ++t) sv[t] = scl[t][4 * q];
    };
    f32x4_t acc[NW];
#pragma unroll
    for (int t = 0; t < NW; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint2 s_cur[NW], s_nxt[NW];
    issue_scales(0, s_cur);
#pragma unroll
    for (int i = 0; i < kRing - 1; ++i) issue(i, wb[i]);
    // A rows two steps ahead: step j + 2 is loaded at step j, staged at step j + 1
    issue_a(0, ab[0]);
    issue_a(1, ab[1]);
    stage(0, ab[0]);
#pragma unroll 1
    for (int j0 = 0; j0 < nsteps; j0 += kRing) {
      // this quad's scales in every lane: sb[t][dword][step of the quad]
      uint32_t sb[NW][2][4];
#pragma unroll
      for (int t = 0; t < NW; ++t) {
        broadcast4(s_cur[t].x, sb[t][0]);
        broadcast4(s_cur[t].y, sb[t][1]);
      }
      issue_scales(j0 / 4 + 1, s_nxt);
#pragma unroll
      for (int u = 0; u < kRing; ++u) {
        const int j = j0 + u;
        // step j's A rows are in their stage; every wave is done with step j - 1's
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);  // no instruction moves between steps: bounded live ranges
        issue(j + kRing - 1, wb[(u + kRing - 1) % kRing]);
        stage(j + 1, ab[(u + 1) % 2]);  // its stage was last read at step j + 1 - kRing
        issue_a(j + 2, ab[u % 2]);      // into the registers step j staged from one step ago
        WStep<NW>& w = wb[u];
        const uint8_t* st = s_a + (j % kRing) * kStageBytes + col * kRowBytes;
#pragma unroll
        for (int t = 0; t < NW; ++t) transpose4(w.w[t]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // one block at a time: other waves of the SIMD supply the overlap, and the
          // registers of four blocks' fragments and products in flight would halve occupancy
          __builtin_amdgcn_sched_barrier(0);
          const f16x8_t ahi = *reinterpret_cast<const f16x8_t*>(st + 16 * a_pos(col, 8 * i + c));
          const f16x8_t alo = *reinterpret_cast<const f16x8_t*>(st + 16 * a_pos(col, 8 * i + 4 + c));
#pragma unroll
          for (int t = 0; t < NW; ++t) {
            const uint32_t wi = i == 0 ? w.w[t].x : i == 1 ? w.w[t].y : i == 2 ? w.w[t].z : w.w[t].w;
            const uint32_t si = sb[t][i >> 1][u];
            block_fma(acc[t], ahi, alo, wi, (i & 1) ? half_hi(si) : half_lo(si));
            // a use of the sums here: otherwise the compiler sinks every block's scale FMAs to
            // the end of the unrolled steps and keeps all their products live
            __asm__ volatile("" : "+v"(acc[t]));
          }
        }
      }
#pragma unroll
      for (int t = 0; t < NW; ++t) s_cur[t] = s_nxt[t];
    }
    // epilogue: lane holds rows 4c + i of column col of each tile
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * c + i;
      if (m >= rows) continue;
      const int p = gr.order[grp.y + r0 + m];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int f = f0 + 16 * t + col;
        if (f >= N) continue;
        if (MODE == 0) {
          const int s = sp.xsig[p / a.k];
          const float g = ldexpf(acc[t][i], -s), u = ldexpf(acc[t + NT][i], -s);
          a.out[(int64_t)p * N + f] = silu(g) * u;
        } else {
          a.ypick[(int64_t)p * N + f] = ldexpf(acc[t][i], -sp.hsig[p]);
        }
      }
    }
    __syncthreads();  // the next row tile refills the stages
  }
}

// ---------------------------------------------------------------------------

namespace {
constexpr int kNtGateUp = 1;  // gate + up: 4 weight tiles per wave
constexpr int kNtDown = 2;    // down: 4 weight tiles per wave
}  // namespace

// steps of four blocks, a multiple of kRing of them per row
bool mfma_grouped_shape_ok(int32_t H, int32_t F) {
  return H > 0 && F > 0 && H % (128 * kRing) == 0 && F % (128 * kRing) == 0;
}

hipError_t launch_split_rows(const float* src, int32_t rows, int32_t K, uint8_t* dst, int32_t* sig, hipStream_t s) {
  if (rows < 1 || K % 32 || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(split_rows_kernel, dim3(rows), dim3(256), 0, s, src, K, reinterpret_cast<uint4*>(dst), sig);
  return hipGetLastError();
}

hipError_t launch_mfma_gateup(const GemvArgs& a, const GroupArgs& g, const SplitArgs& sp, const Launch& l) {
  if (g.P < 1 || !mfma_grouped_shape_ok(a.H, a.F)) return hipErrorInvalidValue;
  const dim3 grid((a.F + 64 * kNtGateUp - 1) / (64 * kNtGateUp), g.P);
  return launch(mfma_grouped_kernel<kNtGateUp, 0>, grid, dim3(256), l, a, g, sp);
}

hipError_t launch_mfma_down(const GemvArgs& a, const GroupArgs& g, const SplitArgs& sp, const Launch& l) {
  if (g.P < 1 || !mfma_grouped_shape_ok(a.H, a.F)) return hipErrorInvalidValue;
  const dim3 grid((a.H + 64 * kNtDown - 1) / (64 * kNtDown), g.P);
  return launch(mfma_grouped_kernel<kNtDown, 1>, grid, dim3(256), l, a, g, sp);
}

}  // namespace moe
