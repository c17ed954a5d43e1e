// prefill.cpp - host side of the prompt pass of one MoE layer: route the
// micro-batch, sort the (token, pick) pairs by expert on the GPU, copy the
// touched experts that are not resident into borrowed HBM staging blocks
// (the "llama.cpp: fork with multi gpu acceleration ..." README, "How it
// works": a prompt pass streams the experts the GPU does not hold and gives
// the borrowed blocks back afterwards), run the grouped gate/up and down
// GEMMs over the used (expert, tile) pairs only, and combine in pick order.
// The cache policy is not touched: no stamps, records, counts or clock.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "kernels.h"
#include "runtime.h"

namespace {
constexpr int kMinTileRows = 64;  // tiles hold 64 or 128 pairs of one expert
// The staging copy runs on a stream of its own; the GEMMs of the experts
// that need no copy run meanwhile, those of the staged ones once their copy
// has landed. Two ways to copy, picked per pass from rough time estimates:
// * the copy would outlast the GEMMs of the experts already in HBM: one
//   gather kernel per chunk (up to kStageChunks of at least kMinChunkExperts
//   experts) reading the pinned weights zero-copy, at the PCIe ceiling; each
//   chunk's GEMMs run while the next chunk is in flight;
// * else DMA copies, one per run of consecutive experts, which take no
//   compute units: the gather kernel's PCIe reads hold up the memory
//   pipelines of the CUs they share with a GEMM, so beside a long GEMM the
//   DMA engines are the better choice even at their lower rate.
constexpr int kStageChunks = 8;
constexpr int kMinChunkExperts = 16;
constexpr double kPcieBytesPerS = 55e9;      // staging rate, either way (measured 49-57.5 GB/s)
constexpr double kGemmFlopsPerS = 600e12;    // grouped GEMMs on long tiles (measured 600-860 TFLOP/s)
constexpr int kMaxGroups = 1 + kStageChunks;  // group 0: experts read where they are
constexpr int kTimed = 3;                     // per group: scale transposition, gate/up, down

// Rows per tile for a pass: 128-row tiles halve the weight conversions per
// MFMA but pad small experts further. A 64-row tile step is taken to cost
// 0.6 of a 128-row one (its weight conversion does not shrink with the
// rows), so 128 is used when it needs fewer than 0.6 x as many tiles.
int tile_rows(const int32_t* counts, int32_t E) {
  int64_t t64 = 0, t128 = 0;
  for (int32_t e = 0; e < E; ++e) {
    t64 += (counts[e] + 63) / 64;
    t128 += (counts[e] + 127) / 128;
  }
  return 10 * t128 < 6 * t64 ? 128 : 64;
}

bool capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) return false;
  return st != hipStreamCaptureStatusNone;
}
}  // namespace

struct Prefill {
  int64_t max_tokens = 0, max_pairs = 0, max_tiles = 0, max_items = 0;
  int32_t last_layer = -1;      // layer of the last completed pass (h_counts / h_eaddr describe it)
  int32_t* ids = nullptr;       // [P]
  float* w = nullptr;           // [P]
  int32_t* perm = nullptr;      // [P] sorted position -> pair
  int32_t* inv = nullptr;       // [P] pair -> sorted position
  int32_t* counts = nullptr;    // [E]
  int32_t* rank = nullptr;      // [P] rank of a pair among its chunk's pairs of the same expert
  int32_t* ccount = nullptr;    // [E][P / 256 chunks] counts, then starts, per chunk
  int32_t* offsets = nullptr;   // [E + 1]
  int4* tiles = nullptr;        // [max_tiles]
  int2* items[2] = {nullptr, nullptr};    // [max_items] work lists of the gate/up and down GEMMs
  const uint8_t** eaddr = nullptr;  // [E]
  int32_t* stage = nullptr;     // [E] experts copied into the staging blocks, in block order
  _Float16* x16 = nullptr;      // [T][H] activations, fp16 in operand order, row t scaled by 2^sig[t]
  int32_t* sig = nullptr;       // [T] row scale exponents
  uint32_t* range_flag = nullptr;    // set by the gate/up GEMM when a scaled h leaves the fp16 range
  uint32_t* h_range_flag = nullptr;  // pinned copy read after the pass
  _Float16* h16 = nullptr;      // [P][F] SwiGLU outputs, fp16 in operand order
  float* ypair = nullptr;       // [P][H]
  uint16_t* sclT = nullptr;     // [E][sclT_elements]: the pass's block scales, transposed
  // pinned staging of the small transfers
  int32_t* h_counts = nullptr;
  int32_t* h_offsets = nullptr;
  int4* h_tiles = nullptr;
  int2* h_items[2] = {nullptr, nullptr};
  const uint8_t** h_eaddr = nullptr;
  int32_t* h_stage = nullptr;   // [E] staged experts in block order, then the experts of group 0
  std::vector<int64_t> tile_begin;  // [E + 1] first tile of each expert
  std::vector<int32_t> direct;      // used experts read where they are
  hipStream_t copy_stream = nullptr;
  hipEvent_t lists_ready = nullptr;              // the staging list is on the device
  hipEvent_t chunk_done[kStageChunks] = {};      // chunk c of the staging copy has landed
  hipEvent_t timing[2 * kTimed * kMaxGroups] = {};  // start/stop of each timed launch
  hipEvent_t stage_timing[2] = {};                  // first and last chunk of the staging copy
};

#define PF_HIP(ctx, expr)                                                                                \
  do {                                                                                                   \
    hipError_t e_ = (expr);                                                                              \
    if (e_ != hipSuccess) return moe_ctx_fail((ctx), MOE_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

int moe_prefill_alloc(moe_ctx* c) {
  const int64_t T = c->cfg.max_prefill_tokens;
  if (T <= 0) return MOE_OK;
  Prefill* p = new Prefill();
  c->pf = p;
  const int64_t E = c->E, P = T * c->k;
  p->max_tokens = T, p->max_pairs = P;
  p->max_tiles = E + P / kMinTileRows + 1;
  p->max_items = p->max_tiles * ((std::max(c->F, c->H) + 127) / 128);  // feature tiles are >= 128 wide
  int rc;
  auto dev = [&](void** q, size_t bytes, const char* what) { return moe_ctx_dev_alloc(c, q, bytes, what); };
  if ((rc = dev((void**)&p->ids, sizeof(int32_t) * P, "prefill ids")) ||
      (rc = dev((void**)&p->w, sizeof(float) * P, "prefill weights")) ||
      (rc = dev((void**)&p->perm, sizeof(int32_t) * P, "prefill perm")) ||
      (rc = dev((void**)&p->inv, sizeof(int32_t) * P, "prefill inverse perm")) ||
      (rc = dev((void**)&p->counts, sizeof(int32_t) * E, "prefill counts")) ||
      (rc = dev((void**)&p->rank, sizeof(int32_t) * P, "prefill ranks")) ||
      (rc = dev((void**)&p->ccount, sizeof(int32_t) * E * moe::sort_chunks((int32_t)P), "prefill chunk counts")) ||
      (rc = dev((void**)&p->offsets, sizeof(int32_t) * (E + 1), "prefill offsets")) ||
      (rc = dev((void**)&p->tiles, sizeof(int4) * p->max_tiles, "prefill tiles")) ||
      (rc = dev((void**)&p->items[0], sizeof(int2) * p->max_items, "prefill gate/up work list")) ||
      (rc = dev((void**)&p->items[1], sizeof(int2) * p->max_items, "prefill down work list")) ||
      (rc = dev((void**)&p->eaddr, sizeof(uint8_t*) * E, "prefill addresses")) ||
      (rc = dev((void**)&p->stage, sizeof(int32_t) * E, "prefill staging list")) ||
      (rc = dev((void**)&p->x16, sizeof(_Float16) * T * c->H, "prefill x fp16")) ||
      (rc = dev((void**)&p->sig, sizeof(int32_t) * T, "prefill row scales")) ||
      (rc = dev((void**)&p->range_flag, sizeof(uint32_t), "prefill range flag")) ||
      (rc = dev((void**)&p->h16, sizeof(_Float16) * P * c->F, "prefill h fp16")) ||
      (rc = dev((void**)&p->ypair, sizeof(float) * P * c->H, "prefill pair outputs")) ||
      (rc = dev((void**)&p->sclT, sizeof(uint16_t) * E * moe::sclT_elements(c->lay), "prefill transposed scales")))
    return rc;
  const unsigned pin = hipHostMallocDefault;
  if ((rc = moe_ctx_host_alloc(c, (void**)&p->h_counts, sizeof(int32_t) * E, pin, "prefill count staging")) ||
      (rc = moe_ctx_host_alloc(c, (void**)&p->h_offsets, sizeof(int32_t) * (E + 1), pin, "prefill offsets staging")) ||
      (rc = moe_ctx_host_alloc(c, (void**)&p->h_tiles, sizeof(int4) * p->max_tiles, pin, "prefill tile staging")) ||
      (rc = moe_ctx_host_alloc(c, (void**)&p->h_items[0], sizeof(int2) * p->max_items, pin, "prefill item staging")) ||
      (rc = moe_ctx_host_alloc(c, (void**)&p->h_items[1], sizeof(int2) * p->max_items, pin, "prefill item staging")) ||
      (rc = moe_ctx_host_alloc(c, (void**)&p->h_eaddr, sizeof(uint8_t*) * E, pin, "prefill address staging")) ||
      (rc = moe_ctx_host_alloc(c, (void**)&p->h_stage, sizeof(int32_t) * E, pin, "prefill staging list")) ||
      (rc = moe_ctx_host_alloc(c, (void**)&p->h_range_flag, sizeof(uint32_t), pin, "prefill range flag")))
    return rc;
  p->tile_begin.assign(E + 1, 0);
  p->direct.reserve(E);
  // default priority, like every stream here
  if (hipStreamCreateWithFlags(&p->copy_stream, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&p->lists_ready, hipEventDisableTiming) != hipSuccess)
    return moe_ctx_fail(c, MOE_E_HIP, "prefill: stream or event creation failed");
  for (hipEvent_t& ev : p->chunk_done)
    if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess)
      return moe_ctx_fail(c, MOE_E_HIP, "prefill: event creation failed");
  for (hipEvent_t& ev : p->timing)
    if (hipEventCreateWithFlags(&ev, hipEventDisableSystemFence) != hipSuccess)
      return moe_ctx_fail(c, MOE_E_HIP, "prefill: event creation failed");
  for (hipEvent_t& ev : p->stage_timing)
    if (hipEventCreateWithFlags(&ev, hipEventDisableSystemFence) != hipSuccess)
      return moe_ctx_fail(c, MOE_E_HIP, "prefill: event creation failed");
  return MOE_OK;
}

// HBM blocks lent to a prompt pass for the touched experts that are not
// resident: E - S of them hold every expert a pass can miss (E with one
// global pool, which may hold none of a layer's experts).
int moe_prefill_alloc_staging(moe_ctx* c) {
  if (c->cfg.max_prefill_tokens <= 0) return MOE_OK;
  // with one global pool a layer may have none of its experts resident
  c->n_staging = c->groups == 1 && c->L > 1 ? (int64_t)c->E : std::max<int64_t>(0, (int64_t)c->E - c->S);
  return moe_ctx_dev_alloc(c, (void**)&c->staging, (size_t)(c->n_staging * c->B), "prefill staging blocks");
}

void moe_prefill_release(moe_ctx* c) {
  Prefill* p = c->pf;
  if (!p) return;
  if (p->copy_stream) {
    (void)hipStreamSynchronize(p->copy_stream);
    (void)hipStreamDestroy(p->copy_stream);
  }
  if (p->lists_ready) (void)hipEventDestroy(p->lists_ready);
  for (hipEvent_t ev : p->chunk_done)
    if (ev) (void)hipEventDestroy(ev);
  for (hipEvent_t ev : p->timing)
    if (ev) (void)hipEventDestroy(ev);
  for (hipEvent_t ev : p->stage_timing)
    if (ev) (void)hipEventDestroy(ev);
  delete p;
  c->pf = nullptr;
}

extern "C" int moe_prefill(moe_ctx* c, int32_t layer, int32_t n_tokens, const float* x, const float* logits,
                           float* y, uint32_t flags) {
  if (!c) return MOE_E_INVAL;
  Prefill* p = c->pf;
  if (!p) return moe_ctx_fail(c, MOE_E_STATE, "prefill: created with max_prefill_tokens = 0");
  if (layer < 0 || layer >= c->L) return moe_ctx_fail(c, MOE_E_INVAL, "prefill: bad layer %d", layer);
  if (n_tokens < 1 || n_tokens > p->max_tokens)
    return moe_ctx_fail(c, MOE_E_INVAL, "prefill: n_tokens %d outside 1..%lld", n_tokens, (long long)p->max_tokens);
  if (!x || !y || ((uintptr_t)x & 15) || ((uintptr_t)y & 15))
    return moe_ctx_fail(c, MOE_E_INVAL, "prefill: x and y must be non-null 16-byte aligned pointers");
  if (y == x && !(flags & MOE_ACCUMULATE))
    return moe_ctx_fail(c, MOE_E_INVAL, "prefill: y may alias x only with MOE_ACCUMULATE");
  if (!logits && !c->routers[layer]) return moe_ctx_fail(c, MOE_E_INVAL, "prefill: no logits and no router");
  if (!c->seeded) return moe_ctx_fail(c, MOE_E_STATE, "prefill before moe_seed");
  if (capturing(c->stream)) return moe_ctx_fail(c, MOE_E_CAPTURING, "prefill while capturing");
  // a pass that failed part-way may have left staging copies running
  PF_HIP(c, hipStreamSynchronize(p->copy_stream));
  hipStream_t s = c->stream;
  const int32_t E = c->E, k = c->k, H = c->H, F = c->F, T = n_tokens;
  const int32_t P = T * k;

  // 1. routing only (no lookup, no policy side effects)
  moe::RouteArgs ra{};
  ra.logits = logits;
  ra.x = x;
  ra.wr = (const float*)c->routers[layer];
  ra.T = T, ra.E = E, ra.k = k, ra.H = H, ra.S = c->S, ra.layer = layer;
  ra.ids = p->ids, ra.w = p->w;
  ra.policy = 0;
  moe::Launch ls;
  ls.stream = s;
  PF_HIP(c, moe::launch_route(ra, ls));

  // 2. pairs per expert, to the host
  PF_HIP(c, moe::launch_expert_counts(p->ids, P, E, p->rank, p->ccount, p->counts, s));
  PF_HIP(c, hipMemcpyAsync(p->h_counts, p->counts, sizeof(int32_t) * E, hipMemcpyDeviceToHost, s));
  PF_HIP(c, hipStreamSynchronize(s));

  // 3. offsets, tiles of the used experts, and where each expert is read from
  int64_t n_tiles = 0, staged = 0, pos = 0;
  const int64_t S = c->S;
  const int bm = tile_rows(p->h_counts, E);
  std::vector<int64_t>& tb = p->tile_begin;
  std::vector<int32_t>& direct = p->direct;
  direct.clear();
  for (int32_t e = 0; e < E; ++e) {
    const int32_t m = p->h_counts[e];
    p->h_offsets[e] = (int32_t)pos;
    p->h_eaddr[e] = nullptr;
    tb[e] = n_tiles;
    if (m > 0) {
      const int32_t slot = c->tbl[(int64_t)layer * E + e];
      if (slot >= 0) {
        p->h_eaddr[e] = c->pool + (c->group_of(layer) * S + slot) * c->B;
        direct.push_back(e);
      } else if (staged < c->n_staging) {
        p->h_eaddr[e] = c->staging + staged * c->B;
        p->h_stage[staged++] = e;
      } else {
        p->h_eaddr[e] = c->host_layers_dev[layer] + (int64_t)e * c->B;  // no block left: read zero-copy
        direct.push_back(e);
      }
      for (int32_t m0 = 0; m0 < m; m0 += bm) p->h_tiles[n_tiles++] = int4{e, (int32_t)(pos + m0), std::min(bm, m - m0), 0};
    }
    pos += m;
  }
  tb[E] = n_tiles;
  p->h_offsets[E] = (int32_t)pos;
  c->last_prefill_staged = staged;
  if (pos != P) return moe_ctx_fail(c, MOE_E_HIP, "prefill: pair count mismatch (%lld != %d)", (long long)pos, P);

  // Groups of experts: 0 = those read where they are (resident, or zero-copy
  // when no staging block is left), 1.. = the chunks of the staging copy in
  // block order. h_stage holds the staged experts, then group 0's.
  const int64_t n_direct = (int64_t)direct.size();
  int64_t direct_pairs = 0;
  for (int32_t e : direct) direct_pairs += p->h_counts[e];
  const double copy_s = (double)staged * c->B / kPcieBytesPerS;
  const double gemm_s = 6.0 * H * F * (double)direct_pairs / kGemmFlopsPerS;
  const bool dma = copy_s < gemm_s;
  const int n_chunks = staged == 0 ? 0
                       : dma      ? 1
                                  : (int)std::min<int64_t>(kStageChunks, std::max<int64_t>(1, staged / kMinChunkExperts));
  const int64_t chunk = n_chunks ? (staged + n_chunks - 1) / n_chunks : 0;
  const int G = 1 + n_chunks;
  std::copy(direct.begin(), direct.end(), p->h_stage + staged);
  int64_t g_first[kMaxGroups], g_count[kMaxGroups];
  g_first[0] = staged, g_count[0] = n_direct;
  for (int g = 1; g < G; ++g) {
    g_first[g] = (g - 1) * chunk;
    g_count[g] = std::max<int64_t>(0, std::min<int64_t>(chunk, staged - g_first[g]));
  }
  // work lists, group by group: per expert, feature tiles outer and row tiles inner
  int64_t item_first[2][kMaxGroups + 1];
  for (int mode = 0; mode < 2; ++mode) {
    const int N = mode == 0 ? F : H, bnw = moe::gemm_features_per_tile(mode, bm);
    if (n_tiles * ((N + bnw - 1) / bnw) > p->max_items)
      return moe_ctx_fail(c, MOE_E_HIP, "prefill: work list larger than its buffer");
    int2* it = p->h_items[mode];
    int64_t n = 0;
    for (int g = 0; g < G; ++g) {
      item_first[mode][g] = n;
      for (int64_t i = 0; i < g_count[g]; ++i) {
        const int32_t e = p->h_stage[g_first[g] + i];
        for (int n0 = 0; n0 < N; n0 += bnw)
          for (int64_t t = tb[e]; t < tb[e + 1]; ++t) it[n++] = int2{(int32_t)t, n0};
      }
    }
    item_first[mode][G] = n;
    PF_HIP(c, hipMemcpyAsync(p->items[mode], it, sizeof(int2) * n, hipMemcpyHostToDevice, s));
  }
  PF_HIP(c, hipMemcpyAsync(p->stage, p->h_stage, sizeof(int32_t) * (staged + n_direct), hipMemcpyHostToDevice, s));
  PF_HIP(c, hipMemcpyAsync(p->offsets, p->h_offsets, sizeof(int32_t) * (E + 1), hipMemcpyHostToDevice, s));
  PF_HIP(c, hipMemcpyAsync(p->tiles, p->h_tiles, sizeof(int4) * n_tiles, hipMemcpyHostToDevice, s));
  PF_HIP(c, hipMemcpyAsync(p->eaddr, p->h_eaddr, sizeof(uint8_t*) * E, hipMemcpyHostToDevice, s));

  // 4. the staging copy, chunk by chunk on its own stream, after everything
  // already queued on the pass's stream (earlier readers of the blocks)
  const bool timed = c->profiling;
  if (n_chunks > 0) {
    PF_HIP(c, hipEventRecord(p->lists_ready, s));
    PF_HIP(c, hipStreamWaitEvent(p->copy_stream, p->lists_ready, 0));
    if (timed) PF_HIP(c, hipEventRecord(p->stage_timing[0], p->copy_stream));
    for (int g = 1; g < G; ++g) {
      if (dma) {
        for (int64_t i = g_first[g], end = g_first[g] + g_count[g]; i < end;) {
          int64_t j = i + 1;
          while (j < end && p->h_stage[j] == p->h_stage[j - 1] + 1) ++j;
          PF_HIP(c, hipMemcpyAsync(c->staging + i * c->B, c->host_layers[layer] + (int64_t)p->h_stage[i] * c->B,
                                   (j - i) * c->B, hipMemcpyHostToDevice, p->copy_stream));
          i = j;
        }
      } else {
        PF_HIP(c, moe::launch_stage_experts(c->host_layers_dev[layer], p->stage + g_first[g], (int32_t)g_count[g],
                                            c->B, c->staging + g_first[g] * c->B, p->copy_stream));
      }
      PF_HIP(c, hipEventRecord(p->chunk_done[g - 1], p->copy_stream));
    }
    if (timed) PF_HIP(c, hipEventRecord(p->stage_timing[1], p->copy_stream));
  }

  // 5. stable sort of the pairs by expert; activations as fp16 rows in
  // operand order, each row scaled by a power of two into the fp16 range
  PF_HIP(c, moe::launch_expert_scatter(p->ids, P, E, p->offsets, p->ccount, p->rank, p->perm, p->inv, s));
  PF_HIP(c, moe::launch_scale_rows(x, T, H, p->x16, p->sig, s));
  PF_HIP(c, hipMemsetAsync(p->range_flag, 0, sizeof(uint32_t), s));

  // 6. per group (a chunk once its copy has landed): the block scales of the
  // group's experts transposed, so each K step of a GEMM reads whole lines of
  // them; then the grouped gate/up and down GEMMs
  bool launched[kMaxGroups][kTimed] = {};
  moe::GemmArgs g{};
  g.a16 = p->x16, g.arow = p->perm, g.arow_div = k;
  g.tiles = p->tiles, g.eaddr = p->eaddr;
  g.K = H, g.N = F;
  g.lay = c->lay;
  g.h16 = p->h16;
  g.sclT = p->sclT;
  g.sclT_per_expert = moe::sclT_elements(c->lay);
  g.perm = p->perm, g.perm_div = k, g.sig = p->sig, g.range_flag = p->range_flag;
  moe::GemmArgs d = g;
  d.a16 = p->h16, d.arow = nullptr, d.arow_div = 1;
  d.K = F, d.N = H;
  d.y = p->ypair;
  for (int gi = 0; gi < G; ++gi) {
    if (gi > 0) PF_HIP(c, hipStreamWaitEvent(s, p->chunk_done[gi - 1], 0));
    if (g_count[gi] == 0) continue;
    auto timer = [&](int kind) {
      moe::Launch l = ls;
      if (timed) {
        l.start = p->timing[2 * (gi * kTimed + kind)], l.stop = p->timing[2 * (gi * kTimed + kind) + 1];
        launched[gi][kind] = true;
      }
      return l;
    };
    PF_HIP(c, moe::launch_transpose_scales(p->eaddr, p->stage + g_first[gi], (int32_t)g_count[gi], c->lay, p->sclT,
                                           timer(0)));
    const int64_t gu0 = item_first[0][gi], gu1 = item_first[0][gi + 1];
    const int64_t dn0 = item_first[1][gi], dn1 = item_first[1][gi + 1];
    g.items = p->items[0] + gu0;
    d.items = p->items[1] + dn0;
    PF_HIP(c, moe::launch_grouped_gemm(g, 0, bm, (int)(gu1 - gu0), timer(1)));
    PF_HIP(c, moe::launch_grouped_gemm(d, 1, bm, (int)(dn1 - dn0), timer(2)));
  }

  // 7. weighted combine in pick order
  PF_HIP(c, moe::launch_combine_pairs(p->ypair, p->inv, p->w, T, k, H, y, (flags & MOE_ACCUMULATE) ? 1 : 0, s));
  PF_HIP(c, hipMemcpyAsync(p->h_range_flag, p->range_flag, sizeof(uint32_t), hipMemcpyDeviceToHost, s));
  PF_HIP(c, hipStreamSynchronize(s));  // the pass is over (it waited for every chunk): the staging blocks are free again
  p->last_layer = layer;
  if (*p->h_range_flag)
    return moe_ctx_fail(c, MOE_E_RANGE,
                        "prefill: a SwiGLU output left the fp16 operand range after the row's power-of-two scaling "
                        "(non-finite activations, or weights too large for the fp16 prompt-pass GEMM); y is not "
                        "valid");

  if (timed) {
    float ms[kTimed] = {};
    for (int gi = 0; gi < G; ++gi)
      for (int kind = 0; kind < kTimed; ++kind) {
        if (!launched[gi][kind]) continue;
        float t = 0;
        PF_HIP(c, hipEventElapsedTime(&t, p->timing[2 * (gi * kTimed + kind)], p->timing[2 * (gi * kTimed + kind) + 1]));
        ms[kind] += t;
      }
    if (n_chunks > 0) {
      float t = 0;
      PF_HIP(c, hipEventElapsedTime(&t, p->stage_timing[0], p->stage_timing[1]));
      c->prof.prefill_stage_ms += t;
    }
    c->prof.prefill_prep_ms += ms[0];
    c->prof.prefill_passes += 1;
    c->prof.prefill_gateup_ms += ms[1];
    c->prof.prefill_down_ms += ms[2];
    c->prof.prefill_pairs += P;
    c->prof.prefill_tiles += n_tiles;
    c->prof.prefill_staged += staged;
  }
  return MOE_OK;
}

// Preheat (the "llama.cpp: fork with multi gpu acceleration ..." README, "How
// it works": after a prompt pass the cache is refilled with the cold experts
// the pass used). The same rule as the policy simulation: the pass's picks
// count as uses at the next token's clock c; resident experts it used are
// stamped c; its cold experts, by pair count (descending, ties: lower id),
// take the lowest free slot, else the slot whose owner has the fewest pass
// picks, then the oldest stamp (ties: highest index), if those picks are
// fewer than the candidate's; at most min(max_experts, S); pending
// admissions are neither candidates nor victims. Their bytes come from the
// staging blocks the pass filled (HBM to HBM), else from pinned memory.
extern "C" int moe_preheat(moe_ctx* c, int32_t layer, int32_t max_experts, int32_t* admitted) {
  if (!c) return MOE_E_INVAL;
  if (admitted) *admitted = 0;
  Prefill* p = c->pf;
  if (!p || p->last_layer < 0) return moe_ctx_fail(c, MOE_E_STATE, "preheat: no prompt pass yet");
  if (layer != p->last_layer)
    return moe_ctx_fail(c, MOE_E_STATE, "preheat: the last prompt pass was of layer %d, not %d", p->last_layer, layer);
  if (capturing(c->stream)) return moe_ctx_fail(c, MOE_E_CAPTURING, "preheat while capturing");
  PF_HIP(c, hipStreamSynchronize(p->copy_stream));  // the staging blocks are read below
  hipStream_t s = c->stream;
  const int64_t E = c->E, S = c->S, GS = (int64_t)c->groups * S, B = c->B;
  const int64_t g0 = c->group_of(layer) * S;
  const uint32_t clk = (uint32_t)c->clock;
  // the device stamps are current (forwards raise them); start from them. The
  // sync also retires any earlier launch still reading the host staging.
  if (S > 0) PF_HIP(c, hipMemcpyAsync(c->h_stamps, c->d_stamps, sizeof(uint32_t) * GS, hipMemcpyDeviceToHost, s));
  PF_HIP(c, hipStreamSynchronize(s));
  if (S > 0) std::memcpy(c->stamps.data(), c->h_stamps, sizeof(uint32_t) * GS);
  const int32_t* cnt = p->h_counts;
  for (int64_t e = 0; e < E; ++e) {
    const int32_t slot = c->tbl[layer * E + e];
    if (cnt[e] > 0 && slot >= 0 && c->stamps[g0 + slot] < clk) c->stamps[g0 + slot] = clk;
  }
  const int64_t limit = std::min<int64_t>(max_experts, S);
  std::vector<int32_t> cand;
  for (int64_t e = 0; e < E; ++e)
    if (cnt[e] > 0 && c->tbl[layer * E + e] < 0 && c->pend[layer * E + e] < 0) cand.push_back((int32_t)e);
  std::stable_sort(cand.begin(), cand.end(), [&](int32_t a, int32_t b) { return cnt[a] > cnt[b]; });
  int32_t n = 0;
  for (size_t i = 0; i < cand.size() && n < limit; ++i) {
    const int64_t e = cand[i], te = layer * E + e;
    int64_t v = -1;
    for (int64_t sl = 0; sl < S; ++sl)
      if (c->owner[g0 + sl] < 0) {
        v = sl;
        break;
      }
    if (v < 0) {
      // victim: the owner with the fewest pass picks (other layers' owners: 0), then the oldest stamp
      int32_t vc = 0;
      for (int64_t sl = 0; sl < S; ++sl) {
        if (c->flip[g0 + sl] >= 0) continue;  // held by a pending admission
        const int32_t o = c->owner[g0 + sl];
        const int32_t oc = o / E == layer ? cnt[o % E] : 0;
        if (v < 0 || oc < vc || (oc == vc && c->stamps[g0 + sl] <= c->stamps[g0 + v])) v = sl, vc = oc;
      }
      if (v < 0 || vc >= cnt[e]) break;  // every owner was used by the pass at least as often
      const int32_t old = c->owner[g0 + v];
      c->tbl[old] = -1;
      c->last_miss[old] = 0;
    }
    c->owner[g0 + v] = (int32_t)te;
    c->tbl[te] = (int32_t)v;
    c->stamps[g0 + v] = clk;
    c->last_miss[te] = 0;
    const uint8_t* src = p->h_eaddr[e];
    const bool staged = src >= c->staging && src < c->staging + c->n_staging * B;
    if (staged)
      PF_HIP(c, hipMemcpyAsync(c->pool + (g0 + v) * B, src, B, hipMemcpyDeviceToDevice, s));
    else
      PF_HIP(c, hipMemcpyAsync(c->pool + (g0 + v) * B, c->host_layers[layer] + e * B, B, hipMemcpyHostToDevice, s));
    ++n;
  }
  // publish: table, stamps, and the last-miss copy the capture decision reads
  std::memcpy(c->h_tbl, c->tbl.data(), sizeof(int32_t) * c->L * E);
  PF_HIP(c, hipMemcpyAsync(c->d_tbl, c->h_tbl, sizeof(int32_t) * c->L * E, hipMemcpyHostToDevice, s));
  if (S > 0) {
    std::memcpy(c->h_stamps, c->stamps.data(), sizeof(uint32_t) * GS);
    PF_HIP(c, hipMemcpyAsync(c->d_stamps, c->h_stamps, sizeof(uint32_t) * GS, hipMemcpyHostToDevice, s));
  }
  if (c->d_last_miss) {
    std::memcpy(c->h_last_miss, c->last_miss.data(), sizeof(uint32_t) * c->L * E);
    PF_HIP(c, hipMemcpyAsync(c->d_last_miss, c->h_last_miss, sizeof(uint32_t) * c->L * E, hipMemcpyHostToDevice, s));
  }
  PF_HIP(c, hipStreamSynchronize(s));  // the staging blocks may be reused by the next pass
  if (admitted) *admitted = n;
  return MOE_OK;
}
