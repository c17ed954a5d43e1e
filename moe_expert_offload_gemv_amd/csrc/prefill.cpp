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
  int32_t* offsets = nullptr;   // [E + 1]
  int4* tiles = nullptr;        // [max_tiles]
  int2* items[2] = {nullptr, nullptr};    // [max_items] work lists of the gate/up and down GEMMs
  const uint8_t** eaddr = nullptr;  // [E]
  int32_t* stage = nullptr;     // [E] experts copied into the staging blocks, in block order
  _Float16* x16 = nullptr;      // [T][H] activations, fp16 in operand order
  _Float16* h16 = nullptr;      // [P][F] SwiGLU outputs, fp16 in operand order
  float* ypair = nullptr;       // [P][H]
  uint16_t* sclT = nullptr;     // [E][sclT_elements]: the pass's block scales, transposed
  // pinned staging of the small transfers
  int32_t* h_counts = nullptr;
  int32_t* h_offsets = nullptr;
  int4* h_tiles = nullptr;
  int2* h_items[2] = {nullptr, nullptr};
  const uint8_t** h_eaddr = nullptr;
  int32_t* h_stage = nullptr;
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
      (rc = dev((void**)&p->offsets, sizeof(int32_t) * (E + 1), "prefill offsets")) ||
      (rc = dev((void**)&p->tiles, sizeof(int4) * p->max_tiles, "prefill tiles")) ||
      (rc = dev((void**)&p->items[0], sizeof(int2) * p->max_items, "prefill gate/up work list")) ||
      (rc = dev((void**)&p->items[1], sizeof(int2) * p->max_items, "prefill down work list")) ||
      (rc = dev((void**)&p->eaddr, sizeof(uint8_t*) * E, "prefill addresses")) ||
      (rc = dev((void**)&p->stage, sizeof(int32_t) * E, "prefill staging list")) ||
      (rc = dev((void**)&p->x16, sizeof(_Float16) * T * c->H, "prefill x fp16")) ||
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
      (rc = moe_ctx_host_alloc(c, (void**)&p->h_stage, sizeof(int32_t) * E, pin, "prefill staging list")))
    return rc;
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
  delete c->pf;
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
  PF_HIP(c, hipMemsetAsync(p->counts, 0, sizeof(int32_t) * E, s));
  PF_HIP(c, moe::launch_expert_histogram(p->ids, P, E, p->counts, s));
  PF_HIP(c, hipMemcpyAsync(p->h_counts, p->counts, sizeof(int32_t) * E, hipMemcpyDeviceToHost, s));
  PF_HIP(c, hipStreamSynchronize(s));

  // 3. offsets, tiles of the used experts, and where each expert is read from
  int64_t n_tiles = 0, staged = 0, pos = 0;
  const int64_t S = c->S;
  const int bm = tile_rows(p->h_counts, E);
  for (int32_t e = 0; e < E; ++e) {
    const int32_t m = p->h_counts[e];
    p->h_offsets[e] = (int32_t)pos;
    p->h_eaddr[e] = nullptr;
    if (m > 0) {
      const int32_t slot = c->tbl[(int64_t)layer * E + e];
      if (slot >= 0) {
        p->h_eaddr[e] = c->pool + (c->group_of(layer) * S + slot) * c->B;
      } else if (staged < c->n_staging) {
        p->h_eaddr[e] = c->staging + staged * c->B;
        p->h_stage[staged++] = e;
      } else {
        p->h_eaddr[e] = c->host_layers_dev[layer] + (int64_t)e * c->B;  // no block left: read zero-copy
      }
      for (int32_t m0 = 0; m0 < m; m0 += bm) p->h_tiles[n_tiles++] = int4{e, (int32_t)(pos + m0), std::min(bm, m - m0), 0};
    }
    pos += m;
  }
  p->h_offsets[E] = (int32_t)pos;
  c->last_prefill_staged = staged;
  if (pos != P) return moe_ctx_fail(c, MOE_E_HIP, "prefill: pair count mismatch (%lld != %d)", (long long)pos, P);
  if (staged > 0) {
    PF_HIP(c, hipMemcpyAsync(p->stage, p->h_stage, sizeof(int32_t) * staged, hipMemcpyHostToDevice, s));
    PF_HIP(c, moe::launch_stage_experts(c->host_layers_dev[layer], p->stage, (int32_t)staged, c->B, c->staging, s));
  }
  PF_HIP(c, hipMemcpyAsync(p->offsets, p->h_offsets, sizeof(int32_t) * (E + 1), hipMemcpyHostToDevice, s));
  PF_HIP(c, hipMemcpyAsync(p->tiles, p->h_tiles, sizeof(int4) * n_tiles, hipMemcpyHostToDevice, s));
  // work lists: per expert, feature tiles outer and row tiles inner
  int n_items[2] = {0, 0};
  for (int mode = 0; mode < 2; ++mode) {
    const int N = mode == 0 ? F : H, bnw = moe::gemm_features_per_tile(mode, bm);
    if (n_tiles * ((N + bnw - 1) / bnw) > p->max_items)
      return moe_ctx_fail(c, MOE_E_HIP, "prefill: work list larger than its buffer");
    int2* it = p->h_items[mode];
    for (int64_t t0 = 0; t0 < n_tiles;) {
      int64_t t1 = t0;
      while (t1 < n_tiles && p->h_tiles[t1].x == p->h_tiles[t0].x) ++t1;
      for (int n0 = 0; n0 < N; n0 += bnw)
        for (int64_t t = t0; t < t1; ++t) it[n_items[mode]++] = int2{(int32_t)t, n0};
      t0 = t1;
    }
    PF_HIP(c, hipMemcpyAsync(p->items[mode], it, sizeof(int2) * n_items[mode], hipMemcpyHostToDevice, s));
  }
  PF_HIP(c, hipMemcpyAsync(p->eaddr, p->h_eaddr, sizeof(uint8_t*) * E, hipMemcpyHostToDevice, s));

  // 4. short tiles (few rows per expert) are bound by weight fetches: give
  // their GEMMs the block scales of the used experts transposed, so each
  // K step reads whole lines of them
  const bool tscl = bm == 64;
  hipEvent_t* ev = nullptr;
  if (c->profiling && c->prefill_events.size() >= 6) ev = c->prefill_events.data();
  if (tscl) {
    moe::Launch lt;
    lt.stream = s;
    if (ev) lt.start = ev[4], lt.stop = ev[5];
    PF_HIP(c, moe::launch_transpose_scales(p->eaddr, E, c->lay, p->sclT, lt));
  }

  // stable sort of the pairs by expert
  PF_HIP(c, moe::launch_expert_scatter(p->ids, P, E, p->offsets, p->perm, p->inv, s));

  // 5. activations as fp16 rows in operand order
  PF_HIP(c, moe::launch_convert_rows(x, T, H, p->x16, s));

  // 6. grouped GEMMs over the used tiles
  moe::GemmArgs g{};
  g.a16 = p->x16, g.arow = p->perm, g.arow_div = k;
  g.tiles = p->tiles, g.eaddr = p->eaddr, g.items = p->items[0];
  g.K = H, g.N = F;
  g.lay = c->lay;
  g.h16 = p->h16;
  g.sclT = tscl ? p->sclT : nullptr;
  g.sclT_per_expert = moe::sclT_elements(c->lay);
  moe::Launch l1 = ls, l2 = ls;
  if (ev) l1.start = ev[0], l1.stop = ev[1], l2.start = ev[2], l2.stop = ev[3];
  PF_HIP(c, moe::launch_grouped_gemm(g, 0, bm, n_items[0], l1));
  moe::GemmArgs d = g;
  d.a16 = p->h16, d.arow = nullptr, d.arow_div = 1;
  d.K = F, d.N = H;
  d.items = p->items[1];
  d.y = p->ypair;
  PF_HIP(c, moe::launch_grouped_gemm(d, 1, bm, n_items[1], l2));

  // 7. weighted combine in pick order
  PF_HIP(c, moe::launch_combine_pairs(p->ypair, p->inv, p->w, T, k, H, y, (flags & MOE_ACCUMULATE) ? 1 : 0, s));
  PF_HIP(c, hipStreamSynchronize(s));  // the pass is over: the staging blocks are free again
  p->last_layer = layer;

  if (ev) {
    float t1 = 0, t2 = 0, t0 = 0;
    PF_HIP(c, hipEventElapsedTime(&t1, ev[0], ev[1]));
    PF_HIP(c, hipEventElapsedTime(&t2, ev[2], ev[3]));
    if (tscl) PF_HIP(c, hipEventElapsedTime(&t0, ev[4], ev[5]));
    c->prof.prefill_prep_ms += t0;
    c->prof.prefill_passes += 1;
    c->prof.prefill_gateup_ms += t1;
    c->prof.prefill_down_ms += t2;
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
  hipStream_t s = c->stream;
  const int64_t E = c->E, S = c->S, GS = (int64_t)c->groups * S, B = c->B;
  const int64_t g0 = c->group_of(layer) * S;
  const uint32_t clk = (uint32_t)c->clock;
  // the device stamps are current (forwards raise them); start from them
  if (S > 0) {
    PF_HIP(c, hipMemcpyAsync(c->h_stamps, c->d_stamps, sizeof(uint32_t) * GS, hipMemcpyDeviceToHost, s));
    PF_HIP(c, hipStreamSynchronize(s));
    std::memcpy(c->stamps.data(), c->h_stamps, sizeof(uint32_t) * GS);
  }
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
