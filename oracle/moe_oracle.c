/*
 * moe_oracle.c - TEST INFRASTRUCTURE. A plain, slow, obviously correct CPU
 * reference of what the routed-expert MoE layer with an HBM expert cache
 * computes. Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load it; the GPU library never does, and the two share no source.
 *
 * Floating point is fp64 (accumulation in natural index order, no blocking,
 * no fused multiply-add contraction: built with -ffp-contract=off), except
 * where an fp32 result decides an integer: router logits are the fp32 fmaf
 * chain the GPU also computes, so expert ids can be compared bit for bit.
 *
 * Sources (page titles as published):
 *  [A6000] "a6000-custom-kernels" README (Zapdev-labs): the pointer-table
 *          GEMV diagram and the paragraph below it: per expert tensor a
 *          table, a pool and a stamp array; a miss recorder packing
 *          (tensor_id << 12 | expert); promotion between decode steps of
 *          experts seen missing for the second time; eviction by a scan of
 *          the use-stamps; pools seeded from routing frequencies; the Q4_0
 *          dot kernels in the list of supported formats.
 *  [FORK]  "llama.cpp: fork with multi gpu acceleration even for models
 *          bigger than total gpu mem" README, "How it works", first bullet:
 *          admission only after repeated use within the last 64 tokens.
 *
 * Readings where the pages are silent (each listed with its reason in the
 * design notes): GGUF Q4_0 nibble order; top-k ties go to the lower expert
 * id and picks are listed by descending logit; routing weights are the
 * softmax over the k chosen logits; SwiGLU h = silu(gate) * up; picks are
 * combined in pick order; the miss-log entry is (t << 32 | layer << 12 | e)
 * processed in ascending order; "within the last W tokens" means
 * t - t_prev < W; the victim is a free slot (lowest index) else the
 * smallest stamp with ties to the highest slot index; admission and
 * eviction both clear the expert's remembered miss.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 -> binary64, from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.                   */
ORC_EXPORT double orc_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int exponent = (h >> 10) & 0x1f;
  int fraction = h & 0x3ff;
  double v;
  if (exponent == 0) {
    v = ldexp((double)fraction, -24); /* subnormal: 0.fraction * 2^-14 */
  } else if (exponent == 31) {
    v = fraction ? NAN : INFINITY;
  } else {
    v = ldexp(1024.0 + (double)fraction, exponent - 25); /* 1.fraction * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* One 18-byte Q4 block -> 32 weights: w = d * (q - 8), d the fp16 scale in
 * the first two bytes (little endian), q_j = low nibble of byte 2+j and
 * q_{j+16} = its high nibble.                                               */
ORC_EXPORT void orc_dequant_block(const uint8_t* blk, double* w) {
  double d = orc_half_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
  for (int j = 0; j < 16; ++j) {
    int lo = blk[2 + j] & 0x0f;
    int hi = blk[2 + j] >> 4;
    w[j] = d * (double)(lo - 8);
    w[j + 16] = d * (double)(hi - 8);
  }
}

/* Dequantise a rows x k matrix stored as rows of k/32 blocks. */
ORC_EXPORT void orc_dequant_matrix(const uint8_t* m, int64_t rows, int64_t k, double* out) {
  int64_t nb = k / 32;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b) orc_dequant_block(m + (r * nb + b) * 18, out + r * k + b * 32);
}

/* y = W x for a Q4 matrix W (rows x k): y_r = sum_c W[r][c] x[c], c ascending. */
ORC_EXPORT void orc_q4_matvec(const uint8_t* m, int64_t rows, int64_t k, const double* x, double* y) {
  int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double w[32];
    double acc = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
      orc_dequant_block(m + (r * nb + b) * 18, w);
      for (int j = 0; j < 32; ++j) acc += w[j] * x[b * 32 + j];
    }
    y[r] = acc;
  }
}

/* ------------------------------------------------------------------------ */
/* Router logits of T tokens: z[t][e] = fmaf chain over j = 0..H-1 of
 * x[t][j] * W[e][j], starting from 0, in fp32 (the GPU computes the same
 * chain, so the comparisons that pick experts see identical values).        */
ORC_EXPORT void orc_router_logits(const float* x, const float* w_router, int32_t T, int32_t E, int32_t H,
                                  float* z) {
  for (int32_t t = 0; t < T; ++t)
    for (int32_t e = 0; e < E; ++e) {
      float acc = 0.0f;
      for (int32_t j = 0; j < H; ++j) acc = fmaf(x[(int64_t)t * H + j], w_router[(int64_t)e * H + j], acc);
      z[(int64_t)t * E + e] = acc;
    }
}

/* Top-k softmax routing of one token: the k experts with the largest logits
 * (equal logits: lower id first), listed in that order; weights are the
 * softmax over the k chosen logits.                                          */
ORC_EXPORT void orc_route(const float* z, int32_t E, int32_t k, int32_t* ids, double* w) {
  for (int32_t i = 0; i < k; ++i) {
    int32_t best = -1;
    for (int32_t e = 0; e < E; ++e) {
      int taken = 0;
      for (int32_t p = 0; p < i; ++p) taken |= (ids[p] == e);
      if (taken) continue;
      if (best < 0 || z[e] > z[best]) best = e; /* strict: ties keep the lower id */
    }
    ids[i] = best;
  }
  double zmax = (double)z[ids[0]];
  double s = 0.0;
  for (int32_t i = 0; i < k; ++i) s += exp((double)z[ids[i]] - zmax);
  for (int32_t i = 0; i < k; ++i) w[i] = exp((double)z[ids[i]] - zmax) / s;
}

/* One expert's SwiGLU FFN: h = silu(W_gate x) * (W_up x), y = W_down h,
 * silu(g) = g / (1 + exp(-g)).                                              */
ORC_EXPORT void orc_expert_ffn(const uint8_t* gate, const uint8_t* up, const uint8_t* down, int32_t H, int32_t F,
                               const double* x, double* y) {
  double* g = (double*)malloc(sizeof(double) * F);
  double* u = (double*)malloc(sizeof(double) * F);
  double* h = (double*)malloc(sizeof(double) * F);
  orc_q4_matvec(gate, F, H, x, g);
  orc_q4_matvec(up, F, H, x, u);
  for (int32_t f = 0; f < F; ++f) h[f] = g[f] / (1.0 + exp(-g[f])) * u[f];
  orc_q4_matvec(down, H, F, h, y);
  free(g);
  free(u);
  free(h);
}

/* One MoE layer for T tokens. gate/up/down are per-expert pointers ([E];
 * entries of experts that no token picks may be NULL). logits fp32 [T][E],
 * or NULL with w_router fp32 [E][H] given (then x32, the fp32 input the GPU
 * sees, must be given too, since the router runs in fp32). x fp64 [T][H].
 * Writes y fp64 [T][H] = sum_i w_i * expert_{ids_i}(x), i = 0..k-1 in
 * order, and ids int32 [T][k], w fp64 [T][k]. Returns 0, or -1 when a
 * picked expert has no weights.                                              */
ORC_EXPORT int orc_moe_layer(int32_t T, int32_t E, int32_t k, int32_t H, int32_t F, const uint8_t* const* gate,
                             const uint8_t* const* up, const uint8_t* const* down, const float* logits,
                             const float* w_router, const float* x32, const double* x, double* y, int32_t* ids,
                             double* w) {
  float* z = (float*)malloc(sizeof(float) * E);
  double* ye = (double*)malloc(sizeof(double) * H);
  int rc = 0;
  for (int32_t t = 0; t < T && rc == 0; ++t) {
    if (logits) {
      memcpy(z, logits + (int64_t)t * E, sizeof(float) * E);
    } else {
      orc_router_logits(x32 + (int64_t)t * H, w_router, 1, E, H, z);
    }
    orc_route(z, E, k, ids + (int64_t)t * k, w + (int64_t)t * k);
    double* yt = y + (int64_t)t * H;
    for (int32_t j = 0; j < H; ++j) yt[j] = 0.0;
    for (int32_t i = 0; i < k; ++i) {
      int32_t e = ids[(int64_t)t * k + i];
      if (!gate[e] || !up[e] || !down[e]) {
        rc = -1;
        break;
      }
      orc_expert_ffn(gate[e], up[e], down[e], H, F, x + (int64_t)t * H, ye);
      double wi = w[(int64_t)t * k + i];
      for (int32_t j = 0; j < H; ++j) yt[j] += wi * ye[j];
    }
  }
  free(z);
  free(ye);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Cache policy, simulated step by step.
 *
 * State per layer (one table per layer: the gate, up and down tensors of an
 * expert are routed together, so [A6000]'s three per-tensor tables of a
 * layer would hold the same entries): slot table tbl[e] (slot or -1), slot
 * owner own[s] (expert or -1), use-stamps st[s], last miss time lm[e]
 * (0 = none since the last reset), lifetime pick counts.
 *
 * A step: every forward of a layer looks its picks up in token order; a hit
 * raises the slot's stamp to the token's clock, a miss appends
 * (t << 32 | layer << 12 | e) to the log. Closing the step sorts the log
 * ascending and walks it: an entry whose expert is already resident (admitted
 * earlier in the walk) is skipped; else with admit == 2 the expert is admitted
 * when lm[e] != 0 and t - lm[e] < window, otherwise lm[e] = t; with admit ==
 * 1 every such entry admits. An admission takes the lowest free slot, else the
 * slot with the smallest stamp (ties: highest index), evicting its expert
 * (whose lm is cleared); the new owner's stamp is t and its lm is cleared.
 * The clock then advances by the step's token count.
 *
 * Pool partition: per layer (S slots for each layer, above), or one global
 * pool of S slots shared by all layers (the "llama.cpp: fork with multi gpu
 * acceleration ..." README, "How it works": one global pool of expert blocks
 * instead of a fixed reserve per layer). The rules are the same with the
 * layer's slots replaced by all slots: a slot's owner is a (layer, expert)
 * pair, the victim is the lowest free slot of the pool, else the pool's
 * smallest stamp (ties: highest index), and seeding fills slots 0..S-1 with
 * the (layer, expert) pairs ordered by count (descending; ties: lower layer,
 * then lower expert).
 * Internally both are "groups": L groups of S slots, or 1 group of S slots;
 * own[] holds layer * E + expert.
 *
 * Swap budget and lead (the same README's tuning keys swaps-per-step and
 * swap-lead, whose meaning it leaves open; this is the plain reading):
 *  - budget > 0: at most budget admissions per step. An entry that would be
 *    admitted beyond it is refused; a refused entry (budget spent, or no slot
 *    that can be taken) remembers t as the expert's last miss.
 *  - lead >= 0: the admission decided when step n closes takes effect when
 *    step n + lead closes (lead 0: at once). Until then the expert is pending:
 *    it stays cold (its picks miss and are logged, and the walk skips them),
 *    it owns its slot, and that slot cannot be a victim. Ownership, the stamp
 *    t and the evictee's loss of its slot and last miss happen at the
 *    decision; only the table entry waits. Pending slots flip after the walk
 *    of the step that closes at n + lead.                                   */
typedef struct {
  int32_t L, E, S, k, window, admit;
  int32_t global;     /* 1: one pool of S slots for all layers */
  int32_t groups;     /* L (per layer) or 1 (global) */
  uint32_t clock;
  uint32_t step_tokens;
  int64_t step;
  int32_t* tbl;      /* [L][E] */
  int32_t* own;      /* [groups][S]: layer * E + expert, or -1 */
  uint32_t* st;      /* [groups][S] */
  uint32_t* lm;      /* [L][E] */
  uint32_t* counts;  /* [L][E] */
  uint64_t* log;     /* current step's log */
  int64_t nlog, caplog;
  uint64_t* last_log; /* log of the last closed step, sorted */
  int64_t nlast;
  int64_t hits, misses;
  /* admissions of the last closed step: (layer, expert, slot, evicted layer, evicted expert) */
  int32_t* adm;
  int64_t nadm, capadm;
  int32_t budget, lead; /* swap budget per step (0: none) and lead in steps */
  int32_t* pend;        /* [L][E]: slot of a pending admission, or -1 */
  int64_t* flip;        /* [groups][S]: step at whose close the slot's pending owner flips in, or -1 */
} orc_policy;

/* global != 0: S is the size of the one pool shared by all layers */
ORC_EXPORT orc_policy* orc_policy_new(int32_t L, int32_t E, int32_t S, int32_t k, int32_t window, int32_t admit,
                                      int64_t log_capacity, int32_t global) {
  orc_policy* p = (orc_policy*)calloc(1, sizeof(orc_policy));
  p->L = L, p->E = E, p->S = S, p->k = k, p->window = window, p->admit = admit;
  p->global = global ? 1 : 0;
  p->groups = global ? 1 : L;
  p->tbl = (int32_t*)malloc(sizeof(int32_t) * L * E);
  p->own = (int32_t*)malloc(sizeof(int32_t) * p->groups * (S > 0 ? S : 1));
  p->st = (uint32_t*)calloc((size_t)p->groups * (S > 0 ? S : 1), sizeof(uint32_t));
  p->lm = (uint32_t*)calloc((size_t)L * E, sizeof(uint32_t));
  p->counts = (uint32_t*)calloc((size_t)L * E, sizeof(uint32_t));
  p->caplog = log_capacity;
  p->log = (uint64_t*)malloc(sizeof(uint64_t) * (log_capacity > 0 ? log_capacity : 1));
  p->last_log = (uint64_t*)malloc(sizeof(uint64_t) * (log_capacity > 0 ? log_capacity : 1));
  p->capadm = log_capacity;
  p->adm = (int32_t*)malloc(sizeof(int32_t) * 5 * (log_capacity > 0 ? log_capacity : 1));
  p->pend = (int32_t*)malloc(sizeof(int32_t) * L * E);
  p->flip = (int64_t*)malloc(sizeof(int64_t) * p->groups * (S > 0 ? S : 1));
  for (int64_t i = 0; i < (int64_t)L * E; ++i) p->tbl[i] = -1, p->pend[i] = -1;
  for (int64_t i = 0; i < (int64_t)p->groups * S; ++i) p->own[i] = -1, p->flip[i] = -1;
  p->clock = 1;
  return p;
}

/* Swap budget per step (0: unlimited) and lead in steps (0: at once). */
ORC_EXPORT void orc_policy_set_swaps(orc_policy* p, int32_t budget, int32_t lead) {
  p->budget = budget > 0 ? budget : 0;
  p->lead = lead > 0 ? lead : 0;
}

ORC_EXPORT void orc_policy_free(orc_policy* p) {
  if (!p) return;
  free(p->tbl), free(p->own), free(p->st), free(p->lm), free(p->counts), free(p->log), free(p->last_log);
  free(p->adm), free(p->pend), free(p->flip);
  free(p);
}

/* Seed: per layer, experts ordered by count (descending, ties: lower id)
 * fill slots 0..S-1 (global pool: all (layer, expert) pairs ordered by count,
 * ties: lower layer, then lower id, fill the pool's slots 0..S-1); freq ==
 * NULL leaves every slot free. Resets stamps, last misses, counts and the
 * log; the clock restarts at 1. The selection is a plain repeated scan for
 * the best pair not yet taken.                                              */
ORC_EXPORT void orc_policy_seed(orc_policy* p, const uint32_t* freq) {
  int32_t L = p->L, E = p->E, S = p->S;
  for (int64_t i = 0; i < (int64_t)L * E; ++i) p->tbl[i] = -1, p->lm[i] = 0, p->counts[i] = 0, p->pend[i] = -1;
  for (int64_t i = 0; i < (int64_t)p->groups * S; ++i) p->own[i] = -1, p->st[i] = 0, p->flip[i] = -1;
  if (freq) {
    char* taken = (char*)calloc((size_t)L * E, 1);
    for (int32_t g = 0; g < p->groups; ++g) {
      /* candidates of group g: layer g (per layer) or every layer (global), in (layer, expert) order */
      int64_t lo = p->global ? 0 : (int64_t)g * E, hi = p->global ? (int64_t)L * E : (int64_t)(g + 1) * E;
      int32_t n = S;
      if (n > hi - lo) n = (int32_t)(hi - lo);
      for (int32_t s = 0; s < n; ++s) {
        int64_t best = -1;
        for (int64_t te = lo; te < hi; ++te) {
          if (taken[te]) continue;
          if (best < 0 || freq[te] > freq[best]) best = te;  /* strict: the first (lowest) index wins ties */
        }
        taken[best] = 1;
        p->tbl[best] = s;
        p->own[(int64_t)g * S + s] = (int32_t)best;
      }
    }
    free(taken);
  }
  p->clock = 1;
  p->step = 0;
  p->nlog = 0;
  p->nlast = 0;
  p->nadm = 0;
  p->hits = p->misses = 0;
  p->step_tokens = 0;
}

/* The cache side of one layer's forward over T tokens with routed ids
 * [T][k]. Returns 0, or -1 if the log would overflow.                       */
ORC_EXPORT int orc_policy_forward(orc_policy* p, int32_t layer, int32_t T, const int32_t* ids) {
  for (int32_t t = 0; t < T; ++t) {
    uint32_t clk = p->clock + (uint32_t)t;
    for (int32_t i = 0; i < p->k; ++i) {
      int32_t e = ids[(int64_t)t * p->k + i];
      p->counts[(int64_t)layer * p->E + e] += 1;
      int32_t s = p->tbl[(int64_t)layer * p->E + e];
      if (s >= 0) {
        uint32_t* stamp = &p->st[(int64_t)(p->global ? 0 : layer) * p->S + s];
        if (clk > *stamp) *stamp = clk;
        p->hits += 1;
      } else {
        if (p->nlog >= p->caplog) return -1;
        p->log[p->nlog++] = ((uint64_t)clk << 32) | ((uint64_t)layer << 12) | (uint64_t)e;
        p->misses += 1;
      }
    }
  }
  if ((uint32_t)T > p->step_tokens) p->step_tokens = (uint32_t)T;
  return 0;
}

static int cmp_u64(const void* a, const void* b) {
  uint64_t x = *(const uint64_t*)a, y = *(const uint64_t*)b;
  return (x > y) - (x < y);
}

/* Close the step. Writes [hits, misses, admissions, evictions, tokens] to
 * stats (may be NULL).                                                       */
ORC_EXPORT void orc_policy_step(orc_policy* p, int64_t* stats) {
  int32_t E = p->E, S = p->S;
  qsort(p->log, (size_t)p->nlog, sizeof(uint64_t), cmp_u64);
  int64_t admissions = 0, evictions = 0;
  p->nadm = 0;
  for (int64_t n = 0; n < p->nlog; ++n) {
    uint64_t entry = p->log[n];
    uint32_t t = (uint32_t)(entry >> 32);
    int32_t layer = (int32_t)((entry >> 12) & 0xfffff);
    int32_t e = (int32_t)(entry & 0xfff);
    int64_t te = (int64_t)layer * E + e;
    if (p->tbl[te] >= 0 || p->pend[te] >= 0) continue; /* admitted earlier in this walk, or pending */
    int admit_now;
    if (p->admit == 1) {
      admit_now = 1;
    } else {
      admit_now = p->lm[te] != 0 && (int64_t)t - (int64_t)p->lm[te] < (int64_t)p->window;
      if (!admit_now) p->lm[te] = t;
    }
    if (!admit_now || S == 0) continue;
    /* victim among the slots of the layer's group that no pending admission
     * holds: lowest free slot, else smallest stamp with ties to the highest
     * index */
    const int64_t g0 = (int64_t)(p->global ? 0 : layer) * S;
    int32_t victim = -1;
    for (int32_t s = 0; s < S; ++s)
      if (p->own[g0 + s] < 0) {
        victim = s;
        break;
      }
    if (victim < 0)
      for (int32_t s = 0; s < S; ++s)
        if (p->flip[g0 + s] < 0 && (victim < 0 || p->st[g0 + s] <= p->st[g0 + victim])) victim = s;
    if (victim < 0 || (p->budget > 0 && admissions == p->budget)) {
      p->lm[te] = t; /* refused: remembered as a miss */
      continue;
    }
    int32_t evicted = -1;  /* layer * E + expert of the evicted owner */
    if (p->own[g0 + victim] >= 0) {
      evicted = p->own[g0 + victim];
      p->tbl[evicted] = -1;
      p->lm[evicted] = 0;
      evictions += 1;
    }
    p->own[g0 + victim] = (int32_t)te;
    p->st[g0 + victim] = t;
    p->lm[te] = 0;
    if (p->lead == 0) {
      p->tbl[te] = victim;
    } else {
      p->pend[te] = victim;
      p->flip[g0 + victim] = p->step + p->lead;
    }
    admissions += 1;
    if (p->nadm < p->capadm) {
      int32_t* a = p->adm + 5 * p->nadm++;
      a[0] = layer, a[1] = e, a[2] = victim;
      a[3] = evicted < 0 ? -1 : evicted / E, a[4] = evicted < 0 ? -1 : evicted % E;
    }
  }
  /* pending admissions whose lead ends with this step flip in */
  for (int64_t i = 0; i < (int64_t)p->groups * S; ++i)
    if (p->flip[i] >= 0 && p->flip[i] <= p->step) {
      int32_t te = p->own[i];
      p->tbl[te] = (int32_t)(i % S);
      p->pend[te] = -1;
      p->flip[i] = -1;
    }
  if (stats) {
    stats[0] = p->hits, stats[1] = p->misses, stats[2] = admissions, stats[3] = evictions;
    stats[4] = p->step_tokens;
  }
  memcpy(p->last_log, p->log, sizeof(uint64_t) * (size_t)p->nlog);
  p->nlast = p->nlog;
  p->nlog = 0;
  p->hits = p->misses = 0;
  p->clock += p->step_tokens;
  p->step_tokens = 0;
  p->step += 1;
}

/* Preheat after a prompt pass of one layer (the "llama.cpp: fork with multi
 * gpu acceleration ..." README, "How it works": after the pass the cache is
 * refilled with the experts the pass used that were cold). The pass's picks
 * count as uses at the clock of the next token, c. counts[E] holds the
 * pass's pairs per expert.
 * 1. Every resident expert with count > 0 gets stamp max(stamp, c).
 * 2. Candidates: experts with count > 0 that are not resident, by count
 *    (descending; ties: lower id). Up to min(max_n, S) of them are admitted,
 *    each into the layer's pool's lowest free slot, else the slot whose
 *    owner has the smallest (pass count, stamp) (ties: highest index; an
 *    owner of another layer, in a global pool, has pass count 0) provided
 *    that count is below the candidate's; the owner is evicted (table entry
 *    and last miss cleared). The new owner's stamp is c and its last miss is
 *    cleared. Preheat stops at the first candidate that finds no such slot:
 *    an expert the pass used is only displaced by one it used more. Pending
 *    admissions (swap lead) are neither candidates nor victims.
 * Returns the number admitted; out (may be NULL) receives the admission
 * records as in the cache step.                                             */
ORC_EXPORT int32_t orc_policy_preheat(orc_policy* p, int32_t layer, const uint32_t* counts, int32_t max_n,
                                      int32_t* out) {
  int32_t E = p->E, S = p->S;
  const uint32_t c = p->clock;
  const int64_t g0 = (int64_t)(p->global ? 0 : layer) * S;
  for (int32_t e = 0; e < E; ++e) {
    int32_t s = p->tbl[(int64_t)layer * E + e];
    if (counts[e] > 0 && s >= 0 && p->st[g0 + s] < c) p->st[g0 + s] = c;
  }
  int32_t limit = max_n < S ? max_n : S;
  if (limit <= 0) return 0;
  char* done = (char*)calloc((size_t)E, 1);
  int32_t n = 0;
  while (n < limit) {
    int32_t best = -1;  /* the next candidate: largest count, lowest id */
    for (int32_t e = 0; e < E; ++e) {
      const int64_t te = (int64_t)layer * E + e;
      if (done[e] || counts[e] == 0 || p->tbl[te] >= 0 || p->pend[te] >= 0) continue;
      if (best < 0 || counts[e] > counts[best]) best = e;
    }
    if (best < 0) break;
    done[best] = 1;
    int32_t victim = -1, evicted = -1;
    for (int32_t s = 0; s < S; ++s)
      if (p->own[g0 + s] < 0) {
        victim = s;
        break;
      }
    if (victim < 0) {
      uint32_t vc = 0; /* pass count of the victim's owner */
      for (int32_t s = 0; s < S; ++s) {
        if (p->flip[g0 + s] >= 0) continue; /* held by a pending admission */
        int32_t o = p->own[g0 + s];
        uint32_t oc = o / E == layer ? counts[o % E] : 0;
        if (victim < 0 || oc < vc || (oc == vc && p->st[g0 + s] <= p->st[g0 + victim])) victim = s, vc = oc;
      }
      if (victim < 0 || vc >= counts[best]) break; /* every owner was used as much as the candidate */
      evicted = p->own[g0 + victim];
      p->tbl[evicted] = -1;
      p->lm[evicted] = 0;
    }
    const int64_t te = (int64_t)layer * E + best;
    p->own[g0 + victim] = (int32_t)te;
    p->tbl[te] = victim;
    p->st[g0 + victim] = c;
    p->lm[te] = 0;
    if (out) {
      int32_t* a = out + 5 * n;
      a[0] = layer, a[1] = best, a[2] = victim;
      a[3] = evicted < 0 ? -1 : evicted / E, a[4] = evicted < 0 ? -1 : evicted % E;
    }
    ++n;
  }
  free(done);
  return n;
}

/* Accessors (copies into caller buffers). */
ORC_EXPORT void orc_policy_tables(const orc_policy* p, int32_t* tbl, int32_t* own, uint32_t* st, uint32_t* lm) {
  if (tbl) memcpy(tbl, p->tbl, sizeof(int32_t) * p->L * p->E);
  if (own) memcpy(own, p->own, sizeof(int32_t) * p->groups * p->S);
  if (st) memcpy(st, p->st, sizeof(uint32_t) * p->groups * p->S);
  if (lm) memcpy(lm, p->lm, sizeof(uint32_t) * p->L * p->E);
}
ORC_EXPORT int64_t orc_policy_last_log(const orc_policy* p, uint64_t* out, int64_t cap) {
  int64_t n = p->nlast < cap ? p->nlast : cap;
  if (out && n > 0) memcpy(out, p->last_log, sizeof(uint64_t) * (size_t)n);
  return p->nlast;
}
ORC_EXPORT int64_t orc_policy_last_admissions(const orc_policy* p, int32_t* out, int64_t cap) {
  int64_t n = p->nadm < cap ? p->nadm : cap;
  if (out && n > 0) memcpy(out, p->adm, sizeof(int32_t) * 5 * (size_t)n);
  return p->nadm;
}
ORC_EXPORT void orc_policy_counts(const orc_policy* p, uint32_t* out) {
  memcpy(out, p->counts, sizeof(uint32_t) * p->L * p->E);
}
ORC_EXPORT uint32_t orc_policy_clock(const orc_policy* p) { return p->clock; }
