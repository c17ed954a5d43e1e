/*
 * moe_offload.h - C ABI of libmoe_offload.so, the routed-expert MoE mat-mul
 * (MUL_MAT_ID) over 4-bit block-quantised expert weights for one MI355X
 * (gfx950), with hot experts in an HBM pool and cold experts read zero-copy
 * from pinned host RAM.
 *
 * Sources for what each call computes (page titles as published):
 *  [A6000]  "a6000-custom-kernels" README (Zapdev-labs): the pointer-table
 *           GEMV diagram and the paragraph under it (one table, pool and stamp
 *           array per expert tensor; miss recorder packing tensor_id<<12|expert;
 *           promotion between decode steps on the 2nd sighting; eviction by
 *           stamp scan; pools seeded from a routing-frequency file; capacity from
 *           free memory minus a safety margin), and the "-lm none" section
 *           (cold experts must sit in pinned host buffers to be read zero-copy).
 *  [FORK]   "llama.cpp: fork with multi gpu acceleration even for models bigger
 *           than total gpu mem" README, "How it works": admission after repeated
 *           use within the last 64 tokens; prompt passes stream the experts the
 *           GPU does not hold and return the borrowed blocks afterwards.
 *  [MAC]    "llama.cpp - very large MoE models on a 64 GB Mac" README, "Metal
 *           kernels": MUL_MAT_ID over used (expert, tile) pairs only.
 *
 * Conventions for every function:
 *  - Returns MOE_OK (0) or a negative MOE_E_* code. Nothing aborts, throws or
 *    prints. moe_last_error(ctx) returns a NUL-terminated message for the last
 *    failing call on ctx; the string is owned by ctx and valid until the next
 *    call on ctx.
 *  - "host" pointers are ordinary CPU pointers; "device" pointers are HIP
 *    device addresses on the context's device (for example torch.Tensor
 *    data_ptr() of a cuda tensor). The library never frees caller memory.
 *  - The library owns the HBM pool, the pinned host arena, the slot tables,
 *    stamps, the miss log and all scratch; they live until moe_destroy.
 *  - A context is used by one host thread at a time; calls are not re-entrant.
 *  - Device work is issued on the context stream (moe_config.stream; NULL is
 *    the device's null stream) in call order.
 *
 * Weight format (MOE_Q4_32_F16): each matrix row is a run of 18-byte blocks
 * along the reduction axis; a block is a little-endian IEEE fp16 scale d
 * followed by 16 bytes qs; element j (0..15) of the block is qs[j] & 0xF and
 * element j+16 is qs[j] >> 4; the weight is d * (q - 8). This is the Q4_0
 * layout that [A6000] lists among its dot kernels, with the public GGUF nibble
 * order. gate and up are [ffn][hidden] (blocks along hidden), down is
 * [hidden][ffn] (blocks along ffn). hidden and ffn must be multiples of 32.
 */
#ifndef MOE_OFFLOAD_H
#define MOE_OFFLOAD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#define MOE_OK            0
#define MOE_E_INVAL      (-1) /* bad argument, shape or call order          */
#define MOE_E_NOMEM      (-2) /* HBM or pinned host allocation failed        */
#define MOE_E_HIP        (-3) /* a HIP runtime call failed                   */
#define MOE_E_STATE      (-4) /* call not allowed in the current state       */
#define MOE_E_CAPTURING  (-5) /* call not allowed while the stream captures  */
#define MOE_E_RANGE      (-6) /* moe_prefill: a value left the range of the
                                 prompt pass's fp16 operands                 */

#define MOE_Q4_32_F16     1   /* the only weight format */

#define MOE_ACCUMULATE    1u  /* moe_forward / moe_prefill: y += result      */

#define MOE_MAX_SWAP_LEAD 8   /* largest moe_config.swap_lead                 */

#define MOE_STATIC_SCRATCH_BYTES 16777216 /* moe_forward_static_scratch's array */

/* Where the cold picks of a decode forward are computed (moe_config.cold_exec). */
#define MOE_COLD_GPU      0   /* the GPU reads the pinned weights zero-copy  */
#define MOE_COLD_CPU      1   /* host threads compute them beside the GPU    */

/* Pinned host arena flavour (moe_config.host_alloc). */
#define MOE_HOST_COHERENT     0 /* hipHostMalloc default: fine-grained      */
#define MOE_HOST_NONCOHERENT  1 /* hipHostMallocNonCoherent: GPU may cache  */

/* Pool partition (moe_config.pool_mode). */
#define MOE_POOL_PER_LAYER    0 /* S slots for each layer                     */
#define MOE_POOL_GLOBAL       1 /* one pool of S slots all layers draw from
                                   ([FORK] "How it works": one global pool of
                                   expert blocks instead of a fixed reserve per
                                   layer); the victim is the pool's lowest free
                                   slot, else its smallest stamp              */

typedef struct moe_ctx moe_ctx;

typedef struct {
  int32_t n_layers;        /* L, 1..2^19 (the miss log keeps l in 19 bits)    */
  int32_t n_experts;       /* E, 1..4096 (the miss log keeps e in 12 bits)    */
  int32_t top_k;           /* k, 1..min(E, 32)                                */
  int32_t hidden;          /* H, multiple of 32                               */
  int32_t ffn;             /* F, multiple of 32                               */
  int32_t quant;           /* MOE_Q4_32_F16                                   */
  int64_t pool_budget_bytes; /* >= 0: HBM pool budget; < 0: free HBM at the
                                time the pool is sized minus reserve_bytes
                                ([A6000]: capacity from free memory minus a
                                safety margin). With both a budget >= 0 and
                                reserve_bytes > 0 the budget is the smaller
                                of the two (a cap on the pool after a
                                reservation). Slots per layer
                                S = min(E, budget / (L * expert_bytes)); with
                                MOE_POOL_GLOBAL, slots of the one pool
                                S = min(L * E, budget / expert_bytes). The
                                small device state and the capture blocks are
                                allocated before the pool is sized.          */
  int64_t reserve_bytes;   /* >= 0: HBM left free for other users (KV cache,
                              dense weights) when the budget comes from free
                              memory; 0 with an explicit budget: no cap      */
  int32_t window_tokens;   /* admission window in tokens (64 in [FORK])       */
  int32_t admit_misses;    /* 2: admit on the 2nd miss inside the window
                              ([A6000] "2nd sighting"); 1: admit every miss  */
  int32_t max_batch_tokens;   /* largest T for moe_forward, 1..256            */
  int32_t max_prefill_tokens; /* largest T for moe_prefill (0: no prefill);
                                 T * top_k at most 2^26 pairs               */
  int32_t device;          /* HIP device ordinal                              */
  int32_t host_alloc;      /* MOE_HOST_COHERENT or MOE_HOST_NONCOHERENT       */
  int32_t host_sets;       /* distinct pinned expert sets, 1..L (0: L). Layer
                              l reads its cold experts from set l % host_sets,
                              so layers that share a set share host weights
                              (their HBM pools stay separate). Bounds the
                              pinned arena where host memory is short.       */
  void*   stream;          /* hipStream_t to issue on; NULL: the null stream  */
  int32_t capture_picks;   /* 0..max_batch_tokens*top_k (0: off). A cold pick
                              p < capture_picks of a layer (p = token * k +
                              pick) that the cache step will admit (judged
                              from the last-miss clocks the step began with)
                              also writes the weight bytes it reads over PCIe
                              into an HBM capture block (L * capture_picks
                              blocks of expert_bytes, allocated before the
                              pool). When the cache step admits that expert,
                              the promotion copies from the capture block
                              (HBM to HBM) instead of from pinned memory.
                              Same bytes, same decisions; applies to forwards
                              that route inside the gate/up GEMV (logits
                              given, E <= 512). Batches of 8 tokens or more
                              on the grouped matrix-core path instead stage
                              each cold expert group g < capture_picks into
                              block g (its weights cross PCIe once, in long
                              contiguous reads, before its products), so its
                              promotion copies that block too. A directory
                              names the expert and clock of each block's
                              last writer. Other forwards copy from pinned. */
  int32_t pool_mode;       /* MOE_POOL_PER_LAYER (0) or MOE_POOL_GLOBAL       */
  int32_t swaps_per_step;  /* >= 0: admissions allowed per cache step (0: no
                              limit); see moe_cache_step ([FORK] "Run": the
                              swaps-per-step key)                            */
  int32_t swap_lead;       /* 0..MOE_MAX_SWAP_LEAD: cache steps an admission
                              waits before its table entry flips (0: at once;
                              [FORK] "Run": the swap-lead key). With a lead,
                              copies from pinned memory run on a stream of the
                              library's own while the next steps decode     */
  int32_t cold_exec;       /* MOE_COLD_GPU (0) or MOE_COLD_CPU ([FORK] "How
                              it works": the GPU computes the cached experts
                              while the CPU computes the misses, in parallel).
                              With MOE_COLD_CPU, capture_picks must be 0 (no
                              GPU read of cold weights exists to capture),
                              moe_forward needs logits and E <= 512 and is not
                              capturable; see moe_forward                    */
  int32_t cpu_threads;     /* host threads for MOE_COLD_CPU, 0..256 (0: one
                              per CPU the process may run on, but two: one
                              left to the thread that launches the forwards,
                              one to the HIP runtime's completion thread)    */
  int32_t decode_launches; /* launches per layer for decode batches of 1..7
                              tokens (0 or 2: two, gate/up then down +
                              combine; 1: one, where logits are given,
                              E <= 512, top-k <= 8 and hidden/ffn is
                              2048/1024, 4096/1536 or 256/512: the down
                              work-groups issue their weight loads at once
                              and wait on device counters for h). Same
                              picks, records, decisions and outputs either
                              way (the same sums in the same order:
                              bit-identical). Two is the default: on MI355X
                              the h hand-over inside one launch (coherent
                              stores, a counter, polls, coherent loads
                              across XCDs) cost more than the launch
                              boundary it saves                            */
  int32_t decode_sync_polls; /* bound of a one-launch down work-group's wait
                              for its token's gate/up work-groups, in polls
                              of at least one memory round trip (0: 2^20,
                              about half a second). Past it the work-group
                              sets a flag, goes on, and the next
                              moe_cache_step returns MOE_E_HIP             */
} moe_config;

typedef struct {
  int64_t slots_per_layer;    /* S: slots of the pool a layer draws from (with
                                 MOE_POOL_GLOBAL the one pool all share)      */
  int64_t expert_bytes;       /* bytes of gate+up+down of one expert          */
  int64_t pool_bytes;         /* HBM pool size: L (or 1) * S * expert_bytes   */
  int64_t host_bytes;         /* pinned arena size, host_sets*E*expert_bytes  */
  int64_t staging_experts;    /* HBM blocks lent to a prefill pass            */
  int64_t clock;              /* token clock of the next step (starts at 1)   */
  int64_t steps;              /* cache steps run since the last seed          */
  int64_t host_threads;       /* threads computing cold picks (0: GPU does)   */
  int64_t host_isa;           /* their dot products: 0 none, 1 scalar C++,
                                 2 AVX2+FMA+F16C, 3 AVX-512                    */
  int64_t pool_budget_bytes;  /* the budget S was sized from (after the rule
                                 of moe_config.pool_budget_bytes)             */
  int64_t free_bytes_at_sizing; /* free HBM when the pool was sized (-1: not
                                 queried: explicit budget, no reserve)        */
} moe_info;

typedef struct {
  int64_t step;               /* index of the step just closed (0-based)      */
  int64_t tokens;             /* tokens in that step (clock advance)          */
  int64_t hits;               /* picks served from the HBM pool               */
  int64_t misses;             /* picks served from pinned host (log entries)  */
  int64_t admissions;         /* experts promoted into the pool               */
  int64_t evictions;          /* resident experts displaced by admissions     */
  int64_t hot_bytes;          /* expert bytes read from HBM by the step       */
  int64_t cold_bytes;         /* expert bytes read over PCIe by the step      */
  int64_t copied_bytes;       /* promotion copies into pool slots issued      */
  int64_t copied_pcie_bytes;  /* the part copied from pinned host memory (the
                                 rest came from capture blocks in HBM)        */
  int64_t distinct_experts;   /* distinct (layer, expert) pairs the step read:
                                 the expert bytes a step must move at least
                                 are distinct_experts * expert_bytes (several
                                 tokens of a batch picking one expert share
                                 its read)                                    */
  int64_t distinct_cold_experts; /* of those, the ones read over PCIe          */
} moe_step_stats;

typedef struct {
  int64_t forwards;           /* moe_forward calls timed                      */
  double  route_ms;           /* summed durations: routing + lookup kernel    */
  double  hot_gateup_ms;      /* gate/up GEMV + SwiGLU of the hot picks (HBM) */
  double  hot_down_ms;        /* down GEMV of the hot picks (HBM)             */
  double  cold_gateup_ms;     /* gate/up GEMV + SwiGLU of the cold picks (PCIe) */
  double  cold_down_ms;       /* down GEMV of the cold picks + combine        */
  int64_t hot_picks;          /* picks the timed forwards served from HBM     */
  int64_t cold_picks;         /* picks they served over PCIe                  */
  int64_t gateup_bytes_per_pick; /* expert bytes of gate + up                 */
  int64_t down_bytes_per_pick;   /* expert bytes of down                      */
  int64_t prefill_passes;     /* moe_prefill calls timed                      */
  double  prefill_gateup_ms;  /* grouped gate/up GEMM (+ SwiGLU)              */
  double  prefill_down_ms;    /* grouped down GEMM                            */
  int64_t prefill_pairs;      /* (token, pick) pairs the timed passes computed */
  int64_t prefill_tiles;      /* (expert, row tile) pairs launched            */
  int64_t prefill_staged;     /* experts copied into borrowed staging blocks  */
  double  prefill_prep_ms;    /* block-scale transposition before the GEMMs
                                 (passes of short tiles only)                 */
  double  prefill_stage_ms;   /* the staging copy (gather kernels or DMA),
                                 start of its first chunk to end of its last  */
  /* cold_exec = MOE_COLD_CPU: the host threads, counted whether or not kernel
     timing is on, since the last moe_profile with enable 0 or 1 (hand-offs
     still in flight are counted once answered)                             */
  int64_t host_forwards;      /* hand-offs answered                           */
  int64_t host_expert_passes; /* distinct cold experts computed (per forward) */
  int64_t host_picks;         /* cold picks computed                          */
  double  host_wait_ms;       /* from taking a hand-off to seeing all picks   */
  double  host_compute_ms;    /* computing the cold picks and answering       */
  /* forwards run as one launch per layer (decode_launches 1): timed as a hot
     launch (routing, gate/up and down of the hot picks) and a cold launch
     (the cold picks, then the combine of all); the per-kernel fields above
     stay 0 for them                                                        */
  int64_t layer_forwards;     /* timed forwards of one launch per layer       */
  double  hot_layer_ms;       /* summed hot launches                          */
  double  cold_layer_ms;      /* summed cold launches                         */
} moe_profile_stats;

/* Size in bytes of one expert (gate + up + down) in MOE_Q4_32_F16. */
MOE_API int64_t moe_expert_bytes(int32_t hidden, int32_t ffn);

/* Create a context. Allocates the HBM pool (pool_budget_bytes, [A6000]
 * capacity rule), the pinned host arena (host_sets*E experts), prefill
 * staging, the slot tables (all -1), stamps, the miss log and scratch, all
 * once: no call below allocates memory (except moe_register_router). *out is
 * set on success. MOE_E_NOMEM if the pool or the arena cannot be allocated;
 * MOE_E_INVAL on a bad config; moe_last_error(NULL) then tells which. */
MOE_API int moe_create(const moe_config* cfg, moe_ctx** out);

/* Release everything the context owns; waits for its stream. NULL is a no-op. */
MOE_API int moe_destroy(moe_ctx* ctx);

/* Copy one layer's expert weights into its pinned host set (layer %
 * host_sets), repacking them into the device layout. gate, up, down are host
 * pointers to E consecutive matrices each, in the canonical format above
 * (gate/up: E*F*(H/32) blocks, down: E*H*(F/32) blocks). The caller may free
 * them on return. Allowed until moe_seed; MOE_E_STATE afterwards. */
MOE_API int moe_register_layer(moe_ctx* ctx, int32_t layer,
                       const void* gate, const void* up, const void* down);

/* Optional router for one layer: host fp32 [E][H], row e is expert e. With a
 * router, moe_forward and moe_prefill may take logits == NULL, and logits are
 * z_e = fmaf chain over j = 0..H-1 of x_j * W[e][j] in fp32, from 0.          */
MOE_API int moe_register_router(moe_ctx* ctx, int32_t layer, const float* w_router);

/* Seed the pools and reset the cache policy ([A6000]: pools are seeded from a
 * routing-frequency table). freq is host uint32 [L][E] or NULL. Per layer the
 * S experts with the highest count (ties: lower id first) take slots 0..S-1 in
 * that order; with freq == NULL every slot stays free (cold start). Resets
 * stamps to 0, the per-expert last-miss times to 0, the miss log, the counts
 * and the token clock to 1. Requires every host set registered (MOE_E_STATE).
 * Synchronises. */
MOE_API int moe_seed(moe_ctx* ctx, const uint32_t* freq);

/* MoE FFN of one layer for a decode batch of n_tokens (1..max_batch_tokens):
 *   ids, w = top-k softmax routing of logits (device fp32 [T][E], or NULL when
 *            a router is registered): k largest logits, ties to the lower id,
 *            in that order; w = softmax over the k chosen logits;
 *   per pick: the expert is found through the layer's slot table ([A6000]
 *            pointer table): resident -> its HBM slot, its use-stamp raised to
 *            the pick's token clock; else -> zero-copy read of pinned host
 *            memory and a miss (t<<32 | layer<<12 | expert) recorded for the
 *            step's miss log;
 *   h = silu(W_gate x) * (W_up x); y_pick = W_down h;
 *   y[t] (=|+=) sum over picks i = 0..k-1 of w_i * y_pick_i, in pick order.
 * Token t of the batch carries clock c + t where c is the context clock.
 * x, y: device fp32 [T][H]; y may equal x only with MOE_ACCUMULATE (residual
 * update in place). ids (int32 [T][k]) and w (fp32 [T][k]) are optional device
 * outputs. Asynchronous on the context stream; allocates nothing and may be
 * captured into a HIP graph. Call it at most once per layer per step.
 *
 * With cold_exec = MOE_COLD_CPU the cold picks are computed by the library's
 * host threads instead ([FORK] "How it works"): the gate/up launch computes
 * the hot picks and hands every pick (expert, hot/cold) and the token's x
 * to pinned host memory; the host threads compute y_pick of each
 * cold pick (same formulas, fp32, AVX-512 where the host has it) and answer;
 * the last launch waits for the answer (bounded) and forms y in pick order.
 * The policy (records, stamps, misses, counts) is the same as with the GPU
 * reading cold weights. Needs logits and E <= 512 (MOE_E_INVAL otherwise);
 * not capturable (MOE_E_CAPTURING). If the host threads cannot answer within
 * 10 s, y leaves those picks out and the step's moe_cache_step returns
 * MOE_E_HIP. */
MOE_API int moe_forward(moe_ctx* ctx, int32_t layer, int32_t n_tokens,
                const float* x, const float* logits, float* y,
                int32_t* ids, float* w, uint32_t flags);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward as moe_forward, same arguments, results and policy side effects,
 * with its per-call scratch (pick ids, weights, addresses and tags, the h
 * rows, per-pick outputs, the grouping by expert) in a static device array of
 * 16 MiB (MOE_STATIC_SCRATCH_BYTES) instead of the context's buffers. The
 * array is the library's, one per device, from the first moe_create on that
 * device until the process ends; moe_create takes its address. Every call on
 * a device shares that device's array and leaves its contents behind
 * (nothing in it needs to start at zero): calls that overlap on one device,
 * on any streams or contexts, race. A forward needs
 *   256-byte-aligned parts for T*k picks: 41 bytes per pick, 8*F + 4*H bytes
 *   per pick for h (fp32 and split) and the per-pick outputs, and 4*H + 4
 *   bytes per token for the split activations,
 * MOE_E_INVAL if that exceeds the array (for example T = 32, k = 8 at
 * H = 4096, F = 1536 needs 7.9 MB; T = 256 there does not fit). Calls no
 * allocating routine; capturable like moe_forward. */
MOE_API int moe_forward_static_scratch(moe_ctx* ctx, int32_t layer, int32_t n_tokens,
                const float* x, const float* logits, float* y,
                int32_t* ids, float* w, uint32_t flags);

/* Prompt pass of one layer for n_tokens (1..max_prefill_tokens): same result
 * as moe_forward, computed as a grouped GEMM over the tokens sorted by expert
 * ([MAC]: only (expert, tile) pairs that hold tokens are computed). Experts
 * the pass touches that are not resident are copied into borrowed HBM staging
 * blocks for the pass and the blocks are returned at its end ([FORK]). The
 * copy runs on a stream the library owns, beside the GEMMs of the resident
 * experts; the pass waits for it before it returns. The cache policy is
 * untouched: no stamps, no miss log, no counts, no clock. Synchronises the
 * stream; not capturable (MOE_E_CAPTURING).
 * Precision: the GEMMs run on fp16 operands with fp32 accumulation (weights
 * d * (q - 8) rounded once to fp16). Each token's row of x is scaled by a
 * power of two so its largest magnitude lies in [4, 8) before the cast, and
 * the SwiGLU output by the square of that factor; both are undone exactly in
 * fp32. If a scaled SwiGLU output is not finite or exceeds 65504 (non-finite
 * activations, or weights far beyond Q4 scales), the pass returns
 * MOE_E_RANGE and y is not valid. */
MOE_API int moe_prefill(moe_ctx* ctx, int32_t layer, int32_t n_tokens,
                const float* x, const float* logits, float* y, uint32_t flags);

/* Preheat after a prompt pass ([FORK] "How it works": after the pass the
 * cache is refilled with the cold experts the pass used). layer must be the
 * layer of the last moe_prefill (else MOE_E_STATE). The pass's picks count as
 * uses at the clock c of the next token: the layer's resident experts the
 * pass used get stamp c; the experts it used that are not resident, ordered
 * by how many of its pairs picked them (descending; ties: lower id), are
 * admitted into the pool the layer draws from, at most min(max_experts, S),
 * each into the lowest free slot, else the slot whose owner has the smallest
 * (pass picks, stamp) (ties: highest index; owners of other layers count 0
 * picks), provided those picks are fewer than the candidate's; the owner is
 * evicted and forgets its last miss. The new owner's stamp is c and it
 * forgets its last miss. Preheat stops at the first candidate that finds no
 * such slot. Pending admissions (swap_lead) are neither candidates nor
 * victims. Bytes are copied from the staging
 * blocks the pass filled, else from pinned memory. *admitted (may be NULL)
 * receives the number admitted. Synchronises the stream; not capturable. */
MOE_API int moe_preheat(moe_ctx* ctx, int32_t layer, int32_t max_experts, int32_t* admitted);

/* Close the current step ([A6000]: promotion pass between decode steps, never
 * graph-captured). Waits for the stream, reads the miss log, sorts it
 * ascending, and walks it in that order: an entry whose expert became resident
 * earlier in this walk is skipped; otherwise, with admit_misses == 2, the
 * expert is admitted if it missed before at t' with t - t' < window_tokens,
 * else t is remembered as its last miss ([FORK] window + admission). An
 * admitted expert takes the lowest free slot, else the slot with the smallest
 * stamp (ties: highest slot index), whose expert is evicted and forgets its
 * last miss; the new slot's stamp is t, and the expert forgets its last miss.
 * Weights are copied into the slot on the stream (from the expert's capture
 * block when a cold read of this step captured it, see capture_picks; else
 * from pinned memory), tables, stamps and the
 * clock (advanced by the step's token count) are uploaded, and the log is
 * cleared. out may be NULL. MOE_E_CAPTURING if the stream is capturing.
 *
 * Swap budget and lead (the [FORK] "Run" keys swaps-per-step and swap-lead,
 * named there without a definition): with swaps_per_step = n > 0, an entry
 * that would be admitted after n admissions of this step is refused; so is
 * one for which every slot of the pool is held by a pending admission. A
 * refused entry remembers t as its last miss. With swap_lead = d > 0 an
 * admission decided by this call is pending until the call d steps later:
 * the victim is evicted, the slot's owner and stamp t are set now, but the
 * expert's table entry stays -1 (its picks read pinned memory and are
 * recorded as misses, which the walk skips) and the slot cannot be a victim.
 * Its copy from pinned memory starts at once on the library's swap stream;
 * a copy from a capture block runs on the context stream. The call d steps
 * later waits for that step's swap copies, then sets the table entries
 * (after its own walk). */
MOE_API int moe_cache_step(moe_ctx* ctx, moe_step_stats* out);

/* Kernel timing for measurement: enable = 1 turns it on and clears the
 * totals, 0 turns it off, -1 leaves it as is; out (may be NULL) receives the
 * totals accumulated so far. While on, moe_forward launches each of its
 * kernels with start/stop events timed by the dispatch (so it must not be
 * captured: MOE_E_CAPTURING), and moe_cache_step adds their durations and the
 * step's hot and cold pick counts once the stream has drained; moe_prefill
 * times its two grouped GEMMs the same way. */
MOE_API int moe_profile(moe_ctx* ctx, int32_t enable, moe_profile_stats* out);

/* Introspection (host outputs; each synchronises the stream). */
MOE_API int moe_get_info(moe_ctx* ctx, moe_info* out);
/* int32 [E]: slot of each expert of the layer in the pool the layer draws
 * from, -1 when not resident. */
MOE_API int moe_get_slot_table(moe_ctx* ctx, int32_t layer, int32_t* out);
/* uint32 [S]: use-stamps of the slots of the pool the layer draws from
 * (with MOE_POOL_GLOBAL the same S stamps for every layer). */
MOE_API int moe_get_stamps(moe_ctx* ctx, int32_t layer, uint32_t* out);
/* uint64: the miss log of the last closed step, ascending; *n = its length.
 * Writes min(cap, n) entries. */
MOE_API int moe_get_miss_log(moe_ctx* ctx, uint64_t* out, int64_t cap, int64_t* n);
/* uint32 [L][E]: picks per expert since the last seed (moe_forward only). */
MOE_API int moe_get_counts(moe_ctx* ctx, uint32_t* out);

MOE_API const char* moe_last_error(moe_ctx* ctx);  /* ctx NULL: the last failed moe_create of this thread */

/* Measurement aid, outside the MoE path: the read bandwidth a plain
 * streaming kernel (128-bit loads, grid-stride, 8 work-groups per CU)
 * achieves on the current device, the ceiling the GEMVs are compared with
 * beside the spec figures.
 *   ptr != NULL: a device address of `bytes` readable bytes (caller-owned,
 *                e.g. HBM); host_coherent is ignored.
 *   ptr == NULL: the call allocates `bytes` of pinned host memory (mapped;
 *                coherent if host_coherent != 0, else non-coherent), reads
 *                it zero-copy over PCIe and frees it before returning.
 * bytes > 0 and a multiple of 16; reps >= 1 timed launches after one
 * untimed one, on `stream` (a hipStream_t; NULL = the default stream). The
 * call synchronises with the stream. *gbps = bytes * reps / time / 1e9.
 * Returns MOE_E_INVAL on bad arguments, MOE_E_NOMEM when an allocation
 * fails, MOE_E_HIP on a HIP error; there is no context, so no message. */
MOE_API int moe_measure_read_bandwidth(const void* ptr, int64_t bytes, int32_t reps, int32_t host_coherent,
                                       void* stream, double* gbps);

#ifdef __cplusplus
}
#endif
#endif /* MOE_OFFLOAD_H */
