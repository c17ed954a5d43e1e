// kernels.h - host-side launchers of the gfx950 kernels (internal to
// libmoe_offload.so; the public boundary is include/moe_offload.h).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Per-device control words read and written by the kernels. Living in device
// memory, they keep their current values across HIP graph replays.
struct Ctrl {
  uint32_t clock;        // token clock of token 0 of the current step
  uint32_t step_tokens;  // max n_tokens over the forwards of the step
  uint32_t host_fault;   // set when a forward's cold picks got no answer from the host threads
  uint32_t sync_fault;   // set when a one-launch layer kernel's down work-group gave up waiting for h
};

// A pick record: (clock << 32) | hit << 31 | layer << 12 | expert. The miss
// log of a step is its records without the hit bit, in ascending order.
constexpr uint64_t kRecordHit = 1ull << 31;

// Device layout of one expert (gate, up, down; each a nibble plane of
// [rows][k/32][16 B] followed by a scale plane of [rows][k/32] fp16).
struct ExpertLayout {
  int32_t H, F;
  int64_t gate_nib, gate_scl, up_nib, up_scl, down_nib, down_scl, bytes;
  static ExpertLayout make(int32_t H, int32_t F) {
    ExpertLayout l;
    l.H = H, l.F = F;
    int64_t kbh = H / 32, kbf = F / 32;
    l.gate_nib = 0;
    l.gate_scl = l.gate_nib + (int64_t)F * kbh * 16;
    l.up_nib = l.gate_scl + (int64_t)F * kbh * 2;
    l.up_scl = l.up_nib + (int64_t)F * kbh * 16;
    l.down_nib = l.up_scl + (int64_t)F * kbh * 2;
    l.down_scl = l.down_nib + (int64_t)H * kbf * 16;
    l.bytes = l.down_scl + (int64_t)H * kbf * 2;
    return l;
  }
};

// Lane mapping of the GEMVs over a reduction of kb blocks: lpr lanes share a
// row (a power of two, 8..64), each lane owns bpl blocks (1..4).
struct GemvShape {
  int lpr, bpl;
};
bool gemv_shape(int kb, GemvShape* out);

// Tag of a pick: where its expert's weights are read from.
constexpr uint8_t kHot = 0;   // HBM pool slot (or prefill staging)
constexpr uint8_t kCold = 1;  // pinned host memory, zero-copy over PCIe
constexpr uint8_t kCaptured = 2;  // flag on a cold pick: its reads are written to its capture block
// which picks a GEMV launch computes
enum { kAll = 0, kOnlyHot = 1, kOnlyCold = 2 };

// Stream of a launch; with start/stop events the launch is timed by the
// dispatch itself (hipExtLaunchKernelGGL).
struct Launch {
  hipStream_t stream = nullptr;
  hipEvent_t start = nullptr, stop = nullptr;
};

struct RouteArgs {
  const float* logits;   // [T][E] or nullptr (router)
  const float* x;        // [T][H] (router input)
  const float* wr;       // [E][H] router weights of the layer or nullptr
  int32_t T, E, k, H, S, layer;
  const int32_t* tbl;    // [E] slot table row of the layer
  uint32_t* stamps;      // [S] stamps of the layer
  uint32_t* counts;      // [E] pick counts of the layer
  uint64_t* records;     // [T][k] pick records of the layer
  Ctrl* ctrl;
  const uint8_t* pool;   // first slot of the layer
  const uint8_t* host;   // device address of the layer's pinned experts
  int64_t expert_bytes;
  int32_t* ids;          // [T][k] internal
  float* w;              // [T][k] internal
  const uint8_t** addr;  // [T][k] per-pick expert address (nullptr: not written)
  uint8_t* kind;         // [T][k] kHot / kCold
  int32_t* ids_user;     // optional copies for the caller
  float* w_user;
  int32_t policy;        // 1: lookup, stamps, records, counts, step tokens; 0: routing only
                         // (fused with the gate/up GEMV: 0 = lookup without side effects)
  uint8_t* xs;           // route_kernel: also split the tokens' activations x (split_dev.h) into
  int32_t* xsig;         //   xs [T][H/32][128 B] and their exponents xsig [T] (nullptr: no)
  uint64_t* cap_dir;     // [capture_picks] the layer's capture directory: block b holds the expert
                         //   (clock << 32) | e whose bytes a forward wrote into it at that clock
  int32_t capture_picks; // picks p < capture_picks of a layer may capture their cold reads:
  const uint32_t* last_miss;  // [E] the layer's last-miss clocks as the step began; a cold
  int32_t window, admit_misses;  // pick captures when the cache step will admit it from them
  // hand-off to the host threads (cold picks computed on the CPU), device
  // addresses of pinned memory; pub_seq == nullptr: off. An extra work-group
  // per pick p writes pub_e/pub_kind[p] (and the token's x row into pub_x
  // for the first pick of a token), then pub_seq[p] = pub_value.
  uint32_t* pub_seq;
  int32_t* pub_e;
  int32_t* pub_kind;
  float* pub_x;
  uint32_t pub_value;
};
hipError_t launch_route(const RouteArgs& a, const Launch& l);

// Launch on l.stream; timed by the dispatch itself when l carries events.
template <typename... Args, typename... P>
inline hipError_t launch(void (*kern)(Args...), dim3 grid, dim3 block, const Launch& l, P... params) {
  if (l.start)
    hipExtLaunchKernelGGL(kern, grid, block, 0, l.stream, l.start, l.stop, 0, params...);
  else
    hipLaunchKernelGGL(kern, grid, block, 0, l.stream, params...);
  return hipGetLastError();
}

struct GemvArgs {
  const float* x;               // gate/up: activations [T][H]; down: h [P][F]
  const uint8_t* const* addr;   // [P] expert base address per pick
  const uint8_t* kind;          // [P] tag of each pick
  const float* w;               // down: routing weights [P]
  float* out;                   // gate/up: h [P][F]; down+combine: y [T][H]
  float* ypick;                 // [P][H] down output of the picks another launch computed
  int32_t T, k, H, F;
  int32_t accumulate;           // combine: y += result
  ExpertLayout lay;
  uint8_t* capture;             // layer's capture blocks: a cold pick p < capture_picks writes the
  int32_t capture_picks;        //   weight bytes it reads into block p (same layout as a slot);
                                //   grouped decode: cold group g < capture_picks is staged in block g
  uint64_t* cap_dir;            // [capture_picks] the layer's capture directory (see RouteArgs)
  const Ctrl* ctrl;             // the step's token clock (directory entries)
};
hipError_t launch_gemv_gateup(const GemvArgs& a, const Launch& l, int mode);
// routing fused into the gate/up GEMV: needs logits and E <= kFusedRouteMaxExperts
constexpr int kFusedRouteMaxExperts = 512;
hipError_t launch_gemv_route_gateup(const GemvArgs& a, const RouteArgs& r, const Launch& l, int mode);
hipError_t launch_gemv_down_pick(const GemvArgs& a, const Launch& l, int mode);
hipError_t launch_gemv_down_combine(const GemvArgs& a, const Launch& l, int mode);

// Decode batches of kGroupedMinTokens tokens or more: the picks are grouped
// by expert on the device and every expert's weight rows are read once for
// all the tokens that picked it (routing and policy as route_kernel's).
constexpr int kGroupedMinTokens = 8;
constexpr int kMaxGroupsSorted = 1024;  // more groups than this stay in expert order
struct GroupArgs {
  const int32_t* ids;    // [P] expert of each pick
  const int32_t* tbl;    // [E] the layer's slot table (cold experts: -1), as the routing read it
  int32_t P, E;
  int4* groups;          // [P] (expert, first position in order, picks, 0), in expert order
  int32_t* order;        // [P] picks by expert
  int32_t* n_groups;     // [1]
};
hipError_t launch_group_picks(const GroupArgs& a, hipStream_t s);
// grouped gate/up (h [P][F] from x) or down (ypick [P][H] from h): a.x / a.out as in
// GemvArgs, the groups from GroupArgs; then a pick-order combine into y.
hipError_t launch_grouped_gateup(const GemvArgs& a, const GroupArgs& g, const Launch& l);
hipError_t launch_grouped_down(const GemvArgs& a, const GroupArgs& g, const Launch& l);
hipError_t launch_combine_picks(const GemvArgs& a, const Launch& l);

// One launch per layer for decode batches of 1 .. kLayerMaxTokens tokens
// (top-k <= 8, logits given, E <= kFusedRouteMaxExperts): gate/up work-groups
// and down + combine work-groups in one grid, the down ones waiting on a
// per-token counter of finished gate/up work-groups (decode_layer.hip).
constexpr int kLayerMaxTokens = kGroupedMinTokens - 1;
struct LayerArgs {
  float* h;              // [T*k][F] exchange buffer of the h rows
  float* y;              // [T][H] layer output
  int32_t accumulate;    // y += result
  uint32_t* sync;        // [kLayerMaxTokens] token counters: 0 between launches, each launch leaves them 0
  uint32_t max_polls;    // bound of a down work-group's wait; past it ctrl->sync_fault is set
};
// the shapes that have a one-launch instantiation (others take the two-launch path)
bool layer_shape_ok(int H, int F, int k, int T, int E);
// mode kAll: the layer; kOnlyHot: hot picks, y_pick rows of a.ypick, no y;
// kOnlyCold: cold picks, combined with the hot picks' a.ypick rows into y
hipError_t launch_decode_layer(const GemvArgs& a, const RouteArgs& r, const LayerArgs& l, const Launch& ln, int mode);

// Grouped decode on the matrix cores (grouped_mfma.hip), for H and F
// multiples of 128: activation rows split into scaled fp16 hi/lo operands.
struct SplitArgs {
  const uint8_t* x;      // [T][H/32][128 B] split activations
  const int32_t* xsig;   // [T] their exponents (row scaled by 2^xsig)
  const uint8_t* h;      // [P][F/32][128 B] split SwiGLU outputs
  const int32_t* hsig;   // [P]
};
bool mfma_grouped_shape_ok(int32_t H, int32_t F);
// rows fp32 [rows][K] -> dst [rows][K/32][128 B], sig [rows]
hipError_t launch_split_rows(const float* src, int32_t rows, int32_t K, uint8_t* dst, int32_t* sig, hipStream_t s);
// h [P][F] (a.out) from the split x; y_pick [P][H] (a.ypick) from the split h
hipError_t launch_mfma_gateup(const GemvArgs& a, const GroupArgs& g, const SplitArgs& sp, const Launch& l);
hipError_t launch_mfma_down(const GemvArgs& a, const GroupArgs& g, const SplitArgs& sp, const Launch& l);

// Combine when the host threads computed the cold picks: a token with a cold
// pick waits until the low half of *done reaches seq (at most max_polls
// polls; a nonzero high half, or no answer, sets ctrl->host_fault and counts
// its cold picks as zero), then y[t] = (y[t] if accumulate) + sum over the
// picks in order of w[p] * (cold ? y_cold[p] : ypick[p]).
struct HostCombineArgs {
  const float* ypick;     // [P][H] hot picks (device)
  const float* w;         // [P]
  const uint8_t* kind;    // [P]
  const float* y_cold;    // [P][H] cold picks (pinned host memory, device address)
  const uint64_t* done;   // pinned host memory, device address: status << 32 | last answered seq
  uint32_t seq;
  uint32_t max_polls;
  float* y;               // [T][H]
  int32_t T, k, H, accumulate;
  Ctrl* ctrl;
};
hipError_t launch_host_combine(const HostCombineArgs& a, const Launch& l);


// ---------------------------------------------------------------------------
// prompt pass (prefill_kernels.hip)

struct GemmArgs {
  const _Float16* a16;          // A rows [rows][K] fp16 in operand order (scale_rows layout)
  const int32_t* arow;          // gate/up: perm (A row = arow[pos] / arow_div); down: nullptr (A row = pos)
  int32_t arow_div;
  const int4* tiles;            // (expert, first sorted position, rows <= BM, 0)
  const int2* items;            // work list: (tile index, first output feature), a multiple of
                                //   gemm_features_per_tile(mode, bm)
  const uint8_t* const* eaddr;  // [E] device address of each expert for the pass
  int32_t K, N;                 // reduction length, output features (both multiples of 64)
  ExpertLayout lay;
  _Float16* h16;                // gate/up output: h rows [P][N] fp16 in operand order
  float* y;                     // down output: y_pair [P][N]
  const uint16_t* sclT;         // the pass's block scales transposed, expert e at sclT + e *
  int64_t sclT_per_expert;      //   sclT_per_expert: gate [H/32][F], up [H/32][F], down [F/32][H]
  const int32_t* perm;          // [P] sorted position -> pair; token of a pair = pair / perm_div
  int32_t perm_div;
  const int32_t* sig;           // [T] exponent s of each token's row scale 2^s (scale_rows)
  uint32_t* range_flag;         // gate/up: set when a scaled h is not finite or above 65504
  int32_t work, work_padded;    // set by the launcher: work items, padded to a multiple of 8
};
// Stable counting sort of pairs by expert (E <= 4096). launch_expert_counts
// fills rank [n_pairs], ccount [E][sort_chunks(n_pairs)] (chunk starts within
// each expert) and counts [E]; launch_expert_scatter, given the offsets (the
// exclusive prefix of counts), writes perm [n_pairs] (sorted position ->
// pair) and inv (pair -> sorted position).
int32_t sort_chunks(int32_t n_pairs);
hipError_t launch_expert_counts(const int32_t* ids, int32_t n_pairs, int32_t E, int32_t* rank, int32_t* ccount,
                                int32_t* counts, hipStream_t s);
hipError_t launch_expert_scatter(const int32_t* ids, int32_t n_pairs, int32_t E, const int32_t* offsets,
                                 const int32_t* ccount, const int32_t* rank, int32_t* perm, int32_t* inv,
                                 hipStream_t s);
// fp32 rows [rows][K] -> fp16 rows in the GEMM's operand order, row r scaled
// by 2^sig[r] so its largest magnitude lies in [4, 8) (sig written here)
hipError_t launch_scale_rows(const float* src, int64_t rows, int32_t K, _Float16* dst, int32_t* sig, hipStream_t s);
// Scale planes of the experts e = experts[0..n) with eaddr[e] != nullptr,
// transposed into out + e * per_expert (layout of GemmArgs::sclT);
// per_expert = sclT_elements(lay).
int64_t sclT_elements(const ExpertLayout& lay);
hipError_t launch_transpose_scales(const uint8_t* const* eaddr, const int32_t* experts, int32_t n,
                                   const ExpertLayout& lay, uint16_t* out, const Launch& l);
int gemm_features_per_tile(int mode, int bm);
// mode 0 gate/up, 1 down; bm = 64 or 128 rows per tile (the tiles were cut to it);
// a.items holds n_items work items
hipError_t launch_grouped_gemm(GemmArgs a, int mode, int bm, int n_items, const Launch& l);
// staging block i of `staging` (blocks of `bytes`, a multiple of 16) <- expert
// experts[i] of the layer whose pinned weights start at host_layer (the
// device-visible address of the mapped allocation), i < n
hipError_t launch_stage_experts(const uint8_t* host_layer, const int32_t* experts, int32_t n, int64_t bytes,
                               uint8_t* staging, hipStream_t s);
hipError_t launch_combine_pairs(const float* ypair, const int32_t* inv, const float* w, int32_t T, int32_t k,
                                int32_t H, float* y, int32_t accumulate, hipStream_t s);

// Copies of the cache step, one launch: transfer i moves op[i].bytes (a
// multiple of 4, 4-byte aligned ends) from op[i].src to op[i].dst, both
// device-accessible (HBM, or pinned host memory mapped for the device).
struct CopyOp {
  const void* src;
  void* dst;
  int64_t bytes;
};
constexpr int kMaxCopyOps = 16;  // a step's usual promotions and its uploads; more take further launches
struct CopyList {
  CopyOp op[kMaxCopyOps];
  int32_t n;
};
hipError_t launch_copy_list(const CopyList& l, hipStream_t s);

// Per-call scratch of a decode forward: device memory beyond its inputs and
// outputs, carved from one block at 256-byte boundaries for P picks.
struct ForwardScratch {
  int32_t* ids;          // [P] expert of each pick
  float* w;              // [P] routing weight
  const uint8_t** addr;  // [P] expert base address
  uint8_t* kind;         // [P] kHot / kCold (+ kCaptured)
  float* h;              // [P][F] SwiGLU outputs
  float* ypick;          // [P][H] down outputs of picks another launch combines
  int4* groups;          // [P] grouped decode: (expert, start, picks, 0)
  int32_t* order;        // [P] picks by expert
  int32_t* n_groups;     // [1]
  uint8_t* xs;           // [T][H/32][128 B] grouped decode: split activations
  int32_t* xsig;         // [T]
  uint8_t* hs;           // [P][F/32][128 B] split SwiGLU outputs
  int32_t* hsig;         // [P]
};
// scratch of a forward of T tokens with top-k (P = T k picks)
int64_t forward_scratch_bytes(int64_t T, int32_t k, int32_t H, int32_t F);
ForwardScratch forward_scratch_carve(uint8_t* base, int64_t T, int32_t k, int32_t H, int32_t F);

// The forward's scratch in a static device array (scratch.hip), for the
// entry point that allocates nothing. static_scratch_init takes the array's
// address on `device`, which must be current; static_scratch returns it
// (null before init).
constexpr int64_t kStaticScratchBytes = 16ll << 20;
hipError_t static_scratch_init(int device);
uint8_t* static_scratch(int device);

}  // namespace moe
