// runtime.h - the context structure shared by the host sources of
// libmoe_offload.so (internal; the public boundary is include/moe_offload.h).
#pragma once
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/moe_offload.h"
#include "host_experts.h"
#include "kernels.h"

// kernels of a forward, in the order of their timing events
enum { kRoute = 0, kHotGateUp, kHotDown, kColdGateUp, kColdDownCombine, kTimedKernels };
// token counters of the one-launch layer kernels (one 64-byte line)
constexpr size_t kLayerSyncBytes = 64;
static_assert(moe::kLayerMaxTokens * sizeof(uint32_t) <= kLayerSyncBytes, "a counter per token");
// bound of a down work-group's wait, in polls of at least a memory round trip
// each (about half a second); a legitimate wait is one gate/up pass, cold
// picks over PCIe included (well under a millisecond)
constexpr uint32_t kLayerMaxPolls = 1u << 20;

struct moe_ctx {
  moe_config cfg{};
  int device = 0;
  int32_t L = 0, E = 0, k = 0, H = 0, F = 0;
  int32_t S = 0;       // slots of one pool
  int64_t budget = 0;          // HBM budget the slots were sized from
  int64_t free_at_sizing = -1; // free HBM when the pool was sized (-1: not queried)
  int32_t groups = 0;  // pools: L (a pool per layer) or 1 (one global pool)
  int64_t group_of(int64_t layer) const { return groups == 1 ? 0 : layer; }
  moe::ExpertLayout lay{};
  int64_t B = 0;
  hipStream_t stream = nullptr;  // caller's stream (nullptr: the null stream)
  bool own_stream = false;

  // device memory
  uint8_t* pool = nullptr;             // [L][S] experts
  int32_t* d_tbl = nullptr;            // [L][E] slot or -1
  uint32_t* d_stamps = nullptr;        // [L][S]
  uint32_t* d_counts = nullptr;        // [L][E]
  uint64_t* d_records = nullptr;       // [L][max_batch*k] pick records of the step
  int64_t rec_stride = 0;              // records per layer
  moe::Ctrl* d_ctrl = nullptr;
  uint8_t** d_host_base = nullptr;     // [L] device addresses of the pinned layers
  uint8_t* d_scratch = nullptr;        // per-forward scratch for max_batch*k picks, carved into sc
  moe::ForwardScratch sc{};
  std::string static_scratch_err;      // why the static scratch's address is unknown, if it is
  int32_t capture_picks = 0;           // picks per layer whose cold reads are captured
  uint8_t* d_capture = nullptr;        // [L][capture_picks] expert blocks
  uint64_t* d_cap_dir = nullptr;       // [L][capture_picks] capture directory: (clock << 32) | expert of
                                       //   the bytes a forward last wrote into each capture block
  uint32_t* d_layer_sync = nullptr;    // token counters of the one-launch layer kernels
  uint32_t* d_last_miss = nullptr;     // [L][E] device copy of last_miss as the step begins
  std::vector<void*> routers;          // per layer fp32 [E][H] or null

  // pinned host memory (host_sets distinct sets; layer l uses set l % host_sets)
  int32_t host_sets = 0;
  std::vector<uint8_t*> host_layers;      // [L] -> E experts in the device layout
  std::vector<uint8_t*> host_layers_dev;  // device addresses of the same
  moe::Ctrl* h_ctrl = nullptr;
  uint64_t* h_records = nullptr;
  uint64_t* h_cap_dir = nullptr;
  uint32_t* h_last_miss = nullptr;
  int32_t* h_tbl = nullptr;
  uint32_t* h_stamps = nullptr;
  // device-side addresses of the same staging (mapped), read by the cache
  // step's copy launch
  const void* h_ctrl_dev = nullptr;
  const void* h_last_miss_dev = nullptr;
  const void* h_tbl_dev = nullptr;
  const void* h_stamps_dev = nullptr;
  void* h_records_dev = nullptr;
  void* h_cap_dir_dev = nullptr;

  // prefill (borrowed staging blocks and per-pass scratch)
  int64_t n_staging = 0;
  uint8_t* staging = nullptr;
  struct Prefill* pf = nullptr;
  int64_t last_prefill_staged = 0;

  // host mirror of the cache state
  std::vector<int32_t> tbl, owner;   // tbl [L][E] slot; owner [groups][S] layer * E + expert or -1
  std::vector<uint32_t> stamps, last_miss;
  std::vector<uint64_t> last_log;
  // swap lead: admissions waiting for their copy (and the copy stream)
  std::vector<int32_t> pend;           // [L][E] slot of a pending admission, or -1
  std::vector<int64_t> flip;           // [groups][S] step whose cache step flips the slot's owner in, or -1
  hipStream_t swap_stream = nullptr;   // copies from pinned memory of pending admissions
  std::vector<hipEvent_t> swap_events; // [swap_lead + 1]: end of a step's swap copies
  std::vector<char> swap_recorded;     // [swap_lead + 1]: the event holds a step's copies
  // cold picks on the host threads (cold_exec CPU): mailbox in pinned memory
  moe_host::Executor* hx = nullptr;
  int32_t hx_threads = 0;
  uint32_t hx_seq = 0;                 // sequence value of the last hand-off
  uint8_t* mbox = nullptr;             // host address
  uint8_t* mbox_dev = nullptr;         // device address of the same
  int64_t mb_off_done = 0, mb_off_seq = 0, mb_off_e = 0, mb_off_kind = 0, mb_off_x = 0, mb_off_y = 0;
  std::vector<int32_t> cap_of;         // [L][E] captured pick of the expert in the step, or -1
  std::vector<uint32_t> seen;          // [L][E] last step (+1) whose records read the expert
  std::vector<int64_t> cap_touched;    // entries of cap_of set in the step
  std::vector<char> registered;        // per host set
  bool seeded = false;
  int64_t clock = 1;
  int64_t steps = 0;

  // kernel timing (moe_profile)
  bool profiling = false;
  std::vector<hipEvent_t> events;      // start/stop per kernel per timed forward
  std::vector<int32_t> timed_tokens;   // n_tokens of each pending timed forward
  std::vector<uint8_t> timed_fused;    // 1: its routing ran inside the gate/up GEMV (no routing interval)
  std::vector<uint8_t> timed_cpu;      // 1: its cold gate/up ran on the host threads (no interval)
  std::vector<uint8_t> timed_grouped;  // 1: grouped by expert (no separate cold gate/up interval)
  std::vector<uint8_t> timed_layer;    // 1: one launch per layer (a hot and a cold launch when timed)
  int32_t timed_pending = 0;
  moe_profile_stats prof{};

  std::vector<void*> dev_allocs, host_allocs;
  std::string err;
};

int moe_ctx_fail(moe_ctx* c, int code, const char* fmt, ...);
int moe_ctx_dev_alloc(moe_ctx* c, void** p, size_t bytes, const char* what);
int moe_ctx_host_alloc(moe_ctx* c, void** p, size_t bytes, unsigned flags, const char* what);

// prefill.cpp
int moe_prefill_alloc(moe_ctx* c);
int moe_prefill_alloc_staging(moe_ctx* c);
void moe_prefill_release(moe_ctx* c);
