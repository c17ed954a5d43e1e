// runtime.cpp - the host side of libmoe_offload.so behind include/moe_offload.h:
// context, HBM pool, pinned host arena, registration (repack into the device
// layout), seeding, the decode forward (two kernel launches when the gate/up
// GEMV routes by itself, else three), and the
// between-step cache policy.
//
// The cache policy is the one the "a6000-custom-kernels" README describes
// under its pointer-table GEMV diagram (table, pool and stamp array per
// expert tensor; cold reads logged by a miss recorder; a promotion pass
// between decode steps, outside graph capture, admitting experts seen
// missing a second time and evicting by a scan of the use-stamps; pools
// seeded from routing frequencies; capacity from free memory minus a margin),
// with the admission window of the "llama.cpp: fork with multi gpu
// acceleration ..." README ("How it works": admission only after repeated use
// within the last 64 tokens).
#include <hip/hip_runtime.h>
#include <sched.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "../../include/moe_offload.h"
#include "host_experts.h"
#include "kernels.h"
#include "runtime.h"

using moe::Ctrl;
using moe::ExpertLayout;

// ---------------------------------------------------------------------------
// error plumbing

static thread_local std::string g_create_error;

int moe_ctx_fail(moe_ctx* c, int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  if (c) c->err = buf;
  return code;
}

#define HIP_TRY(ctx, expr)                                                                             \
  do {                                                                                                 \
    hipError_t e_ = (expr);                                                                            \
    if (e_ != hipSuccess) return moe_ctx_fail((ctx), MOE_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

namespace {

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

bool stream_capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) return false;
  return st != hipStreamCaptureStatusNone;
}

unsigned host_threads() {
  unsigned n = std::thread::hardware_concurrency();
  return std::max(1u, std::min(16u, n ? n : 1u));
}

// Repack E experts of one matrix kind from canonical 18-byte blocks into
// the device layout (nibble plane + scale plane per expert) at dst + e*B.
void repack_matrix(const uint8_t* src, int E, int64_t rows, int64_t kb, uint8_t* dst, int64_t expert_bytes,
                   int64_t nib_off, int64_t scl_off) {
  auto work = [&](int e0, int e1) {
    for (int e = e0; e < e1; ++e) {
      const uint8_t* s = src + (int64_t)e * rows * kb * 18;
      uint8_t* nib = dst + (int64_t)e * expert_bytes + nib_off;
      uint8_t* scl = dst + (int64_t)e * expert_bytes + scl_off;
      const int64_t nb = rows * kb;
      for (int64_t b = 0; b < nb; ++b) {
        std::memcpy(scl + 2 * b, s + 18 * b, 2);
        std::memcpy(nib + 16 * b, s + 18 * b + 2, 16);
      }
    }
  };
  unsigned nt = std::min<unsigned>(host_threads(), (unsigned)E);
  if (nt <= 1) {
    work(0, E);
    return;
  }
  std::vector<std::thread> th;
  for (unsigned i = 0; i < nt; ++i) {
    int e0 = (int)((int64_t)E * i / nt), e1 = (int)((int64_t)E * (i + 1) / nt);
    th.emplace_back(work, e0, e1);
  }
  for (auto& t : th) t.join();
}

}  // namespace

// ---------------------------------------------------------------------------

extern "C" int64_t moe_expert_bytes(int32_t hidden, int32_t ffn) {
  if (hidden <= 0 || ffn <= 0 || hidden % 32 || ffn % 32) return -1;
  return ExpertLayout::make(hidden, ffn).bytes;
}

static void ctx_release(moe_ctx* c) {
  if (!c) return;
  DeviceGuard g(c->device);
  (void)hipStreamSynchronize(c->stream);
  // the stream is drained, so every submitted hand-off was answered; stop the
  // host threads before their mailbox goes away
  if (c->hx) moe_host::executor_destroy(c->hx);
  c->hx = nullptr;
  moe_prefill_release(c);  // drains the staging stream before its blocks are freed
  for (void* p : c->dev_allocs) (void)hipFree(p);
  for (void* p : c->host_allocs) (void)hipHostFree(p);
  for (void* r : c->routers)
    if (r) (void)hipFree(r);
  for (hipEvent_t e : c->events) (void)hipEventDestroy(e);
  if (c->swap_stream) {
    (void)hipStreamSynchronize(c->swap_stream);
    (void)hipStreamDestroy(c->swap_stream);
  }
  for (hipEvent_t e : c->swap_events) (void)hipEventDestroy(e);
  delete c;
}

int moe_ctx_dev_alloc(moe_ctx* c, void** p, size_t bytes, const char* what) {
  *p = nullptr;
  if (bytes == 0) return MOE_OK;
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    *p = nullptr;
    return moe_ctx_fail(c, MOE_E_NOMEM, "hipMalloc(%zu) for %s failed: %s", bytes, what, hipGetErrorString(e));
  }
  c->dev_allocs.push_back(*p);
  return MOE_OK;
}

int moe_ctx_host_alloc(moe_ctx* c, void** p, size_t bytes, unsigned flags, const char* what) {
  *p = nullptr;
  if (bytes == 0) return MOE_OK;
  hipError_t e = hipHostMalloc(p, bytes, flags);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    *p = nullptr;
    return moe_ctx_fail(c, MOE_E_NOMEM, "hipHostMalloc(%zu) for %s failed: %s", bytes, what,
                        hipGetErrorString(e));
  }
  c->host_allocs.push_back(*p);
  return MOE_OK;
}

static int host_exec_create(moe_ctx* c);

extern "C" int moe_create(const moe_config* cfg, moe_ctx** out) {
  g_create_error.clear();
  if (!cfg || !out) return g_create_error = "null config or output", MOE_E_INVAL;
  *out = nullptr;
  const moe_config& k = *cfg;
  if (k.host_sets < 0 || k.host_sets > k.n_layers) return g_create_error = "host_sets outside 0..n_layers", MOE_E_INVAL;
  if (k.reserve_bytes < 0) return g_create_error = "reserve_bytes < 0", MOE_E_INVAL;
  if (k.n_layers < 1 || k.n_layers > (1 << 19) || k.n_experts < 1 || k.n_experts > 4096 || k.top_k < 1 || k.top_k > 32 ||
      k.top_k > k.n_experts || k.hidden < 32 || k.ffn < 32 || k.hidden % 32 || k.ffn % 32 ||
      k.quant != MOE_Q4_32_F16 || k.window_tokens < 1 || (k.admit_misses != 1 && k.admit_misses != 2) ||
      k.max_batch_tokens < 1 || k.max_batch_tokens > 256 || k.max_prefill_tokens < 0 ||
      (int64_t)k.max_prefill_tokens * k.top_k > (1 << 26) || k.n_layers > (1 << 20) ||
      k.capture_picks < 0 || k.capture_picks > k.max_batch_tokens * k.top_k ||
      (k.pool_mode != MOE_POOL_PER_LAYER && k.pool_mode != MOE_POOL_GLOBAL) || k.swaps_per_step < 0 ||
      k.swap_lead < 0 || k.swap_lead > MOE_MAX_SWAP_LEAD ||
      (k.cold_exec != MOE_COLD_GPU && k.cold_exec != MOE_COLD_CPU) || k.cpu_threads < 0 || k.cpu_threads > 256 ||
      k.decode_launches < 0 || k.decode_launches > 2 || k.decode_sync_polls < 0 ||
      (k.cold_exec == MOE_COLD_CPU && k.capture_picks != 0) ||
      (k.host_alloc != MOE_HOST_COHERENT && k.host_alloc != MOE_HOST_NONCOHERENT))
    return g_create_error = "config field out of range", MOE_E_INVAL;
  moe::GemvShape s1, s2;
  if (!moe::gemv_shape(k.hidden / 32, &s1) || !moe::gemv_shape(k.ffn / 32, &s2))
    return g_create_error = "hidden/32 and ffn/32 must each be 2^a*b with 2^a >= 8 (capped at 64) and b <= 4",
           MOE_E_INVAL;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || k.device < 0 || k.device >= ndev)
    return g_create_error = "no such HIP device", MOE_E_INVAL;

  moe_ctx* c = new moe_ctx();
  c->cfg = k;
  c->device = k.device;
  c->L = k.n_layers, c->E = k.n_experts, c->k = k.top_k, c->H = k.hidden, c->F = k.ffn;
  c->lay = ExpertLayout::make(k.hidden, k.ffn);
  c->B = c->lay.bytes;
  DeviceGuard g(c->device);

  auto fail = [&](int rc) {
    g_create_error = c->err.empty() ? "a HIP call failed during create" : c->err;
    ctx_release(c);
    return rc;
  };

  c->stream = (hipStream_t)k.stream;  // NULL: the null stream
  c->own_stream = false;

  // small device state first, so the pool sizing sees what is left
  const int64_t L = c->L, E = c->E, K = c->k;
  c->rec_stride = (int64_t)k.max_batch_tokens * K;
  int rc;
  if ((rc = moe_ctx_dev_alloc(c, (void**)&c->d_tbl, sizeof(int32_t) * L * E, "slot tables"))) return fail(rc);
  if ((rc = moe_ctx_dev_alloc(c, (void**)&c->d_counts, sizeof(uint32_t) * L * E, "counts"))) return fail(rc);
  if ((rc = moe_ctx_dev_alloc(c, (void**)&c->d_records, sizeof(uint64_t) * L * c->rec_stride, "pick records")))
    return fail(rc);
  if ((rc = moe_ctx_dev_alloc(c, (void**)&c->d_ctrl, sizeof(Ctrl), "control"))) return fail(rc);
  if ((rc = moe_ctx_dev_alloc(c, (void**)&c->d_layer_sync, kLayerSyncBytes, "layer counters"))) return fail(rc);
  if ((rc = moe_ctx_dev_alloc(c, (void**)&c->d_host_base, sizeof(uint8_t*) * L, "host bases"))) return fail(rc);
  const int64_t P = (int64_t)k.max_batch_tokens * K;
  if ((rc = moe_ctx_dev_alloc(c, (void**)&c->d_scratch,
                              (size_t)moe::forward_scratch_bytes(k.max_batch_tokens, c->k, c->H, c->F),
                              "forward scratch")))
    return fail(rc);
  c->sc = moe::forward_scratch_carve(c->d_scratch, k.max_batch_tokens, c->k, c->H, c->F);
  // the allocation-free forward's static scratch: its address on this device,
  // taken once; without it only moe_forward_static_scratch is unavailable
  if (hipError_t e = moe::static_scratch_init(c->device); e != hipSuccess) {
    (void)hipGetLastError();
    c->static_scratch_err = std::string("hipGetSymbolAddress of the static scratch: ") + hipGetErrorString(e);
  }
  c->capture_picks = k.capture_picks;
  if (c->capture_picks > 0) {
    if ((rc = moe_ctx_dev_alloc(c, (void**)&c->d_capture, (size_t)(L * c->capture_picks * c->B), "capture blocks")))
      return fail(rc);
    if ((rc = moe_ctx_dev_alloc(c, (void**)&c->d_cap_dir, sizeof(uint64_t) * L * c->capture_picks,
                                "capture directory")))
      return fail(rc);
    if ((rc = moe_ctx_dev_alloc(c, (void**)&c->d_last_miss, sizeof(uint32_t) * L * E, "last-miss copy")))
      return fail(rc);
  }
  if ((rc = moe_prefill_alloc(c))) return fail(rc);

  // pinned host staging for the small transfers of the cache step: mapped
  // and coherent, so the step's copy launch reads the uploads in place
  const unsigned pin = hipHostMallocMapped | hipHostMallocCoherent;
  auto dev_view = [&](const void* host, const void** out) {
    void* dp = nullptr;
    if (host && hipHostGetDevicePointer(&dp, const_cast<void*>(host), 0) != hipSuccess)
      return moe_ctx_fail(c, MOE_E_HIP, "hipHostGetDevicePointer failed for cache-step staging");
    *out = dp;
    return (int)MOE_OK;
  };
  if ((rc = moe_ctx_host_alloc(c, (void**)&c->h_ctrl, sizeof(Ctrl), pin, "ctrl staging"))) return fail(rc);
  if ((rc = moe_ctx_host_alloc(c, (void**)&c->h_records, sizeof(uint64_t) * L * c->rec_stride, pin,
                               "record staging")))
    return fail(rc);
  if ((rc = moe_ctx_host_alloc(c, (void**)&c->h_tbl, sizeof(int32_t) * L * E, pin, "table staging")))
    return fail(rc);
  if (c->capture_picks > 0 &&
      ((rc = moe_ctx_host_alloc(c, (void**)&c->h_cap_dir, sizeof(uint64_t) * L * c->capture_picks, pin,
                                "capture directory staging")) ||
       (rc = moe_ctx_host_alloc(c, (void**)&c->h_last_miss, sizeof(uint32_t) * L * E, pin, "last-miss staging"))))
    return fail(rc);
  const void* rec_view = nullptr;
  const void* tag_view = nullptr;
  if ((rc = dev_view(c->h_ctrl, &c->h_ctrl_dev)) || (rc = dev_view(c->h_tbl, &c->h_tbl_dev)) ||
      (rc = dev_view(c->h_last_miss, &c->h_last_miss_dev)) || (rc = dev_view(c->h_records, &rec_view)) ||
      (rc = dev_view(c->h_cap_dir, &tag_view)))
    return fail(rc);
  c->h_records_dev = const_cast<void*>(rec_view);
  c->h_cap_dir_dev = const_cast<void*>(tag_view);

  // HBM pool: S slots per layer, or one pool of S slots for every layer
  // capacity: an explicit budget, or free HBM minus the reserve, or (both
  // given) the smaller of the two: a cap on the pool after a reservation
  int64_t budget = k.pool_budget_bytes;
  if (budget < 0 || k.reserve_bytes > 0) {
    size_t fr = 0, tot = 0;
    if (hipMemGetInfo(&fr, &tot) != hipSuccess) return fail(moe_ctx_fail(c, MOE_E_HIP, "hipMemGetInfo failed"));
    c->free_at_sizing = (int64_t)fr;
    const int64_t avail = std::max<int64_t>(0, (int64_t)fr - k.reserve_bytes);
    budget = budget < 0 ? avail : std::min(budget, avail);
  }
  c->budget = budget;
  c->groups = k.pool_mode == MOE_POOL_GLOBAL ? 1 : (int32_t)L;
  c->S = (int32_t)(k.pool_mode == MOE_POOL_GLOBAL ? std::min<int64_t>(L * E, budget / c->B)
                                                  : std::min<int64_t>(E, budget / (L * c->B)));
  const int64_t S = c->S, G = c->groups;
  if ((rc = moe_ctx_dev_alloc(c, (void**)&c->pool, (size_t)(G * S * c->B), "expert pool"))) return fail(rc);
  if ((rc = moe_prefill_alloc_staging(c))) return fail(rc);
  if ((rc = moe_ctx_dev_alloc(c, (void**)&c->d_stamps, sizeof(uint32_t) * G * std::max<int64_t>(S, 1), "stamps")))
    return fail(rc);
  if ((rc = moe_ctx_host_alloc(c, (void**)&c->h_stamps, sizeof(uint32_t) * G * std::max<int64_t>(S, 1), pin,
                               "stamp staging")) ||
      (rc = dev_view(c->h_stamps, &c->h_stamps_dev)))
    return fail(rc);

  // pinned host arena, one allocation per host set, mapped for zero-copy reads
  const unsigned hflags =
      hipHostMallocMapped | (k.host_alloc == MOE_HOST_NONCOHERENT ? hipHostMallocNonCoherent : hipHostMallocCoherent);
  c->host_sets = k.host_sets ? k.host_sets : c->L;
  std::vector<uint8_t*> set_host(c->host_sets), set_dev(c->host_sets);
  for (int64_t hs = 0; hs < c->host_sets; ++hs) {
    if ((rc = moe_ctx_host_alloc(c, (void**)&set_host[hs], (size_t)(E * c->B), hflags, "pinned experts")))
      return fail(rc);
    void* dp = nullptr;
    if (hipHostGetDevicePointer(&dp, set_host[hs], 0) != hipSuccess)
      return fail(moe_ctx_fail(c, MOE_E_HIP, "hipHostGetDevicePointer failed"));
    set_dev[hs] = (uint8_t*)dp;
  }
  c->host_layers.assign(L, nullptr);
  c->host_layers_dev.assign(L, nullptr);
  for (int64_t l = 0; l < L; ++l) {
    c->host_layers[l] = set_host[l % c->host_sets];
    c->host_layers_dev[l] = set_dev[l % c->host_sets];
  }
  if (hipMemcpy(c->d_host_base, c->host_layers_dev.data(), sizeof(uint8_t*) * L, hipMemcpyHostToDevice) !=
      hipSuccess)
    return fail(MOE_E_HIP);

  c->routers.assign(L, nullptr);
  c->registered.assign(c->host_sets, 0);
  c->tbl.assign(L * E, -1);
  c->owner.assign(G * std::max<int64_t>(S, 1), -1);
  c->stamps.assign(G * std::max<int64_t>(S, 1), 0);
  c->last_miss.assign(L * E, 0);
  c->cap_of.assign(L * E, -1);
  c->seen.assign(L * E, 0u);
  c->pend.assign(L * E, -1);
  c->flip.assign(G * std::max<int64_t>(S, 1), -1);
  if (k.swap_lead > 0) {
    // default priority, like every stream here
    if (hipStreamCreateWithFlags(&c->swap_stream, hipStreamNonBlocking) != hipSuccess) return fail(MOE_E_HIP);
    for (int i = 0; i <= k.swap_lead; ++i) {
      hipEvent_t ev;
      if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) return fail(MOE_E_HIP);
      c->swap_events.push_back(ev);
    }
    c->swap_recorded.assign(k.swap_lead + 1, 0);
  }
  if (k.cold_exec == MOE_COLD_CPU && (rc = host_exec_create(c))) return fail(rc);
  if (c->d_cap_dir && hipMemset(c->d_cap_dir, 0, sizeof(uint64_t) * L * c->capture_picks) != hipSuccess)
    return fail(MOE_E_HIP);
  if (c->d_last_miss && hipMemset(c->d_last_miss, 0, sizeof(uint32_t) * L * E) != hipSuccess) return fail(MOE_E_HIP);
  if (hipMemset(c->d_tbl, 0xff, sizeof(int32_t) * L * E) != hipSuccess) return fail(MOE_E_HIP);
  if (hipMemset(c->d_counts, 0, sizeof(uint32_t) * L * E) != hipSuccess) return fail(MOE_E_HIP);
  if (hipMemset(c->d_records, 0, sizeof(uint64_t) * L * c->rec_stride) != hipSuccess) return fail(MOE_E_HIP);
  if (hipMemset(c->d_stamps, 0, sizeof(uint32_t) * G * std::max<int64_t>(S, 1)) != hipSuccess)
    return fail(MOE_E_HIP);
  Ctrl z{1, 0, 0, 0};
  if (hipMemcpy(c->d_ctrl, &z, sizeof(z), hipMemcpyHostToDevice) != hipSuccess) return fail(MOE_E_HIP);
  // the one-launch layer kernels leave their token counters at 0; they start there
  if (hipMemset(c->d_layer_sync, 0, kLayerSyncBytes) != hipSuccess) return fail(MOE_E_HIP);
  // events for kernel timing: a start/stop pair per kernel of a forward,
  // enough for one step of every layer
  const int64_t n_timed = L + 16;
  c->events.reserve(2 * kTimedKernels * n_timed);
  for (int64_t i = 0; i < 2 * kTimedKernels * n_timed; ++i) {
    hipEvent_t ev;
    // timing only: no system-scope release fence when the event completes
    if (hipEventCreateWithFlags(&ev, hipEventDisableSystemFence) != hipSuccess) return fail(MOE_E_HIP);
    c->events.push_back(ev);
  }
  c->timed_tokens.assign(n_timed, 0);
  c->timed_fused.assign(n_timed, 0);
  c->timed_cpu.assign(n_timed, 0);
  c->timed_grouped.assign(n_timed, 0);
  c->timed_layer.assign(n_timed, 0);
  if (hipDeviceSynchronize() != hipSuccess) return fail(MOE_E_HIP);
  c->clock = 1;
  *out = c;
  return MOE_OK;
}

extern "C" int moe_destroy(moe_ctx* c) {
  ctx_release(c);
  return MOE_OK;
}

extern "C" const char* moe_last_error(moe_ctx* c) { return c ? c->err.c_str() : g_create_error.c_str(); }

extern "C" int moe_register_layer(moe_ctx* c, int32_t layer, const void* gate, const void* up, const void* down) {
  if (!c) return MOE_E_INVAL;
  if (layer < 0 || layer >= c->L || !gate || !up || !down)
    return moe_ctx_fail(c, MOE_E_INVAL, "register_layer: bad layer %d or null weights", layer);
  if (c->seeded) return moe_ctx_fail(c, MOE_E_STATE, "register_layer after moe_seed");
  const int64_t kbh = c->H / 32, kbf = c->F / 32;
  uint8_t* dst = c->host_layers[layer];
  repack_matrix((const uint8_t*)gate, c->E, c->F, kbh, dst, c->B, c->lay.gate_nib, c->lay.gate_scl);
  repack_matrix((const uint8_t*)up, c->E, c->F, kbh, dst, c->B, c->lay.up_nib, c->lay.up_scl);
  repack_matrix((const uint8_t*)down, c->E, c->H, kbf, dst, c->B, c->lay.down_nib, c->lay.down_scl);
  c->registered[layer % c->host_sets] = 1;
  return MOE_OK;
}

extern "C" int moe_register_router(moe_ctx* c, int32_t layer, const float* w) {
  if (!c) return MOE_E_INVAL;
  if (layer < 0 || layer >= c->L || !w) return moe_ctx_fail(c, MOE_E_INVAL, "register_router: bad arguments");
  DeviceGuard g(c->device);
  if (!c->routers[layer]) {
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, sizeof(float) * (size_t)c->E * c->H);
    if (e != hipSuccess) return moe_ctx_fail(c, MOE_E_NOMEM, "router alloc failed");
    c->routers[layer] = p;
  }
  HIP_TRY(c, hipMemcpy(c->routers[layer], w, sizeof(float) * (size_t)c->E * c->H, hipMemcpyHostToDevice));
  return MOE_OK;
}

extern "C" int moe_seed(moe_ctx* c, const uint32_t* freq) {
  if (!c) return MOE_E_INVAL;
  DeviceGuard g(c->device);
  for (int l = 0; l < c->host_sets; ++l)
    if (!c->registered[l]) return moe_ctx_fail(c, MOE_E_STATE, "seed: host set %d (layer %d) not registered", l, l);
  if (stream_capturing(c->stream)) return moe_ctx_fail(c, MOE_E_CAPTURING, "seed while capturing");
  const int64_t L = c->L, E = c->E, S = c->S;
  std::fill(c->tbl.begin(), c->tbl.end(), -1);
  std::fill(c->owner.begin(), c->owner.end(), -1);
  std::fill(c->stamps.begin(), c->stamps.end(), 0u);
  std::fill(c->last_miss.begin(), c->last_miss.end(), 0u);
  std::fill(c->seen.begin(), c->seen.end(), 0u);  // the step count restarts
  std::fill(c->pend.begin(), c->pend.end(), -1);
  std::fill(c->flip.begin(), c->flip.end(), -1);
  if (c->swap_stream) HIP_TRY(c, hipStreamSynchronize(c->swap_stream));  // copies into slots about to be reseeded
  std::fill(c->swap_recorded.begin(), c->swap_recorded.end(), 0);
  HIP_TRY(c, hipStreamSynchronize(c->stream));
  if (freq) {
    // each pool takes its candidates (the layer's experts, or every layer's
    // with one global pool) by count, descending; ties keep (layer, expert) order
    const int64_t per = c->groups == 1 ? L * E : E;
    std::vector<int32_t> order(per);
    for (int64_t g = 0; g < c->groups; ++g) {
      for (int64_t i = 0; i < per; ++i) order[i] = (int32_t)(g * E + i);  // layer * E + expert
      std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return freq[a] > freq[b]; });
      for (int64_t s = 0; s < std::min(S, per); ++s) {
        const int32_t te = order[s];
        c->tbl[te] = (int32_t)s;
        c->owner[g * S + s] = te;
        HIP_TRY(c, hipMemcpyAsync(c->pool + (g * S + s) * c->B, c->host_layers[te / E] + (int64_t)(te % E) * c->B,
                                  c->B, hipMemcpyHostToDevice, c->stream));
      }
    }
  }
  std::memcpy(c->h_tbl, c->tbl.data(), sizeof(int32_t) * L * E);
  HIP_TRY(c, hipMemcpyAsync(c->d_tbl, c->h_tbl, sizeof(int32_t) * L * E, hipMemcpyHostToDevice, c->stream));
  HIP_TRY(c, hipMemsetAsync(c->d_stamps, 0, sizeof(uint32_t) * c->groups * std::max<int64_t>(S, 1), c->stream));
  HIP_TRY(c, hipMemsetAsync(c->d_counts, 0, sizeof(uint32_t) * L * E, c->stream));
  HIP_TRY(c, hipMemsetAsync(c->d_records, 0, sizeof(uint64_t) * L * c->rec_stride, c->stream));
  if (c->d_cap_dir) HIP_TRY(c, hipMemsetAsync(c->d_cap_dir, 0, sizeof(uint64_t) * L * c->capture_picks, c->stream));
  if (c->d_last_miss) HIP_TRY(c, hipMemsetAsync(c->d_last_miss, 0, sizeof(uint32_t) * L * E, c->stream));
  *c->h_ctrl = Ctrl{1, 0, 0, 0};
  HIP_TRY(c, hipMemcpyAsync(c->d_ctrl, c->h_ctrl, sizeof(Ctrl), hipMemcpyHostToDevice, c->stream));
  HIP_TRY(c, hipStreamSynchronize(c->stream));
  c->clock = 1;
  c->steps = 0;
  c->last_log.clear();
  c->seeded = true;
  return MOE_OK;
}

// The mailbox of the host threads (one pinned, mapped allocation) and the
// threads themselves.
static int host_exec_create(moe_ctx* c) {
  const int64_t P = (int64_t)c->cfg.max_batch_tokens * c->k, T = c->cfg.max_batch_tokens;
  auto up = [](int64_t v) { return (v + 255) / 256 * 256; };
  c->mb_off_done = 0;
  c->mb_off_seq = 256;
  c->mb_off_e = c->mb_off_seq + up(4 * P);
  c->mb_off_kind = c->mb_off_e + up(4 * P);
  c->mb_off_x = c->mb_off_kind + up(4 * P);
  c->mb_off_y = c->mb_off_x + up(4 * T * c->H);
  const int64_t bytes = c->mb_off_y + up(4 * P * c->H);
  int rc;
  if ((rc = moe_ctx_host_alloc(c, (void**)&c->mbox, (size_t)bytes, hipHostMallocMapped | hipHostMallocCoherent,
                               "host hand-off mailbox")))
    return rc;
  std::memset(c->mbox, 0, (size_t)bytes);
  void* dp = nullptr;
  HIP_TRY(c, hipHostGetDevicePointer(&dp, c->mbox, 0));
  c->mbox_dev = (uint8_t*)dp;
  moe_host::ExpertPlanes pl{c->lay.gate_nib, c->lay.gate_scl, c->lay.up_nib, c->lay.up_scl,
                            c->lay.down_nib, c->lay.down_scl, c->lay.bytes};
  moe_host::Mailbox mb;
  mb.done = (uint64_t*)(c->mbox + c->mb_off_done);
  mb.pick_seq = (const uint32_t*)(c->mbox + c->mb_off_seq);
  mb.pick_e = (const int32_t*)(c->mbox + c->mb_off_e);
  mb.pick_kind = (const int32_t*)(c->mbox + c->mb_off_kind);
  mb.x = (const float*)(c->mbox + c->mb_off_x);
  mb.y_cold = (float*)(c->mbox + c->mb_off_y);
  int threads = c->cfg.cpu_threads;
  if (threads == 0) {
    // every CPU of the affinity mask but two: the thread launching the
    // forwards and the HIP runtime's completion thread each keep a CPU busy,
    // and a pool helper that loses its CPU to them stalls every phase
    // barrier for a whole scheduler time slice
    cpu_set_t set;
    int n = sched_getaffinity(0, sizeof(set), &set) == 0 ? CPU_COUNT(&set) : (int)std::thread::hardware_concurrency();
    threads = std::max(1, n - 2);
  }
  std::string err;
  c->hx = moe_host::executor_create(threads, c->H, c->F, c->k, (int)T, pl, mb, &err);
  if (!c->hx) return moe_ctx_fail(c, MOE_E_NOMEM, "%s", err.c_str());
  c->hx_threads = threads;
  return MOE_OK;
}

static_assert(moe::kStaticScratchBytes == MOE_STATIC_SCRATCH_BYTES, "the header states the static scratch size");

// Layout of a forward's scratch for P picks: every part at a 256-byte boundary.
namespace moe {
namespace {
int64_t up256(int64_t v) { return (v + 255) / 256 * 256; }
}  // namespace
int64_t forward_scratch_bytes(int64_t T, int32_t k, int32_t H, int32_t F) {
  const int64_t P = T * k;
  return up256(4 * P) + up256(4 * P) + up256(8 * P) + up256(P) + up256(4 * P * F) + up256(4 * P * H) +
         up256(16 * P) + up256(4 * P) + up256(4) + up256(4 * T * H) + up256(4 * T) + up256(4 * P * F) +
         up256(4 * P);
}
ForwardScratch forward_scratch_carve(uint8_t* base, int64_t T, int32_t k, int32_t H, int32_t F) {
  const int64_t P = T * k;
  ForwardScratch s{};
  int64_t o = 0;
  auto take = [&](int64_t bytes) {
    uint8_t* p = base + o;
    o += up256(bytes);
    return p;
  };
  s.ids = reinterpret_cast<int32_t*>(take(4 * P));
  s.w = reinterpret_cast<float*>(take(4 * P));
  s.addr = reinterpret_cast<const uint8_t**>(take(8 * P));
  s.kind = take(P);
  s.h = reinterpret_cast<float*>(take(4 * P * F));
  s.ypick = reinterpret_cast<float*>(take(4 * P * H));
  s.groups = reinterpret_cast<int4*>(take(16 * P));
  s.order = reinterpret_cast<int32_t*>(take(4 * P));
  s.n_groups = reinterpret_cast<int32_t*>(take(4));
  s.xs = take(4 * T * H);  // 128 bytes per 32 values: hi and lo fp16
  s.xsig = reinterpret_cast<int32_t*>(take(4 * T));
  s.hs = take(4 * P * F);
  s.hsig = reinterpret_cast<int32_t*>(take(4 * P));
  return s;
}
}  // namespace moe

static int check_act(moe_ctx* c, const void* p, const char* what) {
  if (!p || ((uintptr_t)p & 15)) return moe_ctx_fail(c, MOE_E_INVAL, "%s must be a non-null 16-byte aligned pointer", what);
  return MOE_OK;
}

static int forward_impl(moe_ctx* c, int32_t layer, int32_t n_tokens, const float* x, const float* logits, float* y,
                        int32_t* ids, float* w, uint32_t flags, const moe::ForwardScratch& sc);

extern "C" int moe_forward(moe_ctx* c, int32_t layer, int32_t n_tokens, const float* x, const float* logits,
                           float* y, int32_t* ids, float* w, uint32_t flags) {
  if (!c) return MOE_E_INVAL;
  return forward_impl(c, layer, n_tokens, x, logits, y, ids, w, flags, c->sc);
}

extern "C" int moe_forward_static_scratch(moe_ctx* c, int32_t layer, int32_t n_tokens, const float* x,
                                          const float* logits, float* y, int32_t* ids, float* w, uint32_t flags) {
  if (!c) return MOE_E_INVAL;
  if (n_tokens < 1 || n_tokens > c->cfg.max_batch_tokens)
    return moe_ctx_fail(c, MOE_E_INVAL, "forward: n_tokens %d outside 1..%d", n_tokens, c->cfg.max_batch_tokens);
  const int64_t need = moe::forward_scratch_bytes(n_tokens, c->k, c->H, c->F);
  if (need > moe::kStaticScratchBytes)
    return moe_ctx_fail(c, MOE_E_INVAL,
                        "forward_static_scratch: %d tokens x top-%d at hidden %d, ffn %d need %lld bytes of scratch, "
                        "more than the static %lld",
                        n_tokens, c->k, c->H, c->F, (long long)need, (long long)moe::kStaticScratchBytes);
  uint8_t* base = moe::static_scratch(c->device);
  if (!base)
    return moe_ctx_fail(c, MOE_E_HIP, "forward_static_scratch: no static scratch on device %d (%s)", c->device,
                        c->static_scratch_err.c_str());
  return forward_impl(c, layer, n_tokens, x, logits, y, ids, w, flags,
                      moe::forward_scratch_carve(base, n_tokens, c->k, c->H, c->F));
}

static int forward_impl(moe_ctx* c, int32_t layer, int32_t n_tokens, const float* x, const float* logits, float* y,
                        int32_t* ids, float* w, uint32_t flags, const moe::ForwardScratch& sc) {
  if (layer < 0 || layer >= c->L) return moe_ctx_fail(c, MOE_E_INVAL, "forward: bad layer %d", layer);
  if (n_tokens < 1 || n_tokens > c->cfg.max_batch_tokens)
    return moe_ctx_fail(c, MOE_E_INVAL, "forward: n_tokens %d outside 1..%d", n_tokens, c->cfg.max_batch_tokens);
  int rc;
  if ((rc = check_act(c, x, "x")) || (rc = check_act(c, y, "y"))) return rc;
  if (y == x && !(flags & MOE_ACCUMULATE))
    return moe_ctx_fail(c, MOE_E_INVAL, "forward: y may alias x only with MOE_ACCUMULATE");
  if (!logits && !c->routers[layer]) return moe_ctx_fail(c, MOE_E_INVAL, "forward: no logits and no router");
  if (!c->seeded) return moe_ctx_fail(c, MOE_E_STATE, "forward before moe_seed");
  DeviceGuard g(c->device);
  hipEvent_t* ev = nullptr;  // kTimedKernels start/stop pairs
  if (c->profiling) {
    if (stream_capturing(c->stream)) return moe_ctx_fail(c, MOE_E_CAPTURING, "forward with timing on while capturing");
    if ((size_t)c->timed_pending < c->timed_tokens.size()) {
      ev = &c->events[2 * kTimedKernels * (size_t)c->timed_pending];
      c->timed_tokens[c->timed_pending++] = n_tokens;
    }
  }
  auto on = [&](hipStream_t s, int kernel) {
    moe::Launch l;
    l.stream = s;
    if (ev) l.start = ev[2 * kernel], l.stop = ev[2 * kernel + 1];
    return l;
  };
  hipStream_t A = c->stream;

  moe::RouteArgs ra{};
  ra.logits = logits;
  ra.x = x;
  ra.wr = (const float*)c->routers[layer];
  ra.T = n_tokens, ra.E = c->E, ra.k = c->k, ra.H = c->H, ra.S = c->S, ra.layer = layer;
  ra.tbl = c->d_tbl + (int64_t)layer * c->E;
  ra.stamps = c->d_stamps + c->group_of(layer) * std::max(c->S, 1);
  ra.counts = c->d_counts + (int64_t)layer * c->E;
  ra.records = c->d_records + (int64_t)layer * c->rec_stride;
  ra.ctrl = c->d_ctrl;
  ra.pool = c->pool + c->group_of(layer) * c->S * c->B;
  ra.host = c->host_layers_dev[layer];
  ra.expert_bytes = c->B;
  ra.ids = sc.ids, ra.w = sc.w, ra.addr = sc.addr, ra.kind = sc.kind;
  ra.ids_user = ids, ra.w_user = w;
  ra.policy = 1;
  ra.capture_picks = c->capture_picks;
  ra.cap_dir = c->d_cap_dir ? c->d_cap_dir + (int64_t)layer * c->capture_picks : nullptr;
  ra.last_miss = c->d_last_miss ? c->d_last_miss + (int64_t)layer * c->E : nullptr;
  ra.window = c->cfg.window_tokens, ra.admit_misses = c->cfg.admit_misses;
  // with logits at hand the gate/up GEMV routes by itself (one launch less on
  // the critical path); a router chain runs in its own launch first
  const bool fused = logits && c->E <= moe::kFusedRouteMaxExperts;
  if (c->hx) {
    if (!fused)
      return moe_ctx_fail(c, MOE_E_INVAL, "forward: with cold_exec CPU the forward needs logits and E <= %d",
                          moe::kFusedRouteMaxExperts);
    if (stream_capturing(c->stream))
      return moe_ctx_fail(c, MOE_E_CAPTURING, "forward with cold_exec CPU while capturing");
  }
  // a batch of many tokens groups its picks by expert (each expert's weights
  // read once for all the tokens that picked it); the host-thread mode keeps
  // one pass per pick
  const bool grouped = !c->hx && n_tokens >= moe::kGroupedMinTokens;
  if (ev) c->timed_fused[c->timed_pending - 1] = fused && !grouped ? 1 : 0;
  if (ev) c->timed_cpu[c->timed_pending - 1] = c->hx ? 1 : 0;
  if (ev) c->timed_grouped[c->timed_pending - 1] = grouped ? 1 : 0;
  // a few tokens with logits at hand: one launch per layer where the shape has an instantiation
  const bool one_launch = fused && !grouped && !c->hx && c->cfg.decode_launches == 1 &&
                          moe::layer_shape_ok(c->H, c->F, c->k, n_tokens, c->E);
  if (ev) c->timed_layer[c->timed_pending - 1] = one_launch ? 1 : 0;
  // the grouped matrix-core path takes the activations split into fp16 operands, from the routing kernel
  if (grouped && moe::mfma_grouped_shape_ok(c->H, c->F)) ra.xs = sc.xs, ra.xsig = sc.xsig;
  if (!fused || grouped) HIP_TRY(c, moe::launch_route(ra, on(A, kRoute)));

  moe::GemvArgs ga{};
  ga.x = x;
  ga.addr = sc.addr;
  ga.kind = sc.kind;
  ga.w = sc.w;
  ga.out = sc.h;
  ga.ypick = sc.ypick;
  ga.T = n_tokens, ga.k = c->k, ga.H = c->H, ga.F = c->F;
  ga.lay = c->lay;
  ga.capture_picks = c->capture_picks;
  ga.capture = c->d_capture ? c->d_capture + (int64_t)layer * c->capture_picks * c->B : nullptr;
  ga.cap_dir = ra.cap_dir;
  ga.ctrl = c->d_ctrl;
  moe::GemvArgs dn = ga;
  dn.x = sc.h;
  dn.out = y;
  dn.accumulate = (flags & MOE_ACCUMULATE) ? 1 : 0;
  if (grouped) {
    moe::GroupArgs gr{};
    gr.ids = sc.ids, gr.tbl = ra.tbl, gr.P = n_tokens * c->k, gr.E = c->E;
    gr.groups = sc.groups, gr.order = sc.order, gr.n_groups = sc.n_groups;
    HIP_TRY(c, moe::launch_group_picks(gr, A));
    if (moe::mfma_grouped_shape_ok(c->H, c->F)) {
      // each expert's weights dequantised once for all its picks, products on the matrix cores
      moe::SplitArgs sp{sc.xs, sc.xsig, sc.hs, sc.hsig};
      HIP_TRY(c, moe::launch_mfma_gateup(ga, gr, sp, on(A, kHotGateUp)));
      HIP_TRY(c, moe::launch_split_rows(sc.h, n_tokens * c->k, c->F, sc.hs, sc.hsig, A));
      HIP_TRY(c, moe::launch_mfma_down(dn, gr, sp, on(A, kHotDown)));
    } else {
      HIP_TRY(c, moe::launch_grouped_gateup(ga, gr, on(A, kHotGateUp)));
      HIP_TRY(c, moe::launch_grouped_down(dn, gr, on(A, kHotDown)));
    }
    HIP_TRY(c, moe::launch_combine_picks(dn, on(A, kColdDownCombine)));
    return MOE_OK;
  }
  if (c->hx) {
    // the GPU computes the hot picks while the host threads compute the cold
    // ones from the routing and activations the gate/up launch hands over
    const uint32_t seq = ++c->hx_seq ? c->hx_seq : ++c->hx_seq;  // 0 is the mailbox's initial value
    ra.pub_seq = (uint32_t*)(c->mbox_dev + c->mb_off_seq);
    ra.pub_e = (int32_t*)(c->mbox_dev + c->mb_off_e);
    ra.pub_kind = (int32_t*)(c->mbox_dev + c->mb_off_kind);
    ra.pub_x = (float*)(c->mbox_dev + c->mb_off_x);
    ra.pub_value = seq;
    HIP_TRY(c, moe::launch_gemv_route_gateup(ga, ra, on(A, kHotGateUp), moe::kOnlyHot));
    moe_host::executor_submit(c->hx, seq, n_tokens, c->host_layers[layer]);
    HIP_TRY(c, moe::launch_gemv_down_pick(dn, on(A, kHotDown), moe::kOnlyHot));
    moe::HostCombineArgs hc{};
    hc.ypick = sc.ypick, hc.w = sc.w, hc.kind = sc.kind;
    hc.y_cold = (const float*)(c->mbox_dev + c->mb_off_y);
    hc.done = (const uint64_t*)(c->mbox_dev + c->mb_off_done);
    hc.seq = seq;
    hc.max_polls = 1u << 22;  // seconds at the poll rate of pinned memory; the host answers within 10 s
    hc.y = y;
    hc.T = n_tokens, hc.k = c->k, hc.H = c->H, hc.accumulate = dn.accumulate;
    hc.ctrl = c->d_ctrl;
    HIP_TRY(c, moe::launch_host_combine(hc, on(A, kColdDownCombine)));
    return MOE_OK;
  }
  if (one_launch) {
    moe::LayerArgs la{};
    la.h = sc.h;
    la.y = y;
    la.accumulate = dn.accumulate;
    la.sync = c->d_layer_sync;
    la.max_polls = c->cfg.decode_sync_polls > 0 ? (uint32_t)c->cfg.decode_sync_polls : kLayerMaxPolls;
    if (!ev) {
      HIP_TRY(c, moe::launch_decode_layer(ga, ra, la, on(A, 0), moe::kAll));
    } else {
      // timing: the hot picks (with the side effects), then the cold ones and the combine
      moe::RouteArgs quiet = ra;
      quiet.policy = 0;
      HIP_TRY(c, moe::launch_decode_layer(ga, ra, la, on(A, kHotGateUp), moe::kOnlyHot));
      HIP_TRY(c, moe::launch_decode_layer(ga, quiet, la, on(A, kColdDownCombine), moe::kOnlyCold));
    }
    return MOE_OK;
  }
  if (!ev) {
    // hot picks stream from HBM while cold picks stream over PCIe, in one launch
    if (fused)
      HIP_TRY(c, moe::launch_gemv_route_gateup(ga, ra, on(A, 0), moe::kAll));
    else
      HIP_TRY(c, moe::launch_gemv_gateup(ga, on(A, 0), moe::kAll));
    HIP_TRY(c, moe::launch_gemv_down_combine(dn, on(A, 0), moe::kAll));
  } else {
    // timing: the same work split by tag, one launch each, in stream order;
    // fused, both gate/up launches route and only the hot one applies the
    // side effects, and there is no routing interval
    if (fused) {
      moe::RouteArgs quiet = ra;
      quiet.policy = 0;
      HIP_TRY(c, moe::launch_gemv_route_gateup(ga, quiet, on(A, kColdGateUp), moe::kOnlyCold));
      HIP_TRY(c, moe::launch_gemv_route_gateup(ga, ra, on(A, kHotGateUp), moe::kOnlyHot));
    } else {
      HIP_TRY(c, moe::launch_gemv_gateup(ga, on(A, kColdGateUp), moe::kOnlyCold));
      HIP_TRY(c, moe::launch_gemv_gateup(ga, on(A, kHotGateUp), moe::kOnlyHot));
    }
    HIP_TRY(c, moe::launch_gemv_down_pick(dn, on(A, kHotDown), moe::kOnlyHot));
    HIP_TRY(c, moe::launch_gemv_down_combine(dn, on(A, kColdDownCombine), moe::kOnlyCold));
  }
  return MOE_OK;
}

// Add the durations of the pending timed forwards (the stream must be drained).
static int flush_profile(moe_ctx* c) {
  for (int32_t i = 0; i < c->timed_pending; ++i) {
    float t[kTimedKernels];
    if (c->timed_layer[i]) {
      float hot = 0.f, cold = 0.f;
      HIP_TRY(c, hipEventElapsedTime(&hot, c->events[2 * (kTimedKernels * (size_t)i + kHotGateUp)],
                                     c->events[2 * (kTimedKernels * (size_t)i + kHotGateUp) + 1]));
      HIP_TRY(c, hipEventElapsedTime(&cold, c->events[2 * (kTimedKernels * (size_t)i + kColdDownCombine)],
                                     c->events[2 * (kTimedKernels * (size_t)i + kColdDownCombine) + 1]));
      c->prof.forwards += 1;
      c->prof.layer_forwards += 1;
      c->prof.hot_layer_ms += hot;
      c->prof.cold_layer_ms += cold;
      continue;
    }
    for (int j = 0; j < kTimedKernels; ++j) {
      t[j] = 0.f;
      if (j == kRoute && c->timed_fused[i]) continue;
      if (j == kColdGateUp && (c->timed_cpu[i] || c->timed_grouped[i])) continue;  // no separate cold gate/up
      HIP_TRY(c, hipEventElapsedTime(&t[j], c->events[2 * (kTimedKernels * (size_t)i + j)],
                                     c->events[2 * (kTimedKernels * (size_t)i + j) + 1]));
    }
    c->prof.forwards += 1;
    c->prof.route_ms += t[kRoute];
    c->prof.hot_gateup_ms += t[kHotGateUp];
    c->prof.hot_down_ms += t[kHotDown];
    c->prof.cold_gateup_ms += t[kColdGateUp];
    c->prof.cold_down_ms += t[kColdDownCombine];
  }
  c->timed_pending = 0;
  return MOE_OK;
}

extern "C" int moe_profile(moe_ctx* c, int32_t enable, moe_profile_stats* out) {
  if (!c || enable < -1 || enable > 1) return MOE_E_INVAL;
  DeviceGuard g(c->device);
  if (c->timed_pending > 0) {
    HIP_TRY(c, hipStreamSynchronize(c->stream));
    int rc = flush_profile(c);
    if (rc) return rc;
  }
  if (enable == 1) {
    c->profiling = true;
    c->prof = moe_profile_stats{};
    c->prof.gateup_bytes_per_pick = c->lay.down_nib - c->lay.gate_nib;
    c->prof.down_bytes_per_pick = c->lay.bytes - c->lay.down_nib;
  } else if (enable == 0) {
    c->profiling = false;
  }
  if (c->hx && enable != -1) moe_host::executor_stats(c->hx, nullptr, true);
  if (c->hx) {
    moe_host::ExecStats hs{};
    moe_host::executor_stats(c->hx, &hs, false);
    c->prof.host_forwards = hs.forwards, c->prof.host_expert_passes = hs.expert_passes;
    c->prof.host_picks = hs.picks, c->prof.host_wait_ms = hs.wait_ms, c->prof.host_compute_ms = hs.compute_ms;
  }
  if (out) *out = c->prof;
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// the between-step cache policy

static void forget_captures(moe_ctx* c) {
  for (int64_t te : c->cap_touched) c->cap_of[te] = -1;
  c->cap_touched.clear();
}

extern "C" int moe_cache_step(moe_ctx* c, moe_step_stats* out) {
  if (!c) return MOE_E_INVAL;
  if (!c->seeded) return moe_ctx_fail(c, MOE_E_STATE, "cache_step before moe_seed");
  DeviceGuard g(c->device);
  if (stream_capturing(c->stream)) return moe_ctx_fail(c, MOE_E_CAPTURING, "cache_step while capturing");
  const int64_t L = c->L, E = c->E, S = c->S, B = c->B;

  // one round trip: the control words, every layer's pick records, the
  // stamps and capture tags, written into the mapped staging by one launch
  const int64_t GS = (int64_t)c->groups * S;  // slots of every pool
  {
    moe::CopyList rb;
    rb.n = 0;
    rb.op[rb.n++] = moe::CopyOp{c->d_ctrl, const_cast<void*>(c->h_ctrl_dev), (int64_t)sizeof(Ctrl)};
    rb.op[rb.n++] = moe::CopyOp{c->d_records, c->h_records_dev, (int64_t)sizeof(uint64_t) * L * c->rec_stride};
    if (S > 0) rb.op[rb.n++] = moe::CopyOp{c->d_stamps, const_cast<void*>(c->h_stamps_dev), (int64_t)sizeof(uint32_t) * GS};
    if (c->d_cap_dir)
      rb.op[rb.n++] = moe::CopyOp{c->d_cap_dir, c->h_cap_dir_dev, (int64_t)sizeof(uint64_t) * L * c->capture_picks};
    HIP_TRY(c, moe::launch_copy_list(rb, c->stream));
  }
  HIP_TRY(c, hipStreamSynchronize(c->stream));
  const Ctrl st = *c->h_ctrl;
  const bool host_fault = st.host_fault != 0;
  const bool sync_fault = st.sync_fault != 0;
  if (S > 0) std::memcpy(c->stamps.data(), c->h_stamps, sizeof(uint32_t) * GS);
  // records of this step carry clocks in [clock, clock + step tokens); older ones are stale
  int64_t hits = 0, distinct = 0, distinct_cold = 0;
  const uint32_t mark = (uint32_t)(c->steps + 1);  // seen[te] == mark: (layer, expert) already read this step
  c->last_log.clear();
  forget_captures(c);  // left over if an earlier step stopped on an error
  const uint64_t t_lo = (uint64_t)c->clock, t_hi = (uint64_t)c->clock + st.step_tokens;
  for (int64_t i = 0; i < L * c->rec_stride; ++i) {
    const uint64_t r = c->h_records[i];
    const uint64_t t = r >> 32;
    if (t < t_lo || t >= t_hi) continue;
    {
      const int64_t te = (i / c->rec_stride) * E + (int64_t)(r & 0xfff);
      if ((r & 0xfff) < (uint64_t)E && c->seen[te] != mark) {
        c->seen[te] = mark;
        ++distinct;
        distinct_cold += (r & moe::kRecordHit) ? 0 : 1;
      }
    }
    if (r & moe::kRecordHit) {
      ++hits;
      continue;
    }
    c->last_log.push_back(r);
  }
  // capture blocks written during this step hold the experts their directory
  // entries name (the last forward to write a block also wrote its entry)
  for (int64_t i = 0; i < L * c->capture_picks; ++i) {
    const uint64_t d = c->h_cap_dir[i];
    const uint64_t t = d >> 32, e = d & 0xffffffffu;
    if (t < t_lo || t >= t_hi || e >= (uint64_t)E) continue;
    const int64_t te = (i / c->capture_picks) * E + (int64_t)e;
    if (c->cap_of[te] < 0) c->cap_of[te] = (int32_t)(i % c->capture_picks), c->cap_touched.push_back(te);
  }
  const int64_t misses = (int64_t)c->last_log.size();
  if (c->profiling) {
    if (c->timed_pending > 0) {
      int rc = flush_profile(c);
      if (rc) return rc;
    }
    c->prof.hot_picks += hits;
    c->prof.cold_picks += misses;
  }
  // canonical order: ascending 64-bit entries (clock, then layer, then expert)
  std::sort(c->last_log.begin(), c->last_log.end());

  int64_t admissions = 0, evictions = 0, copied_pcie = 0, swap_copies = 0;
  const int32_t lead = c->cfg.swap_lead, budget = c->cfg.swaps_per_step;
  // the step's copies on the context stream go out in one launch (several
  // when there are more than a launch holds). The transfers of a launch run
  // at once, so a slot admitted twice in one walk (its first newcomer evicted
  // again) keeps only the later transfer, as sequential copies would leave it.
  moe::CopyList cl;
  cl.n = 0;
  auto add_copy = [&](const void* src, void* dst, int64_t bytes) -> int {
    for (int i = 0; i < cl.n; ++i)
      if (cl.op[i].dst == dst) {
        cl.op[i] = moe::CopyOp{src, dst, bytes};
        return MOE_OK;
      }
    if (cl.n == moe::kMaxCopyOps) {
      HIP_TRY(c, moe::launch_copy_list(cl, c->stream));
      cl.n = 0;
    }
    cl.op[cl.n++] = moe::CopyOp{src, dst, bytes};
    return MOE_OK;
  };
  int crc;
  for (uint64_t entry : c->last_log) {
    const uint32_t t = (uint32_t)(entry >> 32);
    const int64_t l = (int64_t)((entry >> 12) & 0x7ffff);
    const int64_t e = (int64_t)(entry & 0xfff);
    if (l >= L || e >= E) continue;
    const int64_t te = l * E + e;
    if (c->tbl[te] >= 0 || c->pend[te] >= 0) continue;  // admitted earlier in this walk, or pending
    bool admit;
    if (c->cfg.admit_misses == 1) {
      admit = true;
    } else {
      const uint32_t prev = c->last_miss[te];
      admit = prev != 0 && (int64_t)t - (int64_t)prev < (int64_t)c->cfg.window_tokens;
      if (!admit) c->last_miss[te] = t;
    }
    if (!admit || S == 0) continue;
    // victim in the layer's pool: lowest free slot, else the smallest stamp
    // (ties: highest slot) among slots no pending admission holds; with one
    // global pool the owner may be any layer's
    const int64_t g0 = c->group_of(l) * S;
    int64_t v = -1;
    for (int64_t s = 0; s < S; ++s)
      if (c->owner[g0 + s] < 0) {
        v = s;
        break;
      }
    if (v < 0) {
      uint32_t best = 0xffffffffu;
      for (int64_t s = 0; s < S; ++s)
        if (c->flip[g0 + s] < 0 && c->stamps[g0 + s] <= best) best = c->stamps[g0 + s], v = s;
    }
    if (v < 0 || (budget > 0 && admissions == budget)) {
      c->last_miss[te] = t;  // refused: remembered as a miss
      continue;
    }
    if (c->owner[g0 + v] >= 0) {
      const int32_t old = c->owner[g0 + v];  // layer * E + expert
      c->tbl[old] = -1;
      c->last_miss[old] = 0;
      ++evictions;
    }
    c->owner[g0 + v] = (int32_t)te;
    c->stamps[g0 + v] = t;
    c->last_miss[te] = 0;
    if (lead == 0) {
      c->tbl[te] = (int32_t)v;
    } else {
      c->pend[te] = (int32_t)v;
      c->flip[g0 + v] = c->steps + lead;
    }
    ++admissions;
    uint8_t* dst = c->pool + (g0 + v) * B;
    if (c->cap_of[te] >= 0) {  // before the next step's forwards overwrite the capture block
      if ((crc = add_copy(c->d_capture + (l * c->capture_picks + c->cap_of[te]) * B, dst, B))) return crc;
    } else if (lead == 0) {
      if ((crc = add_copy(c->host_layers_dev[l] + e * B, dst, B))) return crc;  // zero-copy read of the pinned weights
      ++copied_pcie;
    } else {
      // with a lead the slot is read by nobody until the flip: the copy runs beside the next steps
      HIP_TRY(c, hipMemcpyAsync(dst, c->host_layers[l] + e * B, B, hipMemcpyHostToDevice, c->swap_stream));
      ++copied_pcie;
      ++swap_copies;
    }
  }
  forget_captures(c);
  int64_t flips = 0;
  if (lead > 0) {
    const int64_t ring = lead + 1;
    if (swap_copies > 0) {
      HIP_TRY(c, hipEventRecord(c->swap_events[c->steps % ring], c->swap_stream));
      c->swap_recorded[c->steps % ring] = 1;
    }
    // admissions decided lead steps ago flip in once their copies are done
    const int64_t due = c->steps - lead;
    if (due >= 0 && c->swap_recorded[due % ring]) {
      HIP_TRY(c, hipEventSynchronize(c->swap_events[due % ring]));
      c->swap_recorded[due % ring] = 0;
    }
    for (int64_t i = 0; i < GS; ++i)
      if (c->flip[i] >= 0 && c->flip[i] <= c->steps) {
        const int32_t te = c->owner[i];
        c->tbl[te] = (int32_t)(i % S);
        c->pend[te] = -1;
        c->flip[i] = -1;
        ++flips;
      }
  }
  // uploads, read in place from the mapped staging by the same launch
  if (c->d_last_miss && misses > 0) {  // the next step's forwards decide what to capture from it
    std::memcpy(c->h_last_miss, c->last_miss.data(), sizeof(uint32_t) * L * E);
    if ((crc = add_copy(c->h_last_miss_dev, c->d_last_miss, sizeof(uint32_t) * L * E))) return crc;
  }
  if (admissions > 0 || flips > 0) {
    std::memcpy(c->h_tbl, c->tbl.data(), sizeof(int32_t) * L * E);
    if ((crc = add_copy(c->h_tbl_dev, c->d_tbl, sizeof(int32_t) * L * E))) return crc;
    if (S > 0) {
      std::memcpy(c->h_stamps, c->stamps.data(), sizeof(uint32_t) * GS);
      if ((crc = add_copy(c->h_stamps_dev, c->d_stamps, sizeof(uint32_t) * GS))) return crc;
    }
  }
  c->clock += st.step_tokens;
  *c->h_ctrl = Ctrl{(uint32_t)c->clock, 0, 0, 0};
  if ((crc = add_copy(c->h_ctrl_dev, c->d_ctrl, sizeof(Ctrl)))) return crc;
  HIP_TRY(c, moe::launch_copy_list(cl, c->stream));

  if (out) {
    out->step = c->steps;
    out->tokens = st.step_tokens;
    out->hits = hits;
    out->misses = misses;
    out->admissions = admissions;
    out->evictions = evictions;
    out->hot_bytes = hits * B;
    out->cold_bytes = misses * B;
    out->copied_bytes = admissions * B;
    out->copied_pcie_bytes = copied_pcie * B;
    out->distinct_experts = distinct;
    out->distinct_cold_experts = distinct_cold;
  }
  c->steps += 1;
  if (sync_fault) {
    // a wait ran out: the counters may hold a count the protocol did not end at 0
    HIP_TRY(c, hipMemsetAsync(c->d_layer_sync, 0, kLayerSyncBytes, c->stream));
    HIP_TRY(c, hipStreamSynchronize(c->stream));
    return moe_ctx_fail(c, MOE_E_HIP,
                        "cache_step: a one-launch layer forward of this step gave up waiting for its gate/up "
                        "work-groups (its outputs are not valid)");
  }
  if (host_fault)
    return moe_ctx_fail(c, MOE_E_HIP,
                        "cache_step: a forward of this step got no answer from the host threads (its cold picks "
                        "were left out of y)");
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// introspection

extern "C" int moe_get_info(moe_ctx* c, moe_info* out) {
  if (!c || !out) return MOE_E_INVAL;
  out->slots_per_layer = c->S;
  out->expert_bytes = c->B;
  out->pool_bytes = (int64_t)c->groups * c->S * c->B;
  out->host_bytes = (int64_t)c->host_sets * c->E * c->B;
  out->staging_experts = c->n_staging;
  out->host_threads = c->hx ? c->hx_threads : 0;
  out->host_isa = !c->hx ? 0 : std::strcmp(moe_host::executor_isa(c->hx), "avx512") == 0 ? 3
                  : std::strcmp(moe_host::executor_isa(c->hx), "avx2") == 0           ? 2
                                                                                      : 1;
  out->clock = c->clock;
  out->steps = c->steps;
  out->pool_budget_bytes = c->budget;
  out->free_bytes_at_sizing = c->free_at_sizing;
  return MOE_OK;
}

extern "C" int moe_get_slot_table(moe_ctx* c, int32_t layer, int32_t* out) {
  if (!c || !out || layer < 0 || layer >= c->L) return MOE_E_INVAL;
  DeviceGuard g(c->device);
  HIP_TRY(c, hipStreamSynchronize(c->stream));
  HIP_TRY(c, hipMemcpy(out, c->d_tbl + (int64_t)layer * c->E, sizeof(int32_t) * c->E, hipMemcpyDeviceToHost));
  return MOE_OK;
}

extern "C" int moe_get_stamps(moe_ctx* c, int32_t layer, uint32_t* out) {
  if (!c || !out || layer < 0 || layer >= c->L) return MOE_E_INVAL;
  if (c->S == 0) return MOE_OK;
  DeviceGuard g(c->device);
  HIP_TRY(c, hipStreamSynchronize(c->stream));
  HIP_TRY(c, hipMemcpy(out, c->d_stamps + c->group_of(layer) * c->S, sizeof(uint32_t) * c->S, hipMemcpyDeviceToHost));
  return MOE_OK;
}

extern "C" int moe_get_miss_log(moe_ctx* c, uint64_t* out, int64_t cap, int64_t* n) {
  if (!c || !n || cap < 0 || (cap > 0 && !out)) return MOE_E_INVAL;
  *n = (int64_t)c->last_log.size();
  const int64_t m = std::min<int64_t>(cap, *n);
  if (m > 0) std::memcpy(out, c->last_log.data(), sizeof(uint64_t) * m);
  return MOE_OK;
}

extern "C" int moe_get_counts(moe_ctx* c, uint32_t* out) {
  if (!c || !out) return MOE_E_INVAL;
  DeviceGuard g(c->device);
  HIP_TRY(c, hipStreamSynchronize(c->stream));
  HIP_TRY(c, hipMemcpy(out, c->d_counts, sizeof(uint32_t) * (size_t)c->L * c->E, hipMemcpyDeviceToHost));
  return MOE_OK;
}
