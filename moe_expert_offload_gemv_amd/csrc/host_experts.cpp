// host_experts.cpp - CPU execution of the cold picks of a decode forward.
//
// Per forward the coordinator gathers the cold picks, groups them by expert
// (tokens that picked the same expert share one pass over its weights), and
// runs two parallel phases over a persistent pool:
//   1. h[p] = silu(W_gate x_t) * (W_up x_t) for every cold pick p, rows of F
//      split over the threads;
//   2. y_cold[p] = W_down h[p], rows of H split over the threads.
// A row is a run of 32-weight blocks (16 bytes of nibbles + an fp16 scale d);
// its dot with v is sum over blocks of d * sum_j (q_j - 8) v_j in fp32, with
// element j < 16 in the low nibble of byte j and element j + 16 in its high
// nibble. The widest of AVX-512, AVX2 + FMA + F16C or plain C++ that the
// host supports is chosen once, at start.
#include "host_experts.h"

#include <immintrin.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <cstring>
#include <deque>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

namespace moe_host {

namespace {

inline void cpu_relax() { _mm_pause(); }

float half_to_float(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t ex = (h >> 10) & 0x1f, man = h & 0x3ffu;
  float v;
  if (ex == 0) {
    v = std::ldexp((float)man, -24);  // zero or subnormal
  } else if (ex == 31) {
    v = man ? NAN : INFINITY;
  } else {
    v = std::ldexp((float)(man | 0x400u), (int)ex - 25);
  }
  uint32_t b;
  std::memcpy(&b, &v, 4);
  b |= sign;
  std::memcpy(&v, &b, 4);
  return v;
}

// ---------------------------------------------------------------------------
// row dots: out[t] = row . v[t] for nt vectors (nt <= kMaxNt)

constexpr int kMaxNt = 4;
using RowDotFn = void (*)(const uint8_t* nib, const uint16_t* scl, int kb, const float* const* v, int nt,
                          float* out);

void row_dot_scalar(const uint8_t* nib, const uint16_t* scl, int kb, const float* const* v, int nt, float* out) {
  for (int t = 0; t < nt; ++t) {
    float acc = 0.f;
    for (int b = 0; b < kb; ++b) {
      const uint8_t* q = nib + 16 * b;
      const float* x = v[t] + 32 * b;
      float s = 0.f;
      for (int j = 0; j < 16; ++j) {
        s += (float)((int)(q[j] & 15) - 8) * x[j];
        s += (float)((int)(q[j] >> 4) - 8) * x[j + 16];
      }
      acc += half_to_float(scl[b]) * s;
    }
    out[t] = acc;
  }
}

__attribute__((target("avx2,fma,f16c"))) inline float hsum256(__m256 v) {
  __m128 a = _mm_add_ps(_mm256_castps256_ps128(v), _mm256_extractf128_ps(v, 1));
  a = _mm_add_ps(a, _mm_movehl_ps(a, a));
  a = _mm_add_ss(a, _mm_movehdup_ps(a));
  return _mm_cvtss_f32(a);
}

__attribute__((target("avx2,fma,f16c"))) void row_dot_avx2(const uint8_t* nib, const uint16_t* scl, int kb,
                                                          const float* const* v, int nt, float* out) {
  __m256 acc[kMaxNt];
  for (int t = 0; t < nt; ++t) acc[t] = _mm256_setzero_ps();
  const __m256 eight = _mm256_set1_ps(8.f);
  const __m128i m4 = _mm_set1_epi8(0x0f);
  for (int b = 0; b < kb; ++b) {
    const __m128i q = _mm_loadu_si128(reinterpret_cast<const __m128i*>(nib + 16 * b));
    const __m128i lo = _mm_and_si128(q, m4), hi = _mm_and_si128(_mm_srli_epi16(q, 4), m4);
    const __m256 w0 = _mm256_sub_ps(_mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(lo)), eight);
    const __m256 w1 = _mm256_sub_ps(_mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(_mm_srli_si128(lo, 8))), eight);
    const __m256 w2 = _mm256_sub_ps(_mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(hi)), eight);
    const __m256 w3 = _mm256_sub_ps(_mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(_mm_srli_si128(hi, 8))), eight);
    const __m256 d = _mm256_set1_ps(_cvtsh_ss(scl[b]));
    for (int t = 0; t < nt; ++t) {
      const float* x = v[t] + 32 * b;
      __m256 s = _mm256_mul_ps(w0, _mm256_loadu_ps(x));
      s = _mm256_fmadd_ps(w1, _mm256_loadu_ps(x + 8), s);
      s = _mm256_fmadd_ps(w2, _mm256_loadu_ps(x + 16), s);
      s = _mm256_fmadd_ps(w3, _mm256_loadu_ps(x + 24), s);
      acc[t] = _mm256_fmadd_ps(d, s, acc[t]);
    }
  }
  for (int t = 0; t < nt; ++t) out[t] = hsum256(acc[t]);
}

// q - 8 of the 32 elements of block b: elements 0..15 and 16..31
__attribute__((target("avx512f,avx512bw,avx512vl,f16c"))) inline void unpack_block512(const uint8_t* nib, int b,
                                                                                     __m512& lo, __m512& hi) {
  const __m512 eight = _mm512_set1_ps(8.f);
  const __m128i m4 = _mm_set1_epi8(0x0f);
  const __m128i q = _mm_loadu_si128(reinterpret_cast<const __m128i*>(nib + 16 * b));
  lo = _mm512_sub_ps(_mm512_cvtepi32_ps(_mm512_cvtepu8_epi32(_mm_and_si128(q, m4))), eight);
  hi = _mm512_sub_ps(_mm512_cvtepi32_ps(_mm512_cvtepu8_epi32(_mm_and_si128(_mm_srli_epi16(q, 4), m4))), eight);
}

// Two blocks per iteration into two accumulators, so consecutive blocks do
// not wait on each other's FMA.
__attribute__((target("avx512f,avx512bw,avx512vl,avx512dq,fma,f16c"))) void row_dot_avx512(
    const uint8_t* nib, const uint16_t* scl, int kb, const float* const* v, int nt, float* out) {
  __m512 acc0[kMaxNt], acc1[kMaxNt];
  for (int t = 0; t < nt; ++t) acc0[t] = acc1[t] = _mm512_setzero_ps();
  int b = 0;
  for (; b + 1 < kb; b += 2) {
    __m512 l0, h0, l1, h1;
    unpack_block512(nib, b, l0, h0);
    unpack_block512(nib, b + 1, l1, h1);
    const __m512 d0 = _mm512_set1_ps(_cvtsh_ss(scl[b])), d1 = _mm512_set1_ps(_cvtsh_ss(scl[b + 1]));
    for (int t = 0; t < nt; ++t) {
      const float* x = v[t] + 32 * b;
      __m512 s0 = _mm512_mul_ps(l0, _mm512_loadu_ps(x));
      s0 = _mm512_fmadd_ps(h0, _mm512_loadu_ps(x + 16), s0);
      __m512 s1 = _mm512_mul_ps(l1, _mm512_loadu_ps(x + 32));
      s1 = _mm512_fmadd_ps(h1, _mm512_loadu_ps(x + 48), s1);
      acc0[t] = _mm512_fmadd_ps(d0, s0, acc0[t]);
      acc1[t] = _mm512_fmadd_ps(d1, s1, acc1[t]);
    }
  }
  if (b < kb) {
    __m512 l0, h0;
    unpack_block512(nib, b, l0, h0);
    const __m512 d0 = _mm512_set1_ps(_cvtsh_ss(scl[b]));
    for (int t = 0; t < nt; ++t) {
      const float* x = v[t] + 32 * b;
      __m512 s0 = _mm512_mul_ps(l0, _mm512_loadu_ps(x));
      s0 = _mm512_fmadd_ps(h0, _mm512_loadu_ps(x + 16), s0);
      acc0[t] = _mm512_fmadd_ps(d0, s0, acc0[t]);
    }
  }
  for (int t = 0; t < nt; ++t) out[t] = _mm512_reduce_add_ps(_mm512_add_ps(acc0[t], acc1[t]));
}

// ---------------------------------------------------------------------------
// persistent thread pool: run(fn) calls fn(i, n) on every thread i < n and
// returns when all are done. Idle helpers spin briefly, then sleep.

class Pool {
 public:
  explicit Pool(int n) : n_(n) {
    for (int i = 1; i < n; ++i) th_.emplace_back([this, i] { helper(i); });
  }
  ~Pool() {
    {
      std::lock_guard<std::mutex> lk(m_);
      quit_.store(true);
    }
    cv_.notify_all();
    for (auto& t : th_) t.join();
  }
  int size() const { return n_; }
  void run(const std::function<void(int, int)>& fn) {
    fn_ = &fn;
    remaining_.store(n_ - 1);
    gen_.fetch_add(1);  // seq_cst: pairs with the helpers' sleepers_ / gen_ order
    if (sleepers_.load() > 0) {
      std::lock_guard<std::mutex> lk(m_);
      cv_.notify_all();
    }
    fn(0, n_);
    while (remaining_.load(std::memory_order_acquire) > 0) cpu_relax();
  }

 private:
  void helper(int i) {
    uint64_t seen = 0;
    for (;;) {
      uint64_t g;
      int spins = 0;
      while ((g = gen_.load()) == seen) {
        if (quit_.load()) return;
        if (++spins < kSpins) {
          cpu_relax();
          continue;
        }
        std::unique_lock<std::mutex> lk(m_);
        sleepers_.fetch_add(1);
        cv_.wait(lk, [&] { return gen_.load() != seen || quit_.load(); });
        sleepers_.fetch_sub(1);
        spins = 0;
      }
      seen = g;
      (*fn_)(i, n_);
      remaining_.fetch_sub(1, std::memory_order_acq_rel);
    }
  }
  static constexpr int kSpins = 1 << 16;  // a few hundred microseconds
  int n_;
  std::vector<std::thread> th_;
  std::atomic<uint64_t> gen_{0};
  std::atomic<int> remaining_{0}, sleepers_{0};
  std::atomic<bool> quit_{false};
  const std::function<void(int, int)>* fn_ = nullptr;
  std::mutex m_;
  std::condition_variable cv_;
};

struct Job {
  uint32_t seq;
  int T;
  const uint8_t* base;
};

struct Group {  // one cold expert and the picks that chose it
  const uint8_t* w;
  int n;
  int pick[kMaxNt * 64];
};

}  // namespace

class Executor {
 public:
  Executor(int threads, int H, int F, int k, int max_tokens, const ExpertPlanes& pl, const Mailbox& mb)
      : H_(H), F_(F), k_(k), P_(max_tokens * k), pl_(pl), mb_(mb), pool_(threads) {
    if (__builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
        __builtin_cpu_supports("avx512vl") && __builtin_cpu_supports("avx512dq") && __builtin_cpu_supports("f16c") &&
        __builtin_cpu_supports("fma")) {
      dot_ = row_dot_avx512, isa_ = "avx512";
    } else if (__builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma") && __builtin_cpu_supports("f16c")) {
      dot_ = row_dot_avx2, isa_ = "avx2";
    } else {
      dot_ = row_dot_scalar, isa_ = "scalar";
    }
    h_.assign((size_t)P_ * F_, 0.f);
    x_.assign((size_t)max_tokens * H_, 0.f);
    groups_.reserve(P_);
    coord_ = std::thread([this] { coordinate(); });
  }
  ~Executor() {
    {
      std::lock_guard<std::mutex> lk(qm_);
      quit_ = true;
    }
    qcv_.notify_all();
    coord_.join();
  }
  void submit(uint32_t seq, int T, const uint8_t* base) {
    {
      std::lock_guard<std::mutex> lk(qm_);
      q_.push_back(Job{seq, T, base});
      queued_.fetch_add(1, std::memory_order_release);
    }
    qcv_.notify_one();
  }
  const char* isa() const { return isa_; }

 private:
  void coordinate() {
    for (;;) {
      Job j;
      // a hand-off usually follows within microseconds: spin before sleeping
      for (int spins = 0; spins < kSpinsBeforeSleep && queued_.load(std::memory_order_acquire) == 0; ++spins)
        cpu_relax();
      {
        std::unique_lock<std::mutex> lk(qm_);
        qcv_.wait(lk, [&] { return quit_ || !q_.empty(); });
        if (q_.empty()) return;  // quit with nothing left
        j = q_.front();
        q_.pop_front();
        queued_.fetch_sub(1, std::memory_order_relaxed);
      }
      run_job(j);
    }
  }

  static uint32_t load_acquire(const uint32_t* p) { return __atomic_load_n(p, __ATOMIC_ACQUIRE); }

  void run_job(const Job& j) {
    const int P = j.T * k_;
    const auto w0 = std::chrono::steady_clock::now();
    // wait for every pick of the forward (bounded: a forward whose picks
    // never arrive is answered with status 1 so the GPU's combine goes on).
    // A pick already carrying a later forward's value means the GPU went on
    // without this answer, which it does only for a forward with no cold
    // pick: nothing to compute.
    uint32_t status = 0;
    bool superseded = false;
    const auto t0 = std::chrono::steady_clock::now();
    for (int p = 0; p < P && !status && !superseded; ++p) {
      int spins = 0;
      uint32_t v;
      while ((v = load_acquire(&mb_.pick_seq[p])) != j.seq) {
        if ((int32_t)(v - j.seq) > 0) {
          superseded = true;
          break;
        }
        cpu_relax();
        if (++spins == 4096) {
          spins = 0;
          if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(kPickTimeoutS)) {
            status = 1;
            break;
          }
        }
      }
    }
    const auto c0 = std::chrono::steady_clock::now();
    // (if the GPU overtakes while this runs, the forward had no cold pick and
    // nobody reads what this writes)
    if (!status && !superseded) compute(j, P);
    __atomic_store_n(mb_.done, ((uint64_t)status << 32) | j.seq, __ATOMIC_RELEASE);
    const auto c1 = std::chrono::steady_clock::now();
    st_forwards_.fetch_add(1, std::memory_order_relaxed);
    st_wait_ns_.fetch_add(std::chrono::duration_cast<std::chrono::nanoseconds>(c0 - w0).count(),
                          std::memory_order_relaxed);
    st_compute_ns_.fetch_add(std::chrono::duration_cast<std::chrono::nanoseconds>(c1 - c0).count(),
                             std::memory_order_relaxed);
  }

 public:
  void stats(ExecStats* out, bool reset) {
    if (out) {
      out->forwards = st_forwards_.load();
      out->expert_passes = st_passes_.load();
      out->picks = st_picks_.load();
      out->wait_ms = st_wait_ns_.load() * 1e-6;
      out->compute_ms = st_compute_ns_.load() * 1e-6;
    }
    if (reset) st_forwards_ = 0, st_passes_ = 0, st_picks_ = 0, st_wait_ns_ = 0, st_compute_ns_ = 0;
  }

 private:

  void compute(const Job& j, int P) {
    // the activations, once, into private memory: the dot products read each
    // row once per weight row, and the mailbox is pinned memory the host may
    // map uncached
    std::memcpy(x_.data(), mb_.x, sizeof(float) * (size_t)j.T * H_);
    // group the cold picks by expert, in order of first appearance
    groups_.clear();
    for (int p = 0; p < P; ++p) {
      if (!(mb_.pick_kind[p] & 1)) continue;
      const uint8_t* w = j.base + (int64_t)mb_.pick_e[p] * pl_.bytes;
      Group* g = nullptr;
      for (auto& gg : groups_)
        if (gg.w == w) g = &gg;
      if (!g) {
        groups_.push_back(Group{});
        g = &groups_.back();
        g->w = w;
        g->n = 0;
      }
      g->pick[g->n++] = p;
    }
    if (groups_.empty()) return;
    const int G = (int)groups_.size();
    st_passes_.fetch_add(G, std::memory_order_relaxed);
    for (const auto& g : groups_) st_picks_.fetch_add(g.n, std::memory_order_relaxed);
    const int kbh = H_ / 32, kbf = F_ / 32;
    // phase 1: gate/up rows of every group
    pool_.run([&](int i, int n) {
      const int64_t rows = (int64_t)G * F_;
      const int64_t a = rows * i / n, b = rows * (i + 1) / n;
      const float* v[kMaxNt];
      float gv[kMaxNt], uv[kMaxNt];
      for (int64_t r = a; r < b; ++r) {
        const Group& g = groups_[r / F_];
        const int row = (int)(r % F_);
        const uint8_t* gn = g.w + pl_.gate_nib + (int64_t)row * kbh * 16;
        const uint16_t* gs = reinterpret_cast<const uint16_t*>(g.w + pl_.gate_scl) + (int64_t)row * kbh;
        const uint8_t* un = g.w + pl_.up_nib + (int64_t)row * kbh * 16;
        const uint16_t* us = reinterpret_cast<const uint16_t*>(g.w + pl_.up_scl) + (int64_t)row * kbh;
        for (int c = 0; c < g.n; c += kMaxNt) {
          const int nt = std::min(kMaxNt, g.n - c);
          for (int t = 0; t < nt; ++t) v[t] = x_.data() + (int64_t)(g.pick[c + t] / k_) * H_;
          dot_(gn, gs, kbh, v, nt, gv);
          dot_(un, us, kbh, v, nt, uv);
          for (int t = 0; t < nt; ++t) h_[(size_t)g.pick[c + t] * F_ + row] = gv[t] / (1.0f + std::exp(-gv[t])) * uv[t];
        }
      }
    });
    // phase 2: down rows of every group
    pool_.run([&](int i, int n) {
      const int64_t rows = (int64_t)G * H_;
      const int64_t a = rows * i / n, b = rows * (i + 1) / n;
      const float* v[kMaxNt];
      float yv[kMaxNt];
      for (int64_t r = a; r < b; ++r) {
        const Group& g = groups_[r / H_];
        const int row = (int)(r % H_);
        const uint8_t* dn = g.w + pl_.down_nib + (int64_t)row * kbf * 16;
        const uint16_t* ds = reinterpret_cast<const uint16_t*>(g.w + pl_.down_scl) + (int64_t)row * kbf;
        for (int c = 0; c < g.n; c += kMaxNt) {
          const int nt = std::min(kMaxNt, g.n - c);
          for (int t = 0; t < nt; ++t) v[t] = h_.data() + (size_t)g.pick[c + t] * F_;
          dot_(dn, ds, kbf, v, nt, yv);
          for (int t = 0; t < nt; ++t) mb_.y_cold[(int64_t)g.pick[c + t] * H_ + row] = yv[t];
        }
      }
    });
  }

  static constexpr int kPickTimeoutS = 10;
  static constexpr int kSpinsBeforeSleep = 1 << 15;  // about a millisecond of pause instructions
  std::atomic<int> queued_{0};
  std::atomic<int64_t> st_forwards_{0}, st_passes_{0}, st_picks_{0}, st_wait_ns_{0}, st_compute_ns_{0};
  int H_, F_, k_, P_;
  ExpertPlanes pl_;
  Mailbox mb_;
  RowDotFn dot_ = row_dot_scalar;
  const char* isa_ = "scalar";
  std::vector<float> h_, x_;
  std::vector<Group> groups_;
  Pool pool_;
  std::mutex qm_;
  std::condition_variable qcv_;
  std::deque<Job> q_;
  bool quit_ = false;
  std::thread coord_;
};

Executor* executor_create(int threads, int H, int F, int k, int max_tokens, const ExpertPlanes& planes,
                          const Mailbox& mb, std::string* err) {
  if (threads < 1 || H % 32 || F % 32 || k < 1 || max_tokens < 1) {
    if (err) *err = "host executor: bad shape or thread count";
    return nullptr;
  }
  try {
    return new Executor(threads, H, F, k, max_tokens, planes, mb);
  } catch (const std::exception& e) {
    if (err) *err = std::string("host executor: ") + e.what();
    return nullptr;
  }
}

void executor_destroy(Executor* ex) { delete ex; }

void executor_submit(Executor* ex, uint32_t seq, int T, const uint8_t* layer_base) { ex->submit(seq, T, layer_base); }

const char* executor_isa(const Executor* ex) { return ex->isa(); }

void executor_stats(Executor* ex, ExecStats* out, bool reset) { ex->stats(out, reset); }

}  // namespace moe_host
