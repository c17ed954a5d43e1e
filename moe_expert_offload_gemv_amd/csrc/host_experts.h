// host_experts.h - host threads that compute the cold picks of a decode
// forward on the CPU (moe_config.cold_exec = MOE_COLD_CPU), beside the GPU
// computing the hot ones ("llama.cpp: fork with multi gpu acceleration even
// for models bigger than total gpu mem" README, "How it works": the GPUs run
// the cached experts while the CPU runs the misses, in parallel).
//
// Plain C++ (no HIP): the runtime allocates the mailbox in pinned host memory
// and launches the kernels that fill and read it; this side only polls and
// writes host memory.
//
// Hand-off per forward, numbered by a sequence value s:
//   GPU: a work-group of pick p writes expert and kind of the pick (and, for
//        the first pick of a token, the token's activations) with stores that
//        write through to host memory, waits for them, then pick_seq[p] = s.
//   CPU: the coordinator thread waits until pick_seq[p] == s for every pick,
//        computes y_cold[p] = W_down (silu(W_gate x) * (W_up x)) of every cold
//        pick p (unweighted), then done = status << 32 | s (release).
//   GPU: the combine of a token with a cold pick waits (bounded) for done ==
//        s and adds the weighted picks in pick order, cold ones from y_cold.
//        A forward with no cold pick does not wait, so the next forward may
//        overwrite the mailbox before this side has read it: a pick flag
//        already past s tells the coordinator that s needs nothing.
// Forwards are answered in the order they were submitted.
#pragma once
#include <stdint.h>

#include <string>

namespace moe_host {

// Byte offsets of the matrices of one expert (nibble plane [rows][kb][16],
// scale plane [rows][kb] of fp16) and the expert's size.
struct ExpertPlanes {
  int64_t gate_nib, gate_scl, up_nib, up_scl, down_nib, down_scl, bytes;
};

// Host addresses inside the pinned mailbox.
struct Mailbox {
  uint64_t* done;            // status << 32 | last answered sequence value; status 0 ok,
                             // 1 the picks of the forward never arrived (timeout)
  const uint32_t* pick_seq;  // [P]
  const int32_t* pick_e;     // [P]
  const int32_t* pick_kind;  // [P] bit 0 set: cold
  const float* x;            // [T][H]
  float* y_cold;             // [P][H]
};

class Executor;

// threads >= 1 (the coordinator is one of them). Returns nullptr and sets
// *err on failure.
Executor* executor_create(int threads, int H, int F, int k, int max_tokens, const ExpertPlanes& planes,
                          const Mailbox& mb, std::string* err);
// Waits for the submitted forwards, then stops the threads.
void executor_destroy(Executor* ex);
// Queue forward s of T tokens whose experts live at layer_base + e * bytes.
void executor_submit(Executor* ex, uint32_t seq, int T, const uint8_t* layer_base);
// Vector width the dot products use: "avx512", "avx2" or "scalar".
const char* executor_isa(const Executor* ex);

// Totals since the last reset: forwards answered, expert passes (one per
// distinct cold expert of a forward), cold picks computed, time from taking a
// forward to seeing all its picks, and time computing.
struct ExecStats {
  int64_t forwards, expert_passes, picks;
  double wait_ms, compute_ms;
};
void executor_stats(Executor* ex, ExecStats* out, bool reset);

}  // namespace moe_host
