// prefill.cpp - prompt pass of one layer (grouped GEMM over tokens sorted by
// expert, staging of non-resident experts into borrowed HBM blocks).
#include <hip/hip_runtime.h>

#include "runtime.h"

struct Prefill {};

int moe_prefill_alloc(moe_ctx* c) {
  (void)c;
  return MOE_OK;
}

void moe_prefill_release(moe_ctx* c) { (void)c; }

extern "C" int moe_prefill(moe_ctx* c, int32_t layer, int32_t n_tokens, const float* x, const float* logits,
                           float* y, uint32_t flags) {
  (void)layer, (void)n_tokens, (void)x, (void)logits, (void)y, (void)flags;
  if (!c) return MOE_E_INVAL;
  return moe_ctx_fail(c, MOE_E_STATE, "prefill is not available in this build");
}
