// Routing helpers shared by the top-k kernel and the one-token layer kernel,
// so that both select the same experts and produce bit-identical weights.
//
// Selection rule (the C header states it): the k largest router logits, ties
// to the lower expert index, -0 == +0, a NaN below every number; the weights
// are the softmax over the k selected logits ("Beam-1.0-501B-A23B VQ GGUF",
// "What stays native": the router stays FP32).
#pragma once
#include "common.h"

namespace moe {

// One 64-bit key per candidate, unique and ordered like the selection rule:
// the logit's order key above the complement of the expert index.
__device__ __forceinline__ uint64_t topk_key(float logit, int e) {
  return ((uint64_t)order_key(logit) << 32) | (uint64_t)(~(uint32_t)e);
}
__device__ __forceinline__ int topk_key_expert(uint64_t key) { return (int)~(uint32_t)key; }

// Softmax weight of slot `lane` (< k) over the k selected logits sel_v[0..k)
// (sel_v[0] the largest): w = expf(l - l_0) / sum, the sum taken in slot
// order. Called by all 64 lanes of one wave; lanes >= k get 0.
__device__ __forceinline__ float topk_softmax(const float* sel_v, int k, int lane) {
  const float top0 = sel_v[0];
  const float a = (lane < k) ? expf(sel_v[lane] - top0) : 0.0f;
  float sum = 0.0f;
  for (int j = 0; j < k; j++) sum += __shfl(a, j, 64);
  return (lane < k) ? a / sum : 0.0f;
}

}  // namespace moe
