// Routing helpers shared by the router and top-k kernels and the one-token
// layer kernel, so that both paths compute bit-identical logits, select the
// same experts and produce bit-identical weights.
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

// One thread's part of a router logit, for a workgroup of NT threads: the
// f32 fma chain over h = 4j, 4j + 4 NT, ... (h ascending; the four inputs of
// a piece in order). Each pass issues the loads of up to 8 pieces before its
// FMAs, so a row costs one memory round trip per 32 NT inputs, not one per
// piece. row: f32 [H] (16-byte aligned); x: bf16 [H] (8-byte aligned).
template <int NT>
__device__ __forceinline__ float router_thread_sum(const float* __restrict__ row, const uint16_t* __restrict__ x,
                                                   int H, int j) {
  constexpr int U = 8;
  float acc = 0.0f;
  for (int h0 = 4 * j; h0 < H; h0 += 4 * NT * U) {
    f32x4 wv[U];
    u32x2 xv[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int h = h0 + 4 * NT * u;
      if (h < H) {
        wv[u] = *reinterpret_cast<const f32x4*>(row + h);
        xv[u] = *reinterpret_cast<const u32x2*>(x + h);
      }
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      if (h0 + 4 * NT * u < H) {
        acc = fmaf(bf16_to_f32(xv[u].x & 0xFFFFu), wv[u].x, acc);
        acc = fmaf(bf16_to_f32(xv[u].x >> 16), wv[u].y, acc);
        acc = fmaf(bf16_to_f32(xv[u].y & 0xFFFFu), wv[u].z, acc);
        acc = fmaf(bf16_to_f32(xv[u].y >> 16), wv[u].w, acc);
      }
    }
  }
  return acc;
}

// The same chain for the nt <= TT tokens of x (rows H apart) at once: the row
// piece is loaded once for all of them, and each token's FMAs run in exactly
// router_thread_sum's order, so acc[tt] equals router_thread_sum for token tt.
template <int NT, int TT>
__device__ __forceinline__ void router_thread_sums(const float* __restrict__ row, const uint16_t* __restrict__ x,
                                                   int H, int nt, int j, float (&acc)[TT]) {
  constexpr int U = 8;
#pragma unroll
  for (int tt = 0; tt < TT; tt++) acc[tt] = 0.0f;
  for (int h0 = 4 * j; h0 < H; h0 += 4 * NT * U) {
    f32x4 wv[U];
    u32x2 xv[TT][U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int h = h0 + 4 * NT * u;
      if (h < H) {
        wv[u] = *reinterpret_cast<const f32x4*>(row + h);
#pragma unroll
        for (int tt = 0; tt < TT; tt++)
          if (tt < nt) xv[tt][u] = *reinterpret_cast<const u32x2*>(x + (size_t)tt * H + h);
      }
    }
#pragma unroll
    for (int tt = 0; tt < TT; tt++) {
      if (tt >= nt) continue;
#pragma unroll
      for (int u = 0; u < U; u++) {
        if (h0 + 4 * NT * u < H) {
          acc[tt] = fmaf(bf16_to_f32(xv[tt][u].x & 0xFFFFu), wv[u].x, acc[tt]);
          acc[tt] = fmaf(bf16_to_f32(xv[tt][u].x >> 16), wv[u].y, acc[tt]);
          acc[tt] = fmaf(bf16_to_f32(xv[tt][u].y & 0xFFFFu), wv[u].z, acc[tt]);
          acc[tt] = fmaf(bf16_to_f32(xv[tt][u].y >> 16), wv[u].w, acc[tt]);
        }
      }
    }
  }
}

}  // namespace moe
