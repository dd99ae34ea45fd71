// Helpers of the expert-streaming (GEMV) kernels: quads of NVFP4 codes and
// scales, packed-bf16 activation reads from LDS, and row-group reductions.
//
// A quad is 64 inputs of one weight row: 4 E4M3 blocks ("Beam 1.0 501B-A23B,
// streaming pack, NVFP4 experts / MLX 8-bit residents", "What this pack
// holds": one scale per 16 inputs), i.e. 32 bytes of codes (8 U32 words) and
// 4 scale bytes.
#pragma once
#include "common.h"

namespace moe {

// one quad of one projection: 8 code words + 4 scale bytes
struct Quad {
  u32x4 c0, c1;
  uint32_t s;
};

__device__ __forceinline__ Quad load_quad(const uint8_t* row_codes, const uint8_t* row_scales, int q) {
  Quad v;
  const u32x4* cp = reinterpret_cast<const u32x4*>(row_codes + 32 * (size_t)q);
  v.c0 = cp[0];
  v.c1 = cp[1];
  v.s = *reinterpret_cast<const uint32_t*>(row_scales + 4 * (size_t)q);
  return v;
}

// Inputs staged in LDS sit in 16-byte chunks (8 bf16 values), 8 chunks per
// 64-input quad, chunk c of quad q at chunk position 8 q + (c ^ (q & 7)). The
// lanes of a row read different quads at once, 128 bytes apart, i.e. half the
// LDS's 64 four-byte banks apart: stored in order, the 16-byte reads of 8 or
// 16 consecutive quads would fall on two sets of four banks (a 4- or 8-way
// conflict); swizzled, 8 consecutive quads cover every bank once.
__device__ __forceinline__ int xchunk(int q, int c) { return 8 * q + (c ^ (q & 7)); }

// the 8 packed input pairs of block b (0..3) of quad q of an LDS input buffer
// (q counted from the buffer's start)
__device__ __forceinline__ void load_x8(const uint32_t* xbuf, int q, int b, uint32_t* xw) {
  const u32x4 v0 = *reinterpret_cast<const u32x4*>(xbuf + 4 * xchunk(q, 2 * b));
  const u32x4 v1 = *reinterpret_cast<const u32x4*>(xbuf + 4 * xchunk(q, 2 * b + 1));
  xw[0] = v0.x;
  xw[1] = v0.y;
  xw[2] = v0.z;
  xw[3] = v0.w;
  xw[4] = v1.x;
  xw[5] = v1.y;
  xw[6] = v1.z;
  xw[7] = v1.w;
}

// code words of block b of a quad
__device__ __forceinline__ uint32_t quad_word(const Quad& v, int i) {
  switch (i) {
    case 0: return v.c0.x;
    case 1: return v.c0.y;
    case 2: return v.c0.z;
    case 3: return v.c0.w;
    case 4: return v.c1.x;
    case 5: return v.c1.y;
    case 6: return v.c1.z;
    default: return v.c1.w;
  }
}

__device__ __forceinline__ float quad_scale(const Quad& v, int b) {
  switch (b) {
    case 0: return e4m3_f32<0>(v.s);
    case 1: return e4m3_f32<1>(v.s);
    case 2: return e4m3_f32<2>(v.s);
    default: return e4m3_f32<3>(v.s);
  }
}

// Sum over each aligned group of G (2..16) lanes, left in the group's last
// lane (sub == G - 1): DPP row shifts inside a 16-lane row, no LDS traffic.
// Other lanes hold partial sums.
template <int G>
__device__ __forceinline__ float group_sum_last(float v) {
  static_assert(G >= 2 && G <= 16 && (G & (G - 1)) == 0, "G: 2..16, a power of two");
  v += dpp_f32<0x111>(v);                     // row_shr:1
  if (G > 2) v += dpp_f32<0x112>(v);          // row_shr:2
  if (G > 4) v += dpp_f32<0x114>(v);          // row_shr:4
  if (G > 8) v += dpp_f32<0x118>(v);          // row_shr:8
  return v;
}

template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = G / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace moe
