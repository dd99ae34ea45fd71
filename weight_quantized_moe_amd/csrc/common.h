// Device helpers shared by the gfx950 kernels of libmoe_mi355x.so.
//
// Number formats ("Beam 1.0 501B-A23B, streaming pack, NVFP4 experts / MLX 8-bit
// residents", "What this pack holds": E2M1 codes in U32 words, E4M3 block scales,
// f32 globals; BF16 activations) are decoded with gfx950's conversion
// instructions:
//   - v_cvt_scalef32_pk_bf16_fp4 / _f32_fp4 turn one byte (two E2M1 codes, low
//     nibble first) into two values. The instruction scales by a power of two
//     only (it uses the exponent of its f32 scale operand), so it is always
//     called with scale 1.0 and the E4M3 block scale is applied separately.
//   - v_cvt_f32_fp8 decodes an OCP E4M3FN byte exactly.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// f32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  f32x2 v = {f, 0.0f};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b) & 0xFFFFu;
}

__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// E2M1 codes of byte `sel` (0..3) of a U32 word, as two exact bf16 values
// (element 2*sel in the low half, 2*sel+1 in the high half).
template <int SEL>
__device__ __forceinline__ bf16x2 e2m1x2_bf16(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, SEL);
}

template <int SEL>
__device__ __forceinline__ f32x2 e2m1x2_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
}

// E4M3FN byte `sel` of a U32 word as f32 (exact)
template <int SEL>
__device__ __forceinline__ float e4m3_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8(word, SEL);
}

__device__ __forceinline__ float e4m3_f32_dyn(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8(byte, 0);
}

// a.x*b.x + a.y*b.y + c, f32 accumulate (v_dot2c_f32_bf16)
__device__ __forceinline__ float dot2(bf16x2 a, uint32_t b_bits, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2, b_bits), c, false);
}

// sum of the 16 products of one E4M3 block: 8 bytes of codes (two U32 words)
// against 16 bf16 inputs (8 packed pairs)
__device__ __forceinline__ float block_dot16(uint32_t w0, uint32_t w1, const uint32_t* xp) {
  float s = 0.0f;
  s = dot2(e2m1x2_bf16<0>(w0), xp[0], s);
  s = dot2(e2m1x2_bf16<1>(w0), xp[1], s);
  s = dot2(e2m1x2_bf16<2>(w0), xp[2], s);
  s = dot2(e2m1x2_bf16<3>(w0), xp[3], s);
  s = dot2(e2m1x2_bf16<0>(w1), xp[4], s);
  s = dot2(e2m1x2_bf16<1>(w1), xp[5], s);
  s = dot2(e2m1x2_bf16<2>(w1), xp[6], s);
  s = dot2(e2m1x2_bf16<3>(w1), xp[7], s);
  return s;
}

// DPP move of a float from another lane of the same 16-lane row (CTRL: a
// dpp_ctrl value, e.g. 0x111 = row_shr:1); lanes with no source read 0.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// global factor t = f32(g / 2688): IEEE division (hipcc keeps f32 division
// correctly rounded unless fast-math is requested, which this library never
// does)
__device__ __forceinline__ float global_factor(float g) { return g / 2688.0f; }

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

// Total order of logits for top-k as an unsigned key: larger logit first,
// -0 and +0 equal, NaN below every number.
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7FFFFFFFu) == 0) b = 0;                     // -0 -> +0
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0;        // NaN: below everything
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);    // monotone in v
}

}  // namespace moe
