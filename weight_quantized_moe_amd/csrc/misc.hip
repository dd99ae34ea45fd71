// Smaller kernels of libmoe_mi355x.so for gfx950: record pad zeroing (pack),
// the dequant test export, the weightless RMS norm between stacked layers, and
// the affine8_g64 resident linear.
#include "common.h"
#include "internal.h"

namespace moe {

// ---- pack: zero the pad after each record ------------------------------------
__global__ void zero_tails_kernel(uint8_t* base, uint64_t stride, uint64_t record_bytes, int E) {
  const uint64_t pad = stride - record_bytes;
  const uint64_t n = pad * (uint64_t)E;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t e = i / pad, o = i % pad;
    base[e * stride + record_bytes + o] = 0;
  }
}

hipError_t launch_zero_tails(uint8_t* base, uint64_t stride, uint64_t record_bytes, int E,
                             hipStream_t s) {
  const uint64_t n = (stride - record_bytes) * (uint64_t)E;
  if (n == 0) return hipSuccess;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(zero_tails_kernel, dim3(blocks), dim3(256), 0, s, base, stride, record_bytes, E);
  return hipGetLastError();
}

// ---- dequant test export ("Beam 1.0 501B-A23B, streaming pack, NVFP4 experts /
// MLX 8-bit residents", "What this pack holds", global-scales bullet):
// w = e2m1 * f32(e4m3 * f32(g / 2688)), u = e2m1 * e4m3 (exact in bf16). The
// E2M1 values come from the same conversions the layer kernels use: the bf16
// one (decode GEMV) for w, the f32 one (grouped-GEMM tiles) for u.
__global__ void dequant_kernel(const uint8_t* codes, const uint8_t* scales, const uint8_t* gp,
                               int rows, int cols, float* out_f32, uint16_t* out_unit) {
  const int words_per_row = cols / 8;
  const size_t n = (size_t)rows * words_per_row;
  const float t = global_factor(*reinterpret_cast<const float*>(gp));
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / words_per_row, wq = i % words_per_row;
    const uint32_t word = reinterpret_cast<const uint32_t*>(codes + r * (cols / 2))[wq];
    const uint32_t sbyte = scales[r * (cols / 16) + (wq * 8) / 16];
    const float s = e4m3_f32_dyn(sbyte);
    const float S = s * t;
    float e2b[8], e2f[8];
    {
      bf16x2 b0 = e2m1x2_bf16<0>(word), b1 = e2m1x2_bf16<1>(word);
      bf16x2 b2 = e2m1x2_bf16<2>(word), b3 = e2m1x2_bf16<3>(word);
      uint32_t u0 = __builtin_bit_cast(uint32_t, b0), u1 = __builtin_bit_cast(uint32_t, b1);
      uint32_t u2 = __builtin_bit_cast(uint32_t, b2), u3 = __builtin_bit_cast(uint32_t, b3);
      uint32_t us[4] = {u0, u1, u2, u3};
#pragma unroll
      for (int q = 0; q < 4; q++) {
        e2b[2 * q] = bf16_to_f32(us[q] & 0xFFFFu);
        e2b[2 * q + 1] = bf16_to_f32(us[q] >> 16);
      }
      f32x2 f0 = e2m1x2_f32<0>(word), f1 = e2m1x2_f32<1>(word);
      f32x2 f2 = e2m1x2_f32<2>(word), f3 = e2m1x2_f32<3>(word);
      e2f[0] = f0.x; e2f[1] = f0.y; e2f[2] = f1.x; e2f[3] = f1.y;
      e2f[4] = f2.x; e2f[5] = f2.y; e2f[6] = f3.x; e2f[7] = f3.y;
    }
    const size_t o = r * (size_t)cols + wq * 8;
#pragma unroll
    for (int q = 0; q < 8; q++) {
      if (out_f32) out_f32[o + q] = e2b[q] * S;
      if (out_unit) out_unit[o + q] = f32_to_bf16(e2f[q] * s);
    }
  }
}

hipError_t launch_dequant(const BankView& b, int expert, int proj, float* out_f32,
                          uint16_t* out_unit, hipStream_t s) {
  const int rows = (proj == 2) ? b.H : b.I, cols = (proj == 2) ? b.I : b.H;
  const uint8_t* rec = b.base + (size_t)expert * b.stride;
  size_t n = (size_t)rows * cols / 8;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(dequant_kernel, dim3(blocks), dim3(256), 0, s, rec + b.codes[proj],
                     rec + b.scales[proj], rec + b.g[proj], rows, cols, out_f32, out_unit);
  return hipGetLastError();
}

// ---- weightless RMS norm -------------------------------------------------------
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* x, int H, float eps,
                                                      uint16_t* y) {
  const size_t t = blockIdx.x;
  const uint16_t* xr = x + t * H;
  float ss = 0.0f;
  for (int h = threadIdx.x; h < H; h += 256) {
    float v = bf16_to_f32(xr[h]);
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
  for (int h = threadIdx.x; h < H; h += 256) y[t * H + h] = f32_to_bf16(bf16_to_f32(xr[h]) * inv);
}

hipError_t launch_rmsnorm(const uint16_t* x, int T, int H, float eps, uint16_t* y, hipStream_t s) {
  launch_kernel("rmsnorm", rmsnorm_kernel, dim3(T), dim3(256), 0, s, x, H, eps, y);
  return hipGetLastError();
}

// ---- affine8_g64 resident linear ("Beam 1.0 501B-A23B, streaming pack, NVFP4
// experts / MLX 8-bit residents", residents and q8-rule bullets) --------------------
// y[t][n] = sum_g scale[n][g] * (sum_{k in g} x[t][k] q[n][k]) + bias[n][g] * (sum_{k in g} x[t][k]).
// Bandwidth-bound for small T: a wave owns one output row, its lanes sweep the
// row's 8-bit codes 16 bytes at a time (64 lanes x 16 B = 1 KiB per load).
// A code q <= 255 has at most 8 significant bits, so it is exact in bf16: two
// codes become one packed bf16 pair (byte -> f32 -> high half), and v_dot2
// multiplies them with a pair of activations. The activations (bf16 pairs) and
// their 16-element partial sums (for the bias term) sit in LDS, 4 tokens per
// pass.
constexpr int kAffTok = 4;
constexpr int kAffRows = 16;

__device__ __forceinline__ uint32_t u8pair_bf16(uint32_t word, int lo_byte) {
  const float a = (float)((word >> (8 * lo_byte)) & 0xFFu);
  const float b = (float)((word >> (8 * lo_byte + 8)) & 0xFFu);
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
}

__global__ __launch_bounds__(256) void affine8_kernel(const uint16_t* __restrict__ x,
                                                      const uint32_t* __restrict__ codes,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint16_t* __restrict__ biases, int T,
                                                      int K, int N, uint16_t* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  uint32_t* xs = lds;                                          // [kAffTok][K/2] bf16 pairs
  float* xc = reinterpret_cast<float*>(lds + kAffTok * (K / 2));  // [kAffTok][K/16]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = K / 64, C16 = K / 16;
  const int r0 = blockIdx.x * kAffRows, r1 = min(N, r0 + kAffRows);
  for (int t0 = 0; t0 < T; t0 += kAffTok) {
    const int nt = min(kAffTok, T - t0);
    __syncthreads();
    for (int i = threadIdx.x; i < kAffTok * (K / 2); i += 256) {
      int tt = i / (K / 2), kk = i % (K / 2);
      xs[i] = (tt < nt) ? reinterpret_cast<const uint32_t*>(x + (size_t)(t0 + tt) * K)[kk] : 0u;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kAffTok * C16; i += 256) {
      int tt = i / C16, c = i % C16;
      float s = 0.0f;
      for (int q = 0; q < 8; q++) {
        uint32_t pr = xs[tt * (K / 2) + 8 * c + q];
        s += bf16_to_f32(pr & 0xFFFFu) + bf16_to_f32(pr >> 16);
      }
      xc[i] = s;
    }
    __syncthreads();
    for (int r = r0 + wave; r < r1; r += 4) {
      float acc[kAffTok];
#pragma unroll
      for (int tt = 0; tt < kAffTok; tt++) acc[tt] = 0.0f;
      const uint8_t* row = reinterpret_cast<const uint8_t*>(codes) + (size_t)r * K;
      for (int c = lane; c < C16; c += 64) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(row + 16 * (size_t)c);
        const int g = c / 4;
        const float sc = bf16_to_f32(scales[(size_t)r * G + g]);
        const float bi = bf16_to_f32(biases[(size_t)r * G + g]);
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
        uint32_t qp[8];
#pragma unroll
        for (int b = 0; b < 4; b++) {
          qp[2 * b] = u8pair_bf16(wv[b], 0);
          qp[2 * b + 1] = u8pair_bf16(wv[b], 2);
        }
#pragma unroll
        for (int tt = 0; tt < kAffTok; tt++) {
          if (tt < nt) {
            const u32x4* xp = reinterpret_cast<const u32x4*>(xs + tt * (K / 2) + 8 * c);
            const u32x4 xa = xp[0], xb = xp[1];
            const uint32_t xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; j++) s = dot2(__builtin_bit_cast(bf16x2, qp[j]), xv[j], s);
            acc[tt] = fmaf(sc, s, fmaf(bi, xc[tt * C16 + c], acc[tt]));
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < kAffTok; tt++) {
        if (tt < nt) {
          float v = wave_sum(acc[tt]);
          if (lane == 0) y[(size_t)(t0 + tt) * N + r] = f32_to_bf16(v);
        }
      }
    }
  }
}

hipError_t launch_affine8(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                          const uint16_t* biases, int T, int K, int N, uint16_t* y, hipStream_t s) {
  size_t lds = (size_t)kAffTok * (K / 2) * 4 + (size_t)kAffTok * (K / 16) * 4;
  launch_kernel("affine8", affine8_kernel, dim3((N + kAffRows - 1) / kAffRows), dim3(256), (uint32_t)lds, s, x,
                codes, scales, biases, T, K, N, y);
  return hipGetLastError();
}

}  // namespace moe
