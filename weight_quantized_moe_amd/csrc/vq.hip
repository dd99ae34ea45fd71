// Expert-streaming kernels for the 8-dim VQ expert format.
//
// "Beam-1.0-501B-A23B VQ GGUF", "Recipe", routed-experts bullet: every 8
// consecutive weights of an expert row are one index into a codebook of
// E4M3 codewords shared by all experts and by gate/up/down, times one F16
// gain per row; 12-bit indices give 4,096 codewords of 8 bytes (32 KiB, the
// size the page's "Kernel budget on GB10" leaves room for beside 40 KiB of
// mids). Index j of a row is bits 12j..12j+11 of the row's little-endian
// bit stream, so 8 indices (64 weights) are 12 bytes.
//
// Each workgroup stages the codebook into LDS. A weight row is read as
// groups of 8 indices (three U32 words); each index fetches its 8-byte
// codeword from LDS, gfx950 turns each pair of E4M3 bytes into two bf16
// values (exact: E4M3 has 3 mantissa bits), and v_dot2 multiplies them with
// the bf16 inputs, accumulating in f32. The row's F16 gain multiplies the
// row sum. SwiGLU in FP32 and BF16 mids as for the NVFP4 records ([VQ] "What
// stays native", "Kernel budget on GB10").
#include "common.h"
#include "dma.h"
#include "gemv_util.h"
#include "internal.h"

namespace moe {

constexpr int kVqCodebookBytes = 4096 * 8;
constexpr int kVqThreads = 256;

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// the 8 indices of a 12-byte group (words w0, w1, w2, little-endian)
__device__ __forceinline__ void unpack8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t (&c)[8]) {
  c[0] = w0 & 0xFFFu;
  c[1] = (w0 >> 12) & 0xFFFu;
  c[2] = (w0 >> 24) | ((w1 & 0xFu) << 8);
  c[3] = (w1 >> 4) & 0xFFFu;
  c[4] = (w1 >> 16) & 0xFFFu;
  c[5] = (w1 >> 28) | ((w2 & 0xFFu) << 4);
  c[6] = (w2 >> 8) & 0xFFFu;
  c[7] = w2 >> 20;
}

// two E4M3 bytes (the low or high half of a word) as two exact bf16 values,
// the lower byte in the low half
template <bool HI>
__device__ __forceinline__ bf16x2 e4m3x2_bf16(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, HI);
}

// sum over the 8 weights of codeword c (LDS) times 8 inputs (4 packed bf16
// pairs at xp, LDS)
__device__ __forceinline__ float cw_dot8(const uint8_t* cb, uint32_t c, const uint32_t* xp, float s) {
  const u32x2 cw = *reinterpret_cast<const u32x2*>(cb + 8 * c);
  const u32x4 xv = *reinterpret_cast<const u32x4*>(xp);
  s = dot2(e4m3x2_bf16<false>(cw.x), xv.x, s);
  s = dot2(e4m3x2_bf16<true>(cw.x), xv.y, s);
  s = dot2(e4m3x2_bf16<false>(cw.y), xv.z, s);
  s = dot2(e4m3x2_bf16<true>(cw.y), xv.w, s);
  return s;
}

struct Grp {
  uint32_t w0, w1, w2;
};

__device__ __forceinline__ Grp load_grp(const uint8_t* row, int g) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(row + 12 * (size_t)g);
  return Grp{p[0], p[1], p[2]};
}

// sum over group g of an input buffer: 8 indices against its inputs 64 g ..
// 64 g + 63 (xbuf: packed bf16 pairs in LDS in the swizzled chunk layout of
// gemv_util.h, a group being a quad there; g counted from the buffer's
// start). The swizzle keeps the 16-byte input reads of a wave's lanes, which
// take different groups, off each other's banks: 24.4 -> 19.7 us for the
// one-token gate/up launch, 15.3 -> 12.5 us for down.
__device__ __forceinline__ float grp_dot(const uint8_t* cb, const Grp& q, const uint32_t* xbuf, int g, float s) {
  uint32_t c[8];
  unpack8(q.w0, q.w1, q.w2, c);
#pragma unroll
  for (int i = 0; i < 8; i++) s = cw_dot8(cb, c[i], xbuf + 4 * xchunk(g, i), s);
  return s;
}

// Gate/up + SwiGLU. Workgroup (blockIdx.x, pair p = blockIdx.y): wave w takes
// rows 16 blockIdx.x + 4 w .. + 3 of gate and up; 16 lanes share a row, lane
// sub taking the groups sub, sub + 16, ... (all its loads issued before any
// arithmetic). LDS: codebook | x of the pair's token.
__global__ __launch_bounds__(kVqThreads) void vq_gateup_kernel(VqArgs a) {
  constexpr int G = 16, R = 64 / G, QB = 5;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t* cb = lds;
  uint32_t* xs = reinterpret_cast<uint32_t*>(lds + kVqCodebookBytes);
  const int H = a.H, I = a.I, ngrp = H / 64;
  const int p = blockIdx.y, t = p / a.k;
  const int e = a.idx[p];
  if (e < 0 || e >= a.E) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rsub = lane / G, sub = lane % G;
  dma_copy_lds(a.codebook, cb, kVqCodebookBytes, kVqThreads / 64);
  const int r = (blockIdx.x * (kVqThreads / 64) + wave) * R + rsub;
  const bool row_ok = r < I;
  const uint8_t* rec = a.bank + (size_t)e * a.stride;
  const size_t row_bytes = (size_t)H * 3 / 16;
  const uint8_t* rg = rec + a.idx_off[0] + (size_t)(row_ok ? r : 0) * row_bytes;
  const uint8_t* ru = rec + a.idx_off[1] + (size_t)(row_ok ? r : 0) * row_bytes;
  Grp qg[QB], qu[QB];
  float acc_g = 0.0f, acc_u = 0.0f;
  // x of token t -> LDS, while the first index loads are in flight
  const u32x4* xsrc = reinterpret_cast<const u32x4*>(a.x + (size_t)t * H);
  for (int qb = 0; qb < ngrp; qb += G * QB) {
#pragma unroll
    for (int i = 0; i < QB; i++) {
      const int g = qb + sub + G * i;
      if (row_ok && g < ngrp) {
        qg[i] = load_grp(rg, g);
        qu[i] = load_grp(ru, g);
      }
    }
    if (qb == 0) {
      for (int i = threadIdx.x; i < H / 8; i += kVqThreads) reinterpret_cast<u32x4*>(xs)[xchunk(i >> 3, i & 7)] = xsrc[i];
      wait_vmcnt<0>();
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < QB; i++) {
      const int g = qb + sub + G * i;
      if (row_ok && g < ngrp) {
        acc_g = grp_dot(cb, qg[i], xs, g, acc_g);
        acc_u = grp_dot(cb, qu[i], xs, g, acc_u);
      }
    }
  }
  const float sg = group_sum_last<G>(acc_g), su = group_sum_last<G>(acc_u);
  if (sub == G - 1 && row_ok) {
    const uint16_t* gains_g = reinterpret_cast<const uint16_t*>(rec + a.gain_off[0]);
    const uint16_t* gains_u = reinterpret_cast<const uint16_t*>(rec + a.gain_off[1]);
    const float gv = sg * f16_to_f32(gains_g[r]);
    const float uv = su * f16_to_f32(gains_u[r]);
    a.mid[(size_t)p * I + r] = f32_to_bf16(silu_mul(gv, uv));
  }
}

// Down + weighted combine. Workgroup (8 output rows from 8 blockIdx.x, token
// t = blockIdx.y), one wave per pair j < k; 8 lanes share a row. LDS:
// codebook | the token's k rows of mids. The k routing-weighted row sums meet
// in LDS and are added in slot order onto the residual.
__global__ __launch_bounds__(64 * kFlatDecodeMaxK) void vq_down_kernel(VqArgs a) {
  constexpr int G = 8, R = 64 / G, QB = 5;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ float s_d[kFlatDecodeMaxK][R];
  uint8_t* cb = lds;
  uint32_t* ms = reinterpret_cast<uint32_t*>(lds + kVqCodebookBytes);
  const int H = a.H, I = a.I, k = a.k, ngrp = I / 64;
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63, j = threadIdx.x >> 6;
  const int rsub = lane / G, sub = lane % G;
  const int r = blockIdx.x * R + rsub;
  const bool row_ok = r < H;
  const int p = t * k + j;
  const int e = a.idx[p];
  const bool valid = e >= 0 && e < a.E;
  const uint8_t* rec = a.bank + (size_t)(valid ? e : 0) * a.stride;
  const size_t row_bytes = (size_t)I * 3 / 16;
  const uint8_t* rd = rec + a.idx_off[2] + (size_t)(row_ok ? r : 0) * row_bytes;
  dma_copy_lds(a.codebook, cb, kVqCodebookBytes, k);
  dma_copy_lds_swz(a.mid + (size_t)t * k * I, ms, (uint32_t)(k * I * 2), k);
  Grp q[QB];
  if (valid) {
#pragma unroll
    for (int i = 0; i < QB; i++) {
      const int g = sub + G * i;
      if (row_ok && g < ngrp) q[i] = load_grp(rd, g);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();
  float acc = 0.0f;
  if (valid) {
    const int g0 = j * ngrp;  // the pair's mids start at this group of the buffer
    for (int qb = 0; qb < ngrp; qb += G * QB) {
      if (qb > 0) {
#pragma unroll
        for (int i = 0; i < QB; i++) {
          const int g = qb + sub + G * i;
          if (row_ok && g < ngrp) q[i] = load_grp(rd, g);
        }
      }
#pragma unroll
      for (int i = 0; i < QB; i++) {
        const int g = qb + sub + G * i;
        if (row_ok && g < ngrp) acc = grp_dot(cb, q[i], ms, g0 + g, acc);
      }
    }
  }
  const float d = group_sum_last<G>(acc);
  if (sub == G - 1) {
    float v = 0.0f;
    if (valid && row_ok) {
      const uint16_t* gains = reinterpret_cast<const uint16_t*>(rec + a.gain_off[2]);
      v = a.w[p] * (d * f16_to_f32(gains[r]));
    }
    s_d[j][rsub] = v;
  }
  __syncthreads();
  if (threadIdx.x < R) {
    const int rr = blockIdx.x * R + threadIdx.x;
    if (rr < H) {
      const size_t o = (size_t)t * H + rr;
      float y = a.residual ? bf16_to_f32(a.residual[o]) : 0.0f;
      for (int jj = 0; jj < k; jj++) y += s_d[jj][threadIdx.x];  // slot order
      if (a.f32_out)
        reinterpret_cast<float*>(a.y)[o] = y;
      else
        reinterpret_cast<uint16_t*>(a.y)[o] = f32_to_bf16(y);
    }
  }
}

// test export: the f32 weights of one projection through the kernels'
// conversion path (codeword bytes -> bf16 pairs -> f32, times the f32 gain),
// one thread per index
__global__ __launch_bounds__(256) void vq_dequant_kernel(VqArgs a, int expert, int proj, float* out) {
  const int rows = proj == 2 ? a.H : a.I, in = proj == 2 ? a.I : a.H;
  const size_t n_idx = (size_t)rows * (in / 8);
  const size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= n_idx) return;
  const size_t r = q / (in / 8), jj = q % (in / 8);
  const uint8_t* rec = a.bank + (size_t)expert * a.stride;
  const uint8_t* row = rec + a.idx_off[proj] + r * ((size_t)in * 3 / 16);
  const size_t bit = 12 * jj;
  const uint32_t c = ((uint32_t)row[bit / 8] | ((uint32_t)row[bit / 8 + 1] << 8)) >> (bit % 8) & 0xFFFu;
  const float gain = f16_to_f32(reinterpret_cast<const uint16_t*>(rec + a.gain_off[proj])[r]);
  const u32x2 cw = *reinterpret_cast<const u32x2*>(a.codebook + 8 * c);
  const bf16x2 v[4] = {e4m3x2_bf16<false>(cw.x), e4m3x2_bf16<true>(cw.x), e4m3x2_bf16<false>(cw.y),
                       e4m3x2_bf16<true>(cw.y)};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t b = __builtin_bit_cast(uint32_t, v[i]);
    out[r * in + 8 * jj + 2 * i] = bf16_to_f32(b & 0xFFFFu) * gain;
    out[r * in + 8 * jj + 2 * i + 1] = bf16_to_f32(b >> 16) * gain;
  }
}

hipError_t launch_vq_forward(const VqArgs& a, hipStream_t s) {
  const int P = a.T * a.k;
  if (P == 0) return hipSuccess;
  launch_kernel("vq_gateup", vq_gateup_kernel, dim3((a.I + 15) / 16, P), dim3(kVqThreads),
                (uint32_t)(kVqCodebookBytes + a.H * 2), s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_kernel("vq_down", vq_down_kernel, dim3((a.H + 7) / 8, a.T), dim3(64 * a.k),
                (uint32_t)(kVqCodebookBytes + a.k * a.I * 2), s, a);
  return hipGetLastError();
}

hipError_t launch_vq_dequant(const VqArgs& a, int expert, int proj, float* out, hipStream_t s) {
  const int rows = proj == 2 ? a.H : a.I, in = proj == 2 ? a.I : a.H;
  const size_t n_idx = (size_t)rows * (in / 8);
  launch_kernel("vq_dequant", vq_dequant_kernel, dim3((unsigned)((n_idx + 255) / 256)), dim3(256), 0, s, a, expert,
                proj, out);
  return hipGetLastError();
}

}  // namespace moe
