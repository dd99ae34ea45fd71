// Expert-streaming kernels (decode: few tokens per expert) for gfx950.
//
// S4 gate/up, S5 SwiGLU and S6 down of the routed-expert layer over NVFP4
// expert records ("Beam 1.0 501B-A23B, streaming pack, NVFP4 experts / MLX 8-bit
// residents", "What this pack holds": E2M1 codes in U32 words, one E4M3 scale
// per 16 inputs, per-projection f32 global g applied as e4m3 * (g / 2688)).
// SwiGLU in FP32 and BF16 mids follow "Beam-1.0-501B-A23B VQ GGUF" ("What stays
// native", "Kernel budget on GB10").
//
// These kernels are bound by HBM bandwidth: every weight byte is read once per
// call. A block owns one active expert and a tile of output rows; a wave owns
// one row at a time and its 64 lanes sweep the row's input blocks, lane l
// taking blocks l, l+64, ... so each load instruction reads 512 contiguous
// bytes of codes. Each 8-byte chunk is one E4M3 block (16 E2M1 codes): two
// U32 words turn into 8 packed bf16 pairs (v_cvt_scalef32_pk_bf16_fp4), eight
// v_dot2 give the block's partial sum, and one FMA applies the block scale
// S = f32(e4m3 * t). The expert's token activations sit in LDS; the weights
// stay in registers while every token of the pass is applied to them.
#include "common.h"
#include "internal.h"

namespace moe {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kGateUpRows = 16;  // rows of gate (and of up) per block
constexpr int kDownRows = 32;    // rows of down per block
constexpr int kDecTok = 4;       // tokens per pass (activations staged in LDS)
constexpr int kChunksPerLane = 5;

struct DecodeArgs {
  const uint8_t* bank;
  uint64_t stride;
  uint64_t codes[3], scales[3], g[3];
  int H, I, k;
  const uint16_t* in;   // gate/up: x [T][H]; down: mid [P][I] in sorted order
  const float* w;       // down: routing weights [T*k]
  RouteTables rt;
  uint16_t* mid;        // gate/up output [P][I], sorted order
  float* part;          // down output [P][H], pair order
};

// Stage the bf16 input rows of tokens m0..m0+mt-1 of expert slot range s0 into
// LDS: xs[m][0..len/2) as packed pairs. 16-byte copies; len % 8 == 0.
__device__ __forceinline__ void stage_rows(uint32_t* xs, const uint16_t* src, int len,
                                           const int32_t* sorted, int s0, int m0, int mt, int k,
                                           bool by_token) {
  for (int m = 0; m < mt; m++) {
    size_t row = by_token ? (size_t)(sorted[s0 + m0 + m] / k) : (size_t)(s0 + m0 + m);
    const u32x4* s = reinterpret_cast<const u32x4*>(src + row * (size_t)len);
    u32x4* d = reinterpret_cast<u32x4*>(xs + m * (len / 2));
    for (int i = threadIdx.x; i < len / 8; i += kDecThreads) d[i] = s[i];
  }
}

__device__ __forceinline__ void lds_x16(const uint32_t* xrow, int blk, uint32_t* xv) {
  const u32x4* p = reinterpret_cast<const u32x4*>(xrow + 8 * blk);
  u32x4 a = p[0], b = p[1];
  xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
  xv[4] = b.x; xv[5] = b.y; xv[6] = b.z; xv[7] = b.w;
}

// ---- S4 + S5 ------------------------------------------------------------------
__global__ __launch_bounds__(kDecThreads) void decode_gateup_kernel(DecodeArgs a) {
  const int slot = blockIdx.y;
  if (slot >= a.rt.counts[0]) return;
  const int e = a.rt.active[slot];
  const int s0 = a.rt.offsets[e], M = a.rt.offsets[e + 1] - s0;
  const int H = a.H, I = a.I, NB = H / 16;
  const uint8_t* rec = a.bank + (size_t)e * a.stride;
  const uint8_t* cg = rec + a.codes[0];
  const uint8_t* sg = rec + a.scales[0];
  const uint8_t* cu = rec + a.codes[1];
  const uint8_t* su = rec + a.scales[1];
  const float tg = global_factor(*reinterpret_cast<const float*>(rec + a.g[0]));
  const float tu = global_factor(*reinterpret_cast<const float*>(rec + a.g[1]));
  extern __shared__ uint32_t xs[];  // [kDecTok][H/2]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = blockIdx.x * kGateUpRows, r1 = min(I, r0 + kGateUpRows);
  for (int m0 = 0; m0 < M; m0 += kDecTok) {
    const int mt = min(kDecTok, M - m0);
    __syncthreads();
    stage_rows(xs, a.in, H, a.rt.sorted, s0, m0, mt, a.k, true);
    __syncthreads();
    for (int r = r0 + wave; r < r1; r += kDecWaves) {
      float ag[kDecTok], au[kDecTok];
#pragma unroll
      for (int m = 0; m < kDecTok; m++) ag[m] = au[m] = 0.0f;
      const uint8_t* rcg = cg + (size_t)r * (H / 2);
      const uint8_t* rcu = cu + (size_t)r * (H / 2);
      const uint8_t* rsg = sg + (size_t)r * NB;
      const uint8_t* rsu = su + (size_t)r * NB;
      for (int cb = 0; cb < NB; cb += 64 * kChunksPerLane) {
        u32x2 wg[kChunksPerLane], wu[kChunksPerLane];
        uint32_t bg[kChunksPerLane], bu[kChunksPerLane];
#pragma unroll
        for (int i = 0; i < kChunksPerLane; i++) {
          int c = cb + lane + 64 * i;
          if (c < NB) {
            wg[i] = *reinterpret_cast<const u32x2*>(rcg + 8 * (size_t)c);
            wu[i] = *reinterpret_cast<const u32x2*>(rcu + 8 * (size_t)c);
            bg[i] = rsg[c];
            bu[i] = rsu[c];
          }
        }
#pragma unroll
        for (int i = 0; i < kChunksPerLane; i++) {
          int c = cb + lane + 64 * i;
          if (c < NB) {
            const float Sg = e4m3_f32_dyn(bg[i]) * tg;
            const float Su = e4m3_f32_dyn(bu[i]) * tu;
#pragma unroll
            for (int m = 0; m < kDecTok; m++) {
              if (m < mt) {
                uint32_t xv[8];
                lds_x16(xs + m * (H / 2), c, xv);
                ag[m] = fmaf(Sg, block_dot16(wg[i].x, wg[i].y, xv), ag[m]);
                au[m] = fmaf(Su, block_dot16(wu[i].x, wu[i].y, xv), au[m]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int m = 0; m < kDecTok; m++) {
        if (m < mt) {
          float g = wave_sum(ag[m]);
          float u = wave_sum(au[m]);
          if (lane == 0) a.mid[(size_t)(s0 + m0 + m) * I + r] = f32_to_bf16(silu_mul(g, u));
        }
      }
    }
  }
}

hipError_t launch_decode_gateup(const BankView& b, const uint16_t* x, int k, const RouteTables& rt,
                                int slots, uint16_t* mid, hipStream_t s) {
  DecodeArgs a{};
  a.bank = b.base;
  a.stride = b.stride;
  for (int p = 0; p < 3; p++) {
    a.codes[p] = b.codes[p];
    a.scales[p] = b.scales[p];
    a.g[p] = b.g[p];
  }
  a.H = b.H;
  a.I = b.I;
  a.k = k;
  a.in = x;
  a.rt = rt;
  a.mid = mid;
  dim3 grid((b.I + kGateUpRows - 1) / kGateUpRows, slots);
  size_t lds = (size_t)kDecTok * b.H * 2;
  prof_begin("decode_gateup", s);
  hipLaunchKernelGGL(decode_gateup_kernel, grid, dim3(kDecThreads), lds, s, a);
  prof_end("decode_gateup", s);
  return hipGetLastError();
}

// ---- S6: down, per pair, scaled by the routing weight --------------------------
__global__ __launch_bounds__(kDecThreads) void decode_down_kernel(DecodeArgs a) {
  const int slot = blockIdx.y;
  if (slot >= a.rt.counts[0]) return;
  const int e = a.rt.active[slot];
  const int s0 = a.rt.offsets[e], M = a.rt.offsets[e + 1] - s0;
  const int H = a.H, I = a.I, NB = I / 16;
  const uint8_t* rec = a.bank + (size_t)e * a.stride;
  const uint8_t* cd = rec + a.codes[2];
  const uint8_t* sd = rec + a.scales[2];
  const float td = global_factor(*reinterpret_cast<const float*>(rec + a.g[2]));
  extern __shared__ uint32_t ms[];  // [kDecTok][I/2]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = blockIdx.x * kDownRows, r1 = min(H, r0 + kDownRows);
  for (int m0 = 0; m0 < M; m0 += kDecTok) {
    const int mt = min(kDecTok, M - m0);
    __syncthreads();
    stage_rows(ms, a.in, I, a.rt.sorted, s0, m0, mt, a.k, false);
    __syncthreads();
    float wt[kDecTok];
    int pr[kDecTok];
#pragma unroll
    for (int m = 0; m < kDecTok; m++) {
      pr[m] = (m < mt) ? a.rt.sorted[s0 + m0 + m] : 0;
      wt[m] = (m < mt) ? a.w[pr[m]] : 0.0f;
    }
    for (int r = r0 + wave; r < r1; r += kDecWaves) {
      float ad[kDecTok];
#pragma unroll
      for (int m = 0; m < kDecTok; m++) ad[m] = 0.0f;
      const uint8_t* rcd = cd + (size_t)r * (I / 2);
      const uint8_t* rsd = sd + (size_t)r * NB;
      for (int cb = 0; cb < NB; cb += 64 * kChunksPerLane) {
        u32x2 wd[kChunksPerLane];
        uint32_t bd[kChunksPerLane];
#pragma unroll
        for (int i = 0; i < kChunksPerLane; i++) {
          int c = cb + lane + 64 * i;
          if (c < NB) {
            wd[i] = *reinterpret_cast<const u32x2*>(rcd + 8 * (size_t)c);
            bd[i] = rsd[c];
          }
        }
#pragma unroll
        for (int i = 0; i < kChunksPerLane; i++) {
          int c = cb + lane + 64 * i;
          if (c < NB) {
            const float Sd = e4m3_f32_dyn(bd[i]) * td;
#pragma unroll
            for (int m = 0; m < kDecTok; m++) {
              if (m < mt) {
                uint32_t xv[8];
                lds_x16(ms + m * (I / 2), c, xv);
                ad[m] = fmaf(Sd, block_dot16(wd[i].x, wd[i].y, xv), ad[m]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int m = 0; m < kDecTok; m++) {
        if (m < mt) {
          float d = wave_sum(ad[m]);
          if (lane == 0) a.part[(size_t)pr[m] * H + r] = wt[m] * d;
        }
      }
    }
  }
}

hipError_t launch_decode_down(const BankView& b, const uint16_t* mid, const float* w, int k,
                              const RouteTables& rt, int slots, float* part, hipStream_t s) {
  DecodeArgs a{};
  a.bank = b.base;
  a.stride = b.stride;
  for (int p = 0; p < 3; p++) {
    a.codes[p] = b.codes[p];
    a.scales[p] = b.scales[p];
    a.g[p] = b.g[p];
  }
  a.H = b.H;
  a.I = b.I;
  a.k = k;
  a.in = mid;
  a.w = w;
  a.rt = rt;
  a.part = part;
  dim3 grid((b.H + kDownRows - 1) / kDownRows, slots);
  size_t lds = (size_t)kDecTok * b.I * 2;
  prof_begin("decode_down", s);
  hipLaunchKernelGGL(decode_down_kernel, grid, dim3(kDecThreads), lds, s, a);
  prof_end("decode_down", s);
  return hipGetLastError();
}

// ---- S7: weighted combine (the routing weight is already in `part`) -----------
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part,
                                                     const int32_t* __restrict__ idx, int E, int T,
                                                     int H, int k, const uint16_t* __restrict__ res,
                                                     void* y, int f32_out) {
  const size_t n = (size_t)T * H;
  for (size_t o = (size_t)blockIdx.x * blockDim.x + threadIdx.x; o < n;
       o += (size_t)gridDim.x * blockDim.x) {
    const size_t t = o / H, h = o % H;
    float acc = res ? bf16_to_f32(res[o]) : 0.0f;
    for (int j = 0; j < k; j++) {
      const size_t p = t * k + j;
      const int e = idx[p];
      if (e >= 0 && e < E) acc += part[p * H + h];
    }
    if (f32_out)
      reinterpret_cast<float*>(y)[o] = acc;
    else
      reinterpret_cast<uint16_t*>(y)[o] = f32_to_bf16(acc);
  }
}

hipError_t launch_combine(const float* part, const int32_t* idx, int E, int T, int H, int k,
                          const uint16_t* residual, void* y, bool f32_out, hipStream_t s) {
  size_t n = (size_t)T * H;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  prof_begin("combine", s);
  hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, s, part, idx, E, T, H, k,
                     residual, y, f32_out ? 1 : 0);
  prof_end("combine", s);
  return hipGetLastError();
}

}  // namespace moe
