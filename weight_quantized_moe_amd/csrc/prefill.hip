// Grouped-GEMM kernels (prefill: many tokens per expert) on bf16 MFMA, gfx950.
//
// The pairs are sorted by expert; each expert's slots form the M dimension of
// one GEMM. A tile (expert, 128 sorted slots) x (128 output columns) is one
// workgroup of 4 waves, each wave a 64 x 64 quadrant built from
// v_mfma_f32_32x32x16_bf16.
//
// Weights: "Beam 1.0 501B-A23B, streaming pack, NVFP4 experts / MLX 8-bit
// residents", "What this pack holds", gives weight = e2m1 * f32(e4m3 * t) with
// t = f32(g / 2688). The LDS tile holds u = e2m1 * e4m3, which has at most six
// significant bits and so is exact in bf16; t multiplies the f32 accumulator
// in the epilogue. Activations stay bf16 (the pack's intro: the release's
// activation scales are not used). SwiGLU in FP32 and BF16 mids follow
// "Beam-1.0-501B-A23B VQ GGUF" ("What stays native", "Kernel budget on GB10").
#include "common.h"
#include "internal.h"

namespace moe {

constexpr int kPM = kPrefillMTile;  // 128 sorted slots per tile
constexpr int kPN = 128;            // output columns per tile (per projection)
constexpr int kPK = 64;             // inputs per k step
constexpr int kLdsRow = kPK + 8;    // bf16 per LDS row (16-byte pad against bank conflicts)

struct PrefillArgs {
  const uint8_t* bank;
  uint64_t stride;
  uint64_t codes[3], scales[3], g[3];
  int H, I, k;
  const uint16_t* in;  // gate/up: x [T][H]; down: mid [P][I] (sorted order)
  const float* w;      // down: routing weights [T*k]
  RouteTables rt;
  uint16_t* mid;
  float* part;
};

// Dequantize 64 inputs of one weight row (32 code bytes, 4 scale bytes) into
// 64 bf16 unit values u = e2m1 * e4m3 at dst (16-byte aligned).
__device__ __forceinline__ void dequant_row64(const uint8_t* codes, const uint8_t* scales,
                                              uint32_t* dst) {
  const u32x4 c0 = *reinterpret_cast<const u32x4*>(codes);
  const u32x4 c1 = *reinterpret_cast<const u32x4*>(codes + 16);
  const uint32_t sc = *reinterpret_cast<const uint32_t*>(scales);
  const uint32_t words[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float s[4] = {e4m3_f32<0>(sc), e4m3_f32<1>(sc), e4m3_f32<2>(sc), e4m3_f32<3>(sc)};
  uint32_t out[32];
#pragma unroll
  for (int wi = 0; wi < 8; wi++) {
    const float sb = s[wi / 2];
    f32x2 v0 = e2m1x2_f32<0>(words[wi]);
    f32x2 v1 = e2m1x2_f32<1>(words[wi]);
    f32x2 v2 = e2m1x2_f32<2>(words[wi]);
    f32x2 v3 = e2m1x2_f32<3>(words[wi]);
    out[4 * wi + 0] = f32x2_to_bf16x2(v0.x * sb, v0.y * sb);
    out[4 * wi + 1] = f32x2_to_bf16x2(v1.x * sb, v1.y * sb);
    out[4 * wi + 2] = f32x2_to_bf16x2(v2.x * sb, v2.y * sb);
    out[4 * wi + 3] = f32x2_to_bf16x2(v3.x * sb, v3.y * sb);
  }
  u32x4* d = reinterpret_cast<u32x4*>(dst);
#pragma unroll
  for (int q = 0; q < 8; q++) d[q] = u32x4{out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]};
}

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* base, int row, int col) {
  return *reinterpret_cast<const bf16x8*>(base + row * kLdsRow + col);
}

// NPROJ = 2: gate and up side by side (B tile of 256 rows), SwiGLU epilogue
// into mid; NPROJ = 1: down, routing-weighted f32 rows into part.
template <int NPROJ>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  const int tile = blockIdx.y;
  if (tile >= a.rt.counts[1]) return;
  const int e = a.rt.tile_expert[tile];
  const int row0 = a.rt.tile_row0[tile];
  const int rows = min(kPM, a.rt.offsets[e + 1] - row0);
  const int K = (NPROJ == 2) ? a.H : a.I;     // inputs
  const int N = (NPROJ == 2) ? a.I : a.H;     // outputs per projection
  const int n0 = blockIdx.x * kPN;
  const uint8_t* rec = a.bank + (size_t)e * a.stride;
  const int p0 = (NPROJ == 2) ? 0 : 2;

  __shared__ __attribute__((aligned(16))) uint16_t As[kPM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[NPROJ * kPN * kLdsRow];
  __shared__ int src_row[kPM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mh = wave & 1, nh = wave >> 1;
  if (tid < kPM) {
    int r = tid;
    if (r < rows)
      src_row[r] = (NPROJ == 2) ? a.rt.sorted[row0 + r] / a.k : row0 + r;
    else
      src_row[r] = -1;
  }
  float t_p[NPROJ];
#pragma unroll
  for (int q = 0; q < NPROJ; q++) t_p[q] = global_factor(*reinterpret_cast<const float*>(rec + a.g[p0 + q]));
  __syncthreads();

  f32x16 acc[2][2 * NPROJ];
#pragma unroll
  for (int ms = 0; ms < 2; ms++)
#pragma unroll
    for (int ns = 0; ns < 2 * NPROJ; ns++) acc[ms][ns] = f32x16{};

  // A loader: thread -> (row, half): 32 bf16 = four 16-byte loads
  const int a_row = tid >> 1, a_half = tid & 1;
  const int a_src = src_row[a_row];
  // B loader: thread -> one weight row of the tile (NPROJ * 128 rows)
  for (int k0 = 0; k0 < K; k0 += kPK) {
    {
      u32x4* d = reinterpret_cast<u32x4*>(As + a_row * kLdsRow + 32 * a_half);
      if (a_src >= 0) {
        const u32x4* s = reinterpret_cast<const u32x4*>(a.in + (size_t)a_src * K + k0 + 32 * a_half);
        u32x4 v0 = s[0], v1 = s[1], v2 = s[2], v3 = s[3];
        d[0] = v0; d[1] = v1; d[2] = v2; d[3] = v3;
      } else {
        d[0] = d[1] = d[2] = d[3] = u32x4{0, 0, 0, 0};
      }
    }
    for (int j = tid; j < NPROJ * kPN; j += 256) {
      const int q = j / kPN, n = n0 + (j % kPN);
      uint32_t* dst = reinterpret_cast<uint32_t*>(Bs + j * kLdsRow);
      if (n < N) {
        const uint8_t* cp = rec + a.codes[p0 + q] + (size_t)n * (K / 2) + k0 / 2;
        const uint8_t* sp = rec + a.scales[p0 + q] + (size_t)n * (K / 16) + k0 / 16;
        dequant_row64(cp, sp, dst);
      } else {
        u32x4* d = reinterpret_cast<u32x4*>(dst);
#pragma unroll
        for (int q2 = 0; q2 < 8; q2++) d[q2] = u32x4{0, 0, 0, 0};
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kPK; kk += 16) {
      const int col = kk + 8 * (lane >> 5);
      bf16x8 af[2], bfr[2 * NPROJ];
#pragma unroll
      for (int ms = 0; ms < 2; ms++) af[ms] = lds_frag(As, 64 * mh + 32 * ms + (lane & 31), col);
#pragma unroll
      for (int ns = 0; ns < 2 * NPROJ; ns++)
        bfr[ns] = lds_frag(Bs, (ns >> 1) * kPN + 64 * nh + 32 * (ns & 1) + (lane & 31), col);
#pragma unroll
      for (int ms = 0; ms < 2; ms++)
#pragma unroll
        for (int ns = 0; ns < 2 * NPROJ; ns++)
          acc[ms][ns] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ms], bfr[ns], acc[ms][ns], 0, 0, 0);
    }
    __syncthreads();
  }

  // epilogue; accumulator element r of lane l is (row 8(r/4) + 4(l/32) + r%4,
  // column l%32) of its 32 x 32 block
#pragma unroll
  for (int ms = 0; ms < 2; ms++)
#pragma unroll
    for (int ns = 0; ns < 2; ns++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int row = 64 * mh + 32 * ms + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int n = n0 + 64 * nh + 32 * ns + (lane & 31);
        if (row < rows && n < N) {
          if (NPROJ == 2) {
            const float g = t_p[0] * acc[ms][ns][r];
            const float u = t_p[NPROJ - 1] * acc[ms][ns + 2 * (NPROJ - 1)][r];
            a.mid[(size_t)(row0 + row) * N + n] = f32_to_bf16(silu_mul(g, u));
          } else {
            const int pair = a.rt.sorted[row0 + row];
            a.part[(size_t)pair * N + n] = a.w[pair] * (t_p[0] * acc[ms][ns][r]);
          }
        }
      }
}

static PrefillArgs make_args(const BankView& b, int k, const RouteTables& rt) {
  PrefillArgs a{};
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
  a.rt = rt;
  return a;
}

hipError_t launch_prefill_gateup(const BankView& b, const uint16_t* x, int k, const RouteTables& rt,
                                 int max_tiles, uint16_t* mid, hipStream_t s) {
  PrefillArgs a = make_args(b, k, rt);
  a.in = x;
  a.mid = mid;
  dim3 grid((b.I + kPN - 1) / kPN, max_tiles);
  prof_begin("prefill_gateup", s);
  hipLaunchKernelGGL(prefill_kernel<2>, grid, dim3(256), 0, s, a);
  prof_end("prefill_gateup", s);
  return hipGetLastError();
}

hipError_t launch_prefill_down(const BankView& b, const uint16_t* mid, const float* w, int k,
                               const RouteTables& rt, int max_tiles, float* part, hipStream_t s) {
  PrefillArgs a = make_args(b, k, rt);
  a.in = mid;
  a.w = w;
  a.part = part;
  dim3 grid((b.H + kPN - 1) / kPN, max_tiles);
  prof_begin("prefill_down", s);
  hipLaunchKernelGGL(prefill_kernel<1>, grid, dim3(256), 0, s, a);
  prof_end("prefill_down", s);
  return hipGetLastError();
}

}  // namespace moe
