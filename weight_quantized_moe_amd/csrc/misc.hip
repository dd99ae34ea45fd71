// Smaller kernels of libmoe_mi355x.so for gfx950: record pad zeroing (pack),
// the dequant test export, the weightless RMS norm between stacked layers, and
// the affine8_g64 resident linear.
#include "common.h"
#include "dma.h"
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

// ---- status word: cleared by a one-lane store (no memset node, so a caller
// may capture it in a graph)
__global__ void store_u32_kernel(uint32_t* p, uint32_t v) { *p = v; }

hipError_t launch_store_u32(uint32_t* p, uint32_t v, hipStream_t s) {
  hipLaunchKernelGGL(store_u32_kernel, dim3(1), dim3(1), 0, s, p, v);
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
// One workgroup per token. A row of up to 8,192 values (16-byte aligned, H a
// multiple of 8) is read once into registers, all loads in flight together;
// other rows take a strided loop over single values.
constexpr int kRmsU = 4;  // 16-byte pieces per thread held in registers

__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* x, int H, float eps,
                                                      uint16_t* y) {
  const size_t t = blockIdx.x;
  const uint16_t* xr = x + t * H;
  uint16_t* yr = y + t * H;
  const int np = H / 8;
  const bool vec =
      (H % 8 == 0) && np <= kRmsU * 256 && ((uintptr_t)xr & 15) == 0 && ((uintptr_t)yr & 15) == 0;
  u32x4 v[kRmsU];
  float ss = 0.0f;
  if (vec) {
#pragma unroll
    for (int u = 0; u < kRmsU; u++) {
      const int i = threadIdx.x + 256 * u;
      v[u] = i < np ? reinterpret_cast<const u32x4*>(xr)[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kRmsU; u++) {
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const float a = bf16_to_f32(w[q] & 0xFFFFu), b = bf16_to_f32(w[q] >> 16);
        ss = fmaf(a, a, ss);
        ss = fmaf(b, b, ss);
      }
    }
  } else {
    for (int h = threadIdx.x; h < H; h += 256) {
      const float a = bf16_to_f32(xr[h]);
      ss = fmaf(a, a, ss);
    }
  }
  ss = wave_sum(ss);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
  if (vec) {
#pragma unroll
    for (int u = 0; u < kRmsU; u++) {
      const int i = threadIdx.x + 256 * u;
      if (i < np) {
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; q++)
          o[q] = (uint32_t)f32_to_bf16(bf16_to_f32(w[q] & 0xFFFFu) * inv) |
                 ((uint32_t)f32_to_bf16(bf16_to_f32(w[q] >> 16) * inv) << 16);
        reinterpret_cast<u32x4*>(yr)[i] = u32x4{o[0], o[1], o[2], o[3]};
      }
    }
  } else {
    for (int h = threadIdx.x; h < H; h += 256) yr[h] = f32_to_bf16(bf16_to_f32(xr[h]) * inv);
  }
}

hipError_t launch_rmsnorm(const uint16_t* x, int T, int H, float eps, uint16_t* y, hipStream_t s) {
  launch_kernel("rmsnorm", rmsnorm_kernel, dim3(T), dim3(256), 0, s, x, H, eps, y);
  return hipGetLastError();
}

// ---- affine8_g64 resident linear ("Beam 1.0 501B-A23B, streaming pack, NVFP4
// experts / MLX 8-bit residents", residents and q8-rule bullets) --------------------
// y[t][n] = sum_g scale[n][g] * (sum_{k in g} x[t][k] q[n][k]) + bias[n][g] * (sum_{k in g} x[t][k])
// over the 64-input groups g, exactly. Bandwidth-bound for a few tokens (1 B
// per weight plus 4 B per 64 read once), so the arithmetic must stay off the
// critical path: both sums run on v_mfma_f32_16x16x32_bf16 with the tokens as
// M (16 per pass) and weight rows as N. A code q <= 255 is exact in bf16, and
// the group sum of x comes from an MFMA against a B operand of ones, which
// leaves it in the output layout next to the others.
//
// A workgroup of 16 waves owns rw rows, 16 to 32 (two 16-row MFMA blocks that
// share the activations and the ones-MFMA; lanes of the second block past rw
// re-read the last row, from the cache): rw = N / (number of CUs), rounded
// up, so the workgroups run as one round on the chip (20 rows at N = 5120).
// A round of these workgroups costs about the same whether full or not:
// 16-row workgroups left a second round a quarter full and took twice as long. The K groups are split over the waves
// (5 consecutive groups each per block of 5120 inputs), so every wave has all
// its loads (16 bytes of codes per row block and 32 bytes of activations per
// group and lane) in flight at once, straight into registers; the scales and
// biases of the workgroup's rows (adjacent in memory) come in by consecutive
// lanes and wait in LDS. The waves' partial sums meet in LDS and are added in
// wave order.
//
// MFMA layouts (16x16x32): A lane l holds token l%16, inputs 8(l/16)..+7 of
// the k-slice; B lane l holds row l%16, the same inputs; D lane l holds row
// l%16 for tokens 4(l/16)..+3. The 64 inputs of a group go to two k-slices
// so that lane group j = l/16 takes inputs 16j..16j+15 (one 16-byte piece of
// codes), the first 8 in slice 0 and the rest in slice 1; A takes the same
// assignment, which only permutes the order of the sum.
//
// Every load is unconditional (indices are clamped instead): a load under a
// lane-dependent branch makes the compiler wait for it where the branch
// rejoins, which would serialize the round trips. Padding tokens (lanes with
// l%16 >= the pass's token count) load the last real token's row, and rows
// past N load row N-1; neither is stored.
constexpr int kAffWaves = 16;                       // waves per workgroup
constexpr int kAffGW = 5;                           // groups per wave in a K block
constexpr int kAffKB = 64 * kAffGW * kAffWaves;     // inputs per K block (5120)
constexpr int kAffTok = 16;                         // tokens per pass
constexpr int kAffRB = 2;                           // 16-row blocks per workgroup
constexpr int kAffPre = (16 * kAffRB * (kAffKB / 64) + 64 * kAffWaves - 1) / (64 * kAffWaves);

// 8 codes (two words) -> 8 bf16 values (exact: a code has at most 8
// significant bits, so its f32 value has a zero low half)
__device__ __forceinline__ bf16x8 u8x8_bf16(uint32_t w0, uint32_t w1) {
  uint32_t o[4];
  const uint32_t w[2] = {w0, w1};
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const float a = (float)(w[h] & 0xFFu), b = (float)((w[h] >> 8) & 0xFFu);
    const float c = (float)((w[h] >> 16) & 0xFFu), d = (float)(w[h] >> 24);
    o[2 * h] = (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
    o[2 * h + 1] = (__float_as_uint(c) >> 16) | (__float_as_uint(d) & 0xFFFF0000u);
  }
  return __builtin_bit_cast(bf16x8, u32x4{o[0], o[1], o[2], o[3]});
}

template <bool X16>
__global__ __launch_bounds__(64 * kAffWaves) void affine8_kernel(const uint16_t* __restrict__ x,
                                                                 const uint8_t* __restrict__ codes,
                                                                 const uint16_t* __restrict__ scales,
                                                                 const uint16_t* __restrict__ biases, int T,
                                                                 int K, int N, int rw, uint16_t* __restrict__ y) {
  constexpr int R = 16 * kAffRB;                      // rows per workgroup at most
  __shared__ float red[kAffWaves][kAffTok][R];        // [wave][token][row]
  __shared__ uint32_t sbl[R][kAffKB / 64];            // scale | bias << 16 of the block's groups
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, j = lane >> 4;
  const int G = K / 64;
  const int r0 = blockIdx.x * rw, rend = min(r0 + rw, N);  // this workgroup's rows [r0, rend)
  int row[kAffRB];
#pragma unroll
  for (int b = 0; b < kAffRB; b++) row[b] = min(r0 + 16 * b + n, rend - 1);
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  for (int t0 = 0; t0 < T; t0 += kAffTok) {
    const int nt = min(kAffTok, T - t0);
    f32x4 acc[kAffRB];
#pragma unroll
    for (int b = 0; b < kAffRB; b++) acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int kb = 0; kb < K; kb += kAffKB) {
      const int gb = kb / 64, gn = min(kAffKB, K - kb) / 64;  // the block's first group and group count
      const int g0 = gb + wave * kAffGW;
      // the rows' scales and biases of the block, by consecutive lanes from
      // consecutive addresses; loaded first, so storing them to LDS waits
      // for these loads only
      uint16_t ps[kAffPre], pb[kAffPre];
#pragma unroll
      for (int u = 0; u < kAffPre; u++) {
        const int i = min((int)threadIdx.x + 64 * kAffWaves * u, R * gn - 1);
        const size_t o = (size_t)min(r0 + i / gn, rend - 1) * G + gb + i % gn;
        ps[u] = scales[o];
        pb[u] = biases[o];
      }
      // the scale and bias loads go out first: waiting for them (to stage
      // them in LDS) then leaves the codes and activations in flight
      __builtin_amdgcn_sched_barrier(0);
      u32x4 q[kAffRB][kAffGW], xa[kAffGW], xb[kAffGW];
#pragma unroll
      for (int i = 0; i < kAffGW; i++) {
        const int g = min(g0 + i, G - 1);  // groups past G: loaded, weighted by zero
#pragma unroll
        for (int b = 0; b < kAffRB; b++)
          q[b][i] = *reinterpret_cast<const u32x4*>(codes + (size_t)row[b] * K + 64 * g + 16 * j);
        const uint16_t* xp = x + (size_t)(t0 + min(n, nt - 1)) * K + 64 * g + 16 * j;
        if (X16) {
          xa[i] = reinterpret_cast<const u32x4*>(xp)[0];
          xb[i] = reinterpret_cast<const u32x4*>(xp)[1];
        } else {
          const uint32_t* xw = reinterpret_cast<const uint32_t*>(xp);
          xa[i] = u32x4{xw[0], xw[1], xw[2], xw[3]};
          xb[i] = u32x4{xw[4], xw[5], xw[6], xw[7]};
        }
      }
      // keep every load above the first use (the scheduler would otherwise
      // spread them over the MFMAs, one round trip per group)
      __builtin_amdgcn_sched_barrier(0);
      // barriers without a memory fence (a fence would wait for every load in
      // flight): the group MFMAs below start as their own loads land
      step_barrier();  // sbl of the previous block is read
#pragma unroll
      for (int u = 0; u < kAffPre; u++) {
        // unconditional (a conditional store would pull its load below the
        // others); threads past the end rewrite the last entry's own value
        const int i = min((int)threadIdx.x + 64 * kAffWaves * u, R * gn - 1);
        sbl[i / gn][i % gn] = (uint32_t)ps[u] | ((uint32_t)pb[u] << 16);
      }
      step_barrier();  // sbl is written
#pragma unroll
      for (int i = 0; i < kAffGW; i++) {
        const bf16x8 a0 = __builtin_bit_cast(bf16x8, xa[i]), a1 = __builtin_bit_cast(bf16x8, xb[i]);
        const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        f32x4 xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, ones, z, 0, 0, 0);
        xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, ones, xs, 0, 0, 0);
#pragma unroll
        for (int b = 0; b < kAffRB; b++) {
          f32x4 s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, u8x8_bf16(q[b][i].x, q[b][i].y), z, 0, 0, 0);
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, u8x8_bf16(q[b][i].z, q[b][i].w), s, 0, 0, 0);
          const uint32_t sb = (g0 + i < G) ? sbl[16 * b + n][g0 - gb + i] : 0u;
          const float sc = bf16_to_f32(sb & 0xFFFFu), bi = bf16_to_f32(sb >> 16);
#pragma unroll
          for (int e = 0; e < 4; e++) acc[b][e] = fmaf(sc, s[e], fmaf(bi, xs[e], acc[b][e]));
        }
      }
    }
#pragma unroll
    for (int b = 0; b < kAffRB; b++)
#pragma unroll
      for (int e = 0; e < 4; e++) red[wave][4 * j + e][16 * b + n] = acc[b][e];
    __syncthreads();
    if (threadIdx.x < kAffTok * R) {
      const int tt = threadIdx.x / R, nn = threadIdx.x % R;
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kAffWaves; w++) v += red[w][tt][nn];
      if (tt < nt && r0 + nn < rend) y[(size_t)(t0 + tt) * N + r0 + nn] = f32_to_bf16(v);
    }
    __syncthreads();  // red is rewritten by the next pass
  }
}

// The same linear for up to 8 tokens where K is a multiple of 1,024 (G = 16
// GW groups, GW <= 6), as a stream over the codes with the activations in
// LDS. The kernel above reads every group's activations into registers, a
// piece per lane and MFMA, twice over for 8 tokens (the 16-token MFMA is half
// padding), in each of the 256 workgroups; with the codes of the padding rows
// of its second row block that is three times the code bytes through each
// CU's vector memory path, and with the codes removed that kernel still took
// 7.5 of its 13.2 us at 8 x 5120 x 5120. Here:
//   - the activations and the workgroup's scale and bias rows go HBM -> LDS
//     with global_load_lds_dwordx4, once per workgroup, behind one barrier;
//     lanes of padding tokens read a real token's row (their outputs are
//     never stored);
//   - the codes are raw buffer loads straight into registers, all issued at
//     the start (marked volatile, so the compiler keeps them above the wait
//     for the LDS loads); the lanes of rows past the workgroup's last row get
//     an offset past the buffer's range, which the hardware answers with
//     zeros without a memory access;
//   - the arithmetic is the kernel above's: both sums on
//     v_mfma_f32_16x16x32_bf16 (tokens as M, 16 weight rows as N), the group
//     sum of x against a B operand of ones, scale and bias folded per group,
//     the 16 waves' partial sums added in LDS in wave order.
constexpr int kAfsTok = 8;  // tokens at most

template <int GW>
__global__ __launch_bounds__(64 * kAffWaves) void affine8_stream_kernel(const uint16_t* __restrict__ x,
                                                                        const uint8_t* codes,
                                                                        const uint16_t* __restrict__ scales,
                                                                        const uint16_t* __restrict__ biases, int T,
                                                                        int N, int rw, uint16_t* __restrict__ y) {
  constexpr int K = 1024 * GW, G = 16 * GW, R = 16 * kAffRB;
  constexpr uint32_t kXRow = 2 * K + 16;  // bytes per staged token row (16 more: rows start 4 banks apart)
  constexpr int kChunks = 2 * K / 1024;   // 1 KiB loads per token row
  __shared__ __attribute__((aligned(16))) uint8_t xs[kAfsTok * kXRow];
  __shared__ __attribute__((aligned(16))) uint16_t ss[R * G], bs[R * G];  // [row][group]
  __shared__ float red[kAffWaves][kAfsTok][R];                              // [wave][token][row]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, j = lane >> 4;
  const int r0 = blockIdx.x * rw, nr = min(rw, N - r0);  // this workgroup's rows [r0, r0 + nr)
  const int g0 = wave * GW;                              // this wave's groups [g0, g0 + GW)

  // HBM -> LDS: the rows' scales and biases (nr * G * 2 contiguous bytes each,
  // a multiple of 32), and the activations (1 KiB chunk c: token c / kChunks,
  // part c % kChunks)
  dma_copy_lds(scales + (size_t)r0 * G, ss, (uint32_t)(nr * G * 2), kAffWaves);
  dma_copy_lds(biases + (size_t)r0 * G, bs, (uint32_t)(nr * G * 2), kAffWaves);
  {
    const uint8_t* xb = uniform_ptr(x);
    const uint32_t l0 = lds_addr(xs);
    for (int c = wave; c < T * kChunks; c += kAffWaves) {
      const int t = c / kChunks, part = c % kChunks;
      dma16(xb, (uint32_t)(t * 2 * K + 1024 * part + 16 * lane),
            __builtin_amdgcn_readfirstlane(l0 + t * kXRow + 1024 * part));
    }
  }
  // the codes: lane (n, j) of row block b holds 16 bytes of row r0 + 16 b + n
  // for each of the wave's groups
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(codes), (short)0, N * K, 0x00020000);
  u32x4 q[kAffRB][GW];
#pragma unroll
  for (int i = 0; i < GW; i++)
#pragma unroll
    for (int b = 0; b < kAffRB; b++) {
      const int rr = 16 * b + n;
      const uint32_t off = rr < nr ? (uint32_t)((r0 + rr) * K + 64 * (g0 + i) + 16 * j) : 0x80000000u;
      q[b][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
    }
  // the wait covers the HBM -> LDS loads (issued first) and leaves the codes
  // in flight
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<kAffRB * GW>();
  step_barrier();

  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  // A operand: lane (n, j) holds token n (padding rows n >= T read token
  // T - 1), inputs 16 j .. 16 j + 15 of a group (8 per k-slice)
  const uint8_t* xa = xs + min(n, T - 1) * kXRow + 32 * j;
  f32x4 acc[kAffRB];
#pragma unroll
  for (int b = 0; b < kAffRB; b++) acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < GW; i++) {
    const int g = g0 + i;
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(xa + 128 * g);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(xa + 128 * g + 16);
    const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 xsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, ones, z, 0, 0, 0);
    xsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, ones, xsum, 0, 0, 0);
#pragma unroll
    for (int b = 0; b < kAffRB; b++) {
      f32x4 sq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, u8x8_bf16(q[b][i].x, q[b][i].y), z, 0, 0, 0);
      sq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, u8x8_bf16(q[b][i].z, q[b][i].w), sq, 0, 0, 0);
      // rows past nr read another row's entries (their outputs are not stored)
      const float sc = bf16_to_f32(ss[(16 * b + n) * G + g]), bi = bf16_to_f32(bs[(16 * b + n) * G + g]);
#pragma unroll
      for (int e = 0; e < 4; e++) acc[b][e] = fmaf(sc, sq[e], fmaf(bi, xsum[e], acc[b][e]));
    }
  }
  // D layout: lane (n, j) holds row 16 b + n for tokens 4 j .. 4 j + 3
  if (j < kAfsTok / 4) {
#pragma unroll
    for (int b = 0; b < kAffRB; b++)
#pragma unroll
      for (int e = 0; e < 4; e++) red[wave][4 * j + e][16 * b + n] = acc[b][e];
  }
  __syncthreads();
  if (threadIdx.x < kAfsTok * R) {
    const int tt = threadIdx.x / R, rr = threadIdx.x % R;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kAffWaves; w++) v += red[w][tt][rr];
    if (tt < T && rr < nr) y[(size_t)tt * N + r0 + rr] = f32_to_bf16(v);
  }
}

// compute units of the current device (0 if the query fails)
static int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

template <int GW>
static void launch_affine8_stream(dim3 grid, hipStream_t s, const uint16_t* x, const uint8_t* c8,
                                  const uint16_t* scales, const uint16_t* biases, int T, int N, int rw, uint16_t* y) {
  launch_kernel("affine8", affine8_stream_kernel<GW>, grid, dim3(64 * kAffWaves), 0, s, x, c8, scales, biases, T, N,
                rw, y);
}

hipError_t launch_affine8(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                          const uint16_t* biases, int T, int K, int N, uint16_t* y, hipStream_t s) {
  const int cus = device_cus();
  const int rw = std::min(16 * kAffRB, std::max(16, cus > 0 ? (N + cus - 1) / cus : 16 * kAffRB));
  const dim3 grid((N + rw - 1) / rw), block(64 * kAffWaves);
  const uint8_t* c8 = reinterpret_cast<const uint8_t*>(codes);
  // the streaming form: up to 8 tokens, K = 1,024 GW with GW <= 6, 16-byte
  // aligned activations and scale and bias rows, and byte offsets of the
  // codes within 31 bits
  const bool stream = T <= kAfsTok && K % 1024 == 0 && K <= 6144 && ((uintptr_t)x & 15) == 0 &&
                      ((uintptr_t)scales & 15) == 0 &&
                      ((uintptr_t)biases & 15) == 0 && (uint64_t)N * K < (1ull << 31);
  if (stream) {
    switch (K / 1024) {
      case 1: launch_affine8_stream<1>(grid, s, x, c8, scales, biases, T, N, rw, y); break;
      case 2: launch_affine8_stream<2>(grid, s, x, c8, scales, biases, T, N, rw, y); break;
      case 3: launch_affine8_stream<3>(grid, s, x, c8, scales, biases, T, N, rw, y); break;
      case 4: launch_affine8_stream<4>(grid, s, x, c8, scales, biases, T, N, rw, y); break;
      case 5: launch_affine8_stream<5>(grid, s, x, c8, scales, biases, T, N, rw, y); break;
      default: launch_affine8_stream<6>(grid, s, x, c8, scales, biases, T, N, rw, y); break;
    }
  } else if (((uintptr_t)x & 15) == 0) {
    launch_kernel("affine8", affine8_kernel<true>, grid, block, 0, s, x, c8, scales, biases, T, K, N, rw, y);
  } else {
    launch_kernel("affine8", affine8_kernel<false>, grid, block, 0, s, x, c8, scales, biases, T, K, N, rw, y);
  }
  return hipGetLastError();
}

}  // namespace moe
