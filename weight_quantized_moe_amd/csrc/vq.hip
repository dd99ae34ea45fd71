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

struct Grp {
  uint32_t w0, w1, w2;
};

__device__ __forceinline__ Grp load_grp(const uint8_t* row, int g) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(row + 12 * (size_t)g);
  return Grp{p[0], p[1], p[2]};
}

// The LDS reads of one group (8 indices): the 8 codewords (cb: the codebook in
// LDS) and the group's 64 inputs as 8 chunks of 4 packed bf16 pairs (xbuf:
// LDS, in the swizzled chunk layout of gemv_util.h, a group being a quad
// there; g counted from the buffer's start). The swizzle keeps the 16-byte
// input reads of a wave's lanes, which take different groups, off each
// other's banks: 24.4 -> 19.7 us for the one-token gate/up launch, 15.3 ->
// 12.5 us for down. The reads of a group are issued together, so a group
// waits for LDS once, not once per index.
__device__ __forceinline__ void read_codewords(const uint8_t* cb, const Grp& q, u32x2 (&cw)[8]) {
  uint32_t c[8];
  unpack8(q.w0, q.w1, q.w2, c);
#pragma unroll
  for (int i = 0; i < 8; i++) cw[i] = *reinterpret_cast<const u32x2*>(cb + 8 * c[i]);
}

__device__ __forceinline__ void read_inputs(const uint32_t* xbuf, int g, u32x4 (&xv)[8]) {
#pragma unroll
  for (int i = 0; i < 8; i++) xv[i] = *reinterpret_cast<const u32x4*>(xbuf + 4 * xchunk(g, i));
}

// s plus the sum over one group's 64 weights times its inputs, index by
// index, each codeword's E4M3 pairs as exact bf16 pairs against v_dot2
__device__ __forceinline__ float group_dot(const u32x2 (&cw)[8], const u32x4 (&xv)[8], float s) {
#pragma unroll
  for (int i = 0; i < 8; i++) {
    s = dot2(e4m3x2_bf16<false>(cw[i].x), xv[i].x, s);
    s = dot2(e4m3x2_bf16<true>(cw[i].x), xv[i].y, s);
    s = dot2(e4m3x2_bf16<false>(cw[i].y), xv[i].z, s);
    s = dot2(e4m3x2_bf16<true>(cw[i].y), xv[i].w, s);
  }
  return s;
}

// Gate/up + SwiGLU. Workgroup (blockIdx.x, blockIdx.y = token t × pair group):
// rows 16 blockIdx.x .. + 15 of gate and up for kVqGuPairs pairs of token t
// (slots j0, j0 + 1, ...), which share t's inputs and one staged codebook.
// Wave w takes 4 of the rows; 16 lanes share a row, lane sub taking the
// groups sub, sub + 16, ... of each pair's gate and up rows. Every load of a
// pass is issued first: codebook and inputs HBM -> LDS, then the index groups
// into registers, group i of every row before group i + 1, each lane the same
// number (past the row's last group: group 0, not summed; a slot past k or
// with an invalid id: expert 0's rows, not stored). The wait for the LDS
// copies counts on those index loads; the
// groups are then summed in the order their loads return, each group's LDS
// reads (codewords of both projections, the shared inputs) issued together.
constexpr int kVqGuPairs = 2;

__global__ __launch_bounds__(kVqThreads) void vq_gateup_kernel(VqArgs a) {
  constexpr int G = 16, R = 64 / G, QB = 5, NP = kVqGuPairs;
  __shared__ __attribute__((aligned(16))) uint8_t cb[kVqCodebookBytes];
  extern __shared__ __attribute__((aligned(16))) uint32_t xs[];
  const int H = a.H, I = a.I, k = a.k, ngrp = H / 64;
  const int npg = (k + NP - 1) / NP;
  const int t = blockIdx.y / npg, j0 = (blockIdx.y % npg) * NP;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rsub = lane / G, sub = lane % G;
  const int r = (blockIdx.x * (kVqThreads / 64) + wave) * R + rsub;
  const bool row_ok = r < I;
  const size_t row_bytes = (size_t)H * 3 / 16;
  const uint8_t* rows[NP][2];
  int ev[NP];
  bool pv[NP];
#pragma unroll
  for (int q = 0; q < NP; q++) {
    const int e = j0 + q < k ? a.idx[t * k + j0 + q] : -1;
    ev[q] = e;
    pv[q] = e >= 0 && e < a.E;
    const uint8_t* rec = a.bank + (size_t)(pv[q] ? e : 0) * a.stride;
    rows[q][0] = rec + a.idx_off[0] + (size_t)(row_ok ? r : 0) * row_bytes;
    rows[q][1] = rec + a.idx_off[1] + (size_t)(row_ok ? r : 0) * row_bytes;
  }
  dma_copy_lds(a.codebook, cb, kVqCodebookBytes, kVqThreads / 64);
  dma_copy_lds_swz(a.x + (size_t)t * H, xs, (uint32_t)(H * 2), kVqThreads / 64);
  float acc[NP][2] = {};
  Grp qv[QB][NP][2];
  for (int qb = 0; qb < ngrp; qb += G * QB) {
#pragma unroll
    for (int i = 0; i < QB; i++) {
      const int g = qb + sub + G * i;
      const int gl = row_ok && g < ngrp ? g : 0;
#pragma unroll
      for (int q = 0; q < NP; q++) {
        qv[i][q][0] = load_grp(rows[q][0], gl);
        qv[i][q][1] = load_grp(rows[q][1], gl);
      }
    }
    if (qb == 0) {
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<QB * NP * 2>();
      step_barrier();
    }
#pragma unroll
    for (int i = 0; i < QB; i++) {
      const int g = qb + sub + G * i;
      const bool ok = row_ok && g < ngrp;
      u32x4 xv[8];
      read_inputs(xs, ok ? g : 0, xv);
#pragma unroll
      for (int q = 0; q < NP; q++) {
        u32x2 cg[8], cu[8];
        read_codewords(cb, qv[i][q][0], cg);
        read_codewords(cb, qv[i][q][1], cu);
        if (ok) {
          acc[q][0] = group_dot(cg, xv, acc[q][0]);
          acc[q][1] = group_dot(cu, xv, acc[q][1]);
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < NP; q++) {
    const float sg = group_sum_last<G>(acc[q][0]), su = group_sum_last<G>(acc[q][1]);
    if (sub == G - 1 && row_ok && pv[q]) {
      const uint8_t* rec = a.bank + (size_t)ev[q] * a.stride;
      const uint16_t* gains_g = reinterpret_cast<const uint16_t*>(rec + a.gain_off[0]);
      const uint16_t* gains_u = reinterpret_cast<const uint16_t*>(rec + a.gain_off[1]);
      const float gv = sg * f16_to_f32(gains_g[r]);
      const float uv = su * f16_to_f32(gains_u[r]);
      a.mid[(size_t)(t * k + j0 + q) * I + r] = f32_to_bf16(silu_mul(gv, uv));
    }
  }
}

// Down + weighted combine. Workgroup (8 output rows from 8 blockIdx.x, token
// t = blockIdx.y), one wave per pair j < k; 8 lanes share a row. LDS:
// codebook | the token's k rows of mids, copied HBM -> LDS; each lane's index
// groups are loaded after those copies (the same number in every lane, a
// lane past the last row or of an unused slot loading row 0 of expert 0), so
// the wait for the copies counts on them. The k routing-weighted row sums
// meet in LDS and are added in slot order onto the residual.
__global__ __launch_bounds__(64 * kFlatDecodeMaxK) void vq_down_kernel(VqArgs a) {
  constexpr int G = 8, R = 64 / G, QB = 5;
  __shared__ __attribute__((aligned(16))) uint8_t cb[kVqCodebookBytes];
  __shared__ float s_d[kFlatDecodeMaxK][R];
  extern __shared__ __attribute__((aligned(16))) uint32_t ms[];
  const int H = a.H, I = a.I, k = a.k, ngrp = I / 64;
  const int t = blockIdx.y;
  // the wave's slot, uniform: its expert id is a scalar load, which the
  // copies below need not wait for
  const int lane = threadIdx.x & 63, j = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
  float acc = 0.0f;
  const int g0 = j * ngrp;  // the pair's mids start at this group of the buffer
  Grp q[QB];
  for (int qb = 0; qb < ngrp; qb += G * QB) {
#pragma unroll
    for (int i = 0; i < QB; i++) {
      const int g = qb + sub + G * i;
      q[i] = load_grp(rd, row_ok && g < ngrp ? g : 0);
    }
    if (qb == 0) {
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<QB>();
      step_barrier();
    }
#pragma unroll
    for (int i = 0; i < QB; i++) {
      const int g = qb + sub + G * i;
      const bool ok = valid && row_ok && g < ngrp;
      u32x2 cw[8];
      u32x4 mv[8];
      read_codewords(cb, q[i], cw);
      read_inputs(ms, g0 + (ok ? g : 0), mv);
      if (ok) acc = group_dot(cw, mv, acc);
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
  launch_kernel("vq_gateup", vq_gateup_kernel, dim3((a.I + 15) / 16, a.T * ((a.k + kVqGuPairs - 1) / kVqGuPairs)),
                dim3(kVqThreads), (uint32_t)(a.H * 2), s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_kernel("vq_down", vq_down_kernel, dim3((a.H + 7) / 8, a.T), dim3(64 * a.k), (uint32_t)(a.k * a.I * 2), s,
                a);
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
