// Grouped-GEMM kernels (prefill: many tokens per expert) on bf16 MFMA, gfx950.
//
// The pairs are sorted by expert; each expert's slots form the M dimension of
// one GEMM. A tile is (expert, 128 sorted slots) x (256 weight rows), one
// workgroup of 4 waves; wave w owns all 128 slots and 64 weight rows, as a
// 4 x 2 grid of v_mfma_f32_32x32x16_bf16 blocks.
//
// Weights: "Beam 1.0 501B-A23B, streaming pack, NVFP4 experts / MLX 8-bit
// residents", "What this pack holds", gives weight = e2m1 * f32(e4m3 * t) with
// t = f32(g / 2688). The MFMA's B operand holds u = e2m1 * e4m3, which has at
// most six significant bits and so is exact in bf16; t multiplies the f32
// accumulator in the epilogue. Activations stay bf16 (the pack's intro: the
// release's activation scales are not used). SwiGLU in FP32 and BF16 mids
// follow "Beam-1.0-501B-A23B VQ GGUF" ("What stays native", "Kernel budget on
// GB10").
//
// Data paths. B never touches LDS: in the 32x32x16 layout lane l supplies
// 8 consecutive inputs of weight row l%32, which is one U32 word of codes, so
// every lane loads its own codes and scales from HBM and dequantizes them in
// registers right before the MFMA that uses them. The inputs of a 64-wide k
// step are assigned to the MFMA's four k-slices so that lane half h = l/32
// takes inputs 32h..32h+31 (four words, one 16-byte load per row); the A
// operand uses the same assignment, which only permutes the order of the sum.
// A (activation rows, shared by the 4 waves) goes through a double-buffered
// LDS tile.
#include "common.h"
#include "internal.h"

namespace moe {

constexpr int kPM = kPrefillMTile;  // 128 sorted slots per tile
constexpr int kWR = 64;             // weight rows per wave
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

// One k step of this thread's A half row (32 bf16 = 4 blocks of 8).
struct ARegs {
  u32x4 q[4];
};
// One k step of this lane's two weight rows: 32 codes (16 bytes) and the
// row's 4 scale bytes of the step, for each row.
struct BRegs {
  u32x4 c[2];
  uint32_t s[2];
};

struct TileCtx {
  const uint16_t* a_ptr;  // A half row of this thread at k = 0
  const uint8_t* bc[2];   // codes of this lane's rows at k = 0, offset by lane half
  const uint8_t* bs[2];   // scales of this lane's rows at k = 0
};

__device__ __forceinline__ void load_a(const TileCtx& c, int ks, ARegs& r) {
  const u32x4* s = reinterpret_cast<const u32x4*>(c.a_ptr + ks * kPK);
#pragma unroll
  for (int q = 0; q < 4; q++) r.q[q] = s[q];
}

__device__ __forceinline__ void load_b(const TileCtx& c, int ks, BRegs& r) {
#pragma unroll
  for (int f = 0; f < 2; f++) {
    r.c[f] = *reinterpret_cast<const u32x4*>(c.bc[f] + ks * (kPK / 2));
    r.s[f] = *reinterpret_cast<const uint32_t*>(c.bs[f] + ks * (kPK / 16));
  }
}

// LDS row layout: input block j (8 bf16) of a k step sits at position
// 2 (j % 4) + j / 4, so that the fragment of k-slice kk for lane half h
// (block 4h + kk) is at element 16 kk + 8 h.
__device__ __forceinline__ void write_a_q(uint16_t* As, const ARegs& r, int q) {
  const int tid = threadIdx.x, row = tid >> 1, h = tid & 1;
  *reinterpret_cast<u32x4*>(As + row * kLdsRow + 8 * (2 * q + h)) = r.q[q];
}

// word of 8 E2M1 codes -> 8 bf16 unit values e2m1 * e4m3 (exact)
__device__ __forceinline__ bf16x8 deq8(uint32_t word, float sb) {
  const f32x2 v0 = e2m1x2_f32<0>(word), v1 = e2m1x2_f32<1>(word);
  const f32x2 v2 = e2m1x2_f32<2>(word), v3 = e2m1x2_f32<3>(word);
  const u32x4 o = {f32x2_to_bf16x2(v0.x * sb, v0.y * sb), f32x2_to_bf16x2(v1.x * sb, v1.y * sb),
                   f32x2_to_bf16x2(v2.x * sb, v2.y * sb), f32x2_to_bf16x2(v3.x * sb, v3.y * sb)};
  return __builtin_bit_cast(bf16x8, o);
}

// The MFMAs of one k step: A from LDS tile As, B from registers b; the next
// step's A (regs aw) is written to LDS tile As2 along the way.
__device__ __forceinline__ void step_mfma(const uint16_t* As, const BRegs& b, f32x16 (&acc)[4][2],
                                          const ARegs& aw, uint16_t* As2) {
  const int lane = threadIdx.x & 63, h = lane >> 5;
  float sb[2][2];
#pragma unroll
  for (int f = 0; f < 2; f++) {
    const uint32_t sw = b.s[f] >> (16 * h);  // scale bytes 2h, 2h+1: inputs 32h..32h+15, +16..+31
    sb[f][0] = e4m3_f32<0>(sw);
    sb[f][1] = e4m3_f32<1>(sw);
  }
#pragma unroll
  for (int kk = 0; kk < 4; kk++) {
    bf16x8 af[4], bfr[2];
#pragma unroll
    for (int ms = 0; ms < 4; ms++)
      af[ms] = *reinterpret_cast<const bf16x8*>(As + (32 * ms + (lane & 31)) * kLdsRow + 16 * kk + 8 * h);
#pragma unroll
    for (int f = 0; f < 2; f++) bfr[f] = deq8(b.c[f][kk], sb[f][kk >> 1]);
#pragma unroll
    for (int ms = 0; ms < 4; ms++)
#pragma unroll
      for (int f = 0; f < 2; f++)
        acc[ms][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ms], bfr[f], acc[ms][f], 0, 0, 0);
    if (kk >= 2) {
      write_a_q(As2, aw, 2 * (kk - 2));
      write_a_q(As2, aw, 2 * (kk - 2) + 1);
    }
  }
}

// Step s of the k loop (I = s mod 6 picks the register sets): loads of step
// s+2 are issued (A into the set that held step s, B into the set that held
// step s-1), the MFMAs of step s run on LDS tile s%2 and B set s%3 while
// step s+1's A is written to LDS tile (s+1)%2; one barrier.
template <int I>
__device__ __forceinline__ void kstep(const TileCtx& c, int s, int nk, uint16_t* L0, uint16_t* L1,
                                      ARegs& a0, ARegs& a1, BRegs& b0, BRegs& b1, BRegs& b2,
                                      f32x16 (&acc)[4][2]) {
  const int ld = min(s + 2, nk - 1);  // past the end: reload the last step (never used)
  ARegs& a_ld = (I % 2 == 0) ? a0 : a1;
  ARegs& a_wr = (I % 2 == 0) ? a1 : a0;
  BRegs& b_ld = ((I + 2) % 3 == 0) ? b0 : ((I + 2) % 3 == 1) ? b1 : b2;
  BRegs& b_use = (I % 3 == 0) ? b0 : (I % 3 == 1) ? b1 : b2;
  load_a(c, ld, a_ld);
  load_b(c, ld, b_ld);
  step_mfma((I % 2 == 0) ? L0 : L1, b_use, acc, a_wr, (I % 2 == 0) ? L1 : L0);
  __syncthreads();
}

// NPROJ = 2: gate and up (wave w: gate rows n0+32w.. and the same up rows, for
// 128 output columns per tile), SwiGLU epilogue into mid; NPROJ = 1: down
// (wave w: rows n0+64w.., 256 output columns per tile), routing-weighted f32
// rows into part.
//
// Two workgroups share a CU (at most 256 registers per lane, 37 KB of LDS
// each), so one workgroup's MFMAs cover the other's loads and barriers.
//
// Work mapping: the hardware hands out workgroups round-robin over the 8
// XCDs, each with its own L2. Workgroup L runs item (L % 8) * per + L / 8, so
// every XCD walks a contiguous run of items. Items are ordered by expert, and
// within an expert n-tile major with the expert's M tiles adjacent: those
// tiles read the same weight rows at the same time from the same L2, and the
// expert's activation rows stay there across its n-tiles.
template <int NPROJ>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillArgs a) {
  const int ncol = (NPROJ == 2) ? 2 * 64 : 4 * kWR;  // output columns per tile
  const int N = (NPROJ == 2) ? a.I : a.H;
  const int K = (NPROJ == 2) ? a.H : a.I;
  const int ntn = (N + ncol - 1) / ncol;
  const int n_items = a.rt.counts[1] * ntn;
  const int per = (n_items + 7) / 8;
  const int slot = blockIdx.x / 8, xcd = blockIdx.x % 8;
  if (slot >= per) return;
  const int item = xcd * per + slot;
  if (item >= n_items) return;
  // items of one expert: n-tile major, its M tiles adjacent (they share weight rows)
  const int t_any = item / ntn;
  const int e = a.rt.tile_expert[t_any];
  const int e_lo = a.rt.offsets[e], e_hi = a.rt.offsets[e + 1];
  const int ft = t_any - (a.rt.tile_row0[t_any] - e_lo) / kPM;
  const int ce = (e_hi - e_lo + kPM - 1) / kPM;
  const int local = item - ft * ntn;
  const int tile = ft + local % ce;
  const int row0 = a.rt.tile_row0[tile];
  const int rows = min(kPM, e_hi - row0);
  const int n0 = (local / ce) * ncol;
  const uint8_t* rec = a.bank + (size_t)e * a.stride;
  const int p0 = (NPROJ == 2) ? 0 : 2;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kPM * kLdsRow];
  __shared__ int src_row[kPM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  if (tid < kPM) {
    // rows past the tile's end read a valid stand-in row; their outputs are not stored
    const int r = min(tid, rows - 1);
    src_row[tid] = (NPROJ == 2) ? a.rt.sorted[row0 + r] / a.k : row0 + r;
  }
  float t_p[NPROJ];
#pragma unroll
  for (int q = 0; q < NPROJ; q++) t_p[q] = global_factor(*reinterpret_cast<const float*>(rec + a.g[p0 + q]));
  TileCtx c;
#pragma unroll
  for (int f = 0; f < 2; f++) {
    // weight row of fragment f for this lane; rows past N read row 0 (outputs not stored)
    const int q = (NPROJ == 2) ? f : 0;
    int n = (NPROJ == 2) ? n0 + 32 * wave + (lane & 31) : n0 + kWR * wave + 32 * f + (lane & 31);
    if (n >= N) n = 0;
    c.bc[f] = rec + a.codes[p0 + q] + (size_t)n * (K / 2) + 16 * h;
    c.bs[f] = rec + a.scales[p0 + q] + (size_t)n * (K / 16);
  }
  __syncthreads();
  c.a_ptr = a.in + (size_t)src_row[tid >> 1] * K + 32 * (tid & 1);

  f32x16 acc[4][2];
#pragma unroll
  for (int ms = 0; ms < 4; ms++)
#pragma unroll
    for (int f = 0; f < 2; f++) acc[ms][f] = f32x16{};

  const int nk = K / kPK;
  uint16_t* const L0 = lds;
  uint16_t* const L1 = lds + kPM * kLdsRow;
  ARegs a0, a1;
  BRegs b0, b1, b2;
  load_a(c, 0, a0);
  load_b(c, 0, b0);
  load_a(c, min(1, nk - 1), a1);
  load_b(c, min(1, nk - 1), b1);
#pragma unroll
  for (int q = 0; q < 4; q++) write_a_q(L0, a0, q);
  __syncthreads();
  int s = 0;
  for (; s + 6 <= nk; s += 6) {
    kstep<0>(c, s, nk, L0, L1, a0, a1, b0, b1, b2, acc);
    kstep<1>(c, s + 1, nk, L0, L1, a0, a1, b0, b1, b2, acc);
    kstep<2>(c, s + 2, nk, L0, L1, a0, a1, b0, b1, b2, acc);
    kstep<3>(c, s + 3, nk, L0, L1, a0, a1, b0, b1, b2, acc);
    kstep<4>(c, s + 4, nk, L0, L1, a0, a1, b0, b1, b2, acc);
    kstep<5>(c, s + 5, nk, L0, L1, a0, a1, b0, b1, b2, acc);
  }
  if (s < nk) kstep<0>(c, s, nk, L0, L1, a0, a1, b0, b1, b2, acc);
  if (s + 1 < nk) kstep<1>(c, s + 1, nk, L0, L1, a0, a1, b0, b1, b2, acc);
  if (s + 2 < nk) kstep<2>(c, s + 2, nk, L0, L1, a0, a1, b0, b1, b2, acc);
  if (s + 3 < nk) kstep<3>(c, s + 3, nk, L0, L1, a0, a1, b0, b1, b2, acc);
  if (s + 4 < nk) kstep<4>(c, s + 4, nk, L0, L1, a0, a1, b0, b1, b2, acc);

  // epilogue; accumulator element r of lane l is (row 8(r/4) + 4(l/32) + r%4,
  // column l%32) of its 32 x 32 block
#pragma unroll
  for (int ms = 0; ms < 4; ms++)
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int row = 32 * ms + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row >= rows) continue;
      if (NPROJ == 2) {
        const int n = n0 + 32 * wave + (lane & 31);
        if (n < N) {
          const float g = t_p[0] * acc[ms][0][r];
          const float u = t_p[NPROJ - 1] * acc[ms][1][r];
          a.mid[(size_t)(row0 + row) * N + n] = f32_to_bf16(silu_mul(g, u));
        }
      } else {
        const int pair = a.rt.sorted[row0 + row];
        const float wp = a.w[pair] * t_p[0];
#pragma unroll
        for (int f = 0; f < 2; f++) {
          const int n = n0 + kWR * wave + 32 * f + (lane & 31);
          if (n < N) a.part[(size_t)pair * N + n] = wp * acc[ms][f][r];
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
  const int items = ((b.I + 127) / 128) * max_tiles;
  dim3 grid((items + 7) / 8 * 8);
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
  const int items = ((b.H + 255) / 256) * max_tiles;
  dim3 grid((items + 7) / 8 * 8);
  prof_begin("prefill_down", s);
  hipLaunchKernelGGL(prefill_kernel<1>, grid, dim3(256), 0, s, a);
  prof_end("prefill_down", s);
  return hipGetLastError();
}

}  // namespace moe
