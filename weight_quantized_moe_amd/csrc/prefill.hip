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
constexpr int kPN = 128;            // half of the B tile: 128 gate | 128 up rows, or 256 down rows
constexpr int kBR = 2 * kPN;        // B rows per tile
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

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* base, int row, int col) {
  return *reinterpret_cast<const bf16x8*>(base + row * kLdsRow + col);
}

// Global data of one k step held in registers between its load and its LDS
// write: this thread's half row of A (32 bf16) and, for each of its B rows,
// 64 codes (32 bytes) and 4 scale bytes.
template <int NPROJ>
struct StageRegs {
  u32x4 a[4];
  u32x4 b0[1], b1[1];
  uint32_t bs[1];
};

// Per-thread addresses of a tile, computed once before the k loop so the
// loop's loads depend on no other memory access.
template <int NPROJ>
struct TileCtx {
  const uint8_t* rec;
  const uint16_t* in;
  int K, N, n0, p0, a_src;
  const uint16_t* a_ptr;  // this thread's A half row at k = 0 (a valid row even when unused)
  const uint8_t* b_codes[1];   // this thread's B row: codes at k = 0 (always valid)
  const uint8_t* b_scales[1];
  bool b_ok[1];                 // the row exists (else written as 0)
};

// Issue the global loads of k step ks (inputs k0 = 64 ks). The loads are
// unconditional (rows that do not exist read a valid stand-in row and are
// written as zeros), so the loop has no branches and the compiler can wait for
// exactly the loads each use needs.
template <int NPROJ>
__device__ __forceinline__ void stage_load(const TileCtx<NPROJ>& c, int ks, StageRegs<NPROJ>& r) {
  constexpr int BPT = 1;  // B rows per thread
  const int k0 = ks * kPK;
  const u32x4* s = reinterpret_cast<const u32x4*>(c.a_ptr + k0);
  r.a[0] = s[0];
  r.a[1] = s[1];
  r.a[2] = s[2];
  r.a[3] = s[3];
#pragma unroll
  for (int i = 0; i < BPT; i++) {
    const u32x4* cp = reinterpret_cast<const u32x4*>(c.b_codes[i] + k0 / 2);
    r.b0[i] = cp[0];
    r.b1[i] = cp[1];
    r.bs[i] = *reinterpret_cast<const uint32_t*>(c.b_scales[i] + k0 / 16);
  }
}

// Write quarter qt (0..3) of a loaded k step into an LDS stage: A columns
// 16 qt..16 qt+15 of this thread's half row as is, and B inputs
// 16 qt..16 qt+15 of this thread's rows dequantized to bf16 unit values
// u = e2m1 * e4m3 (exact).
template <int NPROJ>
__device__ __forceinline__ void stage_write_q(const TileCtx<NPROJ>& c, const StageRegs<NPROJ>& r,
                                              uint16_t* As, uint16_t* Bs, int qt) {
  constexpr int BPT = 1;
  const int tid = threadIdx.x;
  {
    u32x4* d = reinterpret_cast<u32x4*>(As + (tid >> 1) * kLdsRow + 32 * (tid & 1));
    d[qt] = (c.a_src >= 0) ? r.a[qt] : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < BPT; i++) {
    const int j = tid + 256 * i;
    {
      const u32x4 cw = (qt < 2) ? r.b0[i] : r.b1[i];
      const uint32_t w0 = (qt & 1) ? cw.z : cw.x, w1 = (qt & 1) ? cw.w : cw.y;
      const float sb = e4m3_f32_dyn(r.bs[i] >> (8 * qt));
      const f32x2 v0 = e2m1x2_f32<0>(w0), v1 = e2m1x2_f32<1>(w0), v2 = e2m1x2_f32<2>(w0), v3 = e2m1x2_f32<3>(w0);
      const f32x2 v4 = e2m1x2_f32<0>(w1), v5 = e2m1x2_f32<1>(w1), v6 = e2m1x2_f32<2>(w1), v7 = e2m1x2_f32<3>(w1);
      u32x4 o0 = {f32x2_to_bf16x2(v0.x * sb, v0.y * sb), f32x2_to_bf16x2(v1.x * sb, v1.y * sb),
                  f32x2_to_bf16x2(v2.x * sb, v2.y * sb), f32x2_to_bf16x2(v3.x * sb, v3.y * sb)};
      u32x4 o1 = {f32x2_to_bf16x2(v4.x * sb, v4.y * sb), f32x2_to_bf16x2(v5.x * sb, v5.y * sb),
                  f32x2_to_bf16x2(v6.x * sb, v6.y * sb), f32x2_to_bf16x2(v7.x * sb, v7.y * sb)};
      if (!c.b_ok[i]) o0 = o1 = u32x4{0, 0, 0, 0};
      u32x4* d = reinterpret_cast<u32x4*>(Bs + j * kLdsRow + 16 * qt);
      d[0] = o0;
      d[1] = o1;
    }
  }
}

template <int NPROJ>
__device__ __forceinline__ void stage_write(const TileCtx<NPROJ>& c, const StageRegs<NPROJ>& r,
                                            uint16_t* As, uint16_t* Bs) {
#pragma unroll
  for (int qt = 0; qt < 4; qt++) stage_write_q<NPROJ>(c, r, As, Bs, qt);
}

// The MFMAs of one k step from LDS stage (As, Bs), with the write of the next
// k step (regs r -> LDS stage (As2, Bs2)) interleaved quarter by quarter, so
// the dequant arithmetic overlaps the matrix instructions.
template <int NPROJ>
__device__ __forceinline__ void stage_mfma_write(const uint16_t* As, const uint16_t* Bs,
                                                 f32x16 (&acc)[2][4], const TileCtx<NPROJ>& c,
                                                 const StageRegs<NPROJ>& r, uint16_t* As2,
                                                 uint16_t* Bs2) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mh = wave & 1, nh = wave >> 1;
#pragma unroll
  for (int kk = 0; kk < kPK; kk += 16) {
    const int col = kk + 8 * (lane >> 5);
    bf16x8 af[2], bfr[4];
#pragma unroll
    for (int ms = 0; ms < 2; ms++) af[ms] = lds_frag(As, 64 * mh + 32 * ms + (lane & 31), col);
#pragma unroll
    for (int ns = 0; ns < 4; ns++)
      bfr[ns] = lds_frag(Bs, (ns >> 1) * kPN + 64 * nh + 32 * (ns & 1) + (lane & 31), col);
#pragma unroll
    for (int ms = 0; ms < 2; ms++)
#pragma unroll
      for (int ns = 0; ns < 4; ns++)
        acc[ms][ns] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ms], bfr[ns], acc[ms][ns], 0, 0, 0);
    stage_write_q<NPROJ>(c, r, As2, Bs2, kk / 16);
  }
}

// NPROJ = 2: gate and up side by side (B rows 0..127 gate, 128..255 up, for
// 128 output columns), SwiGLU epilogue into mid; NPROJ = 1: down (B rows =
// 256 output columns), routing-weighted f32 rows into part.
// Pipeline: two LDS stages and a two-deep ring of register stages. While the
// MFMAs of step ks read LDS stage ks%2, the global loads of step ks+2 are in
// flight and step ks+1 is dequantized into the other LDS stage; one barrier
// per step.
//
// Work mapping: the hardware hands out workgroups round-robin over the 8
// XCDs, each with its own L2. Workgroup L runs item (L % 8) * per + L / 8, so
// every XCD walks a contiguous run of items in (tile, n-tile) order: the ~20
// n-tiles of one tile, which read the same activation slice each k step, run
// together on one XCD, and consecutive tiles of one expert read the same
// weight slices there.
template <int NPROJ>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  const int ncol = (NPROJ == 2) ? kPN : kBR;  // output columns per tile
  const int ntn = (((NPROJ == 2) ? a.I : a.H) + ncol - 1) / ncol;  // n-tiles
  const int n_items = a.rt.counts[1] * ntn;
  const int per = (n_items + 7) / 8;
  const int slot = blockIdx.x / 8, xcd = blockIdx.x % 8;
  if (slot >= per) return;
  const int item = xcd * per + slot;
  if (item >= n_items) return;
  const int tile = item / ntn;
  const int e = a.rt.tile_expert[tile];
  const int row0 = a.rt.tile_row0[tile];
  const int rows = min(kPM, a.rt.offsets[e + 1] - row0);
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  constexpr int kStage = kPM * kLdsRow + kBR * kLdsRow;  // bf16 per LDS stage
  __shared__ int src_row[kPM];
  TileCtx<NPROJ> c;
  c.K = (NPROJ == 2) ? a.H : a.I;
  c.N = (NPROJ == 2) ? a.I : a.H;
  c.n0 = (item % ntn) * ncol;
  c.p0 = (NPROJ == 2) ? 0 : 2;
  c.rec = a.bank + (size_t)e * a.stride;
  c.in = a.in;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mh = wave & 1, nh = wave >> 1;
  if (tid < kPM) {
    const int r = tid;
    src_row[r] = (r < rows) ? ((NPROJ == 2) ? a.rt.sorted[row0 + r] / a.k : row0 + r) : -1;
  }
  float t_p[NPROJ];
#pragma unroll
  for (int q = 0; q < NPROJ; q++) t_p[q] = global_factor(*reinterpret_cast<const float*>(c.rec + a.g[c.p0 + q]));
  __syncthreads();
  c.a_src = src_row[tid >> 1];
  c.a_ptr = c.in + (size_t)(c.a_src >= 0 ? c.a_src : 0) * c.K + 32 * (tid & 1);
#pragma unroll
  for (int i = 0; i < 1; i++) {
    const int j = tid;
    const int q = (NPROJ == 2) ? j / kPN : 0, n = c.n0 + ((NPROJ == 2) ? j % kPN : j);
    const bool ok = n < c.N;
    const int qq = ok ? q : 0, nn = ok ? n : 0;  // stand-in: row 0 of the tile's first projection
    c.b_codes[i] = c.rec + a.codes[c.p0 + qq] + (size_t)nn * (c.K / 2);
    c.b_scales[i] = c.rec + a.scales[c.p0 + qq] + (size_t)nn * (c.K / 16);
    c.b_ok[i] = ok;
  }

  f32x16 acc[2][4];
#pragma unroll
  for (int ms = 0; ms < 2; ms++)
#pragma unroll
    for (int ns = 0; ns < 4; ns++) acc[ms][ns] = f32x16{};

  const int nk = c.K / kPK;
  uint16_t* const A0 = lds;
  uint16_t* const B0 = lds + kPM * kLdsRow;
  uint16_t* const A1 = lds + kStage;
  uint16_t* const B1 = lds + kStage + kPM * kLdsRow;
  StageRegs<NPROJ> r0, r1;
  stage_load<NPROJ>(c, 0, r0);
  stage_load<NPROJ>(c, min(1, nk - 1), r1);
  stage_write<NPROJ>(c, r0, A0, B0);
  __syncthreads();
  // Steps past the end reload and rewrite the last step (never read again):
  // the loop body stays branch-free so the scheduler can interleave it.
  for (int ks = 0; ks < nk; ks += 2) {
    // even step: MFMA on stage 0; r0 is free -> loads of ks+2; r1 (ks+1) -> stage 1
    stage_load<NPROJ>(c, min(ks + 2, nk - 1), r0);
    stage_mfma_write<NPROJ>(A0, B0, acc, c, r1, A1, B1);
    __syncthreads();
    if (ks + 1 >= nk) break;
    // odd step: MFMA on stage 1; r1 is free -> loads of ks+3; r0 (ks+2) -> stage 0
    stage_load<NPROJ>(c, min(ks + 3, nk - 1), r1);
    stage_mfma_write<NPROJ>(A1, B1, acc, c, r0, A0, B0);
    __syncthreads();
  }

  // epilogue; accumulator element r of lane l is (row 8(r/4) + 4(l/32) + r%4,
  // column l%32) of its 32 x 32 block
#pragma unroll
  for (int ms = 0; ms < 2; ms++)
#pragma unroll
    for (int ns = 0; ns < ((NPROJ == 2) ? 2 : 4); ns++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int row = 64 * mh + 32 * ms + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (NPROJ == 2) {
          const int n = c.n0 + 64 * nh + 32 * ns + (lane & 31);
          if (row < rows && n < c.N) {
            const float g = t_p[0] * acc[ms][ns][r];
            const float u = t_p[NPROJ - 1] * acc[ms][ns + 2][r];
            a.mid[(size_t)(row0 + row) * c.N + n] = f32_to_bf16(silu_mul(g, u));
          }
        } else {
          const int n = c.n0 + kPN * (ns >> 1) + 64 * nh + 32 * (ns & 1) + (lane & 31);
          if (row < rows && n < c.N) {
            const int pair = a.rt.sorted[row0 + row];
            a.part[(size_t)pair * c.N + n] = a.w[pair] * (t_p[0] * acc[ms][ns][r]);
          }
        }
      }
}

template <int NPROJ>
static size_t prefill_lds_bytes() {
  return 2 * (size_t)(kPM * kLdsRow + kBR * kLdsRow) * sizeof(uint16_t);
}

template <int NPROJ>
static hipError_t prefill_setup() {
  static hipError_t once = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<NPROJ>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)prefill_lds_bytes<NPROJ>());
  return once;
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
  const int items = ((b.I + kPN - 1) / kPN) * max_tiles;
  dim3 grid((items + 7) / 8 * 8);
  hipError_t e = prefill_setup<2>();
  if (e != hipSuccess) return e;
  prof_begin("prefill_gateup", s);
  hipLaunchKernelGGL(prefill_kernel<2>, grid, dim3(256), prefill_lds_bytes<2>(), s, a);
  prof_end("prefill_gateup", s);
  return hipGetLastError();
}

hipError_t launch_prefill_down(const BankView& b, const uint16_t* mid, const float* w, int k,
                               const RouteTables& rt, int max_tiles, float* part, hipStream_t s) {
  PrefillArgs a = make_args(b, k, rt);
  a.in = mid;
  a.w = w;
  a.part = part;
  const int items = ((b.H + kBR - 1) / kBR) * max_tiles;
  dim3 grid((items + 7) / 8 * 8);
  hipError_t e = prefill_setup<1>();
  if (e != hipSuccess) return e;
  prof_begin("prefill_down", s);
  hipLaunchKernelGGL(prefill_kernel<1>, grid, dim3(256), prefill_lds_bytes<1>(), s, a);
  prof_end("prefill_down", s);
  return hipGetLastError();
}

}  // namespace moe
