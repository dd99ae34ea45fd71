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
// call. A block owns one active expert and a tile of output rows. Inside a
// wave, G lanes share a row (64/G rows per wave pass); lane `sub` of a row
// takes the row's 64-input quads sub, sub+G, ... A quad is 4 E4M3 blocks: 32
// bytes of codes (two 16-byte loads) and 4 scale bytes (one 4-byte load), so
// every load is wide and each instruction reads G contiguous pieces of a row.
// All loads of a wave pass are issued before any arithmetic. Each 16-code
// block turns into 8 packed bf16 pairs (v_cvt_scalef32_pk_bf16_fp4, exact),
// eight v_dot2 give its partial sum, and one FMA applies the block scale
// S = f32(e4m3 * t). The expert's token activations sit in LDS (lanes of the
// 64/G rows read the same addresses: broadcast); a row's G partial sums are
// added with shuffles inside the G-lane group.
#include <cstdlib>

#include "common.h"
#include "dma.h"
#include "gemv_util.h"
#include "internal.h"
#include "route_util.h"

namespace moe {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;

struct DecodeArgs {
  const uint8_t* bank;
  uint64_t stride;
  uint64_t codes[3], scales[3], g[3];
  int H, I, k, E, P;
  int passes;           // wave passes (of 64/G rows) per block
  const int32_t* idx;   // [P] expert of each pair
  const uint16_t* in;   // gate/up: x [T][H]; down: mid [P][I] by pair id
  const float* w;       // down: routing weights [P]
  RouteTables rt;       // sorted tables, or rt.active == nullptr: in-block routing
  uint16_t* mid;        // gate/up output [P][I] by pair id
  float* part;          // down output [P][H] by pair id
  uint32_t* status;     // status word, or null
};

// In-block routing for P <= 256 pairs: finds the slot-th smallest expert id
// present in idx and its pairs in ascending pair order (s_pairs). Returns
// the pair count (0 if there are fewer than slot+1 distinct experts).
// Block-uniform result; all threads call it.
__device__ int route_in_block(const int32_t* idx, int P, int E, int slot, int* s_pairs, int* s_e,
                              uint32_t* status) {
  __shared__ uint32_t bits[32];  // E <= 1024
  __shared__ int wcount[kDecWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = (E + 31) / 32;
  if (tid < 32) bits[tid] = 0;
  __syncthreads();
  const int my = (tid < P) ? idx[tid] : -1;
  const bool valid = my >= 0 && my < E;
  if (valid) atomicOr(&bits[my >> 5], 1u << (my & 31));
  if (tid < P && !valid && status && blockIdx.x == 0 && blockIdx.y == 0) atomicOr(status, kStatusBadIdx);
  __syncthreads();
  if (tid == 0) {
    int e = -1, seen = 0;
    for (int i = 0; i < nw && e < 0; i++) {
      const uint32_t wv = bits[i];
      const int pc = __popc(wv);
      if (seen + pc > slot) {
        uint32_t v = wv;
        for (int j = 0; j < slot - seen; j++) v &= v - 1;  // drop lower set bits
        e = 32 * i + __ffs(v) - 1;
      }
      seen += pc;
    }
    *s_e = e;
  }
  __syncthreads();
  const int e = *s_e;
  if (e < 0) return 0;
  const unsigned long long m = __ballot(valid && my == e);
  if (lane == 0) wcount[wave] = __popcll(m);
  __syncthreads();
  int before = 0, total = 0;
  for (int wv = 0; wv < kDecWaves; wv++) {
    if (wv < wave) before += wcount[wv];
    total += wcount[wv];
  }
  if (valid && my == e) s_pairs[before + __popcll(m & ((1ull << lane) - 1ull))] = tid;
  __syncthreads();
  return total;
}

// NPROJ = 2: gate and up rows (input x, SwiGLU into mid); NPROJ = 1: down
// rows (input mid, routing-weighted f32 into part). MT tokens per pass.
// A wave walks its rows in steps (pass, quad batch); all loads of a step are
// issued together before its arithmetic.
template <int G, int kQB, int MT, int NPROJ>
__global__ __launch_bounds__(kDecThreads) void gemv_kernel(DecodeArgs a) {
  constexpr int R = 64 / G;  // rows per wave pass
  __shared__ int s_pairs[kDecInblockMaxP];
  __shared__ int s_e;
  int e, M;
  const int* pairs;
  if (a.rt.active == nullptr) {
    M = route_in_block(a.idx, a.P, a.E, blockIdx.y, s_pairs, &s_e, a.status);
    e = s_e;
    pairs = s_pairs;
  } else {
    if ((int)blockIdx.y >= a.rt.counts[0]) return;
    e = a.rt.active[blockIdx.y];
    const int s0 = a.rt.offsets[e];
    M = a.rt.offsets[e + 1] - s0;
    pairs = a.rt.sorted + s0;
  }
  if (M == 0) return;
  const int K = (NPROJ == 2) ? a.H : a.I;  // inputs
  const int N = (NPROJ == 2) ? a.I : a.H;  // output rows
  const int nquads = K / 64;
  const int nqb = (nquads + G * kQB - 1) / (G * kQB);  // quad batches per row
  const int p0 = (NPROJ == 2) ? 0 : 2;
  const uint8_t* rec = a.bank + (size_t)e * a.stride;
  extern __shared__ __attribute__((aligned(16))) uint32_t xs[];  // [MT][K/2]
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rsub = lane / G, sub = lane % G;
  const int rows_per_block = a.passes * kDecWaves * R;
  const int r0 = blockIdx.x * rows_per_block, r1 = min(N, r0 + rows_per_block);
  // this wave's passes: rows r0 + (p * kDecWaves + wave) * R + rsub
  int np = 0;
  while (np < a.passes && r0 + (np * kDecWaves + wave) * R < r1) np++;
  const int nsteps = np * nqb;

  // One-quad steps over token chunks (gate/up's default) request the next
  // step's weights before this step's arithmetic, into a second register
  // set; wider steps already have all their quads in flight, and in the
  // one-token form the set would cost occupancy.
  constexpr bool kAhead = kQB == 1 && MT > 1;
  Quad v[NPROJ][kQB], vn[kAhead ? NPROJ : 1][kQB];
  auto load_step = [&](int st, Quad (&dst)[NPROJ][kQB]) {
    const int p = st / nqb, qb = (st % nqb) * G * kQB;
    const int r = r0 + (p * kDecWaves + wave) * R + rsub;
    if (r < r1) {
#pragma unroll
      for (int q = 0; q < NPROJ; q++) {
        const uint8_t* rc = rec + a.codes[p0 + q] + (size_t)r * (K / 2);
        const uint8_t* rs = rec + a.scales[p0 + q] + (size_t)r * (K / 16);
#pragma unroll
        for (int i = 0; i < kQB; i++) {
          const int qd = qb + sub + G * i;
          if (qd < nquads) dst[q][i] = load_quad(rc, rs, qd);
        }
      }
    }
  };
  float t[NPROJ];
#pragma unroll
  for (int q = 0; q < NPROJ; q++) t[q] = global_factor(*reinterpret_cast<const float*>(rec + a.g[p0 + q]));

  // The chunk's input rows go HBM -> LDS with no registers (one wave-wide
  // load per 1 KiB of a row). With one load step per wave (every row's quads
  // in one batch: down by default) the weights are loaded once, before the
  // first chunk's rows, and stay in registers for every chunk. Gate/up loads
  // one quad per step and so re-reads its rows, from the L2, for every chunk:
  // its first step's weights are requested with the chunk's rows, and each
  // later step's while the step before is summed. Either way the rows and
  // the first weights are in flight together and one wait covers both. Loads
  // complete in issue order, so nothing waited for between the weights and
  // the rows may be a load: the chunk's row numbers are read before the
  // weights, and the barriers wait for LDS only (step_barrier).
  const int per_row = K / 8, ipr = (per_row + 63) / 64;  // 16-byte pieces and wave loads per row
  // the chunk's pair ids, their input rows and (down) routing weights, all
  // wave-uniform; read once per chunk, ahead of its weights and rows, so the
  // arithmetic waits on none of them
  int pid[MT], prow[MT];
  float wt[MT];
  auto chunk_rows = [&](int m0, int mt) {
#pragma unroll
    for (int m = 0; m < MT; m++) {
      pid[m] = __builtin_amdgcn_readfirstlane(pairs[m0 + min(m, mt - 1)]);
      prow[m] = (NPROJ == 2) ? pid[m] / a.k : pid[m];
    }
#pragma unroll
    for (int m = 0; m < MT; m++) wt[m] = (NPROJ == 1 && m < mt) ? a.w[pid[m]] : 0.0f;
  };
  chunk_rows(0, min(MT, M));
  if (nsteps == 1) load_step(0, v);
  for (int m0 = 0; m0 < M; m0 += MT) {
    const int mt = min(MT, M - m0);
    step_barrier();  // the previous chunk's rows are read
    if (m0 > 0) chunk_rows(m0, mt);
    if constexpr (kAhead) {
      if (nsteps > 1) load_step(0, v);  // in flight together with the chunk's rows
    }
    for (int jj = wave; jj < mt * ipr; jj += kDecWaves) {
      const int m = jj / ipr, blk = jj - m * ipr, pin = 64 * blk + lane;
      int row = prow[0];
#pragma unroll
      for (int mm = 1; mm < MT; mm++)
        if (m == mm) row = prow[mm];
      // swizzled layout (gemv_util.h): position pin holds chunk pin ^ (quad & 7)
      if (pin < per_row)
        dma16(uniform_ptr(a.in + (size_t)row * K), 16u * (uint32_t)xchunk(pin >> 3, pin & 7),
              __builtin_amdgcn_readfirstlane(lds_addr(xs + m * (K / 2)) + 1024u * (uint32_t)blk));
    }
    wait_vmcnt<0>();
    step_barrier();
    float acc[NPROJ][MT];
#pragma unroll
    for (int q = 0; q < NPROJ; q++)
#pragma unroll
      for (int m = 0; m < MT; m++) acc[q][m] = 0.0f;
    for (int st = 0; st < nsteps; st++) {
      if constexpr (kAhead) {
        if (st + 1 < nsteps) load_step(st + 1, vn);
      } else {
        if (nsteps > 1) load_step(st, v);
      }
      const int p = st / nqb, qb = (st % nqb) * G * kQB;
      const int r = r0 + (p * kDecWaves + wave) * R + rsub;
      const bool row_ok = r < r1;
#pragma unroll
      for (int i = 0; i < kQB; i++) {
        const int qd = qb + sub + G * i;
        if (row_ok && qd < nquads) {
#pragma unroll
          for (int m = 0; m < MT; m++) {
            if (m < mt) {
#pragma unroll
              for (int b = 0; b < 4; b++) {
                uint32_t xw[8];
                load_x8(xs + m * (K / 2), qd, b, xw);
#pragma unroll
                for (int q = 0; q < NPROJ; q++) {
                  const float S = quad_scale(v[q][i], b) * t[q];
                  acc[q][m] = fmaf(S, block_dot16(quad_word(v[q][i], 2 * b), quad_word(v[q][i], 2 * b + 1), xw),
                                   acc[q][m]);
                }
              }
            }
          }
        }
      }
      if (st % nqb == nqb - 1) {  // the pass's rows are complete
#pragma unroll
        for (int m = 0; m < MT; m++) {
          if (m < mt) {
            float sm[NPROJ];
#pragma unroll
            for (int q = 0; q < NPROJ; q++) sm[q] = group_sum<G>(acc[q][m]);
            if (sub == 0 && row_ok) {
              if (NPROJ == 2)
                a.mid[(size_t)pid[m] * N + r] = f32_to_bf16(silu_mul(sm[0], sm[NPROJ - 1]));
              else
                a.part[(size_t)pid[m] * N + r] = wt[m] * sm[0];
            }
          }
#pragma unroll
          for (int q = 0; q < NPROJ; q++) acc[q][m] = 0.0f;
        }
      }
      if constexpr (kAhead) {
        if (nsteps > 1) {  // one step: its weights stay in v for every chunk
#pragma unroll
          for (int q = 0; q < NPROJ; q++)
#pragma unroll
            for (int i = 0; i < kQB; i++) v[q][i] = vn[q][i];
        }
      }
    }
  }
}

static int env_int(const char* name, int dflt) {
  const char* s = std::getenv(name);
  return (s && *s) ? std::atoi(s) : dflt;
}

template <int G, int QB, int NPROJ>
static void launch_gemv_g(const DecodeArgs& b, dim3 grid, size_t lds, bool one, hipStream_t s) {
  const char* name = (NPROJ == 2) ? "decode_gateup" : "decode_down";
  if (one)
    launch_kernel(name, gemv_kernel<G, QB, 1, NPROJ>, grid, dim3(kDecThreads), (uint32_t)lds, s, b);
  else
    launch_kernel(name, gemv_kernel<G, QB, 4, NPROJ>, grid, dim3(kDecThreads), (uint32_t)lds, s, b);
}

// Tuning knobs (environment, read at each launch): MOE_GEMV_QB_{GATEUP,DOWN}
// quads per lane per load step (1, 2 or 5; defaults 1 and 5: gate/up with one
// quad per step measured 5-9 % faster from 24 to 127 tokens, e.g. 1,350
// against 1,480 us at 64); MOE_GEMV_PASSES_{GATEUP,DOWN} wave passes per block
// (defaults 2 and 1: two passes of gate/up rows per block, each step's weights
// requested one step ahead, 734 -> 673 us at T = 32 and 1,144 -> 1,055 us at
// T = 64 against one pass loading each step where it is summed).
template <int NPROJ>
static hipError_t launch_gemv(const DecodeArgs& a, int slots, int max_m, hipStream_t s) {
  const int K = (NPROJ == 2) ? a.H : a.I;
  const int N = (NPROJ == 2) ? a.I : a.H;
  const int nquads = K / 64;
  const int G = (nquads % 16 == 0 || nquads > 40) ? 16 : 8;
  const int R = 64 / G;
  const int qb = NPROJ == 2 ? env_int("MOE_GEMV_QB_GATEUP", 1) : env_int("MOE_GEMV_QB_DOWN", 5);
  DecodeArgs b = a;
  b.passes = NPROJ == 2 ? env_int("MOE_GEMV_PASSES_GATEUP", 2) : env_int("MOE_GEMV_PASSES_DOWN", 1);
  if (b.passes < 1) b.passes = 1;
  const int rows_per_block = b.passes * kDecWaves * R;
  dim3 grid((N + rows_per_block - 1) / rows_per_block, slots);
  const bool one = max_m <= 1;
  const size_t lds = (size_t)(one ? 1 : 4) * K * 2;
  if (G == 16) {
    if (qb <= 1) launch_gemv_g<16, 1, NPROJ>(b, grid, lds, one, s);
    else if (qb == 2) launch_gemv_g<16, 2, NPROJ>(b, grid, lds, one, s);
    else launch_gemv_g<16, 5, NPROJ>(b, grid, lds, one, s);
  } else {
    if (qb <= 1) launch_gemv_g<8, 1, NPROJ>(b, grid, lds, one, s);
    else if (qb == 2) launch_gemv_g<8, 2, NPROJ>(b, grid, lds, one, s);
    else launch_gemv_g<8, 5, NPROJ>(b, grid, lds, one, s);
  }
  return hipGetLastError();
}

static DecodeArgs make_args(const BankView& b, const int32_t* idx, int P, int k, const RouteTables* rt) {
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
  a.E = b.E;
  a.k = k;
  a.P = P;
  a.idx = idx;
  if (rt) a.rt = *rt;  // else all-null tables: in-block routing
  return a;
}

hipError_t launch_decode_gateup(const BankView& b, const uint16_t* x, const int32_t* idx, int P, int k,
                                const RouteTables* rt, int slots, int max_m, uint16_t* mid,
                                uint32_t* status, hipStream_t s) {
  DecodeArgs a = make_args(b, idx, P, k, rt);
  a.in = x;
  a.mid = mid;
  a.status = status;
  return launch_gemv<2>(a, slots, max_m, s);
}

hipError_t launch_decode_down(const BankView& b, const uint16_t* mid, const float* w,
                              const int32_t* idx, int P, int k, const RouteTables* rt, int slots,
                              int max_m, float* part, hipStream_t s) {
  DecodeArgs a = make_args(b, idx, P, k, rt);
  a.in = mid;
  a.w = w;
  a.part = part;
  return launch_gemv<1>(a, slots, max_m, s);
}

// ---- one token (T = 1): flat kernels ---------------------------------------------
// With one token every pair has its own expert, so the token's activations are
// shared by all of them. Gate/up: a fixed grid of blocks stages x in LDS once;
// its waves then walk a flat list of (pair, 4-row group) items with no further
// barrier, each item one batch of 16-byte loads (the 4 rows of gate and up).
// Down + combine: a block owns 8 output rows for all k pairs; its k waves take
// one pair each (all loads of a block in flight at once), the routing-weighted
// row sums meet in LDS and
// are added in slot order (j ascending) onto the residual, and y is written
// directly: no per-pair partial rows and no separate combine pass.
struct FlatArgs {
  const uint8_t* bank;
  uint64_t stride;
  uint64_t codes[3], scales[3], g[3];
  int H, I, E, k;
  const int32_t* idx;       // [k]
  const float* w;           // [k]
  const uint16_t* x;        // [H]
  const uint16_t* residual; // [H] or null
  uint16_t* mid;            // [k][I]
  void* y;                  // [H] bf16 or f32
  int f32_out;
  uint32_t* status;         // status word (kStatusBadIdx), or null
};

// x [H] (bf16) -> LDS, as packed pairs in the swizzled chunk layout
// (gemv_util.h); the first 3 rounds of loads are issued before any store
__device__ __forceinline__ void flat_stage_x(const FlatArgs& a, uint32_t* xs) {
  constexpr int U = 3;
  const u32x4* src = reinterpret_cast<const u32x4*>(a.x);
  u32x4* dst = reinterpret_cast<u32x4*>(xs);
  const int n = a.H / 8;
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; u++) {
    const int i = threadIdx.x + u * blockDim.x;
    if (i < n) v[u] = src[i];
  }
#pragma unroll
  for (int u = 0; u < U; u++) {
    const int i = threadIdx.x + u * blockDim.x;
    if (i < n) dst[xchunk(i >> 3, i & 7)] = v[u];
  }
  for (int i = threadIdx.x + U * blockDim.x; i < n; i += blockDim.x) dst[xchunk(i >> 3, i & 7)] = src[i];
}

// The gate/up items of workgroup `blk` of `nblk`: wave w takes items
// blk * 4 + w, then every nblk * 4-th; item (pair j, 4-row group), the pair's
// expert s_idx[j] (-1: none).
__device__ __forceinline__ void flat_gateup_items(const FlatArgs& a, const uint32_t* xs, const int* s_idx,
                                                  int blk, int nblk) {
  // two quads per lane per load step (three steps per 5,120-input row): the
  // one-token launch measured 27.2-27.5 against 28.6-29.4 us with all five
  // at once
  constexpr int G = 16, R = 64 / G, QB = 2;
  const int H = a.H, I = a.I, nquads = H / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rsub = lane / G, sub = lane % G;
  const int groups = (I + R - 1) / R;
  const int n_items = a.k * groups;
  for (int it = blk * kDecWaves + wave; it < n_items; it += nblk * kDecWaves) {
    const int j = it / groups;
    const int r = (it % groups) * R + rsub;
    const int e = s_idx[j];
    if (e < 0) continue;
    const bool row_ok = r < I;
    const uint8_t* rec = a.bank + (size_t)e * a.stride;
    const float tg = global_factor(*reinterpret_cast<const float*>(rec + a.g[0]));
    const float tu = global_factor(*reinterpret_cast<const float*>(rec + a.g[1]));
    const uint8_t* cg = rec + a.codes[0] + (size_t)(row_ok ? r : 0) * (H / 2);
    const uint8_t* sg = rec + a.scales[0] + (size_t)(row_ok ? r : 0) * (H / 16);
    const uint8_t* cu = rec + a.codes[1] + (size_t)(row_ok ? r : 0) * (H / 2);
    const uint8_t* su = rec + a.scales[1] + (size_t)(row_ok ? r : 0) * (H / 16);
    float ag = 0.0f, au = 0.0f;
    for (int qb = 0; qb < nquads; qb += G * QB) {
      Quad vg[QB], vu[QB];
#pragma unroll
      for (int i = 0; i < QB; i++) {
        const int qd = qb + sub + G * i;
        if (row_ok && qd < nquads) {
          vg[i] = load_quad(cg, sg, qd);
          vu[i] = load_quad(cu, su, qd);
        }
      }
#pragma unroll
      for (int i = 0; i < QB; i++) {
        const int qd = qb + sub + G * i;
        if (row_ok && qd < nquads) {
#pragma unroll
          for (int b = 0; b < 4; b++) {
            uint32_t xw[8];
            load_x8(xs, qd, b, xw);
            ag = fmaf(quad_scale(vg[i], b) * tg,
                      block_dot16(quad_word(vg[i], 2 * b), quad_word(vg[i], 2 * b + 1), xw), ag);
            au = fmaf(quad_scale(vu[i], b) * tu,
                      block_dot16(quad_word(vu[i], 2 * b), quad_word(vu[i], 2 * b + 1), xw), au);
          }
        }
      }
    }
    const float g = group_sum_last<G>(ag), u = group_sum_last<G>(au);
    if (sub == G - 1 && row_ok) a.mid[(size_t)j * I + r] = f32_to_bf16(silu_mul(g, u));
  }
}

// A few tokens: the first bpt workgroups serve token 0, the next bpt token 1,
// ... (bpt = k * I/16 with one item per wave, so a workgroup's items belong
// to one token); each stages its token's x.
__global__ __launch_bounds__(kDecThreads) void flat_gateup_kernel(FlatArgs a, int bpt) {
  extern __shared__ __attribute__((aligned(16))) uint32_t xs[];  // [H/2]
  __shared__ int s_idx[kFlatDecodeMaxK];
  const int t = blockIdx.x / bpt;
  FlatArgs b = a;
  b.x = a.x + (size_t)t * a.H;
  b.idx = a.idx + (size_t)t * a.k;
  b.mid = a.mid + (size_t)t * a.k * a.I;
  if (threadIdx.x < a.k) {
    const int e = b.idx[threadIdx.x];
    const bool ok = e >= 0 && e < a.E;
    s_idx[threadIdx.x] = ok ? e : -1;
    // the token's first workgroup reports an expert outside [0, E)
    if (!ok && a.status && blockIdx.x == (unsigned)(t * bpt)) atomicOr(a.status, kStatusBadIdx);
  }
  flat_stage_x(b, xs);
  __syncthreads();
  flat_gateup_items(b, xs, s_idx, blockIdx.x - t * bpt, bpt);
}

__global__ __launch_bounds__(64 * kFlatDecodeMaxK) void flat_down_kernel(FlatArgs a0) {
  // token blockIdx.y of a few: its pairs, mids, residual and output row
  const int tok = blockIdx.y;
  FlatArgs a = a0;
  a.idx = a0.idx + (size_t)tok * a0.k;
  a.w = a0.w + (size_t)tok * a0.k;
  a.mid = a0.mid + (size_t)tok * a0.k * a0.I;
  if (a0.residual) a.residual = a0.residual + (size_t)tok * a0.H;
  a.y = a0.f32_out ? static_cast<void*>(static_cast<float*>(a0.y) + (size_t)tok * a0.H)
                   : static_cast<void*>(static_cast<uint16_t*>(a0.y) + (size_t)tok * a0.H);
  constexpr int G = 8, R = 64 / G, QB = 5;
  extern __shared__ __attribute__((aligned(16))) uint32_t ms[];  // [k][I/2]
  __shared__ float s_d[kFlatDecodeMaxK][R];
  const int H = a.H, I = a.I, k = a.k, nquads = I / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rsub = lane / G, sub = lane % G;
  const int r = blockIdx.x * R + rsub;
  const bool row_ok = r < H;
  {
    const int j = wave;  // one wave per pair
    int e = a.idx[j];
    e = (e >= 0 && e < a.E) ? e : -1;
    const float wj = a.w[j];
    // this pair's mids (I * 2 bytes, whole KiB chunks) into its part of the
    // swizzled buffer, by this wave alone
    {
      const uint8_t* base = uniform_ptr(a.mid);
      const uint32_t l0 = lds_addr(ms);
      // whole 64-chunk loads covering the pair's chunks [8 q0, 8 q0 + 8 nquads);
      // a load that straddles two pairs is made by both waves (the same
      // bytes to the same places)
      const int p0 = 8 * j * nquads, p1 = 8 * (j + 1) * nquads, ptot = 8 * k * nquads;
      for (int c = p0 / 64; 64 * c < p1; c++) {
        const uint32_t pos = c * 64 + lane;
        const uint32_t q = pos >> 3;
        const uint32_t off = 16u * (8u * q + ((pos & 7u) ^ (q & 7u)));
        if ((int)pos < ptot) dma16(base, off, __builtin_amdgcn_readfirstlane(l0 + c * 1024));
      }
    }
    float ad = 0.0f;
    if (e >= 0) {
      const uint8_t* rec = a.bank + (size_t)e * a.stride;
      const float td = global_factor(*reinterpret_cast<const float*>(rec + a.g[2]));
      const uint8_t* cd = rec + a.codes[2] + (size_t)(row_ok ? r : 0) * (I / 2);
      const uint8_t* sd = rec + a.scales[2] + (size_t)(row_ok ? r : 0) * (I / 16);
      const int q0 = j * nquads;  // pair j's mids start at this quad of the buffer
      for (int qb = 0; qb < nquads; qb += G * QB) {
        Quad vd[QB];
#pragma unroll
        for (int i = 0; i < QB; i++) {
          const int qd = qb + sub + G * i;
          if (row_ok && qd < nquads) vd[i] = load_quad(cd, sd, qd);
        }
        // the mids copy and the weights have landed (the copy was issued first)
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<0>();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < QB; i++) {
          const int qd = qb + sub + G * i;
          if (row_ok && qd < nquads) {
#pragma unroll
            for (int b = 0; b < 4; b++) {
              uint32_t xw[8];
              load_x8(ms, q0 + qd, b, xw);
              ad = fmaf(quad_scale(vd[i], b) * td,
                        block_dot16(quad_word(vd[i], 2 * b), quad_word(vd[i], 2 * b + 1), xw), ad);
            }
          }
        }
      }
    }
    wait_vmcnt<0>();  // (no expert: the copy still lands before the workgroup ends)
    const float d = group_sum_last<G>(ad);
    if (sub == G - 1) s_d[j][rsub] = (e >= 0) ? wj * d : 0.0f;
  }
  __syncthreads();
  if (threadIdx.x < R) {
    const int rr = blockIdx.x * R + threadIdx.x;
    if (rr < H) {
      float acc = a.residual ? bf16_to_f32(a.residual[rr]) : 0.0f;
      for (int j = 0; j < k; j++) acc += s_d[j][threadIdx.x];  // slot order
      if (a.f32_out)
        reinterpret_cast<float*>(a.y)[rr] = acc;
      else
        reinterpret_cast<uint16_t*>(a.y)[rr] = f32_to_bf16(acc);
    }
  }
}

// ---- one token, router and top-k in the gate/up launch -----------------------
// A launch costs a few microseconds of start-up and drain, more than the router
// (5 MB of f32 weights) and the top-k need, so the layer entry point runs both
// in the gate/up launch. Its first E workgroups are router workgroups: each
// computes one logit (expert e = blockIdx.x) with the router kernel's
// arithmetic (thread j sums h = 4j, 4j + 1024, ... by f32 fma, then the wave
// sums in wave order), publishes it in the workspace as a 64-bit tag (this
// call's number above the logit's bits, one atomic store) and ends. The other
// workgroups stage x and then need the routing. A workgroup that finds the
// routing record of this call (k tagged words: call number above the expert
// index) takes it from there; one that does not waits for all E tags and
// selects the top-k itself. The first of these workgroups publishes the
// record and writes logits, idx and w out (one writer: many stores to the
// same words from all workgroups would queue behind each other). Tags and
// records left by earlier
// calls carry other numbers, so nothing is reset between calls. A router
// workgroup waits for nothing, and workgroups are dispatched in id order, so
// the waits end once the router workgroups have run, however few workgroups
// fit on the GPU at a time. The wait is bounded anyway (about 0.1 s of
// polling): past the bound the workgroup sets bit 0 of the workspace's status
// word, writes idx as -1 and skips its items; the call's outputs are then
// invalid.
//
// Selection, with 256 threads: thread t waits for the tags t, t + 256, ...
// and turns each logit into a key (topk_key: unique, ordered as the
// selection rule); one wave then takes the k largest keys in k rounds of a
// wave-wide maximum (wave_topk: DPP, no barrier). A workgroup that starts once
// the record is out reads k words instead.
struct RouteFuse {
  const float* wr;    // [E][H] router weights, f32
  float* logits;      // [E] out
  int32_t* idx;       // [k] out (the down launch reads it as FlatArgs::idx)
  float* w;           // [k] out (FlatArgs::w)
  uint64_t* tags;     // [1024] workspace: router logits
  uint64_t* route;    // [kFlatDecodeMaxK] workspace: the routing record
  uint32_t* status;   // workspace status word
  uint32_t call;      // this call's number
  uint32_t spins;     // polls of one tag before the wait gives up
  int publish;        // router workgroups store their tags (0 only to exercise the give-up path)
};

constexpr uint32_t kTagSpins = 1u << 20;

__device__ __forceinline__ uint64_t ld_tag(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_tag(uint64_t* p, uint32_t call, uint32_t v) {
  __hip_atomic_store(p, ((uint64_t)call << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Maximum of v over the wave, uniform: DPP row shifts leave each 16-lane
// row's maximum in its lane 15, two row broadcasts carry them to lane 63
// (lanes without a source read 0, the identity here)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true));  // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true));  // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true));  // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true));  // row_shr:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xF, 0xF, true));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xF, 0xF, true));  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

// The k largest of the E keys (E <= 64 PER), by one wave: lane l holds keys
// l, l + 64, ... in registers; each round takes the largest remaining key of
// the wave (its high word, then among the lanes holding that the low word:
// keys are unique) and removes it from its lane. Writes s_idx[round] and
// sel_v[round] in the order of the selection rule, as ranking all keys does.
template <int PER>
__device__ __forceinline__ void wave_topk(const uint64_t* keys, const float* lv, int E, int k, int* s_idx,
                                          float* sel_v) {
  const int lane = threadIdx.x & 63;
  uint64_t kk[PER];
#pragma unroll
  for (int i = 0; i < PER; i++) kk[i] = lane + 64 * i < E ? keys[lane + 64 * i] : 0;  // 0: below every key
  for (int round = 0; round < k; round++) {
    uint64_t h = kk[0];
#pragma unroll
    for (int i = 1; i < PER; i++) h = kk[i] > h ? kk[i] : h;
    const uint32_t hi = wave_max_u32((uint32_t)(h >> 32));
    const uint32_t lo = wave_max_u32((uint32_t)(h >> 32) == hi ? (uint32_t)h : 0u);
    const uint64_t win = ((uint64_t)hi << 32) | lo;
#pragma unroll
    for (int i = 0; i < PER; i++)
      if (kk[i] == win) kk[i] = 0;
    if (lane == 0) {
      const int e = topk_key_expert(win);
      s_idx[round] = e;
      sel_v[round] = lv[e];
    }
  }
}

__global__ __launch_bounds__(kDecThreads) void flat_route_gateup_kernel(FlatArgs a, RouteFuse r) {
  extern __shared__ __attribute__((aligned(16))) uint32_t xs[];  // [H/2]
  __shared__ uint64_t keys[1024];
  __shared__ float lv[1024];
  __shared__ int failed, have_route;
  __shared__ float red[kDecWaves];
  __shared__ float sel_v[kFlatDecodeMaxK];
  __shared__ int s_idx[kFlatDecodeMaxK];
  const int H = a.H, E = a.E, k = a.k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (blockIdx.x < (unsigned)E) {
    const int e = blockIdx.x;
    const float sw = wave_sum(router_thread_sum<kDecThreads>(r.wr + (size_t)e * H, a.x, H, tid));
    if (lane == 0) red[wave] = sw;
    __syncthreads();
    if (tid == 0 && r.publish) st_tag(r.tags + e, r.call, __float_as_uint(((red[0] + red[1]) + red[2]) + red[3]));
    return;
  }
  const int blk = blockIdx.x - E, nblk = gridDim.x - E;
  if (tid == 0) {
    failed = 0;
    have_route = 1;
  }
  if (tid < kFlatDecodeMaxK) s_idx[tid] = -1;
  __syncthreads();
  flat_stage_x(a, xs);
  // the routing record, if a workgroup has published it already
  if (tid < k) {
    const uint64_t v = ld_tag(r.route + tid);
    if ((uint32_t)(v >> 32) == r.call)
      s_idx[tid] = (int)(uint32_t)v;
    else
      have_route = 0;
  }
  __syncthreads();
  if (!have_route) {
    for (int e = tid; e < E; e += kDecThreads) {
      uint64_t v = ld_tag(r.tags + e);
      uint32_t n = 0;
      while ((uint32_t)(v >> 32) != r.call) {
        if (++n > r.spins) {
          failed = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
        v = ld_tag(r.tags + e);
      }
      lv[e] = __uint_as_float((uint32_t)v);
      keys[e] = topk_key(lv[e], e);
    }
    __syncthreads();
    if (failed) {
      if (tid < k) {
        r.w[tid] = 0.0f;
        r.idx[tid] = -1;
      }
      if (tid == 0) atomicOr(r.status, kStatusRouteTimeout);
      return;
    }
    // the selecting wave differs between neighbouring workgroups, so that the
    // several workgroups on a CU select on different SIMDs
    if (wave == (blk & (kDecWaves - 1))) {
      if (E <= 64)
        wave_topk<1>(keys, lv, E, k, s_idx, sel_v);
      else if (E <= 128)
        wave_topk<2>(keys, lv, E, k, s_idx, sel_v);
      else if (E <= 256)
        wave_topk<4>(keys, lv, E, k, s_idx, sel_v);
      else if (E <= 512)
        wave_topk<8>(keys, lv, E, k, s_idx, sel_v);
      else
        wave_topk<16>(keys, lv, E, k, s_idx, sel_v);
    }
    __syncthreads();
    // one workgroup writes the outputs and the record (the first gate/up
    // workgroup, which always selects: no record exists before it does)
    if (blk == 0) {
      if (wave == 0) {
        const float wl = topk_softmax(sel_v, k, lane);
        if (lane < k) {
          r.w[lane] = wl;
          r.idx[lane] = s_idx[lane];
          st_tag(r.route + lane, r.call, (uint32_t)s_idx[lane]);
        }
      }
      for (int e = tid; e < E; e += kDecThreads) r.logits[e] = lv[e];
    }
  }
  flat_gateup_items(a, xs, s_idx, blk, nblk);
}

static int flat_blocks(int n_items) {
  // one item per wave: every wave's loads are issued at once and the hardware
  // starts the next workgroup on a SIMD as soon as one finishes (measured
  // 25.1 us against 27.6 us with two items per wave at T = 1, k = 8)
  int b = env_int("MOE_FLAT_GATEUP_BLOCKS", 0);
  if (b <= 0) b = (n_items + kDecWaves - 1) / kDecWaves;
  return b < 1 ? 1 : b;
}

static FlatArgs flat_args(const BankView& b, const uint16_t* x, const int32_t* idx, const float* w, int k,
                          const uint16_t* residual, uint16_t* mid, void* y, bool f32_out, uint32_t* status) {
  FlatArgs a{};
  a.bank = b.base;
  a.stride = b.stride;
  for (int p = 0; p < 3; p++) {
    a.codes[p] = b.codes[p];
    a.scales[p] = b.scales[p];
    a.g[p] = b.g[p];
  }
  a.H = b.H;
  a.I = b.I;
  a.E = b.E;
  a.k = k;
  a.idx = idx;
  a.w = w;
  a.x = x;
  a.residual = residual;
  a.mid = mid;
  a.y = y;
  a.f32_out = f32_out ? 1 : 0;
  a.status = status;
  return a;
}

static hipError_t launch_flat_down(const FlatArgs& a, int T, hipStream_t s) {
  launch_kernel("decode_down", flat_down_kernel, dim3((a.H + 7) / 8, T), dim3(64 * a.k),
                (uint32_t)(a.k * a.I * 2), s, a);
  return hipGetLastError();
}

hipError_t launch_flat_decode(const BankView& b, const uint16_t* x, int T, const int32_t* idx,
                              const float* w, int k, const uint16_t* residual, uint16_t* mid,
                              void* y, bool f32_out, uint32_t* status, hipStream_t s) {
  const FlatArgs a = flat_args(b, x, idx, w, k, residual, mid, y, f32_out, status);
  const int groups = (b.I + 3) / 4;
  // one token may take the tuned block count; several take one item per wave
  const int bpt = T == 1 ? flat_blocks(k * groups) : k * groups / kDecWaves;
  launch_kernel("decode_gateup", flat_gateup_kernel, dim3(bpt * T), dim3(kDecThreads), (uint32_t)(b.H * 2), s, a,
                bpt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_flat_down(a, T, s);
}

hipError_t launch_flat_layer(const BankView& b, const uint16_t* x, const float* wr, int k,
                             const uint16_t* residual, float* logits, int32_t* idx, float* w,
                             uint16_t* mid, uint64_t* tags, uint32_t* status, uint32_t call, void* y,
                             bool f32_out, hipStream_t s, bool debug_giveup) {
  // (the one-token layer computes idx itself, so only its wait can set a bit)
  const FlatArgs a = flat_args(b, x, idx, w, k, residual, mid, y, f32_out, nullptr);
  RouteFuse r{};
  r.wr = wr;
  r.logits = logits;
  r.idx = idx;
  r.w = w;
  r.tags = tags;
  r.route = tags + 1024;
  r.status = status;
  r.call = call;
  // debug_giveup: the router workgroups keep their logits to themselves and
  // the waits give up after a few polls, so every gate/up workgroup takes
  // the give-up path and every kernel still ends normally
  r.spins = debug_giveup ? 64u : kTagSpins;
  r.publish = debug_giveup ? 0 : 1;
  const int groups = (b.I + 3) / 4;
  const dim3 grid(b.E + flat_blocks(k * groups)), block(kDecThreads);
  const uint32_t lds = b.H * 2;
  launch_kernel("decode_route_gateup", flat_route_gateup_kernel, grid, block, lds, s, a, r);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_flat_down(a, 1, s);
}

// ---- S7: weighted combine (the routing weight is already in `part`) -----------
// y[t] = residual[t] + sum_j part[t*k + j] in slot order j (f32), four
// consecutive outputs per thread (16-byte loads of part). With k <= KMAX the
// k rows' loads are all issued before the first add (the rows of pairs with
// an expert outside [0, E) are read but not added), so a thread waits for one
// round trip instead of k; KMAX = 0 takes any k one row at a time.
template <int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part,
                                                     const int32_t* __restrict__ idx, int E, int T,
                                                     int H, int k, const uint16_t* __restrict__ res,
                                                     void* y, int f32_out) {
  const size_t n4 = (size_t)T * H / 4;  // H is a multiple of 4
  for (size_t o = (size_t)blockIdx.x * blockDim.x + threadIdx.x; o < n4;
       o += (size_t)gridDim.x * blockDim.x) {
    const size_t t = o * 4 / H, hh = o * 4 % H;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (res) {
      const u32x2 r = *reinterpret_cast<const u32x2*>(res + t * H + hh);
      acc = f32x4{bf16_to_f32(r.x & 0xFFFFu), bf16_to_f32(r.x >> 16), bf16_to_f32(r.y & 0xFFFFu),
                  bf16_to_f32(r.y >> 16)};
    }
    if (KMAX > 0) {
      f32x4 v[KMAX > 0 ? KMAX : 1];
      bool ok[KMAX > 0 ? KMAX : 1];
#pragma unroll
      for (int j = 0; j < KMAX; j++) {
        const size_t p = t * k + (j < k ? j : 0);
        const int e = idx[p];
        ok[j] = j < k && e >= 0 && e < E;
        v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(part + p * H + hh));
      }
#pragma unroll
      for (int j = 0; j < KMAX; j++)
        if (ok[j]) acc += v[j];
    } else {
      for (int j = 0; j < k; j++) {
        const size_t p = t * k + j;
        const int e = idx[p];
        if (e >= 0 && e < E) acc += *reinterpret_cast<const f32x4*>(part + p * H + hh);
      }
    }
    if (f32_out) {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(y) + t * H + hh) = acc;
    } else {
      const u32x2 b = {f32x2_to_bf16x2(acc.x, acc.y), f32x2_to_bf16x2(acc.z, acc.w)};
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(y) + t * H + hh) = b;
    }
  }
}

hipError_t launch_combine(const float* part, const int32_t* idx, int E, int T, int H, int k,
                          const uint16_t* residual, void* y, bool f32_out, hipStream_t s) {
  const size_t n4 = (size_t)T * H / 4;
  size_t blocks = (n4 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks), block(256);
  const int fo = f32_out ? 1 : 0;
  if (k <= 8)
    launch_kernel("combine", combine_kernel<8>, grid, block, 0, s, part, idx, E, T, H, k, residual, y, fo);
  else if (k <= 16)
    launch_kernel("combine", combine_kernel<16>, grid, block, 0, s, part, idx, E, T, H, k, residual, y, fo);
  else
    launch_kernel("combine", combine_kernel<0>, grid, block, 0, s, part, idx, E, T, H, k, residual, y, fo);
  return hipGetLastError();
}

}  // namespace moe
