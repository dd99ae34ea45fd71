// Routing kernels for gfx950: router logits (S1), wave64 top-k + softmax (S2)
// and the stable token -> expert counting sort (S3).
//
// Router numerics follow "Beam-1.0-501B-A23B VQ GGUF", "What stays native"
// (router logits in FP32); the top-k of 256 experts with 8 active per token is
// the routed-expert shape of "Beam 1.0 501B-A23B, streaming pack, NVFP4
// experts / MLX 8-bit residents" (intro). The selection rule (top-k by logit,
// softmax over the k selected) and the tie rule (lower expert index first) are
// the readings the C header states.
#include "common.h"
#include "internal.h"

namespace moe {

// ---- S1: partial logits ----------------------------------------------------
// Block (chunk c, token group tg): rows h in [64c, 64c+64) of Wr, up to 8
// tokens. Thread j owns experts j, j+256, j+512, j+768. Each Wr row is read
// once per block with coalesced 4-byte loads (1 KiB per row at E = 256); the x
// values are uniform across the block. Output partial[c][t][e] (f32); the
// top-k kernel sums the chunks in ascending order, so logits are deterministic.
__global__ __launch_bounds__(256) void router_partial_kernel(const uint16_t* __restrict__ x,
                                                             const float* __restrict__ Wr,
                                                             float* __restrict__ partial, int T,
                                                             int H, int E) {
  const int c = blockIdx.x, t0 = blockIdx.y * kRouterTok;
  const int nt = min(kRouterTok, T - t0);
  const int h0 = c * kRouterRows, h1 = min(H, h0 + kRouterRows);
  __shared__ float xs[kRouterTok][kRouterRows];
  for (int i = threadIdx.x; i < kRouterTok * kRouterRows; i += blockDim.x) {
    int tt = i / kRouterRows, hh = i % kRouterRows;
    xs[tt][hh] = (tt < nt && h0 + hh < h1) ? bf16_to_f32(x[(size_t)(t0 + tt) * H + h0 + hh]) : 0.0f;
  }
  __syncthreads();
  float acc[kRouterTok][4];
#pragma unroll
  for (int tt = 0; tt < kRouterTok; tt++)
#pragma unroll
    for (int q = 0; q < 4; q++) acc[tt][q] = 0.0f;
  for (int h = h0; h < h1; h++) {
    const float* wrow = Wr + (size_t)h * E;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      int e = threadIdx.x + 256 * q;
      float wv = (e < E) ? wrow[e] : 0.0f;
#pragma unroll
      for (int tt = 0; tt < kRouterTok; tt++) acc[tt][q] = fmaf(xs[tt][h - h0], wv, acc[tt][q]);
    }
  }
  for (int tt = 0; tt < nt; tt++)
#pragma unroll
    for (int q = 0; q < 4; q++) {
      int e = threadIdx.x + 256 * q;
      if (e < E) partial[((size_t)c * T + t0 + tt) * E + e] = acc[tt][q];
    }
}

hipError_t launch_router_partial(const uint16_t* x, const float* Wr, float* partial, int T, int H,
                                 int E, hipStream_t s) {
  dim3 grid((H + kRouterRows - 1) / kRouterRows, (T + kRouterTok - 1) / kRouterTok);
  prof_begin("router", s);
  hipLaunchKernelGGL(router_partial_kernel, grid, dim3(256), 0, s, x, Wr, partial, T, H, E);
  prof_end("router", s);
  return hipGetLastError();
}

// ---- S2: top-k + softmax, one wave64 per token --------------------------------
// Ordering key: larger logit first, then lower expert index; NaN ranks below
// every number; -0 and +0 compare equal (IEEE comparison).
__device__ __forceinline__ bool better(float a, int ea, float b, int eb) {
  bool na = a != a, nb = b != b;
  if (na != nb) return nb;  // the non-NaN one wins
  if (!na && a != b) return a > b;
  return ea < eb;
}

constexpr int kTopkMaxPerLane = 16;  // E <= 1024

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ partial, int nchunk,
                                                   float* __restrict__ logits, int T, int E, int k,
                                                   int32_t* __restrict__ idx, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[kTopkMaxPerLane];
  const int per = (E + 63) / 64;
#pragma unroll
  for (int i = 0; i < kTopkMaxPerLane; i++) {
    int e = lane + 64 * i;
    float a = -__builtin_inff();
    if (i < per && e < E) {
      if (partial) {
        a = 0.0f;
        for (int c = 0; c < nchunk; c++) a += partial[((size_t)c * T + t) * E + e];
        logits[(size_t)t * E + e] = a;
      } else {
        a = logits[(size_t)t * E + e];
      }
    }
    v[i] = a;
  }
  uint32_t taken = 0;  // bit i: candidate i of this lane already selected
  float top0 = 0.0f, sel_v = 0.0f;
  int sel_e = 0;
  for (int j = 0; j < k; j++) {
    float bv = 0.0f;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kTopkMaxPerLane; i++) {
      int e = lane + 64 * i;
      if (i < per && e < E && !((taken >> i) & 1u) && (be == 0x7FFFFFFF || better(v[i], e, bv, be))) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      float ov = __shfl_xor(bv, o, 64);
      int oe = __shfl_xor(be, o, 64);
      if (oe != 0x7FFFFFFF && (be == 0x7FFFFFFF || better(ov, oe, bv, be))) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (j == 0) top0 = bv;
    if (lane == j) {
      sel_v = bv;
      sel_e = be;
    }
  }
  // softmax over the k selected logits, f32, summed in slot order
  float a = (lane < k) ? expf(sel_v - top0) : 0.0f;
  float sum = 0.0f;
  for (int j = 0; j < k; j++) sum += __shfl(a, j, 64);
  if (lane < k) {
    idx[(size_t)t * k + lane] = sel_e;
    w[(size_t)t * k + lane] = a / sum;
  }
}

hipError_t launch_topk(const float* partial, int nchunk, float* logits, int T, int E, int k,
                       int32_t* idx, float* w, hipStream_t s) {
  prof_begin("topk", s);
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, partial, nchunk, logits, T,
                     E, k, idx, w);
  prof_end("topk", s);
  return hipGetLastError();
}

// ---- S3: stable counting sort of the pairs -----------------------------------
// One workgroup of 1024 threads (16 waves). Pass 1 counts pairs per expert
// (integer LDS atomics: order-independent). Pass 2 scans the counts. Pass 3
// places chunks of 1024 pairs in order: inside a wave, lanes with the same
// expert find each other by matching the expert id bit by bit with ballots;
// a pair's slot is the expert's running cursor + the same-expert pairs of the
// earlier waves of the chunk + its rank among the earlier lanes of its wave.
constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kMaxE = 1024;

__global__ __launch_bounds__(kSortThreads) void sort_kernel(const int32_t* __restrict__ idx, int P,
                                                            int E, RouteTables rt, int mtile,
                                                            int max_tiles) {
  __shared__ int cnt[kMaxE];
  __shared__ int cursor[kMaxE];
  __shared__ uint16_t wcnt[kSortWaves][kMaxE];
  __shared__ int scan_tmp[kSortThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < kMaxE; e += kSortThreads) {
    cnt[e] = 0;
    for (int wv = 0; wv < kSortWaves; wv++) wcnt[wv][e] = 0;
  }
  __syncthreads();
  for (int p = tid; p < P; p += kSortThreads) {
    int e = idx[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  // exclusive scan of cnt[0..E) -> cursor, one expert per thread (E <= 1024)
  int my = (tid < E) ? cnt[tid] : 0;
  int incl = my;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int n = __shfl_up(incl, o, 64);
    if (lane >= o) incl += n;
  }
  if (lane == 63) scan_tmp[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int wv = 0; wv < wave; wv++) base += scan_tmp[wv];
  int excl = base + incl - my;
  if (tid < E) {
    cursor[tid] = excl;
    rt.offsets[tid] = excl;
  }
  if (tid == kSortThreads - 1) {
    int total = 0;
    for (int wv = 0; wv < kSortWaves; wv++) total += scan_tmp[wv];
    rt.offsets[E] = total;
  }
  // active experts (count > 0) in ascending order, and the grouped-GEMM tiles
  {
    int flag = (tid < E && my > 0) ? 1 : 0;
    int ntile = (flag && mtile > 0) ? (my + mtile - 1) / mtile : 0;
    unsigned long long fb = __ballot(flag);
    int fpos = __popcll(fb & ((1ull << lane) - 1ull));
    int tincl = ntile;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int n = __shfl_up(tincl, o, 64);
      if (lane >= o) tincl += n;
    }
    __shared__ int fsum[kSortWaves], tsum[kSortWaves];
    if (lane == 63) {
      fsum[wave] = __popcll(fb);
      tsum[wave] = tincl;
    }
    __syncthreads();
    int fbase = 0, tbase = 0;
    for (int wv = 0; wv < wave; wv++) {
      fbase += fsum[wv];
      tbase += tsum[wv];
    }
    if (flag && rt.active) rt.active[fbase + fpos] = tid;
    int t0 = tbase + tincl - ntile;
    for (int q = 0; q < ntile; q++) {
      if (t0 + q < max_tiles && rt.tile_expert) {
        rt.tile_expert[t0 + q] = tid;
        rt.tile_row0[t0 + q] = excl + q * mtile;
      }
    }
    if (tid == kSortThreads - 1 && rt.counts) {
      int na = 0, nt = 0;
      for (int wv = 0; wv < kSortWaves; wv++) {
        na += fsum[wv];
        nt += tsum[wv];
      }
      rt.counts[0] = na;
      rt.counts[1] = nt < max_tiles ? nt : max_tiles;
    }
  }
  __syncthreads();
  // placement, chunk by chunk
  for (int p0 = 0; p0 < P; p0 += kSortThreads) {
    int p = p0 + tid;
    int e = (p < P) ? idx[p] : -1;
    bool valid = e >= 0 && e < E;
    int key = valid ? e : kMaxE;  // 11-bit key; invalid pairs group together
    unsigned long long peers = __ballot(1);
#pragma unroll
    for (int b = 0; b < 11; b++) {
      unsigned long long bb = __ballot((key >> b) & 1);
      peers &= ((key >> b) & 1) ? bb : ~bb;
    }
    int rank = __popcll(peers & ((1ull << lane) - 1ull));
    bool leader = rank == 0;
    if (valid && leader) wcnt[wave][e] = (uint16_t)__popcll(peers);
    __syncthreads();
    int slot = 0;
    if (valid) {
      int before = 0;
      for (int wv = 0; wv < wave; wv++) before += wcnt[wv][e];
      slot = cursor[e] + before + rank;
      rt.sorted[slot] = p;
    }
    __syncthreads();
    if (valid && leader) {
      atomicAdd(&cursor[e], (int)wcnt[wave][e]);
    }
    __syncthreads();
    if (valid && leader) wcnt[wave][e] = 0;
  }
}

hipError_t launch_sort(const int32_t* idx, int P, int E, RouteTables rt, int mtile, int max_tiles,
                       hipStream_t s) {
  prof_begin("sort", s);
  hipLaunchKernelGGL(sort_kernel, dim3(1), dim3(kSortThreads), 0, s, idx, P, E, rt, mtile,
                     max_tiles);
  prof_end("sort", s);
  return hipGetLastError();
}

}  // namespace moe
