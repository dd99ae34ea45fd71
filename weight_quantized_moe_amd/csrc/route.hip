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
#include "route_util.h"

namespace moe {

// ---- S1: router logits --------------------------------------------------------
// Router weights are f32 [E][H], one contiguous row per expert. Block
// (expert e, token group) computes the whole dot product of that row with up
// to 8 token rows: thread j sums 16-byte pieces h = 4j, 4j + 1024, ... of the
// row (coalesced) against the matching x values (router_thread_sum's
// arithmetic, which the one-token layer kernel uses too); the sum is reduced
// in the wave, then over the 4 waves in wave order. The row's pieces are
// loaded once for all the block's tokens, with every token's x pieces in the
// same round trip. One block per expert keeps every CU busy at E = 256
// without partial sums across blocks.
__global__ __launch_bounds__(256) void router_kernel(const uint16_t* x, const float* Wr, float* logits, int T,
                                                     int H, int E) {
  const int e = blockIdx.x, t0 = blockIdx.y * kRouterTok;
  const int nt = min(kRouterTok, T - t0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ float red[4][kRouterTok];
  const float* row = Wr + (size_t)e * H;
  float acc[kRouterTok];
  router_thread_sums<256, kRouterTok>(row, x + (size_t)t0 * H, H, nt, threadIdx.x, acc);
#pragma unroll
  for (int tt = 0; tt < kRouterTok; tt++) {
    if (tt < nt) {
      const float s = wave_sum(acc[tt]);
      if (lane == 0) red[wave][tt] = s;
    }
  }
  __syncthreads();
  if (threadIdx.x < nt) {
    const int tt = threadIdx.x;
    logits[(size_t)(t0 + tt) * E + e] = ((red[0][tt] + red[1][tt]) + red[2][tt]) + red[3][tt];
  }
}

hipError_t launch_router(const uint16_t* x, const float* Wr, float* logits, int T, int H, int E,
                         hipStream_t s) {
  dim3 grid(E, (T + kRouterTok - 1) / kRouterTok);
  launch_kernel("router", router_kernel, grid, dim3(256), 0, s, x, Wr, logits, T, H, E);
  return hipGetLastError();
}

// ---- S2: top-k + softmax ------------------------------------------------------
// Order: larger logit first, then lower expert index; -0 and +0 are equal; a
// NaN ranks below every number (topk_key turns a logit and its index into one
// unique 64-bit key with that order). One wave per token, four tokens per
// workgroup. Lane l owns the stripe of experts l, l + 64, ... (NS stripes,
// 64 NS >= E). tau, the k-th largest of the 64 stripe maxima, is at most the
// k-th largest key (k stripes reach it), so every top-k key is >= tau, and
// the keys >= tau (at most k NS) are ranked among themselves by counting:
// a key's rank among them is its rank among all keys. The softmax over the
// k selected logits is f32, summed in slot order (topk_softmax).
constexpr int kTopkWaves = 4;

template <int NS>
__global__ __launch_bounds__(64 * kTopkWaves) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                              int k, int32_t* __restrict__ idx,
                                                              float* __restrict__ w) {
  __shared__ uint64_t lmax_all[kTopkWaves][64];
  __shared__ uint64_t cand_all[kTopkWaves][64 * NS];
  __shared__ float sel_v_all[kTopkWaves][64];
  __shared__ int sel_e_all[kTopkWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * kTopkWaves + wave;
  if (t >= T) return;
  uint64_t* lmax = lmax_all[wave];
  uint64_t* cand = cand_all[wave];
  float* sel_v = sel_v_all[wave];
  int* sel_e = sel_e_all[wave];
  const float* lt = logits + (size_t)t * E;
  uint64_t key[NS];
  uint64_t m = 0;
#pragma unroll
  for (int i = 0; i < NS; i++) {
    const int e = lane + 64 * i;
    key[i] = (e < E) ? topk_key(lt[e], e) : 0;
    m = max(m, key[i]);
  }
  lmax[lane] = m;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  int ahead = 0;
#pragma unroll
  for (int j = 0; j < 64; j++) ahead += lmax[j] > m ? 1 : 0;
  // the lane whose stripe maximum has k - 1 larger ones (keys are unique and
  // non-zero; lanes without a key hold 0 and never qualify)
  const uint64_t hit = __ballot(ahead == k - 1 && m != 0);
  const int src = hit ? __builtin_ctzll(hit) : 0;
  const uint64_t tau = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(m >> 32), src) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)m, src);
  int nc = 0;
#pragma unroll
  for (int i = 0; i < NS; i++) {
    const bool c = key[i] != 0 && key[i] >= tau;
    const uint64_t mask = __ballot(c);
    const int pos = nc + __popcll(mask & ((1ull << lane) - 1ull));
    if (c && pos < 64 * NS) cand[pos] = key[i];
    nc += __popcll(mask);
  }
  nc = min(nc, 64 * NS);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  for (int i0 = 0; i0 < nc; i0 += 64) {
    const int i = i0 + lane;
    const uint64_t c = (i < nc) ? cand[i] : 0;
    int rank = 0;
    for (int j = 0; j < nc; j++) rank += cand[j] > c ? 1 : 0;
    if (i < nc && rank < k) {
      const int e = topk_key_expert(c);
      sel_e[rank] = e;
      sel_v[rank] = lt[e];
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  const float wl = topk_softmax(sel_v, k, lane);
  if (lane < k) {
    idx[(size_t)t * k + lane] = sel_e[lane];
    w[(size_t)t * k + lane] = wl;
  }
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                       hipStream_t s) {
  const dim3 grid((T + kTopkWaves - 1) / kTopkWaves), block(64 * kTopkWaves);
  const int ns = (E + 63) / 64;
  if (ns <= 1)
    launch_kernel("topk", topk_kernel<1>, grid, block, 0, s, logits, T, E, k, idx, w);
  else if (ns <= 2)
    launch_kernel("topk", topk_kernel<2>, grid, block, 0, s, logits, T, E, k, idx, w);
  else if (ns <= 4)
    launch_kernel("topk", topk_kernel<4>, grid, block, 0, s, logits, T, E, k, idx, w);
  else if (ns <= 8)
    launch_kernel("topk", topk_kernel<8>, grid, block, 0, s, logits, T, E, k, idx, w);
  else
    launch_kernel("topk", topk_kernel<16>, grid, block, 0, s, logits, T, E, k, idx, w);
  return hipGetLastError();
}

// ---- S3: stable counting sort of the pairs -----------------------------------
// Pairs are placed in chunks of 1024 (one per 16-wave workgroup pass): inside
// a wave, lanes with the same expert find each other by matching the expert
// id bit by bit with ballots; a pair's slot is the expert's cursor at the
// chunk's start + the same-expert pairs of the earlier waves of the chunk +
// its rank among the earlier lanes of its wave. Counts use integer LDS
// atomics (order-independent). Pairs with an expert outside [0, E) are
// dropped, and reported in the status word when the caller gives one.
//
// Few pairs: one workgroup counts, scans and places every chunk in order.
// Many pairs (with a histogram buffer): three launches. sort_count_kernel
// counts each chunk's pairs per expert; sort_scan_kernel turns the counts
// into each chunk's starting cursor per expert (the expert's first slot +
// the pairs of the earlier chunks) and builds the tables; sort_place_kernel
// places each chunk from its cursors. Both give the same stable order.
constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kMaxE = 1024;

// From per-expert counts cnt[0..E) (LDS): offsets, and when asked the active
// list and the grouped-GEMM tile table; cursor[e] (LDS) = first slot of e.
// Called by all kSortThreads threads of one workgroup.
__device__ void sort_tables(const int* cnt, int* cursor, int E, const RouteTables& rt, int mtile, int max_tiles) {
  __shared__ int scan_tmp[kSortWaves];
  __shared__ int fsum[kSortWaves], tsum[kSortWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  __syncthreads();
}

// Place the chunk of pairs p0 .. p0 + 1023 from the per-expert cursors (LDS);
// the cursors advance past the chunk's pairs. wcnt [kSortWaves][E] must be 0
// and is left 0. Called by all kSortThreads threads.
__device__ void sort_place_chunk(const int32_t* __restrict__ idx, int p0, int P, int E, int* cursor,
                                 uint16_t (*wcnt)[kMaxE], int32_t* __restrict__ sorted) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p = p0 + tid;
  const int e = (p < P) ? idx[p] : -1;
  const bool valid = e >= 0 && e < E;
  const int key = valid ? e : kMaxE;  // 11-bit key; invalid pairs group together
  unsigned long long peers = __ballot(1);
#pragma unroll
  for (int b = 0; b < 11; b++) {
    unsigned long long bb = __ballot((key >> b) & 1);
    peers &= ((key >> b) & 1) ? bb : ~bb;
  }
  const int rank = __popcll(peers & ((1ull << lane) - 1ull));
  const bool leader = rank == 0;
  if (valid && leader) wcnt[wave][e] = (uint16_t)__popcll(peers);
  __syncthreads();
  if (valid) {
    int before = 0;
    for (int wv = 0; wv < wave; wv++) before += wcnt[wv][e];
    sorted[cursor[e] + before + rank] = p;
  }
  __syncthreads();
  if (valid && leader) atomicAdd(&cursor[e], (int)wcnt[wave][e]);
  __syncthreads();
  if (valid && leader) wcnt[wave][e] = 0;
}

__global__ __launch_bounds__(kSortThreads) void sort_kernel(const int32_t* __restrict__ idx, int P,
                                                            int E, RouteTables rt, int mtile,
                                                            int max_tiles) {
  __shared__ int cnt[kMaxE];
  __shared__ int cursor[kMaxE];
  __shared__ uint16_t wcnt[kSortWaves][kMaxE];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kSortThreads) {
    cnt[e] = 0;
    for (int wv = 0; wv < kSortWaves; wv++) wcnt[wv][e] = 0;
  }
  __shared__ int bad;
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int p = tid; p < P; p += kSortThreads) {
    int e = idx[p];
    if (e >= 0 && e < E)
      atomicAdd(&cnt[e], 1);
    else
      bad = 1;
  }
  __syncthreads();
  if (tid == 0 && bad && rt.status) atomicOr(rt.status, kStatusBadIdx);
  sort_tables(cnt, cursor, E, rt, mtile, max_tiles);
  for (int p0 = 0; p0 < P; p0 += kSortThreads) sort_place_chunk(idx, p0, P, E, cursor, wcnt, rt.sorted);
}

// chunk b's count per expert -> hist[b][e]
__global__ __launch_bounds__(kSortThreads) void sort_count_kernel(const int32_t* __restrict__ idx, int P, int E,
                                                                  int32_t* __restrict__ hist, uint32_t* status) {
  __shared__ int cnt[kMaxE];
  __shared__ int bad;
  const int tid = threadIdx.x, b = blockIdx.x;
  for (int e = tid; e < E; e += kSortThreads) cnt[e] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  const int p = b * kSortThreads + tid;
  if (p < P) {
    const int e = idx[p];
    if (e >= 0 && e < E)
      atomicAdd(&cnt[e], 1);
    else
      bad = 1;
  }
  __syncthreads();
  if (tid == 0 && bad && status) atomicOr(status, kStatusBadIdx);
  for (int e = tid; e < E; e += kSortThreads) hist[(size_t)b * E + e] = cnt[e];
}

// hist[b][e] -> the number of expert e's pairs in chunks before b; the tables
__global__ __launch_bounds__(kSortThreads) void sort_scan_kernel(int nb, int E, int32_t* __restrict__ hist,
                                                                 RouteTables rt, int mtile, int max_tiles) {
  __shared__ int cnt[kMaxE];
  __shared__ int cursor[kMaxE];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kSortThreads) {
    int run = 0;
    int b = 0;
    // 16 loads in flight per pass over the chunks
    for (; b + 16 <= nb; b += 16) {
      int v[16];
#pragma unroll
      for (int u = 0; u < 16; u++) v[u] = hist[(size_t)(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < 16; u++) {
        hist[(size_t)(b + u) * E + e] = run;
        run += v[u];
      }
    }
    for (; b < nb; b++) {
      const int v = hist[(size_t)b * E + e];
      hist[(size_t)b * E + e] = run;
      run += v;
    }
    cnt[e] = run;
  }
  __syncthreads();
  sort_tables(cnt, cursor, E, rt, mtile, max_tiles);
}

// chunk b placed from its cursors: the expert's first slot + hist[b][e]
__global__ __launch_bounds__(kSortThreads) void sort_place_kernel(const int32_t* __restrict__ idx, int P, int E,
                                                                  const int32_t* __restrict__ hist, RouteTables rt) {
  __shared__ int cursor[kMaxE];
  __shared__ uint16_t wcnt[kSortWaves][kMaxE];
  const int tid = threadIdx.x, b = blockIdx.x;
  for (int e = tid; e < E; e += kSortThreads) {
    cursor[e] = rt.offsets[e] + hist[(size_t)b * E + e];
    for (int wv = 0; wv < kSortWaves; wv++) wcnt[wv][e] = 0;
  }
  __syncthreads();
  sort_place_chunk(idx, b * kSortThreads, P, E, cursor, wcnt, rt.sorted);
}

int sort_hist_ints(int P, int E) { return (P + kSortThreads - 1) / kSortThreads * E; }

hipError_t launch_sort(const int32_t* idx, int P, int E, RouteTables rt, int mtile, int max_tiles,
                       hipStream_t s) {
  const int nb = (P + kSortThreads - 1) / kSortThreads;
  if (!rt.hist || nb <= 2) {
    launch_kernel("sort", sort_kernel, dim3(1), dim3(kSortThreads), 0, s, idx, P, E, rt, mtile, max_tiles);
    return hipGetLastError();
  }
  launch_kernel("sort_count", sort_count_kernel, dim3(nb), dim3(kSortThreads), 0, s, idx, P, E, rt.hist, rt.status);
  launch_kernel("sort_scan", sort_scan_kernel, dim3(1), dim3(kSortThreads), 0, s, nb, E, rt.hist, rt, mtile,
                max_tiles);
  launch_kernel("sort_place", sort_place_kernel, dim3(nb), dim3(kSortThreads), 0, s, idx, P, E,
                (const int32_t*)rt.hist, rt);
  return hipGetLastError();
}

}  // namespace moe
