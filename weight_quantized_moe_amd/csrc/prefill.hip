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
// Data paths. Every load of the k loop goes from HBM straight into LDS
// (global_load_lds_dwordx4: lane l's 16 bytes land at a wave-uniform LDS base
// + 16 l), so no registers hold data in flight, and each wave-wide load covers
// whole 64- or 128-byte row segments (the texture unit's cost grows with the
// number of distinct rows a load touches, not with its bytes):
//   A    the tile's 128 activation rows, 128 bytes (64 inputs) per row and step,
//        8 rows per load, double-buffered and shared by the 4 waves;
//   B    each wave's 64 weight rows, 64 bytes of codes (two steps) per row,
//        16 rows per load, double-buffered, private to the wave;
//   S    each wave's 64 rows' scales, 16 bytes (four steps) per row, one row
//        per lane, double-buffered, private to the wave.
// 16-byte pieces are stored XOR-swizzled within their row so the fragment
// reads of 16 consecutive rows fall in distinct banks. The B operand is
// dequantized in registers right before the MFMA: in the 32x32x16 layout lane
// l supplies 8 consecutive inputs of weight row l%32, one U32 word of codes.
// The inputs of a 64-wide k step are assigned to the MFMA's four k-slices so
// that lane half h = l/32 takes inputs 32h..32h+31 (one 16-byte piece of codes
// per row); the A operand uses the same assignment, which only permutes the
// order of the sum.
#include "common.h"
#include "dma.h"
#include "internal.h"

namespace moe {

constexpr int kPM = kPrefillMTile;  // 128 sorted slots per tile
constexpr int kWR = 64;             // weight rows per wave
constexpr int kPK = 64;             // inputs per k step
constexpr int kABuf = kPM * kPK * 2;          // bytes of one A tile (16 KiB)
constexpr int kBStage = kWR * kPK;            // bytes of one wave's codes for two k steps (4 KiB)
constexpr int kSGroup = kWR * 16;             // bytes of one wave's scales for four k steps (1 KiB)

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

// 16-byte slot of piece j in A row r (8 pieces per row)
__device__ __forceinline__ int a_slot(int r, int j) { return j ^ ((r & 7) ^ ((r >> 3) & 1)); }
// 16-byte slot of piece c in B row r (4 pieces per row)
__device__ __forceinline__ int b_slot(int r, int c) { return c ^ (((r >> 1) ^ (r >> 3)) & 3); }

// NW waves per workgroup: the A tile is shared by all of them, and an A ring
// of RA tiles gives the A loads RA-1 steps to land. The launches use 4 waves
// (two workgroups per CU); 8 waves with a 3-deep A ring (one workgroup per
// CU) measured slower on the T=8192 workload.
constexpr int kWaves = 4;
template <int NW>
struct Cfg {
  static constexpr int kRA = (NW == 8) ? 3 : 2;
  static constexpr int kALoads = kPM / NW / 8;  // wave-wide A loads per step (8 rows each)
};

template <int NW>
struct TileCtx {
  const uint8_t* in;      // A matrix (bytes), uniform
  const uint8_t* rec;     // the expert's record, uniform
  uint32_t a_off[Cfg<NW>::kALoads];  // byte offsets in A of this lane's pieces at k = 0
  uint32_t b_off[4];      // byte offsets in the record of this lane's code pieces at k = 0
  uint32_t s_off;         // byte offset in the record of weight row (wave row = lane)'s scales at k = 0
  uint32_t a_lds;         // LDS base of this wave's A rows in A tile 0
  uint32_t b_lds[2];      // the wave's code stages
  uint32_t s_lds[2];      // the wave's scale groups
};

// A of step ks -> A tile t: the wave loads rows (kPM/NW) w + 8i + l/8.
template <int NW>
__device__ __forceinline__ void dma_a(const TileCtx<NW>& c, int ks, int t) {
#pragma unroll
  for (int i = 0; i < Cfg<NW>::kALoads; i++)
    dma16(c.in + ks * (kPK * 2), c.a_off[i], c.a_lds + t * kABuf + 1024 * i);
}
// codes of stage g (k steps 2g, 2g+1) -> the wave's stage buffer t
template <int NW>
__device__ __forceinline__ void dma_b(const TileCtx<NW>& c, int g, int t) {
#pragma unroll
  for (int i = 0; i < 4; i++) dma16(c.rec + g * 64, c.b_off[i], c.b_lds[t] + 1024 * i);
}
// scales of group G (k steps 4G..4G+3) -> the wave's group buffer t
template <int NW>
__device__ __forceinline__ void dma_s(const TileCtx<NW>& c, int G, int t) {
  dma16(c.rec + G * 16, c.s_off, c.s_lds[t]);
}

// word of 8 E2M1 codes -> 8 bf16 unit values e2m1 * e4m3 (exact)
__device__ __forceinline__ bf16x8 deq8(uint32_t word, float sb) {
  const f32x2 v0 = e2m1x2_f32<0>(word), v1 = e2m1x2_f32<1>(word);
  const f32x2 v2 = e2m1x2_f32<2>(word), v3 = e2m1x2_f32<3>(word);
  const u32x4 o = {f32x2_to_bf16x2(v0.x * sb, v0.y * sb), f32x2_to_bf16x2(v1.x * sb, v1.y * sb),
                   f32x2_to_bf16x2(v2.x * sb, v2.y * sb), f32x2_to_bf16x2(v3.x * sb, v3.y * sb)};
  return __builtin_bit_cast(bf16x8, o);
}

// The B operand of one k step as each lane holds it: the code words of its
// two 32-row fragments (four k-slices each) and their E4M3 block scales.
struct BStep {
  u32x4 bc[2];
  float sb[2][2];
};

// Reads step (t, q)'s B operand from the wave's code stage Bs (half t) and
// scale group Ss (step q within it).
__device__ __forceinline__ void load_bstep(const uint8_t* Bs, int t, const uint8_t* Ss, int q, BStep& b) {
  const int lane = threadIdx.x & 63, h = lane >> 5, n = lane & 31;
#pragma unroll
  for (int f = 0; f < 2; f++) {
    const int r = 32 * f + n;
    b.bc[f] = *reinterpret_cast<const u32x4*>(Bs + r * 64 + 16 * b_slot(r, 2 * t + h));
    // scale bytes 2h, 2h+1 of the step: inputs 32h..32h+15 and +16..+31
    const uint32_t v = *reinterpret_cast<const uint32_t*>(Ss + r * 16 + 4 * q) >> (16 * h);
    b.sb[f][0] = e4m3_f32<0>(v);
    b.sb[f][1] = e4m3_f32<1>(v);
  }
}

// MFMAs of one k-slice interleaved with the VALU work beside them: each MFMA
// is followed by up to four VALU instructions (the dequant of the next
// slice), so the wave's in-order issue fills the MFMA's shadow instead of
// stalling on back-to-back MFMAs and then running the VALU work alone.
template <int NMS>
__device__ __forceinline__ void interleave_slice() {
#pragma unroll
  for (int i = 0; i < 2 * NMS; i++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // up to four VALU
  }
}

// The MFMAs of one k step on A tile As, with this step's B operand in cur and
// its first k-slice already dequantized in bfr. Software pipeline over the
// four k-slices: the A fragments and the dequantized B fragments of slice
// kk+1 are prepared while the MFMAs of slice kk run (the A reads of a slice
// are issued before the MFMAs of the one before, kept apart by scheduling
// barriers). The next step's B operand (codes and scales of this wave's own
// stage, so no barrier is needed; the caller has waited for its loads) is
// read into nxt during slice 2 and its first slice dequantized into bfr
// during slice 3, so the next step starts with its first MFMAs ready.
// Measured on the T = 8192 workload: gate/up 3.25 against 3.33-3.35 ms for
// the form that read each step's B operand at its start.
template <int NMS>
__device__ __forceinline__ void step_mfma(const uint8_t* As, BStep& cur, BStep& nxt, const uint8_t* nBs, int nt,
                                          const uint8_t* nSs, int nq, bf16x8 (&bfr)[2], f32x16 (&acc)[4][2]) {
  const int lane = threadIdx.x & 63, h = lane >> 5, n = lane & 31;
  bf16x8 af[4];
#pragma unroll
  for (int ms = 0; ms < NMS; ms++) {
    const int r = 32 * ms + n;
    af[ms] = *reinterpret_cast<const bf16x8*>(As + r * 128 + 16 * a_slot(r, 4 * h));
  }
#pragma unroll
  for (int kk = 0; kk < 4; kk++) {
    bf16x8 an[4], bn[2];
    if (kk < 3) {
#pragma unroll
      for (int ms = 0; ms < NMS; ms++) {
        const int r = 32 * ms + n;
        an[ms] = *reinterpret_cast<const bf16x8*>(As + r * 128 + 16 * a_slot(r, 4 * h + kk + 1));
      }
    }
    // the next step's B operand is read a slice ahead of its use
    if (kk == 2) load_bstep(nBs, nt, nSs, nq, nxt);
    __builtin_amdgcn_sched_barrier(0);
    if (kk < 3) {
#pragma unroll
      for (int f = 0; f < 2; f++) bn[f] = deq8(cur.bc[f][kk + 1], cur.sb[f][(kk + 1) >> 1]);
    } else {
#pragma unroll
      for (int f = 0; f < 2; f++) bn[f] = deq8(nxt.bc[f][0], nxt.sb[f][0]);
    }
#pragma unroll
    for (int ms = 0; ms < NMS; ms++)
#pragma unroll
      for (int f = 0; f < 2; f++)
        acc[ms][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ms], bfr[f], acc[ms][f], 0, 0, 0);
    interleave_slice<NMS>();
    __builtin_amdgcn_sched_barrier(0);
    if (kk < 3) {
#pragma unroll
      for (int ms = 0; ms < NMS; ms++) af[ms] = an[ms];
    }
#pragma unroll
    for (int f = 0; f < 2; f++) bfr[f] = bn[f];
  }
}

// Step s of the k loop, I = s mod 8. Issue order (the waits count on it):
// A of step s+1 into A tile (s+1)%2; on even steps the codes of the next
// stage (4 loads); every fourth step the scales of the next group (1 load).
// Then the MFMAs of step s on A tile s%2. The next step's B operand is read
// during the last k-slice: on odd steps it comes from the next stage, issued
// on the step before, so first wait until only this step's A loads may be
// outstanding (on even steps it is in the current stage, which has landed).
// Before the barrier, wait until A of step s+1 has landed (the first loads of
// this step). Buffers written here were last read on the step before, which
// every wave has finished (barrier). Loads past the last step repeat it (into
// buffers never read again), and the last step's look-ahead reads LDS that
// nothing uses.
template <int NW, int NMS, int I>
__device__ __forceinline__ void kstep(const TileCtx<NW>& c, int s, int nk, const uint8_t* As, const uint8_t* B0,
                                      const uint8_t* B1, const uint8_t* S0, const uint8_t* S1, BStep (&bs)[2],
                                      bf16x8 (&bfr)[2], f32x16 (&acc)[4][2]) {
  static_assert(Cfg<NW>::kRA == 2, "two A tiles");
  dma_a(c, min(s + 1, nk - 1), (s + 1) % 2);
  if (I % 2 == 0) dma_b(c, min(s / 2 + 1, (nk - 1) / 2), (I / 2 + 1) % 2);
  if (I % 4 == 0) dma_s(c, min(s / 4 + 1, (nk - 1) / 4), (I / 4 + 1) % 2);
  constexpr int J = (I + 1) % 8;  // the next step
  if (I % 2 == 1) wait_vmcnt<Cfg<NW>::kALoads>();
  __builtin_amdgcn_sched_barrier(0);
  // the MFMA section at raised wave priority: the SIMD's arbiter then
  // favours the wave feeding the matrix core over the other workgroup's wave
  // in its load issue, waits or epilogue (gate/up 1-1.5 % faster on the
  // T = 8192 workload, down within 1 % either way; raised per k-slice
  // instead: 8 % slower)
  __builtin_amdgcn_s_setprio(1);
  step_mfma<NMS>(As + (s % 2) * kABuf, bs[I % 2], bs[J % 2], ((J / 2) % 2) ? B1 : B0, J % 2, ((J / 4) % 2) ? S1 : S0,
                 J % 4, bfr, acc);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
  constexpr int later = ((I % 2 == 0) ? 4 : 0) + ((I % 4 == 0) ? 1 : 0);  // issued after this step's A
  wait_vmcnt<later>();
  step_barrier();
}

template <int NW, int NMS>
__device__ __forceinline__ void kloop(const TileCtx<NW>& c, int nk, const uint8_t* lds_a, const uint8_t* B0,
                                      const uint8_t* B1, const uint8_t* S0, const uint8_t* S1,
                                      f32x16 (&acc)[4][2]) {
  BStep bs[2];
  bf16x8 bfr[2];
  load_bstep(B0, 0, S0, 0, bs[0]);
#pragma unroll
  for (int f = 0; f < 2; f++) bfr[f] = deq8(bs[0].bc[f][0], bs[0].sb[f][0]);
  int s = 0;
  for (; s + 8 <= nk; s += 8) {
    kstep<NW, NMS, 0>(c, s, nk, lds_a, B0, B1, S0, S1, bs, bfr, acc);
    kstep<NW, NMS, 1>(c, s + 1, nk, lds_a, B0, B1, S0, S1, bs, bfr, acc);
    kstep<NW, NMS, 2>(c, s + 2, nk, lds_a, B0, B1, S0, S1, bs, bfr, acc);
    kstep<NW, NMS, 3>(c, s + 3, nk, lds_a, B0, B1, S0, S1, bs, bfr, acc);
    kstep<NW, NMS, 4>(c, s + 4, nk, lds_a, B0, B1, S0, S1, bs, bfr, acc);
    kstep<NW, NMS, 5>(c, s + 5, nk, lds_a, B0, B1, S0, S1, bs, bfr, acc);
    kstep<NW, NMS, 6>(c, s + 6, nk, lds_a, B0, B1, S0, S1, bs, bfr, acc);
    kstep<NW, NMS, 7>(c, s + 7, nk, lds_a, B0, B1, S0, S1, bs, bfr, acc);
  }
  if (s < nk) kstep<NW, NMS, 0>(c, s, nk, lds_a, B0, B1, S0, S1, bs, bfr, acc);
  if (s + 1 < nk) kstep<NW, NMS, 1>(c, s + 1, nk, lds_a, B0, B1, S0, S1, bs, bfr, acc);
  if (s + 2 < nk) kstep<NW, NMS, 2>(c, s + 2, nk, lds_a, B0, B1, S0, S1, bs, bfr, acc);
  if (s + 3 < nk) kstep<NW, NMS, 3>(c, s + 3, nk, lds_a, B0, B1, S0, S1, bs, bfr, acc);
  if (s + 4 < nk) kstep<NW, NMS, 4>(c, s + 4, nk, lds_a, B0, B1, S0, S1, bs, bfr, acc);
  if (s + 5 < nk) kstep<NW, NMS, 5>(c, s + 5, nk, lds_a, B0, B1, S0, S1, bs, bfr, acc);
  if (s + 6 < nk) kstep<NW, NMS, 6>(c, s + 6, nk, lds_a, B0, B1, S0, S1, bs, bfr, acc);
}

// NPROJ = 2: gate and up (wave w: gate rows n0+32w.. and the same up rows,
// 32 NW output columns per tile), SwiGLU epilogue into mid; NPROJ = 1: down
// (wave w: rows n0+64w.., 64 NW output columns per tile), routing-weighted
// f32 rows into part.
//
// NW = 4: two workgroups share a CU (at most 256 registers per lane, 73 KB
// of LDS each), so one workgroup's MFMAs cover the other's loads and
// barriers.
//
// Work mapping: the hardware hands out workgroups round-robin over the 8
// XCDs, each with its own L2. Workgroup L runs item (L % 8) * per + L / 8, so
// every XCD walks a contiguous run of items. Items are ordered by expert, and
// within an expert n-tile major with the expert's M tiles adjacent: those
// tiles read the same weight rows at the same time from the same L2, and the
// expert's activation rows stay there across its n-tiles.
template <int NPROJ, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void prefill_kernel(PrefillArgs a) {
  constexpr int RA = Cfg<NW>::kRA;
  const int ncol = (NPROJ == 2) ? 32 * NW : kWR * NW;  // output columns per tile
  const int N = (NPROJ == 2) ? a.I : a.H;
  const int K = (NPROJ == 2) ? a.H : a.I;
  const int ntn = (N + ncol - 1) / ncol;
  const int n_items = a.rt.counts[1] * ntn;
  const int per = (n_items + 7) / 8;
  const int slot = blockIdx.x / 8, xcd = blockIdx.x % 8;
  if (slot >= per) return;
  int item = xcd * per + slot;
  if (item >= n_items) return;
  if (NPROJ == 1) item = n_items - 1 - item;  // down: most recently written mids first
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
  const int p0 = (NPROJ == 2) ? 0 : 2;
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[RA * kABuf];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b0[NW * kBStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b1[NW * kBStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds_s0[NW * kSGroup];
  __shared__ __attribute__((aligned(16))) uint8_t lds_s1[NW * kSGroup];
  __shared__ int src_row[kPM];
  __shared__ int out_pair[NPROJ == 1 ? kPM : 1];   // down: pair id of each tile row
  __shared__ float out_w[NPROJ == 1 ? kPM : 1];    // down: its routing weight
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid < kPM) {
    // rows past the tile's end read a valid stand-in row; their outputs are not stored
    const int r = min(tid, rows - 1);
    if (NPROJ == 2) {
      src_row[tid] = a.rt.sorted[row0 + r] / a.k;
    } else {
      src_row[tid] = r;  // mid rows counted from the tile's first slot (c.in)
      const int pair = a.rt.sorted[row0 + r];
      out_pair[tid] = pair;
      out_w[tid] = a.w[pair];
    }
  }
  TileCtx<NW> c;
  // A's base: gate/up the activations x (a token's row at its token id; the
  // host keeps T * H * 2 below 2^31 bytes per launch), down the tile's first
  // mid row, so the 32-bit per-lane offsets stay below 128 rows
  c.in = uniform_ptr(NPROJ == 2 ? a.in : a.in + (size_t)row0 * K);
  c.rec = uniform_ptr(a.bank + (size_t)e * a.stride);
  float t_p[NPROJ];
#pragma unroll
  for (int q = 0; q < NPROJ; q++) t_p[q] = global_factor(*reinterpret_cast<const float*>(c.rec + a.g[p0 + q]));
  // weight row (output index, projection) of the wave's row r (0..63); rows
  // past N read row 0 (their outputs are not stored)
  auto wrow = [&](int r, int& q) {
    q = (NPROJ == 2) ? (r >> 5) : 0;
    const int n = (NPROJ == 2) ? n0 + 32 * wave + (r & 31) : n0 + kWR * wave + r;
    return n < N ? n : 0;
  };
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int r = 16 * i + (lane >> 2);
    int q;
    const int n = wrow(r, q);
    const int piece = b_slot(r, lane & 3);  // slot lane&3 of row r holds this piece
    c.b_off[i] = (uint32_t)(a.codes[p0 + q] + (size_t)n * (K / 2) + 16 * piece);
  }
  {
    int q;
    const int n = wrow(lane, q);
    c.s_off = (uint32_t)(a.scales[p0 + q] + (size_t)n * (K / 16));
  }
  constexpr int arows = kPM / NW;  // A rows loaded by each wave
  const uint8_t* const B0 = lds_b0 + wave * kBStage;
  const uint8_t* const B1 = lds_b1 + wave * kBStage;
  const uint8_t* const S0 = lds_s0 + wave * kSGroup;
  const uint8_t* const S1 = lds_s1 + wave * kSGroup;
  c.a_lds = __builtin_amdgcn_readfirstlane(lds_addr(lds_a + arows * wave * 128));
  c.b_lds[0] = __builtin_amdgcn_readfirstlane(lds_addr(B0));
  c.b_lds[1] = __builtin_amdgcn_readfirstlane(lds_addr(B1));
  c.s_lds[0] = __builtin_amdgcn_readfirstlane(lds_addr(S0));
  c.s_lds[1] = __builtin_amdgcn_readfirstlane(lds_addr(S1));
  __syncthreads();
#pragma unroll
  for (int i = 0; i < Cfg<NW>::kALoads; i++) {
    const int r = arows * wave + 8 * i + (lane >> 3);
    const int piece = a_slot(r, lane & 7);
    c.a_off[i] = (uint32_t)src_row[r] * (uint32_t)(K * 2) + 16 * piece;
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int ms = 0; ms < 4; ms++)
#pragma unroll
    for (int f = 0; f < 2; f++) acc[ms][f] = f32x16{};

  const int nk = K / kPK;
#pragma unroll
  for (int j = 0; j < RA - 1; j++) dma_a(c, min(j, nk - 1), j);
  dma_b(c, 0, 0);
  dma_s(c, 0, 0);
  wait_vmcnt<0>();
  step_barrier();
  // 32-row blocks that hold rows of this tile: a partial last tile of an
  // expert runs the k loop without the MFMAs of the rest
  switch (min(4, (rows + 31) / 32)) {
    case 1: kloop<NW, 1>(c, nk, lds_a, B0, B1, S0, S1, acc); break;
    case 2: kloop<NW, 2>(c, nk, lds_a, B0, B1, S0, S1, acc); break;
    case 3: kloop<NW, 3>(c, nk, lds_a, B0, B1, S0, S1, acc); break;
    default: kloop<NW, 4>(c, nk, lds_a, B0, B1, S0, S1, acc); break;
  }
  wait_vmcnt<0>();  // the loads past the last step

  // Epilogue. Accumulator element r of lane l is (row 8(r/4) + 4(l/32) + r%4,
  // column l%32) of its 32 x 32 block, so a lane's values lie in 16 rows of
  // one column. Each 32-row block goes through the wave's own code stages
  // (free once the k loop's loads have landed) and comes back as 16-byte
  // row pieces, so each store writes whole row segments: 8 stores per wave
  // for the bf16 mids instead of 64, 32 for the f32 rows instead of 128
  // (down 1.88 -> 1.77 ms on the T = 8192 workload). 16-byte groups are
  // XOR-swizzled by row bit 2, so the two lane halves' writes (rows 4 apart)
  // fall in different banks.
  if (NPROJ == 2) {
    uint16_t* const tb = reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(B0));  // [32 rows][32 mids]
#pragma unroll
    for (int ms = 0; ms < 4; ms++) {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int rb = 8 * (r >> 2) + 4 * h + (r & 3), col = lane & 31;
        const float g = t_p[0] * acc[ms][0][r];
        const float u = t_p[NPROJ - 1] * acc[ms][1][r];
        tb[rb * 32 + 8 * ((col >> 3) ^ (2 * ((rb >> 2) & 1))) + (col & 7)] = f32_to_bf16(silu_mul(g, u));
      }
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const int rb = (lane >> 2) + 16 * j, cg = lane & 3, row = 32 * ms + rb;
        const u32x4 v = *reinterpret_cast<const u32x4*>(tb + rb * 32 + 8 * (cg ^ (2 * ((rb >> 2) & 1))));
        const int n = n0 + 32 * wave + 8 * cg;  // N % 8 == 0: n < N covers all 8
        if (row < rows && n < N) *reinterpret_cast<u32x4*>(a.mid + (size_t)(row0 + row) * N + n) = v;
      }
    }
  } else {
    float* const tb[2] = {reinterpret_cast<float*>(const_cast<uint8_t*>(B0)),
                          reinterpret_cast<float*>(const_cast<uint8_t*>(B1))};  // [32 rows][32 columns] per f
#pragma unroll
    for (int ms = 0; ms < 4; ms++) {
#pragma unroll
      for (int f = 0; f < 2; f++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int rb = 8 * (r >> 2) + 4 * h + (r & 3), col = lane & 31;
          tb[f][rb * 32 + 4 * ((col >> 2) ^ (4 * ((rb >> 2) & 1))) + (col & 3)] = acc[ms][f][r];
        }
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int rb = (lane >> 3) + 8 * j, cg = lane & 7, row = 32 * ms + rb;
        const int pair = out_pair[row];
        const float wp = out_w[row] * t_p[0];
#pragma unroll
        for (int f = 0; f < 2; f++) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(tb[f] + rb * 32 + 4 * (cg ^ (4 * ((rb >> 2) & 1))));
          const int n = n0 + kWR * wave + 32 * f + 4 * cg;  // N % 4 == 0: n < N covers all 4
          if (row < rows && n < N)
            *reinterpret_cast<f32x4*>(a.part + (size_t)pair * N + n) = f32x4{wp * v.x, wp * v.y, wp * v.z, wp * v.w};
        }
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
  const int items = ((b.I + 32 * kWaves - 1) / (32 * kWaves)) * max_tiles;
  dim3 grid((items + 7) / 8 * 8);
  launch_kernel("prefill_gateup", prefill_kernel<2, kWaves>, grid, dim3(64 * kWaves), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefill_down(const BankView& b, const uint16_t* mid, const float* w, int k,
                               const RouteTables& rt, int max_tiles, float* part, hipStream_t s) {
  PrefillArgs a = make_args(b, k, rt);
  a.in = mid;
  a.w = w;
  a.part = part;
  const int items = ((b.H + 64 * kWaves - 1) / (64 * kWaves)) * max_tiles;
  dim3 grid((items + 7) / 8 * 8);
  launch_kernel("prefill_down", prefill_kernel<1, kWaves>, grid, dim3(64 * kWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
