// The affine8_g64 resident linear for many tokens, on bf16 MFMA (gfx950).
//
// "Beam 1.0 501B-A23B, streaming pack, NVFP4 experts / MLX 8-bit residents",
// "What this pack holds" (residents and q8-rule bullets): W[n][k] =
// scale[n][g] * q[n][k] + bias[n][g] for the group g = k / 64, 8-bit codes q,
// BF16 scale and bias. Per group,
//   sum_{k in g} x[t][k] W[n][k] = scale[n][g] * (sum_{k in g} x[t][k] q[n][k])
//                                + bias[n][g] * (sum_{k in g} x[t][k]),
// exactly. q <= 255 is exact in bf16, so the inner sums run on
// v_mfma_f32_32x32x16_bf16 into a per-group accumulator that the group's
// scale then folds into the output accumulator (f32 FMA, one per output
// element and group). The bias term is one more MFMA per group: the group
// sum of x (f32) is split exactly into three bf16 values x1 + x2 + x3 and
// multiplied with (bias, bias, bias) over three of the k-slice's inputs.
//
// Tile: 128 tokens x 128 output rows per workgroup of 4 waves; wave w owns
// output rows 32 w .. 32 w + 31 for all 128 tokens (4 MFMA blocks of 32 x
// 32). Per group of 64 inputs: the activations (16 KiB) pass through LDS,
// double-buffered and shared by the waves; each lane loads its row's 32
// codes (two 16-byte loads) and its scale straight into registers, one
// group ahead. The 64 inputs of a group are assigned to the MFMA's four
// k-slices so that lane half h = l / 32 takes inputs 32 h .. 32 h + 31 (one
// 32-byte code piece per lane); the activations use the same assignment,
// which only permutes the order of the sum.
//
// Work order: workgroups are dealt round-robin to the 8 XCDs, each with its
// own L2. Workgroup b runs on XCD b mod 8; when the number of row tiles is a
// multiple of 8, XCD x takes the row tiles x, x + 8, ... (a fifth of the
// codes at K = N = 5120, which stay in its L2) for one token tile after the
// other, so the activations stream through each XCD once and the codes are
// read from HBM once per XCD.
#include <mutex>

#include "common.h"
#include "dma.h"
#include "internal.h"

namespace moe {

constexpr int kA8M = 128, kA8N = 128, kA8Threads = 256;

// 16-byte slot of piece j (0..7) in activation row r (128 bytes per row)
__device__ __forceinline__ int a8_slot(int r, int j) { return j ^ ((r & 7) ^ ((r >> 3) & 1)); }

// 4 bytes of codes -> two packed bf16 pairs (exact: a code has at most 8
// significant bits, so its f32 value has a zero low half): v_cvt_f32_ubyte0..3,
// then one byte permute per pair takes the two high halves
__device__ __forceinline__ void u8x4_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const float a = (float)(w & 0xFFu), b = (float)((w >> 8) & 0xFFu);
  const float c = (float)((w >> 16) & 0xFFu), d = (float)(w >> 24);
  lo = __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
  hi = __builtin_amdgcn_perm(__float_as_uint(d), __float_as_uint(c), 0x07060302u);
}

// sum of the 8 bf16 values of a 16-byte piece, by four v_dot2 against (1, 1)
// from 0 (the products are exact). The words go through a plain array: this
// compiler turned a bit cast of a vector element access (v.y) into a read of
// element 0.
__device__ __forceinline__ float piece_sum(const u32x4& v, float s) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  const bf16x2 one2 = __builtin_bit_cast(bf16x2, 0x3F803F80u);
#pragma unroll
  for (int q = 0; q < 4; q++) s = __builtin_amdgcn_fdot2_f32_bf16(one2, __builtin_bit_cast(bf16x2, w[q]), s, false);
  return s;
}

// f32 -> bf16 by truncation (used only where the value is exact in bf16)
__device__ __forceinline__ uint32_t bf16_trunc(float v) { return __float_as_uint(v) >> 16; }

// The group sum of an activation row: thread t takes row t / 2, pieces
// 4 (t % 2) .. 4 (t % 2) + 3 (piece_sum in piece order), and the two halves
// meet by one DPP swap of neighbouring lanes. Thread t % 2 == 0 splits the sum
// exactly into three bf16 values x1 + x2 + x3 and stores them for the bias
// MFMA: x1 | x2 << 16, x3.
__device__ __forceinline__ void store_group_sum(float s, uint32_t (*xs)[2], int r, bool first) {
  s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, true));
  if (first) {
    const float x1 = bf16_to_f32(f32_to_bf16(s));
    const float r1 = s - x1;  // exact
    const float x2 = bf16_to_f32(f32_to_bf16(r1));
    const float x3 = r1 - x2;  // exact, and exact in bf16 (at most 8 significant bits left)
    xs[r][0] = bf16_trunc(x1) | (bf16_trunc(x2) << 16);
    xs[r][1] = bf16_trunc(x3);
  }
}


// two waves per SIMD: the compiler keeps the 128 accumulators and the
// fragments in 216 VGPRs (without the bound: 324 VGPRs and 128 AGPRs, one wave)
__global__ __launch_bounds__(kA8Threads) __attribute__((amdgpu_waves_per_eu(2))) void affine8_gemm_kernel(const uint16_t* __restrict__ x,
                                                                  const uint8_t* __restrict__ codes,
                                                                  const uint16_t* __restrict__ scales,
                                                                  const uint16_t* __restrict__ biases, int T,
                                                                  int K, int N, int n_tiles, int gps,
                                                                  uint16_t* __restrict__ y, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint8_t As[2][kA8M * 128];
  __shared__ __attribute__((aligned(16))) uint32_t Xs[2][kA8M][2];  // group sums of x as bf16 (x1, x2 | x3, 0)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int G = K / 64;
  const int g0 = (int)blockIdx.y * gps, g1 = min(G, g0 + gps);  // this split's groups
  int mt, nt;
  if (n_tiles % 8 == 0) {
    const int per = n_tiles / 8, i = blockIdx.x / 8;
    mt = i / per;
    nt = (int)(blockIdx.x % 8) + 8 * (i % per);
  } else {
    mt = blockIdx.x / n_tiles;
    nt = blockIdx.x % n_tiles;
  }
  const int m0 = mt * kA8M;
  const int n = nt * kA8N + wave * 32 + l32;  // this lane's output row (MFMA column)
  const int nc = n < N ? n : N - 1;
  const uint8_t* crow = codes + (size_t)nc * K + 32 * h;
  // activation pieces of this thread: row tid / 2, pieces 4 (tid % 2) + i
  const int ar = tid >> 1, ah = tid & 1;
  u32x4 av[4];
  auto load_a = [&](int g) {
    const int t = m0 + ar;
#pragma unroll
    for (int i = 0; i < 4; i++)
      av[i] = t < T ? *reinterpret_cast<const u32x4*>(x + (size_t)t * K + 64 * g + 8 * (4 * ah + i))
                    : u32x4{0u, 0u, 0u, 0u};
  };
  // the pieces into LDS, and the row's group sum
  auto store_a = [&](int buf) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      *reinterpret_cast<u32x4*>(&As[buf][ar * 128 + 16 * a8_slot(ar, 4 * ah + i)]) = av[i];
      s = piece_sum(av[i], s);
    }
    store_group_sum(s, Xs[buf], ar, ah == 0);
  };
  u32x4 bc[2], bn[2];
  float sc = 0.0f, scn = 0.0f, bi = 0.0f, bin = 0.0f;
  auto load_b = [&](int g, u32x4 (&b)[2], float& s, float& bb) {
    b[0] = *reinterpret_cast<const u32x4*>(crow + 64 * g);
    b[1] = *reinterpret_cast<const u32x4*>(crow + 64 * g + 16);
    s = bf16_to_f32(scales[(size_t)nc * G + g]);
    bb = bf16_to_f32(biases[(size_t)nc * G + g]);
  };

  f32x16 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; mb++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[mb][r] = 0.0f;

  load_a(g0);
  load_b(g0, bc, sc, bi);
  store_a(g0 & 1);
  __syncthreads();
  for (int g = g0; g < g1; g++) {
    const int buf = g & 1;
    if (g + 1 < g1) {
      load_a(g + 1);
      load_b(g + 1, bn, scn, bin);
    }
    const uint8_t* A = As[buf];
    f32x16 tmp[4];
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      // B: this lane's 8 codes of slice kk (bytes 8 kk .. 8 kk + 7 of its piece)
      const uint32_t w0 = kk < 2 ? (kk == 0 ? bc[0].x : bc[0].z) : (kk == 2 ? bc[1].x : bc[1].z);
      const uint32_t w1 = kk < 2 ? (kk == 0 ? bc[0].y : bc[0].w) : (kk == 2 ? bc[1].y : bc[1].w);
      uint32_t q0, q1, q2, q3;
      u8x4_bf16(w0, q0, q1);
      u8x4_bf16(w1, q2, q3);
      const bf16x8 bfr = __builtin_bit_cast(bf16x8, u32x4{q0, q1, q2, q3});
#pragma unroll
      for (int mb = 0; mb < 4; mb++) {
        const int r = 32 * mb + l32;
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(A + r * 128 + 16 * a8_slot(r, 4 * h + kk));
        if (kk == 0) {
          f32x16 z;
#pragma unroll
          for (int e = 0; e < 16; e++) z[e] = 0.0f;
          tmp[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr, z, 0, 0, 0);
        } else {
          tmp[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr, tmp[mb], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int mb = 0; mb < 4; mb++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[mb][e] = fmaf(sc, tmp[mb][e], acc[mb][e]);
    // bias: inputs 0..2 of a k-slice carry (x1, x2, x3) against (b, b, b)
    {
      const uint32_t bb = bf16_trunc(bi);
      const bf16x8 bbf = __builtin_bit_cast(
          bf16x8, h == 0 ? u32x4{bb | (bb << 16), bb, 0u, 0u} : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
      for (int mb = 0; mb < 4; mb++) {
        const int r = 32 * mb + l32;
        const bf16x8 xf = __builtin_bit_cast(
            bf16x8, h == 0 ? u32x4{Xs[buf][r][0], Xs[buf][r][1], 0u, 0u} : u32x4{0u, 0u, 0u, 0u});
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf, bbf, acc[mb], 0, 0, 0);
      }
    }
    if (g + 1 < g1) {
      store_a(buf ^ 1);
      bc[0] = bn[0];
      bc[1] = bn[1];
      sc = scn;
      bi = bin;
    }
    __syncthreads();
  }
  // element e of lane l: token 8 (e / 4) + 4 h + e % 4 of block mb, row n
  if (n < N) {
#pragma unroll
    for (int mb = 0; mb < 4; mb++)
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int t = m0 + 32 * mb + 8 * (e / 4) + 4 * h + (e % 4);
        if (t < T) {
          if (part)
            part[((size_t)blockIdx.y * T + t) * N + n] = acc[mb][e];
          else
            y[(size_t)t * N + n] = f32_to_bf16(acc[mb][e]);
        }
      }
  }
}

// The same GEMM with every operand going HBM -> LDS by global_load_lds_dwordx4
// (K a multiple of 512, scale and bias rows 16-byte aligned). The kernel above
// loads the next group's activations into registers during a group and
// stores them to LDS at its end, so each group waits out the round trip of
// loads issued one group earlier. Here the loads write no registers and the
// loop waits for them itself, by count:
//   - activations: three LDS stages, loaded two groups ahead (4 loads per
//     wave: rows 32 w + 8 i + l / 8, the 16-byte piece that belongs in slot
//     l % 8 of the swizzled row);
//   - codes: two stages, one group ahead, each wave its own 32 rows (2 loads:
//     rows 16 i + l / 4, piece (l % 4) ^ ((row / 4) % 4) in slot l % 4, so
//     that 16 lanes' reads of 16 consecutive rows fall in distinct banks);
//   - scales and biases: 16 bytes (8 groups) of each row, a block ahead
//     (wave w loads 64 rows of one of the two arrays), double-buffered.
// Per group g: wait for group g's loads (the only loads issued later are the
// activations of group g + 1: vmcnt(4)), barrier, issue the next loads; read
// the step's small LDS operands together (the pieces of group g's sums, the
// lane's codes, group g - 1's sums and bias, group g's scale); then group g's
// MFMAs into tmp, each slice's A fragments and codes prepared while the
// previous slice's MFMAs run and one piece of the sums added per slice; store
// group g's sums into a double-buffered Xs; the bias MFMA of group g - 1
// (whose sums the barrier has completed); group g's scale fold. The last
// group's bias follows a barrier after the loop. The accumulator sees the
// same operations in the same order as in the kernel above (fold g, bias g,
// fold g + 1, ...), so the output is the same bit for bit, with one barrier
// per group.
constexpr int kA8DStages = 3;  // activation stages

__device__ __forceinline__ int a8_cslot(int r, int p) { return p ^ ((r >> 2) & 3); }

__global__ __launch_bounds__(kA8Threads) __attribute__((amdgpu_waves_per_eu(2))) void affine8_gemm_dma_kernel(
    const uint16_t* __restrict__ x, const uint8_t* codes, const uint16_t* scales, const uint16_t* biases, int T,
    int K, int N, int n_tiles, int gps, uint16_t* __restrict__ y, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint8_t As[kA8DStages][kA8M * 128];
  __shared__ __attribute__((aligned(16))) uint8_t Cs[2][kA8N * 64];            // [row][64 codes], swizzled
  __shared__ __attribute__((aligned(16))) uint16_t Ss[2][2][kA8N][8];          // [block][scale|bias][row][group]
  __shared__ __attribute__((aligned(16))) uint32_t Xs[2][kA8M][2];            // group sums of x as bf16
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int G = K / 64;
  int mt, nt;
  if (n_tiles % 8 == 0) {
    const int per = n_tiles / 8, i = blockIdx.x / 8;
    mt = i / per;
    nt = (int)(blockIdx.x % 8) + 8 * (i % per);
  } else {
    mt = blockIdx.x / n_tiles;
    nt = blockIdx.x % n_tiles;
  }
  const int m0 = mt * kA8M, n0 = nt * kA8N;
  const int n = n0 + wave * 32 + l32;  // this lane's output row (MFMA column)
  const int g0 = (int)blockIdx.y * gps, g1 = min(G, g0 + gps);  // this split's groups (whole blocks of 8)

  // load sources: uniform bases and per-lane 32-bit offsets
  const uint8_t* xb = uniform_ptr(x + (size_t)m0 * K);
  const uint8_t* cb = uniform_ptr(codes + (size_t)n0 * K);
  const uint8_t* sb = uniform_ptr((wave < 2 ? scales : biases) + (size_t)n0 * G);
  uint32_t a_off[4], c_off[2];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int r = 32 * wave + 8 * i + (lane >> 3);
    a_off[i] = (uint32_t)((min(m0 + r, T - 1) - m0) * K * 2 + 16 * a8_slot(r, lane & 7));
  }
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int r = 32 * wave + 16 * i + (lane >> 2);
    c_off[i] = (uint32_t)((min(n0 + r, N - 1) - n0) * K + 16 * a8_cslot(r, lane & 3));
  }
  const int s_row = 64 * (wave & 1) + lane;
  const uint32_t s_off = (uint32_t)((min(n0 + s_row, N - 1) - n0) * G * 2);
  // LDS destinations: wave-uniform bases, the stage or buffer added per load
  const uint32_t a_lds = __builtin_amdgcn_readfirstlane(lds_addr(&As[0][0]) + 32 * wave * 128);
  const uint32_t c_lds = __builtin_amdgcn_readfirstlane(lds_addr(&Cs[0][0]) + 32 * wave * 64);
  const uint32_t s_lds = __builtin_amdgcn_readfirstlane(lds_addr(&Ss[0][wave >> 1][64 * (wave & 1)][0]));
  // group g's activations into stage g % 3 (4 loads)
  auto issue_a = [&](int g) {
    const uint32_t l = __builtin_amdgcn_readfirstlane(a_lds + (uint32_t)(g % kA8DStages) * (kA8M * 128));
#pragma unroll
    for (int i = 0; i < 4; i++) dma16(xb + 128 * g, a_off[i], l + 1024 * i);
  };
  // group g's codes into buffer g % 2 (2 loads), and at the start of a block
  // of 8 groups the block's scales or biases (1 load)
  auto issue_c = [&](int g) {
    const uint32_t l = __builtin_amdgcn_readfirstlane(c_lds + (uint32_t)(g & 1) * (kA8N * 64));
#pragma unroll
    for (int i = 0; i < 2; i++) dma16(cb + 64 * g, c_off[i], l + 1024 * i);
    if ((g & 7) == 0)
      dma16(sb + 2 * g, s_off,
            __builtin_amdgcn_readfirstlane(s_lds + (uint32_t)((g >> 3) & 1) * (uint32_t)sizeof(Ss[0])));
  };

  f32x16 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; mb++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[mb][r] = 0.0f;
  const int cr = 32 * wave + l32;         // this lane's code row in the tile
  const int ar = tid >> 1, ah = tid & 1;  // group sums: row tid / 2, pieces 4 (tid % 2) ..

  // a group's bias: inputs 0..2 of a k-slice carry the sums (x1, x2, x3) of
  // row 32 mb + l32 (xv[mb]) against (b, b, b), b this lane's bias bits
  auto bias_mfma = [&](const uint32_t (&xv)[4][2], uint32_t bb) {
    const bf16x8 bbf =
        __builtin_bit_cast(bf16x8, h == 0 ? u32x4{bb | (bb << 16), bb, 0u, 0u} : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
    for (int mb = 0; mb < 4; mb++) {
      const bf16x8 xf =
          __builtin_bit_cast(bf16x8, h == 0 ? u32x4{xv[mb][0], xv[mb][1], 0u, 0u} : u32x4{0u, 0u, 0u, 0u});
      acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf, bbf, acc[mb], 0, 0, 0);
    }
  };
  // group gb's sums and this lane's bias, from LDS
  auto read_bias = [&](int gb, uint32_t (&xv)[4][2], uint32_t& bb) {
    bb = Ss[(gb >> 3) & 1][1][cr][gb & 7];
#pragma unroll
    for (int mb = 0; mb < 4; mb++) {
      xv[mb][0] = Xs[gb & 1][32 * mb + l32][0];
      xv[mb][1] = Xs[gb & 1][32 * mb + l32][1];
    }
  };

  issue_c(g0);
  issue_a(g0);
  if (g0 + 1 < g1) issue_a(g0 + 1);
  for (int g = g0; g < g1; g++) {
    // group g's codes, scales and activations have landed for this wave: the
    // loads issued after them are group g + 1's activations
    if (g + 1 < g1)
      wait_vmcnt<4>();
    else
      wait_vmcnt<0>();
    // every wave's loads of group g have landed, and every wave is done with
    // group g - 1 (codes buffer (g + 1) % 2, activation stage (g + 2) % 3)
    step_barrier();
    if (g + 1 < g1) issue_c(g + 1);
    if (g + 2 < g1) issue_a(g + 2);
    const uint8_t* A = As[g % kA8DStages];
    // the step's small LDS reads, all issued before the MFMAs: this thread's
    // pieces for group g's sums, the lane's 32 codes (row cr, bytes 32 h ..
    // 32 h + 31), group g - 1's sums and bias, group g's scale
    u32x4 pv[4];
#pragma unroll
    for (int i = 0; i < 4; i++) pv[i] = *reinterpret_cast<const u32x4*>(A + ar * 128 + 16 * a8_slot(ar, 4 * ah + i));
    const uint8_t* crow = Cs[g & 1] + cr * 64;
    const u32x4 bc0 = *reinterpret_cast<const u32x4*>(crow + 16 * a8_cslot(cr, 2 * h));
    const u32x4 bc1 = *reinterpret_cast<const u32x4*>(crow + 16 * a8_cslot(cr, 2 * h + 1));
    uint32_t xv[4][2] = {}, bb = 0;
    if (g > g0) read_bias(g - 1, xv, bb);
    const uint32_t scb = Ss[(g >> 3) & 1][0][cr][g & 7];
    __builtin_amdgcn_sched_barrier(0);
    // slice kk: inputs 8 kk .. 8 kk + 7 of each lane half's 32; its A
    // fragments and dequantized codes are read and prepared while the MFMAs
    // of slice kk - 1 run (scheduling barriers keep the reads ahead)
    auto codes_of = [&](int kk) {
      const uint32_t w0 = kk < 2 ? (kk == 0 ? bc0.x : bc0.z) : (kk == 2 ? bc1.x : bc1.z);
      const uint32_t w1 = kk < 2 ? (kk == 0 ? bc0.y : bc0.w) : (kk == 2 ? bc1.y : bc1.w);
      uint32_t q0, q1, q2, q3;
      u8x4_bf16(w0, q0, q1);
      u8x4_bf16(w1, q2, q3);
      return __builtin_bit_cast(bf16x8, u32x4{q0, q1, q2, q3});
    };
    auto a_frag = [&](int mb, int kk) {
      const int r = 32 * mb + l32;
      return *reinterpret_cast<const bf16x8*>(A + r * 128 + 16 * a8_slot(r, 4 * h + kk));
    };
    // the MFMAs at raised wave priority, so the SIMD's arbiter favours the
    // wave feeding the matrix core (0.755-0.770 -> 0.731-0.734 ms at
    // 8192 x 5120 x 5120)
    __builtin_amdgcn_s_setprio(1);
    f32x16 tmp[4];
    float gsum = 0.0f;  // group g's sum over this thread's four pieces, one per slice
    bf16x8 af[4], bfr = codes_of(0);
#pragma unroll
    for (int mb = 0; mb < 4; mb++) af[mb] = a_frag(mb, 0);
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      bf16x8 an[4], bn;
      if (kk < 3) {
#pragma unroll
        for (int mb = 0; mb < 4; mb++) an[mb] = a_frag(mb, kk + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kk < 3) bn = codes_of(kk + 1);
#pragma unroll
      for (int mb = 0; mb < 4; mb++) {
        if (kk == 0) {
          f32x16 z;
#pragma unroll
          for (int e = 0; e < 16; e++) z[e] = 0.0f;
          tmp[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr, z, 0, 0, 0);
        } else {
          tmp[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr, tmp[mb], 0, 0, 0);
        }
      }
      gsum = piece_sum(pv[kk], gsum);
      __builtin_amdgcn_sched_barrier(0);
      if (kk < 3) {
#pragma unroll
        for (int mb = 0; mb < 4; mb++) af[mb] = an[mb];
        bfr = bn;
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // group g's sums (store_group_sum), for its bias in the next step
    store_group_sum(gsum, Xs[g & 1], ar, ah == 0);
    // group g - 1's bias, then group g's scale fold
    if (g > g0) bias_mfma(xv, bb);
    const float scf = bf16_to_f32(scb);
#pragma unroll
    for (int mb = 0; mb < 4; mb++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[mb][e] = fmaf(scf, tmp[mb][e], acc[mb][e]);
  }
  step_barrier();  // the last group's sums are complete
  {
    uint32_t xv[4][2], bb;
    read_bias(g1 - 1, xv, bb);
    bias_mfma(xv, bb);
  }
  // element e of lane l: token 8 (e / 4) + 4 h + e % 4 of block mb, row n
  if (n < N) {
#pragma unroll
    for (int mb = 0; mb < 4; mb++)
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int t = m0 + 32 * mb + 8 * (e / 4) + 4 * h + (e % 4);
        if (t < T) {
          if (part)
            part[((size_t)blockIdx.y * T + t) * N + n] = acc[mb][e];
          else
            y[(size_t)t * N + n] = f32_to_bf16(acc[mb][e]);
        }
      }
  }
}

// y = bf16 of the splits' f32 partial sums, added in split order
__global__ __launch_bounds__(256) void affine8_split_sum_kernel(const float* __restrict__ part, int S, size_t tn,
                                                               uint16_t* __restrict__ y) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < tn; i += (size_t)gridDim.x * 256) {
    float v = part[i];
    for (int sp = 1; sp < S; sp++) v += part[(size_t)sp * tn + i];
    y[i] = f32_to_bf16(v);
  }
}

// The split form's scratch comes from a stream-ordered pool of this library,
// one per device, that keeps its memory (release threshold at the maximum):
// after the first calls an allocation is a stream-ordered reuse, not a trip
// to the driver (7-10 us per call at T = 64 to 256 with the default pool).
static hipMemPool_t split_pool() {
  static std::mutex mu;
  static hipMemPool_t pools[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!pools[dev]) {
    hipMemPoolProps props{};
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t p = nullptr;
    if (hipMemPoolCreate(&p, &props) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    uint64_t keep = UINT64_MAX;
    if (hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep) != hipSuccess) (void)hipGetLastError();
    pools[dev] = p;
  }
  return pools[dev];
}

// workgroups of this GEMM resident at once on the current device (two per CU)
static int gemm_slots() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return 2 * cus;
}

hipError_t launch_affine8_gemm(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                               const uint16_t* biases, int T, int K, int N, uint16_t* y, hipStream_t s) {
  const int n_tiles = (N + kA8N - 1) / kA8N, m_tiles = (T + kA8M - 1) / kA8M, tiles = n_tiles * m_tiles;
  const int G = K / 64;
  // Few tiles (fewer than the CUs: a prefill of a few hundred tokens) leave
  // most of the chip idle while each walks all G groups. Then K is split into
  // S ranges of whole 8-group blocks (the largest even split whose
  // workgroups still all fit at once); each range's sum, fold and bias go to
  // f32 partials (stream-ordered scratch, split_pool), added in range order
  // into y.
  int S = 1, gps = G;
  const int slots = gemm_slots();
  if (slots > 0 && 2 * tiles <= slots && G >= 16) {
    const int nb = (G + 7) / 8;
    for (int d = nb; d >= 2; d--)
      if (nb % d == 0 && tiles * d <= slots) {
        S = d;
        break;
      }
    gps = (nb / S) * 8;
  }
  float* part = nullptr;
  hipMemPool_t pool = S > 1 ? split_pool() : nullptr;
  if (S > 1 && (!pool || hipMallocFromPoolAsync(reinterpret_cast<void**>(&part), (size_t)S * T * N * sizeof(float),
                                                 pool, s) != hipSuccess)) {
    (void)hipGetLastError();  // no scratch: the single-range form
    S = 1;
    gps = G;
    part = nullptr;
  }
  // the HBM -> LDS form: K a multiple of 512 (blocks of 8 groups), 16-byte
  // aligned scale and bias rows, and 32-bit load offsets within a tile
  const bool dma = K % 512 == 0 && ((uintptr_t)scales & 15) == 0 && ((uintptr_t)biases & 15) == 0 &&
                   (uint64_t)kA8M * K * 2 < (1ull << 31);
  const dim3 grid(tiles, S);
  if (dma)
    launch_kernel("affine8_gemm", affine8_gemm_dma_kernel, grid, dim3(kA8Threads), 0, s, x,
                  reinterpret_cast<const uint8_t*>(codes), scales, biases, T, K, N, n_tiles, gps, y, part);
  else
    launch_kernel("affine8_gemm", affine8_gemm_kernel, grid, dim3(kA8Threads), 0, s, x,
                  reinterpret_cast<const uint8_t*>(codes), scales, biases, T, K, N, n_tiles, gps, y, part);
  hipError_t e = hipGetLastError();
  if (S > 1) {
    if (e == hipSuccess) {
      const size_t tn = (size_t)T * N;
      const unsigned blocks = (unsigned)std::min<size_t>((tn + 255) / 256, 4096);
      launch_kernel("affine8_split_sum", affine8_split_sum_kernel, dim3(blocks), dim3(256), 0, s, part, S, tn, y);
      e = hipGetLastError();
    }
    const hipError_t ef = hipFreeAsync(part, s);
    if (e == hipSuccess) e = ef;
  }
  return e;
}

}  // namespace moe
