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
#include "common.h"
#include "internal.h"

namespace moe {

constexpr int kA8M = 128, kA8N = 128, kA8Threads = 256;

// 16-byte slot of piece j (0..7) in activation row r (128 bytes per row)
__device__ __forceinline__ int a8_slot(int r, int j) { return j ^ ((r & 7) ^ ((r >> 3) & 1)); }

// 4 bytes of codes -> two packed bf16 pairs (exact: a code has at most 8
// significant bits, so its f32 value has a zero low half)
__device__ __forceinline__ void u8x4_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const float a = (float)(w & 0xFFu), b = (float)((w >> 8) & 0xFFu);  // v_cvt_f32_ubyte0..3
  const float c = (float)((w >> 16) & 0xFFu), d = (float)(w >> 24);
  lo = (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
  hi = (__float_as_uint(c) >> 16) | (__float_as_uint(d) & 0xFFFF0000u);
}

// f32 -> bf16 by truncation (used only where the value is exact in bf16)
__device__ __forceinline__ uint32_t bf16_trunc(float v) { return __float_as_uint(v) >> 16; }

// two waves per SIMD: the compiler keeps the 128 accumulators and the
// fragments in 216 VGPRs (without the bound: 324 VGPRs and 128 AGPRs, one wave)
__global__ __launch_bounds__(kA8Threads) __attribute__((amdgpu_waves_per_eu(2))) void affine8_gemm_kernel(const uint16_t* __restrict__ x,
                                                                  const uint8_t* __restrict__ codes,
                                                                  const uint16_t* __restrict__ scales,
                                                                  const uint16_t* __restrict__ biases, int T,
                                                                  int K, int N, int n_tiles,
                                                                  uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t As[2][kA8M * 128];
  __shared__ __attribute__((aligned(16))) uint32_t Xs[2][kA8M][2];  // group sums of x as bf16 (x1, x2 | x3, 0)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  const int m0 = mt * kA8M;
  const int n = nt * kA8N + wave * 32 + l32;  // this lane's output row (MFMA column)
  const int nc = n < N ? n : N - 1;
  const uint8_t* crow = codes + (size_t)nc * K + 32 * h;
  // activation pieces of this thread: p = tid + 256 i, row p / 8, piece p % 8
  u32x4 av[4];
  auto load_a = [&](int g) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int p = tid + kA8Threads * i, r = p >> 3, j = p & 7;
      const int t = m0 + r;
      av[i] = t < T ? *reinterpret_cast<const u32x4*>(x + (size_t)t * K + 64 * g + 8 * j) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // the pieces into LDS, and the group sums of the 128 rows (8 threads per
  // row: consecutive lanes) split into three bf16 values
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int p = tid + kA8Threads * i, r = p >> 3, j = p & 7;
      *reinterpret_cast<u32x4*>(&As[buf][r * 128 + 16 * a8_slot(r, j)]) = av[i];
      const uint32_t w[4] = {av[i].x, av[i].y, av[i].z, av[i].w};
      float s = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; q++) s += bf16_to_f32(w[q] & 0xFFFFu) + bf16_to_f32(w[q] >> 16);
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      s += __shfl_xor(s, 4, 64);
      if (j == 0) {
        const float x1 = bf16_to_f32(f32_to_bf16(s));
        const float r1 = s - x1;  // exact
        const float x2 = bf16_to_f32(f32_to_bf16(r1));
        const float x3 = r1 - x2;  // exact, and exact in bf16 (at most 8 significant bits left)
        Xs[buf][r][0] = bf16_trunc(x1) | (bf16_trunc(x2) << 16);
        Xs[buf][r][1] = bf16_trunc(x3);
      }
    }
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

  load_a(0);
  load_b(0, bc, sc, bi);
  store_a(0);
  __syncthreads();
  for (int g = 0; g < G; g++) {
    const int buf = g & 1;
    if (g + 1 < G) {
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
#pragma unroll
    for (int mb = 0; mb < 4; mb++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[mb][e] = fmaf(sc, tmp[mb][e], acc[mb][e]);
    if (g + 1 < G) {
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
        if (t < T) y[(size_t)t * N + n] = f32_to_bf16(acc[mb][e]);
      }
  }
}

hipError_t launch_affine8_gemm(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                               const uint16_t* biases, int T, int K, int N, uint16_t* y, hipStream_t s) {
  const int n_tiles = (N + kA8N - 1) / kA8N, m_tiles = (T + kA8M - 1) / kA8M;
  launch_kernel("affine8_gemm", affine8_gemm_kernel, dim3(n_tiles * m_tiles), dim3(kA8Threads), 0, s, x,
                reinterpret_cast<const uint8_t*>(codes), scales, biases, T, K, N, n_tiles, y);
  return hipGetLastError();
}

}  // namespace moe
