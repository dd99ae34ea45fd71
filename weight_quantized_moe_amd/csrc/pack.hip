// Pack-side helpers of the expert bank: the f32 global g recovered from the
// release's per-projection weight_scale_2, and the SHA-256 of each record for
// the bank's manifest.
//
// "Beam 1.0 501B-A23B, streaming pack, NVFP4 experts / MLX 8-bit residents",
// "What this pack holds": the block scale is e4m3(scale) * (g / 2688) in f32,
// and the pack stores, per projection, the g whose f32(g / 2688) equals the
// release's weight_scale_2; where none does it stores the nearest g, about one
// f32 ulp away, and the manifest lists those projections. The same bullet list
// gives the manifest: format and layout names, the 9 parts of a record, and
// each record's offset, length and sha256.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>

#include "common.h"
#include "internal.h"

namespace moe {

// ---- g from weight_scale_2 (host) ------------------------------------------------
// g -> f32(g / 2688) is monotone, and every g with f32(g / 2688) == ws2 lies
// within 0.66 ulp(g) of the exact product ws2 * 2688 (ulp(g) is 2^11 or 2^12
// times ulp(ws2) and 2688 / 2^12 < 2688 / 2^11 < 2 * 0.66), so the candidates
// are the f32 values next to that product. Among them: the smallest
// |f32(g / 2688) - ws2| (zero when an exact g exists), then the smallest
// |g - ws2 * 2688|, then an even significand.
bool global_from_ws2_one(float ws2, float* g_out) {
  const double target = (double)ws2 * 2688.0;  // exact: 24 + 12 significant bits
  const float g0 = (float)target;               // round to nearest even
  float c[5];
  c[2] = g0;
  c[1] = nextafterf(g0, 0.0f);
  c[0] = nextafterf(c[1], 0.0f);
  c[3] = nextafterf(g0, INFINITY);
  c[4] = nextafterf(c[3], INFINITY);
  float best = 0.0f;
  double best_err = INFINITY, best_dist = INFINITY;
  bool have = false;
  for (float g : c) {
    if (!(g > 0.0f) || !std::isfinite(g)) continue;
    const volatile float img = g / 2688.0f;  // IEEE f32 division
    const double err = std::fabs((double)img - (double)ws2);
    const double dist = std::fabs((double)g - target);
    uint32_t bits;
    std::memcpy(&bits, &g, 4);
    bool take = !have || err < best_err || (err == best_err && dist < best_dist);
    if (have && err == best_err && dist == best_dist) take = (bits & 1u) == 0;
    if (take) {
      best = g;
      best_err = err;
      best_dist = dist;
      have = true;
    }
  }
  *g_out = best;
  return best_err == 0.0;
}

// ---- SHA-256 of records (device) -------------------------------------------------
// FIPS 180-4. The 64 round constants and the initial hash value are the first
// 32 bits of the fractional parts of the cube roots of the first 64 primes and
// of the square roots of the first 8 primes; the host computes them from that
// definition.
struct Sha256Consts {
  uint32_t k[64];
  uint32_t h0[8];
};

static uint32_t frac32(long double v) {
  const long double f = v - floorl(v);
  return (uint32_t)floorl(f * 4294967296.0L);
}

Sha256Consts sha256_consts() {
  Sha256Consts c;
  int n = 0;
  for (int p = 2; n < 64; p++) {
    bool prime = true;
    for (int d = 2; d * d <= p; d++)
      if (p % d == 0) {
        prime = false;
        break;
      }
    if (!prime) continue;
    if (n < 8) c.h0[n] = frac32(sqrtl((long double)p));
    c.k[n] = frac32(cbrtl((long double)p));
    n++;
  }
  return c;
}

__device__ __forceinline__ uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

// one 64-byte block (big-endian words w[0..15]) into the state h
__device__ __forceinline__ void sha256_block(uint32_t (&h)[8], const uint32_t (&m)[16], const Sha256Consts& c) {
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 16; i++) w[i] = m[i];
  uint32_t a = h[0], b = h[1], cc = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
#pragma unroll
  for (int t = 0; t < 64; t++) {
    uint32_t wt;
    if (t < 16) {
      wt = w[t];
    } else {
      const uint32_t w15 = w[(t - 15) & 15], w2 = w[(t - 2) & 15];
      const uint32_t s0 = rotr(w15, 7) ^ rotr(w15, 18) ^ (w15 >> 3);
      const uint32_t s1 = rotr(w2, 17) ^ rotr(w2, 19) ^ (w2 >> 10);
      wt = w[t & 15] + s0 + w[(t - 7) & 15] + s1;
      w[t & 15] = wt;
    }
    const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
    const uint32_t ch = (e & f) ^ (~e & g);
    const uint32_t t1 = hh + S1 + ch + c.k[t] + wt;
    const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
    const uint32_t maj = (a & b) ^ (a & cc) ^ (b & cc);
    const uint32_t t2 = S0 + maj;
    hh = g;
    g = f;
    f = e;
    e = d + t1;
    d = cc;
    cc = b;
    b = a;
    a = t1 + t2;
  }
  h[0] += a;
  h[1] += b;
  h[2] += cc;
  h[3] += d;
  h[4] += e;
  h[5] += f;
  h[6] += g;
  h[7] += hh;
}

__device__ __forceinline__ void load_block(const uint8_t* p, uint32_t (&m)[16]) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const u32x4 v = q[i];
    m[4 * i + 0] = __builtin_bswap32(v.x);
    m[4 * i + 1] = __builtin_bswap32(v.y);
    m[4 * i + 2] = __builtin_bswap32(v.z);
    m[4 * i + 3] = __builtin_bswap32(v.w);
  }
}

// Lane i hashes record e0 + i (i < n): its nbytes bytes from the record start
// (16-byte aligned). The message is processed one 64-byte block at a time, the
// next block's loads issued before the current block's rounds; the tail and
// the padding (0x80, zeros, the 64-bit big-endian bit length) form the last
// one or two blocks. out: [n][32] bytes, the digests (4-byte aligned).
__global__ __launch_bounds__(64) void record_sha256_kernel(const uint8_t* __restrict__ base, uint64_t stride,
                                                           uint64_t nbytes, int e0, int n, Sha256Consts c,
                                                           uint8_t* __restrict__ out) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= n) return;
  const uint8_t* rec = base + (uint64_t)(e0 + i) * stride;
  uint32_t h[8];
#pragma unroll
  for (int j = 0; j < 8; j++) h[j] = c.h0[j];
  const uint64_t nfull = nbytes / 64;
  uint32_t cur[16], nxt[16];
  if (nfull > 0) load_block(rec, cur);
  for (uint64_t b = 0; b < nfull; b++) {
    if (b + 1 < nfull) load_block(rec + (b + 1) * 64, nxt);
    sha256_block(h, cur, c);
#pragma unroll
    for (int j = 0; j < 16; j++) cur[j] = nxt[j];
  }
  // tail + padding: one block when the tail leaves room for the 0x80 byte
  // and the length (tail <= 55), else two
  const uint32_t tail = (uint32_t)(nbytes % 64);
  const uint8_t* tp = rec + nfull * 64;
  const uint64_t bits = nbytes * 8;
  const int nlast = tail <= 55 ? 1 : 2;
  for (int blk = 0; blk < nlast; blk++) {
    uint32_t m[16];
#pragma unroll
    for (int j = 0; j < 16; j++) {
      uint32_t wv = 0;
#pragma unroll
      for (int bb = 0; bb < 4; bb++) {
        const uint32_t pos = (uint32_t)blk * 64 + 4 * j + bb;  // byte position after the full blocks
        uint32_t byte = 0;
        if (pos < tail)
          byte = tp[pos];
        else if (pos == tail)
          byte = 0x80;
        else if (pos >= (uint32_t)nlast * 64 - 8)
          byte = (uint32_t)(bits >> (8 * ((uint32_t)nlast * 64 - 1 - pos))) & 0xFF;
        wv = (wv << 8) | byte;
      }
      m[j] = wv;
    }
    sha256_block(h, m, c);
  }
#pragma unroll
  for (int j = 0; j < 8; j++) reinterpret_cast<uint32_t*>(out + (size_t)i * 32)[j] = __builtin_bswap32(h[j]);
}

hipError_t launch_record_sha256(const uint8_t* base, uint64_t stride, uint64_t nbytes, int e0, int n,
                                uint8_t* digests, hipStream_t s) {
  static const Sha256Consts c = sha256_consts();
  launch_kernel("sha256", record_sha256_kernel, dim3((n + 63) / 64), dim3(64), 0, s, base, stride, nbytes, e0, n, c,
                digests);
  return hipGetLastError();
}

}  // namespace moe
