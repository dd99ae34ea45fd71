/* Runs every oracle entry point once on small seeded inputs, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py):
 * any out-of-bounds access, use of freed memory or undefined operation in the
 * oracle aborts the run. The values are not checked here; the pinning tests
 * check them. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
  /* xorshift64*, a small seeded generator for the inputs */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

static uint16_t bf16_of(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static float unit_float(void) { return (float)(next_u32() >> 8) / 16777216.0f - 0.5f; }

int main(void) {
  const int H = 128, I = 64, E = 4, k = 2, T = 3;
  for (unsigned c = 0; c < 16; c++) (void)orc_e2m1_value(c);
  for (unsigned b = 0; b < 256; b++) (void)orc_e4m3_value(b);
  (void)orc_f64_to_bf16(1.0 / 3.0);
  (void)orc_weight(7, 0x38, 2688.0f);

  uint64_t off[9], bytes, stride;
  if (orc_record_layout(H, I, off, &bytes, &stride) != 0) return 1;
  uint8_t* recs[E];
  for (int e = 0; e < E; e++) {
    uint32_t* codes[3];
    uint8_t* scales[3];
    float g[3];
    for (int p = 0; p < 3; p++) {
      size_t n = (size_t)H * I;
      codes[p] = malloc(n / 8 * 4);
      scales[p] = malloc(n / 16);
      for (size_t i = 0; i < n / 8; i++) codes[p][i] = next_u32();
      for (size_t i = 0; i < n / 16; i++) scales[p][i] = (uint8_t)(next_u32() % 0x7F);
      g[p] = 2688.0f * (0.5f + unit_float() + 0.5f);
    }
    recs[e] = malloc(stride);
    orc_pack_record(H, I, (const uint32_t* const*)codes, (const uint8_t* const*)scales, g, recs[e]);
    for (int p = 0; p < 3; p++) {
      free(codes[p]);
      free(scales[p]);
    }
  }
  float* wbuf = malloc(sizeof(float) * H * I);
  uint16_t* ubuf = malloc(sizeof(uint16_t) * H * I);
  for (int p = 0; p < 3; p++) orc_dequant_projection(recs[1], H, I, p, wbuf, ubuf);

  uint16_t* x = malloc(sizeof(uint16_t) * T * H);
  uint16_t* res = malloc(sizeof(uint16_t) * T * H);
  float* Wr = malloc(sizeof(float) * E * H);
  for (int i = 0; i < T * H; i++) {
    x[i] = bf16_of(4.0f * unit_float());
    res[i] = bf16_of(unit_float());
  }
  for (int i = 0; i < E * H; i++) Wr[i] = 0.1f * unit_float();
  float logits[T * E], w[T * k];
  int32_t idx[T * k], offs[E + 1], sorted[T * k];
  orc_router_logits(x, Wr, T, H, E, logits);
  if (orc_route_topk(logits, T, E, k, idx, w) != 0) return 2;
  if (orc_sort_pairs(idx, T * k, E, offs, sorted) != 0) return 3;
  float* yf = malloc(sizeof(float) * T * H);
  uint16_t* yb = malloc(sizeof(uint16_t) * T * H);
  uint16_t* mid = malloc(sizeof(uint16_t) * T * k * I);
  for (int acc = 0; acc < 2; acc++)
    if (orc_moe_forward((const uint8_t* const*)recs, E, H, I, x, T, idx, w, k, res, acc, yf, yb, mid) != 0) return 4;
  int32_t bad[T * k];
  memcpy(bad, idx, sizeof(bad));
  bad[1] = E;
  if (orc_moe_forward((const uint8_t* const*)recs, E, H, I, x, T, bad, w, k, NULL, 0, yf, yb, NULL) != -1) return 5;

  /* 8-dim VQ records */
  uint64_t voff[6], vbytes, vstride;
  if (orc_vq_layout(H, I, voff, &vbytes, &vstride) != 0) return 6;
  uint8_t* book = malloc(4096 * 8);
  for (int i = 0; i < 4096 * 8; i++) book[i] = (uint8_t)(next_u32() % 0x7F);
  uint8_t* vrecs[E];
  for (int e = 0; e < E; e++) {
    uint8_t* vi[3];
    uint16_t* vg[3];
    for (int p = 0; p < 3; p++) {
      int out = p == 2 ? H : I, in = p == 2 ? I : H;
      size_t nb = (size_t)out * in * 3 / 16;
      vi[p] = malloc(nb);
      vg[p] = malloc(sizeof(uint16_t) * out);
      for (size_t i = 0; i < nb; i++) vi[p][i] = (uint8_t)next_u32();
      for (int i = 0; i < out; i++) vg[p][i] = 0x2000 + (uint16_t)(next_u32() % 0x800);
    }
    vrecs[e] = malloc(vstride);
    orc_vq_pack_record(H, I, (const uint8_t* const*)vi, (const uint16_t* const*)vg, vrecs[e]);
    for (int p = 0; p < 3; p++) {
      free(vi[p]);
      free(vg[p]);
    }
  }
  orc_vq_dequant_projection(vrecs[0], book, H, I, 2, wbuf);
  if (orc_vq_moe_forward((const uint8_t* const*)vrecs, book, E, H, I, x, T, idx, w, k, res, 0, yf, yb) != 0) return 7;

  /* residents */
  const int N = 5, K = 128;
  uint16_t* v = malloc(sizeof(uint16_t) * N * K);
  for (int i = 0; i < N * K; i++) v[i] = bf16_of(0.02f * unit_float());
  for (int i = 0; i < 64; i++) v[i] = v[0]; /* one flat group */
  uint32_t* qc = malloc(sizeof(uint32_t) * N * K / 4);
  uint16_t* qs = malloc(sizeof(uint16_t) * N * K / 64);
  uint16_t* qb = malloc(sizeof(uint16_t) * N * K / 64);
  if (orc_q8_quantize(v, N, K, qc, qs, qb) != 0) return 8;
  uint16_t* xa = malloc(sizeof(uint16_t) * T * K);
  for (int i = 0; i < T * K; i++) xa[i] = bf16_of(unit_float());
  float* ya = malloc(sizeof(float) * T * N);
  uint16_t* yab = malloc(sizeof(uint16_t) * T * N);
  if (orc_affine8_linear(xa, qc, qs, qb, T, K, N, ya, yab) != 0) return 9;
  orc_rmsnorm(x, T, H, 1e-6, yb);

  for (int e = 0; e < E; e++) {
    free(recs[e]);
    free(vrecs[e]);
  }
  free(wbuf), free(ubuf), free(x), free(res), free(Wr), free(yf), free(yb), free(mid), free(book);
  free(v), free(qc), free(qs), free(qb), free(xa), free(ya), free(yab);
  printf("oracle driver: ok\n");
  return 0;
}
