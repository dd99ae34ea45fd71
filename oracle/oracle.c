/*
 * CPU oracle for the NVFP4 MoE layer. TEST INFRASTRUCTURE ONLY: see oracle.h
 * for the sources and the readings. Build: gcc -O2 -fopenmp -ffp-contract=off
 * (no fast-math), so every float operation rounds as written.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* number formats                                                            */
/* ------------------------------------------------------------------------ */

double orc_e2m1_value(unsigned code) {
  /* 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit. Exponent field 0 is
   * the subnormal range: m * 2^(1-1) * 2^-1. */
  unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
  double v = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
  return s ? -v : v;
}

double orc_e4m3_value(unsigned byte) {
  /* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; the FN variant has
   * no infinities and uses all-ones exponent and mantissa for NaN only. */
  unsigned s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9); /* m/8 * 2^(1-7) */
  else
    v = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return s ? -v : v;
}

float orc_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

uint16_t orc_f64_to_bf16(double v) {
  /* Round the exact value v to the bf16 grid, nearest with ties to even:
   * find the grid spacing q at v's binade, round v/q to an integer with
   * rint() (ties to even in the default rounding mode), scale back. The
   * result is a bf16 value, so it converts to f32 exactly. */
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  int ex;
  frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
  int E = ex - 1;
  if (E < -126) E = -126; /* subnormal range: fixed spacing 2^-133 */
  double q = ldexp(1.0, E - 7);
  double r = rint(a / q) * q;
  if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80); /* rounds past max */
  float f = (float)r;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | (u >> 16));
}

/* ------------------------------------------------------------------------ */
/* dequantization                                                            */
/* ------------------------------------------------------------------------ */

float orc_global_factor(float g) {
  float d = 2688.0f;
  return g / d; /* IEEE f32 division, round to nearest even */
}

float orc_block_scale(unsigned s_byte, float g) {
  float s = (float)orc_e4m3_value(s_byte); /* exact in f32 */
  float t = orc_global_factor(g);
  return s * t; /* one f32 rounding */
}

float orc_weight(unsigned code, unsigned s_byte, float g) {
  float c = (float)orc_e2m1_value(code); /* exact in f32 */
  float S = orc_block_scale(s_byte, g);
  return c * S; /* one f32 rounding */
}

/* ------------------------------------------------------------------------ */
/* record layout                                                             */
/* ------------------------------------------------------------------------ */

static void proj_shape(int H, int I, int p, int* out, int* in) {
  if (p == ORC_DOWN) {
    *out = H;
    *in = I;
  } else {
    *out = I;
    *in = H;
  }
}

int orc_record_layout(int H, int I, uint64_t part_off[9], uint64_t* record_bytes,
                      uint64_t* stride) {
  if (H <= 0 || I <= 0 || H % 16 || I % 16) return -1;
  uint64_t n = (uint64_t)H * (uint64_t)I; /* weights per projection */
  uint64_t codes = n / 2;                 /* 4 bits per weight */
  uint64_t scales = n / 16;               /* 1 byte per 16 weights */
  uint64_t off = 0;
  for (int p = 0; p < 3; p++) {
    part_off[2 * p] = off;
    off += codes;
    part_off[2 * p + 1] = off;
    off += scales;
  }
  for (int p = 0; p < 3; p++) {
    part_off[6 + p] = off;
    off += 4;
  }
  *record_bytes = off;
  *stride = (off + 4095) / 4096 * 4096;
  return 0;
}

void orc_pack_record(int H, int I, const uint32_t* const codes[3],
                     const uint8_t* const scales[3], const float g[3], uint8_t* dst) {
  uint64_t off[9], bytes, stride;
  orc_record_layout(H, I, off, &bytes, &stride);
  memset(dst, 0, stride);
  uint64_t n = (uint64_t)H * (uint64_t)I;
  for (int p = 0; p < 3; p++) {
    /* U32 words stored little-endian, so the word's low nibble comes first */
    for (uint64_t wi = 0; wi < n / 8; wi++) {
      uint32_t v = codes[p][wi];
      uint8_t* q = dst + off[2 * p] + 4 * wi;
      q[0] = (uint8_t)(v & 0xFF);
      q[1] = (uint8_t)((v >> 8) & 0xFF);
      q[2] = (uint8_t)((v >> 16) & 0xFF);
      q[3] = (uint8_t)((v >> 24) & 0xFF);
    }
    memcpy(dst + off[2 * p + 1], scales[p], n / 16);
    memcpy(dst + off[6 + p], &g[p], 4);
  }
}

/* code of element `e` of a row whose words start at byte pointer `w`:
 * element 8*q + j is nibble j (bits 4j..4j+3) of little-endian word q */
static unsigned code_at(const uint8_t* row_codes, uint64_t e) {
  uint8_t b = row_codes[e / 2];
  return (e & 1) ? (b >> 4) : (b & 15u);
}

void orc_dequant_projection(const uint8_t* record, int H, int I, int proj, float* w_out,
                            uint16_t* unit_out) {
  uint64_t off[9], bytes, stride;
  orc_record_layout(H, I, off, &bytes, &stride);
  int out, in;
  proj_shape(H, I, proj, &out, &in);
  const uint8_t* codes = record + off[2 * proj];
  const uint8_t* scales = record + off[2 * proj + 1];
  float g;
  memcpy(&g, record + off[6 + proj], 4);
#pragma omp parallel for schedule(static)
  for (int r = 0; r < out; r++) {
    const uint8_t* rc = codes + (uint64_t)r * (uint64_t)(in / 2);
    const uint8_t* rs = scales + (uint64_t)r * (uint64_t)(in / 16);
    for (int b = 0; b < in / 16; b++) {
      unsigned sb = rs[b];
      float S = orc_block_scale(sb, g); /* one block scale per 16 inputs */
      double s_exact = orc_e4m3_value(sb);
      for (int c = 16 * b; c < 16 * b + 16; c++) {
        unsigned code = code_at(rc, (uint64_t)c);
        uint64_t o = (uint64_t)r * (uint64_t)in + (uint64_t)c;
        if (w_out) w_out[o] = (float)orc_e2m1_value(code) * S;
        if (unit_out) unit_out[o] = orc_f64_to_bf16(orc_e2m1_value(code) * s_exact);
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* routing                                                                   */
/* ------------------------------------------------------------------------ */

void orc_router_logits(const uint16_t* x, const float* Wr, int T, int H, int E,
                       float* logits) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int t = 0; t < T; t++)
    for (int e = 0; e < E; e++) {
      double acc = 0.0;
      for (int h = 0; h < H; h++)
        acc += (double)orc_bf16_to_f32(x[(size_t)t * H + h]) * (double)Wr[(size_t)e * H + h];
      logits[(size_t)t * E + e] = (float)acc;
    }
}

typedef struct {
  float l;
  int e;
} cand_t;

static int cand_cmp(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a;
  const cand_t* y = (const cand_t*)b;
  if (x->l > y->l) return -1; /* larger logit first */
  if (x->l < y->l) return 1;
  return (x->e < y->e) ? -1 : (x->e > y->e); /* equal (incl. -0 == +0): lower index */
}

int orc_route_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w) {
  if (k < 1 || k > E) return -1;
  cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)E);
  if (!c) return -1;
  for (int t = 0; t < T; t++) {
    for (int e = 0; e < E; e++) {
      c[e].l = logits[(size_t)t * E + e];
      c[e].e = e;
      if (isnan(c[e].l)) {
        free(c);
        return -1;
      }
    }
    qsort(c, (size_t)E, sizeof(cand_t), cand_cmp);
    double m = (double)c[0].l, sum = 0.0;
    for (int j = 0; j < k; j++) sum += exp((double)c[j].l - m);
    for (int j = 0; j < k; j++) {
      idx[(size_t)t * k + j] = c[j].e;
      w[(size_t)t * k + j] = (float)(exp((double)c[j].l - m) / sum);
    }
  }
  free(c);
  return 0;
}

int orc_sort_pairs(const int32_t* idx, int P, int E, int32_t* offsets, int32_t* sorted) {
  for (int p = 0; p < P; p++)
    if (idx[p] < 0 || idx[p] >= E) return -1;
  int32_t* cursor = (int32_t*)calloc((size_t)E + 1, sizeof(int32_t));
  if (!cursor) return -1;
  for (int p = 0; p < P; p++) cursor[idx[p] + 1]++; /* counts */
  for (int e = 0; e < E; e++) cursor[e + 1] += cursor[e]; /* exclusive scan */
  for (int e = 0; e <= E; e++) offsets[e] = cursor[e];
  for (int p = 0; p < P; p++) sorted[cursor[idx[p]]++] = p; /* stable placement */
  free(cursor);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* the layer                                                                 */
/* ------------------------------------------------------------------------ */

/* y = A x for a dense f32 matrix A [rows][cols] and a vector of f32 values xv,
 * one entry per row; accumulation in f64 (or f32 in index order). */
static void matvec(const float* A, int rows, int cols, const float* xv, int acc, double* y) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; r++) {
    const float* a = A + (size_t)r * cols;
    if (acc == ORC_ACC_F32) {
      float s = 0.0f;
      for (int c = 0; c < cols; c++) s = s + xv[c] * a[c];
      y[r] = (double)s;
    } else {
      double s = 0.0;
      for (int c = 0; c < cols; c++) s += (double)xv[c] * (double)a[c];
      y[r] = s;
    }
  }
}

/* The layer over any expert format: deq(ctx, e, proj, W) writes expert e's
 * dense f32 matrix of projection proj ([out][in]). */
typedef void (*orc_deq_fn)(const void* ctx, int e, int H, int I, int proj, float* W);

static int moe_forward_core(const uint8_t* const* records, orc_deq_fn deq, const void* ctx, int E, int H,
                            int I, const uint16_t* x, int T, const int32_t* idx, const float* w, int k,
                            const uint16_t* residual, int acc, float* y_f32, uint16_t* y_bf16,
                            uint16_t* mid_bf16) {
  if (H <= 0 || I <= 0 || H % 16 || I % 16 || T < 0 || k < 1 || k > E) return -1;
  size_t P = (size_t)T * (size_t)k;
  for (size_t p = 0; p < P; p++)
    if (idx[p] < 0 || idx[p] >= E || records[idx[p]] == NULL) return -1;
  size_t nw = (size_t)H * (size_t)I;
  float* Wg = (float*)malloc(nw * sizeof(float));
  float* Wu = (float*)malloc(nw * sizeof(float));
  float* Wd = (float*)malloc(nw * sizeof(float));
  float* xv = (float*)malloc((size_t)H * sizeof(float));
  float* mv = (float*)malloc((size_t)I * sizeof(float));
  double* gv = (double*)malloc((size_t)I * sizeof(double));
  double* uv = (double*)malloc((size_t)I * sizeof(double));
  double* d_all = (double*)malloc((P ? P : 1) * (size_t)H * sizeof(double));
  int rc = 0;
  if (!Wg || !Wu || !Wd || !xv || !mv || !gv || !uv || !d_all) {
    rc = -1;
    goto done;
  }
  /* Each pair (t, j) is computed on its own; experts are visited in index
   * order so that each used expert is dequantized once per call. */
  for (int e = 0; e < E; e++) {
    int used = 0;
    for (size_t p = 0; p < P && !used; p++) used = (idx[p] == e);
    if (!used) continue;
    deq(ctx, e, H, I, ORC_GATE, Wg);
    deq(ctx, e, H, I, ORC_UP, Wu);
    deq(ctx, e, H, I, ORC_DOWN, Wd);
    for (size_t p = 0; p < P; p++) {
      if (idx[p] != e) continue;
      size_t t = p / (size_t)k;
      for (int h = 0; h < H; h++) xv[h] = orc_bf16_to_f32(x[t * (size_t)H + h]);
      matvec(Wg, I, H, xv, acc, gv);
      matvec(Wu, I, H, xv, acc, uv);
      for (int i = 0; i < I; i++) {
        /* SwiGLU on the f32 gate and up values ([VQ] keeps SwiGLU in FP32),
         * rounded to a bf16 mid ([VQ] kernel budget: BF16 mid values). */
        float gi = (float)gv[i], ui = (float)uv[i];
        uint16_t mb;
        if (acc == ORC_ACC_F32) {
          float silu = gi / (1.0f + expf(-gi));
          mb = orc_f64_to_bf16((double)(silu * ui));
        } else {
          double silu = (double)gi / (1.0 + exp(-(double)gi));
          mb = orc_f64_to_bf16(silu * (double)ui);
        }
        mv[i] = orc_bf16_to_f32(mb);
        if (mid_bf16) mid_bf16[p * (size_t)I + i] = mb;
      }
      matvec(Wd, H, I, mv, acc, d_all + p * (size_t)H);
    }
  }
  /* combine: residual plus the weighted expert outputs, slot j ascending */
  for (int t = 0; t < T; t++)
    for (int h = 0; h < H; h++) {
      size_t o = (size_t)t * H + h;
      double r = residual ? (double)orc_bf16_to_f32(residual[o]) : 0.0;
      double v;
      if (acc == ORC_ACC_F32) {
        float s = (float)r;
        for (int j = 0; j < k; j++) {
          size_t p = (size_t)t * k + j;
          s = s + w[p] * (float)d_all[p * (size_t)H + h];
        }
        v = (double)s;
      } else {
        double s = r;
        for (int j = 0; j < k; j++) {
          size_t p = (size_t)t * k + j;
          s += (double)w[p] * d_all[p * (size_t)H + h];
        }
        v = s;
      }
      if (y_f32) y_f32[o] = (float)v;
      if (y_bf16) y_bf16[o] = orc_f64_to_bf16(v);
    }
done:
  free(Wg);
  free(Wu);
  free(Wd);
  free(xv);
  free(mv);
  free(gv);
  free(uv);
  free(d_all);
  return rc;
}

static void nvfp4_deq(const void* ctx, int e, int H, int I, int proj, float* W) {
  const uint8_t* const* records = (const uint8_t* const*)ctx;
  orc_dequant_projection(records[e], H, I, proj, W, NULL);
}

int orc_moe_forward(const uint8_t* const* records, int E, int H, int I, const uint16_t* x,
                    int T, const int32_t* idx, const float* w, int k,
                    const uint16_t* residual, int acc, float* y_f32, uint16_t* y_bf16,
                    uint16_t* mid_bf16) {
  return moe_forward_core(records, nvfp4_deq, records, E, H, I, x, T, idx, w, k, residual, acc, y_f32,
                          y_bf16, mid_bf16);
}

/* ------------------------------------------------------------------------ */
/* 8-dim VQ experts ([VQ] "Recipe", routed-experts bullet)                   */
/* ------------------------------------------------------------------------ */

double orc_f16_value(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-14 / 1024 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp(1.0 + (double)m / 1024.0, e - 15);
  return s ? -v : v;
}

unsigned orc_vq_index(const uint8_t* row, uint64_t j) {
  /* bits 12j .. 12j+11 of the row's little-endian bit stream */
  uint64_t bit = 12 * j;
  unsigned lo = row[bit / 8], hi = row[bit / 8 + 1];
  return ((lo | (hi << 8)) >> (bit % 8)) & 0xFFFu;
}

static uint64_t up16(uint64_t n) { return (n + 15) / 16 * 16; }

int orc_vq_layout(int H, int I, uint64_t part_off[6], uint64_t* record_bytes, uint64_t* stride) {
  if (H <= 0 || I <= 0 || H % 64 || I % 64) return -1;
  uint64_t off = 0;
  for (int p = 0; p < 3; p++) {
    int out, in;
    proj_shape(H, I, p, &out, &in);
    part_off[2 * p] = off;
    off = up16(off + (uint64_t)out * ((uint64_t)in / 8 * 12 / 8)); /* 12 bits per 8 weights */
    part_off[2 * p + 1] = off;
    off = up16(off + (uint64_t)out * 2); /* one f16 gain per row */
  }
  *record_bytes = off;
  *stride = (off + 4095) / 4096 * 4096;
  return 0;
}

void orc_vq_pack_record(int H, int I, const uint8_t* const idx[3], const uint16_t* const gain[3],
                        uint8_t* dst) {
  uint64_t off[6], bytes, stride;
  orc_vq_layout(H, I, off, &bytes, &stride);
  memset(dst, 0, stride);
  for (int p = 0; p < 3; p++) {
    int out, in;
    proj_shape(H, I, p, &out, &in);
    memcpy(dst + off[2 * p], idx[p], (uint64_t)out * ((uint64_t)in / 8 * 12 / 8));
    for (int r = 0; r < out; r++) {
      dst[off[2 * p + 1] + 2 * (uint64_t)r] = (uint8_t)(gain[p][r] & 0xFF);
      dst[off[2 * p + 1] + 2 * (uint64_t)r + 1] = (uint8_t)(gain[p][r] >> 8);
    }
  }
}

void orc_vq_dequant_projection(const uint8_t* record, const uint8_t* codebook, int H, int I, int proj,
                               float* w_out) {
  uint64_t off[6], bytes, stride;
  orc_vq_layout(H, I, off, &bytes, &stride);
  int out, in;
  proj_shape(H, I, proj, &out, &in);
  const uint64_t row_bytes = (uint64_t)in / 8 * 12 / 8;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < out; r++) {
    const uint8_t* row = record + off[2 * proj] + (uint64_t)r * row_bytes;
    uint16_t gb = (uint16_t)(record[off[2 * proj + 1] + 2 * (uint64_t)r] |
                             (record[off[2 * proj + 1] + 2 * (uint64_t)r + 1] << 8));
    double gain = orc_f16_value(gb);
    for (int j = 0; j < in / 8; j++) {
      unsigned c = orc_vq_index(row, (uint64_t)j);
      for (int i = 0; i < 8; i++) /* exact: 11 x 4 significant bits */
        w_out[(uint64_t)r * in + 8 * j + i] = (float)(gain * orc_e4m3_value(codebook[8 * c + i]));
    }
  }
}

typedef struct {
  const uint8_t* const* records;
  const uint8_t* codebook;
} vq_ctx;

static void vq_deq(const void* ctx, int e, int H, int I, int proj, float* W) {
  const vq_ctx* c = (const vq_ctx*)ctx;
  orc_vq_dequant_projection(c->records[e], c->codebook, H, I, proj, W);
}

int orc_vq_moe_forward(const uint8_t* const* records, const uint8_t* codebook, int E, int H, int I,
                       const uint16_t* x, int T, const int32_t* idx, const float* w, int k,
                       const uint16_t* residual, int acc, float* y_f32, uint16_t* y_bf16) {
  vq_ctx c = {records, codebook};
  if (H % 64 || I % 64) return -1;
  return moe_forward_core(records, vq_deq, &c, E, H, I, x, T, idx, w, k, residual, acc, y_f32, y_bf16, NULL);
}

/* ------------------------------------------------------------------------ */
/* residents                                                                 */
/* ------------------------------------------------------------------------ */

/* the bf16 value that follows b on the grid (b finite, >= 0) */
static uint16_t bf16_next_up(uint16_t b) { return (uint16_t)(b + 1); }

int orc_q8_quantize(const uint16_t* v, int N, int K, uint32_t* codes, uint16_t* scales,
                    uint16_t* biases) {
  if (N <= 0 || K <= 0 || K % 64) return -1;
  int G = K / 64;
  for (int n = 0; n < N; n++)
    for (int gi = 0; gi < G; gi++) {
      const uint16_t* grp = v + (size_t)n * K + (size_t)gi * 64;
      double mn = INFINITY, mx = -INFINITY;
      uint16_t mn_bits = 0;
      for (int i = 0; i < 64; i++) {
        double a = (double)orc_bf16_to_f32(grp[i]);
        if (a < mn) {
          mn = a;
          mn_bits = grp[i];
        }
        if (a > mx) mx = a;
      }
      double d = mx - mn; /* exact: both are bf16 values */
      /* smallest bf16 b >= 0 with 255 * b >= d (255*b is exact in f64):
       * start from the bf16 truncation of d/255 and walk up the grid */
      uint16_t sb = 0;
      if (d > 0.0) {
        float c = (float)(d / 255.0);
        uint32_t cu;
        memcpy(&cu, &c, 4);
        sb = (uint16_t)(cu >> 16);
        if (sb > 0) sb = (uint16_t)(sb - 1); /* margin below the candidate */
        while (255.0 * (double)orc_bf16_to_f32(sb) < d) sb = bf16_next_up(sb);
      }
      double s = (double)orc_bf16_to_f32(sb);
      /* a negative zero minimum is still the group minimum; keep its bits */
      biases[(size_t)n * G + gi] = mn_bits;
      scales[(size_t)n * G + gi] = sb;
      for (int i = 0; i < 64; i++) {
        double r = (double)orc_bf16_to_f32(grp[i]) - mn; /* exact, >= 0 */
        unsigned q = 0;
        if (s > 0.0) {
          /* nearest integer to r / s with exact ties to even: compare 2r with
           * (2q + 1) s, all exact in f64 */
          q = (unsigned)floor(r / s);
          while ((double)q * s > r) q--;
          while ((double)(q + 1) * s <= r) q++;
          double twice = 2.0 * r, mid = (double)(2 * q + 1) * s;
          if (twice > mid || (twice == mid && (q & 1u))) q++;
        }
        size_t e = (size_t)n * K + (size_t)gi * 64 + (size_t)i;
        uint32_t* wd = &codes[e / 4];
        if (e % 4 == 0) *wd = 0;
        *wd |= (uint32_t)(q & 0xFFu) << (8 * (e % 4));
      }
    }
  return 0;
}

int orc_affine8_linear(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                       const uint16_t* biases, int T, int K, int N, float* y_f32,
                       uint16_t* y_bf16) {
  if (T < 0 || N <= 0 || K <= 0 || K % 64) return -1;
  int G = K / 64;
#pragma omp parallel for collapse(2) schedule(static)
  for (int t = 0; t < T; t++)
    for (int n = 0; n < N; n++) {
      double acc = 0.0;
      for (int kk = 0; kk < K; kk++) {
        size_t e = (size_t)n * K + (size_t)kk;
        unsigned q = (codes[e / 4] >> (8 * (e % 4))) & 0xFFu;
        double s = (double)orc_bf16_to_f32(scales[(size_t)n * G + kk / 64]);
        double b = (double)orc_bf16_to_f32(biases[(size_t)n * G + kk / 64]);
        double wv = s * (double)q + b; /* exact in f64 */
        acc += (double)orc_bf16_to_f32(x[(size_t)t * K + kk]) * wv;
      }
      if (y_f32) y_f32[(size_t)t * N + n] = (float)acc;
      if (y_bf16) y_bf16[(size_t)t * N + n] = orc_f64_to_bf16(acc);
    }
  return 0;
}

void orc_rmsnorm(const uint16_t* x, int T, int H, double eps, uint16_t* y) {
  for (int t = 0; t < T; t++) {
    double ss = 0.0;
    for (int h = 0; h < H; h++) {
      double a = (double)orc_bf16_to_f32(x[(size_t)t * H + h]);
      ss += a * a;
    }
    double inv = 1.0 / sqrt(ss / (double)H + eps);
    for (int h = 0; h < H; h++)
      y[(size_t)t * H + h] = orc_f64_to_bf16((double)orc_bf16_to_f32(x[(size_t)t * H + h]) * inv);
  }
}
