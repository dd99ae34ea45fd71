/*
 * CPU oracle for the routed-expert MoE layer over weight-only NVFP4 experts.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link or
 * call this code: only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark use it. It shares no code, header, table or constant with
 * the HIP library.
 *
 * It is a plain, slow, obviously-correct statement of what the layer computes.
 * Sources, cited by page title and section (the pages are the text of public web
 * pages about serving Reflection's Beam-1.0-501B-A23B):
 *   [PACK]  "Beam 1.0 501B-A23B, streaming pack, NVFP4 experts / MLX 8-bit
 *           residents", section "What this pack holds" (bullets: routed experts,
 *           global scales, residents, q8 rule) and its intro paragraph.
 *   [VQ]    "Beam-1.0-501B-A23B VQ GGUF", sections "What stays native" (FP32
 *           router logits and SwiGLU) and "Kernel budget on GB10" (BF16 mids,
 *           H = 5,120, I = 2,560).
 * Readings of what the pages leave open are listed beside each function.
 *
 * Precision: every accumulation is in double (f64). Values are rounded to f32
 * or bf16 exactly where the pages fix that precision: router logits (f32),
 * the SwiGLU inputs (f32), the mid values (bf16), the dequantized weight
 * (f32, by the pack's block-scale rule). An f32-accumulating mode (ORC_ACC_F32)
 * reproduces plain float loops in index order, for comparison.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_ACC_F64 = 0, ORC_ACC_F32 = 1 };
enum { ORC_GATE = 0, ORC_UP = 1, ORC_DOWN = 2 };

/* ---- number formats --------------------------------------------------- */
/* E2M1 value of a 4-bit code (sign, 2 exponent bits with bias 1, 1 mantissa
 * bit); [PACK] routed-experts bullet names E2M1 codes. */
double orc_e2m1_value(unsigned code);
/* E4M3 value of a byte, OCP "FN" variant (bias 7, max 448, no infinities,
 * 0x7F/0xFF are NaN). The variant is fixed by the divisor 2688 = 448 * 6 in
 * [PACK] global-scales bullet (max E4M3 times max E2M1). */
double orc_e4m3_value(unsigned byte);
/* bf16 <-> f32/f64; rounding is to nearest, ties to even. */
float orc_bf16_to_f32(uint16_t b);
uint16_t orc_f64_to_bf16(double v);

/* ---- dequantization, [PACK] global-scales bullet ---------------------- */
/* t = f32(g / 2688), IEEE f32 division */
float orc_global_factor(float g);
/* S = f32(e4m3(s) * t) */
float orc_block_scale(unsigned s_byte, float g);
/* w = f32(e2m1(c) * S): the dequantized weight */
float orc_weight(unsigned code, unsigned s_byte, float g);

/* ---- record layout, [PACK] routed-experts bullet ----------------------- */
/* One expert record holds gate, up and down, each with E2M1 codes (U32 words,
 * 8 codes per word), E4M3 block scales (one per 16 inputs) and an f32 global.
 * Reading: gate and up are [I rows][H inputs], down is [H rows][I inputs]
 * (row-major, blocks run along inputs); parts are laid out
 * gate.codes, gate.scales, up.codes, up.scales, down.codes, down.scales,
 * g_gate, g_up, g_down; records start on 4 KiB boundaries.
 * part_off[2p] = codes of projection p, part_off[2p+1] = its scales,
 * part_off[6+p] = its f32 global. Returns 0, or -1 on a bad shape. */
int orc_record_layout(int H, int I, uint64_t part_off[9], uint64_t* record_bytes,
                      uint64_t* stride);
/* Writes one record (stride bytes, zero padded) from its 9 parts.
 * codes[p]: U32 [out_p][in_p/8]; scales[p]: bytes [out_p][in_p/16]. */
void orc_pack_record(int H, int I, const uint32_t* const codes[3],
                     const uint8_t* const scales[3], const float g[3], uint8_t* dst);
/* Dense dequantized matrix of projection `proj` of a record, [out][in]:
 * w_out gets the f32 weight; unit_out (nullable) gets bf16(e2m1 * e4m3), which
 * is exact in bf16. */
void orc_dequant_projection(const uint8_t* record, int H, int I, int proj,
                            float* w_out, uint16_t* unit_out);

/* ---- 8-dim VQ experts, [VQ] "Recipe" routed-experts bullet ------------------
 * Every 8 consecutive weights of an expert row are one index into a codebook
 * of 8-dim E4M3 codewords (one book per layer, shared by all experts and by
 * gate/up/down), times one F16 gain per row. 12-bit indices: 4,096 codewords
 * of 8 bytes, 32 KiB (the [VQ] kernel budget leaves 27 KiB of 99 KiB beside
 * 40 KiB of mids at 12 bits). Readings: index j of a row is bits 12j..12j+11 of
 * the row's little-endian bit stream; codeword c is bytes 8c..8c+7, element i
 * at byte 8c+i; a record holds gate.idx, gate.gain, up.idx, up.gain,
 * down.idx, down.gain, each part starting on 16 bytes, records on 4 KiB; the
 * weight is gain * e4m3(codeword element), exact in f32. */
double orc_f16_value(uint16_t h);
unsigned orc_vq_index(const uint8_t* row, uint64_t j);
/* part_off[2p] = index rows of projection p, part_off[2p+1] = its gains;
 * H and I multiples of 64; returns 0 or -1 */
int orc_vq_layout(int H, int I, uint64_t part_off[6], uint64_t* record_bytes, uint64_t* stride);
/* idx[p]: packed index rows [out_p][in_p * 3 / 16] bytes; gain[p]: f16 bits [out_p] */
void orc_vq_pack_record(int H, int I, const uint8_t* const idx[3], const uint16_t* const gain[3],
                        uint8_t* dst);
void orc_vq_dequant_projection(const uint8_t* record, const uint8_t* codebook, int H, int I, int proj,
                               float* w_out);
/* the layer of orc_moe_forward over VQ records (codebook: 4096 x 8 bytes) */
int orc_vq_moe_forward(const uint8_t* const* records, const uint8_t* codebook, int E, int H, int I,
                       const uint16_t* x, int T, const int32_t* idx, const float* w, int k,
                       const uint16_t* residual, int acc, float* y_f32, uint16_t* y_bf16);

/* ---- routing ------------------------------------------------------------ */
/* logits[t][e] = f32( sum_h x[t][h] * Wr[e][h] ), sum in f64; [VQ] "What stays
 * native" keeps router logits in FP32. x bf16 [T][H], Wr f32 [E][H] (one row
 * per expert, the layout of a Linear layer's weight; [PACK] residents bullet
 * keeps the routers in F32 as released). */
void orc_router_logits(const uint16_t* x, const float* Wr, int T, int H, int E,
                       float* logits);
/* Per token: the k largest logits (ties: lower expert index first; -0 == +0),
 * idx[t][j] in that order, and softmax over the k selected logits,
 * w = f32(exp(l_j - l_0) / sum), evaluated in f64. Returns -1 on a NaN logit
 * or a bad k, else 0. */
int orc_route_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w);
/* Stable counting sort of the P = T*k (token, slot) pairs by expert:
 * offsets[e] = first sorted slot of expert e (offsets[E] = P), sorted[s] = pair
 * id p = t*k + j, pairs of one expert in increasing p. Returns -1 if an
 * index is out of [0, E). */
int orc_sort_pairs(const int32_t* idx, int P, int E, int32_t* offsets, int32_t* sorted);

/* ---- the layer ---------------------------------------------------------- */
/* y[t] = residual[t] + sum_j w[t][j] * down_e( bf16( silu(gate_e x) * up_e x ) )
 * with e = idx[t][j]. records[e] points at expert e's record (may be NULL for
 * experts no token uses). x, residual (nullable): bf16 [T][H].
 * Outputs: y_f32 [T][H] and y_bf16 [T][H] (either nullable), mid_bf16 [T*k][I]
 * in pair order (nullable). acc: ORC_ACC_F64 or ORC_ACC_F32. Returns -1 on a
 * bad argument. */
int orc_moe_forward(const uint8_t* const* records, int E, int H, int I,
                    const uint16_t* x, int T, const int32_t* idx, const float* w, int k,
                    const uint16_t* residual, int acc, float* y_f32, uint16_t* y_bf16,
                    uint16_t* mid_bf16);

/* ---- residents, [PACK] residents bullet and q8-rule bullet ------------- */
/* Quantizes v bf16 [N][K] (K % 64 == 0) group-wise along K: per group of 64,
 * bias = min, scale = the smallest bf16 b with 255*b >= max - min, code = the
 * nearest step (exact ties to even). Codes packed 4 per U32, first code in the
 * low byte: codes U32 [N][K/4]; scales, biases bf16 [N][K/64].
 * A group with max == min gets scale +0 and all codes 0. Returns -1 on a bad
 * shape. */
int orc_q8_quantize(const uint16_t* v, int N, int K, uint32_t* codes, uint16_t* scales,
                    uint16_t* biases);
/* y[t][n] = sum_k x[t][k] * (scale[n][k/64] * q[n][k] + bias[n][k/64]), f64,
 * outputs f32 and/or bf16 (nullable). */
int orc_affine8_linear(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                       const uint16_t* biases, int T, int K, int N, float* y_f32,
                       uint16_t* y_bf16);
/* Weightless RMS norm, y = bf16( x / sqrt(mean(x^2) + eps) ), f64. */
void orc_rmsnorm(const uint16_t* x, int T, int H, double eps, uint16_t* y);

#ifdef __cplusplus
}
#endif
#endif
