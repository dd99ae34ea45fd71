/*
 * moe_mi355x.h -- C ABI of libmoe_mi355x.so: the routed-expert MoE layer over
 * weight-only NVFP4 experts (BF16 activations) on AMD Instinct MI355X (gfx950).
 *
 * Sources, by page title and section:
 *   [PACK] "Beam 1.0 501B-A23B, streaming pack, NVFP4 experts / MLX 8-bit
 *          residents": "What this pack holds" (routed-experts, global-scales,
 *          residents and q8-rule bullets) and the intro (49 routed layers of
 *          256 experts, 8 active per token).
 *   [VQ]   "Beam-1.0-501B-A23B VQ GGUF": "What stays native" (router logits and
 *          SwiGLU in FP32) and "Kernel budget on GB10" (BF16 mids, 5,120 and
 *          2,560 row widths).
 *
 * Conventions (every entry point):
 *   - Returns MOE_OK (0) or a negative MOE_E* code; moe_last_error() then gives
 *     a message (thread-local). No C++ exception crosses this boundary.
 *   - Tensor pointers are caller-owned DEVICE memory unless stated otherwise;
 *     the library keeps no pointer after a call returns.
 *   - Arguments are validated before anything is enqueued: on an error return
 *     nothing has been launched.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*, NULL = the
 *     null stream) and the call returns without waiting. Launch failures are
 *     reported as MOE_EHIP from hipGetLastError at enqueue time.
 *   - bf16 values travel as uint16_t bit patterns; f32 is IEEE binary32.
 *   - Results are deterministic: no floating-point atomics on any path.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_EINVAL (-1)     /* null pointer or value out of range */
#define MOE_ESHAPE (-2)     /* a size breaks a shape rule */
#define MOE_EALIGN (-3)     /* a pointer or offset is not aligned as required */
#define MOE_EWORKSPACE (-4) /* workspace too small */
#define MOE_EHIP (-5)       /* the HIP runtime reported an error */

/* forward flags */
#define MOE_F32_OUT 1u      /* y is f32 [T][H] instead of bf16 */
#define MOE_FORCE_DECODE 2u /* always use the expert-streaming (GEMV) kernels */
#define MOE_FORCE_PREFILL 4u /* always use the grouped-GEMM (MFMA) kernels */

enum { MOE_GATE = 0, MOE_UP = 1, MOE_DOWN = 2 };

/* The status word of a forward / layer workspace: the 32-bit word at byte
 * offset MOE_STATUS_OFFSET. Kernels only ever set its bits; the library never
 * clears them (moe_status_clear does, when the caller asks), so a caller that
 * checks the word clears it before the calls it wants to cover. */
#define MOE_STATUS_OFFSET 8
#define MOE_STATUS_ROUTE_TIMEOUT 1u /* moe_nvfp4_layer, one token: the wait for the router expired */
#define MOE_STATUS_BAD_IDX 2u       /* moe_nvfp4_forward: a pair named an expert outside [0, E) */

/* Message for the last error on the calling thread ("" if none). */
const char* moe_last_error(void);

/* ---- the expert record, [PACK] routed-experts bullet ----------------------
 * One record per expert: gate, up and down, each with E2M1 codes (U32 words,
 * 8 codes per word, element 8q+j in bits 4j..4j+3 of word q), E4M3 block
 * scales (one byte per 16 inputs) and an f32 global g. Gate and up are
 * [I rows][H inputs], down is [H rows][I inputs], row-major. Default part
 * order: gate.codes, gate.scales, up.codes, up.scales, down.codes,
 * down.scales, g_gate, g_up, g_down; records start every `stride` bytes, the
 * record size rounded up to 4 KiB. At H = 5120, I = 2560: 22,118,412 B per
 * record at a 22,122,496 B stride. */
size_t moe_nvfp4_record_bytes(int H, int I);  /* 3*(H*I/2 + H*I/16) + 12; 0 on bad shape */
size_t moe_nvfp4_record_stride(int H, int I); /* record bytes rounded up to 4096 */

typedef struct moe_nvfp4_bank {
  int32_t H, I, E, reserved;
  uint64_t record_bytes, stride;
  /* part_off[2p] codes, part_off[2p+1] scales, part_off[6+p] global of
   * projection p (gate, up, down), bytes from the record start */
  uint64_t part_off[9];
  void* base; /* device, E * stride bytes, 4096-byte aligned */
} moe_nvfp4_bank;

/* Fills *b for E records of shape (H, I) at `base` with the default layout.
 * Shape rules: H, I positive multiples of 16, 1 <= E <= 1024.
 * Errors: MOE_EINVAL (null b/base), MOE_ESHAPE, MOE_EALIGN (base not
 * 4096-aligned). */
int moe_nvfp4_bank_init(moe_nvfp4_bank* b, void* base, int H, int I, int E);

/* S0, pack: copies the 9 parts of each of the b->E experts into their records
 * and zeroes each record's tail pad. Per projection p:
 *   codes[p]  U32 [E][out_p][in_p/8], scales[p] u8 [E][out_p][in_p/16],
 *   g[p]      f32 [E],
 * host or device memory (the runtime picks the copy direction). Host sources
 * must stay valid until the stream reaches the copies. */
int moe_pack_nvfp4_bank(const moe_nvfp4_bank* b, const uint32_t* const codes[3],
                        const uint8_t* const scales[3], const float* const g[3], void* stream);

/* Pack side, [PACK] global-scales bullet: the release gives per projection an
 * f32 weight_scale_2 (ws2); the bank stores g with f32(g / 2688) == ws2. For
 * each of the n values (host arrays): g[i] is the f32 whose f32(g / 2688) is
 * nearest to ws2[i] (equal to it when such a g exists); among several, the
 * one nearest to the exact product ws2[i] * 2688, then the one with an even
 * significand. inexact (nullable) u8 [n]: 1 where no g gives ws2[i] exactly
 * (the manifest's global_scale_inexact list), else 0. Runs on the host, no
 * GPU needed. Errors: MOE_EINVAL for n < 0, null ws2/g (n > 0), or a ws2 that
 * is not a positive f32 whose g = ws2 * 2688 is finite; nothing is written
 * then. */
int moe_nvfp4_global_from_ws2(const float* ws2, int64_t n, float* g, uint8_t* inexact);

/* Manifest digests, [PACK] routed-experts bullet (each record's sha256): the
 * SHA-256 (FIPS 180-4) of records e0 .. e0+n-1 of the bank over their
 * record_bytes bytes (not the pad), computed on the device from the records
 * as they sit in memory. digests: device u8 [n][32], 4-byte aligned. Errors:
 * MOE_EINVAL for a range outside [0, E) or null digests (n > 0), MOE_EALIGN;
 * bank errors as for the pack. Stream-ordered like the other calls. */
int moe_nvfp4_record_sha256(const moe_nvfp4_bank* b, int e0, int n, uint8_t* digests, void* stream);

/* Expert cache: a bounded set of expert records in HBM fed from host memory
 * ([PACK] "What it is for": the selected experts stream into a bounded cache
 * of expert rows on the GPU; "Beam-1.0-501B-A23B, EXL3 3-bit, for 2x RTX PRO
 * 6000 Blackwell", "How it fits": cold experts in pinned host RAM, moved over
 * PCIe on a side stream).
 * moe_cache_create: host_bank describes the full bank in HOST memory (base
 * pinned by the caller, e.g. hipHostMalloc; stride a multiple of 4096; any E
 * >= 1), slot_base is DEVICE memory of nslots * stride bytes (4096-byte
 * aligned, 1 <= nslots <= min(E, 1024)). The cache keeps both pointers until
 * moe_cache_destroy; it creates one copy stream (default priority) and two
 * events. Errors: MOE_EINVAL, MOE_ESHAPE, MOE_EALIGN, MOE_EHIP.
 * moe_cache_prepare: makes experts ids[0..n) (host i32, in [0, E), at most
 * nslots distinct; duplicates allowed) resident and writes their slots into
 * slot_of (host i32 [n]). A resident expert is a hit; a miss takes the least
 * recently used slot that this call does not name (empty slots first, then
 * the lowest slot) and is copied (stride bytes) on the copy stream, which first
 * waits for the work already on `stream`; `stream` then waits for the copies.
 * So a forward enqueued on `stream` after the call, over moe_cache_bank's
 * descriptor with idx mapped through slot_of, reads the right records, and no
 * slot is overwritten while earlier work on `stream` may read it. Calls on one
 * cache must not overlap (the cache has no lock). Errors are returned before
 * any state changes.
 * moe_cache_bank: the slot pool as a bank descriptor (E = nslots) for
 * moe_nvfp4_forward / moe_nvfp4_layer.
 * moe_cache_stats: hits and misses counted per id since creation, and bytes
 * copied (nullable outputs). */
typedef struct moe_expert_cache moe_expert_cache;
int moe_cache_create(const moe_nvfp4_bank* host_bank, void* slot_base, int nslots, moe_expert_cache** out);
int moe_cache_destroy(moe_expert_cache* c);
int moe_cache_prepare(moe_expert_cache* c, const int32_t* ids, int n, int32_t* slot_of, void* stream);
int moe_cache_bank(const moe_expert_cache* c, moe_nvfp4_bank* out);
int moe_cache_stats(const moe_expert_cache* c, int64_t* hits, int64_t* misses, int64_t* bytes_copied);

/* S1 + S2, routing ([PACK] intro: 8 of 256 experts per token; [VQ] "What
 * stays native": FP32 router logits).
 *   If x and w_router are both non-null: logits[t][e] = sum_h x[t][h]*Wr[e][h]
 *   (f32 accumulation) is computed into `logits` first. Otherwise `logits` is
 *   the input. Then per token: the k largest logits (ties: lower expert index;
 *   -0 == +0; a NaN ranks below every number), idx i32 [T][k] in descending
 *   order, and w f32 [T][k] = softmax over the k selected logits (f32, summed
 *   in slot order).
 *   x bf16 [T][H] (8-byte aligned); w_router f32 [E][H], one row per expert
 *   (16-byte aligned; the routers stay F32 as released, [PACK] residents
 *   bullet); logits f32 [T][E].
 *   Rules: T >= 0, 1 <= k <= min(E, 64), 1 <= E <= 1024, H % 16 == 0. */
int moe_route_topk(const uint16_t* x, const float* w_router, float* logits, int T, int H,
                   int E, int k, int32_t* idx, float* w, void* stream);

/* S3, token -> expert counting sort of the P = T*k pairs (pair p = t*k + j):
 * offsets i32 [E+1] (offsets[e] = first sorted slot of expert e, offsets[E] = P)
 * and sorted i32 [P] (pair ids, ascending within one expert: a stable sort).
 * idx values outside [0, E) are a caller error; they are dropped and
 * offsets[E] then counts only the valid pairs. */
int moe_sort_pairs(const int32_t* idx, int T, int k, int E, int32_t* offsets, int32_t* sorted,
                   void* stream);

/* The same sort with a caller scratch buffer, the form moe_nvfp4_forward uses
 * internally: above 2048 pairs it runs on many workgroups (per-chunk counts,
 * a scan, per-chunk placement) instead of one. Same results as
 * moe_sort_pairs, bit for bit. workspace: device, 4-byte aligned, at least
 * moe_sort_workspace_bytes(T, k, E) bytes (0 on bad arguments), not shared
 * with a concurrent call. */
size_t moe_sort_workspace_bytes(int T, int k, int E);
int moe_sort_pairs_ws(const int32_t* idx, int T, int k, int E, int32_t* offsets, int32_t* sorted,
                      void* workspace, size_t workspace_bytes, void* stream);

/* S3..S7, the layer (shape rules: H and I multiples of 64, T >= 0,
 * 1 <= k <= min(E, 64); a bank accepts multiples of 16, but every layer
 * kernel walks a weight row in 64-input quads of four E4M3 blocks, 32 bytes
 * of codes and 4 scale bytes per load, so a row that ends inside a quad is
 * rejected with MOE_ESHAPE rather than read past its end):
 *   y[t] = residual[t] + sum_j w[t][j] * down_e( bf16( silu(gate_e x[t]) * up_e x[t] ) )
 * with e = idx[t][j], each projection dequantized by the [PACK] global-scales
 * rule (weight = e2m1 * f32(e4m3 * f32(g / 2688))), f32 accumulation, FP32
 * SwiGLU and BF16 mids ([VQ]). x, residual (nullable): bf16 [T][H]; idx i32
 * [T][k]; w f32 [T][k]; y bf16 [T][H], or f32 with MOE_F32_OUT. Alignment:
 * x and y 16 bytes, residual 8 bytes, idx and w 4 bytes (else MOE_EALIGN).
 * Expert-streaming (GEMV) kernels are used for small T*k, grouped-GEMM (bf16
 * MFMA) kernels for large T*k; flags can force either.
 * workspace: device, >= moe_nvfp4_workspace_bytes(T, k, H, I, E) bytes,
 * 256-byte aligned, not shared with a concurrent call. idx values outside
 * [0, E) are a caller error: those pairs contribute nothing, and the kernels
 * set MOE_STATUS_BAD_IDX in the workspace's status word (the call itself
 * returns MOE_OK: the values are only seen on the device). Prefills of more
 * than 2 GiB of activations (T * H * 2 bytes) run as several passes over
 * token chunks, with the same results. */
size_t moe_nvfp4_workspace_bytes(int T, int k, int H, int I, int E);
int moe_nvfp4_forward(const moe_nvfp4_bank* b, const uint16_t* x, int T, const int32_t* idx,
                      const float* w, int k, const uint16_t* residual, void* y, unsigned flags,
                      void* workspace, size_t workspace_bytes, void* stream);

/* moe_nvfp4_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, rules and results as moe_nvfp4_forward, without
 * the workspace: the scratch is a library-owned static device array of
 * MOE_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, held from the library's first
 * use on that GPU until the process ends. A call whose
 * moe_nvfp4_workspace_bytes(T, k, H, I, E) exceeds it returns MOE_EWORKSPACE
 * before anything is enqueued (at H = 5120, I = 2560, k = 8: up to 163
 * tokens). The call allocates nothing. All calls on one GPU share its array
 * and each leaves its contents behind: calls that can overlap on one GPU (on
 * different streams, or from several threads) race and must not be made.
 * status (nullable): device u32 word into which the kernels OR the
 * MOE_STATUS_* bits (4-byte aligned; the caller clears it). */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_nvfp4_forward_noalloc(const moe_nvfp4_bank* b, const uint16_t* x, int T, const int32_t* idx,
                              const float* w, int k, const uint16_t* residual, void* y, unsigned flags,
                              uint32_t* status, void* stream);

/* S1..S7 in one call: the router, the top-k with its softmax and the layer,
 * i.e. moe_route_topk(x, w_router, logits, ...) followed by
 * moe_nvfp4_forward(..., idx, w, ...), with the same results: logits f32
 * [T][E], idx i32 [T][k] and w f32 [T][k] are written as moe_route_topk
 * writes them, y as moe_nvfp4_forward writes it. Arguments, flags, alignment
 * and workspace as for those two calls (w_router f32 [E][H], 16-byte
 * aligned; logits 4-byte aligned; E <= 1024).
 * For one token (T = 1, k <= 16, k*I*2 <= 65536 bytes of mids, no
 * MOE_FORCE_PREFILL) the router and the top-k run inside the gate/up launch
 * (two launches in all): the router logits pass through the workspace as
 * 64-bit tags stamped with a per-call number, so the workspace needs no
 * clearing between calls, must not be shared by calls that can overlap, and
 * a region never written by this library matches a call number with
 * probability 2^-32 per tag. The wait for the tags is bounded (about 0.1 s);
 * if it ever expires (it does not in a correct launch), MOE_STATUS_ROUTE_TIMEOUT
 * is set in the workspace's status word, idx holds -1, w holds 0 and y holds
 * the residual (or 0): the call's routing is lost and it returns MOE_OK,
 * so a caller that must know checks the status word. (The environment
 * variable MOE_DEBUG_ROUTE_GIVEUP=1 forces this path, for tests.) Otherwise
 * the call runs the router, top-k and forward launches in order. */
int moe_nvfp4_layer(const moe_nvfp4_bank* b, const uint16_t* x, const float* w_router, int T, int k,
                    const uint16_t* residual, float* logits, int32_t* idx, float* w, void* y,
                    unsigned flags, void* workspace, size_t workspace_bytes, void* stream);

/* The status word of `workspace` (256-byte aligned): moe_status_read waits for
 * `stream` and copies the word into *status (host); moe_status_clear enqueues
 * a store of 0 on `stream` (a kernel, not a memset, so it may be captured in
 * a graph). Errors: MOE_EINVAL (null), MOE_EALIGN, MOE_EHIP. */
int moe_status_read(const void* workspace, uint32_t* status, void* stream);
int moe_status_clear(void* workspace, void* stream);

/* S8, resident linear in MLX affine 8-bit, group 64 ([PACK] residents and
 * q8-rule bullets): y[t][n] = sum_k x[t][k] * (scale[n][k/64]*q[n][k] +
 * bias[n][k/64]), f32 accumulation, bf16 out.
 * x bf16 [T][K]; codes U32 [N][K/4] (4 codes per word, first in the low
 * byte); scales, biases bf16 [N][K/64]; y bf16 [T][N].
 * Rules: K % 64 == 0, N >= 1, T >= 0; codes 16-byte aligned, x 4-byte
 * aligned (MOE_EALIGN otherwise). From 33 tokens (env
 * MOE_AFFINE8_GEMM_MIN_T) with x 16-byte aligned the call runs as a tiled
 * MFMA GEMM, below that as a bandwidth-bound pass that reads the weights
 * once per 16 tokens; both accumulate in f32. When the GEMM's 128 x 128
 * tiles number fewer than the device's CUs (a few hundred tokens), K is
 * split into ranges of whole 64 x 8 blocks whose f32 partial outputs are
 * added in range order: the call then takes S * T * N * 4 bytes of scratch
 * (at most 32 MiB on a 256-CU device: S times the tiles stays within two
 * workgroups per CU)
 * from a stream-ordered memory pool the library keeps per device
 * (hipMallocFromPoolAsync / hipFreeAsync on `stream`, so calls on different
 * streams do not share it; the pool keeps its memory for reuse until the
 * process ends), and without it runs unsplit. Errors: MOE_ESHAPE, MOE_EINVAL (null), MOE_EALIGN, MOE_EHIP. */
int affine8_g64_linear(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                       const uint16_t* biases, int T, int K, int N, uint16_t* y, void* stream);

/* S9, weightless RMS norm used between stacked layers:
 * y = bf16( x / sqrt(mean(x^2) + eps) ), f32 math. x, y bf16 [T][H]. */
int moe_rmsnorm(const uint16_t* x, int T, int H, float eps, uint16_t* y, void* stream);

/* Test export of the dequant rule ([PACK] global-scales bullet) for one
 * projection of one record: out_f32 [out][in] (nullable) = e2m1 * f32(e4m3 *
 * f32(g/2688)); out_unit (nullable) bf16 [out][in] = e2m1 * e4m3, exact. */
int moe_nvfp4_dequant(const moe_nvfp4_bank* b, int expert, int proj, float* out_f32,
                      uint16_t* out_unit, void* stream);

/* ---- 8-dim VQ experts, a second record format for the same layer ----------
 * "Beam-1.0-501B-A23B VQ GGUF", "Recipe", routed-experts bullet: every 8
 * consecutive weights of an expert row are one 12-bit index into a codebook
 * of 4,096 codewords of 8 E4M3 bytes (one codebook per layer, shared by all
 * experts and by gate/up/down), times one F16 gain per row: weight =
 * gain * e4m3(codeword[index][i]), exact in f32. Index j of a row is bits
 * 12j..12j+11 of the row's little-endian bit stream (8 indices in 12 bytes).
 * Record: gate.idx [I][H*3/16] bytes, gate.gain f16 [I], up.idx, up.gain,
 * down.idx [H][I*3/16], down.gain [H], each part on 16 bytes; records every
 * `stride` bytes (record size rounded up to 4 KiB). At H = 5120, I = 2560:
 * 7,393,280 B per record, 1.5 bits per weight. H and I multiples of 64. */
size_t moe_vq_record_bytes(int H, int I);  /* 0 on bad shape */
size_t moe_vq_record_stride(int H, int I);

typedef struct moe_vq_bank {
  int32_t H, I, E, reserved;
  uint64_t record_bytes, stride;
  uint64_t part_off[6]; /* part_off[2p] index rows, part_off[2p+1] gains of projection p */
  void* base;           /* device, E * stride bytes, 4096-byte aligned */
  const void* codebook; /* device, 4096 * 8 bytes (E4M3), 16-byte aligned */
} moe_vq_bank;

/* Fills *b with the default layout. Errors: MOE_EINVAL (null), MOE_ESHAPE
 * (H, I not positive multiples of 64; E outside [1, 1024]), MOE_EALIGN. */
int moe_vq_bank_init(moe_vq_bank* b, void* base, const void* codebook, int H, int I, int E);
/* Copies each expert's parts into its record and zeroes the pad:
 * idx[p] bytes [E][out_p][in_p*3/16], gain[p] f16 bits [E][out_p], host or
 * device memory (host sources must stay valid until the stream reaches the
 * copies). */
int moe_vq_pack_bank(const moe_vq_bank* b, const uint8_t* const idx[3], const uint16_t* const gain[3],
                     void* stream);
/* Test export: f32 [out][in] weights of one projection of one record, through
 * the kernels' own conversion path. */
int moe_vq_dequant(const moe_vq_bank* b, int expert, int proj, float* out_f32, void* stream);
/* The layer of moe_nvfp4_forward over VQ records (same arguments, flags
 * MOE_F32_OUT only; expert-streaming kernels for any T, k <= 16, and
 * 32 KiB + k*I*2 bytes of codebook and mids must fit the LDS). workspace:
 * device, 256-byte aligned, >= moe_vq_workspace_bytes(T, k, H, I) (0 on bad
 * arguments). idx values outside [0, E) contribute nothing. */
size_t moe_vq_workspace_bytes(int T, int k, int H, int I);
int moe_vq_forward(const moe_vq_bank* b, const uint16_t* x, int T, const int32_t* idx, const float* w, int k,
                   const uint16_t* residual, void* y, unsigned flags, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Achievable-peak probes, the measured denominators beside the data-sheet
 * peaks of the rooflines (measurement only; no step of the layer uses them).
 * moe_probe_hbm_read: reads nbytes (a multiple of 16) at buf (device,
 * 16-byte aligned) once, with `blocks` workgroups of 256 threads in
 * grid-stride order, 16-byte loads, 4 (variant 0, 2) or 8 (1, 3) in flight per
 * thread, nontemporal in variants 2 and 3. moe_probe_mfma_bf16: `blocks`
 * workgroups of 4 waves, each wave 4 independent chains of `iters`
 * v_mfma_f32_32x32x16_bf16 (32,768 flop each) on register operands. sink:
 * device, `blocks` words, which the probes do not write for real data (they
 * only keep the compiler from dropping the work). Errors: MOE_EINVAL,
 * MOE_EALIGN, MOE_EHIP. */
int moe_probe_hbm_read(const void* buf, size_t nbytes, int variant, int blocks, uint32_t* sink, void* stream);
int moe_probe_mfma_bf16(int blocks, int iters, float* sink, void* stream);

/* Kernel timing with HIP events that hipExtLaunchKernel records at each
 * kernel's own start and end on its stream. moe_profile_enable(1) clears and
 * starts collection; moe_profile_read(name, ...) synchronizes the events and
 * returns the summed duration and count of the kernel family `name` since the
 * last enable. Names: "router", "topk", "sort", "decode_gateup", "decode_down",
 * "combine", "prefill_gateup", "prefill_down", "affine8", "rmsnorm", "sha256",
 * "vq_gateup", "vq_down", "vq_dequant", "probe_hbm_read", "probe_mfma". */
int moe_profile_enable(int on);
int moe_profile_read(const char* name, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif
