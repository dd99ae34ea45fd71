// Internal launch interface of libmoe_mi355x.so (not part of the C ABI).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

struct moe_nvfp4_bank;
struct moe_expert_cache;

namespace moe {

// Where one bank's parts live: byte offsets inside every record.
struct BankView {
  const uint8_t* base;
  uint64_t stride;
  uint64_t codes[3], scales[3], g[3];
  int H, I, E;
};

// Bits of the forward's status word (a 32-bit word in the workspace): the
// one-token layer's bounded wait for the router expired; a pair named an
// expert outside [0, E). Kernels only set bits; the library never clears them.
constexpr uint32_t kStatusRouteTimeout = 1u;
constexpr uint32_t kStatusBadIdx = 2u;

// Routing tables written by the pair sort into the forward's workspace.
struct RouteTables {
  int32_t* offsets;     // [E+1] first sorted slot of each expert
  int32_t* sorted;      // [P] pair ids, grouped by expert, stable
  int32_t* active;      // [E] experts with at least one pair, ascending
  int32_t* counts;      // [0] n_active, [1] n_tiles
  int32_t* tile_expert; // [max_tiles] grouped-GEMM tiles: expert
  int32_t* tile_row0;   // [max_tiles] first sorted slot of the tile
  int32_t* hist;        // [sort_hist_ints(P, E)] scratch of the multi-workgroup sort, or null
  uint32_t* status;     // status word (kStatusBadIdx set for a pair outside [0, E)), or null
};

// router: logits = x . Wr^T with Wr f32 [E][H]; one block per (expert, 8 tokens)
constexpr int kRouterTok = 8;
hipError_t launch_router(const uint16_t* x, const float* Wr, float* logits, int T, int H, int E,
                         hipStream_t s);
// top-k + softmax over given logits, one wave per token
hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                       hipStream_t s);
// stable counting sort of the T*k pairs; also the active list and, when
// mtile > 0, the grouped-GEMM tile table (tiles of mtile sorted slots). With
// rt.hist set and more than 2048 pairs it runs as three multi-workgroup
// launches (same order).
int sort_hist_ints(int P, int E);
hipError_t launch_sort(const int32_t* idx, int P, int E, RouteTables rt, int mtile, int max_tiles,
                       hipStream_t s);

// pack side: g with f32(g / 2688) == ws2 if one exists, else the nearest
// (returns whether it is exact); SHA-256 of records e0 .. e0 + n - 1 over
// their first nbytes bytes, digests [n][32] (device, 4-byte aligned)
bool global_from_ws2_one(float ws2, float* g);
// 8-dim VQ records (vq.hip): byte offsets of each projection's index rows and
// gains inside a record; the codebook is 4096 x 8 E4M3 bytes
struct VqArgs {
  const uint8_t* bank;
  uint64_t stride;
  uint64_t idx_off[3], gain_off[3];
  const uint8_t* codebook;
  int H, I, E, k, T;
  const int32_t* idx;       // [T][k]
  const float* w;           // [T][k]
  const uint16_t* x;        // [T][H]
  const uint16_t* residual; // [T][H] or null
  uint16_t* mid;            // [T*k][I] scratch
  void* y;                  // [T][H] bf16 or f32
  int f32_out;
};
hipError_t launch_vq_forward(const VqArgs& a, hipStream_t s);
hipError_t launch_vq_dequant(const VqArgs& a, int expert, int proj, float* out, hipStream_t s);
// the expert cache's host logic and copies (arguments checked by the caller;
// prepare's ids are in [0, E) with at most nslots distinct)
int cache_create(const moe_nvfp4_bank* host, void* slot_base, int nslots, moe_expert_cache** out);
void cache_destroy(moe_expert_cache* c);
int cache_prepare(moe_expert_cache* c, const int32_t* ids, int n, int32_t* slot_of, hipStream_t stream, char* err,
                  size_t errlen);
int cache_view(const moe_expert_cache* c, moe_nvfp4_bank* out);
int cache_experts(const moe_expert_cache* c);
void cache_stats(const moe_expert_cache* c, int64_t* hits, int64_t* misses, int64_t* bytes);
hipError_t launch_record_sha256(const uint8_t* base, uint64_t stride, uint64_t nbytes, int e0, int n,
                                uint8_t* digests, hipStream_t s);

// expert-streaming (GEMV) kernels. rt == nullptr: each block finds its
// expert (the slot-th smallest present in idx) and that expert's pairs itself,
// which needs P <= kDecInblockMaxP; else the sorted tables are used. mid and part
// are indexed by pair id. max_m: the expected largest pair count of one
// expert, a hint only (1 picks the single-token kernels, which still loop
// over any number of pairs).
constexpr int kDecInblockMaxP = 256;
hipError_t launch_decode_gateup(const BankView& b, const uint16_t* x, const int32_t* idx, int P, int k,
                                const RouteTables* rt, int slots, int max_m, uint16_t* mid,
                                uint32_t* status, hipStream_t s);
hipError_t launch_decode_down(const BankView& b, const uint16_t* mid, const float* w,
                              const int32_t* idx, int P, int k, const RouteTables* rt, int slots,
                              int max_m, float* part, hipStream_t s);
// up to kFlatDecodeMaxT tokens (k <= kFlatDecodeMaxK, k * I * 2 <= 64 KiB of
// mids in LDS, I % 16 == 0): gate/up then down with the combine folded in;
// mid [T*k][I] is scratch, y [T][H] the layer output
constexpr int kFlatDecodeMaxK = 16;
// tokens the one-item-per-wave decode kernels take by default: they stream
// every pair's record at about 6 TB/s, the routed GEMV reads each distinct
// record once; on skewed routing the two cross between 8 and 10 tokens
// (226-228 against 226-253 us at 8, 278 against 271 us at 10, 328 against
// 311 us at 12, 381 against 351 us at 14)
constexpr int kFlatDecodeMaxT = 9;
hipError_t launch_flat_decode(const BankView& b, const uint16_t* x, int T, const int32_t* idx,
                              const float* w, int k, const uint16_t* residual, uint16_t* mid,
                              void* y, bool f32_out, uint32_t* status, hipStream_t s);
// router + top-k + gate/up in one launch, then down (T = 1, the same limits
// as launch_flat_decode, E <= 1024): logits [E], idx [k] and w [k] are
// written; tags [E] and status live in the workspace; call is this call's
// number (tags carrying it are this call's logits); tags spans 1024 router
// tags followed by kFlatDecodeMaxK routing-record words
hipError_t launch_flat_layer(const BankView& b, const uint16_t* x, const float* wr, int k,
                             const uint16_t* residual, float* logits, int32_t* idx, float* w,
                             uint16_t* mid, uint64_t* tags, uint32_t* status, uint32_t call, void* y,
                             bool f32_out, hipStream_t s, bool debug_giveup = false);
// y[t] = residual[t] + sum_j part[t*k+j] (j ascending); pairs with idx
// outside [0, E) contribute nothing
hipError_t launch_combine(const float* part, const int32_t* idx, int E, int T, int H, int k,
                          const uint16_t* residual, void* y, bool f32_out, hipStream_t s);

// grouped-GEMM (bf16 MFMA) kernels
constexpr int kPrefillMTile = 128;
hipError_t launch_prefill_gateup(const BankView& b, const uint16_t* x, int k, const RouteTables& rt,
                                 int max_tiles, uint16_t* mid, hipStream_t s);
hipError_t launch_prefill_down(const BankView& b, const uint16_t* mid, const float* w, int k,
                               const RouteTables& rt, int max_tiles, float* part, hipStream_t s);

// misc
hipError_t launch_store_u32(uint32_t* p, uint32_t v, hipStream_t s);
hipError_t launch_zero_tails(uint8_t* base, uint64_t stride, uint64_t record_bytes, int E,
                             hipStream_t s);
hipError_t launch_dequant(const BankView& b, int expert, int proj, float* out_f32,
                          uint16_t* out_unit, hipStream_t s);
hipError_t launch_rmsnorm(const uint16_t* x, int T, int H, float eps, uint16_t* y, hipStream_t s);
hipError_t launch_affine8(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                          const uint16_t* biases, int T, int K, int N, uint16_t* y, hipStream_t s);
// the same linear on bf16 MFMA for many tokens (x 16-byte aligned)
hipError_t launch_affine8_gemm(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                               const uint16_t* biases, int T, int K, int N, uint16_t* y, hipStream_t s);

// achievable-peak probes (peak.hip): a streaming read of nbytes (a multiple of
// 16, 16-byte aligned) in one of 4 load variants, and a bf16 MFMA loop of
// blocks x 4 waves x iters x 4 instructions; sink: device scratch of `blocks`
// words that a real run never writes
hipError_t launch_probe_hbm_read(const void* buf, uint64_t nbytes, int variant, int blocks, uint32_t* sink,
                                 hipStream_t s);
hipError_t launch_probe_mfma(int blocks, int iters, float* sink, hipStream_t s);

// kernel timing (api.hip)
// Kernel timing (moe_profile_enable). When on, prof_events hands out a pair
// of events for one launch of kernel `name`; launch_kernel passes them to
// hipExtLaunchKernel, which records them at the kernel's own start and end.
bool prof_events(const char* name, hipEvent_t* start, hipEvent_t* stop);

template <typename F, typename... Args>
inline void launch_kernel(const char* name, F kernel, dim3 grid, dim3 block, uint32_t shm, hipStream_t s,
                          Args... args) {
  hipEvent_t e0, e1;
  if (prof_events(name, &e0, &e1))
    hipExtLaunchKernelGGL(kernel, grid, block, shm, s, e0, e1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shm, s, args...);
}

}  // namespace moe
