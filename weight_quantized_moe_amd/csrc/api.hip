// C ABI of libmoe_mi355x.so: argument validation, workspace layout, dispatch
// and kernel timing. Every check happens before the first enqueue, so an
// error return means nothing was launched. See include/moe_mi355x.h.
#include <hip/hip_runtime.h>

#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe_mi355x.h"
#include "internal.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t up256(size_t n) { return (n + 255) / 256 * 256; }

// ---- kernel timing -------------------------------------------------------------
struct ProfEntry {
  hipEvent_t start, end;
};
struct Profiler {
  std::mutex mu;
  bool on = false;
  std::map<std::string, std::vector<ProfEntry>> done;
  void clear() {
    for (auto& kv : done)
      for (auto& pe : kv.second) {
        hipEventDestroy(pe.start);
        hipEventDestroy(pe.end);
      }
    done.clear();
  }
};
Profiler& prof() {
  static Profiler p;
  return p;
}

}  // namespace

namespace moe {

bool prof_events(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  if (!p.on) return false;
  if (hipEventCreate(start) != hipSuccess) return false;
  if (hipEventCreate(stop) != hipSuccess) {
    hipEventDestroy(*start);
    return false;
  }
  p.done[name].push_back({*start, *stop});
  return true;
}

}  // namespace moe

using namespace moe;

// ---- sizes and the bank descriptor ---------------------------------------------
static bool record_shape_ok(int H, int I) { return H > 0 && I > 0 && H % 16 == 0 && I % 16 == 0; }

MOE_API const char* moe_last_error(void) { return g_err; }

MOE_API size_t moe_nvfp4_record_bytes(int H, int I) {
  if (!record_shape_ok(H, I)) return 0;
  const size_t n = (size_t)H * (size_t)I;
  return 3 * (n / 2 + n / 16) + 12;
}

MOE_API size_t moe_nvfp4_record_stride(int H, int I) {
  const size_t b = moe_nvfp4_record_bytes(H, I);
  return (b + 4095) / 4096 * 4096;
}

MOE_API int moe_nvfp4_bank_init(moe_nvfp4_bank* b, void* base, int H, int I, int E) {
  if (!b || !base) return fail(MOE_EINVAL, "bank_init: null pointer");
  if (!record_shape_ok(H, I)) return fail(MOE_ESHAPE, "bank_init: H=%d I=%d must be positive multiples of 16", H, I);
  if (E < 1 || E > 1024) return fail(MOE_ESHAPE, "bank_init: E=%d outside [1, 1024]", E);
  if (!aligned(base, 4096)) return fail(MOE_EALIGN, "bank_init: base not 4096-byte aligned");
  std::memset(b, 0, sizeof(*b));
  b->H = H;
  b->I = I;
  b->E = E;
  const uint64_t n = (uint64_t)H * (uint64_t)I;
  uint64_t off = 0;
  for (int p = 0; p < 3; p++) {
    b->part_off[2 * p] = off;
    off += n / 2;
    b->part_off[2 * p + 1] = off;
    off += n / 16;
  }
  for (int p = 0; p < 3; p++) {
    b->part_off[6 + p] = off;
    off += 4;
  }
  b->record_bytes = off;
  b->stride = (off + 4095) / 4096 * 4096;
  b->base = base;
  return MOE_OK;
}

// Checks a descriptor and turns it into the kernels' view.
static int bank_view(const moe_nvfp4_bank* b, BankView* v, const char* who) {
  if (!b || !b->base) return fail(MOE_EINVAL, "%s: null bank", who);
  if (!record_shape_ok(b->H, b->I) || b->E < 1 || b->E > 1024)
    return fail(MOE_ESHAPE, "%s: bank shape H=%d I=%d E=%d", who, b->H, b->I, b->E);
  if (b->stride < b->record_bytes || b->record_bytes != moe_nvfp4_record_bytes(b->H, b->I))
    return fail(MOE_EINVAL, "%s: record size/stride inconsistent with H, I", who);
  if (!aligned(b->base, 256) || b->stride % 256) return fail(MOE_EALIGN, "%s: base/stride alignment", who);
  const uint64_t n = (uint64_t)b->H * (uint64_t)b->I;
  for (int p = 0; p < 3; p++) {
    if (b->part_off[2 * p] % 16 || b->part_off[2 * p + 1] % 16 || b->part_off[6 + p] % 4)
      return fail(MOE_EALIGN, "%s: part offsets of projection %d not aligned (16 B codes/scales, 4 B g)", who, p);
    if (b->part_off[2 * p] + n / 2 > b->record_bytes || b->part_off[2 * p + 1] + n / 16 > b->record_bytes ||
        b->part_off[6 + p] + 4 > b->record_bytes)
      return fail(MOE_EINVAL, "%s: part of projection %d outside the record", who, p);
  }
  v->base = static_cast<const uint8_t*>(b->base);
  v->stride = b->stride;
  for (int p = 0; p < 3; p++) {
    v->codes[p] = b->part_off[2 * p];
    v->scales[p] = b->part_off[2 * p + 1];
    v->g[p] = b->part_off[6 + p];
  }
  v->H = b->H;
  v->I = b->I;
  v->E = b->E;
  return MOE_OK;
}

// ---- S0 pack -------------------------------------------------------------------
MOE_API int moe_pack_nvfp4_bank(const moe_nvfp4_bank* b, const uint32_t* const codes[3],
                                const uint8_t* const scales[3], const float* const g[3],
                                void* stream) {
  BankView v;
  int rc = bank_view(b, &v, "pack");
  if (rc) return rc;
  if (!codes || !scales || !g) return fail(MOE_EINVAL, "pack: null part arrays");
  for (int p = 0; p < 3; p++)
    if (!codes[p] || !scales[p] || !g[p]) return fail(MOE_EINVAL, "pack: null part of projection %d", p);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t n = (size_t)b->H * (size_t)b->I;
  uint8_t* base = static_cast<uint8_t*>(b->base);
  for (int e = 0; e < b->E; e++) {
    uint8_t* rec = base + (size_t)e * b->stride;
    for (int p = 0; p < 3; p++) {
      rc = hip_check(hipMemcpyAsync(rec + b->part_off[2 * p], reinterpret_cast<const uint8_t*>(codes[p]) + e * (n / 2),
                                    n / 2, hipMemcpyDefault, s), "pack codes");
      if (rc) return rc;
      rc = hip_check(hipMemcpyAsync(rec + b->part_off[2 * p + 1], scales[p] + e * (n / 16), n / 16,
                                    hipMemcpyDefault, s), "pack scales");
      if (rc) return rc;
      rc = hip_check(hipMemcpyAsync(rec + b->part_off[6 + p], g[p] + e, 4, hipMemcpyDefault, s), "pack g");
      if (rc) return rc;
    }
  }
  return hip_check(launch_zero_tails(base, b->stride, b->record_bytes, b->E, s), "pack zero pad");
}

// ---- pack side: global scales and record digests --------------------------------
MOE_API int moe_nvfp4_global_from_ws2(const float* ws2, int64_t n, float* g, uint8_t* inexact) {
  if (n < 0) return fail(MOE_EINVAL, "global_from_ws2: n=%lld < 0", (long long)n);
  if (n > 0 && (!ws2 || !g)) return fail(MOE_EINVAL, "global_from_ws2: null ws2/g");
  for (int64_t i = 0; i < n; i++)
    if (!(ws2[i] > 0.0f) || !((double)ws2[i] * 2688.0 <= 3.4028234663852886e38))
      return fail(MOE_EINVAL, "global_from_ws2: ws2[%lld] = %g is not a positive f32 with a finite g",
                  (long long)i, (double)ws2[i]);
  for (int64_t i = 0; i < n; i++) {
    const bool exact = global_from_ws2_one(ws2[i], &g[i]);
    if (inexact) inexact[i] = exact ? 0 : 1;
  }
  return MOE_OK;
}

MOE_API int moe_nvfp4_record_sha256(const moe_nvfp4_bank* b, int e0, int n, uint8_t* digests, void* stream) {
  BankView v;
  int rc = bank_view(b, &v, "record_sha256");
  if (rc) return rc;
  if (e0 < 0 || n < 0 || (int64_t)e0 + n > b->E)
    return fail(MOE_EINVAL, "record_sha256: records [%d, %d) outside [0, %d)", e0, e0 + n, b->E);
  if (n == 0) return MOE_OK;
  if (!digests) return fail(MOE_EINVAL, "record_sha256: null digests");
  if (!aligned(digests, 4)) return fail(MOE_EALIGN, "record_sha256: digests not 4-byte aligned");
  return hip_check(launch_record_sha256(v.base, v.stride, b->record_bytes, e0, n, digests,
                                        static_cast<hipStream_t>(stream)),
                   "record_sha256");
}

// ---- expert cache (host bank, HBM slots) ------------------------------------------
// The host bank's checks are the device bank's, without the device alignment
// of its base (host memory from the caller's pinned allocation).
static int host_bank_ok(const moe_nvfp4_bank* b, const char* who) {
  if (!b || !b->base) return fail(MOE_EINVAL, "%s: null bank", who);
  if (!record_shape_ok(b->H, b->I) || b->E < 1)
    return fail(MOE_ESHAPE, "%s: bank shape H=%d I=%d E=%d", who, b->H, b->I, b->E);
  if (b->stride < b->record_bytes || b->record_bytes != moe_nvfp4_record_bytes(b->H, b->I) || b->stride % 4096)
    return fail(MOE_EINVAL, "%s: record size/stride inconsistent with H, I", who);
  return MOE_OK;
}

MOE_API int moe_cache_create(const moe_nvfp4_bank* host_bank, void* slot_base, int nslots, moe_expert_cache** out) {
  int rc = host_bank_ok(host_bank, "cache_create");
  if (rc) return rc;
  if (!out) return fail(MOE_EINVAL, "cache_create: null out");
  if (nslots < 1 || nslots > 1024 || nslots > host_bank->E)
    return fail(MOE_ESHAPE, "cache_create: nslots=%d outside [1, min(E, 1024)]", nslots);
  if (!slot_base) return fail(MOE_EINVAL, "cache_create: null slot_base");
  if (!aligned(slot_base, 4096)) return fail(MOE_EALIGN, "cache_create: slot_base not 4096-byte aligned");
  rc = cache_create(host_bank, slot_base, nslots, out);
  if (rc == MOE_EHIP) return fail(MOE_EHIP, "cache_create: stream or event creation failed");
  if (rc) return fail(rc, "cache_create: out of host memory");
  return MOE_OK;
}

MOE_API int moe_cache_destroy(moe_expert_cache* c) {
  cache_destroy(c);
  return MOE_OK;
}

MOE_API int moe_cache_prepare(moe_expert_cache* c, const int32_t* ids, int n, int32_t* slot_of, void* stream) {
  if (!c) return fail(MOE_EINVAL, "cache_prepare: null cache");
  if (n < 0) return fail(MOE_EINVAL, "cache_prepare: n=%d < 0", n);
  if (n > 0 && (!ids || !slot_of)) return fail(MOE_EINVAL, "cache_prepare: null ids/slot_of");
  const int E = cache_experts(c);
  moe_nvfp4_bank view;
  cache_view(c, &view);
  std::vector<uint8_t> mark(E, 0);
  int distinct = 0;
  for (int i = 0; i < n; i++) {
    if (ids[i] < 0 || ids[i] >= E) return fail(MOE_EINVAL, "cache_prepare: ids[%d] = %d outside [0, %d)", i, ids[i], E);
    if (!mark[ids[i]]) {
      mark[ids[i]] = 1;
      distinct++;
    }
  }
  if (distinct > view.E) return fail(MOE_EINVAL, "cache_prepare: %d distinct experts do not fit %d slots", distinct, view.E);
  char err[256] = "";
  const int rc = cache_prepare(c, ids, n, slot_of, static_cast<hipStream_t>(stream), err, sizeof(err));
  if (rc) return fail(rc, "%s", err);
  return MOE_OK;
}

MOE_API int moe_cache_bank(const moe_expert_cache* c, moe_nvfp4_bank* out) {
  if (!c || !out) return fail(MOE_EINVAL, "cache_bank: null argument");
  return cache_view(c, out);
}

MOE_API int moe_cache_stats(const moe_expert_cache* c, int64_t* hits, int64_t* misses, int64_t* bytes_copied) {
  if (!c) return fail(MOE_EINVAL, "cache_stats: null cache");
  cache_stats(c, hits, misses, bytes_copied);
  return MOE_OK;
}

// ---- 8-dim VQ experts --------------------------------------------------------------
static bool vq_shape_ok(int H, int I) { return H > 0 && I > 0 && H % 64 == 0 && I % 64 == 0; }

MOE_API size_t moe_vq_record_bytes(int H, int I) {
  if (!vq_shape_ok(H, I)) return 0;
  size_t off = 0;
  for (int p = 0; p < 3; p++) {
    const size_t out = p == 2 ? H : I, in = p == 2 ? I : H;
    off = (off + out * in * 3 / 16 + 15) / 16 * 16;
    off = (off + out * 2 + 15) / 16 * 16;
  }
  return off;
}

MOE_API size_t moe_vq_record_stride(int H, int I) { return (moe_vq_record_bytes(H, I) + 4095) / 4096 * 4096; }

MOE_API int moe_vq_bank_init(moe_vq_bank* b, void* base, const void* codebook, int H, int I, int E) {
  if (!b || !base || !codebook) return fail(MOE_EINVAL, "vq_bank_init: null pointer");
  if (!vq_shape_ok(H, I)) return fail(MOE_ESHAPE, "vq_bank_init: H=%d I=%d must be positive multiples of 64", H, I);
  if (E < 1 || E > 1024) return fail(MOE_ESHAPE, "vq_bank_init: E=%d outside [1, 1024]", E);
  if (!aligned(base, 4096)) return fail(MOE_EALIGN, "vq_bank_init: base not 4096-byte aligned");
  if (!aligned(codebook, 16)) return fail(MOE_EALIGN, "vq_bank_init: codebook not 16-byte aligned");
  b->H = H;
  b->I = I;
  b->E = E;
  b->reserved = 0;
  size_t off = 0;
  for (int p = 0; p < 3; p++) {
    const size_t out = p == 2 ? H : I, in = p == 2 ? I : H;
    b->part_off[2 * p] = off;
    off = (off + out * in * 3 / 16 + 15) / 16 * 16;
    b->part_off[2 * p + 1] = off;
    off = (off + out * 2 + 15) / 16 * 16;
  }
  b->record_bytes = off;
  b->stride = moe_vq_record_stride(H, I);
  b->base = base;
  b->codebook = codebook;
  return MOE_OK;
}

static int vq_args(const moe_vq_bank* b, VqArgs* a, const char* who) {
  if (!b || !b->base || !b->codebook) return fail(MOE_EINVAL, "%s: null bank", who);
  if (!vq_shape_ok(b->H, b->I) || b->E < 1 || b->E > 1024)
    return fail(MOE_ESHAPE, "%s: bank shape H=%d I=%d E=%d", who, b->H, b->I, b->E);
  if (b->record_bytes != moe_vq_record_bytes(b->H, b->I) || b->stride < b->record_bytes || b->stride % 256)
    return fail(MOE_EINVAL, "%s: record size/stride inconsistent with H, I", who);
  if (!aligned(b->base, 256) || !aligned(b->codebook, 16)) return fail(MOE_EALIGN, "%s: base/codebook alignment", who);
  for (int p = 0; p < 3; p++) {
    const uint64_t out = p == 2 ? b->H : b->I, in = p == 2 ? b->I : b->H;
    if (b->part_off[2 * p] % 16 || b->part_off[2 * p + 1] % 16)
      return fail(MOE_EALIGN, "%s: part offsets of projection %d not 16-byte aligned", who, p);
    if (b->part_off[2 * p] + out * in * 3 / 16 > b->record_bytes || b->part_off[2 * p + 1] + out * 2 > b->record_bytes)
      return fail(MOE_EINVAL, "%s: part of projection %d outside the record", who, p);
  }
  *a = VqArgs{};
  a->bank = static_cast<const uint8_t*>(b->base);
  a->stride = b->stride;
  for (int p = 0; p < 3; p++) {
    a->idx_off[p] = b->part_off[2 * p];
    a->gain_off[p] = b->part_off[2 * p + 1];
  }
  a->codebook = static_cast<const uint8_t*>(b->codebook);
  a->H = b->H;
  a->I = b->I;
  a->E = b->E;
  return MOE_OK;
}

MOE_API int moe_vq_pack_bank(const moe_vq_bank* b, const uint8_t* const idx[3], const uint16_t* const gain[3],
                             void* stream) {
  VqArgs a;
  int rc = vq_args(b, &a, "vq_pack");
  if (rc) return rc;
  if (!idx || !gain) return fail(MOE_EINVAL, "vq_pack: null part arrays");
  for (int p = 0; p < 3; p++)
    if (!idx[p] || !gain[p]) return fail(MOE_EINVAL, "vq_pack: null part of projection %d", p);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* base = static_cast<uint8_t*>(b->base);
  for (int e = 0; e < b->E; e++) {
    uint8_t* rec = base + (size_t)e * b->stride;
    for (int p = 0; p < 3; p++) {
      const size_t out = p == 2 ? b->H : b->I, in = p == 2 ? b->I : b->H;
      const size_t nb = out * in * 3 / 16;
      rc = hip_check(hipMemcpyAsync(rec + b->part_off[2 * p], idx[p] + e * nb, nb, hipMemcpyDefault, s), "vq_pack idx");
      if (rc) return rc;
      rc = hip_check(hipMemcpyAsync(rec + b->part_off[2 * p + 1], gain[p] + e * out, out * 2, hipMemcpyDefault, s),
                     "vq_pack gains");
      if (rc) return rc;
    }
  }
  return hip_check(launch_zero_tails(base, b->stride, b->record_bytes, b->E, s), "vq_pack zero pad");
}

MOE_API int moe_vq_dequant(const moe_vq_bank* b, int expert, int proj, float* out_f32, void* stream) {
  VqArgs a;
  int rc = vq_args(b, &a, "vq_dequant");
  if (rc) return rc;
  if (expert < 0 || expert >= b->E || proj < 0 || proj > 2 || !out_f32)
    return fail(MOE_EINVAL, "vq_dequant: expert/proj out of range or null output");
  return hip_check(launch_vq_dequant(a, expert, proj, out_f32, static_cast<hipStream_t>(stream)), "vq_dequant");
}

MOE_API size_t moe_vq_workspace_bytes(int T, int k, int H, int I) {
  if (T < 0 || k < 1 || k > kFlatDecodeMaxK || !vq_shape_ok(H, I)) return 0;
  return up256((size_t)T * k * I * 2) + 256;
}

MOE_API int moe_vq_forward(const moe_vq_bank* b, const uint16_t* x, int T, const int32_t* idx, const float* w, int k,
                           const uint16_t* residual, void* y, unsigned flags, void* workspace,
                           size_t workspace_bytes, void* stream) {
  VqArgs a;
  int rc = vq_args(b, &a, "vq_forward");
  if (rc) return rc;
  if (T < 0) return fail(MOE_ESHAPE, "vq_forward: T=%d < 0", T);
  if (k < 1 || k > kFlatDecodeMaxK || k > b->E)
    return fail(MOE_ESHAPE, "vq_forward: k=%d outside [1, min(E, %d)]", k, kFlatDecodeMaxK);
  if (32768 + (size_t)k * b->I * 2 > 160 * 1024 - 2048)
    return fail(MOE_ESHAPE, "vq_forward: k*I*2 = %zu bytes of mids do not fit LDS beside the codebook",
                (size_t)k * b->I * 2);
  if (T == 0) return MOE_OK;
  if (!x || !idx || !w || !y || !workspace) return fail(MOE_EINVAL, "vq_forward: null pointer");
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(idx, 4) || !aligned(w, 4) || (residual && !aligned(residual, 8)) ||
      !aligned(workspace, 256))
    return fail(MOE_EALIGN, "vq_forward: x, y 16 B; idx, w 4 B; residual 8 B; workspace 256 B");
  if (workspace_bytes < moe_vq_workspace_bytes(T, k, b->H, b->I))
    return fail(MOE_EWORKSPACE, "vq_forward: workspace %zu < %zu bytes", workspace_bytes,
                moe_vq_workspace_bytes(T, k, b->H, b->I));
  a.k = k;
  a.T = T;
  a.idx = idx;
  a.w = w;
  a.x = x;
  a.residual = residual;
  a.mid = static_cast<uint16_t*>(workspace);
  a.y = y;
  a.f32_out = (flags & MOE_F32_OUT) ? 1 : 0;
  return hip_check(launch_vq_forward(a, static_cast<hipStream_t>(stream)), "vq_forward");
}

// ---- S1 + S2 routing -----------------------------------------------------------
MOE_API int moe_route_topk(const uint16_t* x, const float* w_router, float* logits, int T, int H,
                           int E, int k, int32_t* idx, float* w, void* stream) {
  if (T < 0) return fail(MOE_ESHAPE, "route: T=%d < 0", T);
  if (E < 1 || E > 1024) return fail(MOE_ESHAPE, "route: E=%d outside [1, 1024]", E);
  if (k < 1 || k > E || k > 64) return fail(MOE_ESHAPE, "route: k=%d outside [1, min(E, 64)]", k);
  if (!logits || !idx || !w) return fail(MOE_EINVAL, "route: null logits/idx/w");
  const bool gemm = x && w_router;
  if ((x == nullptr) != (w_router == nullptr)) return fail(MOE_EINVAL, "route: give both x and w_router, or neither");
  if (gemm) {
    if (H <= 0 || H % 16) return fail(MOE_ESHAPE, "route: H=%d must be a positive multiple of 16", H);
    if (!aligned(x, 8) || !aligned(w_router, 16)) return fail(MOE_EALIGN, "route: x must be 8-byte, w_router 16-byte aligned");
  }
  if (!aligned(logits, 4)) return fail(MOE_EALIGN, "route: logits alignment");
  if (T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (gemm) {
    int rc = hip_check(launch_router(x, w_router, logits, T, H, E, s), "router");
    if (rc) return rc;
  }
  return hip_check(launch_topk(logits, T, E, k, idx, w, s), "topk");
}

// ---- S3 sort ---------------------------------------------------------------------
struct FwdLayout {
  size_t counts, offsets, sorted, active, tile_e, tile_r, hist, tags, mid, part, total;
  int max_tiles;
};
// counts area (256 bytes): [0] active experts, [1] tiles (pair sort),
// [2] the status word (byte offset MOE_STATUS_OFFSET)
static_assert(MOE_STATUS_OFFSET == 8, "status word is counts[2]");

static FwdLayout fwd_layout(int T, int k, int H, int I, int E) {
  FwdLayout L{};
  const size_t P = (size_t)T * (size_t)k;
  L.max_tiles = (int)(P / kPrefillMTile + (P < (size_t)E ? P : (size_t)E) + 1);
  size_t o = 0;
  L.counts = o;
  o += 256;
  L.offsets = o;
  o += up256(((size_t)E + 1) * 4);
  L.sorted = o;
  o += up256(P * 4 + 4);
  L.active = o;
  o += up256((size_t)E * 4);
  L.tile_e = o;
  o += up256((size_t)L.max_tiles * 4);
  L.tile_r = o;
  o += up256((size_t)L.max_tiles * 4);
  L.hist = o;
  o += up256((size_t)sort_hist_ints((int)(P < (1u << 30) ? P : 0), E) * 4);
  L.tags = o;
  o += up256((1024 + kFlatDecodeMaxK) * 8);  // router tags (1024 slots), then the routing record
  L.mid = o;
  o += up256(P * (size_t)I * 2);
  L.part = o;
  o += up256(P * (size_t)H * 4);
  L.total = o;
  return L;
}

MOE_API int moe_sort_pairs(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                           int32_t* sorted, void* stream) {
  if (T < 0 || k < 1 || k > 64) return fail(MOE_ESHAPE, "sort: T=%d k=%d", T, k);
  if (E < 1 || E > 1024) return fail(MOE_ESHAPE, "sort: E=%d outside [1, 1024]", E);
  if (!idx || !offsets || !sorted) return fail(MOE_EINVAL, "sort: null pointer");
  const long long P = (long long)T * k;
  if (P > (1LL << 30)) return fail(MOE_ESHAPE, "sort: too many pairs");
  hipStream_t s = static_cast<hipStream_t>(stream);
  RouteTables rt{};  // no active list, counters or tile table for this entry point
  rt.offsets = offsets;
  rt.sorted = sorted;
  return hip_check(launch_sort(idx, (int)P, E, rt, 0, 0, s), "sort");
}

MOE_API size_t moe_sort_workspace_bytes(int T, int k, int E) {
  if (T < 0 || k < 1 || k > 64 || E < 1 || E > 1024) return 0;
  const long long P = (long long)T * k;
  if (P > (1LL << 30)) return 0;
  return (size_t)sort_hist_ints((int)P, E) * 4 + 4;
}

MOE_API int moe_sort_pairs_ws(const int32_t* idx, int T, int k, int E, int32_t* offsets, int32_t* sorted,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (T < 0 || k < 1 || k > 64) return fail(MOE_ESHAPE, "sort: T=%d k=%d", T, k);
  if (E < 1 || E > 1024) return fail(MOE_ESHAPE, "sort: E=%d outside [1, 1024]", E);
  if (!idx || !offsets || !sorted || !workspace) return fail(MOE_EINVAL, "sort: null pointer");
  const long long P = (long long)T * k;
  if (P > (1LL << 30)) return fail(MOE_ESHAPE, "sort: too many pairs");
  if (!aligned(workspace, 4)) return fail(MOE_EALIGN, "sort: workspace not 4-byte aligned");
  if (workspace_bytes < moe_sort_workspace_bytes(T, k, E))
    return fail(MOE_EWORKSPACE, "sort: workspace %zu < %zu bytes", workspace_bytes, moe_sort_workspace_bytes(T, k, E));
  RouteTables rt{};
  rt.offsets = offsets;
  rt.sorted = sorted;
  rt.hist = static_cast<int32_t*>(workspace);
  return hip_check(launch_sort(idx, (int)P, E, rt, 0, 0, static_cast<hipStream_t>(stream)), "sort");
}

// ---- S3..S7 forward --------------------------------------------------------------
MOE_API size_t moe_nvfp4_workspace_bytes(int T, int k, int H, int I, int E) {
  if (T < 0 || k < 1 || E < 1 || H <= 0 || I <= 0) return 0;
  return fwd_layout(T, k, H, I, E).total;
}

static int prefill_min_pairs() {
  static int v = -1;
  if (v < 0) {
    const char* s = std::getenv("MOE_PREFILL_MIN_PAIRS");
    v = (s && *s) ? std::atoi(s) : 1024;
    if (v < 1) v = 1;
  }
  return v;
}

// Checks shared by the forward and layer entry points (idx and w are checked
// by the callers: inputs of one, outputs of the other).
static int layer_checks(const char* who, const BankView& v, const uint16_t* x, int T, int k,
                        const uint16_t* residual, void* y, unsigned flags, void* workspace,
                        size_t workspace_bytes, FwdLayout* L) {
  if (v.H % 64 || v.I % 64) return fail(MOE_ESHAPE, "%s: H=%d and I=%d must be multiples of 64", who, v.H, v.I);
  if (T < 0) return fail(MOE_ESHAPE, "%s: T=%d < 0", who, T);
  if (k < 1 || k > v.E || k > 64) return fail(MOE_ESHAPE, "%s: k=%d outside [1, min(E, 64)]", who, k);
  if ((flags & MOE_FORCE_DECODE) && (flags & MOE_FORCE_PREFILL))
    return fail(MOE_EINVAL, "%s: both FORCE flags set", who);
  if (flags & ~(MOE_F32_OUT | MOE_FORCE_DECODE | MOE_FORCE_PREFILL)) return fail(MOE_EINVAL, "%s: unknown flags", who);
  if ((long long)T * k > (1LL << 30)) return fail(MOE_ESHAPE, "%s: too many pairs", who);
  if (T == 0) return MOE_OK;
  if (!x || !y || !workspace) return fail(MOE_EINVAL, "%s: null pointer", who);
  if (!aligned(x, 16) || (residual && !aligned(residual, 8)) || !aligned(y, 16))
    return fail(MOE_EALIGN, "%s: x and y must be 16-byte aligned, residual 8-byte", who);
  if (!aligned(workspace, 256)) return fail(MOE_EALIGN, "%s: workspace not 256-byte aligned", who);
  *L = fwd_layout(T, k, v.H, v.I, v.E);
  if (workspace_bytes < L->total)
    return fail(MOE_EWORKSPACE, "%s: workspace %zu < %zu bytes", who, workspace_bytes, L->total);
  return MOE_OK;
}

// read at each call (a test compares both routings in one process)
static bool gemv_inblock() {
  const char* s = std::getenv("MOE_GEMV_INBLOCK");
  return s && *s && std::atoi(s) != 0;
}

// read at each call (a test runs both sides of the limit in one process)
static int flat_max_t() {
  const char* s = std::getenv("MOE_FLAT_MAX_T");
  const int v = (s && *s) ? std::atoi(s) : kFlatDecodeMaxT;
  return v < 1 ? 1 : v;
}

// up to kFlatDecodeMaxT tokens of at most kFlatDecodeMaxK pairs each, whose
// mids fit in 64 KiB of LDS
static bool flat_path(const BankView& v, int T, int k, unsigned flags) {
  return T >= 1 && T <= flat_max_t() && !(flags & MOE_FORCE_PREFILL) && k <= kFlatDecodeMaxK &&
         (size_t)k * v.I * 2 <= 65536 && v.I % 16 == 0;
}

// The grouped-GEMM kernels address activation rows with 32-bit byte offsets
// from one base, so a prefill runs over token chunks whose activations span
// at most 2 GiB (209,715 tokens at H = 5120); each chunk is a forward of its
// own (rows of y depend only on their own tokens).
static long long prefill_chunk_tokens(int H) { return (1LL << 31) / (2LL * H); }

static int forward_run(const BankView& v, const uint16_t* x, int T, const int32_t* idx, const float* w, int k,
                       const uint16_t* residual, void* y, unsigned flags, uint8_t* ws, const FwdLayout& L,
                       hipStream_t s, uint32_t* status) {
  int rc;
  RouteTables rt{};
  rt.counts = reinterpret_cast<int32_t*>(ws + L.counts);
  rt.offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  rt.sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
  rt.active = reinterpret_cast<int32_t*>(ws + L.active);
  rt.tile_expert = reinterpret_cast<int32_t*>(ws + L.tile_e);
  rt.tile_row0 = reinterpret_cast<int32_t*>(ws + L.tile_r);
  rt.hist = reinterpret_cast<int32_t*>(ws + L.hist);
  rt.status = status;
  uint16_t* mid = reinterpret_cast<uint16_t*>(ws + L.mid);
  float* part = reinterpret_cast<float*>(ws + L.part);
  const int P = T * k;
  bool prefill = P >= prefill_min_pairs();
  if (flags & MOE_FORCE_DECODE) prefill = false;
  if (flags & MOE_FORCE_PREFILL) prefill = true;
  const bool f32_out = (flags & MOE_F32_OUT) != 0;
  if (!prefill && flat_path(v, T, k, flags))
    return hip_check(launch_flat_decode(v, x, T, idx, w, k, residual, mid, y, f32_out, rt.status, s), "decode");

  if (prefill) {
    const size_t ysize = f32_out ? 4 : 2;
    const int tc_max = (int)std::min<long long>(T, prefill_chunk_tokens(v.H));
    for (int t0 = 0; t0 < T; t0 += tc_max) {
      const int tc = std::min(tc_max, T - t0), pc = tc * k;
      const uint16_t* xc = x + (size_t)t0 * v.H;
      const int32_t* ic = idx + (size_t)t0 * k;
      const float* wc = w + (size_t)t0 * k;
      const uint16_t* rc_res = residual ? residual + (size_t)t0 * v.H : nullptr;
      void* yc = static_cast<uint8_t*>(y) + (size_t)t0 * v.H * ysize;
      rc = hip_check(launch_sort(ic, pc, v.E, rt, kPrefillMTile, L.max_tiles, s), "sort");
      if (rc) return rc;
      rc = hip_check(launch_prefill_gateup(v, xc, k, rt, L.max_tiles, mid, s), "prefill gate/up");
      if (rc) return rc;
      rc = hip_check(launch_prefill_down(v, mid, wc, k, rt, L.max_tiles, part, s), "prefill down");
      if (rc) return rc;
      rc = hip_check(launch_combine(part, ic, v.E, tc, v.H, k, rc_res, yc, f32_out, s), "combine");
      if (rc) return rc;
    }
    return MOE_OK;
  }
  // few pairs: the GEMV blocks take their expert and its pairs from the
  // sorted tables (one small sort launch). Routing inside every block
  // (env MOE_GEMV_INBLOCK=1, up to kDecInblockMaxP pairs) saves the launch
  // but measured slower: 1.01 against 0.88 ms at T = 32, k = 8.
  const bool inblock = gemv_inblock() && P <= kDecInblockMaxP;
  if (!inblock) {
    rc = hip_check(launch_sort(idx, P, v.E, rt, 0, L.max_tiles, s), "sort");
    if (rc) return rc;
  }
  const RouteTables* rtp = inblock ? nullptr : &rt;
  const int slots = P < v.E ? P : v.E;
  const int max_m = T;  // top-k selects an expert at most once per token
  rc = hip_check(launch_decode_gateup(v, x, idx, P, k, rtp, slots, max_m, mid, rt.status, s), "decode gate/up");
  if (rc) return rc;
  rc = hip_check(launch_decode_down(v, mid, w, idx, P, k, rtp, slots, max_m, part, s), "decode down");
  if (rc) return rc;
  return hip_check(launch_combine(part, idx, v.E, T, v.H, k, residual, y, f32_out, s), "combine");
}

MOE_API int moe_nvfp4_forward(const moe_nvfp4_bank* b, const uint16_t* x, int T, const int32_t* idx,
                              const float* w, int k, const uint16_t* residual, void* y,
                              unsigned flags, void* workspace, size_t workspace_bytes,
                              void* stream) {
  BankView v;
  int rc = bank_view(b, &v, "forward");
  if (rc) return rc;
  FwdLayout L;
  rc = layer_checks("forward", v, x, T, k, residual, y, flags, workspace, workspace_bytes, &L);
  if (rc || T == 0) return rc;
  if (!idx || !w) return fail(MOE_EINVAL, "forward: null idx/w");
  if (!aligned(idx, 4) || !aligned(w, 4)) return fail(MOE_EALIGN, "forward: idx/w must be 4-byte aligned");
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  return forward_run(v, x, T, idx, w, k, residual, y, flags, ws, L, static_cast<hipStream_t>(stream),
                     reinterpret_cast<uint32_t*>(ws + L.counts) + 2);
}

// ---- the forward with no allocation ------------------------------------------------
// For callers that cannot allocate (code under graph capture, tight serving
// loops): the workspace of moe_nvfp4_forward taken from a file-scope device
// array. Each GPU the library runs on holds its own copy until the process
// ends. In host code `scratch` is only a stand-in for the device symbol: the
// address kernels must use comes from hipGetSymbolAddress, once per device.
static_assert(MOE_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

// The current device's copy of `scratch` (its address on that device).
static int scratch_ptr(uint8_t** out) {
  int dev = -1;
  int rc = hip_check(hipGetDevice(&dev), "forward_noalloc: hipGetDevice");
  if (rc) return rc;
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EINVAL, "forward_noalloc: device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    rc = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "forward_noalloc: hipGetSymbolAddress");
    if (rc) return rc;
    if (!p || !aligned(p, 256)) return fail(MOE_EHIP, "forward_noalloc: scratch address not 256-byte aligned");
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<uint8_t*>(g_scratch_ptr[dev]);
  return MOE_OK;
}

MOE_API int moe_nvfp4_forward_noalloc(const moe_nvfp4_bank* b, const uint16_t* x, int T, const int32_t* idx,
                                      const float* w, int k, const uint16_t* residual, void* y, unsigned flags,
                                      uint32_t* status, void* stream) {
  BankView v;
  int rc = bank_view(b, &v, "forward_noalloc");
  if (rc) return rc;
  if (status && !aligned(status, 4)) return fail(MOE_EALIGN, "forward_noalloc: status not 4-byte aligned");
  const size_t need = moe_nvfp4_workspace_bytes(T, k, v.H, v.I, v.E);
  if (need > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_EWORKSPACE, "forward_noalloc: the call needs %zu bytes of scratch, the library holds %zu per GPU",
                need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  uint8_t* ws = nullptr;
  if (T > 0) {
    rc = scratch_ptr(&ws);
    if (rc) return rc;
  }
  FwdLayout L;
  // the scratch stands in for the workspace: the same checks, the same layout
  rc = layer_checks("forward_noalloc", v, x, T, k, residual, y, flags, ws, MOE_NOALLOC_SCRATCH_BYTES, &L);
  if (rc || T == 0) return rc;
  if (!idx || !w) return fail(MOE_EINVAL, "forward_noalloc: null idx/w");
  if (!aligned(idx, 4) || !aligned(w, 4)) return fail(MOE_EALIGN, "forward_noalloc: idx/w must be 4-byte aligned");
  // without a status word of the caller's, bad expert ids go to the scratch's
  // own word, which nobody reads
  uint32_t* st = status ? status : reinterpret_cast<uint32_t*>(ws + L.counts) + 2;
  return forward_run(v, x, T, idx, w, k, residual, y, flags, ws, L, static_cast<hipStream_t>(stream), st);
}

// ---- S1..S7 in one call ------------------------------------------------------------
// Call numbers stamp the router tags in the workspace. They start from a
// clock-derived value per process and skip 0 (the value a zero-filled
// workspace holds).
static uint32_t next_call_number() {
  static std::atomic<uint32_t> counter{(uint32_t)std::chrono::steady_clock::now().time_since_epoch().count() ^
                                       ((uint32_t)getpid() << 16)};
  uint32_t c;
  do {
    c = counter.fetch_add(1) + 1;
  } while (c == 0);
  return c;
}

// Read at each call: MOE_DEBUG_ROUTE_GIVEUP=1 makes the one-token layer's
// router workgroups withhold their logits and the waits give up after a few
// polls, so that a test can check the give-up contract (every kernel still
// ends normally).
static bool debug_route_giveup() {
  const char* s = std::getenv("MOE_DEBUG_ROUTE_GIVEUP");
  return s && *s && std::atoi(s) != 0;
}

MOE_API int moe_nvfp4_layer(const moe_nvfp4_bank* b, const uint16_t* x, const float* w_router, int T, int k,
                            const uint16_t* residual, float* logits, int32_t* idx, float* w, void* y,
                            unsigned flags, void* workspace, size_t workspace_bytes, void* stream) {
  BankView v;
  int rc = bank_view(b, &v, "layer");
  if (rc) return rc;
  if (v.E > 1024) return fail(MOE_ESHAPE, "layer: E=%d above 1024", v.E);
  FwdLayout L;
  rc = layer_checks("layer", v, x, T, k, residual, y, flags, workspace, workspace_bytes, &L);
  if (rc || T == 0) return rc;
  if (!w_router || !logits || !idx || !w) return fail(MOE_EINVAL, "layer: null w_router/logits/idx/w");
  if (!aligned(w_router, 16) || !aligned(logits, 4) || !aligned(idx, 4) || !aligned(w, 4))
    return fail(MOE_EALIGN, "layer: w_router must be 16-byte aligned, logits/idx/w 4-byte");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  if (T == 1 && flat_path(v, T, k, flags)) {
    uint64_t* tags = reinterpret_cast<uint64_t*>(ws + L.tags);
    uint32_t* status = reinterpret_cast<uint32_t*>(ws + L.counts) + 2;
    uint16_t* mid = reinterpret_cast<uint16_t*>(ws + L.mid);
    return hip_check(launch_flat_layer(v, x, w_router, k, residual, logits, idx, w, mid, tags, status,
                                       next_call_number(), y, (flags & MOE_F32_OUT) != 0, s, debug_route_giveup()),
                     "layer");
  }
  rc = hip_check(launch_router(x, w_router, logits, T, v.H, v.E, s), "router");
  if (rc) return rc;
  rc = hip_check(launch_topk(logits, T, v.E, k, idx, w, s), "topk");
  if (rc) return rc;
  return forward_run(v, x, T, idx, w, k, residual, y, flags, ws, L, s, reinterpret_cast<uint32_t*>(ws + L.counts) + 2);
}

// ---- the workspace status word --------------------------------------------------
static_assert(MOE_STATUS_ROUTE_TIMEOUT == kStatusRouteTimeout && MOE_STATUS_BAD_IDX == kStatusBadIdx,
              "status bits");

MOE_API int moe_status_read(const void* workspace, uint32_t* status, void* stream) {
  if (!workspace || !status) return fail(MOE_EINVAL, "status_read: null pointer");
  if (!aligned(workspace, 256)) return fail(MOE_EALIGN, "status_read: workspace not 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  int rc = hip_check(hipMemcpyAsync(&v, static_cast<const uint8_t*>(workspace) + MOE_STATUS_OFFSET, 4,
                                    hipMemcpyDeviceToHost, s), "status_read");
  if (rc) return rc;
  rc = hip_check(hipStreamSynchronize(s), "status_read");
  if (rc) return rc;
  *status = v;
  return MOE_OK;
}

MOE_API int moe_status_clear(void* workspace, void* stream) {
  if (!workspace) return fail(MOE_EINVAL, "status_clear: null workspace");
  if (!aligned(workspace, 256)) return fail(MOE_EALIGN, "status_clear: workspace not 256-byte aligned");
  uint32_t* p = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(workspace) + MOE_STATUS_OFFSET);
  return hip_check(launch_store_u32(p, 0u, static_cast<hipStream_t>(stream)), "status_clear");
}

// ---- S8 affine8_g64 --------------------------------------------------------------
// tokens from which the linear runs as an MFMA GEMM instead of the
// weight-streaming kernel
static int affine8_gemm_min_t() {
  static int v = -1;
  if (v < 0) {
    const char* s = std::getenv("MOE_AFFINE8_GEMM_MIN_T");
    // from 33 tokens: with K split over the chip the GEMM takes 25-27 us at
    // any T up to 128 (K = N = 5120), the bandwidth-bound pass 25 us at
    // T = 32 and 37-48 us at 48-63
    v = (s && *s) ? std::atoi(s) : 33;
    if (v < 1) v = 1;
  }
  return v;
}

MOE_API int affine8_g64_linear(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                               const uint16_t* biases, int T, int K, int N, uint16_t* y,
                               void* stream) {
  if (T < 0 || N < 1 || K < 64 || K % 64) return fail(MOE_ESHAPE, "affine8: T=%d K=%d N=%d", T, K, N);
  if (T == 0) return MOE_OK;
  if (!x || !codes || !scales || !biases || !y) return fail(MOE_EINVAL, "affine8: null pointer");
  if (!aligned(codes, 16) || !aligned(x, 4) || !aligned(y, 2) || !aligned(scales, 2) || !aligned(biases, 2))
    return fail(MOE_EALIGN, "affine8: codes must be 16-byte aligned, x 4-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T >= affine8_gemm_min_t() && aligned(x, 16))
    return hip_check(launch_affine8_gemm(x, codes, scales, biases, T, K, N, y, s), "affine8 gemm");
  return hip_check(launch_affine8(x, codes, scales, biases, T, K, N, y, s), "affine8");
}

// ---- S9 rmsnorm --------------------------------------------------------------------
MOE_API int moe_rmsnorm(const uint16_t* x, int T, int H, float eps, uint16_t* y, void* stream) {
  if (T < 0 || H < 1) return fail(MOE_ESHAPE, "rmsnorm: T=%d H=%d", T, H);
  if (!(eps >= 0.0f)) return fail(MOE_EINVAL, "rmsnorm: eps must be >= 0");
  if (T == 0) return MOE_OK;
  if (!x || !y) return fail(MOE_EINVAL, "rmsnorm: null pointer");
  return hip_check(launch_rmsnorm(x, T, H, eps, y, static_cast<hipStream_t>(stream)), "rmsnorm");
}

// ---- dequant test export -----------------------------------------------------------
MOE_API int moe_nvfp4_dequant(const moe_nvfp4_bank* b, int expert, int proj, float* out_f32,
                              uint16_t* out_unit, void* stream) {
  BankView v;
  int rc = bank_view(b, &v, "dequant");
  if (rc) return rc;
  if (expert < 0 || expert >= v.E) return fail(MOE_EINVAL, "dequant: expert %d outside [0, %d)", expert, v.E);
  if (proj < 0 || proj > 2) return fail(MOE_EINVAL, "dequant: proj %d outside [0, 2]", proj);
  if (!out_f32 && !out_unit) return fail(MOE_EINVAL, "dequant: no output");
  if ((out_f32 && !aligned(out_f32, 4)) || (out_unit && !aligned(out_unit, 2)))
    return fail(MOE_EALIGN, "dequant: output alignment");
  return hip_check(launch_dequant(v, expert, proj, out_f32, out_unit, static_cast<hipStream_t>(stream)),
                   "dequant");
}

// ---- achievable-peak probes -----------------------------------------------------------
MOE_API int moe_probe_hbm_read(const void* buf, size_t nbytes, int variant, int blocks, uint32_t* sink,
                               void* stream) {
  if (!buf || !sink) return fail(MOE_EINVAL, "probe_hbm_read: null pointer");
  if (!aligned(buf, 16) || nbytes % 16) return fail(MOE_EALIGN, "probe_hbm_read: buf and nbytes must be 16-byte multiples");
  if (variant < 0 || variant > 3 || blocks < 1 || blocks > (1 << 20))
    return fail(MOE_EINVAL, "probe_hbm_read: variant %d outside [0, 3] or blocks %d outside [1, 2^20]", variant, blocks);
  if (nbytes == 0) return MOE_OK;
  return hip_check(launch_probe_hbm_read(buf, nbytes, variant, blocks, sink, static_cast<hipStream_t>(stream)),
                   "probe_hbm_read");
}

MOE_API int moe_probe_mfma_bf16(int blocks, int iters, float* sink, void* stream) {
  if (!sink) return fail(MOE_EINVAL, "probe_mfma_bf16: null sink");
  if (blocks < 1 || blocks > (1 << 20) || iters < 1) return fail(MOE_EINVAL, "probe_mfma_bf16: blocks %d, iters %d", blocks, iters);
  return hip_check(launch_probe_mfma(blocks, iters, sink, static_cast<hipStream_t>(stream)), "probe_mfma_bf16");
}

// ---- timing --------------------------------------------------------------------------
MOE_API int moe_profile_enable(int on) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  p.clear();
  p.on = on != 0;
  return MOE_OK;
}

MOE_API int moe_profile_read(const char* name, double* total_ms, int64_t* launches) {
  if (!name || !total_ms || !launches) return fail(MOE_EINVAL, "profile_read: null pointer");
  Profiler& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  double tot = 0.0;
  int64_t n = 0;
  auto it = p.done.find(name);
  if (it != p.done.end()) {
    for (auto& pe : it->second) {
      int rc = hip_check(hipEventSynchronize(pe.end), "profile_read");
      if (rc) return rc;
      float ms = 0.0f;
      rc = hip_check(hipEventElapsedTime(&ms, pe.start, pe.end), "profile_read");
      if (rc) return rc;
      tot += ms;
      n++;
    }
  }
  *total_ms = tot;
  *launches = n;
  return MOE_OK;
}
