// A bounded cache of expert records in HBM, fed from host memory.
//
// "Beam 1.0 501B-A23B, streaming pack, NVFP4 experts / MLX 8-bit residents",
// "What it is for": the routed experts the router selects stream into a
// bounded cache of expert rows on the GPU, so a machine serves a bank larger
// than its GPU memory; the memory section counts the rows (prompt rows and
// decode rows). "Beam-1.0-501B-A23B, EXL3 3-bit, for 2x RTX PRO 6000
// Blackwell" ("How it fits") keeps the
// coldest experts in pinned host RAM and moves them over PCIe on a side
// stream. Here the full bank sits in host memory (pinned by the caller), a
// pool of slots in HBM holds the records in use, and misses are copied on the
// cache's own stream.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/moe_mi355x.h"
#include "internal.h"

struct moe_expert_cache {
  moe_nvfp4_bank host;            // the full bank, base in host memory
  uint8_t* slots;                 // device, nslots * stride
  int nslots;
  std::vector<int32_t> slot_expert;  // expert held by each slot (-1: none)
  std::vector<int32_t> expert_slot;  // slot of each expert (-1: not resident)
  std::vector<uint64_t> last_use;    // tick of each slot's last request
  std::vector<uint64_t> in_call;     // call tick that named the slot, so it is not evicted within the call
  uint64_t tick = 0;
  int64_t hits = 0, misses = 0, bytes = 0;
  hipStream_t copy = nullptr;
  hipEvent_t compute_done = nullptr, copies_done = nullptr;
};

namespace moe {

int cache_create(const moe_nvfp4_bank* host, void* slot_base, int nslots, moe_expert_cache** out) {
  moe_expert_cache* c = new (std::nothrow) moe_expert_cache();
  if (!c) return MOE_EINVAL;
  c->host = *host;
  c->slots = static_cast<uint8_t*>(slot_base);
  c->nslots = nslots;
  c->slot_expert.assign(nslots, -1);
  c->expert_slot.assign(host->E, -1);
  c->last_use.assign(nslots, 0);
  c->in_call.assign(nslots, 0);
  if (hipStreamCreateWithFlags(&c->copy, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&c->compute_done, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&c->copies_done, hipEventDisableTiming) != hipSuccess) {
    cache_destroy(c);
    return MOE_EHIP;
  }
  *out = c;
  return MOE_OK;
}

void cache_destroy(moe_expert_cache* c) {
  if (!c) return;
  if (c->copy) {
    hipStreamSynchronize(c->copy);
    hipStreamDestroy(c->copy);
  }
  if (c->compute_done) hipEventDestroy(c->compute_done);
  if (c->copies_done) hipEventDestroy(c->copies_done);
  delete c;
}

// The least recently used slot that the current call (tick) has not named;
// empty slots first (their tick is 0), then the lowest slot index. The caller
// has checked that the call's distinct experts fit the slots, so one exists.
static int pick_victim(const moe_expert_cache* c) {
  int best = -1;
  for (int s = 0; s < c->nslots; s++) {
    if (c->in_call[s] == c->tick) continue;
    if (best < 0 || c->last_use[s] < c->last_use[best]) best = s;
  }
  return best;
}

// ids: experts in [0, E) whose distinct count is at most nslots (checked by
// the caller). An id resident before the call, or placed earlier in the same
// call, is a hit; the others are misses, each given the victim slot.
int cache_prepare(moe_expert_cache* c, const int32_t* ids, int n, int32_t* slot_of, hipStream_t stream,
                  char* err, size_t errlen) {
  c->tick++;
  std::vector<int> miss_slot(n, -1);
  // resident experts named by the call are not evicted by its misses
  for (int i = 0; i < n; i++)
    if (c->expert_slot[ids[i]] >= 0) c->in_call[c->expert_slot[ids[i]]] = c->tick;
  int n_miss = 0;
  for (int i = 0; i < n; i++) {
    const int e = ids[i];
    if (c->expert_slot[e] < 0) {
      const int s = pick_victim(c);
      if (c->slot_expert[s] >= 0) c->expert_slot[c->slot_expert[s]] = -1;
      c->slot_expert[s] = e;
      c->expert_slot[e] = s;
      c->in_call[s] = c->tick;
      miss_slot[i] = s;
      n_miss++;
    }
    slot_of[i] = c->expert_slot[e];
  }
  for (int i = 0; i < n; i++) c->last_use[slot_of[i]] = c->tick;
  if (n_miss > 0) {
    // a slot may still be read by work already on the compute stream: the
    // copies wait for it, and the compute stream waits for the copies
    if (hipEventRecord(c->compute_done, stream) != hipSuccess ||
        hipStreamWaitEvent(c->copy, c->compute_done, 0) != hipSuccess) {
      snprintf(err, errlen, "cache_prepare: stream ordering failed");
      return MOE_EHIP;
    }
    const uint8_t* src = static_cast<const uint8_t*>(c->host.base);
    for (int i = 0; i < n; i++) {
      if (miss_slot[i] < 0) continue;
      if (hipMemcpyAsync(c->slots + (size_t)miss_slot[i] * c->host.stride, src + (size_t)ids[i] * c->host.stride,
                         c->host.stride, hipMemcpyHostToDevice, c->copy) != hipSuccess) {
        snprintf(err, errlen, "cache_prepare: copy of expert %d failed", ids[i]);
        return MOE_EHIP;
      }
      c->bytes += (int64_t)c->host.stride;
    }
    if (hipEventRecord(c->copies_done, c->copy) != hipSuccess ||
        hipStreamWaitEvent(stream, c->copies_done, 0) != hipSuccess) {
      snprintf(err, errlen, "cache_prepare: stream ordering failed");
      return MOE_EHIP;
    }
  }
  c->misses += n_miss;
  c->hits += n - n_miss;
  return MOE_OK;
}

// the slot pool as a bank of nslots records
int cache_view(const moe_expert_cache* c, moe_nvfp4_bank* out) {
  *out = c->host;
  out->base = c->slots;
  out->E = c->nslots;
  return MOE_OK;
}

int cache_experts(const moe_expert_cache* c) { return c->host.E; }

void cache_stats(const moe_expert_cache* c, int64_t* hits, int64_t* misses, int64_t* bytes) {
  if (hits) *hits = c->hits;
  if (misses) *misses = c->misses;
  if (bytes) *bytes = c->bytes;
}

}  // namespace moe
