// HBM -> LDS loads for gfx950 kernels that manage their own waits.
#pragma once
#include "common.h"

namespace moe {

// One wave-wide HBM -> LDS load (global_load_lds_dwordx4): lane l's 16 bytes
// at base + voff land at LDS byte address lds + 16 l; base and lds are
// wave-uniform. Issued from inline asm so the compiler's wait insertion does
// not make every later LDS access and barrier wait for it: a kernel using it
// waits for these loads itself (wait_vmcnt) before it reads their data, and
// must not have other vector-memory loads in flight that the count would
// miss. The instruction writes no registers.
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base), "s"(lds)
               : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ const uint8_t* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

// A linear copy of nbytes (a multiple of 16; src and dst 16-byte aligned)
// from global memory to LDS by the nwaves waves of a workgroup: wave w copies
// the 1 KiB chunks w, w + nwaves, ... with one wave-wide load each, all in
// flight together. The caller waits (wait_vmcnt<0>, then a barrier) before any
// wave reads the copy.
__device__ __forceinline__ void dma_copy_lds(const void* src, void* dst, uint32_t nbytes, int nwaves) {
  const uint8_t* base = uniform_ptr(src);
  const uint32_t l0 = lds_addr(dst);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (uint32_t c = wave; c * 1024 < nbytes; c += nwaves) {
    const uint32_t off = c * 1024 + 16 * lane;
    if (off < nbytes) dma16(base, off, __builtin_amdgcn_readfirstlane(l0 + c * 1024));
  }
}

// The same copy into the swizzled input layout of the expert-streaming
// kernels (16-byte chunk c of 64-input quad q at chunk position 8 q + (c ^
// (q & 7)), quads counted from src): lane l of a load fills position l of its
// 64 chunks, so it reads the chunk that belongs there (the XOR is its own
// inverse, and a KiB holds 8 whole quads). nbytes: whole quads (128 bytes).
__device__ __forceinline__ void dma_copy_lds_swz(const void* src, void* dst, uint32_t nbytes, int nwaves) {
  const uint8_t* base = uniform_ptr(src);
  const uint32_t l0 = lds_addr(dst);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (uint32_t c = wave; c * 1024 < nbytes; c += nwaves) {
    const uint32_t pos = c * 64 + lane;  // chunk position this lane fills
    const uint32_t q = pos >> 3;
    const uint32_t off = 16u * (8u * q + ((pos & 7u) ^ (q & 7u)));
    if (16u * pos < nbytes) dma16(base, off, __builtin_amdgcn_readfirstlane(l0 + c * 1024));
  }
}

// Workgroup barrier after this wave's LDS accesses have completed. No memory
// fence: __syncthreads()'s fence would also wait for every load in flight
// (weights loaded into registers ahead of their use, HBM -> LDS copies). The
// asm statement keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void step_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// s_waitcnt vmcnt(n) alone (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace moe
