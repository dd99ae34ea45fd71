// Probes of what this GPU reaches in practice, the second denominators of the
// rooflines the layer's kernels are held to: a streaming read of HBM (the
// decode kernels are bound by reading expert records once) and a bf16 MFMA
// loop with its operands in registers (the grouped GEMM of the prefill).
// Measurement only: no step of the layer uses them.
#include "common.h"
#include "internal.h"

namespace moe {

// Every thread reads 16-byte pieces with U loads in flight, the workgroups in
// grid-stride order (consecutive workgroups read consecutive 4 KiB). The XOR
// of all pieces decides a store that never happens for real data, which keeps
// the loads. NT: nontemporal loads (no reuse expected).
template <int U, bool NT>
__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4* __restrict__ p, uint64_t n16, uint32_t* sink) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; u++) v[u] = NT ? __builtin_nontemporal_load(p + i + u * stride) : p[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; u++) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= p[i];
  const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (r == 0x9E3779B9u) sink[blockIdx.x] = r;
}

// Each wave runs 4 independent chains of v_mfma_f32_32x32x16_bf16 on operands
// built from its lane id (2 * 32 * 32 * 16 flop per instruction).
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    a[j] = (__bf16)(1.0f + 0.001f * (float)(lane + j));
    b[j] = (__bf16)(0.5f - 0.002f * (float)(lane ^ j));
  }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; c++) acc[c] = f32x16{};
  for (int i = 0; i < iters; i++) {
#pragma unroll
    for (int c = 0; c < 4; c++) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; c++)
#pragma unroll
    for (int r = 0; r < 16; r++) s += acc[c][r];
  if (s == 1.2345678f) sink[blockIdx.x] = s;
}

hipError_t launch_probe_hbm_read(const void* buf, uint64_t nbytes, int variant, int blocks, uint32_t* sink,
                                 hipStream_t s) {
  const u32x4* p = static_cast<const u32x4*>(buf);
  const uint64_t n16 = nbytes / 16;
  const dim3 grid(blocks), block(256);
  switch (variant) {
    case 0: launch_kernel("probe_hbm_read", hbm_read_kernel<4, false>, grid, block, 0, s, p, n16, sink); break;
    case 1: launch_kernel("probe_hbm_read", hbm_read_kernel<8, false>, grid, block, 0, s, p, n16, sink); break;
    case 2: launch_kernel("probe_hbm_read", hbm_read_kernel<4, true>, grid, block, 0, s, p, n16, sink); break;
    default: launch_kernel("probe_hbm_read", hbm_read_kernel<8, true>, grid, block, 0, s, p, n16, sink); break;
  }
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int blocks, int iters, float* sink, hipStream_t s) {
  launch_kernel("probe_mfma", mfma_loop_kernel, dim3(blocks), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace moe
