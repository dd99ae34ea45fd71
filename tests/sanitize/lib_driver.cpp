// Runs the host-only entry points of libmoe_mi355x (global scales from
// weight_scale_2) and the argument checks of every entry point that returns
// before any HIP call, for a build whose host code has AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitizers.py). No GPU is touched:
// the pointers handed to the checks are never dereferenced.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/moe_mi355x.h"

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); \
      return 1;                                                        \
    }                                                                  \
  } while (0)

int main() {
  // g from weight_scale_2: subnormal, tiny, ordinary, largest finite-g values
  std::vector<float> ws2;
  for (int i = 1; i < 4000; i++) ws2.push_back(std::ldexp(1.0f + 0.000731f * (float)i, -140 + (i % 230)));
  ws2.push_back(1.4e-45f);
  ws2.push_back(3.4028234e38f / 2688.0f);
  std::vector<float> g(ws2.size());
  std::vector<uint8_t> inexact(ws2.size());
  EXPECT(moe_nvfp4_global_from_ws2(ws2.data(), (int64_t)ws2.size(), g.data(), inexact.data()) == MOE_OK);
  float bad = -1.0f;
  EXPECT(moe_nvfp4_global_from_ws2(&bad, 1, g.data(), nullptr) == MOE_EINVAL);
  EXPECT(moe_nvfp4_global_from_ws2(nullptr, 3, g.data(), nullptr) == MOE_EINVAL);
  EXPECT(std::strlen(moe_last_error()) > 0);

  // sizes and descriptors
  EXPECT(moe_nvfp4_record_bytes(5120, 2560) == 22118412u);
  EXPECT(moe_nvfp4_record_stride(5120, 2560) == 22122496u);
  EXPECT(moe_nvfp4_record_bytes(24, 16) == 0);
  void* fake = reinterpret_cast<void*>(uintptr_t(1) << 40);
  moe_nvfp4_bank b;
  EXPECT(moe_nvfp4_bank_init(&b, fake, 256, 128, 16) == MOE_OK);
  EXPECT(moe_nvfp4_bank_init(&b, fake, 256, 120, 16) == MOE_ESHAPE);
  EXPECT(moe_nvfp4_bank_init(&b, fake, 256, 128, 16) == MOE_OK);
  const size_t ws = moe_nvfp4_workspace_bytes(4, 2, 256, 128, 16);
  EXPECT(ws > 0 && moe_sort_workspace_bytes(4096, 8, 256) > 0);

  // argument checks that return before anything is enqueued
  const uint16_t* x = static_cast<const uint16_t*>(fake);
  void* y = fake;
  EXPECT(moe_nvfp4_forward(&b, x, 4, nullptr, nullptr, 0, nullptr, y, 0, fake, ws, nullptr) == MOE_ESHAPE);
  EXPECT(moe_nvfp4_forward(&b, x, 4, static_cast<int32_t*>(fake), static_cast<float*>(fake), 2, nullptr, y, 0,
                           fake, ws - 1, nullptr) == MOE_EWORKSPACE);
  EXPECT(moe_nvfp4_forward(&b, x, 4, static_cast<int32_t*>(fake), static_cast<float*>(fake), 2, nullptr, y, 7u,
                           fake, ws, nullptr) == MOE_EINVAL);
  EXPECT(moe_nvfp4_layer(&b, x, nullptr, 1, 2, nullptr, nullptr, nullptr, nullptr, y, 0, fake, ws, nullptr) ==
         MOE_EINVAL);
  EXPECT(moe_route_topk(x, nullptr, static_cast<float*>(fake), 4, 256, 16, 2, static_cast<int32_t*>(fake),
                        static_cast<float*>(fake), nullptr) == MOE_EINVAL);
  EXPECT(moe_route_topk(nullptr, nullptr, static_cast<float*>(fake), 4, 256, 16, 17, static_cast<int32_t*>(fake),
                        static_cast<float*>(fake), nullptr) == MOE_ESHAPE);
  EXPECT(moe_sort_pairs(nullptr, 4, 2, 16, nullptr, nullptr, nullptr) == MOE_EINVAL);
  EXPECT(affine8_g64_linear(x, static_cast<const uint32_t*>(fake), x, x, 4, 100, 8, static_cast<uint16_t*>(y),
                            nullptr) == MOE_ESHAPE);
  EXPECT(moe_rmsnorm(x, 4, 256, -1.0f, static_cast<uint16_t*>(y), nullptr) == MOE_EINVAL);
  EXPECT(moe_nvfp4_dequant(&b, 16, 0, static_cast<float*>(fake), nullptr, nullptr) == MOE_EINVAL);
  EXPECT(moe_status_read(nullptr, nullptr, nullptr) == MOE_EINVAL);
  EXPECT(moe_status_clear(static_cast<uint8_t*>(fake) + 8, nullptr) == MOE_EALIGN);
  moe_vq_bank vb;
  EXPECT(moe_vq_bank_init(&vb, fake, fake, 256, 96, 4) == MOE_ESHAPE);
  EXPECT(moe_vq_record_bytes(5120, 2560) > 0);
  EXPECT(moe_probe_hbm_read(fake, 24, 0, 16, static_cast<uint32_t*>(fake), nullptr) == MOE_EALIGN);
  EXPECT(moe_probe_mfma_bf16(0, 1, static_cast<float*>(fake), nullptr) == MOE_EINVAL);
  std::printf("library driver: ok (%zu scales, %d inexact)\n", ws2.size(),
              (int)std::count_if(inexact.begin(), inexact.end(), [](uint8_t v) { return v != 0; }));
  return 0;
}
