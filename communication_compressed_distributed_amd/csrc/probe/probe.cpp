// probe.cpp -- C ABI of the measurement library (include/lioncub_probe.h):
// argument checks and launches of the reference streams and the step-pattern
// probe.  Allocates nothing; no part of the method runs here.
#include "lioncub_probe.h"

#include <hip/hip_runtime.h>

#include "../layout.hpp"

namespace lioncub {
hipError_t launch_stream(int kind, const float* a, const float* b, float* c, int64_t n,
                         hipStream_t st);
hipError_t launch_pattern(void* theta, float* m, const void* g, int64_t d, int64_t ld, int W,
                          int theta_bf16, int grad_bf16, float beta2, float lr, int flags,
                          hipStream_t st);
hipError_t launch_panel_pattern(void* theta, float* m, const void* g, int64_t d, int64_t ld, int W,
                                int theta_bf16, int grad_bf16, float beta2, float lr, int panel,
                                hipStream_t st);
}  // namespace lioncub

namespace {
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int dev_status(hipError_t e) { return e == hipSuccess ? LIONCUB_OK : LIONCUB_EDEVICE; }
}  // namespace

extern "C" {

int lioncub_probe_stream(int32_t kind, const float* a, const float* b, float* c, int64_t n,
                         void* hip_stream) {
  if (kind < LIONCUB_PROBE_READ || kind > LIONCUB_PROBE_TRIAD) return LIONCUB_EINVAL;
  if (n < lioncub::kBlock || n % lioncub::kBlock != 0 || n / lioncub::kBlock > 0x7FFFFFFF)
    return LIONCUB_EINVAL;
  if (!a || !c || (kind == LIONCUB_PROBE_TRIAD && !b)) return LIONCUB_EINVAL;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return LIONCUB_EALIGN;
  return dev_status(
      lioncub::launch_stream(kind, a, b, c, n, static_cast<hipStream_t>(hip_stream)));
}

int lioncub_probe_step_pattern(void* theta, float* m, const void* g, int64_t d, int64_t ld,
                               int32_t W, int32_t theta_dtype, int32_t grad_dtype, float beta2,
                               float lr, int32_t flags, void* hip_stream) {
  if (!theta || !m || !g) return LIONCUB_EINVAL;
  if (d < 1 || ld < d || ld % 64 != 0 || (d + lioncub::kBlock - 1) / lioncub::kBlock > 0x7FFFFFFF)
    return LIONCUB_EINVAL;
  if (W < 1 || W > 255) return LIONCUB_EINVAL;
  if ((theta_dtype != LIONCUB_F32 && theta_dtype != LIONCUB_BF16) ||
      (grad_dtype != LIONCUB_F32 && grad_dtype != LIONCUB_BF16))
    return LIONCUB_EINVAL;
  if (!aligned16(theta) || !aligned16(m) || !aligned16(g)) return LIONCUB_EALIGN;
  const int32_t shaping = LIONCUB_PROBE_CAP_MASK | LIONCUB_PROBE_DRAIN_MASK;
  if (flags & ~(LIONCUB_PROBE_CACHED | LIONCUB_PROBE_MASKED | shaping)) return LIONCUB_EINVAL;
  if ((flags & shaping) && (flags & (LIONCUB_PROBE_CACHED | LIONCUB_PROBE_MASKED)))
    return LIONCUB_EINVAL;
  if ((flags & LIONCUB_PROBE_CAP_MASK) && (flags & LIONCUB_PROBE_DRAIN_MASK)) return LIONCUB_EINVAL;
  return dev_status(lioncub::launch_pattern(theta, m, g, d, ld, W, theta_dtype == LIONCUB_BF16,
                                            grad_dtype == LIONCUB_BF16, beta2, lr, flags,
                                            static_cast<hipStream_t>(hip_stream)));
}

int lioncub_probe_panel_pattern(void* theta, float* m, const void* g, int64_t d, int64_t ld,
                                int32_t W, int32_t theta_dtype, int32_t grad_dtype, float beta2,
                                float lr, int32_t panel_blocks, void* hip_stream) {
  if (!theta || !m || !g) return LIONCUB_EINVAL;
  if (d < 1 || ld < d || ld % 64 != 0) return LIONCUB_EINVAL;
  if (W < 1 || W > 255 || panel_blocks < 1) return LIONCUB_EINVAL;
  // one workgroup of 256 work-items per (block, worker): the grid's
  // work-item count must fit 32 bits
  if ((d + lioncub::kBlock - 1) / lioncub::kBlock * W * lioncub::kThreads > 0xFFFFFFFFll)
    return LIONCUB_EINVAL;
  if ((theta_dtype != LIONCUB_F32 && theta_dtype != LIONCUB_BF16) ||
      (grad_dtype != LIONCUB_F32 && grad_dtype != LIONCUB_BF16))
    return LIONCUB_EINVAL;
  if (!aligned16(theta) || !aligned16(m) || !aligned16(g)) return LIONCUB_EALIGN;
  return dev_status(lioncub::launch_panel_pattern(
      theta, m, g, d, ld, W, theta_dtype == LIONCUB_BF16, grad_dtype == LIONCUB_BF16, beta2, lr,
      panel_blocks, static_cast<hipStream_t>(hip_stream)));
}

}  // extern "C"
