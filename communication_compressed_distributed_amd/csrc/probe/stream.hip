// stream.hip -- STREAM-style reference kernels of the measurement library
// (lioncub_probe_stream): what plain read-only, copy and triad streams
// achieve on this device, reported beside the published 8 TB/s peak.  Same
// shape as the step library's kernels: 256 threads, 4096 elements per
// workgroup, four nontemporal 16-byte quads per lane.
#include "../device.hpp"
#include "../layout.hpp"

namespace lioncub {

// Sum of the workgroup's elements, stored only if it equals an impossible
// sentinel, so the loads cannot be removed and nothing is written.
__global__ __launch_bounds__(kThreads) void k_stream_read(const float* __restrict__ a,
                                                          float* __restrict__ sink) {
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * kBlock + kQuad * threadIdx.x;
  F4 x[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) x[r] = ldnt_f32x4(a + j0 + kThreads * kQuad * r, kQuad);
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < kRounds; ++r) s += (x[r].v[0] + x[r].v[1]) + (x[r].v[2] + x[r].v[3]);
  if (s == -1234.5f) sink[0] = s;
}

__global__ __launch_bounds__(kThreads) void k_stream_copy(const float* __restrict__ a,
                                                          float* __restrict__ c) {
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * kBlock + kQuad * threadIdx.x;
  F4 x[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) x[r] = ldnt_f32x4(a + j0 + kThreads * kQuad * r, kQuad);
#pragma unroll
  for (int r = 0; r < kRounds; ++r) stnt_f32x4(c + j0 + kThreads * kQuad * r, x[r], kQuad);
}

__global__ __launch_bounds__(kThreads) void k_stream_triad(const float* __restrict__ a,
                                                           const float* __restrict__ b,
                                                           float* __restrict__ c, float s) {
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * kBlock + kQuad * threadIdx.x;
  F4 x[kRounds], y[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    x[r] = ldnt_f32x4(a + j0 + kThreads * kQuad * r, kQuad);
    y[r] = ldnt_f32x4(b + j0 + kThreads * kQuad * r, kQuad);
  }
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    F4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o.v[k] = x[r].v[k] + s * y[r].v[k];
    stnt_f32x4(c + j0 + kThreads * kQuad * r, o, kQuad);
  }
}

// n: elements, a multiple of kBlock (checked by the caller).
hipError_t launch_stream(int kind, const float* a, const float* b, float* c, int64_t n,
                         hipStream_t st) {
  const dim3 g(static_cast<unsigned>(n / kBlock)), t(kThreads);
  if (kind == 0) hipLaunchKernelGGL(k_stream_read, g, t, 0, st, a, c);
  else if (kind == 1) hipLaunchKernelGGL(k_stream_copy, g, t, 0, st, a, c);
  else hipLaunchKernelGGL(k_stream_triad, g, t, 0, st, a, b, c, 0.5f);
  return hipGetLastError();
}

}  // namespace lioncub
