// pattern.hip -- the fused step's HBM access pattern with trivial arithmetic
// (measurement only; see lioncub_probe.h).  Mirrors the step kernel's
// grid, per-thread quads, worker batches of two, nontemporal accesses and
// store order, so its rate is the ceiling of that pattern on this device.
#include "../device.hpp"
#include "../layout.hpp"

namespace lioncub {

struct PatternParams {
  void* theta;
  float* m;
  const void* g;
  int64_t d, ld;
  int32_t W;
  float beta2, omega2, lr;
};

template <int TT, int GT, int WT>
__global__ __launch_bounds__(kThreads) void k_pattern(PatternParams p) {
  constexpr int Q = kRounds;
  constexpr int WB = 2;
  const int W = WT > 0 ? WT : p.W;
  const int64_t start = static_cast<int64_t>(blockIdx.x) * kBlock;
  const int len = static_cast<int>(p.d - start < kBlock ? p.d - start : kBlock);
  int64_t j[Q];
  int nv[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int loc = kThreads * kQuad * q + kQuad * static_cast<int>(threadIdx.x);
    j[q] = start + loc;
    nv[q] = max(0, min(kQuad, len - loc));
  }
  F4 th[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q)
    if (nv[q] > 0) th[q] = ld_x4<TT>(p.theta, j[q], nv[q]);
  uint32_t cnt[Q] = {0, 0, 0, 0};
#pragma unroll 1
  for (int i0 = 0; i0 < W; i0 += WB) {
    F4 mv[WB][Q], gv[WB][Q];
#pragma unroll
    for (int b = 0; b < WB; ++b)
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        if (i0 + b < W && nv[q] > 0) {
          const int64_t idx = static_cast<int64_t>(i0 + b) * p.ld + j[q];
          mv[b][q] = ldnt_f32x4(p.m + idx, nv[q]);
          gv[b][q] = ldnt_x4<GT>(p.g, idx, nv[q]);
        }
      }
#pragma unroll
    for (int b = 0; b < WB; ++b) {
      if (i0 + b >= W) break;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        if (nv[q] == 0) continue;
        F4 mn;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          mn.v[k] = (p.beta2 * mv[b][q].v[k]) + (p.omega2 * gv[b][q].v[k]);
          cnt[q] += mn.v[k] > 0.0f ? 1u : 0u;
        }
        stnt_f32x4(p.m + static_cast<int64_t>(i0 + b) * p.ld + j[q], mn, nv[q]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    if (nv[q] == 0) continue;
    const float s = 2 * static_cast<int>(cnt[q]) > 4 * W ? p.lr : -p.lr;
#pragma unroll
    for (int k = 0; k < 4; ++k) th[q].v[k] = th[q].v[k] - s;
    stnt_x4<TT>(p.theta, j[q], th[q], nv[q]);
  }
}

// The same bytes in another arrangement: one workgroup per (block, worker)
// and the grid worker-major within panels of `panel` consecutive blocks
// (workgroup k: panel k / (panel*W), then worker, then block), so the
// workgroups resident together read one worker's rows over a contiguous
// range; theta is read and written by the workgroup of the last worker.
// No cross-worker aggregation: this measures what the arrangement streams at.
template <int TT, int GT>
__global__ __launch_bounds__(kThreads) void k_panel_pattern(PatternParams p, int panel,
                                                            int nblk) {
  const int64_t k = blockIdx.x;
  const int64_t per_panel = static_cast<int64_t>(panel) * p.W;
  const int64_t pn = k / per_panel;
  const int64_t first = pn * panel;
  const int width = static_cast<int>(nblk - first < panel ? nblk - first : panel);
  const int64_t r = k - pn * per_panel;
  const int w = static_cast<int>(r / width);
  const int64_t b = first + r % width;
  const int64_t start = b * kBlock;
  const int len = static_cast<int>(p.d - start < kBlock ? p.d - start : kBlock);
  int64_t j[kRounds];
  int nv[kRounds];
  F4 mv[kRounds], gv[kRounds];
#pragma unroll
  for (int q = 0; q < kRounds; ++q) {
    const int loc = kThreads * kQuad * q + kQuad * static_cast<int>(threadIdx.x);
    j[q] = start + loc;
    nv[q] = max(0, min(kQuad, len - loc));
    if (nv[q] > 0) {
      const int64_t idx = static_cast<int64_t>(w) * p.ld + j[q];
      mv[q] = ldnt_f32x4(p.m + idx, nv[q]);
      gv[q] = ldnt_x4<GT>(p.g, idx, nv[q]);
    }
  }
  uint32_t cnt = 0;
#pragma unroll
  for (int q = 0; q < kRounds; ++q) {
    if (nv[q] == 0) continue;
    F4 mn;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mn.v[e] = (p.beta2 * mv[q].v[e]) + (p.omega2 * gv[q].v[e]);
      cnt += mn.v[e] > 0.0f ? 1u : 0u;
    }
    stnt_f32x4(p.m + static_cast<int64_t>(w) * p.ld + j[q], mn, nv[q]);
  }
  if (w == p.W - 1) {
    const float s = 2 * static_cast<int>(cnt) > 16 ? p.lr : -p.lr;
#pragma unroll
    for (int q = 0; q < kRounds; ++q) {
      if (nv[q] == 0) continue;
      F4 th = ld_x4<TT>(p.theta, j[q], nv[q]);
#pragma unroll
      for (int e = 0; e < 4; ++e) th.v[e] = th.v[e] - s;
      stnt_x4<TT>(p.theta, j[q], th, nv[q]);
    }
  }
}

template <int TT, int GT>
static void launch_panel_t(const PatternParams& p, int panel, hipStream_t st) {
  const int64_t nblk = (p.d + kBlock - 1) / kBlock;
  const dim3 g(static_cast<unsigned>(nblk * p.W)), b(kThreads);
  hipLaunchKernelGGL((k_panel_pattern<TT, GT>), g, b, 0, st, p, panel, static_cast<int>(nblk));
}

hipError_t launch_panel_pattern(void* theta, float* m, const void* g, int64_t d, int64_t ld, int W,
                                int theta_bf16, int grad_bf16, float beta2, float lr, int panel,
                                hipStream_t st) {
  PatternParams p;
  p.theta = theta;
  p.m = m;
  p.g = g;
  p.d = d;
  p.ld = ld;
  p.W = W;
  p.beta2 = beta2;
  p.omega2 = 1.0f - beta2;
  p.lr = lr;
  if (theta_bf16) {
    if (grad_bf16) launch_panel_t<1, 1>(p, panel, st);
    else launch_panel_t<1, 0>(p, panel, st);
  } else {
    if (grad_bf16) launch_panel_t<0, 1>(p, panel, st);
    else launch_panel_t<0, 0>(p, panel, st);
  }
  return hipGetLastError();
}

template <int TT, int GT>
static void launch_pattern_t(const PatternParams& p, hipStream_t st) {
  const dim3 g(static_cast<unsigned>((p.d + kBlock - 1) / kBlock)), b(kThreads);
  switch (p.W) {
    case 4: hipLaunchKernelGGL((k_pattern<TT, GT, 4>), g, b, 0, st, p); break;
    case 8: hipLaunchKernelGGL((k_pattern<TT, GT, 8>), g, b, 0, st, p); break;
    case 16: hipLaunchKernelGGL((k_pattern<TT, GT, 16>), g, b, 0, st, p); break;
    default: hipLaunchKernelGGL((k_pattern<TT, GT, 0>), g, b, 0, st, p); break;
  }
}

hipError_t launch_pattern(void* theta, float* m, const void* g, int64_t d, int64_t ld, int W,
                          int theta_bf16, int grad_bf16, float beta2, float lr, hipStream_t st) {
  PatternParams p;
  p.theta = theta;
  p.m = m;
  p.g = g;
  p.d = d;
  p.ld = ld;
  p.W = W;
  p.beta2 = beta2;
  p.omega2 = 1.0f - beta2;
  p.lr = lr;
  if (theta_bf16) {
    if (grad_bf16) launch_pattern_t<1, 1>(p, st);
    else launch_pattern_t<1, 0>(p, st);
  } else {
    if (grad_bf16) launch_pattern_t<0, 1>(p, st);
    else launch_pattern_t<0, 0>(p, st);
  }
  return hipGetLastError();
}

}  // namespace lioncub
