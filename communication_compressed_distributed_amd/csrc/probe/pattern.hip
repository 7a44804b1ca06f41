// pattern.hip -- the fused step's HBM access pattern with trivial arithmetic
// (measurement only; see lioncub_probe.h).  Mirrors the step kernel's
// grid, per-thread quads, worker batches of two, nontemporal accesses and
// store order, so its rate is the ceiling of that pattern on this device.
#include "../device.hpp"
#include "../layout.hpp"

namespace lioncub {

// Wait until at most N vector-memory operations of this wave are still
// outstanding (s_waitcnt vmcnt(N), the other counters left unconstrained).
// gfx9 encoding of the immediate: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

struct PatternParams {
  void* theta;
  float* m;
  const void* g;
  int64_t d, ld;
  int32_t W;
  float beta2, omega2, lr;
};

// NT: nontemporal loads and stores (as the step kernels use) or plain ones,
// which let a working set smaller than the last-level cache stay there from
// one call to the next.
// FULL: a whole 4096-element block, no per-lane predicates (as the step
// kernel's full-block path); otherwise the block's ragged tail.
// CAP > 0: at most CAP vector-memory operations of a wave in flight while
// a batch's loads are issued (an explicit wait before each load).
// DRAIN 1: the wave waits for all its memory operations (the previous
// batch's stores included) before a batch's loads; DRAIN 2: before every
// quad's pair of loads; DRAIN 3: before every quad's pair of loads and
// before every store (memory operations of a wave one after another).
template <int TT, int GT, int WT, bool NT, bool FULL, int CAP = 0, int DRAIN = 0>
__device__ __forceinline__ void pattern_block(const PatternParams& p, int64_t start, int len) {
  constexpr int Q = kRounds;
  constexpr int WB = 2;
  const int W = WT > 0 ? WT : p.W;
  int64_t j[Q];
  int nv[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int loc = kThreads * kQuad * q + kQuad * static_cast<int>(threadIdx.x);
    j[q] = start + loc;
    nv[q] = FULL ? kQuad : max(0, min(kQuad, len - loc));
  }
  F4 th[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q)
    if (nv[q] > 0) th[q] = ld_x4<TT>(p.theta, j[q], nv[q]);
  uint32_t cnt[Q] = {0, 0, 0, 0};
#pragma unroll 1
  for (int i0 = 0; i0 < W; i0 += WB) {
    F4 mv[WB][Q], gv[WB][Q];
    if constexpr (DRAIN == 1) vm_wait<0>();
#pragma unroll
    for (int b = 0; b < WB; ++b)
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        if (((WT > 0 && WT % WB == 0) || i0 + b < W) && (FULL || nv[q] > 0)) {
          const int64_t idx = static_cast<int64_t>(i0 + b) * p.ld + j[q];
          if constexpr (DRAIN >= 2) vm_wait<0>();
          if constexpr (CAP > 0) vm_wait<CAP - 1>();
          mv[b][q] = NT ? ldnt_f32x4(p.m + idx, nv[q]) : ld_f32x4(p.m + idx, nv[q]);
          if constexpr (CAP > 0) vm_wait<CAP - 1>();
          gv[b][q] = NT ? ldnt_x4<GT>(p.g, idx, nv[q]) : ld_x4<GT>(p.g, idx, nv[q]);
        }
      }
#pragma unroll
    for (int b = 0; b < WB; ++b) {
      if (!(WT > 0 && WT % WB == 0) && i0 + b >= W) break;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        if (!FULL && nv[q] == 0) continue;
        F4 mn;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          mn.v[k] = (p.beta2 * mv[b][q].v[k]) + (p.omega2 * gv[b][q].v[k]);
          cnt[q] += mn.v[k] > 0.0f ? 1u : 0u;
        }
        if constexpr (DRAIN == 3) vm_wait<0>();
        if (NT) stnt_f32x4(p.m + static_cast<int64_t>(i0 + b) * p.ld + j[q], mn, nv[q]);
        else st_f32x4(p.m + static_cast<int64_t>(i0 + b) * p.ld + j[q], mn, nv[q]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    if (!FULL && nv[q] == 0) continue;
    const float s = 2 * static_cast<int>(cnt[q]) > 4 * W ? p.lr : -p.lr;
#pragma unroll
    for (int k = 0; k < 4; ++k) th[q].v[k] = th[q].v[k] - s;
    if (NT) stnt_x4<TT>(p.theta, j[q], th[q], nv[q]);
    else st_x4<TT>(p.theta, j[q], th[q], nv[q]);
  }
}

// MASKED: every block takes the per-lane predicated path of a ragged block
// (a second arrangement of the same bytes, with more instructions between a
// batch's loads and its stores).
template <int TT, int GT, int WT, bool NT, bool MASKED, int CAP, int DRAIN>
__global__ __launch_bounds__(kThreads) void k_pattern(PatternParams p) {
  const int64_t start = static_cast<int64_t>(blockIdx.x) * kBlock;
  const int len = static_cast<int>(p.d - start < kBlock ? p.d - start : kBlock);
  if (!MASKED && len == kBlock) pattern_block<TT, GT, WT, NT, true, CAP, DRAIN>(p, start, len);
  else pattern_block<TT, GT, WT, NT, false>(p, start, len);
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

template <int TT, int GT, bool NT, bool MASKED, int CAP, int DRAIN>
static void launch_pattern_t(const PatternParams& p, hipStream_t st) {
  const dim3 g(static_cast<unsigned>((p.d + kBlock - 1) / kBlock)), b(kThreads);
  switch (p.W) {
    case 4: hipLaunchKernelGGL((k_pattern<TT, GT, 4, NT, MASKED, CAP, DRAIN>), g, b, 0, st, p); break;
    case 8: hipLaunchKernelGGL((k_pattern<TT, GT, 8, NT, MASKED, CAP, DRAIN>), g, b, 0, st, p); break;
    case 16: hipLaunchKernelGGL((k_pattern<TT, GT, 16, NT, MASKED, CAP, DRAIN>), g, b, 0, st, p); break;
    default: hipLaunchKernelGGL((k_pattern<TT, GT, 0, NT, MASKED, CAP, DRAIN>), g, b, 0, st, p); break;
  }
}

template <bool NT, bool MASKED, int CAP, int DRAIN = 0>
static void launch_pattern_d(const PatternParams& p, int theta_bf16, int grad_bf16,
                             hipStream_t st) {
  if (theta_bf16) {
    if (grad_bf16) launch_pattern_t<1, 1, NT, MASKED, CAP, DRAIN>(p, st);
    else launch_pattern_t<1, 0, NT, MASKED, CAP, DRAIN>(p, st);
  } else {
    if (grad_bf16) launch_pattern_t<0, 1, NT, MASKED, CAP, DRAIN>(p, st);
    else launch_pattern_t<0, 0, NT, MASKED, CAP, DRAIN>(p, st);
  }
}

hipError_t launch_pattern(void* theta, float* m, const void* g, int64_t d, int64_t ld, int W,
                          int theta_bf16, int grad_bf16, float beta2, float lr, int flags,
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
  const bool cached = flags & 1, masked = flags & 2;
  const int cap = (flags >> 2) & 3;  // 0: no cap; 1, 2, 3: 2, 4, 8 loads in flight
  const int drain = (flags >> 4) & 3;
  if (drain == 1) {
    launch_pattern_d<true, false, 0, 1>(p, theta_bf16, grad_bf16, st);
  } else if (drain == 2) {
    launch_pattern_d<true, false, 0, 2>(p, theta_bf16, grad_bf16, st);
  } else if (drain == 3) {
    launch_pattern_d<true, false, 0, 3>(p, theta_bf16, grad_bf16, st);
  } else if (cached) {
    if (masked) launch_pattern_d<false, true, 0>(p, theta_bf16, grad_bf16, st);
    else launch_pattern_d<false, false, 0>(p, theta_bf16, grad_bf16, st);
  } else if (masked) {
    launch_pattern_d<true, true, 0>(p, theta_bf16, grad_bf16, st);
  } else if (cap == 1) {
    launch_pattern_d<true, false, 2>(p, theta_bf16, grad_bf16, st);
  } else if (cap == 2) {
    launch_pattern_d<true, false, 4>(p, theta_bf16, grad_bf16, st);
  } else if (cap == 3) {
    launch_pattern_d<true, false, 8>(p, theta_bf16, grad_bf16, st);
  } else {
    launch_pattern_d<true, false, 0>(p, theta_bf16, grad_bf16, st);
  }
  return hipGetLastError();
}

}  // namespace lioncub
