// l1.hip -- mean |c| (the M1 of Eq. (1)) and standalone L1 codes, gfx950.
//
// Eq. (1) of the Lion Cub page (pith.science review, "What carries the
// argument"): Q1(x) = clamp(round((2^(n-1)-1) x / M1(x)), 2^(n-1)-1), M1 the
// mean absolute value.  The codes need the mean of the whole (worker,
// tensor) row first, so the L1 path reads m and g twice: once here, once in
// the fused step.
//
// Summation order (fixed, so that every run and the CPU reference agree to
// the bit): a workgroup of 256 lanes owns a block of 4096 elements; lane l
// sums, in fp64 from 0, ((e0+e1)+(e2+e3)) of its quads at 1024*r + 4*l for
// r = 0..3; each wave64 folds its lanes with xor-shuffles at distances 32,
// 16, .., 1 (lane q < s adds lane q+s: the halving tree; the mirrored lanes
// compute the same sums since IEEE addition commutes); the block partial is
// (w0+w1)+(w2+w3) over the four waves, combined through LDS.  The finalize
// folds each group of 256 consecutive block partials of a tensor the same
// way (partial l in lane l), then one wave gives lane l the group values l,
// l+64, ... in order, folds, and divides by the element count.  Only magnitudes are added, so
// the partials are non-negative and independent of sign.
#include "device.hpp"
#include "layout.hpp"

#pragma clang fp contract(off)

namespace lioncub {

__device__ __forceinline__ double wave_fold(double v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = v + __shfl_xor(v, s, kWave);
  return v;
}

// SRC 0: e = |x|.  SRC 1: e = |beta1*m + omega1*g| (g fp32 or bf16 per GT).
// One workgroup per block; it walks all W workers of that block, two at a
// time (16 outstanding 16-byte loads per lane).
template <int SRC, int GT>
__global__ __launch_bounds__(kThreads) void k_m1_partial(M1Params p) {
  __shared__ double sh_w[4][256];  // [wave][worker]
  const BlockEnt be = p.blk[blockIdx.x];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int W = p.W;
  constexpr int WB = 2;

#pragma unroll 1
  for (int i0 = 0; i0 < W; i0 += WB) {
    F4 a[WB][kRounds], b[WB][kRounds];
#pragma unroll
    for (int u = 0; u < WB; ++u) {
#pragma unroll
      for (int r = 0; r < kRounds; ++r) {
        const int loc = kThreads * kQuad * r + kQuad * tid;
        const int nv = max(0, min(kQuad, be.len - loc));
        const int64_t idx = static_cast<int64_t>(i0 + u) * p.ld + be.start + loc;
        if (i0 + u < W && nv > 0) {
          if (SRC == 0) {
            a[u][r] = ldnt_f32x4(p.x + idx, nv);
          } else {
            a[u][r] = ldnt_f32x4(p.m + idx, nv);
            b[u][r] = ldnt_x4<GT>(p.g, idx, nv);
          }
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) a[u][r].v[k] = b[u][r].v[k] = 0.0f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < WB; ++u) {
      if (i0 + u >= W) break;
      double acc = 0.0;
#pragma unroll
      for (int r = 0; r < kRounds; ++r) {
        double e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float c;
          if (SRC == 0) c = a[u][r].v[k];
          else c = (p.beta1 * a[u][r].v[k]) + (p.omega1 * b[u][r].v[k]);
          e[k] = fabs(static_cast<double>(c));  // zero-filled past the end
        }
        acc = acc + ((e[0] + e[1]) + (e[2] + e[3]));
      }
      acc = wave_fold(acc);
      if (lane == 0) sh_w[wave][i0 + u] = acc;
    }
  }
  __syncthreads();
  for (int i = tid; i < W; i += kThreads) {
    const double P = (sh_w[0][i] + sh_w[1][i]) + (sh_w[2][i] + sh_w[3][i]);
    p.partial[static_cast<int64_t>(i) * p.nblk + blockIdx.x] = P;
  }
}

// Group values: one workgroup per (worker, group of 256 consecutive block
// partials of one tensor); lane l takes partial l (0.0 past the tensor's last
// block), each wave folds, then (w0+w1)+(w2+w3).
__global__ __launch_bounds__(kThreads) void k_m1_group(M1Params p) {
  __shared__ double sh[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t gid = blockIdx.x;
  const int i = static_cast<int>(gid / p.ngrp), gg = static_cast<int>(gid % p.ngrp);
  const GroupEnt ge = p.grp[gg];
  double v = tid < ge.cnt ? p.partial[static_cast<int64_t>(i) * p.nblk + ge.blk + tid] : 0.0;
  v = wave_fold(v);
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  if (tid == 0) p.gval[static_cast<int64_t>(i) * p.ngrp + gg] = (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

// One wave per (worker, tensor): lane l sums group values l, l+64, ... in
// order, the wave folds, M1 = total / n, scale = Qmax / M1 (0 when M1 == 0,
// which makes every code 0).
__global__ __launch_bounds__(kThreads) void k_m1_finalize(M1Params p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (pair >= static_cast<int64_t>(p.W) * p.nT) return;
  const int i = static_cast<int>(pair / p.nT), T = static_cast<int>(pair % p.nT);
  const TensorEnt te = p.tens[T];
  const double* G = p.gval + static_cast<int64_t>(i) * p.ngrp + te.grp0;
  double acc = 0.0;
  for (int k = lane; k < te.ngrp; k += kWave) acc = acc + G[k];
  acc = wave_fold(acc);
  if (lane == 0) {
    const double M = acc / static_cast<double>(te.n);
    p.m1[pair] = M;
    if (p.m1_out) p.m1_out[pair] = M;
    if (p.qmax > 0) p.scale[pair] = M == 0.0 ? 0.0 : static_cast<double>(p.qmax) / M;
  }
}

// Eq. (1) codes of x: one workgroup per block, all workers.
__global__ __launch_bounds__(kThreads) void k_quant_codes(M1Params p, int8_t* __restrict__ codes) {
  const BlockEnt be = p.blk[blockIdx.x];
  const int tid = threadIdx.x;
  const double qm = static_cast<double>(p.qmax);
#pragma unroll 1
  for (int i = 0; i < p.W; ++i) {
    const double s = p.scale[static_cast<int64_t>(i) * p.nT + be.tensor];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int loc = kThreads * kQuad * r + kQuad * tid;
      const int nv = max(0, min(kQuad, be.len - loc));
      if (nv == 0) continue;
      const int64_t idx = static_cast<int64_t>(i) * p.ld + be.start + loc;
      const F4 x = ldnt_f32x4(p.x + idx, nv);
      uint32_t packed = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        double y = __builtin_rint(static_cast<double>(x.v[k]) * s);
        y = fmin(fmax(y, -qm), qm);
        packed |= (static_cast<uint32_t>(static_cast<int>(y)) & 0xFFu) << (8 * k);
      }
      st_b4(codes + idx, packed, nv);
    }
  }
}

hipError_t launch_m1(const M1Params& p, int src_x, int grad_bf16, hipStream_t st) {
  const dim3 blk(kThreads);
  if (src_x) hipLaunchKernelGGL((k_m1_partial<0, 0>), dim3(p.nblk), blk, 0, st, p);
  else if (grad_bf16) hipLaunchKernelGGL((k_m1_partial<1, 1>), dim3(p.nblk), blk, 0, st, p);
  else hipLaunchKernelGGL((k_m1_partial<1, 0>), dim3(p.nblk), blk, 0, st, p);
  return hipGetLastError();
}

hipError_t launch_m1_finalize(const M1Params& p, hipStream_t st) {
  const int64_t groups = static_cast<int64_t>(p.W) * p.ngrp;
  hipLaunchKernelGGL(k_m1_group, dim3(static_cast<unsigned>(groups)), dim3(kThreads), 0, st, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t pairs = static_cast<int64_t>(p.W) * p.nT;
  hipLaunchKernelGGL(k_m1_finalize, dim3(static_cast<unsigned>((pairs + 3) / 4)), dim3(kThreads),
                     0, st, p);
  return hipGetLastError();
}

hipError_t launch_quant_codes(const M1Params& p, int8_t* codes, hipStream_t st) {
  hipLaunchKernelGGL(k_quant_codes, dim3(p.nblk), dim3(kThreads), 0, st, p, codes);
  return hipGetLastError();
}

}  // namespace lioncub
