// l1.hip -- mean |c| (the M1 of Eq. (1)) or max |c| (the max-norm
// baseline), and standalone codes of both quantisers, gfx950.
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
//
// The max-norm baseline (MX = true) runs the same tree with max in place of
// the sum and no division: a maximum is exact in any order.  Its codes round
// stochastically (sr_code): element j of worker i at step t takes 32 bits of
// SplitMix64 output number (t*W + i)*d + (j with its lowest bit cleared), the
// low half for even j and the high half for odd j.
#include "device.hpp"
#include "layout.hpp"

#pragma clang fp contract(off)

namespace lioncub {

// The tree's combining step: a sum, or for the max-norm a maximum.
template <bool MX>
__device__ __forceinline__ double red(double a, double b) {
  if constexpr (MX) return fmax(a, b);
  else return a + b;
}

template <bool MX = false>
__device__ __forceinline__ double wave_fold(double v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = red<MX>(v, __shfl_xor(v, s, kWave));
  return v;
}

// Lane sum of one worker over the block: acc = sum over the 4 rounds of
// ((e0+e1)+(e2+e3)), e = |c| in fp64 (zero past the end of the tensor).
template <int SRC, int GT, bool MX>
__device__ __forceinline__ double lane_sum(const M1Params& p, const F4 (&a)[kRounds],
                                           const F4 (&b)[kRounds]) {
  double acc = 0.0;
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    double e[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float c;
      if (SRC == 0) c = a[r].v[k];
      else c = (p.beta1 * a[r].v[k]) + (p.omega1 * b[r].v[k]);
      e[k] = fabs(static_cast<double>(c));
    }
    acc = red<MX>(acc, red<MX>(red<MX>(e[0], e[1]), red<MX>(e[2], e[3])));
  }
  return acc;
}

// Loads of workers i0 .. i0+WB-1 for the thread's 4 quads (zeros for absent
// workers and elements).
template <int SRC, int GT, bool FULL, int WB>
__device__ __forceinline__ void m1_load(const M1Params& p, const BlockEnt& be, int i0, int W,
                                        const int (&nv)[kRounds], F4 (&a)[WB][kRounds],
                                        F4 (&b)[WB][kRounds]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < WB; ++u) {
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int64_t idx = static_cast<int64_t>(i0 + u) * p.ld + be.start +
                          (kThreads * kQuad * r + kQuad * tid);
      if (FULL && i0 + u < W) {
        if (SRC == 0) {
          a[u][r] = ldnt_f32x4(p.x + idx, kQuad);
        } else {
          a[u][r] = ldnt_f32x4(p.m + idx, kQuad);
          b[u][r] = ldnt_x4<GT>(p.g, idx, kQuad);
        }
      } else if (!FULL && i0 + u < W) {
        const int n = nv[r];
        if (SRC == 0) {
          a[u][r] = ldm_f32x4(p.x + idx, n);
        } else {
          a[u][r] = ldm_f32x4(p.m + idx, n);
          b[u][r] = ldm_x4<GT>(p.g, idx, n);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) a[u][r].v[k] = b[u][r].v[k] = 0.0f;
      }
    }
  }
}

// Fold NW (a power of two, 4..16) workers' lane sums at once.  A reduce-
// scatter over the halving tree: at distance s, lane q keeps half of its
// workers (the lower half if bit s of q is clear) and adds the partner's
// value of the same worker, so each worker is still summed exactly as the
// halving tree a[q] + a[q+s] (the mirrored lanes add the same pair, and IEEE
// addition commutes).  After log2(NW) such steps each lane holds one worker;
// the remaining distances fold it like wave_fold.  17 shuffles instead of 96
// for 16 workers.  Returns the total of worker wk(lane) in `out`.
template <int NW, bool MX>
__device__ __forceinline__ double fold_many(double (&v)[NW], int* wk) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  int n = NW;
  int s = 32;
#pragma unroll
  for (int step = 0; (1 << step) < NW; ++step) {
    const int h = n >> 1;
    const bool upper = (lane & s) != 0;
#pragma unroll
    for (int k = 0; k < NW / 2; ++k) {
      if (k >= h) break;
      const double send = upper ? v[k] : v[k + h];
      const double keep = upper ? v[k + h] : v[k];
      const double recv = __shfl_xor(send, s, kWave);
      v[k] = red<MX>(keep, recv);
    }
    if (upper) base += h;
    n = h;
    s >>= 1;
  }
  double r = v[0];
  for (; s >= 1; s >>= 1) r = red<MX>(r, __shfl_xor(r, s, kWave));
  *wk = base;
  return r;
}

// SRC 0: e = |x|.  SRC 1: e = |beta1*m + omega1*g| (g fp32 or bf16 per GT).
// One workgroup per block; it walks all W workers of that block, two at a
// time (16 outstanding 16-byte loads per lane).  FULL blocks take straight
// vector loads with no per-lane predicates; the ragged last block of a
// tensor takes the masked path.  With WT = 4, 8 or 16 workers the lane sums
// stay in registers and are folded together at the end (fold_many).
template <int SRC, int GT, bool FULL, int WT, bool MX>
__device__ __forceinline__ void m1_block(const M1Params& p, const BlockEnt& be,
                                         double (*sh_w)[256]) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int W = WT > 0 ? WT : p.W;
  constexpr int WB = 2;  // workers per batch on the fixed-W path
  int nv[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r)
    nv[r] = FULL ? kQuad : max(0, min(kQuad, be.len - (kThreads * kQuad * r + kQuad * tid)));

  if constexpr (WT > 0) {
    // fully unrolled over the fixed worker count: every index is static
    double acc[WT];
#pragma unroll
    for (int i0 = 0; i0 < WT; i0 += WB) {
      F4 a[WB][kRounds], b[WB][kRounds];
      m1_load<SRC, GT, FULL, WB>(p, be, i0, W, nv, a, b);
#pragma unroll
      for (int u = 0; u < WB; ++u) acc[i0 + u] = lane_sum<SRC, GT, MX>(p, a[u], b[u]);
    }
    int wk = 0;
    const double tot = fold_many<WT, MX>(acc, &wk);
    if ((lane & (64 / WT - 1)) == 0) sh_w[wave][wk] = tot;
  } else {
    // generic W or a ragged block: one worker at a time, folded at once
#pragma unroll 1
    for (int i = 0; i < W; ++i) {
      F4 a[1][kRounds], b[1][kRounds];
      m1_load<SRC, GT, FULL, 1>(p, be, i, W, nv, a, b);
      const double tot = wave_fold<MX>(lane_sum<SRC, GT, MX>(p, a[0], b[0]));
      if (lane == 0) sh_w[wave][i] = tot;
    }
  }
}

template <int SRC, int GT, int WT, bool MX>
__global__ __launch_bounds__(kThreads) void k_m1_partial(M1Params p) {
  __shared__ double sh_w[4][256];  // [wave][worker]
  const BlockEnt be = block_of(p.blk, p.flat, p.d);
  const int tid = threadIdx.x;
  if (be.len == kBlock) m1_block<SRC, GT, true, WT, MX>(p, be, sh_w);
  else m1_block<SRC, GT, false, 0, MX>(p, be, sh_w);
  __syncthreads();
  for (int i = tid; i < p.W; i += kThreads) {
    const double P = red<MX>(red<MX>(sh_w[0][i], sh_w[1][i]), red<MX>(sh_w[2][i], sh_w[3][i]));
    // one run per block, nontemporal (same-process A/B on 350M x 16:
    // 6.59-6.63 ms against 6.65-6.67 with plain stores)
    __builtin_nontemporal_store(P, p.partial + static_cast<int64_t>(blockIdx.x) * p.W + i);
  }
}

// Group values: one workgroup per group of 256 consecutive block partials
// of one tensor, for all W workers; for worker i, lane l takes partial l of
// the group (0.0 past the tensor's last block), each wave folds, then
// (w0+w1)+(w2+w3).  Thread l reads block l's W partials, one contiguous run
// of the block-major array, so each partial is fetched from HBM once.
template <bool MX>
__global__ __launch_bounds__(kThreads) void k_m1_group(M1Params p) {
  __shared__ double sh[4][256];  // [wave][worker]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int gg = blockIdx.x;
  const GroupEnt ge = p.grp[gg];
  const double* __restrict__ row = p.partial + static_cast<int64_t>(ge.blk + tid) * p.W;
  const bool have = tid < ge.cnt;
#pragma unroll 1
  for (int i0 = 0; i0 < p.W; i0 += 4) {
    double v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = (have && i0 + u < p.W) ? row[i0 + u] : 0.0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (i0 + u >= p.W) break;  // uniform
      const double f = wave_fold<MX>(v[u]);
      if (lane == 0) sh[wave][i0 + u] = f;
    }
  }
  __syncthreads();
  for (int i = tid; i < p.W; i += kThreads)
    p.gval[static_cast<int64_t>(i) * p.ngrp + gg] =
        red<MX>(red<MX>(sh[0][i], sh[1][i]), red<MX>(sh[2][i], sh[3][i]));
}

// One wave per (worker, tensor): lane l sums group values l, l+64, ... in
// order, the wave folds, M1 = total / n, scale = Qmax / M1 (0 when M1 == 0,
// which makes every code 0).  Max-norm: the maximum, not divided.
template <bool MX>
__global__ __launch_bounds__(kThreads) void k_m1_finalize(M1Params p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (pair >= static_cast<int64_t>(p.W) * p.nT) return;
  const int i = static_cast<int>(pair / p.nT), T = static_cast<int>(pair % p.nT);
  const TensorEnt te = p.tens[T];
  const double* G = p.gval + static_cast<int64_t>(i) * p.ngrp + te.grp0;
  double acc = 0.0;
  for (int k = lane; k < te.ngrp; k += kWave) acc = red<MX>(acc, G[k]);
  acc = wave_fold<MX>(acc);
  if (lane == 0) {
    const double M = MX ? acc : acc / static_cast<double>(te.n);
    p.m1[pair] = M;
    if (p.m1_out) p.m1_out[pair] = M;
    if (p.qmax > 0) p.scale[pair] = M == 0.0 ? 0.0 : static_cast<double>(p.qmax) / M;
  }
}

// Eq. (1) codes of x: one workgroup per (block, worker), grid (nblk, W);
// the thread's four quads are loaded before any code is formed, and the
// codes leave through nontemporal stores.  (Measured on MI355X, 350M x 16:
// 4.6 ms, against 4.9 ms for one workgroup per block walking the workers.)
__global__ __launch_bounds__(kThreads) void k_quant_codes(M1Params p, int8_t* __restrict__ codes) {
  const BlockEnt be = block_of(p.blk, p.flat, p.d);
  const int tid = threadIdx.x;
  const int i = blockIdx.y;
  const int qm = p.qmax;
  const double s = p.scale[static_cast<int64_t>(i) * p.nT + be.tensor];
  const int64_t row = static_cast<int64_t>(i) * p.ld + be.start;
  F4 x[kRounds];
  int nv[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int loc = kThreads * kQuad * r + kQuad * tid;
    nv[r] = max(0, min(kQuad, be.len - loc));
    if (nv[r] == kQuad) x[r] = ldnt_f32x4(p.x + row + loc, kQuad);
    else x[r] = ldm_f32x4(p.x + row + loc, nv[r]);
  }
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    if (nv[r] == 0) continue;
    const int loc = kThreads * kQuad * r + kQuad * tid;
    uint32_t packed = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      double y = __builtin_rint(static_cast<double>(x[r].v[k]) * s);
      y = fmin(fmax(y, -qm), qm);
      packed |= (static_cast<uint32_t>(static_cast<int>(y)) & 0xFFu) << (8 * k);
    }
    stnt_b4(codes + row + loc, packed, nv[r]);
  }
}

// Stochastic max-norm codes: one workgroup per block walking all workers,
// quad by quad.  This kernel is bound by the generator's 64-bit arithmetic,
// not by HBM, and the long-lived workgroups keep the loads of the next quads
// in flight behind it (the one-worker-per-workgroup form of the L1 kernel
// above measured 7.0 ms here against 6.4).
__global__ __launch_bounds__(kThreads) void k_quant_codes_sr(M1Params p, int8_t* __restrict__ codes) {
  const BlockEnt be = block_of(p.blk, p.flat, p.d);
  const int tid = threadIdx.x;
  const int qm = p.qmax;
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
      // elements j, j+1 (j = be.start + loc + 0 or 2, even) share output
      // number (t*W + i)*d + j of the stream
      const uint64_t z0 = p.seed + (static_cast<uint64_t>(
          (static_cast<uint64_t>(p.t) * static_cast<uint64_t>(p.W) + static_cast<uint64_t>(i)) *
              static_cast<uint64_t>(p.d) + static_cast<uint64_t>(be.start + loc)) + 1u) * kGamma;
      const uint64_t r01 = mix64(z0), r23 = mix64(z0 + 2u * kGamma);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int qc = sr_code(x.v[k], s, qm, quad_bits(r01, r23, k));
        packed |= (static_cast<uint32_t>(qc) & 0xFFu) << (8 * k);
      }
      stnt_b4(codes + idx, packed, nv);
    }
  }
}

template <int SRC, int GT, bool MX>
static void launch_m1_t(const M1Params& p, hipStream_t st) {
  const dim3 g(p.nblk), b(kThreads);
  switch (p.W) {
    case 4: hipLaunchKernelGGL((k_m1_partial<SRC, GT, 4, MX>), g, b, 0, st, p); break;
    case 8: hipLaunchKernelGGL((k_m1_partial<SRC, GT, 8, MX>), g, b, 0, st, p); break;
    case 16: hipLaunchKernelGGL((k_m1_partial<SRC, GT, 16, MX>), g, b, 0, st, p); break;
    default: hipLaunchKernelGGL((k_m1_partial<SRC, GT, 0, MX>), g, b, 0, st, p); break;
  }
}

template <bool MX>
static void launch_m1_m(const M1Params& p, int src_x, int grad_bf16, hipStream_t st) {
  if (src_x) launch_m1_t<0, 0, MX>(p, st);
  else if (grad_bf16) launch_m1_t<1, 1, MX>(p, st);
  else launch_m1_t<1, 0, MX>(p, st);
}

hipError_t launch_m1(const M1Params& p, int src_x, int grad_bf16, int maxnorm, hipStream_t st) {
  if (maxnorm) launch_m1_m<true>(p, src_x, grad_bf16, st);
  else launch_m1_m<false>(p, src_x, grad_bf16, st);
  return hipGetLastError();
}

hipError_t launch_m1_finalize(const M1Params& p, int maxnorm, hipStream_t st) {
  const dim3 gg(static_cast<unsigned>(p.ngrp)), b(kThreads);
  if (maxnorm) hipLaunchKernelGGL(k_m1_group<true>, gg, b, 0, st, p);
  else hipLaunchKernelGGL(k_m1_group<false>, gg, b, 0, st, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t pairs = static_cast<int64_t>(p.W) * p.nT;
  const dim3 gf(static_cast<unsigned>((pairs + 3) / 4));
  if (maxnorm) hipLaunchKernelGGL(k_m1_finalize<true>, gf, b, 0, st, p);
  else hipLaunchKernelGGL(k_m1_finalize<false>, gf, b, 0, st, p);
  return hipGetLastError();
}

hipError_t launch_quant_codes(const M1Params& p, int8_t* codes, int maxnorm, hipStream_t st) {
  if (maxnorm) {
    hipLaunchKernelGGL(k_quant_codes_sr, dim3(static_cast<unsigned>(p.nblk)), dim3(kThreads), 0,
                       st, p, codes);
  } else {
    const dim3 g(static_cast<unsigned>(p.nblk), static_cast<unsigned>(p.W));
    hipLaunchKernelGGL(k_quant_codes, g, dim3(kThreads), 0, st, p, codes);
  }
  return hipGetLastError();
}

}  // namespace lioncub
