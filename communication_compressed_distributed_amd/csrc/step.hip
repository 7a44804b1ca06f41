// step.hip -- fused Lion Cub step kernels for gfx950.
//
// One workgroup (256 threads, 4 wave64) per block of 4096 elements of one
// tensor; each thread owns one quad (4 consecutive elements) per round, 4
// rounds.  For its quad a thread walks the W workers: loads m_i and g_i
// (coalesced 16-byte / 8-byte vector loads), forms c_i = beta1*m_i +
// omega1*g_i, compresses it (sign bit, or Eq. (1) code), accumulates the
// aggregate (vote count, or integer sum) and immediately writes the new
// momentum m_i' = beta2*m_i + omega2*g_i -- m_i' does not depend on the
// global sign, so each worker's state is touched exactly once.  After the
// last worker it applies the global sign to theta.  On averaging steps of a
// designated tensor the new momenta are summed in worker order instead and
// their mean is written to every worker.
//
// Method: "Lion Cub: Minimizing Communication Overhead in Distributed Lion"
// (pith.science review, "What carries the argument": c_{i,t}, 0/1 packing
// with parity zeros, Eq. (1), the quantised sum and global sign; selective
// momentum synchronisation of the embedding and output layers), and the
// D-Lion summary page ("Approach": per-worker momentum, majority vote).
// The max-norm baseline (kAggLinf) is the L1 path with the codes rounded
// stochastically against max |c|: the quantiser the Lion Cub page compares
// Eq. (1) with (Figure 4).
//
// Workers are processed in batches of WB: the 2*WB*4 loads of a batch (m and
// g of WB workers for the thread's 4 quads) are issued before any use, so
// every lane keeps 16 vector loads in flight at WB = 2; the batch's momentum
// stores follow.  HBM-bound: per element it moves W*(4 + s_g + 4) + 2*s_theta
// bytes on every path -- nothing else (the quantised paths' norm pass is a
// separate kernel).

#include "device.hpp"
#include "layout.hpp"

#pragma clang fp contract(off)

namespace lioncub {

// Sum the workgroup's diagnostic counters and take its largest variance;
// thread 0 writes them to the block's slots (no atomics: a second kernel
// folds the blocks of each tensor in order).
__device__ __forceinline__ void block_stats(const StepParams& p, unsigned tie, unsigned match,
                                         unsigned flip, unsigned zero, double var) {
  __shared__ unsigned sh_c[4][4];
  __shared__ double sh_v[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    tie += __shfl_xor(tie, s, kWave);
    match += __shfl_xor(match, s, kWave);
    flip += __shfl_xor(flip, s, kWave);
    zero += __shfl_xor(zero, s, kWave);
    var = fmax(var, __shfl_xor(var, s, kWave));
  }
  if (lane == 0) {
    sh_c[wave][0] = tie;
    sh_c[wave][1] = match;
    sh_c[wave][2] = flip;
    sh_c[wave][3] = zero;
    sh_v[wave] = var;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t* out = p.bstat + static_cast<int64_t>(blockIdx.x) * kStat;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      out[k] = static_cast<uint64_t>(sh_c[0][k]) + sh_c[1][k] + sh_c[2][k] + sh_c[3][k];
    const double v = fmax(fmax(sh_v[0], sh_v[1]), fmax(sh_v[2], sh_v[3]));
    out[4] = static_cast<uint64_t>(__double_as_longlong(v));
  }
}

// Fold 256 (count, count, count, count, max) slots held one per thread:
// thread 0 returns the workgroup's totals.  Integer sums and maxima are exact
// in any order.
__device__ __forceinline__ void fold_stats(uint64_t (&c)[4], double& v) {
  __shared__ uint64_t sh_c[4][4];
  __shared__ double sh_v[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] += __shfl_xor(c[k], s, kWave);
    v = fmax(v, __shfl_xor(v, s, kWave));
  }
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) sh_c[wave][k] = c[k];
    sh_v[wave] = v;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = (sh_c[0][k] + sh_c[1][k]) + (sh_c[2][k] + sh_c[3][k]);
    v = fmax(fmax(sh_v[0], sh_v[1]), fmax(sh_v[2], sh_v[3]));
  }
}

// Level 1: one workgroup per group of up to 256 consecutive blocks of one
// tensor (the same group table as the mean-|c| finalize); thread l takes
// block l's slots.
__global__ __launch_bounds__(kThreads) void k_stats_group(StepParams p) {
  const GroupEnt ge = p.grp[blockIdx.x];
  uint64_t c[4] = {0, 0, 0, 0};
  double v = 0.0;
  if (static_cast<int>(threadIdx.x) < ge.cnt) {
    const uint64_t* in = p.bstat + static_cast<int64_t>(ge.blk + threadIdx.x) * kStat;
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = in[k];
    v = __longlong_as_double(static_cast<long long>(in[4]));
  }
  fold_stats(c, v);
  if (threadIdx.x == 0) {
    uint64_t* out = p.gstat + static_cast<int64_t>(blockIdx.x) * kStat;
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = c[k];
    out[4] = static_cast<uint64_t>(__double_as_longlong(v));
  }
}

// Level 2: one workgroup per tensor over its groups' slots.
__global__ __launch_bounds__(kThreads) void k_stats_reduce(StepParams p) {
  const int T = blockIdx.x;
  const TensorEnt te = p.tens[T];
  uint64_t c[4] = {0, 0, 0, 0};
  double v = 0.0;
  for (int g = te.grp0 + static_cast<int>(threadIdx.x); g < te.grp0 + te.ngrp; g += kThreads) {
    const uint64_t* in = p.gstat + static_cast<int64_t>(g) * kStat;
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] += in[k];
    v = fmax(v, __longlong_as_double(static_cast<long long>(in[4])));
  }
  fold_stats(c, v);
  if (threadIdx.x == 0) {
    if (p.stats) {
#pragma unroll
      for (int k = 0; k < 4; ++k) p.stats[static_cast<int64_t>(T) * 4 + k] = c[k];
    }
    if (p.mvar_max) p.mvar_max[T] = v;
  }
}

hipError_t launch_stats_reduce(const StepParams& p, int nT, hipStream_t st) {
  hipLaunchKernelGGL(k_stats_group, dim3(p.ngrp), dim3(kThreads), 0, st, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_stats_reduce, dim3(nT), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

// One workgroup, one block.  Each thread owns the quads j[q] = start +
// 1024*q + 4*tid (q = 0..3) and walks the workers in the outer loop, so each
// worker row is read as one 16 KB contiguous run per workgroup before the
// next row (measured: longer runs per row stream better than interleaving
// the rows quad by quad).  FULL blocks (all 4096 elements present) have no
// per-lane predicates; WT > 0 fixes W at compile time; AVG selects the
// averaging path (new momenta summed, their mean written to every worker).
template <int TT, int GT, bool DBG, int AGG, int WB, int WT, bool FULL, bool AVG>
__device__ __forceinline__ void step_block(const StepParams& p, const BlockEnt& be, uint32_t par) {
  constexpr int Q = kRounds;
  const int W = WT > 0 ? WT : p.W;
  const int tid = threadIdx.x;
  constexpr bool kQ = AGG == kAggL1 || AGG == kAggLinf;  // quantised paths
  const double* __restrict__ scl = p.scale + be.tensor;  // scl[i*nT]
  float* __restrict__ m = p.m;

  int64_t j[Q];
  int nv[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int loc = kThreads * kQuad * q + kQuad * tid;
    j[q] = be.start + loc;
    nv[q] = FULL ? kQuad : max(0, min(kQuad, be.len - loc));
  }
  // max-norm draws: the quad at j (a multiple of 4) of worker i takes outputs
  // (t*W + i)*d + j and + j + 2 of the stream, mix64(seed + (n + 1) * gamma)
  // = mix64(zrow_i + j*gamma) and mix64(zrow_i + (j + 2)*gamma), mod 2^64;
  // each output gives its pair of elements 32 bits apiece
  uint64_t jg[AGG == kAggLinf ? Q : 1];
  if constexpr (AGG == kAggLinf) {
#pragma unroll
    for (int q = 0; q < Q; ++q) jg[q] = static_cast<uint64_t>(j[q]) * kGamma;
  }

  // theta does not change until the end: fetch it first
  F4 th[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q)
    if (FULL || nv[q] > 0) th[q] = ld_x4<TT>(p.theta, j[q], nv[q]);

  uint32_t cnt[Q];    // vote: per-element counts, one byte each
  int sum[Q][4];      // quantised paths: per-element integer sums
  F4 acc[Q];          // averaging: running sum of new momenta
  // diagnostics (debug instantiations): unquantised sum of c in worker order,
  // fp64 sums of the new momenta and of their squares
  constexpr bool ST = DBG && AGG != kAggApply;
  const bool want_st = ST && (p.stats || p.mvar_max);
  float csum[ST ? Q : 1][4];
  double s1[ST ? Q : 1][4], s2[ST ? Q : 1][4];
  if constexpr (ST) {
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int k = 0; k < 4; ++k) csum[q][k] = 0.0f, s1[q][k] = 0.0, s2[q][k] = 0.0;
  }
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    cnt[q] = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) sum[q][k] = 0;
  }

  // The W scales of this tensor (quantised paths) are staged in LDS once per block:
  // a vector load after the batch's data loads would make every wave wait
  // for all of them before its first product; an LDS read is counted apart
  // from the memory loads and arrives first.
  __shared__ double sh_sc[256];
  if (kQ) {
    for (int i = tid; i < W; i += kThreads) sh_sc[i] = scl[static_cast<int64_t>(i) * p.nT];
    __syncthreads();
  }

  constexpr bool kExact = WT > 0 && WT % WB == 0;
#pragma unroll 1
  for (int i0 = 0; i0 < W; i0 += WB) {
    double sc_b[WB];
    if (kQ) {
#pragma unroll
      for (int b = 0; b < WB; ++b) sc_b[b] = (kExact || i0 + b < W) ? sh_sc[i0 + b] : 0.0;
    }
    F4 mv[WB][Q], gv[WB][Q];
#pragma unroll
    for (int b = 0; b < WB; ++b) {
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        if ((kExact || i0 + b < W) && (FULL || nv[q] > 0)) {
          const int64_t idx = static_cast<int64_t>(i0 + b) * p.ld + j[q];
          mv[b][q] = ldnt_f32x4(m + idx, nv[q]);
          gv[b][q] = ldnt_x4<GT>(p.g, idx, nv[q]);
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) mv[b][q].v[k] = gv[b][q].v[k] = 0.0f;
        }
      }
    }
#pragma unroll
    for (int b = 0; b < WB; ++b) {
      const int i = i0 + b;
      if (!kExact && i >= W) break;
      const double s_i = kQ ? sc_b[b] : 0.0;
      uint64_t zrow = 0;
      if constexpr (AGG == kAggLinf)
        zrow = p.seed + ((static_cast<uint64_t>(p.t) * static_cast<uint64_t>(W) +
                          static_cast<uint64_t>(i)) * static_cast<uint64_t>(p.d) + 1u) * kGamma;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int64_t idx = static_cast<int64_t>(i) * p.ld + j[q];
        F4 mn;
        uint32_t nib = 0;
        uint64_t r01 = 0, r23 = 0;
        if constexpr (AGG == kAggLinf) {
          r01 = mix64(zrow + jg[q]);
          r23 = mix64(zrow + jg[q] + 2u * kGamma);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float c = (p.beta1 * mv[b][q].v[k]) + (p.omega1 * gv[b][q].v[k]);
          if (AGG == kAggVote || AGG == kAggAvg) {
            nib |= ((FULL || k < nv[q]) ? sign_bit(c, par) : 0u) << k;
          } else if (kQ) {
            int qc;
            if constexpr (AGG == kAggLinf) {
              qc = sr_code(c, s_i, p.qmax, quad_bits(r01, r23, k));
            } else {
              double y = __builtin_rint(static_cast<double>(c) * s_i);
              y = fmin(fmax(y, -static_cast<double>(p.qmax)), static_cast<double>(p.qmax));
              qc = static_cast<int>(y);
            }
            sum[q][k] += qc;
            if (DBG) nib |= (static_cast<uint32_t>(qc) & 0xFFu) << (8 * k);
          }
          mn.v[k] = (p.beta2 * mv[b][q].v[k]) + (p.omega2 * gv[b][q].v[k]);
          if constexpr (ST) {
            if (want_st) {
              csum[q][k] = i == 0 ? c : csum[q][k] + c;
              const double v = static_cast<double>(mn.v[k]);
              s1[q][k] = s1[q][k] + v;
              s2[q][k] = s2[q][k] + (v * v);
            }
          }
        }
        if (AGG == kAggVote || AGG == kAggAvg) {
          cnt[q] += nibble_to_bytes(nib);
          if (DBG && p.bits) {
            const uint64_t word = row_pack_word(nib);  // every lane takes part
            // the row's last lane stores the word if its first element exists
            // (in a ragged tail that lane itself may hold none)
            if ((tid & 15) == 15 && (FULL || (j[q] & ~int64_t{63}) < be.start + be.len))
              stnt_u64(p.bits + static_cast<int64_t>(i) * (p.ld >> 6) + (j[q] >> 6), word);
          }
        } else if (kQ && DBG && p.codes && (FULL || nv[q] > 0)) {
          stnt_b4(p.codes + idx, nib, nv[q]);
        }
        if (FULL || nv[q] > 0) {
          if (!AVG) {
            stnt_f32x4(m + idx, mn, nv[q]);
          } else if (i == 0) {
            acc[q] = mn;
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[q].v[k] = acc[q].v[k] + mn.v[k];
          }
        }
      }
    }
  }

  unsigned st_tie = 0, st_match = 0, st_flip = 0, st_zero = 0;
  double st_var = 0.0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    if (!FULL && nv[q] == 0) continue;
    // global sign s (the int8 record) and the applied update sf
    int s[4];
    float sf[4];
    if (AGG == kAggVote) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int twice = 2 * static_cast<int>((cnt[q] >> (8 * k)) & 0xFFu);
        s[k] = twice > W ? 1 : (twice < W ? -1 : (p.tie_zero ? 0 : (par ? 1 : -1)));
        sf[k] = static_cast<float>(s[k]);
      }
      if (DBG && p.counts) stnt_b4(p.counts + j[q], cnt[q], nv[q]);
    } else if (AGG == kAggAvg) {
      // D-Lion averaging: the mean of the W signs, (2v - W) / W in fp32
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int net = 2 * static_cast<int>((cnt[q] >> (8 * k)) & 0xFFu) - W;
        s[k] = (net > 0) - (net < 0);
        sf[k] = static_cast<float>(net) / static_cast<float>(W);
      }
      if (DBG && p.counts) stnt_b4(p.counts + j[q], cnt[q], nv[q]);
    } else if (kQ) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        s[k] = (sum[q][k] > 0) - (sum[q][k] < 0);
        sf[k] = static_cast<float>(s[k]);
      }
      if (DBG && p.sums) stnt_i32x4(p.sums + j[q], sum[q], nv[q]);
    } else {
      // apply mode: the sign arrives as bit planes (16 lanes share a word)
      const int sh = static_cast<int>(j[q] & 63);
      const uint32_t pos = static_cast<uint32_t>(p.sign_bits[j[q] >> 6] >> sh) & 0xFu;
      const uint32_t zer =
          p.zero_bits ? static_cast<uint32_t>(p.zero_bits[j[q] >> 6] >> sh) & 0xFu : 0u;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        s[k] = ((zer >> k) & 1u) ? 0 : (((pos >> k) & 1u) ? 1 : -1);
        sf[k] = static_cast<float>(s[k]);
      }
    }
    if constexpr (ST) {
      if (want_st) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (!FULL && k >= nv[q]) break;
          const int ref = (csum[q][k] > 0.0f) - (csum[q][k] < 0.0f);
          if ((AGG == kAggVote || AGG == kAggAvg) &&
              2 * static_cast<int>((cnt[q] >> (8 * k)) & 0xFFu) == W)
            st_tie++;
          if (s[k] != 0 && s[k] == ref) st_match++;
          if (s[k] != 0 && s[k] == -ref) st_flip++;
          if (s[k] == 0) st_zero++;
          const double mean = s1[q][k] / static_cast<double>(W);
          double var = (s2[q][k] / static_cast<double>(W)) - (mean * mean);
          if (var < 0.0) var = 0.0;
          st_var = fmax(st_var, var);
        }
      }
    }
    if (DBG && p.sign) {
      const uint32_t packed = (static_cast<uint32_t>(s[0]) & 0xFFu) |
                              ((static_cast<uint32_t>(s[1]) & 0xFFu) << 8) |
                              ((static_cast<uint32_t>(s[2]) & 0xFFu) << 16) |
                              ((static_cast<uint32_t>(s[3]) & 0xFFu) << 24);
      stnt_b4(p.sign + j[q], packed, nv[q]);
    }
    // theta <- theta - lr*(sign + wd*theta)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float x = th[q].v[k];
      th[q].v[k] = x - (p.lr * (sf[k] + (p.wd * x)));
    }
    stnt_x4<TT>(p.theta, j[q], th[q], nv[q]);
    // worker mean of the new momenta on averaging steps
    if (AVG) {
      const float fw = static_cast<float>(W);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[q].v[k] = acc[q].v[k] / fw;
#pragma unroll 4
      for (int i = 0; i < W; ++i)
        stnt_f32x4(m + static_cast<int64_t>(i) * p.ld + j[q], acc[q], nv[q]);
    }
  }
  if constexpr (ST) {
    if (want_st) block_stats(p, st_tie, st_match, st_flip, st_zero, st_var);
  }
}

template <int TT, int GT, bool DBG, int AGG, int WB, int WT>
__global__ __launch_bounds__(kThreads) void k_step(StepParams p) {
  const BlockEnt be = block_of(p.blk, p.flat, p.d);
  const bool avg = p.avg_step && p.any_sync && p.tens[be.tensor].sync;
  const uint32_t par = static_cast<uint32_t>(p.parity);
  if (be.len == kBlock) {
    if (avg) step_block<TT, GT, DBG, AGG, WB, WT, true, true>(p, be, par);
    else step_block<TT, GT, DBG, AGG, WB, WT, true, false>(p, be, par);
  } else {
    if (avg) step_block<TT, GT, DBG, AGG, WB, 0, false, true>(p, be, par);
    else step_block<TT, GT, DBG, AGG, WB, 0, false, false>(p, be, par);
  }
}

// Zero the words of each row that lie wholly past d (debug bitmaps).
__global__ void k_zero_tail_words(uint64_t* bits, int64_t words, int64_t first, int W) {
  const int64_t n = words - first;
  const int64_t k = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (k >= n * W) return;
  const int64_t i = k / n, w = first + k % n;
  bits[i * words + w] = 0;
}

constexpr int kWB = 2;

template <int TT, int GT, bool DBG, int AGG>
static hipError_t launch_t(const StepParams& p, int nblk, hipStream_t st) {
  const dim3 g(nblk), b(kThreads);
  if constexpr (!DBG) {
    if (p.W == 4) {
      hipLaunchKernelGGL((k_step<TT, GT, DBG, AGG, kWB, 4>), g, b, 0, st, p);
      return hipGetLastError();
    }
    if (p.W == 8) {
      hipLaunchKernelGGL((k_step<TT, GT, DBG, AGG, kWB, 8>), g, b, 0, st, p);
      return hipGetLastError();
    }
    if (p.W == 16) {
      hipLaunchKernelGGL((k_step<TT, GT, DBG, AGG, kWB, 16>), g, b, 0, st, p);
      return hipGetLastError();
    }
  }
  // debug outputs and diagnostics keep many more values live: one worker per
  // batch keeps them in registers
  hipLaunchKernelGGL((k_step<TT, GT, DBG, AGG, DBG ? 1 : kWB, 0>), g, b, 0, st, p);
  return hipGetLastError();
}

hipError_t launch_step(const StepParams& p, int nblk, int theta_bf16, int grad_bf16, int agg,
                       hipStream_t st) {
  const bool dbg = p.bits || p.codes || p.counts || p.sums || p.sign || p.stats || p.mvar_max;
  if (agg < 0 || agg > kAggLinf) return hipErrorInvalidValue;
  const int key = (theta_bf16 << 5) | (grad_bf16 << 4) | ((dbg ? 1 : 0) << 3) | agg;
  switch (key) {
#define LC_CASE(TT, GT, D, A) \
  case ((TT << 5) | (GT << 4) | (D << 3) | A): return launch_t<TT, GT, (D != 0), A>(p, nblk, st);
#define LC_AGGS(TT, GT, D) \
  LC_CASE(TT, GT, D, 0) LC_CASE(TT, GT, D, 1) LC_CASE(TT, GT, D, 2) LC_CASE(TT, GT, D, 4)
    LC_AGGS(0, 0, 0) LC_AGGS(0, 0, 1) LC_AGGS(0, 1, 0) LC_AGGS(0, 1, 1)
    LC_AGGS(1, 0, 0) LC_AGGS(1, 0, 1) LC_AGGS(1, 1, 0) LC_AGGS(1, 1, 1)
    LC_CASE(0, 0, 0, 3) LC_CASE(0, 1, 0, 3) LC_CASE(1, 0, 0, 3) LC_CASE(1, 1, 0, 3)
#undef LC_AGGS
#undef LC_CASE
    default: return hipErrorInvalidValue;
  }
}


hipError_t launch_zero_tail_words(uint64_t* bits, int64_t words, int64_t first, int W,
                                  hipStream_t st) {
  const int64_t n = (words - first) * W;
  if (n <= 0) return hipSuccess;
  const int64_t grid = (n + 255) / 256;
  hipLaunchKernelGGL(k_zero_tail_words, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, bits,
                     words, first, W);
  return hipGetLastError();
}

}  // namespace lioncub
