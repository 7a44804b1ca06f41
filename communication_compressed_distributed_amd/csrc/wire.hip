// wire.hip -- receive-side and wire-format kernels of the worker-sharded
// exchange, gfx950.
//
// On a cluster the pages' 1-bit path sends packed sign bitmaps through an
// AlltoAll, each worker votes on its slice and the 1-bit result is
// all-gathered; the p-bit path sends n-bit Eq. (1) codes and sums them
// ("Lion Cub: Minimizing Communication Overhead in Distributed Lion",
// pith.science review: "What carries the argument", the Figure 1 caption,
// the referee report on summation width).  These kernels are the per-GPU
// halves of that exchange, so the single-GPU pieces compose into it:
//
//   pack_codes: int8 codes -> n-bit two's complement fields, 32 elements per
//               group of n 32-bit words
//   unpack_sum: W packed rows -> int32 sums and their signs
//
// (The global sign of the vote as bit planes comes from the bit-sliced vote
// kernel; applying a global sign bitmap to theta and the momenta is a mode of
// the fused step kernel.)
#include "device.hpp"
#include "layout.hpp"

namespace lioncub {

struct WireParams {
  const int8_t* codes;   // [W][ld]
  uint32_t* wire;        // [W][(ld/32)*n]
  int32_t* sums;         // [d] or null
  int8_t* sign;          // [d] or null
  int64_t d, ld;
  int32_t W;
};

// One thread per (worker, group of 32 elements): 32 codes (two 16-byte
// loads) -> N words.  Field k sits at bit N*k of the group's bit string; all
// positions are compile-time, so a field that straddles two words is two
// shifts.
template <int N>
__global__ __launch_bounds__(kThreads) void k_pack_codes(WireParams p) {
  const int64_t groups = p.ld >> 5;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (gid >= groups * p.W) return;
  const int64_t i = gid / groups, gi = gid % groups;
  const int64_t j0 = gi << 5;
  const int8_t* src = p.codes + i * p.ld + j0;
  uint32_t c[8];
  const uint4 a = *reinterpret_cast<const uint4*>(src);
  const uint4 b = *reinterpret_cast<const uint4*>(src + 16);
  c[0] = a.x; c[1] = a.y; c[2] = a.z; c[3] = a.w;
  c[4] = b.x; c[5] = b.y; c[6] = b.z; c[7] = b.w;
  const int64_t valid = p.d - j0;  // elements at or past d pack as 0
  uint32_t w[N];
#pragma unroll
  for (int k = 0; k < N; ++k) w[k] = 0;
  constexpr uint32_t mask = (1u << N) - 1u;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const uint32_t f = k < valid ? ((c[k >> 2] >> (8 * (k & 3))) & mask) : 0u;
    const int bit = N * k;
    w[bit >> 5] |= f << (bit & 31);
    if ((bit & 31) + N > 32) w[(bit >> 5) + 1] |= f >> (32 - (bit & 31));
  }
  uint32_t* dst = p.wire + i * (groups * N) + gi * N;
  if constexpr (N == 4 || N == 8) {  // 16-byte aligned runs
#pragma unroll
    for (int k = 0; k < N; k += 4) stnt_u128(dst + k, make_uint4(w[k], w[k + 1], w[k + 2], w[k + 3]));
  } else {
#pragma unroll
    for (int k = 0; k < N; ++k) __builtin_nontemporal_store(w[k], dst + k);
  }
}

// The W workers' n-bit fields of group gi (32 elements), sign-extended and
// summed in int32.  The words of four workers are loaded before any is
// unpacked (same-process timing on 350M x 16, n = 4: 0.80-0.81 ms against
// 0.83 ms one worker at a time; 0.0055 against 0.0080 ms on 1M elements,
// where latency dominates).
template <int N>
__device__ __forceinline__ void unpack_group(const WireParams& p, int64_t gi, int32_t (&S)[32]) {
  const int64_t groups = p.ld >> 5;
#pragma unroll
  for (int k = 0; k < 32; ++k) S[k] = 0;
  auto add = [&](const uint32_t (&w)[N]) {
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int bit = N * k;
      uint32_t f = w[bit >> 5] >> (bit & 31);
      if ((bit & 31) + N > 32) f |= w[(bit >> 5) + 1] << (32 - (bit & 31));
      // sign-extend the low N bits
      const int32_t q = static_cast<int32_t>(f << (32 - N)) >> (32 - N);
      S[k] += q;
    }
  };
  const int64_t rstride = groups * N;
  const uint32_t* base = p.wire + gi * N;
  int i = 0;
#pragma unroll 1
  for (; i + 4 <= p.W; i += 4) {
    uint32_t w[4][N];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int k = 0; k < N; ++k) w[u][k] = __builtin_nontemporal_load(base + (i + u) * rstride + k);
#pragma unroll
    for (int u = 0; u < 4; ++u) add(w[u]);
  }
#pragma unroll 1
  for (; i < p.W; ++i) {
    uint32_t w[N];
#pragma unroll
    for (int k = 0; k < N; ++k) w[k] = base[i * rstride + k];
    add(w);
  }
}

// One thread per group of 32 elements: the sums (unpack_group), then sums
// and signs stored.
template <int N>
__global__ __launch_bounds__(kThreads) void k_unpack_sum(WireParams p) {
  const int64_t gi = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t j0 = gi << 5;
  if (j0 >= p.d) return;
  int32_t S[32];
  unpack_group<N>(p, gi, S);
  const int64_t valid = p.d - j0;
  // A workgroup whose 256 groups all lie below d writes through LDS: each
  // wave's 8 KB of sums (and 2 KB of signs) is stored as instructions of 64
  // consecutive 16-byte pieces instead of pieces 128 (32) bytes apart; the
  // XOR swizzles spread the LDS writes and reads over the banks (measured
  // about 5% faster).  Every thread of such a workgroup is present (none
  // returned above).
  const int64_t wg_end = (static_cast<int64_t>(blockIdx.x) + 1) * kThreads * 32;
  if (wg_end <= p.d) {
    __shared__ int4 sh_s[kThreads * 8];
    __shared__ uint4 sh_g[kThreads * 2];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t sg[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) sg[k] = 0;
#pragma unroll
    for (int k = 0; k < 32; ++k)
      sg[k >> 2] |= (static_cast<uint32_t>((S[k] > 0) - (S[k] < 0)) & 0xFFu) << (8 * (k & 3));
#pragma unroll
    for (int q = 0; q < 8; ++q)
      sh_s[wave * 512 + 8 * lane + (q ^ (lane & 7))] =
          make_int4(S[4 * q], S[4 * q + 1], S[4 * q + 2], S[4 * q + 3]);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      sh_g[wave * 128 + 2 * lane + (q ^ (lane & 1))] =
          make_uint4(sg[4 * q], sg[4 * q + 1], sg[4 * q + 2], sg[4 * q + 3]);
    __syncthreads();
    const int64_t wave_j0 = (static_cast<int64_t>(blockIdx.x) * kThreads + 64 * wave) << 5;
    if (p.sums) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {  // piece 64k + lane: lane src's quad lane % 8
        const int src = 8 * k + (lane >> 3);
        const int4 v = sh_s[wave * 512 + 8 * src + ((lane & 7) ^ (src & 7))];
        stnt_u128(p.sums + wave_j0 + 4 * (64 * k + lane),
                  make_uint4(static_cast<uint32_t>(v.x), static_cast<uint32_t>(v.y),
                             static_cast<uint32_t>(v.z), static_cast<uint32_t>(v.w)));
      }
    }
    if (p.sign) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int src = 32 * k + (lane >> 1);
        stnt_u128(p.sign + wave_j0 + 16 * (64 * k + lane),
                  sh_g[wave * 128 + 2 * src + ((lane & 1) ^ (src & 1))]);
      }
    }
  } else if (valid >= 32) {
    if (p.sums) {
#pragma unroll
      for (int k = 0; k < 32; k += 4)
        *reinterpret_cast<int4*>(p.sums + j0 + k) = make_int4(S[k], S[k + 1], S[k + 2], S[k + 3]);
    }
    if (p.sign) {
      uint32_t sg[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) sg[k] = 0;
#pragma unroll
      for (int k = 0; k < 32; ++k)
        sg[k >> 2] |= (static_cast<uint32_t>((S[k] > 0) - (S[k] < 0)) & 0xFFu) << (8 * (k & 3));
      *reinterpret_cast<uint4*>(p.sign + j0) = make_uint4(sg[0], sg[1], sg[2], sg[3]);
      *reinterpret_cast<uint4*>(p.sign + j0 + 16) = make_uint4(sg[4], sg[5], sg[6], sg[7]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      if (k >= valid) break;
      if (p.sums) p.sums[j0 + k] = S[k];
      if (p.sign) p.sign[j0 + k] = static_cast<int8_t>((S[k] > 0) - (S[k] < 0));
    }
  }
}

// The same sums as 2-bit global signs, in the bit planes the apply mode of
// the step kernel reads: one thread per group of 32 elements over all ld/32
// groups writes the 32-bit half gi of the sign plane (bit k: sum > 0) and of
// the zero plane (sum == 0); elements past d, and groups wholly past d
// (whose wire words are not read), give 0 bits.
template <int N>
__global__ __launch_bounds__(kThreads) void k_unpack_bits(WireParams p, uint32_t* __restrict__ sign_h,
                                                          uint32_t* __restrict__ zero_h) {
  const int64_t gi = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (gi >= (p.ld >> 5)) return;
  const int64_t j0 = gi << 5;
  uint32_t sb = 0, zb = 0;
  if (j0 < p.d) {
    int32_t S[32];
    unpack_group<N>(p, gi, S);
    const int64_t valid = p.d - j0;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      if (k < valid) {
        sb |= static_cast<uint32_t>(S[k] > 0) << k;
        zb |= static_cast<uint32_t>(S[k] == 0) << k;
      }
    }
  }
  __builtin_nontemporal_store(sb, sign_h + gi);
  if (zero_h) __builtin_nontemporal_store(zb, zero_h + gi);
}

hipError_t launch_pack_codes(const int8_t* codes, uint32_t* wire, int64_t d, int64_t ld, int W,
                             int n, hipStream_t st) {
  WireParams p{codes, wire, nullptr, nullptr, d, ld, W};
  const int64_t threads = (ld >> 5) * W;
  const dim3 g(static_cast<unsigned>((threads + kThreads - 1) / kThreads)), b(kThreads);
  switch (n) {
    case 2: hipLaunchKernelGGL(k_pack_codes<2>, g, b, 0, st, p); break;
    case 3: hipLaunchKernelGGL(k_pack_codes<3>, g, b, 0, st, p); break;
    case 4: hipLaunchKernelGGL(k_pack_codes<4>, g, b, 0, st, p); break;
    case 5: hipLaunchKernelGGL(k_pack_codes<5>, g, b, 0, st, p); break;
    case 6: hipLaunchKernelGGL(k_pack_codes<6>, g, b, 0, st, p); break;
    case 7: hipLaunchKernelGGL(k_pack_codes<7>, g, b, 0, st, p); break;
    case 8: hipLaunchKernelGGL(k_pack_codes<8>, g, b, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_unpack_sum(const uint32_t* wire, int32_t* sums, int8_t* sign, int64_t d,
                             int64_t ld, int W, int n, hipStream_t st) {
  WireParams p{nullptr, const_cast<uint32_t*>(wire), sums, sign, d, ld, W};
  const int64_t threads = (d + 31) >> 5;
  const dim3 g(static_cast<unsigned>((threads + kThreads - 1) / kThreads)), b(kThreads);
  switch (n) {
    case 2: hipLaunchKernelGGL(k_unpack_sum<2>, g, b, 0, st, p); break;
    case 3: hipLaunchKernelGGL(k_unpack_sum<3>, g, b, 0, st, p); break;
    case 4: hipLaunchKernelGGL(k_unpack_sum<4>, g, b, 0, st, p); break;
    case 5: hipLaunchKernelGGL(k_unpack_sum<5>, g, b, 0, st, p); break;
    case 6: hipLaunchKernelGGL(k_unpack_sum<6>, g, b, 0, st, p); break;
    case 7: hipLaunchKernelGGL(k_unpack_sum<7>, g, b, 0, st, p); break;
    case 8: hipLaunchKernelGGL(k_unpack_sum<8>, g, b, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_unpack_bits(const uint32_t* wire, uint64_t* sign_bits, uint64_t* zero_bits,
                              int64_t d, int64_t ld, int W, int n, hipStream_t st) {
  WireParams p{nullptr, const_cast<uint32_t*>(wire), nullptr, nullptr, d, ld, W};
  uint32_t* sh = reinterpret_cast<uint32_t*>(sign_bits);
  uint32_t* zh = reinterpret_cast<uint32_t*>(zero_bits);
  const int64_t threads = ld >> 5;
  const dim3 g(static_cast<unsigned>((threads + kThreads - 1) / kThreads)), b(kThreads);
  switch (n) {
    case 2: hipLaunchKernelGGL(k_unpack_bits<2>, g, b, 0, st, p, sh, zh); break;
    case 3: hipLaunchKernelGGL(k_unpack_bits<3>, g, b, 0, st, p, sh, zh); break;
    case 4: hipLaunchKernelGGL(k_unpack_bits<4>, g, b, 0, st, p, sh, zh); break;
    case 5: hipLaunchKernelGGL(k_unpack_bits<5>, g, b, 0, st, p, sh, zh); break;
    case 6: hipLaunchKernelGGL(k_unpack_bits<6>, g, b, 0, st, p, sh, zh); break;
    case 7: hipLaunchKernelGGL(k_unpack_bits<7>, g, b, 0, st, p, sh, zh); break;
    case 8: hipLaunchKernelGGL(k_unpack_bits<8>, g, b, 0, st, p, sh, zh); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lioncub
