// device.hpp -- gfx950 device helpers: quad loads/stores, bf16, bit tricks.
//
// All floating point here is one IEEE operation at a time (the translation
// units are built with -ffp-contract=off and carry the pragma below).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace lioncub {

// ---------------------------------------------------------------- bf16 ----

__device__ __forceinline__ float bf16_widen(uint32_t h) {
  return __uint_as_float(h << 16);
}

// fp32 -> bf16, round to nearest even on the 16 dropped bits; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t bf16_narrow(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// --------------------------------------------------------- quad loads ----
// A "quad" is 4 consecutive elements owned by one thread.  nv (0..4) is the
// number that exist; the rest read as 0 and are never stored.  nv == 4 takes
// one vector access (16 bytes fp32, 8 bytes bf16).

struct F4 { float v[4]; };

__device__ __forceinline__ F4 ld_f32x4(const float* __restrict__ p, int nv) {
  F4 r;
  if (nv == 4) {
    float4 q = *reinterpret_cast<const float4*>(p);
    r.v[0] = q.x; r.v[1] = q.y; r.v[2] = q.z; r.v[3] = q.w;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) r.v[k] = k < nv ? p[k] : 0.0f;
  }
  return r;
}

__device__ __forceinline__ F4 ld_bf16x4(const uint16_t* __restrict__ p, int nv) {
  F4 r;
  if (nv == 4) {
    uint2 q = *reinterpret_cast<const uint2*>(p);
    r.v[0] = bf16_widen(q.x & 0xFFFFu); r.v[1] = bf16_widen(q.x >> 16);
    r.v[2] = bf16_widen(q.y & 0xFFFFu); r.v[3] = bf16_widen(q.y >> 16);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) r.v[k] = k < nv ? bf16_widen(p[k]) : 0.0f;
  }
  return r;
}

template <int BF16>
__device__ __forceinline__ F4 ld_x4(const void* __restrict__ base, int64_t idx, int nv) {
  if (BF16) return ld_bf16x4(static_cast<const uint16_t*>(base) + idx, nv);
  return ld_f32x4(static_cast<const float*>(base) + idx, nv);
}

// Element-wise masked quad loads for ragged blocks: no vector/scalar branch,
// so lanes of one wave that hold whole and partial quads share one path.
__device__ __forceinline__ F4 ldm_f32x4(const float* __restrict__ p, int nv) {
  F4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) r.v[k] = k < nv ? p[k] : 0.0f;
  return r;
}

template <int BF16>
__device__ __forceinline__ F4 ldm_x4(const void* __restrict__ base, int64_t idx, int nv) {
  F4 r;
  if (BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + idx;
#pragma unroll
    for (int k = 0; k < 4; ++k) r.v[k] = k < nv ? bf16_widen(p[k]) : 0.0f;
  } else {
    const float* p = static_cast<const float*>(base) + idx;
#pragma unroll
    for (int k = 0; k < 4; ++k) r.v[k] = k < nv ? p[k] : 0.0f;
  }
  return r;
}

// Streaming (nontemporal) variants for data touched once per step: the
// whole-quad case uses the nontemporal hint, which on gfx950 lifts a pure
// read stream from ~6.4 to ~7.1 TB/s; partial quads fall back to plain loads.
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef unsigned int v2u_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ F4 ldnt_f32x4(const float* __restrict__ p, int nv) {
  if (nv != 4) return ld_f32x4(p, nv);
  const v4f_t q = __builtin_nontemporal_load(reinterpret_cast<const v4f_t*>(p));
  F4 r;
  r.v[0] = q.x; r.v[1] = q.y; r.v[2] = q.z; r.v[3] = q.w;
  return r;
}

__device__ __forceinline__ F4 ldnt_bf16x4(const uint16_t* __restrict__ p, int nv) {
  if (nv != 4) return ld_bf16x4(p, nv);
  const v2u_t q = __builtin_nontemporal_load(reinterpret_cast<const v2u_t*>(p));
  F4 r;
  r.v[0] = bf16_widen(q.x & 0xFFFFu); r.v[1] = bf16_widen(q.x >> 16);
  r.v[2] = bf16_widen(q.y & 0xFFFFu); r.v[3] = bf16_widen(q.y >> 16);
  return r;
}

template <int BF16>
__device__ __forceinline__ F4 ldnt_x4(const void* __restrict__ base, int64_t idx, int nv) {
  if (BF16) return ldnt_bf16x4(static_cast<const uint16_t*>(base) + idx, nv);
  return ldnt_f32x4(static_cast<const float*>(base) + idx, nv);
}

__device__ __forceinline__ void st_f32x4(float* __restrict__ p, const F4& a, int nv) {
  if (nv == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(a.v[0], a.v[1], a.v[2], a.v[3]);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < nv) p[k] = a.v[k];
  }
}

__device__ __forceinline__ void st_bf16x4(uint16_t* __restrict__ p, const F4& a, int nv) {
  if (nv == 4) {
    uint2 q;
    q.x = bf16_narrow(a.v[0]) | (bf16_narrow(a.v[1]) << 16);
    q.y = bf16_narrow(a.v[2]) | (bf16_narrow(a.v[3]) << 16);
    *reinterpret_cast<uint2*>(p) = q;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < nv) p[k] = static_cast<uint16_t>(bf16_narrow(a.v[k]));
  }
}

__device__ __forceinline__ void stnt_f32x4(float* __restrict__ p, const F4& a, int nv) {
  if (nv != 4) {
    st_f32x4(p, a, nv);
    return;
  }
  const v4f_t q = {a.v[0], a.v[1], a.v[2], a.v[3]};
  __builtin_nontemporal_store(q, reinterpret_cast<v4f_t*>(p));
}

template <int BF16>
__device__ __forceinline__ void st_x4(void* __restrict__ base, int64_t idx, const F4& a, int nv) {
  if (BF16) st_bf16x4(static_cast<uint16_t*>(base) + idx, a, nv);
  else st_f32x4(static_cast<float*>(base) + idx, a, nv);
}

// Four bytes (one per element) as one 32-bit store when the quad is whole.
__device__ __forceinline__ void st_b4(void* __restrict__ p, uint32_t packed, int nv) {
  if (nv == 4) {
    *reinterpret_cast<uint32_t*>(p) = packed;
  } else {
    uint8_t* b = static_cast<uint8_t*>(p);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < nv) b[k] = static_cast<uint8_t>(packed >> (8 * k));
  }
}

__device__ __forceinline__ void st_i32x4(int32_t* __restrict__ p, const int (&s)[4], int nv) {
  if (nv == 4) {
    *reinterpret_cast<int4*>(p) = make_int4(s[0], s[1], s[2], s[3]);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < nv) p[k] = s[k];
  }
}

// Nontemporal stores for outputs written once per call.  Measured on MI355X
// (350M x 16 fp32 input): where the output is a small fraction of the bytes
// (sign words, 1-byte codes), plain stores trickle partial write-backs into
// the read stream and cost far more than their size; with the nontemporal
// hint the 1-bit pack went from 4.3 to 3.8 ms and the L1 codes kernel from
// 5.5 to 4.55 ms.  Partial quads fall back to plain stores.
typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void stnt_u64(uint64_t* __restrict__ p, uint64_t v) {
  __builtin_nontemporal_store(v, p);
}

__device__ __forceinline__ void stnt_u128(void* __restrict__ p, const uint4& v) {
  const v4u_t q = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(q, reinterpret_cast<v4u_t*>(p));
}

__device__ __forceinline__ void stnt_b4(void* __restrict__ p, uint32_t packed, int nv) {
  if (nv == 4) __builtin_nontemporal_store(packed, reinterpret_cast<uint32_t*>(p));
  else st_b4(p, packed, nv);
}

__device__ __forceinline__ void stnt_i32x4(int32_t* __restrict__ p, const int (&s)[4], int nv) {
  if (nv != 4) {
    st_i32x4(p, s, nv);
    return;
  }
  const v4u_t q = {static_cast<uint32_t>(s[0]), static_cast<uint32_t>(s[1]),
                   static_cast<uint32_t>(s[2]), static_cast<uint32_t>(s[3])};
  __builtin_nontemporal_store(q, reinterpret_cast<v4u_t*>(p));
}

__device__ __forceinline__ void stnt_bf16x4(uint16_t* __restrict__ p, const F4& a, int nv) {
  if (nv != 4) {
    st_bf16x4(p, a, nv);
    return;
  }
  const v2u_t q = {bf16_narrow(a.v[0]) | (bf16_narrow(a.v[1]) << 16),
                   bf16_narrow(a.v[2]) | (bf16_narrow(a.v[3]) << 16)};
  __builtin_nontemporal_store(q, reinterpret_cast<v2u_t*>(p));
}

template <int BF16>
__device__ __forceinline__ void stnt_x4(void* __restrict__ base, int64_t idx, const F4& a, int nv) {
  if (BF16) stnt_bf16x4(static_cast<uint16_t*>(base) + idx, a, nv);
  else stnt_f32x4(static_cast<float*>(base) + idx, a, nv);
}

// ------------------------------------------------------------ bit tricks --

// Bit k of a 4-bit nibble -> bit 0 of byte k (the four partial products of
// the multiply land in disjoint bit ranges, so no carries mix them).
__device__ __forceinline__ uint32_t nibble_to_bytes(uint32_t nib) {
  return (nib * 0x00204081u) & 0x01010101u;
}

// Wave64 sign bitmap of the 256 consecutive elements held 4 per lane: lane l
// holds bits nib (bit r = element 4l+r).  Each row of 16 lanes owns one
// 64-bit word (elements 64*(l/16) .. +63, LSB first): lane l%16 = r places
// its nibble at bit 4r of the low (r < 8) or high half, and an OR prefix scan
// over the row with DPP row shifts by 1, 2, 4 and 8 lanes leaves the whole
// word in lane r = 15.  Returns it there (partial ORs elsewhere).  Every lane
// of the wave must call it, with all 64 lanes active.
__device__ __forceinline__ uint64_t row_pack_word(uint32_t nib) {
  const int r = threadIdx.x & 15;
  uint32_t lo = r < 8 ? nib << (4 * r) : 0u;
  uint32_t hi = r >= 8 ? nib << (4 * (r - 8)) : 0u;
  // dpp_ctrl 0x110 + n = row_shr:n; lanes with no source in the row read 0
  lo |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(lo), 0x111, 0xF, 0xF, true));
  hi |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(hi), 0x111, 0xF, 0xF, true));
  lo |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(lo), 0x112, 0xF, 0xF, true));
  hi |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(hi), 0x112, 0xF, 0xF, true));
  lo |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(lo), 0x114, 0xF, 0xF, true));
  hi |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(hi), 0x114, 0xF, 0xF, true));
  lo |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(lo), 0x118, 0xF, 0xF, true));
  hi |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(hi), 0x118, 0xF, 0xF, true));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Sign bit of one element: 1 for c > 0, 0 for c < 0, parity for an exact
// zero (and for anything unordered).
__device__ __forceinline__ uint32_t sign_bit(float c, uint32_t parity) {
  return c > 0.0f ? 1u : (c < 0.0f ? 0u : parity);
}

// SplitMix64 output function (the finaliser of Steele, Lea and Flood's
// generator; see kGamma for the counter that feeds it).
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// The 32 random bits of element k (0..3) of a quad whose first element is
// even: the pair (k = 0, 1) shares draw r01 and the pair (2, 3) draw r23,
// the even element taking the low half and the odd one the high half.
__device__ __forceinline__ uint32_t quad_bits(uint64_t r01, uint64_t r23, int k) {
  const uint64_t r = k < 2 ? r01 : r23;
  return (k & 1) ? static_cast<uint32_t>(r >> 32) : static_cast<uint32_t>(r);
}

// Stochastic rounding of y = c * scale (fp64) onto the integers: floor(y) + 1
// when u < y - floor(y), u = r * 2^-32 uniform in [0, 1) for 32 random bits
// r, else floor(y); then clamped to +-qmax.  Every step is exact except the
// product; |c| <= max|c| keeps floor(y) within +-(qmax + 1), so the integer
// form of the last two steps is exact.
__device__ __forceinline__ int sr_code(float c, double scale, int qmax, uint32_t r) {
  const double y = static_cast<double>(c) * scale;
  const double fl = __builtin_floor(y);
  const double u = static_cast<double>(r) * 0x1.0p-32;
  const int q = static_cast<int>(fl) + (u < (y - fl) ? 1 : 0);
  return min(max(q, -qmax), qmax);
}

}  // namespace lioncub
