// bits.hip -- 1-bit sign packing and majority vote over packed bitmaps, gfx950.
//
// Lion Cub page (pith.science review, "What carries the argument"): signs are
// sent packed as 0/1 and exact zeros alternate between +1 and -1 with the
// iteration parity; the receiving side takes the majority of the workers'
// signs (D-Lion summary page, "Approach": majority vote).  These are the two
// halves of the 1-bit exchange; the fused step does both in registers.
//
// Pack: each lane loads a 16-byte quad, forms a 4-bit nibble, and four wave
// ballots give the 256 bits of the wave; the LSB-first 64-bit word of
// elements 64k..64k+63 is assembled from bits 16k..16k+15 of the ballots by a
// 4-way bit spread and stored by lane 16k.
//
// Vote: each lane owns a quad; for every worker it loads the 64-bit word that
// holds its quad (16 lanes share one word: one cache line per 16 lanes),
// extracts its nibble and adds it to four byte-wide counters held in one
// register (W <= 255, so no byte overflows).
#include "device.hpp"
#include "layout.hpp"

namespace lioncub {

struct PackParams {
  const float* x;   // [W][ld]
  uint64_t* bits;   // [W][ld/64]
  int64_t d, ld;
  uint32_t parity;
};

// grid: (ceil(ld/1024), W); 256 threads; 1024 elements (16 words) per group.
__global__ __launch_bounds__(kThreads) void k_pack(PackParams p) {
  const int tid = threadIdx.x;
  const int64_t i = blockIdx.y;
  const int64_t j = static_cast<int64_t>(blockIdx.x) * (kThreads * kQuad) + kQuad * tid;
  const int64_t rem = p.d - j;
  const int nv = rem >= 4 ? 4 : (rem > 0 ? static_cast<int>(rem) : 0);
  uint32_t nib = 0;
  if (nv > 0) {
    const F4 x = ld_f32x4(p.x + i * p.ld + j, nv);
#pragma unroll
    for (int k = 0; k < 4; ++k) nib |= (k < nv ? sign_bit(x.v[k], p.parity) : 0u) << k;
  }
  const uint64_t word = wave_pack_words(nib);
  if ((tid & 15) == 0 && j < p.ld) p.bits[i * (p.ld >> 6) + (j >> 6)] = word;
}

struct VoteParams {
  const uint64_t* bits;  // [W][ld/64]
  uint8_t* counts;       // [d] or null
  int8_t* sign;          // [d] or null
  int64_t d, words;
  int32_t W;
  uint32_t parity;
  int32_t tie_zero;
};

// grid: ceil(d/1024); 256 threads; 4 elements per thread.
__global__ __launch_bounds__(kThreads) void k_vote(VoteParams p) {
  const int64_t j = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * kQuad;
  if (j >= p.d) return;
  const int nv = p.d - j >= 4 ? 4 : static_cast<int>(p.d - j);
  const uint64_t* __restrict__ col = p.bits + (j >> 6);
  const int sh = static_cast<int>(j & 63);
  uint32_t cnt = 0;
  int i = 0;
  for (; i + 8 <= p.W; i += 8) {
    uint64_t w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) w[u] = col[static_cast<int64_t>(i + u) * p.words];
#pragma unroll
    for (int u = 0; u < 8; ++u) cnt += nibble_to_bytes(static_cast<uint32_t>(w[u] >> sh) & 0xFu);
  }
  for (; i < p.W; ++i)
    cnt += nibble_to_bytes(static_cast<uint32_t>(col[static_cast<int64_t>(i) * p.words] >> sh) & 0xFu);
  if (nv < 4) cnt &= (1u << (8 * nv)) - 1u;  // bits past d are 0 anyway
  if (p.counts) st_b4(p.counts + j, cnt, nv);
  if (p.sign) {
    uint32_t packed = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int twice = 2 * static_cast<int>((cnt >> (8 * k)) & 0xFFu);
      const int s = twice > p.W ? 1 : (twice < p.W ? -1 : (p.tie_zero ? 0 : (p.parity ? 1 : -1)));
      packed |= (static_cast<uint32_t>(s) & 0xFFu) << (8 * k);
    }
    st_b4(p.sign + j, packed, nv);
  }
}

hipError_t launch_pack(const float* x, uint64_t* bits, int64_t d, int64_t ld, int W,
                       uint32_t parity, hipStream_t st) {
  PackParams p{x, bits, d, ld, parity};
  const dim3 grid(static_cast<unsigned>((ld + kThreads * kQuad - 1) / (kThreads * kQuad)),
                  static_cast<unsigned>(W));
  hipLaunchKernelGGL(k_pack, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_vote(const uint64_t* bits, uint8_t* counts, int8_t* sign, int64_t d, int64_t ld,
                       int W, uint32_t parity, int tie_zero, hipStream_t st) {
  VoteParams p{bits, counts, sign, d, ld >> 6, W, parity, tie_zero};
  const int64_t grid = (d + kThreads * kQuad - 1) / (kThreads * kQuad);
  hipLaunchKernelGGL(k_vote, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace lioncub
