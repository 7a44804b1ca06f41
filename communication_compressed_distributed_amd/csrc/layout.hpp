// layout.hpp -- host/device shared tables and kernel parameter blocks.
//
// The flat parameter vector is cut into tensors (offsets multiples of 64) and
// every tensor into blocks of kBlock elements; a block never straddles a
// tensor, so a workgroup sees one tensor's flags and scales.  The tables live
// in the caller's workspace (or the allocation-free step's fixed array),
// written by the table kernels of tables.hip.
#pragma once
#include <stdint.h>

namespace lioncub {

constexpr int kBlock = 4096;    // elements per block (and per mean-|x| partial)
constexpr int kThreads = 256;   // threads per workgroup (4 wave64)
constexpr int kQuad = 4;        // consecutive elements per thread and round
constexpr int kRounds = kBlock / (kThreads * kQuad);  // 4
constexpr int kWave = 64;

struct BlockEnt {      // 16 bytes
  int64_t start;       // first element (global index)
  int32_t len;         // 1..kBlock
  int32_t tensor;
};

constexpr int kGroup = 256;     // block partials folded together in the finalize

struct TensorEnt {     // 40 bytes
  int64_t off;         // first element
  int64_t n;           // elements
  int32_t blk0;        // first block id
  int32_t nblk;        // blocks
  int32_t grp0;        // first group id (groups of kGroup consecutive blocks)
  int32_t ngrp;        // groups
  int32_t sync;        // momentum averaged over workers on averaging steps
  int32_t pad;
};

struct GroupEnt {      // 16 bytes: kGroup consecutive blocks of one tensor
  int32_t tensor;
  int32_t blk;         // first block id
  int32_t cnt;         // 1..kGroup
  int32_t pad;
};

struct StepParams {
  const BlockEnt* blk;
  const TensorEnt* tens;
  void* theta;         // [d] fp32 or bf16
  float* m;            // [W][ld]
  const void* g;       // [W][ld] fp32 or bf16
  const double* scale; // [W][nT] (quantised paths): Qmax / M1 or Qmax / max|c|,
                       // 0 when that norm is 0
  int64_t ld;
  int32_t W;
  int32_t nT;
  float beta1, omega1, beta2, omega2, lr, wd;
  int32_t parity;      // t & 1
  int32_t avg_step;    // t % sync_every == 0
  int32_t tie_zero;
  int32_t qmax;
  int32_t flat;        // one tensor: block b starts at b*kBlock (no table load)
  int32_t any_sync;    // some tensor is averaged (else no tensor-table load)
  int64_t d;
  // stochastic rounding (max-norm path): element j of worker i takes 32 bits
  // of output (t*W + i)*d + (j & ~1) of the SplitMix64 stream keyed by seed
  uint64_t seed;
  int64_t t;
  // global sign given as bit planes (apply mode): [ld/64] each, zero may be null
  const uint64_t* sign_bits;
  const uint64_t* zero_bits;
  // optional outputs
  uint64_t* bits;
  int8_t* codes;
  uint8_t* counts;
  int32_t* sums;
  int8_t* sign;
  // diagnostics: per-block partials [nblk][kStat] and per-group partials
  // [ngrp][kStat] (workspace), then per tensor
  uint64_t* bstat;
  uint64_t* gstat;
  const GroupEnt* grp;  // groups of kGroup consecutive blocks of one tensor
  int32_t ngrp;
  uint64_t* stats;     // [nT][4]: ties, sign matches, flips, zero signs
  double* mvar_max;    // [nT]: largest inter-worker variance of the new momenta
};

constexpr int kStat = 8;  // per-block diagnostic slots: 4 counters, variance bits, pad

struct M1Params {
  const BlockEnt* blk;
  const TensorEnt* tens;
  const float* x;      // [W][ld] source c (quant_l1), or
  const float* m;      // [W][ld] with
  const void* g;       // [W][ld]: c = beta1*m + omega1*g
  const GroupEnt* grp;
  double* partial;     // [nblk][W]: each block's W partials written as one run
  double* gval;        // [W][ngrp]
  double* m1;          // [W][nT]
  double* scale;       // [W][nT]
  double* m1_out;      // optional caller copy of m1 [W][nT]
  int64_t ld;
  int32_t W;
  int32_t nT;
  int32_t nblk;
  int32_t ngrp;
  int32_t qmax;
  int32_t flat;        // one tensor: block b starts at b*kBlock (no table load)
  int64_t d;
  float beta1, omega1;
  uint64_t seed;       // max-norm codes: stochastic-rounding key and step
  int64_t t;
};

// Aggregation modes of the fused step kernel.
enum Agg : int { kAggVote = 0, kAggL1 = 1, kAggAvg = 2, kAggApply = 3, kAggLinf = 4 };

// SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014) as a counter-based generator: output k of the
// stream keyed by s is mix(s + (k+1)*gamma).
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

// Block b's descriptor; a single-tensor vector needs no table load.
__device__ __forceinline__ BlockEnt block_of(const BlockEnt* blk, int flat, int64_t d) {
  if (flat) {
    BlockEnt be;
    be.start = static_cast<int64_t>(blockIdx.x) * kBlock;
    const int64_t rem = d - be.start;
    be.len = static_cast<int32_t>(rem < kBlock ? rem : kBlock);
    be.tensor = 0;
    return be;
  }
  return blk[blockIdx.x];
}

}  // namespace lioncub
