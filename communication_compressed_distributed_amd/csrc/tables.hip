// tables.hip -- the tensor, block and group tables of a configuration,
// written into device memory with kernel launches only (no copies from host
// memory, no memsets), so that a table build can sit in a captured stream or
// in a call that may not allocate.
//
// The tensor table is computed on the host and handed to the device as
// kernel arguments, kTensChunk entries per launch.  The block and group
// tables follow from it: block b belongs to the last tensor whose first block
// id is <= b (every tensor has at least one block, so first block ids rise
// strictly), and likewise for groups.  A list of at most kTensChunk tensors
// gets all three tables from one launch.
#include "ctx.hpp"

namespace lioncub {

constexpr int kTensChunk = 32;  // 32 x 40 bytes of kernel arguments per launch

struct TensorChunk {
  TensorEnt ent[kTensChunk];
  int32_t first;  // index of ent[0] in the table
  int32_t count;  // 1..kTensChunk
};

__global__ void k_put_tensors(TensorChunk c, TensorEnt* __restrict__ tens) {
  const int k = threadIdx.x;
  if (k < c.count) tens[c.first + k] = c.ent[k];
}

// Last tensor T with key(T) <= id, keys strictly increasing from key(0) = 0.
template <typename Key>
__device__ __forceinline__ int owner(const TensorEnt* __restrict__ tens, int nT, int id, Key key) {
  int lo = 0, hi = nT - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (key(tens[mid]) <= id) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__global__ void k_put_blocks(const TensorEnt* __restrict__ tens, int nT, BlockEnt* __restrict__ blk,
                             int nblk) {
  const int b = static_cast<int>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (b >= nblk) return;
  const int T = owner(tens, nT, b, [](const TensorEnt& e) { return e.blk0; });
  const TensorEnt te = tens[T];
  const int64_t s = static_cast<int64_t>(b - te.blk0) * kBlock;
  BlockEnt be;
  be.start = te.off + s;
  be.len = static_cast<int32_t>(te.n - s < kBlock ? te.n - s : kBlock);
  be.tensor = T;
  blk[b] = be;
}

__global__ void k_put_groups(const TensorEnt* __restrict__ tens, int nT, GroupEnt* __restrict__ grp,
                             int ngrp) {
  const int gq = static_cast<int>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gq >= ngrp) return;
  const int T = owner(tens, nT, gq, [](const TensorEnt& e) { return e.grp0; });
  const TensorEnt te = tens[T];
  const int k = gq - te.grp0;
  GroupEnt ge;
  ge.tensor = T;
  ge.blk = te.blk0 + k * kGroup;
  ge.cnt = te.nblk - k * kGroup < kGroup ? te.nblk - k * kGroup : kGroup;
  ge.pad = 0;
  grp[gq] = ge;
}

// Every table in one launch when the whole tensor list fits one chunk of
// kernel arguments: items [0, nT) are tensor entries, [nT, nT + ngrp) groups,
// the rest blocks; a group or block finds its tensor among the argument
// entries themselves.  Used on vectors of up to kTensChunk tensors, where the
// table build is otherwise three launches beside a step that may itself be
// a few microseconds long.
__global__ void k_put_tables(TensorChunk c, TensorEnt* __restrict__ tens,
                             BlockEnt* __restrict__ blk, GroupEnt* __restrict__ grp, int ngrp,
                             int nblk) {
  const int64_t k = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int nT = c.count;
  if (k < nT) {
    tens[k] = c.ent[k];
    return;
  }
  if (k < nT + ngrp) {
    const int gq = static_cast<int>(k - nT);
    int T = 0;
    while (T + 1 < nT && c.ent[T + 1].grp0 <= gq) ++T;
    const TensorEnt& te = c.ent[T];
    const int r = gq - te.grp0;
    GroupEnt ge;
    ge.tensor = T;
    ge.blk = te.blk0 + r * kGroup;
    ge.cnt = te.nblk - r * kGroup < kGroup ? te.nblk - r * kGroup : kGroup;
    ge.pad = 0;
    grp[gq] = ge;
    return;
  }
  if (k < static_cast<int64_t>(nT) + ngrp + nblk) {
    const int b = static_cast<int>(k - nT - ngrp);
    int T = 0;
    while (T + 1 < nT && c.ent[T + 1].blk0 <= b) ++T;
    const TensorEnt& te = c.ent[T];
    const int64_t s = static_cast<int64_t>(b - te.blk0) * kBlock;
    BlockEnt be;
    be.start = te.off + s;
    be.len = static_cast<int32_t>(te.n - s < kBlock ? te.n - s : kBlock);
    be.tensor = T;
    blk[b] = be;
  }
}

hipError_t build_tables(const lioncub_config* c, int64_t nblk, int64_t ngrp, TensorEnt* tens,
                        BlockEnt* blk, GroupEnt* grp, int32_t* any_sync, hipStream_t st) {
  TensorChunk ch;
  int32_t blk0 = 0, grp0 = 0, sync = 0;
  for (int T0 = 0; T0 < c->n_tensors; T0 += kTensChunk) {
    ch.first = T0;
    ch.count = c->n_tensors - T0 < kTensChunk ? c->n_tensors - T0 : kTensChunk;
    for (int k = 0; k < ch.count; ++k) {
      const int T = T0 + k;
      TensorEnt& te = ch.ent[k];
      te.off = c->tensor_offsets[T];
      te.n = c->tensor_offsets[T + 1] - te.off;
      te.blk0 = blk0;
      te.nblk = static_cast<int32_t>((te.n + kBlock - 1) / kBlock);
      te.grp0 = grp0;
      te.ngrp = (te.nblk + kGroup - 1) / kGroup;
      te.sync = c->sync_m ? (c->sync_m[T] ? 1 : 0) : 0;
      te.pad = 0;
      blk0 += te.nblk;
      grp0 += te.ngrp;
      sync |= te.sync;
    }
    if (c->n_tensors <= kTensChunk) break;  // one chunk: all tables in one launch below
    hipLaunchKernelGGL(k_put_tensors, dim3(1), dim3(kTensChunk), 0, st, ch, tens);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (blk0 != nblk || grp0 != ngrp) return hipErrorInvalidValue;  // checked config: cannot happen
  *any_sync = sync;
  if (c->n_tensors <= kTensChunk) {
    const int64_t items = c->n_tensors + ngrp + nblk;
    hipLaunchKernelGGL(k_put_tables, dim3(static_cast<unsigned>((items + 255) / 256)), dim3(256),
                       0, st, ch, tens, blk, grp, static_cast<int>(ngrp), static_cast<int>(nblk));
    return hipGetLastError();
  }
  const unsigned nb = static_cast<unsigned>((nblk + 255) / 256);
  hipLaunchKernelGGL(k_put_blocks, dim3(nb), dim3(256), 0, st, tens, c->n_tensors, blk,
                     static_cast<int>(nblk));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned ng = static_cast<unsigned>((ngrp + 255) / 256);
  hipLaunchKernelGGL(k_put_groups, dim3(ng), dim3(256), 0, st, tens, c->n_tensors, grp,
                     static_cast<int>(ngrp));
  return hipGetLastError();
}

}  // namespace lioncub
