// ctx.hpp -- the host-side context of the C ABI, the layout of its device
// workspace and the configuration checks, shared by the context entry points
// (lioncub.cpp) and the allocation-free step (static.hip).
#pragma once
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "layout.hpp"
#include "lioncub.h"

namespace lioncub {

constexpr size_t kWsAlign = 256;

// Byte offsets of the workspace pieces, each 256-byte aligned.
struct WsLayout {
  size_t blk, tens, grp, partial, gval, m1, scale, bstat, gstat, total;
};

WsLayout ws_layout(int64_t nblk, int64_t ngrp, int64_t nT, int64_t W);

// Checks every field of c; on success *nblk = number of tensor-aligned
// blocks and *ngrp = number of groups of kGroup consecutive blocks.
int check_config(const lioncub_config* c, int64_t* nblk, int64_t* ngrp);

// Writes the tensor table (from c's offsets and flags, passed as kernel
// arguments) and then the block and group tables (derived on the device from
// the tensor table) into tens/blk/grp, asynchronously on st.  Enqueues kernel
// launches only.  *any_sync receives whether some tensor is averaged.
hipError_t build_tables(const lioncub_config* c, int64_t nblk, int64_t ngrp, TensorEnt* tens,
                        BlockEnt* blk, GroupEnt* grp, int32_t* any_sync, hipStream_t st);

}  // namespace lioncub

struct lioncub_ctx {
  lioncub_config cfg;  // host pointers cleared after the tables are built
  hipStream_t stream = nullptr;
  int32_t nblk = 0;
  int32_t ngrp = 0;
  int32_t any_sync = 0;
  lioncub::BlockEnt* blk = nullptr;
  lioncub::TensorEnt* tens = nullptr;
  lioncub::GroupEnt* grp = nullptr;
  double* partial = nullptr;
  double* gval = nullptr;
  double* m1 = nullptr;
  double* scale = nullptr;
  uint64_t* bstat = nullptr;
  uint64_t* gstat = nullptr;
  // profiling hook
  bool prof = false;
  int32_t prof_cap = 0;
  int32_t prof_n = 0;
  std::vector<hipEvent_t> prof_ev;  // 2 per record
  std::vector<int32_t> prof_kind;
};

namespace lioncub {

// Point c's device tables and buffers into the workspace ws laid out by L.
void bind_workspace(lioncub_ctx* c, char* ws, const WsLayout& L);

}  // namespace lioncub
