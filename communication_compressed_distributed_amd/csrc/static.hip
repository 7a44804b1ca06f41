// static.hip -- lioncub_step_static: the compressed-update step for callers
// that cannot allocate device memory (code under stream capture, tight
// serving loops, harnesses that forbid allocation).  The tables and norm
// partials a step needs live in `scratch`, a fixed array of device memory
// every GPU the library runs on holds from the time the library's code is
// loaded there until the process ends.  Each call rebuilds the tables in it
// (kernel launches only) and then runs the same kernels as lioncub_step, so
// nothing carries over between calls: every byte a call reads from scratch
// it has written first (tables, then block partials, group values, norms and
// scales, each fully written before it is read).  Calls that overlap on one
// GPU (two streams, two threads) race on the array.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address on the current GPU comes from hipGetSymbolAddress, taken
// once per device and kept, and only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ctx.hpp"
#include "lioncub.h"

static_assert(LIONCUB_STATIC_SCRATCH_BYTES % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[LIONCUB_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
char* g_scratch[kMaxDevices];  // device address of `scratch` per device, or null

// Device address of this GPU's scratch array: the current device must be the
// one `st` belongs to.
int scratch_of(hipStream_t st, char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return LIONCUB_EDEVICE;
  if (st) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(st, &sdev) != hipSuccess) return LIONCUB_EDEVICE;
    if (sdev != dev) return LIONCUB_EINVAL;
  }
  if (dev < 0 || dev >= kMaxDevices) return LIONCUB_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LIONCUB_EDEVICE;
    g_scratch[dev] = static_cast<char*>(p);
  }
  *out = g_scratch[dev];
  return LIONCUB_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int lioncub_step_static(const lioncub_config* cfg, void* hip_stream, void* theta,
                                   float* m, const void* g, int64_t t) {
  int64_t nblk = 0, ngrp = 0;
  int st = lioncub::check_config(cfg, &nblk, &ngrp);
  if (st != LIONCUB_OK) return st;
  if (!theta || !m || !g || t < 1) return LIONCUB_EINVAL;
  if (!aligned16(theta) || !aligned16(m) || !aligned16(g)) return LIONCUB_EALIGN;
  const lioncub::WsLayout L = lioncub::ws_layout(nblk, ngrp, cfg->n_tensors, cfg->W);
  if (L.total > LIONCUB_STATIC_SCRATCH_BYTES) return LIONCUB_ESCRATCH;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  char* base = nullptr;
  st = scratch_of(s, &base);
  if (st != LIONCUB_OK) return st;

  lioncub_ctx c;  // host stack only: no member allocates
  c.cfg = *cfg;
  c.stream = s;
  c.nblk = static_cast<int32_t>(nblk);
  c.ngrp = static_cast<int32_t>(ngrp);
  lioncub::bind_workspace(&c, base, L);
  if (lioncub::build_tables(cfg, nblk, ngrp, c.tens, c.blk, c.grp, &c.any_sync, s) !=
      hipSuccess)
    return LIONCUB_EDEVICE;
  c.cfg.tensor_offsets = nullptr;
  c.cfg.sync_m = nullptr;
  return lioncub_step(&c, theta, m, g, t, nullptr);
}
