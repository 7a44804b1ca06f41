// lioncub.cpp -- C ABI of the Lion Cub compressed-update step (see
// include/lioncub.h): configuration checks, workspace layout, kernel
// selection, profiling hook.  No device memory is allocated here; the caller
// provides the workspace (the allocation-free step in static.hip uses a
// fixed device array instead).
#include "lioncub.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include "ctx.hpp"
#include "layout.hpp"

namespace lioncub {
hipError_t launch_step(const StepParams& p, int nblk, int theta_bf16, int grad_bf16, int agg,
                       hipStream_t st);
hipError_t launch_zero_tail_words(uint64_t* bits, int64_t words, int64_t first, int W,
                                  hipStream_t st);
hipError_t launch_stats_reduce(const StepParams& p, int nT, hipStream_t st);
hipError_t launch_m1(const M1Params& p, int src_x, int grad_bf16, int maxnorm, hipStream_t st);
hipError_t launch_m1_finalize(const M1Params& p, int maxnorm, hipStream_t st);
hipError_t launch_quant_codes(const M1Params& p, int8_t* codes, int maxnorm, hipStream_t st);
hipError_t launch_pack(const float* x, uint64_t* bits, int64_t d, int64_t ld, int W,
                       uint32_t parity, hipStream_t st);
hipError_t launch_vote(const uint64_t* bits, uint8_t* counts, int8_t* sign, int64_t d, int64_t ld,
                       int W, uint32_t parity, int tie_zero, hipStream_t st);
hipError_t launch_vote_bits(const uint64_t* bits, uint64_t* sign_bits, uint64_t* zero_bits,
                            int64_t d, int64_t ld, int W, uint32_t parity, int tie_zero,
                            hipStream_t st);
hipError_t launch_pack_codes(const int8_t* codes, uint32_t* wire, int64_t d, int64_t ld, int W,
                             int n, hipStream_t st);
hipError_t launch_unpack_sum(const uint32_t* wire, int32_t* sums, int8_t* sign, int64_t d,
                             int64_t ld, int W, int n, hipStream_t st);
hipError_t launch_unpack_bits(const uint32_t* wire, uint64_t* sign_bits, uint64_t* zero_bits,
                              int64_t d, int64_t ld, int W, int n, hipStream_t st);
}  // namespace lioncub

using namespace lioncub;

namespace lioncub {

namespace {
constexpr int64_t kMaxLd = int64_t{1} << 40;

size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

bool finite(float x) { return std::isfinite(x); }
}  // namespace

WsLayout ws_layout(int64_t nblk, int64_t ngrp, int64_t nT, int64_t W) {
  WsLayout L;
  size_t o = 0;
  L.blk = o;
  o = align_up(o + static_cast<size_t>(nblk) * sizeof(BlockEnt));
  L.tens = o;
  o = align_up(o + static_cast<size_t>(nT) * sizeof(TensorEnt));
  L.grp = o;
  o = align_up(o + static_cast<size_t>(ngrp) * sizeof(GroupEnt));
  L.partial = o;
  o = align_up(o + static_cast<size_t>(W * nblk) * sizeof(double));
  L.gval = o;
  o = align_up(o + static_cast<size_t>(W * ngrp) * sizeof(double));
  L.m1 = o;
  o = align_up(o + static_cast<size_t>(W * nT) * sizeof(double));
  L.scale = o;
  o = align_up(o + static_cast<size_t>(W * nT) * sizeof(double));
  L.bstat = o;
  o = align_up(o + static_cast<size_t>(nblk) * kStat * sizeof(uint64_t));
  L.gstat = o;
  o = align_up(o + static_cast<size_t>(ngrp) * kStat * sizeof(uint64_t));
  L.total = o;
  return L;
}

// Checks every field; on success *nblk = number of tensor-aligned blocks and
// *ngrp = number of groups of kGroup consecutive blocks (per tensor).
int check_config(const lioncub_config* c, int64_t* nblk, int64_t* ngrp) {
  if (!c) return LIONCUB_EINVAL;
  if (c->d < 1 || c->ld < c->d || c->ld % 64 != 0) return LIONCUB_EINVAL;
  if (c->W < 1 || c->W > 255) return LIONCUB_EINVAL;
  if (c->n_tensors < 1 || !c->tensor_offsets) return LIONCUB_EINVAL;
  if (c->sync_every < 1) return LIONCUB_EINVAL;
  if ((c->theta_dtype != LIONCUB_F32 && c->theta_dtype != LIONCUB_BF16) ||
      (c->grad_dtype != LIONCUB_F32 && c->grad_dtype != LIONCUB_BF16))
    return LIONCUB_EINVAL;
  if (c->agg != LIONCUB_AGG_VOTE && c->agg != LIONCUB_AGG_L1SUM && c->agg != LIONCUB_AGG_AVG &&
      c->agg != LIONCUB_AGG_LINFSUM)
    return LIONCUB_EINVAL;
  if ((c->agg == LIONCUB_AGG_L1SUM || c->agg == LIONCUB_AGG_LINFSUM) &&
      (c->qbits < 2 || c->qbits > 8))
    return LIONCUB_EINVAL;
  if (c->tie_mode != LIONCUB_TIE_PARITY && c->tie_mode != LIONCUB_TIE_ZERO) return LIONCUB_EINVAL;
  if (!finite(c->beta1) || !finite(c->beta2) || !finite(c->lr) || !finite(c->wd))
    return LIONCUB_EINVAL;
  const int64_t* off = c->tensor_offsets;
  if (off[0] != 0 || off[c->n_tensors] != c->d) return LIONCUB_EINVAL;
  int64_t nb = 0, ng = 0;
  for (int k = 0; k < c->n_tensors; ++k) {
    if (off[k + 1] <= off[k] || off[k] % 64 != 0) return LIONCUB_EINVAL;
    const int64_t b = (off[k + 1] - off[k] + kBlock - 1) / kBlock;
    nb += b;
    ng += (b + kGroup - 1) / kGroup;
  }
  // blocks index a 1-D grid; element offsets i*ld + j (and their byte
  // offsets) must stay far inside int64
  if (nb > 0x7FFFFFFF || c->ld > kMaxLd) return LIONCUB_EUNSUPPORTED;
  *nblk = nb;
  *ngrp = ng;
  return LIONCUB_OK;
}

void bind_workspace(lioncub_ctx* c, char* ws, const WsLayout& L) {
  c->blk = reinterpret_cast<BlockEnt*>(ws + L.blk);
  c->tens = reinterpret_cast<TensorEnt*>(ws + L.tens);
  c->grp = reinterpret_cast<GroupEnt*>(ws + L.grp);
  c->partial = reinterpret_cast<double*>(ws + L.partial);
  c->gval = reinterpret_cast<double*>(ws + L.gval);
  c->m1 = reinterpret_cast<double*>(ws + L.m1);
  c->scale = reinterpret_cast<double*>(ws + L.scale);
  c->bstat = reinterpret_cast<uint64_t*>(ws + L.bstat);
  c->gstat = reinterpret_cast<uint64_t*>(ws + L.gstat);
}

}  // namespace lioncub

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Launch through the profiling hook when it is on.
template <typename F>
hipError_t run(lioncub_ctx* c, int kind, F&& f) {
  if (c->prof && c->prof_n < c->prof_cap) {
    const int k = c->prof_n++;
    c->prof_kind[k] = kind;
    hipError_t e = hipEventRecord(c->prof_ev[2 * k], c->stream);
    if (e != hipSuccess) return e;
    e = f();
    if (e != hipSuccess) return e;
    return hipEventRecord(c->prof_ev[2 * k + 1], c->stream);
  }
  return f();
}

void fill_step_params(const lioncub_ctx* c, StepParams* p) {
  std::memset(p, 0, sizeof(*p));
  p->blk = c->blk;
  p->tens = c->tens;
  p->scale = c->scale;
  p->bstat = c->bstat;
  p->gstat = c->gstat;
  p->grp = c->grp;
  p->ngrp = c->ngrp;
  p->ld = c->cfg.ld;
  p->W = c->cfg.W;
  p->nT = c->cfg.n_tensors;
  p->beta1 = c->cfg.beta1;
  p->omega1 = 1.0f - c->cfg.beta1;
  p->beta2 = c->cfg.beta2;
  p->omega2 = 1.0f - c->cfg.beta2;
  p->lr = c->cfg.lr;
  p->wd = c->cfg.wd;
  p->tie_zero = c->cfg.tie_mode == LIONCUB_TIE_ZERO;
  p->flat = c->cfg.n_tensors == 1;
  p->any_sync = c->any_sync;
  p->d = c->cfg.d;
  p->qmax = c->cfg.qbits >= 2 ? (1 << (c->cfg.qbits - 1)) - 1 : 0;
  p->seed = c->cfg.sr_seed;
}

void fill_m1_params(const lioncub_ctx* c, M1Params* p) {
  std::memset(p, 0, sizeof(*p));
  p->blk = c->blk;
  p->tens = c->tens;
  p->grp = c->grp;
  p->partial = c->partial;
  p->gval = c->gval;
  p->m1 = c->m1;
  p->scale = c->scale;
  p->ld = c->cfg.ld;
  p->W = c->cfg.W;
  p->nT = c->cfg.n_tensors;
  p->nblk = c->nblk;
  p->ngrp = c->ngrp;
  p->qmax = c->cfg.qbits >= 2 && c->cfg.qbits <= 8 ? (1 << (c->cfg.qbits - 1)) - 1 : 0;
  p->beta1 = c->cfg.beta1;
  p->omega1 = 1.0f - c->cfg.beta1;
  p->flat = c->cfg.n_tensors == 1;
  p->d = c->cfg.d;
  p->seed = c->cfg.sr_seed;
}

int dev_status(hipError_t e) { return e == hipSuccess ? LIONCUB_OK : LIONCUB_EDEVICE; }

}  // namespace

extern "C" {

size_t lioncub_workspace_bytes(const lioncub_config* cfg) {
  int64_t nblk = 0, ngrp = 0;
  if (check_config(cfg, &nblk, &ngrp) != LIONCUB_OK) return 0;
  return ws_layout(nblk, ngrp, cfg->n_tensors, cfg->W).total;
}

int lioncub_init(lioncub_ctx** out, const lioncub_config* cfg, void* hip_stream, void* workspace,
                 size_t ws_bytes) {
  if (!out) return LIONCUB_EINVAL;
  *out = nullptr;
  int64_t nblk = 0, ngrp = 0;
  int st = check_config(cfg, &nblk, &ngrp);
  if (st != LIONCUB_OK) return st;
  const WsLayout L = ws_layout(nblk, ngrp, cfg->n_tensors, cfg->W);
  if (!workspace || !aligned(workspace, kWsAlign) || ws_bytes < L.total) return LIONCUB_EWORKSPACE;

  lioncub_ctx* c = new (std::nothrow) lioncub_ctx();
  if (!c) return LIONCUB_ENOMEM;
  c->cfg = *cfg;
  c->stream = static_cast<hipStream_t>(hip_stream);
  c->nblk = static_cast<int32_t>(nblk);
  c->ngrp = static_cast<int32_t>(ngrp);
  bind_workspace(c, static_cast<char*>(workspace), L);
  hipError_t e =
      build_tables(cfg, nblk, ngrp, c->tens, c->blk, c->grp, &c->any_sync, c->stream);
  c->cfg.tensor_offsets = nullptr;
  c->cfg.sync_m = nullptr;
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) {
    delete c;
    return LIONCUB_EDEVICE;
  }
  *out = c;
  return LIONCUB_OK;
}

int lioncub_set_stream(lioncub_ctx* ctx, void* hip_stream) {
  if (!ctx) return LIONCUB_EINVAL;
  ctx->stream = static_cast<hipStream_t>(hip_stream);
  return LIONCUB_OK;
}

int lioncub_step(lioncub_ctx* ctx, void* theta, float* m, const void* g, int64_t t,
                 const lioncub_debug* dbg) {
  if (!ctx || !theta || !m || !g || t < 1) return LIONCUB_EINVAL;
  if (!aligned(theta, 16) || !aligned(m, 16) || !aligned(g, 16)) return LIONCUB_EALIGN;
  const lioncub_config& cf = ctx->cfg;
  const bool linf = cf.agg == LIONCUB_AGG_LINFSUM;
  const bool l1 = cf.agg == LIONCUB_AGG_L1SUM || linf;  // the quantised paths
  StepParams p;
  fill_step_params(ctx, &p);
  p.theta = theta;
  p.m = m;
  p.g = g;
  p.parity = static_cast<int32_t>(t & 1);
  p.avg_step = (t % cf.sync_every) == 0;
  p.t = t;
  const int kind = linf ? LIONCUB_K_LINF_STEP
                 : l1   ? LIONCUB_K_L1_STEP
                 : (cf.agg == LIONCUB_AGG_AVG ? LIONCUB_K_AVG_STEP : LIONCUB_K_VOTE_STEP);
  const int agg = linf ? kAggLinf : cf.agg;
  if (dbg) {
    if ((dbg->bits || dbg->counts) && l1) return LIONCUB_EINVAL;
    if ((dbg->codes || dbg->sums || dbg->m1) && !l1) return LIONCUB_EINVAL;
    if (!aligned(dbg->bits, 16) || !aligned(dbg->codes, 16) || !aligned(dbg->counts, 16) ||
        !aligned(dbg->sums, 16) || !aligned(dbg->sign, 16) || !aligned(dbg->m1, 16) ||
        !aligned(dbg->stats, 16) || !aligned(dbg->mvar_max, 16))
      return LIONCUB_EALIGN;
    p.bits = dbg->bits;
    p.codes = dbg->codes;
    p.counts = dbg->counts;
    p.sums = dbg->sums;
    p.sign = dbg->sign;
    p.stats = dbg->stats;
    p.mvar_max = dbg->mvar_max;
  }
  hipError_t e = hipSuccess;
  if (l1) {
    M1Params q;
    fill_m1_params(ctx, &q);
    q.m = m;
    q.g = g;
    q.m1_out = dbg ? dbg->m1 : nullptr;
    e = run(ctx, LIONCUB_K_M1_PARTIAL,
            [&] { return launch_m1(q, 0, cf.grad_dtype, linf, ctx->stream); });
    if (e == hipSuccess)
      e = run(ctx, LIONCUB_K_M1_FINALIZE, [&] { return launch_m1_finalize(q, linf, ctx->stream); });
  }
  if (e == hipSuccess)
    e = run(ctx, kind, [&] {
      return launch_step(p, ctx->nblk, cf.theta_dtype, cf.grad_dtype, agg, ctx->stream);
    });
  if (e == hipSuccess && p.bits)
    e = launch_zero_tail_words(p.bits, cf.ld / 64, (cf.d + 63) / 64, cf.W, ctx->stream);
  if (e == hipSuccess && (p.stats || p.mvar_max))
    e = run(ctx, LIONCUB_K_STATS, [&] { return launch_stats_reduce(p, cf.n_tensors, ctx->stream); });
  return dev_status(e);
}

int lioncub_vote_bits(lioncub_ctx* ctx, const uint64_t* bits, int64_t t, uint64_t* sign_bits,
                      uint64_t* zero_bits) {
  if (!ctx || !bits || !sign_bits || t < 1) return LIONCUB_EINVAL;
  if (!aligned(bits, 16) || !aligned(sign_bits, 16) || !aligned(zero_bits, 16))
    return LIONCUB_EALIGN;
  const lioncub_config& cf = ctx->cfg;
  return dev_status(run(ctx, LIONCUB_K_VOTE_BITS, [&] {
    return launch_vote_bits(bits, sign_bits, zero_bits, cf.d, cf.ld, cf.W,
                            static_cast<uint32_t>(t & 1), cf.tie_mode == LIONCUB_TIE_ZERO,
                            ctx->stream);
  }));
}

int lioncub_apply(lioncub_ctx* ctx, void* theta, float* m, const void* g, int64_t t,
                  const uint64_t* sign_bits, const uint64_t* zero_bits) {
  if (!ctx || !theta || !m || !g || !sign_bits || t < 1) return LIONCUB_EINVAL;
  if (!aligned(theta, 16) || !aligned(m, 16) || !aligned(g, 16) || !aligned(sign_bits, 16) ||
      !aligned(zero_bits, 16))
    return LIONCUB_EALIGN;
  const lioncub_config& cf = ctx->cfg;
  StepParams p;
  fill_step_params(ctx, &p);
  p.theta = theta;
  p.m = m;
  p.g = g;
  p.parity = static_cast<int32_t>(t & 1);
  p.avg_step = (t % cf.sync_every) == 0;
  p.sign_bits = sign_bits;
  p.zero_bits = zero_bits;
  return dev_status(run(ctx, LIONCUB_K_APPLY, [&] {
    return launch_step(p, ctx->nblk, cf.theta_dtype, cf.grad_dtype, kAggApply, ctx->stream);
  }));
}

int lioncub_pack_codes(lioncub_ctx* ctx, const int8_t* codes, uint32_t* wire) {
  if (!ctx || !codes || !wire) return LIONCUB_EINVAL;
  if (ctx->cfg.qbits < 2 || ctx->cfg.qbits > 8) return LIONCUB_EINVAL;
  if (!aligned(codes, 16) || !aligned(wire, 16)) return LIONCUB_EALIGN;
  const lioncub_config& cf = ctx->cfg;
  return dev_status(run(ctx, LIONCUB_K_PACK_CODES, [&] {
    return launch_pack_codes(codes, wire, cf.d, cf.ld, cf.W, cf.qbits, ctx->stream);
  }));
}

int lioncub_unpack_sum(lioncub_ctx* ctx, const uint32_t* wire, int32_t* sums, int8_t* sign) {
  if (!ctx || !wire || (!sums && !sign)) return LIONCUB_EINVAL;
  if (ctx->cfg.qbits < 2 || ctx->cfg.qbits > 8) return LIONCUB_EINVAL;
  if (!aligned(wire, 16) || !aligned(sums, 16) || !aligned(sign, 16)) return LIONCUB_EALIGN;
  const lioncub_config& cf = ctx->cfg;
  return dev_status(run(ctx, LIONCUB_K_UNPACK_SUM, [&] {
    return launch_unpack_sum(wire, sums, sign, cf.d, cf.ld, cf.W, cf.qbits, ctx->stream);
  }));
}

int lioncub_unpack_sum_bits(lioncub_ctx* ctx, const uint32_t* wire, uint64_t* sign_bits,
                            uint64_t* zero_bits) {
  if (!ctx || !wire || !sign_bits) return LIONCUB_EINVAL;
  if (ctx->cfg.qbits < 2 || ctx->cfg.qbits > 8) return LIONCUB_EINVAL;
  if (!aligned(wire, 16) || !aligned(sign_bits, 16) || !aligned(zero_bits, 16))
    return LIONCUB_EALIGN;
  const lioncub_config& cf = ctx->cfg;
  return dev_status(run(ctx, LIONCUB_K_UNPACK_BITS, [&] {
    return launch_unpack_bits(wire, sign_bits, zero_bits, cf.d, cf.ld, cf.W, cf.qbits,
                              ctx->stream);
  }));
}

int lioncub_pack(lioncub_ctx* ctx, const float* x, int64_t t, uint64_t* bits) {
  if (!ctx || !x || !bits || t < 1) return LIONCUB_EINVAL;
  if (!aligned(x, 16) || !aligned(bits, 16)) return LIONCUB_EALIGN;
  const lioncub_config& cf = ctx->cfg;
  return dev_status(run(ctx, LIONCUB_K_PACK, [&] {
    return launch_pack(x, bits, cf.d, cf.ld, cf.W, static_cast<uint32_t>(t & 1), ctx->stream);
  }));
}

int lioncub_vote(lioncub_ctx* ctx, const uint64_t* bits, int64_t t, uint8_t* counts,
                 int8_t* sign) {
  if (!ctx || !bits || t < 1 || (!counts && !sign)) return LIONCUB_EINVAL;
  if (!aligned(bits, 16) || !aligned(counts, 16) || !aligned(sign, 16)) return LIONCUB_EALIGN;
  const lioncub_config& cf = ctx->cfg;
  return dev_status(run(ctx, LIONCUB_K_VOTE, [&] {
    return launch_vote(bits, counts, sign, cf.d, cf.ld, cf.W, static_cast<uint32_t>(t & 1),
                       cf.tie_mode == LIONCUB_TIE_ZERO, ctx->stream);
  }));
}

int lioncub_quant_l1(lioncub_ctx* ctx, const float* x, int8_t* codes, double* m1) {
  if (!ctx || !x || !codes) return LIONCUB_EINVAL;
  if (ctx->cfg.qbits < 2 || ctx->cfg.qbits > 8) return LIONCUB_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(m1, 16)) return LIONCUB_EALIGN;
  M1Params q;
  fill_m1_params(ctx, &q);
  q.x = x;
  q.m1_out = m1;
  hipError_t e = run(ctx, LIONCUB_K_M1_PARTIAL, [&] { return launch_m1(q, 1, 0, 0, ctx->stream); });
  if (e == hipSuccess)
    e = run(ctx, LIONCUB_K_M1_FINALIZE, [&] { return launch_m1_finalize(q, 0, ctx->stream); });
  if (e == hipSuccess)
    e = run(ctx, LIONCUB_K_QUANT, [&] { return launch_quant_codes(q, codes, 0, ctx->stream); });
  return dev_status(e);
}

int lioncub_quant_linf(lioncub_ctx* ctx, const float* x, int64_t t, int8_t* codes,
                       double* minf) {
  if (!ctx || !x || !codes || t < 1) return LIONCUB_EINVAL;
  if (ctx->cfg.qbits < 2 || ctx->cfg.qbits > 8) return LIONCUB_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(minf, 16)) return LIONCUB_EALIGN;
  M1Params q;
  fill_m1_params(ctx, &q);
  q.x = x;
  q.m1_out = minf;
  q.t = t;
  hipError_t e = run(ctx, LIONCUB_K_M1_PARTIAL, [&] { return launch_m1(q, 1, 0, 1, ctx->stream); });
  if (e == hipSuccess)
    e = run(ctx, LIONCUB_K_M1_FINALIZE, [&] { return launch_m1_finalize(q, 1, ctx->stream); });
  if (e == hipSuccess)
    e = run(ctx, LIONCUB_K_QUANT_LINF,
            [&] { return launch_quant_codes(q, codes, 1, ctx->stream); });
  return dev_status(e);
}

int lioncub_profile_begin(lioncub_ctx* ctx, int32_t capacity) {
  if (!ctx || capacity < 1 || ctx->prof) return LIONCUB_EINVAL;
  try {
    ctx->prof_ev.assign(2 * static_cast<size_t>(capacity), nullptr);
    ctx->prof_kind.assign(capacity, 0);
  } catch (const std::bad_alloc&) {
    ctx->prof_ev.clear();
    ctx->prof_kind.clear();
    return LIONCUB_ENOMEM;
  }
  for (auto& ev : ctx->prof_ev) {
    if (hipEventCreate(&ev) != hipSuccess) {
      for (auto& e2 : ctx->prof_ev)
        if (e2) (void)hipEventDestroy(e2);
      ctx->prof_ev.clear();
      return LIONCUB_EDEVICE;
    }
  }
  ctx->prof_cap = capacity;
  ctx->prof_n = 0;
  ctx->prof = true;
  return LIONCUB_OK;
}

int lioncub_profile_end(lioncub_ctx* ctx, double* ms_total, int32_t* launches) {
  if (!ctx || !ctx->prof || !ms_total || !launches) return LIONCUB_EINVAL;
  for (int k = 0; k < LIONCUB_K_COUNT; ++k) {
    ms_total[k] = 0.0;
    launches[k] = 0;
  }
  int st = LIONCUB_OK;
  for (int r = 0; r < ctx->prof_n; ++r) {
    float ms = 0.0f;
    if (hipEventSynchronize(ctx->prof_ev[2 * r + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, ctx->prof_ev[2 * r], ctx->prof_ev[2 * r + 1]) != hipSuccess) {
      st = LIONCUB_EDEVICE;
      continue;
    }
    ms_total[ctx->prof_kind[r]] += ms;
    launches[ctx->prof_kind[r]] += 1;
  }
  for (auto& ev : ctx->prof_ev) (void)hipEventDestroy(ev);
  ctx->prof_ev.clear();
  ctx->prof = false;
  ctx->prof_n = 0;
  return st;
}

int lioncub_destroy(lioncub_ctx* ctx) {
  if (!ctx) return LIONCUB_OK;
  int st = LIONCUB_OK;
  if (hipStreamSynchronize(ctx->stream) != hipSuccess) st = LIONCUB_EDEVICE;
  for (auto& ev : ctx->prof_ev) (void)hipEventDestroy(ev);
  delete ctx;
  return st;
}

const char* lioncub_strerror(int status) {
  switch (status) {
    case LIONCUB_OK: return "ok";
    case LIONCUB_EINVAL: return "invalid argument or configuration";
    case LIONCUB_EALIGN: return "pointer not aligned as required";
    case LIONCUB_EWORKSPACE: return "workspace missing, misaligned or too small";
    case LIONCUB_EDEVICE: return "HIP runtime or kernel launch failure";
    case LIONCUB_EUNSUPPORTED: return "configuration not supported by this library";
    case LIONCUB_ENOMEM: return "out of host memory";
    case LIONCUB_ESCRATCH:
      return "configuration needs more than the library's fixed scratch array";
    default: return "unknown status";
  }
}

}  // extern "C"
