/*
 * example.c -- the C ABI used from plain C (no Python, no torch): allocate
 * the state with the HIP runtime, run three steps of each aggregation mode
 * through lioncub_step, and compare theta and the momenta bit for bit with
 * the CPU oracle (liblco, test infrastructure) run on host copies; then the
 * p-bit exchange composed of the standalone calls against the fused step, and
 * two cases through the allocation-free lioncub_step_static.  Also
 * checks that argument errors come back as status codes before anything
 * runs.  Prints one line per case and exits non-zero on any mismatch.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lioncub.h"
#include "../../oracle/lco.h"

#define CHECK_HIP(x)                                                        \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__);      \
      exit(2);                                                              \
    }                                                                       \
  } while (0)

/* Inputs: a small xorshift generator (test data only). */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static float rnd(float scale) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  const double u = (double)(rng_state >> 11) * (1.0 / 9007199254740992.0);
  return (float)((u - 0.5) * 2.0 * scale);
}

/* use_static: step through lioncub_step_static (no context, no workspace:
 * the library's fixed scratch array) instead of lioncub_step. */
static int run_case(int32_t agg, int32_t qbits, const char *name, int use_static) {
  const int64_t d = 3 * 4096 + 1000, ld = (d + 63) / 64 * 64;
  const int32_t W = 5;
  const int64_t off[3] = {0, 8192, d};
  const uint8_t sync[2] = {1, 0};

  lioncub_config cfg;
  memset(&cfg, 0, sizeof cfg);
  cfg.d = d;
  cfg.ld = ld;
  cfg.W = W;
  cfg.n_tensors = 2;
  cfg.tensor_offsets = off;
  cfg.sync_m = sync;
  cfg.sync_every = 2;
  cfg.theta_dtype = LIONCUB_F32;
  cfg.grad_dtype = LIONCUB_F32;
  cfg.agg = agg;
  cfg.qbits = qbits;
  cfg.tie_mode = LIONCUB_TIE_PARITY;
  cfg.beta1 = 0.9f;
  cfg.beta2 = 0.99f;
  cfg.lr = 1e-4f;
  cfg.wd = 0.1f;
  cfg.sr_seed = 12345u;

  const size_t nth = (size_t)d, nwl = (size_t)W * (size_t)ld;
  float *h_theta = calloc(nth, 4), *h_m = calloc(nwl, 4), *h_g = calloc(nwl, 4);
  float *o_theta = calloc(nth, 4), *o_m = calloc(nwl, 4), *r_theta = calloc(nth, 4),
        *r_m = calloc(nwl, 4);
  for (size_t j = 0; j < nth; ++j) h_theta[j] = rnd(0.02f);
  for (int32_t i = 0; i < W; ++i)
    for (int64_t j = 0; j < d; ++j) h_m[(size_t)i * ld + j] = rnd(1e-3f);
  memcpy(o_theta, h_theta, nth * 4);
  memcpy(o_m, h_m, nwl * 4);

  const size_t ws_bytes = lioncub_workspace_bytes(&cfg);
  if (ws_bytes == 0) { fprintf(stderr, "%s: config rejected\n", name); return 1; }
  void *ws, *d_theta, *d_m, *d_g;
  CHECK_HIP(hipMalloc(&ws, ws_bytes));
  CHECK_HIP(hipMalloc(&d_theta, nth * 4));
  CHECK_HIP(hipMalloc(&d_m, nwl * 4));
  CHECK_HIP(hipMalloc(&d_g, nwl * 4));
  CHECK_HIP(hipMemcpy(d_theta, h_theta, nth * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_m, h_m, nwl * 4, hipMemcpyHostToDevice));

  lioncub_ctx *ctx = NULL;
  int st = lioncub_init(&ctx, &cfg, NULL, ws, ws_bytes);
  if (st != LIONCUB_OK) { fprintf(stderr, "%s: init %s\n", name, lioncub_strerror(st)); return 1; }

  /* argument errors are returned before anything is enqueued */
  if (lioncub_step(ctx, d_theta, (float *)d_m, d_g, 0, NULL) != LIONCUB_EINVAL ||
      lioncub_step(ctx, (char *)d_theta + 4, (float *)d_m, d_g, 1, NULL) != LIONCUB_EALIGN ||
      lioncub_step(NULL, d_theta, (float *)d_m, d_g, 1, NULL) != LIONCUB_EINVAL) {
    fprintf(stderr, "%s: argument errors not reported\n", name);
    return 1;
  }

  /* the oracle's configuration: the same numbers */
  lco_cfg oc;
  memset(&oc, 0, sizeof oc);
  oc.d = d;
  oc.W = W;
  oc.n_tensors = 2;
  oc.off = off;
  oc.sync_m = sync;
  oc.sync_every = 2;
  oc.theta_bf16 = 0;
  oc.grad_bf16 = 0;
  oc.agg = agg;  /* the two enums share values */
  oc.qbits = qbits;
  oc.tie_mode = LCO_TIE_PARITY;
  oc.beta1 = 0.9f;
  oc.beta2 = 0.99f;
  oc.lr = 1e-4f;
  oc.wd = 0.1f;
  oc.seed = 12345u;

  for (int64_t t = 1; t <= 3; ++t) {
    memset(h_g, 0, nwl * 4);
    for (int32_t i = 0; i < W; ++i)
      for (int64_t j = 0; j < d; ++j) {
        float v = rnd(1e-3f);
        if ((j % 97) == 0) v = 0.0f;   /* exact zeros: the parity rule */
        h_g[(size_t)i * ld + j] = v;
      }
    CHECK_HIP(hipMemcpy(d_g, h_g, nwl * 4, hipMemcpyHostToDevice));
    st = use_static ? lioncub_step_static(&cfg, NULL, d_theta, (float *)d_m, d_g, t)
                    : lioncub_step(ctx, d_theta, (float *)d_m, d_g, t, NULL);
    if (st != LIONCUB_OK) { fprintf(stderr, "%s: step %s\n", name, lioncub_strerror(st)); return 1; }
    lco_step(&oc, ld, o_theta, o_m, h_g, t, NULL);
  }
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(r_theta, d_theta, nth * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(r_m, d_m, nwl * 4, hipMemcpyDeviceToHost));

  int64_t bad = 0;
  for (size_t j = 0; j < nth; ++j) bad += memcmp(&r_theta[j], &o_theta[j], 4) != 0;
  for (int32_t i = 0; i < W; ++i)
    for (int64_t j = 0; j < d; ++j)
      bad += memcmp(&r_m[(size_t)i * ld + j], &o_m[(size_t)i * ld + j], 4) != 0;
  printf("%s: %lld values differ from the oracle\n", name, (long long)bad);

  lioncub_destroy(ctx);
  hipFree(ws); hipFree(d_theta); hipFree(d_m); hipFree(d_g);
  free(h_theta); free(h_m); free(h_g); free(o_theta); free(o_m); free(r_theta); free(r_m);
  return bad != 0;
}

/* The worker-sharded p-bit exchange through the C ABI alone: each worker's
 * c (formed on the host with the oracle's lco_c_row) is quantised
 * (lioncub_quant_l1), packed to n-bit fields (lioncub_pack_codes), unpacked
 * and summed into sign and zero planes (lioncub_unpack_sum_bits) and
 * applied (lioncub_apply); theta and m must equal the oracle's fused step. */
static int run_exchange(void) {
  const int64_t d = 2 * 4096 + 700, ld = (d + 63) / 64 * 64;
  const int32_t W = 6, n = 4;
  const int64_t off[2] = {0, d};
  lioncub_config cfg;
  memset(&cfg, 0, sizeof cfg);
  cfg.d = d; cfg.ld = ld; cfg.W = W; cfg.n_tensors = 1; cfg.tensor_offsets = off;
  cfg.sync_every = 1; cfg.theta_dtype = LIONCUB_F32; cfg.grad_dtype = LIONCUB_F32;
  cfg.agg = LIONCUB_AGG_L1SUM; cfg.qbits = n; cfg.tie_mode = LIONCUB_TIE_PARITY;
  cfg.beta1 = 0.9f; cfg.beta2 = 0.99f; cfg.lr = 1e-4f; cfg.wd = 0.1f;
  lco_cfg oc;
  memset(&oc, 0, sizeof oc);
  oc.d = d; oc.W = W; oc.n_tensors = 1; oc.off = off; oc.sync_every = 1;
  oc.agg = LCO_AGG_L1SUM; oc.qbits = n; oc.tie_mode = LCO_TIE_PARITY;
  oc.beta1 = 0.9f; oc.beta2 = 0.99f; oc.lr = 1e-4f; oc.wd = 0.1f;

  const size_t nwl = (size_t)W * (size_t)ld, words = (size_t)(ld / 64);
  const size_t nwire = (size_t)W * (size_t)(ld / 32) * (size_t)n;
  float *h_theta = calloc((size_t)d, 4), *h_m = calloc(nwl, 4), *h_g = calloc(nwl, 4),
        *h_c = calloc(nwl, 4), *r_theta = calloc((size_t)d, 4), *r_m = calloc(nwl, 4);
  for (int64_t j = 0; j < d; ++j) h_theta[j] = rnd(0.02f);
  for (int32_t i = 0; i < W; ++i)
    for (int64_t j = 0; j < d; ++j) {
      h_m[(size_t)i * ld + j] = rnd(1e-3f);
      h_g[(size_t)i * ld + j] = rnd(1e-3f);
    }
  for (int32_t i = 0; i < W; ++i)
    lco_c_row(&oc, d, h_m + (size_t)i * ld, h_g + (size_t)i * ld, h_c + (size_t)i * ld);

  const size_t ws_bytes = lioncub_workspace_bytes(&cfg);
  void *ws, *d_theta, *d_m, *d_g, *d_c, *d_codes, *d_wire, *d_sb, *d_zb;
  CHECK_HIP(hipMalloc(&ws, ws_bytes));
  CHECK_HIP(hipMalloc(&d_theta, (size_t)d * 4));
  CHECK_HIP(hipMalloc(&d_m, nwl * 4));
  CHECK_HIP(hipMalloc(&d_g, nwl * 4));
  CHECK_HIP(hipMalloc(&d_c, nwl * 4));
  CHECK_HIP(hipMalloc(&d_codes, nwl));
  CHECK_HIP(hipMalloc(&d_wire, nwire * 4));
  CHECK_HIP(hipMalloc(&d_sb, words * 8));
  CHECK_HIP(hipMalloc(&d_zb, words * 8));
  CHECK_HIP(hipMemcpy(d_theta, h_theta, (size_t)d * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_m, h_m, nwl * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_g, h_g, nwl * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_c, h_c, nwl * 4, hipMemcpyHostToDevice));

  lioncub_ctx *ctx = NULL;
  int st = lioncub_init(&ctx, &cfg, NULL, ws, ws_bytes);
  if (st == LIONCUB_OK) st = lioncub_quant_l1(ctx, (const float *)d_c, (int8_t *)d_codes, NULL);
  if (st == LIONCUB_OK) st = lioncub_pack_codes(ctx, (const int8_t *)d_codes, (uint32_t *)d_wire);
  if (st == LIONCUB_OK)
    st = lioncub_unpack_sum_bits(ctx, (const uint32_t *)d_wire, (uint64_t *)d_sb,
                                 (uint64_t *)d_zb);
  if (st == LIONCUB_OK)
    st = lioncub_apply(ctx, d_theta, (float *)d_m, d_g, 1, (const uint64_t *)d_sb,
                       (const uint64_t *)d_zb);
  if (st != LIONCUB_OK) {
    fprintf(stderr, "exchange: %s\n", lioncub_strerror(st));
    return 1;
  }
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(r_theta, d_theta, (size_t)d * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(r_m, d_m, nwl * 4, hipMemcpyDeviceToHost));
  lco_step(&oc, ld, h_theta, h_m, h_g, 1, NULL);

  int64_t bad = 0;
  for (int64_t j = 0; j < d; ++j) bad += memcmp(&r_theta[j], &h_theta[j], 4) != 0;
  for (int32_t i = 0; i < W; ++i)
    for (int64_t j = 0; j < d; ++j)
      bad += memcmp(&r_m[(size_t)i * ld + j], &h_m[(size_t)i * ld + j], 4) != 0;
  printf("p-bit exchange (quant_l1, pack_codes, unpack_sum_bits, apply): %lld values differ "
         "from the oracle's fused step\n", (long long)bad);
  lioncub_destroy(ctx);
  hipFree(ws); hipFree(d_theta); hipFree(d_m); hipFree(d_g); hipFree(d_c); hipFree(d_codes);
  hipFree(d_wire); hipFree(d_sb); hipFree(d_zb);
  free(h_theta); free(h_m); free(h_g); free(h_c); free(r_theta); free(r_m);
  return bad != 0;
}

int main(void) {
  int fails = 0;
  fails += run_exchange();
  fails += run_case(LIONCUB_AGG_VOTE, 0, "vote", 0);
  fails += run_case(LIONCUB_AGG_L1SUM, 4, "l1-sum n=4", 0);
  fails += run_case(LIONCUB_AGG_AVG, 0, "average", 0);
  fails += run_case(LIONCUB_AGG_LINFSUM, 3, "max-norm n=3", 0);
  fails += run_case(LIONCUB_AGG_L1SUM, 8, "allocation-free l1-sum n=8", 1);
  fails += run_case(LIONCUB_AGG_VOTE, 0, "allocation-free vote", 1);
  printf(fails ? "FAILED\n" : "OK\n");
  return fails;
}
