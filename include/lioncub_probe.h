/*
 * lioncub_probe.h -- C ABI of liblioncub_probe.so, the measurement library
 * that sits beside the Lion Cub step library (lioncub.h).  Nothing here is
 * part of the method: these kernels measure what the device's memory system
 * delivers for the access patterns the step's kernels use, so a benchmark
 * can report the step's rate against the published 8 TB/s peak and against
 * what the same bytes reach when the arithmetic is trivial.
 *
 * Conventions as in lioncub.h: device buffers belong to the caller, every
 * call is asynchronous on the given stream (a hipStream_t; NULL = the null
 * stream), arguments are checked before anything is enqueued, status codes
 * are the LIONCUB_* codes, data pointers must be 16-byte aligned.
 */
#ifndef LIONCUB_PROBE_H
#define LIONCUB_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "lioncub.h"

#ifdef __cplusplus
extern "C" {
#endif

/* STREAM-style reference kernels with the step library's launch shape (256
 * threads, 4096 elements per workgroup, nontemporal 16-byte accesses):
 *   LIONCUB_PROBE_READ:  reads a[n] (c receives nothing; pass any buffer)
 *   LIONCUB_PROBE_COPY:  c[j] = a[j]
 *   LIONCUB_PROBE_TRIAD: c[j] = a[j] + 0.5f * b[j]
 * a, b, c: device fp32, not overlapping (b only for the triad); n: elements,
 * a positive multiple of 4096. */
enum { LIONCUB_PROBE_READ = 0, LIONCUB_PROBE_COPY = 1, LIONCUB_PROBE_TRIAD = 2 };
int lioncub_probe_stream(int32_t kind, const float *a, const float *b, float *c, int64_t n,
                         void *hip_stream);

/* The fused step's access pattern with trivial arithmetic: the same grid
 * (one 256-thread workgroup per 4096-element block of a flat vector), the
 * same per-thread quads (4 rounds of 4 consecutive elements), theta read
 * first, the workers walked two per batch with every m and g quad of the
 * batch loaded (nontemporal) before use, each worker's new m stored
 * (nontemporal) as soon as it is formed, theta written at the end -- so it
 * moves exactly the step's bytes, W*(4 + s_g + 4) + 2*s_theta per element,
 * in the step's order.  The arithmetic is only the momentum update
 * m <- beta2*m + (1 - beta2)*g and a count of positive new momenta that
 * moves theta by lr; no compression, no norms.
 *   theta: device [d] fp32 or bf16 per theta_dtype (read, written)
 *   m:     device [W][ld] fp32 (read, written)
 *   g:     device [W][ld] fp32 or bf16 per grad_dtype (read)
 *   d >= 1, ld >= d and a multiple of 64, W in 1..255.
 *   flags: 0, or any of
 *     LIONCUB_PROBE_CACHED: plain loads and stores instead of nontemporal
 *       ones (a working set smaller than the last-level cache can then stay
 *       there from one call to the next);
 *     LIONCUB_PROBE_MASKED: every block takes the per-lane predicated path
 *       the step kernel uses only for a ragged last block (the same bytes;
 *       its generated code waits for a wave's loads before each new quad,
 *       so about two are in flight per wave);
 *     LIONCUB_PROBE_CAP2 / _CAP4 / _CAP8 (not with the two above): the
 *       full-block path with at most 2, 4 or 8 vector-memory operations of
 *       a wave in flight while a batch's loads are issued;
 *     LIONCUB_PROBE_DRAIN_BATCH / _DRAIN_QUAD / _SERIAL (alone): the
 *       full-block path with the wave waiting for all its memory operations
 *       (stores included) before each batch's loads, before each quad's
 *       pair of loads, or before each pair of loads and each store. */
enum {
  LIONCUB_PROBE_CACHED = 1,
  LIONCUB_PROBE_MASKED = 2,
  LIONCUB_PROBE_CAP2 = 4,
  LIONCUB_PROBE_CAP4 = 8,
  LIONCUB_PROBE_CAP8 = 12,
  LIONCUB_PROBE_CAP_MASK = 12,
  LIONCUB_PROBE_DRAIN_BATCH = 16,
  LIONCUB_PROBE_DRAIN_QUAD = 32,
  LIONCUB_PROBE_SERIAL = 48,
  LIONCUB_PROBE_DRAIN_MASK = 48
};
int lioncub_probe_step_pattern(void *theta, float *m, const void *g, int64_t d, int64_t ld,
                               int32_t W, int32_t theta_dtype, int32_t grad_dtype, float beta2,
                               float lr, int32_t flags, void *hip_stream);

/* The same bytes in the arrangement the step does not use: one workgroup
 * per (4096-element block, worker), the grid worker-major within panels of
 * panel_blocks consecutive blocks (workgroup k: panel k/(panel_blocks*W),
 * then worker, then block), so the workgroups resident together stream one
 * worker's rows over a contiguous range, as a plain triad does; theta is
 * read and written by the last worker's workgroup.  Same arithmetic as
 * above per worker, but no aggregation across workers (theta moves by +-lr
 * from the last worker's momenta only): it measures what that arrangement
 * streams at, not a step.  Arguments as above; panel_blocks >= 1. */
int lioncub_probe_panel_pattern(void *theta, float *m, const void *g, int64_t d, int64_t ld,
                                int32_t W, int32_t theta_dtype, int32_t grad_dtype, float beta2,
                                float lr, int32_t panel_blocks, void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif
