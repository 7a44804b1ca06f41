/*
 * lioncub.h -- C ABI of the MI355X (gfx950) Lion Cub compressed-update step.
 *
 * The method (sources: "Lion Cub: Minimizing Communication Overhead in
 * Distributed Lion", pith.science review page, section "What carries the
 * argument", Eq. (1) and the Figure 1 / Figure 10 captions; "Communication
 * Efficient Distributed Training with Distributed Lion", atlas.scime.ai
 * summary, section "Approach"):
 *
 *   W data-parallel workers each keep their own momentum m_i and gradient g_i.
 *   1. every worker forms c_i = beta1*m_i + (1-beta1)*g_i;
 *   2. c_i is compressed, either to a 0/1 sign bitmap (exact zeros take +1 on
 *      odd and -1 on even steps) or to n-bit integers by L1 quantisation,
 *      Q1(x) = clamp(round((2^(n-1)-1) * x / mean|x|), +-(2^(n-1)-1));
 *   3. the W compressed vectors are aggregated, by majority vote over the
 *      bitmaps or by an integer sum of the codes;
 *   4. the global sign is applied: theta <- theta - lr*(sign + wd*theta);
 *   5. each worker's momentum is updated, m_i <- beta2*m_i + (1-beta2)*g_i,
 *      and, for designated tensors (the input-embedding and output layers) on
 *      averaging steps, replaced by the worker mean.
 *
 * Here the W workers are stacked buffers in one GPU's memory and the
 * aggregation is a local kernel.
 *
 * Conventions for every entry point:
 *  - Buffers named "device" are device pointers owned by the caller; the
 *    library never allocates, frees or retains them past the call.
 *  - Every call is asynchronous, enqueued on the stream given at init (or by
 *    lioncub_set_stream), ordered with other work on that stream; no call
 *    synchronises the host except lioncub_init, lioncub_destroy and
 *    lioncub_profile_end.
 *  - Argument errors are detected before anything is enqueued and returned as
 *    a negative status; nothing is written then.  A failed launch returns
 *    LIONCUB_EDEVICE.  Faults inside a kernel surface at the caller's next
 *    synchronisation of the stream.
 *  - [W][ld] is worker-major: element j of worker i is at index i*ld + j.
 *    Rows hold d valid elements; ld >= d is a multiple of 64.
 *  - Bitmaps are little-endian uint64 words, least-significant bit first:
 *    element j of worker i is bit j%64 of word i*(ld/64) + j/64.  Bit 1 means
 *    +1 (c > 0, or c == 0 on an odd step).  Bits at j >= d are 0.
 *  - Data pointers must be 16-byte aligned; inputs and outputs must not
 *    overlap.  A context is not thread-safe; many contexts may coexist.
 *  - Floating point is IEEE round-to-nearest-even, one operation at a time,
 *    no fused multiply-add contraction, subnormals kept.  bf16 values are
 *    widened exactly and narrowed round-to-nearest-even; a NaN narrows to
 *    the quiet NaN 0x7FC0.
 */
#ifndef LIONCUB_H
#define LIONCUB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lioncub_ctx lioncub_ctx; /* opaque, host memory, owned by the library */

enum {
  LIONCUB_OK = 0,
  LIONCUB_EINVAL = -1,       /* bad argument or configuration             */
  LIONCUB_EALIGN = -2,       /* pointer not aligned as required           */
  LIONCUB_EWORKSPACE = -3,   /* workspace missing, misaligned or too small */
  LIONCUB_EDEVICE = -4,      /* HIP runtime / launch failure              */
  LIONCUB_EUNSUPPORTED = -5, /* valid request this library does not support */
  LIONCUB_ENOMEM = -6,       /* host memory for the context or its
                                profiling events could not be allocated   */
  LIONCUB_ESCRATCH = -7      /* lioncub_step_static: the configuration
                                needs more than the library's fixed device
                                scratch array (LIONCUB_STATIC_SCRATCH_BYTES) */
};

enum { LIONCUB_F32 = 0, LIONCUB_BF16 = 1 };
enum { LIONCUB_AGG_VOTE = 0, LIONCUB_AGG_L1SUM = 1, LIONCUB_AGG_AVG = 2, LIONCUB_AGG_LINFSUM = 3 };
enum { LIONCUB_TIE_PARITY = 0, LIONCUB_TIE_ZERO = 1 };

typedef struct {
  int64_t d;                     /* parameters per worker, >= 1                  */
  int64_t ld;                    /* row stride of [W][ld] buffers, >= d, % 64 == 0;
                                    above 2^40 (or more than 2^31-1 blocks of
                                    4096 per tensor summed) LIONCUB_EUNSUPPORTED */
  int32_t W;                     /* workers, 1..255                              */
  int32_t n_tensors;             /* tensors in the flat vector, >= 1             */
  const int64_t *tensor_offsets; /* HOST, n_tensors+1: off[0]=0 < off[1] < ... <
                                    off[n]=d; off[k] % 64 == 0 for k < n.  Read
                                    during lioncub_init (or lioncub_step_static) only. */
  const uint8_t *sync_m;         /* HOST, n_tensors flags (1 = momentum averaged
                                    over workers on averaging steps) or NULL.
                                    Read during lioncub_init (or
                                    lioncub_step_static) only.                   */
  int32_t sync_every;            /* >= 1: averaging on steps with t % sync_every == 0 */
  int32_t theta_dtype;           /* LIONCUB_F32 or LIONCUB_BF16                  */
  int32_t grad_dtype;            /* LIONCUB_F32 or LIONCUB_BF16; m is always fp32 */
  int32_t agg;                   /* LIONCUB_AGG_VOTE (majority vote of the sign
                                    bitmaps), LIONCUB_AGG_L1SUM (integer sum of
                                    Eq. (1) codes), LIONCUB_AGG_AVG (D-Lion
                                    averaging: the applied update is the mean
                                    of the W signs, (2*count - W) / W in fp32)
                                    or LIONCUB_AGG_LINFSUM (integer sum of the
                                    max-norm baseline's stochastic codes; see
                                    lioncub_quant_linf)                         */
  int32_t qbits;                 /* n of Eq. (1), 2..8; required for L1SUM,
                                    LINFSUM, lioncub_quant_l1 and
                                    lioncub_quant_linf, else ignored            */
  int32_t tie_mode;              /* vote ties (2*count == W): LIONCUB_TIE_PARITY
                                    (+1 odd t, -1 even t) or LIONCUB_TIE_ZERO (0) */
  float beta1, beta2, lr, wd;    /* finite                                       */
  uint64_t sr_seed;              /* key of the stochastic rounding of the
                                    max-norm codes (any value)                   */
} lioncub_config;

/* Optional per-element outputs of lioncub_step (each member may be NULL). */
typedef struct {
  uint64_t *bits;  /* device [W][ld/64]: the workers' sign bitmaps (vote path)  */
  int8_t *codes;   /* device [W][ld]: Eq. (1) or max-norm codes (quantised
                      paths); j >= d untouched                                 */
  uint8_t *counts; /* device [d]: number of +1 bits per element (vote path)     */
  int32_t *sums;   /* device [d]: integer sum of the codes (quantised paths)   */
  int8_t *sign;    /* device [d]: the global sign applied, in {-1, 0, +1}       */
  double *m1;      /* device [W][n_tensors]: the norm the codes divide by per
                      (worker, tensor): mean |c| (L1SUM) or max |c|
                      (LINFSUM); does not change which step kernel runs     */
  /* Per-tensor diagnostics of this step (written, not accumulated).
   * Sources: the Lion Cub page's Figure 4 / Figure 11 (does the quantised
   * update's sign match or flip the unquantised one), its note on majority
   * ties, and Figure 6 (spread of the workers' momenta).                  */
  uint64_t *stats; /* device [n_tensors][4]: ties (2*count == W, vote and
                      averaging paths), matches (applied sign == sgn of the
                      fp32 worker-order sum of c, nonzero), flips (== minus
                      it, nonzero), zero applied signs                        */
  double *mvar_max; /* device [n_tensors]: largest inter-worker variance of
                      the new momenta, S2/W - (S1/W)^2 with fp64 worker-order
                      sums S1, S2 of m' and m'^2, floored at 0                */
} lioncub_debug;

/* Bytes of device workspace lioncub_init needs for cfg (0 if cfg is invalid):
 * the block, tensor and group tables, the norm partials and scales, the
 * diagnostics' counters.  Pure host computation. */
size_t lioncub_workspace_bytes(const lioncub_config *cfg);

/* Validate cfg, lay out the caller's workspace (device, >= the bytes above,
 * 256-byte aligned, owned by the caller, must outlive the context and not be
 * touched by the caller while the context lives) and write the tensor, block
 * and group tables into it on hip_stream (a hipStream_t; NULL = the null
 * stream) with kernel launches.  Synchronises that stream once.  On success
 * *out receives a new context; LIONCUB_ENOMEM if the context's host memory
 * cannot be allocated. */
int lioncub_init(lioncub_ctx **out, const lioncub_config *cfg, void *hip_stream,
                 void *workspace, size_t ws_bytes);

/* Switch the stream later calls enqueue on. */
int lioncub_set_stream(lioncub_ctx *ctx, void *hip_stream);

/* One compressed-update step, steps 1-5 above, in place.
 *   theta: device [d], fp32 or bf16 per theta_dtype (read, written)
 *   m:     device [W][ld] fp32 (read, written; columns j >= d untouched)
 *   g:     device [W][ld], fp32 or bf16 per grad_dtype (read only)
 *   t:     1-based step index; decides zero and tie parity and averaging steps
 *   dbg:   NULL, or optional outputs (bits/counts on the vote and averaging
 *          paths, codes/sums/m1 on the quantised paths, sign and the
 *          diagnostics on all); an output of another path is an error
 *          (LIONCUB_EINVAL)
 * The vote and averaging paths are one kernel; the quantised paths are
 * three (norm block partials, per-(worker, tensor) norm and scale, then the
 * fused quantise-sum-apply). */
int lioncub_step(lioncub_ctx *ctx, void *theta, float *m, const void *g, int64_t t,
                 const lioncub_debug *dbg);

/* For callers that cannot allocate any memory -- code under stream capture,
 * tight serving loops, harnesses that forbid allocation: lioncub_step
 * without a context or a caller workspace.  The tables and norm partials of
 * the step live in a fixed array of device memory inside the library,
 * LIONCUB_STATIC_SCRATCH_BYTES per GPU, which each GPU the library runs on
 * holds from the time the library's code is loaded there until the process
 * ends.  The call allocates nothing (host or device), enqueues kernel
 * launches only on hip_stream (a hipStream_t of the current device, NULL =
 * its null stream) and rebuilds the tables in the array every call, so it
 * carries no state from one call to the next and needs no set-up or
 * teardown.
 *   cfg:   as for lioncub_init (its host arrays are read during the call
 *          only); the configuration must satisfy lioncub_workspace_bytes(cfg)
 *          <= LIONCUB_STATIC_SCRATCH_BYTES, else LIONCUB_ESCRATCH and
 *          nothing is enqueued
 *   theta, m, g, t: as for lioncub_step (no debug outputs)
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (on two streams, or from two host threads) race and their results are
 * undefined; calls ordered on one stream are safe.  LIONCUB_EINVAL if
 * hip_stream belongs to another device than the current one.  The first call
 * on each device looks up the array's device address there (the only
 * call that may synchronise). */
#define LIONCUB_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int lioncub_step_static(const lioncub_config *cfg, void *hip_stream, void *theta, float *m,
                        const void *g, int64_t t);

/* Sign packing of x = c directly: bits[W][ld/64] (device) from x[W][ld]
 * (device fp32), zeros by the parity of t (>= 1).  Every word of every row is
 * written, words past d with zeros. */
int lioncub_pack(lioncub_ctx *ctx, const float *x, int64_t t, uint64_t *bits);

/* Majority vote over bits[W][ld/64] (device): counts[d] (device, may be NULL)
 * = number of 1 bits, sign[d] (device, may be NULL) = +1 if 2*count > W, -1 if
 * 2*count < W, ties per tie_mode with the parity of t (>= 1).  At least one
 * output must be given. */
int lioncub_vote(lioncub_ctx *ctx, const uint64_t *bits, int64_t t, uint8_t *counts,
                 int8_t *sign);

/* L1 quantisation, Eq. (1), of x = c directly: codes[W][ld] (device int8,
 * columns j >= d untouched) and, if m1 != NULL, m1[W][n_tensors] (device
 * fp64) = mean |x| of each (worker, tensor), summed in fp64 in the library's
 * fixed order (blocks of 4096; within a block 256 lanes x 4 rounds of 4
 * consecutive values, acc += ((e0+e1)+(e2+e3)); 64-lane halving folds; block
 * partial (w0+w1)+(w2+w3); lane l of one 64-lane group sums partials l, l+64,
 * ... then folds), then divided by the tensor's element count.  A tensor
 * with mean 0 gets all-zero codes.  Needs qbits in 2..8 in the config. */
int lioncub_quant_l1(lioncub_ctx *ctx, const float *x, int8_t *codes, double *m1);

/* The max-norm baseline Eq. (1) is measured against (Lion Cub page, pith.
 * science review, Figure 4 caption and the referee report on Eq. (1): the
 * standard max-normalised quantiser with stochastic rounding; its formula is
 * not printed there, this is the reading taken):
 *   q = clamp(floor(y) + [u < y - floor(y)], +-(2^(n-1)-1)),
 *   y = (2^(n-1)-1) / max|x| * x in fp64 (scale 0 when max|x| == 0),
 *   u = b * 2^-32, b = the low 32 bits (even j) or the high 32 bits (odd j)
 *   of SplitMix64 output number (t*W + i)*d + (j & ~1) of the stream keyed
 *   by cfg.sr_seed, i.e. mix(sr_seed + (number+1)*0x9E3779B97F4A7C15) with
 *   Steele-Lea-Flood's mixer (shifts 30/27/31, multipliers
 *   0xBF58476D1CE4E5B9 and 0x94D049BB133111EB), all mod 2^64.
 * x[W][ld] (device fp32) -> codes[W][ld] (device int8, columns j >= d
 * untouched) and, if minf != NULL, minf[W][n_tensors] (device fp64) = max |x|
 * per (worker, tensor).  t >= 1 selects the draws (the fused step with
 * LIONCUB_AGG_LINFSUM at step t draws the same ones for c).  Needs qbits in
 * 2..8 in the config.  Codes of a row holding NaN or infinity are
 * unspecified. */
int lioncub_quant_linf(lioncub_ctx *ctx, const float *x, int64_t t, int8_t *codes,
                       double *minf);

/* ---- receive side and wire formats of the worker-sharded exchange -------
 * Sources: "Lion Cub: Minimizing Communication Overhead in Distributed Lion",
 * pith.science review ("What carries the argument": the 1-bit path packs
 * signs, votes and all-gathers a 1-bit result; the p-bit path sums n-bit
 * codes; Figure 1 caption; the referee report's note that the sum needs more
 * bits than a code).  On one GPU these operate on the context's whole
 * vector; on a cluster each GPU would run them on its slice.              */

/* Global sign of the majority vote over bits[W][ld/64] (device) as bit
 * planes: sign_bits[ld/64] (device, required) gets bit 1 where the sign is
 * +1; zero_bits[ld/64] (device, may be NULL) gets bit 1 where it is 0 (ties
 * under LIONCUB_TIE_ZERO; under LIONCUB_TIE_PARITY a tie is carried by the
 * parity of t in the sign plane, as a 1-bit all-gather carries it).  Every
 * word is written; bits past d are 0. */
int lioncub_vote_bits(lioncub_ctx *ctx, const uint64_t *bits, int64_t t,
                      uint64_t *sign_bits, uint64_t *zero_bits);

/* Steps 4-5 from a global sign given as bit planes (as lioncub_vote_bits
 * writes them; zero_bits may be NULL = no zeros): theta <- theta - lr*(s +
 * wd*theta) with s = zero ? 0 : (sign ? +1 : -1), then every worker's
 * momentum update and the selective averaging, exactly as lioncub_step.
 * theta/m/g as in lioncub_step; sign_bits/zero_bits device [ld/64]. */
int lioncub_apply(lioncub_ctx *ctx, void *theta, float *m, const void *g, int64_t t,
                  const uint64_t *sign_bits, const uint64_t *zero_bits);

/* n-bit wire packing of Eq. (1) codes, n = qbits of the config (2..8):
 * codes[W][ld] (device int8; values in [-(2^(n-1)-1), 2^(n-1)-1]; columns
 * j >= d ignored) -> wire[W][(ld/32)*n] (device uint32).  Per row, each 32
 * elements form a group of n words; element k of a group is the n-bit two's
 * complement field at bit n*k of the group's little-endian bit string.
 * Elements past d pack as 0. */
int lioncub_pack_codes(lioncub_ctx *ctx, const int8_t *codes, uint32_t *wire);

/* Receive side of the p-bit exchange: for every element, the W workers'
 * fields are unpacked from wire[W][(ld/32)*n] (device) and summed in int32:
 * sums[d] (device, may be NULL) and sign[d] (device int8, may be NULL; sgn,
 * 0 for a zero sum).  At least one output must be given. */
int lioncub_unpack_sum(lioncub_ctx *ctx, const uint32_t *wire, int32_t *sums, int8_t *sign);

/* The same receive side delivering the global sign as the 2-bit value per
 * element that lioncub_apply takes (the p-bit sum can be 0, so a 1-bit
 * plane does not carry it): from wire[W][(ld/32)*n] (device), sign_bits
 * [ld/64] (device, required) gets bit 1 where the int32 sum is > 0 and
 * zero_bits[ld/64] (device, may be NULL) bit 1 where it is 0.  Every word is
 * written; bits past d are 0.  quant_l1 -> pack_codes -> unpack_sum_bits ->
 * apply on the same state is exactly lioncub_step on the L1 path. */
int lioncub_unpack_sum_bits(lioncub_ctx *ctx, const uint32_t *wire, uint64_t *sign_bits,
                            uint64_t *zero_bits);

/* Measurement hook: while enabled, every kernel the context launches is
 * bracketed by HIP events on its stream (at most `capacity` launches are
 * recorded).  lioncub_profile_end synchronises on the events, disables the
 * hook and writes, per kernel kind k (LIONCUB_K_*), the summed duration in
 * ms_total[k] and the launch count in launches[k] (arrays of
 * LIONCUB_K_COUNT entries, host memory).  The norm pass of both quantised
 * paths (mean |c| or max |c|) is counted as M1_PARTIAL and M1_FINALIZE. */
enum {
  LIONCUB_K_VOTE_STEP = 0,
  LIONCUB_K_M1_PARTIAL = 1,
  LIONCUB_K_M1_FINALIZE = 2,
  LIONCUB_K_L1_STEP = 3,
  LIONCUB_K_PACK = 4,
  LIONCUB_K_VOTE = 5,
  LIONCUB_K_QUANT = 6,
  LIONCUB_K_VOTE_BITS = 7,
  LIONCUB_K_APPLY = 8,
  LIONCUB_K_PACK_CODES = 9,
  LIONCUB_K_UNPACK_SUM = 10,
  LIONCUB_K_AVG_STEP = 11,
  LIONCUB_K_STATS = 12,
  LIONCUB_K_LINF_STEP = 13,
  LIONCUB_K_QUANT_LINF = 14,
  LIONCUB_K_UNPACK_BITS = 15,
  LIONCUB_K_COUNT = 16
};
int lioncub_profile_begin(lioncub_ctx *ctx, int32_t capacity);
int lioncub_profile_end(lioncub_ctx *ctx, double *ms_total, int32_t *launches);

/* Release the context (host memory).  Synchronises its stream first.  NULL
 * is accepted. */
int lioncub_destroy(lioncub_ctx *ctx);

/* Static description of a status code. */
const char *lioncub_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif
