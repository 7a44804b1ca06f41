/*
 * lco.h -- plain serial CPU oracle for the Lion Cub compressed-update step.
 *
 * TEST INFRASTRUCTURE ONLY.  This library defines, in slow and obviously
 * correct loops, what the GPU library computes.  Only the test-suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * source, header, table or helper with the GPU library, and the GPU library
 * never calls it.
 *
 * Sources (the web pages this method is described on):
 *   [LC]  "Lion Cub: Minimizing Communication Overhead in Distributed Lion",
 *         pith.science review page: section "What carries the argument"
 *         (the pre-sign update vector c_{i,t}, the 0/1 sign packing with
 *         exact zeros alternated by iteration parity, Eq. (1) L1
 *         quantisation), "Core claim", the assumptions list (zeros sent as
 *         +1 on odd and -1 on even iterations), Figure 1 and
 *         Figure 10 captions, and the reference-graph note that with 4
 *         workers over 30% of majority votes tie.
 *   [DL]  "Communication Efficient Distributed Training with Distributed
 *         Lion", atlas.scime.ai summary page: section "Approach" (each worker
 *         keeps its own momentum; majority vote / averaging of the binary
 *         update vectors).
 * The Lion update and momentum rules themselves (theta -= lr*(sign+wd*theta),
 * m = beta2*m + (1-beta2)*g) are the standard Lion optimizer the Lion Cub page
 * builds on (its reference "Symbolic Discovery of Optimization Algorithms").
 *
 * Every floating-point expression below is evaluated exactly as written, one
 * IEEE operation at a time, round-to-nearest-even, no contraction into FMA,
 * subnormals kept (build with -O2 -ffp-contract=off -fno-fast-math).
 *
 * Parity status of each function is stated beside it.
 */
#ifndef LCO_H
#define LCO_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { LCO_AGG_VOTE = 0, LCO_AGG_L1SUM = 1, LCO_AGG_AVG = 2, LCO_AGG_LINFSUM = 3 };
enum { LCO_TIE_PARITY = 0, LCO_TIE_ZERO = 1 };

/* Block / lane constants of the fixed mean-|x| summation tree (D-M1). */
enum { LCO_M1_BLOCK = 4096, LCO_M1_LANES = 256, LCO_M1_WAVE = 64 };

typedef struct {
  int64_t d;               /* parameters per worker                        */
  int32_t W;               /* simulated workers                            */
  int32_t n_tensors;       /* tensors in the flat parameter vector         */
  const int64_t *off;      /* n_tensors+1 ascending offsets, off[0]=0, off[n]=d */
  const uint8_t *sync_m;   /* n_tensors flags (momentum averaged) or NULL  */
  int32_t sync_every;      /* averaging on steps with t % sync_every == 0  */
  int32_t theta_bf16;      /* theta stored as bf16 (else fp32)             */
  int32_t grad_bf16;       /* g stored as bf16 (else fp32)                 */
  int32_t agg;             /* LCO_AGG_VOTE, _L1SUM, _AVG or _LINFSUM        */
  int32_t qbits;           /* n of Eq. (1), 2..8, L1 and max-norm paths    */
  int32_t tie_mode;        /* LCO_TIE_PARITY or LCO_TIE_ZERO, vote path    */
  float beta1, beta2, lr, wd;
  uint64_t seed;           /* stochastic rounding of the max-norm baseline  */
} lco_cfg;

/* bf16 <-> fp32: widening is exact; narrowing rounds to nearest-even,
 * NaN -> 0x7FC0.  Pinned against torch's fp32->bf16 conversion. */
float    lco_bf16_to_f32(uint16_t b);
uint16_t lco_f32_to_bf16(float f);

/* [LC] sign packing: 1 for c > 0, 0 for c < 0, exact zero (either sign)
 * takes the step parity: 1 on odd t, 0 on even t. */
int lco_bit(float c, int64_t t);

/* Pack x[W][ld] (first d of each row used) into bits[W][ld/64]: element j of
 * worker i is bit j%64 of word i*(ld/64) + j/64; bits at j >= d are 0. */
void lco_pack(int32_t W, int64_t d, int64_t ld, const float *x, int64_t t,
              uint64_t *bits);

/* Majority vote over the W bitmaps.  counts[j] = number of 1 bits; sign[j]
 * = +1 if 2*counts > W, -1 if 2*counts < W; a tie takes the step parity
 * (+1 odd t, -1 even t) under LCO_TIE_PARITY or 0 under LCO_TIE_ZERO.
 * Either output may be NULL. */
void lco_vote(int32_t W, int64_t d, int64_t ld, const uint64_t *bits,
              int64_t t, int32_t tie_mode, uint8_t *counts, int8_t *sign);

/* Fixed-order fp64 sum of |a| over one block of n <= 4096 values (D-M1
 * block partial).  Values past n count as +0.0. */
double lco_m1_block(const float *a, int64_t n);

/* M1 from the nb block partials of one (worker, tensor) of nT elements:
 * groups of 256 partials folded like a block, group values summed per lane
 * (lane l takes groups l, l+64, ...), lanes folded, divided by nT. */
double lco_m1_finalize(const double *P, int64_t nb, int64_t nT);

/* M1 of one row of n values (block partials + finalize). */
double lco_m1(const float *x, int64_t n);

/* Eq. (1) code of one value given the row's M1 and n = qbits. */
int8_t lco_q1(float c, double m1, int32_t qbits);

/* Standalone L1 quantisation of x[W][ld]: codes[W][ld] (first d of each row
 * written) and, if m1 != NULL, m1[W][n_tensors]. */
void lco_quant_l1(const lco_cfg *cfg, int64_t ld, const float *x,
                  int8_t *codes, double *m1);

/* c = beta1*m + (1-beta1)*G for n elements of one worker row (G = g widened
 * to fp32). */
void lco_c_row(const lco_cfg *cfg, int64_t n, const float *m, const void *g,
               float *c);

/* Block partials of n consecutive elements of one worker's row, starting at
 * a block boundary of its tensor: P[b] for the ceil(n/4096) blocks, c formed
 * from m and g as in lco_c_row.  Lets a caller stream a row in chunks. */
void lco_m1_partials(const lco_cfg *cfg, int64_t n, const float *m, const void *g,
                     double *P);

/* max |c| of every (worker, tensor) from the full state: [W][n_tensors]. */
void lco_minf_all(const lco_cfg *cfg, int64_t ld, const float *m, const void *g,
                  double *minf);

/* M1 of every (worker, tensor) from the full state: m1[W][n_tensors]. */
void lco_m1_all(const lco_cfg *cfg, int64_t ld, const float *m, const void *g,
                double *m1);

/* Optional per-element outputs of a step (any member may be NULL). */
typedef struct {
  uint64_t *bits;   /* [W][ldc/64]; needs j0 % 64 == 0 and ldc % 64 == 0 */
  int8_t   *codes;  /* [W][ldc]                                          */
  uint8_t  *counts; /* [j1-j0]                                           */
  int32_t  *sums;   /* [j1-j0]                                           */
  int8_t   *sign;   /* [j1-j0]                                           */
  /* Per-tensor diagnostics, accumulated (the caller zeroes them):
   * stats[T][0] ties (2*count == W, vote and averaging paths),
   * stats[T][1] match: applied sign == sgn(sum_i c_i) != 0,
   * stats[T][2] flip:  applied sign == -sgn(sum_i c_i) != 0,
   * stats[T][3] zero:  applied sign == 0;
   * mvar_max[T] = max over the tensor's elements of the inter-worker
   * variance of the new momenta (before any averaging). */
  uint64_t *stats;    /* [n_tensors][4] */
  double   *mvar_max; /* [n_tensors]    */
} lco_debug;

/* One step over the element range [j0, j1).  Chunk layout: element j of
 * worker i lives at m[i*ldc + (j-j0)], g likewise, theta at theta[j-j0].
 * m1 is m1[W][n_tensors] (L1 path: mean |c|; max-norm path: max |c|; may be
 * NULL on the vote and averaging paths). */
void lco_step_range(const lco_cfg *cfg, int64_t j0, int64_t j1,
                    const double *m1, void *theta, float *m, const void *g,
                    int64_t ldc, int64_t t, const lco_debug *dbg);

/* ---- max-norm (Q-infinity) stochastic quantisation: the baseline ------
 * A READING, PINNED STEP BY STEP: the pages name this quantiser as the baseline
 * that L1 replaces (Lion Cub review, Figure 4 caption: with stochastic
 * rounding it sends most entries to zero; the referee report on Eq. (1)
 * says the paper's section 2 defines that stochastic rounding) but never
 * print its formula.  Reading taken: the form of
 * Eq. (1) with the max |x| in place of the mean |x| and stochastic rounding
 * in place of rounding to nearest:
 *   q = clamp(floor(y) + [u < y - floor(y)], +-Qmax),  y = (Qmax / max|x|) * x
 * in fp64, u uniform in [0, 1) from the counter-based generator below.
 * Pinned: the generator's published first outputs, which output and half
 * an element draws (tuples worked by hand onto those published outputs),
 * exactness of max|x|, integer y (no randomness), the threshold's
 * direction, the clamp, unbiasedness E[q] = y, and the pages' claim that on
 * heavy-tailed updates most codes become 0.  What no pin can settle is
 * whether the paper's quantiser is this formula: the pages do not print it. */

/* SplitMix64 (Steele, Lea and Flood, 2014) used as a counter-based
 * generator: the counter-th output of the stream started at `seed`. */
uint64_t lco_splitmix64(uint64_t seed, uint64_t counter);

/* max |x| of one row of n values (exact: fp32 magnitudes, no rounding). */
double lco_minf(const float *x, int64_t n);

/* The 32 random bits of element j of worker i at step t: output number
 * (t*W + i)*d + (j with its lowest bit cleared) of the stream, its low 32
 * bits for even j and its high 32 bits for odd j (counters mod 2^64). */
uint32_t lco_sr_u32(uint64_t seed, int64_t d, int32_t W, int64_t t, int32_t i, int64_t j);

/* One stochastic code, u = r * 2^-32 for the element's 32 random bits r. */
int8_t lco_qinf(float c, double minf, int32_t qbits, uint32_t r);

/* Standalone max-norm quantisation of x[W][ld] for step t: element j of
 * worker i uses lco_sr_u32(seed, d, W, t, i, j). */
void lco_quant_linf(const lco_cfg *cfg, int64_t ld, const float *x, int64_t t,
                    int8_t *codes, double *minf);

/* ---- receive side and wire formats of the worker-sharded exchange ---- */

/* Global sign of the majority vote as bit planes: sign_bits[ld/64] has bit
 * 1 where the sign is +1; zero_bits[ld/64] (may be NULL) has bit 1 where it
 * is 0 (ties under LCO_TIE_ZERO).  Under LCO_TIE_PARITY a tie is carried by
 * the parity bit, as a 1-bit all-gather would carry it.  Bits past d are 0. */
void lco_vote_bits(int32_t W, int64_t d, int64_t ld, const uint64_t *bits,
                   int64_t t, int32_t tie_mode, uint64_t *sign_bits,
                   uint64_t *zero_bits);

/* Apply a global sign given as bit planes (zero_bits may be NULL: no zeros):
 * theta <- theta - lr*(s + wd*theta), then every worker's momentum update and
 * the selective averaging, exactly as steps 4-5 of lco_step. */
void lco_apply(const lco_cfg *cfg, int64_t ld, void *theta, float *m,
               const void *g, int64_t t, const uint64_t *sign_bits,
               const uint64_t *zero_bits);

/* n-bit wire packing of Eq. (1) codes: per worker row, every 32 elements
 * form one group of n 32-bit words; element k of a group occupies bits
 * n*k .. n*k+n-1 of the group's little-endian bit string, as an n-bit two's
 * complement integer.  Row stride (ld/32)*n words; elements past d are 0. */
void lco_pack_codes(int32_t W, int64_t d, int64_t ld, int32_t qbits,
                    const int8_t *codes, uint32_t *wire);

/* Receive side of the p-bit exchange: unpack every worker's codes of each
 * element, sum them in int32 and take the sign (sgn(0) = 0).  Either output
 * may be NULL. */
void lco_unpack_sum(int32_t W, int64_t d, int64_t ld, int32_t qbits,
                    const uint32_t *wire, int32_t *sums, int8_t *sign);

/* The same sums as lco_unpack_sum, delivered as the bit planes lco_apply
 * takes: sign_bits[ld/64] has bit 1 where the sum is > 0, zero_bits[ld/64]
 * (may be NULL) where it is 0; bits past d are 0. */
void lco_unpack_sum_bits(int32_t W, int64_t d, int64_t ld, int32_t qbits,
                         const uint32_t *wire, uint64_t *sign_bits, uint64_t *zero_bits);

/* One whole step in place on the full state (theta[d], m[W][ld], g[W][ld]). */
void lco_step(const lco_cfg *cfg, int64_t ld, void *theta, float *m,
              const void *g, int64_t t, const lco_debug *dbg);

#ifdef __cplusplus
}
#endif
#endif
