/*
 * lco.c -- plain serial CPU oracle for the Lion Cub compressed-update step.
 *
 * TEST INFRASTRUCTURE ONLY (see lco.h): loaded by the tests, the smoke check
 * and the benchmark's CPU-baseline leg, never by the GPU library.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared
 *
 * Each function cites the passage it follows.  [LC] is the pith.science
 * review page of "Lion Cub: Minimizing Communication Overhead in Distributed
 * Lion"; [DL] is the atlas.scime.ai summary page of "Communication Efficient
 * Distributed Training with Distributed Lion".
 *
 * Parity pins (tests/test_oracle_pins.py): Lion closed forms, hand-worked
 * pack/vote/quantisation examples, brute force over all sign patterns for
 * W <= 5, exact rational arithmetic for Eq. (1) and for exactly summable
 * mean-|x| inputs, the summation error bound for the rest, invariants, and
 * torch's bf16 conversion.  The fixed order of the mean-|x| tree is a
 * definition of this project (the pages define M1 only as the mean of the
 * absolute values, with no order of summation); each level of it is pinned
 * by a hand-worked case (tests/golden/m1_order.json) whose sum a different
 * order would change.
 */
#include "lco.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- bf16 -- */

float lco_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

uint16_t lco_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0; /* NaN */
  /* round to nearest, ties to even, on the 16 dropped bits */
  uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

static float load_g(const lco_cfg *cfg, const void *g, int64_t k) {
  if (cfg->grad_bf16) return lco_bf16_to_f32(((const uint16_t *)g)[k]);
  return ((const float *)g)[k];
}

/* tensor holding element j (linear search: plain, not fast) */
static int32_t tensor_of(const lco_cfg *cfg, int64_t j) {
  int32_t T = 0;
  while (T + 1 < cfg->n_tensors && cfg->off[T + 1] <= j) T++;
  return T;
}

/* ------------------------------------------------- 1-bit compression [LC] */

/* [LC] "What carries the argument": signs packed as 0/1, exact zeros forced
 * to +1 or -1 on alternating iterations; the assumptions list fixes the order
 * (+1 on odd, -1 on even iterations).  t counts steps from 1.  Anything that
 * is neither > 0 nor < 0 (+0, -0, NaN) is treated as an exact zero. */
int lco_bit(float c, int64_t t) {
  if (c > 0.0f) return 1;
  if (c < 0.0f) return 0;
  return (int)(t & 1);
}

void lco_pack(int32_t W, int64_t d, int64_t ld, const float *x, int64_t t,
              uint64_t *bits) {
  int64_t words = ld / 64;
  for (int32_t i = 0; i < W; i++) {
    for (int64_t k = 0; k < words; k++) bits[i * words + k] = 0;
    for (int64_t j = 0; j < d; j++) {
      if (lco_bit(x[i * ld + j], t))
        bits[i * words + j / 64] |= (uint64_t)1 << (j % 64);
    }
  }
}

/* [LC] majority vote of the workers' signs; [DL] "Approach" (MaVo).  A tie
 * (2*count == W) is the zero that a 1-bit result cannot carry, so it follows
 * the same parity rule as an exact zero of c (LCO_TIE_PARITY), or stays 0
 * (LCO_TIE_ZERO). */
static int8_t vote_sign(int32_t W, int32_t count, int64_t t, int32_t tie_mode) {
  if (2 * count > W) return 1;
  if (2 * count < W) return -1;
  if (tie_mode == LCO_TIE_ZERO) return 0;
  return (t & 1) ? 1 : -1;
}

void lco_vote(int32_t W, int64_t d, int64_t ld, const uint64_t *bits,
              int64_t t, int32_t tie_mode, uint8_t *counts, int8_t *sign) {
  int64_t words = ld / 64;
  for (int64_t j = 0; j < d; j++) {
    int32_t v = 0;
    for (int32_t i = 0; i < W; i++)
      v += (int32_t)((bits[i * words + j / 64] >> (j % 64)) & 1u);
    if (counts) counts[j] = (uint8_t)v;
    if (sign) sign[j] = vote_sign(W, v, t, tie_mode);
  }
}

/* -------------------------------------------------- mean |x| (Eq. (1) M1) */

/* [LC] Eq. (1): M1 is the mean absolute value.  Summation order (D-M1, a
 * definition of this project so that any two implementations agree bit for
 * bit): a row is cut into blocks of 4096; in a block, lane l (0..255) takes
 * four rounds r, each over the four consecutive values at 1024*r + 4*l,
 * accumulating acc += ((e0 + e1) + (e2 + e3)) in fp64 from acc = 0; each group
 * of 64 lanes is folded by halving (a[q] += a[q+s] for s = 32, 16, .., 1); the
 * block partial is (w0 + w1) + (w2 + w3) over its four groups. */
static double fold64(double *a) {
  for (int s = LCO_M1_WAVE / 2; s >= 1; s /= 2)
    for (int q = 0; q < s; q++) a[q] = a[q] + a[q + s];
  return a[0];
}

double lco_m1_block(const float *a, int64_t n) {
  double acc[LCO_M1_LANES];
  for (int l = 0; l < LCO_M1_LANES; l++) {
    acc[l] = 0.0;
    for (int r = 0; r < 4; r++) {
      double e[4];
      for (int k = 0; k < 4; k++) {
        int64_t idx = 1024 * r + 4 * l + k;
        e[k] = idx < n ? fabs((double)a[idx]) : 0.0;
      }
      acc[l] = acc[l] + ((e[0] + e[1]) + (e[2] + e[3]));
    }
  }
  double wv[4];
  for (int w = 0; w < 4; w++) wv[w] = fold64(acc + LCO_M1_WAVE * w);
  return (wv[0] + wv[1]) + (wv[2] + wv[3]);
}

/* Finalize (three levels, so that no summation chain is long): the block
 * partials of a tensor, in block order, are cut into groups of 256; a group
 * value folds its partials like a block (partial l of the group in lane l,
 * 0.0 past the last block, halving folds per 64 lanes, then (w0 + w1) +
 * (w2 + w3)); lane l (0..63) sums group values l, l+64, l+128, ... in
 * increasing order from 0.0; the 64 lane sums are folded by halving; the
 * total is divided by the element count. */
static double fold_group(const double *P, int64_t cnt) {
  double acc[LCO_M1_LANES];
  for (int l = 0; l < LCO_M1_LANES; l++) acc[l] = l < cnt ? P[l] : 0.0;
  double wv[4];
  for (int w = 0; w < 4; w++) wv[w] = fold64(acc + LCO_M1_WAVE * w);
  return (wv[0] + wv[1]) + (wv[2] + wv[3]);
}

double lco_m1_finalize(const double *P, int64_t nb, int64_t nT) {
  int64_t ng = (nb + LCO_M1_LANES - 1) / LCO_M1_LANES;
  double p[LCO_M1_WAVE];
  for (int l = 0; l < LCO_M1_WAVE; l++) p[l] = 0.0;
  for (int64_t g = 0; g < ng; g++) {
    int64_t cnt = nb - g * LCO_M1_LANES;
    if (cnt > LCO_M1_LANES) cnt = LCO_M1_LANES;
    double G = fold_group(P + g * LCO_M1_LANES, cnt);
    p[g % LCO_M1_WAVE] = p[g % LCO_M1_WAVE] + G;
  }
  return fold64(p) / (double)nT;
}

double lco_m1(const float *x, int64_t n) {
  int64_t nb = (n + LCO_M1_BLOCK - 1) / LCO_M1_BLOCK;
  double *P = (double *)malloc((size_t)(nb > 0 ? nb : 1) * sizeof(double));
  for (int64_t b = 0; b < nb; b++) {
    int64_t len = n - b * LCO_M1_BLOCK;
    if (len > LCO_M1_BLOCK) len = LCO_M1_BLOCK;
    P[b] = lco_m1_block(x + b * LCO_M1_BLOCK, len);
  }
  double M = lco_m1_finalize(P, nb, n);
  free(P);
  return M;
}

/* [LC] Eq. (1): Q1(x) = clamp(round((2^(n-1)-1) * x / M1(x)), 2^(n-1)-1).
 * Readings: the clamp is symmetric, [-Qmax, +Qmax]; round is deterministic
 * half-to-even; the scale Qmax/M1 and the product c*scale are fp64; a row
 * with M1 == 0 (all zeros) gives all-zero codes. */
int8_t lco_q1(float c, double m1, int32_t qbits) {
  int32_t qmax = (1 << (qbits - 1)) - 1;
  if (m1 == 0.0) return 0;
  double scale = (double)qmax / m1;
  double r = rint((double)c * scale);
  if (r > (double)qmax) r = (double)qmax;
  if (r < -(double)qmax) r = -(double)qmax;
  return (int8_t)r;
}

void lco_quant_l1(const lco_cfg *cfg, int64_t ld, const float *x,
                  int8_t *codes, double *m1) {
  for (int32_t i = 0; i < cfg->W; i++) {
    for (int32_t T = 0; T < cfg->n_tensors; T++) {
      int64_t a = cfg->off[T], n = cfg->off[T + 1] - cfg->off[T];
      double M = lco_m1(x + i * ld + a, n);
      if (m1) m1[(int64_t)i * cfg->n_tensors + T] = M;
      for (int64_t j = a; j < a + n; j++)
        codes[i * ld + j] = lco_q1(x[i * ld + j], M, cfg->qbits);
    }
  }
}

/* ------------------------------------------------------------- the step -- */

/* [LC] "What carries the argument": c_{i,t} = beta1*m_{i,t-1} +
 * (1-beta1)*grad f_i(theta_{t-1}).  (1-beta1) is formed once in fp32. */
void lco_c_row(const lco_cfg *cfg, int64_t n, const float *m, const void *g,
               float *c) {
  float omega1 = 1.0f - cfg->beta1;
  for (int64_t k = 0; k < n; k++)
    c[k] = (cfg->beta1 * m[k]) + (omega1 * load_g(cfg, g, k));
}

void lco_m1_partials(const lco_cfg *cfg, int64_t n, const float *m, const void *g,
                     double *P) {
  float c[LCO_M1_BLOCK];
  size_t gsz = cfg->grad_bf16 ? 2 : 4;
  for (int64_t b = 0; b * LCO_M1_BLOCK < n; b++) {
    int64_t len = n - b * LCO_M1_BLOCK;
    if (len > LCO_M1_BLOCK) len = LCO_M1_BLOCK;
    lco_c_row(cfg, len, m + b * LCO_M1_BLOCK,
              (const char *)g + (size_t)(b * LCO_M1_BLOCK) * gsz, c);
    P[b] = lco_m1_block(c, len);
  }
}

void lco_m1_all(const lco_cfg *cfg, int64_t ld, const float *m, const void *g,
                double *m1) {
  size_t gsz = cfg->grad_bf16 ? 2 : 4;
  float *c = (float *)malloc((size_t)(cfg->d > 0 ? cfg->d : 1) * sizeof(float));
  for (int32_t i = 0; i < cfg->W; i++) {
    lco_c_row(cfg, cfg->d, m + i * ld, (const char *)g + (size_t)(i * ld) * gsz, c);
    for (int32_t T = 0; T < cfg->n_tensors; T++) {
      int64_t a = cfg->off[T], n = cfg->off[T + 1] - cfg->off[T];
      m1[(int64_t)i * cfg->n_tensors + T] = lco_m1(c + a, n);
    }
  }
  free(c);
}

/* Diagnostics of one column ([LC] Figure 4 and Figure 11: whether the
 * quantised update's sign matches or flips the sign of the unquantised one;
 * the reference-graph note on majority-vote ties; Figure 6: the spread of
 * the workers' momenta).  The unquantised aggregate is sum_i c_i in fp32,
 * summed in worker order; the momentum variance is S2/W - (S1/W)^2 with S1,
 * S2 the fp64 sums of m'_i and m'_i*m'_i in worker order, floored at 0. */
static void lco_column_stats(const lco_cfg *cfg, int32_t T, int32_t count, int8_t s,
                             float csum, const float *mcol, int64_t ldc,
                             const lco_debug *dbg) {
  const int32_t W = cfg->W;
  if (dbg->stats) {
    uint64_t *st = dbg->stats + 4 * (int64_t)T;
    int ref = (csum > 0.0f) - (csum < 0.0f);
    if ((cfg->agg == LCO_AGG_VOTE || cfg->agg == LCO_AGG_AVG) && 2 * count == W) st[0] += 1;
    if (s != 0 && s == ref) st[1] += 1;
    if (s != 0 && s == -ref) st[2] += 1;
    if (s == 0) st[3] += 1;
  }
  if (dbg->mvar_max) {
    double S1 = 0.0, S2 = 0.0;
    for (int32_t i = 0; i < W; i++) {
      double v = (double)mcol[i * ldc];
      S1 = S1 + v;
      S2 = S2 + (v * v);
    }
    double mean = S1 / (double)W;
    double var = (S2 / (double)W) - (mean * mean);
    if (var < 0.0) var = 0.0;
    if (var > dbg->mvar_max[T]) dbg->mvar_max[T] = var;
  }
}

/* One element column j: every worker's c from the pre-step m, compression,
 * aggregation, the global sign applied to theta (decoupled weight decay, the
 * Lion rule), then each worker's momentum update and, on averaging steps for
 * designated tensors, the worker mean of the new momenta ([LC] selective
 * momentum synchronisation of the input-embedding and output layers; the
 * interval is the sync_every parameter, 10 in the pages' runs). */
void lco_step_range(const lco_cfg *cfg, int64_t j0, int64_t j1,
                    const double *m1, void *theta, float *m, const void *g,
                    int64_t ldc, int64_t t, const lco_debug *dbg) {
  const int32_t W = cfg->W;
  const float omega1 = 1.0f - cfg->beta1;
  const float omega2 = 1.0f - cfg->beta2;
  const int avg_step = (t % cfg->sync_every) == 0;
  const int64_t words = ldc / 64;

  if (dbg && dbg->bits)
    for (int64_t k = 0; k < (int64_t)W * words; k++) dbg->bits[k] = 0;

  int32_t T = tensor_of(cfg, j0);
  for (int64_t j = j0; j < j1; j++) {
    const int64_t col = j - j0;
    while (T + 1 < cfg->n_tensors && cfg->off[T + 1] <= j) T++;

    /* 1-2: c per worker, compressed; 3: aggregated */
    int32_t count = 0, sum = 0;
    float csum = 0.0f;
    for (int32_t i = 0; i < W; i++) {
      float G = load_g(cfg, g, i * ldc + col);
      float c = (cfg->beta1 * m[i * ldc + col]) + (omega1 * G);
      csum = i == 0 ? c : csum + c;
      if (cfg->agg == LCO_AGG_VOTE || cfg->agg == LCO_AGG_AVG) {
        int b = lco_bit(c, t);
        count += b;
        if (dbg && dbg->bits && b)
          dbg->bits[i * words + col / 64] |= (uint64_t)1 << (col % 64);
      } else {
        int8_t q;
        if (cfg->agg == LCO_AGG_LINFSUM) {
          q = lco_qinf(c, m1[(int64_t)i * cfg->n_tensors + T], cfg->qbits,
                       lco_sr_u32(cfg->seed, cfg->d, W, t, i, j));
        } else {
          q = lco_q1(c, m1[(int64_t)i * cfg->n_tensors + T], cfg->qbits);
        }
        sum += q;
        if (dbg && dbg->codes) dbg->codes[i * ldc + col] = q;
      }
    }
    int8_t s;
    float sf;
    if (cfg->agg == LCO_AGG_VOTE) {
      s = vote_sign(W, count, t, cfg->tie_mode);
      sf = (float)s;
    } else if (cfg->agg == LCO_AGG_AVG) {
      /* [DL] "Approach": the server averages the workers' binary update
       * vectors, so the applied update is the mean of the W signs,
       * (count*(+1) + (W-count)*(-1)) / W, one fp32 division; the int8
       * sign output records its sign. */
      int32_t net = 2 * count - W;
      sf = (float)net / (float)W;
      s = (int8_t)((net > 0) - (net < 0));
    } else {
      /* [LC]: a global sign of the integer sum; the p-bit sum can carry
       * zero, so sgn(0) = 0 and the parameter only decays. */
      s = (int8_t)((sum > 0) - (sum < 0));
      sf = (float)s;
    }
    if (dbg && dbg->counts) dbg->counts[col] = (uint8_t)count;
    if (dbg && dbg->sums) dbg->sums[col] = sum;
    if (dbg && dbg->sign) dbg->sign[col] = s;

    /* 4: theta <- theta - lr*(sign + wd*theta) */
    if (cfg->theta_bf16) {
      uint16_t *th = (uint16_t *)theta;
      float x = lco_bf16_to_f32(th[col]);
      float y = x - (cfg->lr * (sf + (cfg->wd * x)));
      th[col] = lco_f32_to_bf16(y);
    } else {
      float *th = (float *)theta;
      float x = th[col];
      th[col] = x - (cfg->lr * (sf + (cfg->wd * x)));
    }

    /* 5: m_i <- beta2*m_i + (1-beta2)*g_i, then optional worker mean */
    for (int32_t i = 0; i < W; i++) {
      float G = load_g(cfg, g, i * ldc + col);
      m[i * ldc + col] = (cfg->beta2 * m[i * ldc + col]) + (omega2 * G);
    }
    if (dbg && (dbg->stats || dbg->mvar_max))
      lco_column_stats(cfg, T, count, s, csum, m + col, ldc, dbg);
    if (avg_step && cfg->sync_m && cfg->sync_m[T]) {
      float acc = m[col];
      for (int32_t i = 1; i < W; i++) acc = acc + m[i * ldc + col];
      float avg = acc / (float)W;
      for (int32_t i = 0; i < W; i++) m[i * ldc + col] = avg;
    }
  }
}

/* ------------------------------------ max-norm stochastic baseline ---- */

/* SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): the generator adds the
 * odd constant gamma to its state and mixes; as a counter-based generator
 * output k of the stream seeded s is mix(s + (k+1)*gamma).  Pinned to the
 * published first outputs. */
uint64_t lco_splitmix64(uint64_t seed, uint64_t counter) {
  uint64_t z = seed + (counter + 1u) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* The 32 random bits of element j of worker i at step t: the elements j and
 * j + 1 (j even) share output number (t*W + i)*d + j of the stream, the even
 * one taking its low 32 bits and the odd one its high 32 bits.  Counters
 * wrap mod 2^64.  (A reading: the pages give no generator.) */
uint32_t lco_sr_u32(uint64_t seed, int64_t d, int32_t W, int64_t t, int32_t i, int64_t j) {
  uint64_t ctr = ((uint64_t)t * (uint64_t)W + (uint64_t)i) * (uint64_t)d + ((uint64_t)j & ~(uint64_t)1);
  uint64_t r = lco_splitmix64(seed, ctr);
  return (j & 1) ? (uint32_t)(r >> 32) : (uint32_t)r;
}

double lco_minf(const float *x, int64_t n) {
  double mx = 0.0;
  for (int64_t k = 0; k < n; k++) {
    double a = fabs((double)x[k]);
    if (a > mx) mx = a;
  }
  return mx;
}

/* [LC] Figure 4 caption and the referee report on Eq. (1): the standard
 * max-normalised quantiser with stochastic rounding, the baseline Eq. (1) is
 * measured against; the pages name it but print no formula, so this is the
 * reading of Eq. (1) with max |x| for M1 and stochastic rounding:
 * floor(y) + [u < y - floor(y)], y = (2^(n-1)-1)/max|x| * x in fp64,
 * u = r * 2^-32 for 32 random bits r (lco_sr_u32), clamped.  The formula
 * is a reading; each of its steps is pinned: integer y, the threshold's
 * direction, the clamp, unbiasedness, the pages' zero-collapse finding, and
 * which published generator output and half each element draws
 * (tests/golden/sr_draws.json). */
int8_t lco_qinf(float c, double minf, int32_t qbits, uint32_t r) {
  int32_t qmax = (1 << (qbits - 1)) - 1;
  if (minf == 0.0) return 0;
  double scale = (double)qmax / minf;
  double y = (double)c * scale;
  double fl = floor(y);
  double frac = y - fl;
  double u = (double)r * 0x1.0p-32;
  double q = fl + (u < frac ? 1.0 : 0.0);
  if (q > (double)qmax) q = (double)qmax;
  if (q < -(double)qmax) q = -(double)qmax;
  return (int8_t)q;
}

void lco_quant_linf(const lco_cfg *cfg, int64_t ld, const float *x, int64_t t,
                    int8_t *codes, double *minf) {
  for (int32_t i = 0; i < cfg->W; i++) {
    for (int32_t T = 0; T < cfg->n_tensors; T++) {
      int64_t a = cfg->off[T], n = cfg->off[T + 1] - cfg->off[T];
      double M = lco_minf(x + i * ld + a, n);
      if (minf) minf[(int64_t)i * cfg->n_tensors + T] = M;
      for (int64_t j = a; j < a + n; j++)
        codes[i * ld + j] = lco_qinf(x[i * ld + j], M, cfg->qbits,
                                     lco_sr_u32(cfg->seed, cfg->d, cfg->W, t, i, j));
    }
  }
}

void lco_minf_all(const lco_cfg *cfg, int64_t ld, const float *m, const void *g,
                  double *minf) {
  size_t gsz = cfg->grad_bf16 ? 2 : 4;
  float *c = (float *)malloc((size_t)(cfg->d > 0 ? cfg->d : 1) * sizeof(float));
  for (int32_t i = 0; i < cfg->W; i++) {
    lco_c_row(cfg, cfg->d, m + i * ld, (const char *)g + (size_t)(i * ld) * gsz, c);
    for (int32_t T = 0; T < cfg->n_tensors; T++) {
      int64_t a = cfg->off[T], n = cfg->off[T + 1] - cfg->off[T];
      minf[(int64_t)i * cfg->n_tensors + T] = lco_minf(c + a, n);
    }
  }
  free(c);
}

/* ------------------- receive side and wire formats of the exchange ---- */

/* [LC] the 1-bit path: after the AlltoAll each worker votes on its slice and
 * the 1-bit result is all-gathered; a 2-bit result can also carry zero. */
void lco_vote_bits(int32_t W, int64_t d, int64_t ld, const uint64_t *bits,
                   int64_t t, int32_t tie_mode, uint64_t *sign_bits,
                   uint64_t *zero_bits) {
  int64_t words = ld / 64;
  for (int64_t k = 0; k < words; k++) {
    sign_bits[k] = 0;
    if (zero_bits) zero_bits[k] = 0;
  }
  for (int64_t j = 0; j < d; j++) {
    int32_t v = 0;
    for (int32_t i = 0; i < W; i++)
      v += (int32_t)((bits[i * words + j / 64] >> (j % 64)) & 1u);
    int8_t s = vote_sign(W, v, t, tie_mode);
    if (s > 0) sign_bits[j / 64] |= (uint64_t)1 << (j % 64);
    if (s == 0 && zero_bits) zero_bits[j / 64] |= (uint64_t)1 << (j % 64);
  }
}

void lco_apply(const lco_cfg *cfg, int64_t ld, void *theta, float *m,
               const void *g, int64_t t, const uint64_t *sign_bits,
               const uint64_t *zero_bits) {
  const int32_t W = cfg->W;
  const float omega2 = 1.0f - cfg->beta2;
  const int avg_step = (t % cfg->sync_every) == 0;
  int32_t T = 0;
  for (int64_t j = 0; j < cfg->d; j++) {
    while (T + 1 < cfg->n_tensors && cfg->off[T + 1] <= j) T++;
    int pos = (int)((sign_bits[j / 64] >> (j % 64)) & 1u);
    int zer = zero_bits ? (int)((zero_bits[j / 64] >> (j % 64)) & 1u) : 0;
    float sf = zer ? 0.0f : (pos ? 1.0f : -1.0f);
    if (cfg->theta_bf16) {
      uint16_t *th = (uint16_t *)theta;
      float x = lco_bf16_to_f32(th[j]);
      th[j] = lco_f32_to_bf16(x - (cfg->lr * (sf + (cfg->wd * x))));
    } else {
      float *th = (float *)theta;
      float x = th[j];
      th[j] = x - (cfg->lr * (sf + (cfg->wd * x)));
    }
    for (int32_t i = 0; i < W; i++) {
      float G = load_g(cfg, g, i * ld + j);
      m[i * ld + j] = (cfg->beta2 * m[i * ld + j]) + (omega2 * G);
    }
    if (avg_step && cfg->sync_m && cfg->sync_m[T]) {
      float acc = m[j];
      for (int32_t i = 1; i < W; i++) acc = acc + m[i * ld + j];
      float avg = acc / (float)W;
      for (int32_t i = 0; i < W; i++) m[i * ld + j] = avg;
    }
  }
}

/* [LC] the p-bit path sends Eq. (1) codes in n bits each (Figure 1: 1-bit
 * vs p-bit allreduce); the sum needs more bits than one code (the referee
 * report's note that a uint8 only fits 0/1 sums), hence int32 here. */
void lco_pack_codes(int32_t W, int64_t d, int64_t ld, int32_t qbits,
                    const int8_t *codes, uint32_t *wire) {
  int64_t wpr = (ld / 32) * qbits;
  uint32_t mask = (1u << qbits) - 1u;
  for (int32_t i = 0; i < W; i++) {
    for (int64_t k = 0; k < wpr; k++) wire[i * wpr + k] = 0;
    for (int64_t j = 0; j < d; j++) {
      uint32_t field = (uint32_t)(int32_t)codes[i * ld + j] & mask;
      int64_t bit = (j / 32) * 32 * qbits + (j % 32) * qbits;  /* bit offset in row */
      for (int32_t b = 0; b < qbits; b++)
        if ((field >> b) & 1u)
          wire[i * wpr + (bit + b) / 32] |= 1u << ((bit + b) % 32);
    }
  }
}

void lco_unpack_sum(int32_t W, int64_t d, int64_t ld, int32_t qbits,
                    const uint32_t *wire, int32_t *sums, int8_t *sign) {
  int64_t wpr = (ld / 32) * qbits;
  for (int64_t j = 0; j < d; j++) {
    int32_t S = 0;
    int64_t bit = (j / 32) * 32 * qbits + (j % 32) * qbits;
    for (int32_t i = 0; i < W; i++) {
      uint32_t field = 0;
      for (int32_t b = 0; b < qbits; b++)
        field |= ((wire[i * wpr + (bit + b) / 32] >> ((bit + b) % 32)) & 1u) << b;
      int32_t q = (field & (1u << (qbits - 1))) ? (int32_t)field - (1 << qbits)
                                                 : (int32_t)field;
      S += q;
    }
    if (sums) sums[j] = S;
    if (sign) sign[j] = (int8_t)((S > 0) - (S < 0));
  }
}

/* The p-bit receive side with the global sign as a 2-bit value per element
 * (the planes lco_apply takes): the integer sum of the W unpacked fields as
 * in lco_unpack_sum, sign bit where it is > 0, zero bit where it is 0 (the
 * p-bit sum can carry zero, so the parameter then only decays).  Every word
 * of the [ld/64] planes is written; bits past d are 0. */
void lco_unpack_sum_bits(int32_t W, int64_t d, int64_t ld, int32_t qbits,
                         const uint32_t *wire, uint64_t *sign_bits, uint64_t *zero_bits) {
  int64_t words = ld / 64;
  int32_t *S = (int32_t *)malloc((size_t)(d > 0 ? d : 1) * sizeof(int32_t));
  lco_unpack_sum(W, d, ld, qbits, wire, S, 0);
  for (int64_t w = 0; w < words; w++) {
    uint64_t sb = 0, zb = 0;
    for (int64_t k = 0; k < 64; k++) {
      int64_t j = 64 * w + k;
      if (j >= d) break;
      if (S[j] > 0) sb |= 1ull << k;
      if (S[j] == 0) zb |= 1ull << k;
    }
    sign_bits[w] = sb;
    if (zero_bits) zero_bits[w] = zb;
  }
  free(S);
}

void lco_step(const lco_cfg *cfg, int64_t ld, void *theta, float *m,
              const void *g, int64_t t, const lco_debug *dbg) {
  double *m1 = 0;
  if (cfg->agg == LCO_AGG_L1SUM || cfg->agg == LCO_AGG_LINFSUM) {
    m1 = (double *)malloc((size_t)cfg->W * cfg->n_tensors * sizeof(double));
    if (cfg->agg == LCO_AGG_L1SUM) lco_m1_all(cfg, ld, m, g, m1);
    else lco_minf_all(cfg, ld, m, g, m1);
  }
  lco_step_range(cfg, 0, cfg->d, m1, theta, m, g, ld, t, dbg);
  free(m1);
}
