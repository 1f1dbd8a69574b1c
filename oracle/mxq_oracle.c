/*
 * mxq_oracle.c - plain, slow, scalar CPU oracle for MXNorm, RMSNorm -> MXCast
 * (two-pass, and the single-pass exact-RMS comparator), MXCast, the
 * straight-through backward of the normalisation, and the MX GEMM that
 * consumes the MX output.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this. It shares no code, header, table or constant
 * with the HIP library: every rule below is written out again here from the
 * pages and from the definitions of the number formats.
 *
 * Sources (page titles and sections):
 *  [MXN]  "MXNorm: Reusing MXFP block scales for efficient tensor normalisation"
 *         (gist.science technical summary): §1.1 (RMSNorm statistic over the
 *         hidden dim), §1.2 (RMSNorm and MXCast as separate steps), §2.1 (MX
 *         blocks of size B with one scale per block from the block absmax;
 *         m_k; the power mean G_K^(p); normalise by the approximation and cast
 *         in the same pass), §2.2 (Theorem 1, output bounds), §2.3 (gain folded
 *         into the next linear layer), §4 (drop-in, no new hyperparameter).
 *  [R8]   "Recipes for Pre-training LLMs with MXFP8" (fugumt abstract page):
 *         E4M3 as the MX element type; its related-paper entries
 *         "Microscaling Data Formats for Deep Learning" (per-block scale with
 *         narrow elements) and "FP8 Formats for Deep Learning" (E4M3 has no
 *         infinities and a single NaN mantissa pattern).
 *  [SR]   aibr.jp explainer on stochastic rounding with BF16 and Adam (opening
 *         dialogue and the core-technique paragraph): pick one of the two
 *         neighbouring representable values with probability set by the
 *         distance, so that the expectation equals the input.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *  - B = 32 elements per block along the hidden dim, D % 32 == 0.
 *  - E4M3 is the OCP "FN" variant: bias 7, no Inf, NaN = S.1111.111, max 448.
 *  - E2M1: bias 1, values {0, .5, 1, 1.5, 2, 3, 4, 6}, no Inf/NaN; element 2j
 *    in bits 3:0 of byte j, element 2j+1 in bits 7:4.
 *  - E8M0 scale of a block with absmax a: s = floor(log2 a) - emax, clamped to
 *    [-127, 127], stored as s + 127 (emax = 8 for E4M3, 2 for E2M1); a == 0
 *    gives code 0; a non-finite block gives code 0xFF and every element code
 *    is the NaN pattern (0x7F for E4M3, 0x7 for E2M1).
 *  - element rounding: round to nearest, ties to even, saturating at the
 *    format's largest finite value; the sign of zero is kept.
 *  - stochastic rounding: with q the value in units of the local quantum,
 *    n = floor(q), f = q - n, round up iff the top B bits of a 32-bit random
 *    word r are below the top B bits of f, i.e. r < 2^(32-B) * floor(f * 2^B),
 *    where B = 23 - (stored mantissa bits) is the number of fp32 mantissa bits
 *    the format drops at a normal target (20 for E4M3, 22 for E2M1);
 *    saturating; r comes from Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
 *    "Parallel random numbers: as easy as 1, 2, 3", SC'11) keyed by the
 *    64-bit seed, counter (n>>2 as two words, offset as two words), word
 *    (n & 3), n = t*D + d the logical element index. P(up) is f to within
 *    2^-B: unbiased to that precision.
 *  - MXNorm divides by G itself (no c(p,B) correction) and has no epsilon;
 *    G == 0 gives a zero normaliser; a row holding a NaN or Inf gives a NaN
 *    normaliser.
 *  - RMSNorm: y = gamma * x / sqrt(mean(x^2) + eps), rounded once to bf16 (the
 *    separate normalisation op emits a bf16 tensor). The single-pass
 *    comparator uses the same statistic but casts y without the bf16 step.
 *
 * NVFP4 (named by the MXNorm page, §3.2, and by a related-paper title on the
 * MXFP8 recipes page, but defined on neither; the reading below is the
 * published two-level format, written out in the design notes):
 *  - elements E2M1 as above, packed the same way; blocks of 16 consecutive
 *    elements along the row; one E4M3 scale byte per block; one fp32 tensor
 *    scale s_t in [2^-32, 2^32] given by the caller (decode: e2m1 * e4m3(scale)
 *    * s_t).
 *  - per block with a = max |y|: the scale byte is the E4M3 encoding (round
 *    to nearest even, saturating at 448) of RN32(a * k), k = RN32(1 / (6 s_t));
 *    with Sd its value, each element is the E2M1 encoding (RNE, saturating) of
 *    RN32(y * r), r = RN32(1 / RN32(Sd * s_t)), or r = 0 when Sd == 0 (the
 *    block then holds signed zeros); a block holding NaN or Inf gets scale
 *    0x7F (the E4M3 NaN) and element codes 0x7.
 *  - MXNorm over NVFP4 takes its statistic from the same blocks: m_k over 16
 *    elements, K = D / 16.
 *
 * Two modes for the normalising ops:
 *  (R) reference: statistic and normaliser in fp64, y in fp64, cast directly.
 *  (I) injected: takes a per-row fp32 normaliser and applies the fp32
 *      operation order y = RN32(RN32(x*gamma) * inv) (RMSNorm then rounds y to
 *      bf16); x*gamma of two bf16 values is exact in fp32.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_E4M3 0
#define ORC_E2M1 1
#define ORC_RNE 0
#define ORC_SR 1
#define ORC_SCALE_FLOOR 0
#define ORC_SCALE_CEIL 1

/* ------------------------------------------------------------------ */
/* Plain helpers                                                       */
/* ------------------------------------------------------------------ */

/* bf16 is the top half of an fp32; widening is exact. */
double orc_bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* floor(log2(a)) for a finite a > 0 (exact, via frexp: a = fr * 2^e, fr in [0.5, 1)). */
static int floor_log2(double a) {
  int e;
  frexp(a, &e);
  return e - 1;
}

/* Round a double to fp32 (C conversion: round to nearest even). */
static float rn32(double v) { return (float)v; }

/* Round to nearest, ties to even, of a >= 0 on the grid of multiples of 2^qe. */
static double rne_on_grid(double a, int qe) {
  double q = ldexp(a, -qe); /* exact */
  double n = floor(q);
  double f = q - n; /* exact */
  int up = (f > 0.5) || (f == 0.5 && fmod(n, 2.0) == 1.0);
  return ldexp(n + up, qe);
}

/* bf16 round-to-nearest-even of a double. Every NaN becomes the canonical
 * quiet NaN 0x7FC0: the pages give a NaN in the normalised tensor no sign or
 * payload, and the sign of a NaN made by arithmetic (Inf * 0 in RMSNorm of a
 * row holding an Inf) depends on the machine (x86 gives a negative one), so
 * the oracle fixes one pattern and comparisons treat all NaN patterns alike. */
uint16_t orc_bf16_rne(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isinf(a)) return sign | 0x7F80;
  if (a == 0) return sign;
  int e = floor_log2(a);
  if (e < -126) e = -126;           /* bf16 subnormals share fp32's exponent range */
  double mag = rne_on_grid(a, e - 7); /* 7 stored mantissa bits */
  if (mag >= ldexp(1.0, 128)) return sign | 0x7F80; /* overflow to Inf */
  float f = (float)mag;             /* exact: mag is on the bf16 grid */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return sign | (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ */
/* Element formats                                                     */
/* ------------------------------------------------------------------ */

/* E4M3 (OCP FN): s eeee mmm, bias 7; e == 0 subnormal m * 2^-9;
 * S.1111.111 is NaN; no Inf. */
double orc_e4m3_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return s ? -mag : mag;
}

/* E2M1: s ee m, bias 1; e == 0 subnormal m * 2^-1; no Inf or NaN. */
double orc_e2m1_decode(uint8_t c) {
  int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  double mag = (e == 0) ? ldexp((double)m, -1) : ldexp((double)(2 + m), e - 2);
  return s ? -mag : mag;
}

typedef struct {
  int ebits;     /* exponent bits */
  int mbits;     /* stored mantissa bits */
  int emin;      /* exponent of the smallest normal */
  double maxval; /* largest finite magnitude */
  int emax;      /* exponent of the largest binade (for the E8M0 rule) */
  uint8_t nan_code;
} fmt_t;

static const fmt_t FMT_E4M3 = {4, 3, -6, 448.0, 8, 0x7F};
static const fmt_t FMT_E2M1 = {2, 1, 0, 6.0, 2, 0x7};

static const fmt_t* fmt_of(int elem) { return elem == ORC_E2M1 ? &FMT_E2M1 : &FMT_E4M3; }

/* Bits of a magnitude that is exactly representable (and <= maxval). */
static uint8_t magnitude_bits(const fmt_t* F, double mag) {
  if (mag < ldexp(1.0, F->emin)) /* subnormal: mantissa = mag / quantum */
    return (uint8_t)ldexp(mag, F->mbits - F->emin);
  int e = floor_log2(mag);
  int bias = 1 - F->emin;
  int m = (int)ldexp(mag, F->mbits - e) - (1 << F->mbits);
  return (uint8_t)(((e + bias) << F->mbits) | m);
}

/* Encode a finite value already divided by the block scale.
 * RNE: nearest on the format grid, ties to the even code, saturating.
 * SR : round up iff r < 2^(32-B) * floor(f * 2^B), B = 23 - mbits (the top B
 *      bits of r against the top B bits of the fraction), saturating. */
static uint8_t encode_value(const fmt_t* F, int rnd, double v, uint32_t r) {
  uint8_t sign = signbit(v) ? (uint8_t)(1 << (F->ebits + F->mbits)) : 0;
  double a = fabs(v);
  if (a == 0) return sign;
  int e = floor_log2(a);
  if (e < F->emin) e = F->emin;
  int qe = e - F->mbits; /* quantum of the binade */
  double mag;
  if (rnd == ORC_RNE) {
    mag = rne_on_grid(a, qe);
  } else {
    double q = ldexp(a, -qe);
    double n = floor(q);
    double f = q - n;
    int B = 23 - F->mbits;
    double thr = ldexp(floor(ldexp(f, B)), 32 - B); /* exact: power-of-two scalings */
    int up = (double)r < thr;
    mag = ldexp(n + up, qe);
  }
  if (mag > F->maxval) mag = F->maxval;
  return sign | magnitude_bits(F, mag);
}

uint8_t orc_encode(int elem, int rnd, double v, uint32_t r) {
  return encode_value(fmt_of(elem), rnd, v, r);
}

/* Element-wise encode of n finite values (r may be NULL for RNE). */
void orc_encode_array(int elem, int rnd, const double* v, const uint32_t* r, int64_t n,
                      uint8_t* out) {
  const fmt_t* F = fmt_of(elem);
  for (int64_t i = 0; i < n; ++i) out[i] = encode_value(F, rnd, v[i], r ? r[i] : 0u);
}

/* E8M0 block scale from the block absmax. */
/* E8M0 scale of a block with absmax amax under one of two rules:
 *   floor (the OCP MX rule): s = floor(log2 amax) - emax;
 *   ceil  (round the scale up): the smallest s with amax <= maxval * 2^s, so
 *         no element of the block saturates (the pages' MXFP8 recipes abstract
 *         mentions a specific conversion algorithm without printing it; this
 *         is the reading that takes the scale up rather than clipping).
 * Clamped to [-127, 127], stored as s + 127; amax == 0 gives 0, NaN/Inf 0xFF. */
uint8_t orc_e8m0_scale_rule(int elem, double amax, int rule) {
  const fmt_t* F = fmt_of(elem);
  if (isnan(amax) || isinf(amax)) return 0xFF;
  if (amax == 0) return 0;
  int s = floor_log2(amax) - F->emax;
  if (rule == ORC_SCALE_CEIL) {
    while (ldexp(F->maxval, s) < amax) ++s;       /* smallest s that holds amax */
    while (ldexp(F->maxval, s - 1) >= amax) --s;
  }
  if (s < -127) s = -127;
  if (s > 127) s = 127;
  return (uint8_t)(s + 127);
}

uint8_t orc_e8m0_scale(int elem, double amax) {
  return orc_e8m0_scale_rule(elem, amax, ORC_SCALE_FLOOR);
}

/* ------------------------------------------------------------------ */
/* Philox (Salmon et al., SC'11): N = 4 words, 10 rounds.              */
/* Round: (c0,c1,c2,c3) -> (hi(M1*c2)^c1^k0, lo(M1*c2),                 */
/*                          hi(M0*c0)^c3^k1, lo(M0*c0));                */
/* the key is bumped by the Weyl constants between rounds.             */
/* One body serves both word widths so the 64-bit form, which numpy    */
/* also implements, checks the structure shared with the 32-bit form.  */
/* ------------------------------------------------------------------ */
#define PHILOX4_BODY(W, WW, M0, M1, W0, W1)                                 \
  W c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];                     \
  W k0 = key[0], k1 = key[1];                                               \
  for (int round = 0; round < 10; ++round) {                                \
    if (round > 0) {                                                        \
      k0 += (W)(W0);                                                        \
      k1 += (W)(W1);                                                        \
    }                                                                       \
    WW p0 = (WW)(M0) * (WW)c0;                                              \
    WW p1 = (WW)(M1) * (WW)c2;                                              \
    W n0 = (W)(p1 >> (8 * sizeof(W))) ^ c1 ^ k0;                            \
    W n1 = (W)p1;                                                           \
    W n2 = (W)(p0 >> (8 * sizeof(W))) ^ c3 ^ k1;                            \
    W n3 = (W)p0;                                                           \
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;                                     \
  }                                                                         \
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  PHILOX4_BODY(uint32_t, uint64_t, 0xD2511F53u, 0xCD9E8D57u, 0x9E3779B9u, 0xBB67AE85u)
}

void orc_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]) {
  PHILOX4_BODY(uint64_t, unsigned __int128, 0xD2E7470EE14C6C93ull, 0xCA5A826395121157ull,
               0x9E3779B97F4A7C15ull, 0xBB67AE8584CAA73Bull)
}

/* Random word for logical element index n under (seed, offset). */
uint32_t orc_sr_word(uint64_t seed, uint64_t offset, uint64_t n) {
  uint64_t blk = n >> 2;
  uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), (uint32_t)offset,
                     (uint32_t)(offset >> 32)};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  return out[n & 3];
}

/* Words for logical element indices n0 .. n0+count-1. */
void orc_sr_words(uint64_t seed, uint64_t offset, uint64_t n0, int64_t count, uint32_t* out) {
  for (int64_t i = 0; i < count; ++i) out[i] = orc_sr_word(seed, offset, n0 + (uint64_t)i);
}

/* ------------------------------------------------------------------ */
/* MXCast of one row of doubles                                        */
/* ------------------------------------------------------------------ */

/* v: D values of row t; writes D codes (unpacked, one per byte) and D/32 scales.
 * Element index for SR is t*D + d. */
static void mxcast_row_f64(const double* v, int64_t D, int64_t t, int elem, int rnd, int rule,
                           uint64_t seed, uint64_t offset, uint8_t* code_row,
                           uint8_t* scale_row) {
  const fmt_t* F = fmt_of(elem);
  for (int64_t k = 0; k < D / 32; ++k) {
    const double* b = v + 32 * k;
    double amax = 0;
    int nonfinite = 0;
    for (int i = 0; i < 32; ++i) {
      if (!isfinite(b[i])) nonfinite = 1;
      else if (fabs(b[i]) > amax) amax = fabs(b[i]);
    }
    uint8_t sc = orc_e8m0_scale_rule(elem, nonfinite ? NAN : amax, rule);
    scale_row[k] = sc;
    for (int i = 0; i < 32; ++i) {
      uint8_t c;
      if (sc == 0xFF) {
        c = F->nan_code;
      } else {
        double w = ldexp(b[i], -(sc - 127)); /* exact power-of-two division */
        uint32_t r = 0;
        if (rnd == ORC_SR) r = orc_sr_word(seed, offset, (uint64_t)t * (uint64_t)D + 32 * k + i);
        c = encode_value(F, rnd, w, r);
      }
      code_row[32 * k + i] = c;
    }
  }
}

/* Write one row's unpacked codes into the output layout. */
static void store_codes(int elem, const uint8_t* unpacked, int64_t D, uint8_t* out_row) {
  if (elem == ORC_E2M1) {
    for (int64_t j = 0; j < D / 2; ++j)
      out_row[j] = (uint8_t)((unpacked[2 * j] & 0xF) | ((unpacked[2 * j + 1] & 0xF) << 4));
  } else {
    memcpy(out_row, unpacked, (size_t)D);
  }
}

static int64_t code_bytes_per_row(int elem, int64_t D) { return elem == ORC_E2M1 ? D / 2 : D; }

static int check_args(int64_t T, int64_t D, int elem, int rnd, int rule, int64_t row_base) {
  if (T < 0 || D <= 0 || D % 32 != 0 || row_base < 0) return 2;
  if (elem != ORC_E4M3 && elem != ORC_E2M1) return 4;
  if (rnd != ORC_RNE && rnd != ORC_SR) return 4;
  if (rule != ORC_SCALE_FLOOR && rule != ORC_SCALE_CEIL) return 4;
  return 0;
}

/* MXCast on an arbitrary row of doubles (test helper for compositions). */
int orc_mxcast_f64(const double* v, int64_t D, int64_t t, int elem, int rnd, int rule,
                   uint64_t seed, uint64_t offset, uint8_t* codes_unpacked, uint8_t* scales) {
  if (check_args(1, D, elem, rnd, rule, t)) return 2;
  mxcast_row_f64(v, D, t, elem, rnd, rule, seed, offset, codes_unpacked, scales);
  return 0;
}

/* ------------------------------------------------------------------ */
/* The three operations                                                */
/* ------------------------------------------------------------------ */

/* Buffer conventions of the three operations: x holds T rows of D bf16 values
 * with row stride ldx; buffer row t is logical row row_base + t (the logical
 * row only enters the stochastic-rounding element index); codes [T, D] (E4M3)
 * or [T, D/2] (E2M1), scales [T, D/32] and the per-row arrays are contiguous. */

/* MXCast of a bf16 activation. */
int orc_mxcast(const uint16_t* x, int64_t ldx, int64_t T, int64_t D, int elem, int rnd, int rule,
               uint64_t seed, uint64_t offset, int64_t row_base, uint8_t* codes,
               uint8_t* scales) {
  int rc = check_args(T, D, elem, rnd, rule, row_base);
  if (rc) return rc;
  double* v = (double*)malloc(sizeof(double) * (size_t)D);
  uint8_t* cu = (uint8_t*)malloc((size_t)D);
  if (!v || !cu) { free(v); free(cu); return 6; }
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t d = 0; d < D; ++d) v[d] = orc_bf16_to_f64(x[t * ldx + d]);
    mxcast_row_f64(v, D, row_base + t, elem, rnd, rule, seed, offset, cu, scales + t * (D / 32));
    store_codes(elem, cu, D, codes + t * code_bytes_per_row(elem, D));
  }
  free(v);
  free(cu);
  return 0;
}

/* Generalised p-mean of K block maxima: ((1/K) sum m_k^p)^(1/p); p = inf -> max. */
double orc_pmean(const double* m, int64_t K, double p) {
  if (isinf(p)) {
    double g = 0;
    for (int64_t k = 0; k < K; ++k)
      if (m[k] > g) g = m[k];
    return g;
  }
  double s = 0;
  for (int64_t k = 0; k < K; ++k) s += pow(m[k], p);
  return pow(s / (double)K, 1.0 / p);
}

/* Fused MXNorm -> MX cast. inv_inject == NULL selects mode (R); otherwise mode
 * (I) with inv_inject[t] as the fp32 normaliser. inv_out (nullable) receives
 * the normaliser used (fp64 1/G in mode R). gamma == NULL means gamma == 1. */
int orc_mxnorm(const uint16_t* x, int64_t ldx, const uint16_t* gamma, int64_t T, int64_t D,
               double p, int elem, int rnd, int rule, uint64_t seed, uint64_t offset,
               int64_t row_base, const float* inv_inject, uint8_t* codes, uint8_t* scales,
               double* inv_out) {
  int rc = check_args(T, D, elem, rnd, rule, row_base);
  if (rc) return rc;
  if (!(p > 0)) return 5;
  const int64_t K = D / 32;
  double* y = (double*)malloc(sizeof(double) * (size_t)D);
  double* m = (double*)malloc(sizeof(double) * (size_t)K);
  uint8_t* cu = (uint8_t*)malloc((size_t)D);
  if (!y || !m || !cu) { free(y); free(m); free(cu); return 6; }
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* xr = x + t * ldx;
    double inv;
    if (inv_inject) {
      inv = (double)inv_inject[t];
    } else {
      int nonfinite = 0;
      for (int64_t k = 0; k < K; ++k) {
        double mk = 0;
        for (int i = 0; i < 32; ++i) {
          double xi = orc_bf16_to_f64(xr[32 * k + i]);
          if (!isfinite(xi)) nonfinite = 1;
          else if (fabs(xi) > mk) mk = fabs(xi);
        }
        m[k] = mk;
      }
      double G = orc_pmean(m, K, p);
      inv = nonfinite ? NAN : (G == 0 ? 0.0 : 1.0 / G);
    }
    if (inv_out) inv_out[t] = inv;
    for (int64_t d = 0; d < D; ++d) {
      double xi = orc_bf16_to_f64(xr[d]);
      double gi = gamma ? orc_bf16_to_f64(gamma[d]) : 1.0;
      if (inv_inject)
        y[d] = (double)rn32((double)rn32(xi * gi) * inv);
      else
        y[d] = xi * gi * inv; /* x*gamma is exact in double */
    }
    mxcast_row_f64(y, D, row_base + t, elem, rnd, rule, seed, offset, cu, scales + t * K);
    store_codes(elem, cu, D, codes + t * code_bytes_per_row(elem, D));
  }
  free(y);
  free(m);
  free(cu);
  return 0;
}

/* Two-pass comparison: RMSNorm (bf16 y) then MXCast(y). */
int orc_rmsnorm_mxcast(const uint16_t* x, int64_t ldx, const uint16_t* gamma, int64_t T,
                       int64_t D, double eps, int elem, int rnd, int rule, uint64_t seed,
                       uint64_t offset, int64_t row_base, const float* inv_inject,
                       uint16_t* ybf, uint8_t* codes, uint8_t* scales, double* inv_out) {
  int rc = check_args(T, D, elem, rnd, rule, row_base);
  if (rc) return rc;
  if (!(eps >= 0)) return 5;
  const int64_t K = D / 32;
  double* y = (double*)malloc(sizeof(double) * (size_t)D);
  uint8_t* cu = (uint8_t*)malloc((size_t)D);
  if (!y || !cu) { free(y); free(cu); return 6; }
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* xr = x + t * ldx;
    double inv;
    if (inv_inject) {
      inv = (double)inv_inject[t];
    } else {
      double s = 0;
      for (int64_t d = 0; d < D; ++d) {
        double xi = orc_bf16_to_f64(xr[d]);
        s += xi * xi;
      }
      inv = 1.0 / sqrt(s / (double)D + eps);
    }
    if (inv_out) inv_out[t] = inv;
    for (int64_t d = 0; d < D; ++d) {
      double xi = orc_bf16_to_f64(xr[d]);
      double gi = gamma ? orc_bf16_to_f64(gamma[d]) : 1.0;
      double yd = inv_inject ? (double)rn32((double)rn32(xi * gi) * inv) : xi * gi * inv;
      uint16_t b = orc_bf16_rne(yd);
      ybf[t * D + d] = b;
      y[d] = orc_bf16_to_f64(b);
    }
    mxcast_row_f64(y, D, row_base + t, elem, rnd, rule, seed, offset, cu, scales + t * K);
    store_codes(elem, cu, D, codes + t * code_bytes_per_row(elem, D));
  }
  free(y);
  free(cu);
  return 0;
}

/* Single-pass exact-RMS comparator: RMSNorm's statistic over all D elements
 * (MXNorm page, §1.1) in place of MXNorm's power mean, with y cast straight to
 * MX in the same pass as MXNorm does (§2.1), so y is never rounded to bf16.
 * (R): inv = 1/sqrt(mean(x^2) + eps) and y = x*gamma*inv in fp64. (I): the
 * injected fp32 inv and y = RN32(RN32(x*gamma)*inv). Outputs as orc_mxnorm. */
int orc_rmsnorm_fused_mxcast(const uint16_t* x, int64_t ldx, const uint16_t* gamma, int64_t T,
                             int64_t D, double eps, int elem, int rnd, int rule, uint64_t seed,
                             uint64_t offset, int64_t row_base, const float* inv_inject,
                             uint8_t* codes, uint8_t* scales, double* inv_out) {
  int rc = check_args(T, D, elem, rnd, rule, row_base);
  if (rc) return rc;
  if (!(eps >= 0)) return 5;
  const int64_t K = D / 32;
  double* y = (double*)malloc(sizeof(double) * (size_t)D);
  uint8_t* cu = (uint8_t*)malloc((size_t)D);
  if (!y || !cu) { free(y); free(cu); return 6; }
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* xr = x + t * ldx;
    double inv;
    if (inv_inject) {
      inv = (double)inv_inject[t];
    } else {
      double s = 0;
      for (int64_t d = 0; d < D; ++d) {
        double xi = orc_bf16_to_f64(xr[d]);
        s += xi * xi;
      }
      inv = 1.0 / sqrt(s / (double)D + eps);
    }
    if (inv_out) inv_out[t] = inv;
    for (int64_t d = 0; d < D; ++d) {
      double xi = orc_bf16_to_f64(xr[d]);
      double gi = gamma ? orc_bf16_to_f64(gamma[d]) : 1.0;
      y[d] = inv_inject ? (double)rn32((double)rn32(xi * gi) * inv) : xi * gi * inv;
    }
    mxcast_row_f64(y, D, row_base + t, elem, rnd, rule, seed, offset, cu, scales + t * K);
    store_codes(elem, cu, D, codes + t * code_bytes_per_row(elem, D));
  }
  free(y);
  free(cu);
  return 0;
}

/* ------------------------------------------------------------------ */
/* NVFP4                                                               */
/* ------------------------------------------------------------------ */

/* One row of values y (D of them, D % 16 == 0) to NVFP4: unpacked E2M1 codes
 * and D/16 E4M3 scale bytes. fp32 == 1: the fp32 operation order of the
 * reading (RN32 after each product and reciprocal; every product here is
 * exact in double, and the reciprocal of an fp32 value is never close enough
 * to an fp32 rounding midpoint for the double-then-float rounding to differ
 * from a direct one). fp32 == 0: the same rules in fp64 (reference mode of
 * the normalising op). */
static void nvfp4_row_f64(const double* y, int64_t D, double s_t, int fp32, uint8_t* code_row,
                          uint8_t* scale_row) {
  const double k = fp32 ? (double)rn32(1.0 / (6.0 * s_t)) : 1.0 / (6.0 * s_t);
  for (int64_t b = 0; b < D / 16; ++b) {
    const double* v = y + 16 * b;
    double amax = 0;
    int nonfinite = 0;
    for (int i = 0; i < 16; ++i) {
      if (!isfinite(v[i])) nonfinite = 1;
      else if (fabs(v[i]) > amax) amax = fabs(v[i]);
    }
    if (nonfinite) {
      scale_row[b] = 0x7F;
      for (int i = 0; i < 16; ++i) code_row[16 * b + i] = 0x7;
      continue;
    }
    double q = fp32 ? (double)rn32(amax * k) : amax * k;
    if (q > FMT_E4M3.maxval) q = FMT_E4M3.maxval; /* saturating (also keeps an fp32 Inf out) */
    const uint8_t sc = encode_value(&FMT_E4M3, ORC_RNE, q, 0);
    scale_row[b] = sc;
    const double Sd = orc_e4m3_decode(sc);
    for (int i = 0; i < 16; ++i) {
      double z;
      if (Sd == 0) {
        z = copysign(0.0, v[i]);
      } else if (fp32) {
        const double r = (double)rn32(1.0 / (double)rn32(Sd * s_t));
        z = (double)rn32(v[i] * r);
      } else {
        z = v[i] / (Sd * s_t);
      }
      code_row[16 * b + i] = encode_value(&FMT_E2M1, ORC_RNE, z, 0);
    }
  }
}

/* The tensor scale is taken in [2^-32, 2^32], where every quantity above stays
 * a finite, normal fp32 value. */
static int nvfp4_scale_ok(double s_t) { return s_t >= ldexp(1.0, -32) && s_t <= ldexp(1.0, 32); }

static int nvfp4_args(int64_t T, int64_t D, double s_t) {
  if (T < 0 || D <= 0 || D % 32 != 0) return 2;
  if (!nvfp4_scale_ok(s_t)) return 4;
  return 0;
}

/* NVFP4 cast of a bf16 activation: codes [T, D/2], scales [T, D/16]. The
 * fp32 order of the reading is the definition, so there is one mode. */
int orc_nvfp4_cast(const uint16_t* x, int64_t ldx, int64_t T, int64_t D, double s_t,
                   uint8_t* codes, uint8_t* scales) {
  int rc = nvfp4_args(T, D, s_t);
  if (rc) return rc;
  double* v = (double*)malloc(sizeof(double) * (size_t)D);
  uint8_t* cu = (uint8_t*)malloc((size_t)D);
  if (!v || !cu) { free(v); free(cu); return 6; }
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t d = 0; d < D; ++d) v[d] = orc_bf16_to_f64(x[t * ldx + d]);
    nvfp4_row_f64(v, D, s_t, 1, cu, scales + t * (D / 16));
    store_codes(ORC_E2M1, cu, D, codes + t * (D / 2));
  }
  free(v);
  free(cu);
  return 0;
}

/* MXNorm over NVFP4: G is the p-mean of the 16-element block maxima of |x|;
 * y as in orc_mxnorm; then the NVFP4 cast of y. inv_inject == NULL: mode (R)
 * (fp64 throughout); otherwise mode (I) with the given fp32 normalisers and
 * the fp32 order. */
int orc_mxnorm_nvfp4(const uint16_t* x, int64_t ldx, const uint16_t* gamma, int64_t T,
                     int64_t D, double p, double s_t, const float* inv_inject, uint8_t* codes,
                     uint8_t* scales, double* inv_out) {
  int rc = nvfp4_args(T, D, s_t);
  if (rc) return rc;
  if (!(p > 0)) return 5;
  const int64_t K = D / 16;
  double* y = (double*)malloc(sizeof(double) * (size_t)D);
  double* m = (double*)malloc(sizeof(double) * (size_t)K);
  uint8_t* cu = (uint8_t*)malloc((size_t)D);
  if (!y || !m || !cu) { free(y); free(m); free(cu); return 6; }
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* xr = x + t * ldx;
    double inv;
    if (inv_inject) {
      inv = (double)inv_inject[t];
    } else {
      int nonfinite = 0;
      for (int64_t b = 0; b < K; ++b) {
        double mb = 0;
        for (int i = 0; i < 16; ++i) {
          double xi = orc_bf16_to_f64(xr[16 * b + i]);
          if (!isfinite(xi)) nonfinite = 1;
          else if (fabs(xi) > mb) mb = fabs(xi);
        }
        m[b] = mb;
      }
      double G = orc_pmean(m, K, p);
      inv = nonfinite ? NAN : (G == 0 ? 0.0 : 1.0 / G);
    }
    if (inv_out) inv_out[t] = inv;
    for (int64_t d = 0; d < D; ++d) {
      double xi = orc_bf16_to_f64(xr[d]);
      double gi = gamma ? orc_bf16_to_f64(gamma[d]) : 1.0;
      y[d] = inv_inject ? (double)rn32((double)rn32(xi * gi) * inv) : xi * gi * inv;
    }
    nvfp4_row_f64(y, D, s_t, inv_inject != NULL, cu, scales + t * K);
    store_codes(ORC_E2M1, cu, D, codes + t * (D / 2));
  }
  free(y);
  free(m);
  free(cu);
  return 0;
}

/* NVFP4 block encode of 16 doubles (test helper for the pins): fp32 as in
 * nvfp4_row_f64. */
int orc_nvfp4_block(const double* v, double s_t, int fp32, uint8_t* codes_unpacked,
                    uint8_t* scale) {
  if (!nvfp4_scale_ok(s_t)) return 4;
  nvfp4_row_f64(v, 16, s_t, fp32, codes_unpacked, scale);
  return 0;
}

/* ------------------------------------------------------------------ */
/* Backward (straight-through)                                         */
/* ------------------------------------------------------------------ */

/* Backward of the normalisation with the cast taken as the identity (MXNorm
 * page, §2.3, gradient paragraph: RMSNorm's gradient computation is reused as a
 * straight-through estimator), with the forward's normaliser inv_t = 1/G_t in
 * the place of RMSNorm's 1/rms. Per row t, with g_i = gamma_i * dy_i:
 *   s_t  = sum_i g_i * x_i
 *   dx_i = inv_t * g_i - inv_t^3 * (s_t / D) * x_i
 * which is d/dx of gamma * x * r(x) for r = (mean(x^2))^(-1/2), with r's value
 * replaced by inv_t. (R): everything in fp64, dx rounded once to bf16.
 * (I): s_inject[t] is the kernel's fp32 row dot and the fp32 order is
 *   k = RN(RN(inv*inv)*inv); c = RN(k * RN(s/D)); dx = bf16(RN(RN(inv*g) - RN(c*x))).
 * s_out (nullable) receives the s used. dx is contiguous [T, D]. */
int orc_mxnorm_bwd(const uint16_t* x, int64_t ldx, const uint16_t* gamma, const uint16_t* dy,
                   int64_t lddy, const float* inv, int64_t T, int64_t D, const float* s_inject,
                   uint16_t* dx, double* s_out) {
  if (T < 0 || D <= 0) return 2;
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* xr = x + t * ldx;
    const uint16_t* dr = dy + t * lddy;
    double s;
    if (s_inject) {
      s = (double)s_inject[t];
    } else {
      s = 0;
      for (int64_t d = 0; d < D; ++d) {
        double gi = gamma ? orc_bf16_to_f64(gamma[d]) : 1.0;
        s += gi * orc_bf16_to_f64(dr[d]) * orc_bf16_to_f64(xr[d]);
      }
    }
    if (s_out) s_out[t] = s;
    const double a = (double)inv[t];
    for (int64_t d = 0; d < D; ++d) {
      double gi = gamma ? orc_bf16_to_f64(gamma[d]) : 1.0;
      double g = gi * orc_bf16_to_f64(dr[d]); /* exact in fp32 and fp64 */
      double xi = orc_bf16_to_f64(xr[d]);
      double v;
      if (s_inject) {
        float k = rn32((double)rn32(a * a) * a);
        float c = rn32((double)k * (double)rn32(s / (double)D));
        v = (double)rn32((double)rn32(a * g) - (double)rn32((double)c * xi));
      } else {
        v = a * g - a * a * a * (s / (double)D) * xi;
      }
      dx[t * D + d] = orc_bf16_rne(v);
    }
  }
  return 0;
}

/* Gradient of the gain: dgamma_i = sum_t dy_ti * x_ti * inv_t, in fp64, rows in
 * order (MXNorm page, §2.3: the gain of the normalisation). */
int orc_mxnorm_bwd_dgamma(const uint16_t* x, int64_t ldx, const uint16_t* dy, int64_t lddy,
                          const float* inv, int64_t T, int64_t D, double* dgamma,
                          double* abs_sum) {
  if (T < 0 || D <= 0) return 2;
  for (int64_t d = 0; d < D; ++d) {
    dgamma[d] = 0;
    if (abs_sum) abs_sum[d] = 0;
  }
  for (int64_t t = 0; t < T; ++t)
    for (int64_t d = 0; d < D; ++d) {
      double v = orc_bf16_to_f64(dy[t * lddy + d]) * orc_bf16_to_f64(x[t * ldx + d]) * (double)inv[t];
      dgamma[d] += v;
      if (abs_sum) abs_sum[d] += fabs(v);
    }
  return 0;
}

/* ------------------------------------------------------------------ */
/* MX GEMM (the consumer of the MX output)                             */
/* ------------------------------------------------------------------ */

/* Decoded value of element k of an MX row: code (unpacked from the E2M1 byte
 * pair when elem is E2M1) times the block's scale 2^(s - 127); a 0xFF scale
 * is NaN. */
static double mx_value(const uint8_t* codes_row, const uint8_t* scales_row, int elem, int64_t k) {
  uint8_t c;
  if (elem == ORC_E2M1) c = (uint8_t)((codes_row[k / 2] >> (4 * (k & 1))) & 0xF);
  else c = codes_row[k];
  uint8_t s = scales_row[k / 32];
  if (s == 0xFF) return NAN;
  double v = elem == ORC_E2M1 ? orc_e2m1_decode(c) : orc_e4m3_decode(c);
  return v * ldexp(1.0, (int)s - 127);
}

/* C[m][n] = sum_k A[m][k] * B[n][k] over MX operands: A is [M, K] with its
 * scales [M, K/32] (the MX cast of the activation, MXNorm page §2.1), B is
 * [N, K] with scales [N, K/32] (the next linear layer's weight, gain folded and
 * MX-cast along K, §2.3). fp64, k in order. abs_out (nullable) receives
 * sum_k |A[m][k] B[n][k]|. lda / ldb are code bytes per row, ldsa / ldsb scale
 * bytes per row. */
int orc_mx_gemm(const uint8_t* a, int64_t lda, const uint8_t* sa, int64_t ldsa, int elem_a,
                const uint8_t* b, int64_t ldb, const uint8_t* sb, int64_t ldsb, int elem_b,
                int64_t M, int64_t N, int64_t K, double* c, double* abs_out) {
  if (M < 0 || N < 0 || K <= 0 || K % 32 != 0) return 2;
  double* av = (double*)malloc(sizeof(double) * (size_t)K);
  if (!av) return 6;
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t k = 0; k < K; ++k) av[k] = mx_value(a + m * lda, sa + m * ldsa, elem_a, k);
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0, ab = 0;
      for (int64_t k = 0; k < K; ++k) {
        double p = av[k] * mx_value(b + n * ldb, sb + n * ldsb, elem_b, k);
        acc += p;
        ab += fabs(p);
      }
      c[m * N + n] = acc;
      if (abs_out) abs_out[m * N + n] = ab;
    }
  }
  free(av);
  return 0;
}
