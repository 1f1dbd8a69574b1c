/* Drives every entry point of the oracle (oracle/mxq_oracle.c, included
 * below) on small inputs, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer: every buffer is a heap allocation of exactly the
 * size the entry point's contract gives, so a read or write one byte outside it
 * stops the program. Covers both element formats and roundings, both scale
 * rules, p in {1, 2, 3.5, inf}, row strides above D, rows with zero, -0, NaN,
 * +-Inf, bf16-subnormal and extreme values, gains present and absent, both
 * oracle modes, the NVFP4 paths, the backward, the MX GEMM, and the status
 * codes of invalid arguments. Exits 0 when every call returned the status it
 * should; a sanitizer report exits non-zero. Test infrastructure only. */

#include "../../oracle/mxq_oracle.c"

#include <stdio.h>

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void) { /* xorshift64 */
  g_state ^= g_state << 13;
  g_state ^= g_state >> 7;
  g_state ^= g_state << 17;
  return (uint32_t)(g_state >> 32);
}

/* A bf16 pattern: mostly moderate magnitudes, sometimes a special value. */
static uint16_t next_bf16(void) {
  static const uint16_t special[] = {0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1,
                                     0x0001, 0x807F, 0x7F7F, 0xFF7F, 0x0080, 0x3F80};
  const uint32_t r = next_u32();
  if ((r & 63) == 0) return special[(r >> 6) % (sizeof special / sizeof special[0])];
  const uint32_t e = 112 + ((r >> 8) % 32);
  return (uint16_t)(((r >> 31) << 15) | (e << 7) | ((r >> 16) & 0x7F));
}

static void* xalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) abort();
  return p;
}

static uint16_t* bf16_buffer(int64_t n) {
  uint16_t* p = (uint16_t*)xalloc(sizeof(uint16_t) * (size_t)n);
  for (int64_t i = 0; i < n; ++i) p[i] = next_bf16();
  return p;
}

static int g_failures = 0;

#define EXPECT(expr, want)                                                                  \
  do {                                                                                      \
    const int rc_ = (int)(expr);                                                            \
    if (rc_ != (want)) {                                                                    \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #expr,    \
              rc_, (int)(want));                                                            \
      ++g_failures;                                                                         \
    }                                                                                       \
  } while (0)

static void scalars(void) {
  for (uint32_t h = 0; h < 65536; ++h) (void)orc_bf16_rne(orc_bf16_to_f64((uint16_t)h));
  for (int c = 0; c < 256; ++c) (void)orc_e4m3_decode((uint8_t)c);
  for (int c = 0; c < 16; ++c) (void)orc_e2m1_decode((uint8_t)c);
  /* the element encoder takes finite values (its contract); the scale rule
     takes any absmax, NaN and Inf included */
  const double vals[] = {0.0, -0.0, 1e-45, 0.3, -1.75, 6.5, 448.0, 480.0, 1e30, -1e30,
                         INFINITY, -INFINITY, NAN};
  for (size_t i = 0; i < sizeof vals / sizeof vals[0]; ++i)
    for (int elem = 0; elem < 2; ++elem) {
      if (isfinite(vals[i]))
        for (int rnd = 0; rnd < 2; ++rnd) (void)orc_encode(elem, rnd, vals[i], next_u32());
      for (int rule = 0; rule < 2; ++rule) (void)orc_e8m0_scale_rule(elem, fabs(vals[i]), rule);
      (void)orc_e8m0_scale(elem, fabs(vals[i]));
    }
  const int64_t n = 37;
  double* v = (double*)xalloc(sizeof(double) * n);
  uint32_t* r = (uint32_t*)xalloc(sizeof(uint32_t) * n);
  uint8_t* out = (uint8_t*)xalloc((size_t)n);
  for (int64_t i = 0; i < n; ++i) {
    do v[i] = orc_bf16_to_f64(next_bf16()); while (!isfinite(v[i]));
    r[i] = next_u32();
  }
  for (int elem = 0; elem < 2; ++elem)
    for (int rnd = 0; rnd < 2; ++rnd) orc_encode_array(elem, rnd, v, r, n, out);
  free(v), free(r), free(out);

  uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, o32[4];
  orc_philox4x32_10(ctr, key, o32);
  uint64_t c64[4] = {1, 2, 3, 4}, k64[2] = {5, 6}, o64[4];
  orc_philox4x64_10(c64, k64, o64);
  (void)orc_sr_word(0x5EED, 7, 123456789);
  uint32_t* words = (uint32_t*)xalloc(sizeof(uint32_t) * 13);
  orc_sr_words(0x5EED, 7, 5, 13, words);
  free(words);

  double* m = (double*)xalloc(sizeof(double) * 5);
  const double ps[] = {1.0, 2.0, 3.5, INFINITY};
  for (int k = 0; k < 5; ++k) m[k] = k == 2 ? 0.0 : 0.25 * (k + 1);
  for (int i = 0; i < 4; ++i) (void)orc_pmean(m, 5, ps[i]);
  free(m);
}

/* The three forward operations and MXCast of a double row, on T rows of D
 * elements with row stride ldx. */
/* MXQ_PLANT_SHORT_SCALES: the scales buffer of the forward operations one
 * byte short, so that a build of this drive shows the sanitizer reporting the
 * oracle's last scale write (a check of the check, on the CPU). */
#ifdef MXQ_PLANT_SHORT_SCALES
#define SCALES_SHORT 1
#else
#define SCALES_SHORT 0
#endif

static void forward_ops(int64_t T, int64_t D, int64_t ldx) {
  const int64_t K = D / 32;
  uint16_t* x = bf16_buffer(T * ldx);
  uint16_t* gamma = bf16_buffer(D);
  float* inj = (float*)xalloc(sizeof(float) * (size_t)T);
  for (int64_t t = 0; t < T; ++t) inj[t] = t == 1 ? INFINITY : 0.5f + (float)t;
  double* inv_out = (double*)xalloc(sizeof(double) * (size_t)T);
  uint16_t* ybf = (uint16_t*)xalloc(sizeof(uint16_t) * (size_t)(T * D));
  uint8_t* scales = (uint8_t*)xalloc((size_t)(T * K) - SCALES_SHORT);
  const double ps[] = {1.0, 2.0, 3.5, INFINITY};
  for (int elem = 0; elem < 2; ++elem) {
    const int64_t cb = elem == ORC_E2M1 ? D / 2 : D;
    uint8_t* codes = (uint8_t*)xalloc((size_t)(T * cb));
    for (int rnd = 0; rnd < 2; ++rnd)
      for (int rule = 0; rule < 2; ++rule) {
        EXPECT(orc_mxcast(x, ldx, T, D, elem, rnd, rule, 0x5EED, 3, 11, codes, scales), 0);
        for (int pi = 0; pi < 4; ++pi)
          for (int g = 0; g < 2; ++g)
            for (int mode = 0; mode < 2; ++mode)
              EXPECT(orc_mxnorm(x, ldx, g ? gamma : NULL, T, D, ps[pi], elem, rnd, rule, 0x5EED,
                                3, 11, mode ? inj : NULL, codes, scales, inv_out),
                     0);
        for (int g = 0; g < 2; ++g)
          for (int mode = 0; mode < 2; ++mode) {
            EXPECT(orc_rmsnorm_mxcast(x, ldx, g ? gamma : NULL, T, D, 1e-5, elem, rnd, rule, 0x5EED,
                                      3, 11, mode ? inj : NULL, ybf, codes, scales, inv_out),
                   0);
            EXPECT(orc_rmsnorm_fused_mxcast(x, ldx, g ? gamma : NULL, T, D, 1e-5, elem, rnd, rule,
                                            0x5EED, 3, 11, mode ? inj : NULL, codes, scales,
                                            inv_out),
                   0);
          }
      }
    free(codes);
  }
  double* row = (double*)xalloc(sizeof(double) * (size_t)D);
  uint8_t* cu = (uint8_t*)xalloc((size_t)D);
  uint8_t* srow = (uint8_t*)xalloc((size_t)K);
  for (int64_t d = 0; d < D; ++d) row[d] = orc_bf16_to_f64(x[d]) * 3.0;
  for (int elem = 0; elem < 2; ++elem)
    EXPECT(orc_mxcast_f64(row, D, 5, elem, ORC_SR, ORC_SCALE_CEIL, 1, 2, cu, srow), 0);
  free(row), free(cu), free(srow);
  free(x), free(gamma), free(inj), free(inv_out), free(ybf), free(scales);
}

static void nvfp4_ops(int64_t T, int64_t D, int64_t ldx) {
  uint16_t* x = bf16_buffer(T * ldx);
  uint16_t* gamma = bf16_buffer(D);
  float* inj = (float*)xalloc(sizeof(float) * (size_t)T);
  for (int64_t t = 0; t < T; ++t) inj[t] = 0.75f;
  double* inv_out = (double*)xalloc(sizeof(double) * (size_t)T);
  uint8_t* codes = (uint8_t*)xalloc((size_t)(T * D / 2));
  uint8_t* scales = (uint8_t*)xalloc((size_t)(T * D / 16));
  const double sts[] = {1.0, 0.375, 3000.0};
  for (int i = 0; i < 3; ++i) {
    EXPECT(orc_nvfp4_cast(x, ldx, T, D, sts[i], codes, scales), 0);
    for (int g = 0; g < 2; ++g)
      for (int mode = 0; mode < 2; ++mode)
        EXPECT(orc_mxnorm_nvfp4(x, ldx, g ? gamma : NULL, T, D, 2.0, sts[i], mode ? inj : NULL,
                                codes, scales, inv_out),
               0);
  }
  double* v = (double*)xalloc(sizeof(double) * 16);
  uint8_t* cu = (uint8_t*)xalloc(16);
  uint8_t* sc = (uint8_t*)xalloc(1);
  for (int i = 0; i < 16; ++i) v[i] = orc_bf16_to_f64(next_bf16());
  for (int fp32 = 0; fp32 < 2; ++fp32) EXPECT(orc_nvfp4_block(v, 1.0, fp32, cu, sc), 0);
  free(v), free(cu), free(sc);
  free(x), free(gamma), free(inj), free(inv_out), free(codes), free(scales);
}

static void backward_ops(int64_t T, int64_t D, int64_t ldx, int64_t lddy) {
  uint16_t* x = bf16_buffer(T * ldx);
  uint16_t* dy = bf16_buffer(T * lddy);
  uint16_t* gamma = bf16_buffer(D);
  float* inv = (float*)xalloc(sizeof(float) * (size_t)T);
  float* s_inj = (float*)xalloc(sizeof(float) * (size_t)T);
  for (int64_t t = 0; t < T; ++t) inv[t] = 0.5f + (float)t, s_inj[t] = 2.0f - (float)t;
  uint16_t* dx = (uint16_t*)xalloc(sizeof(uint16_t) * (size_t)(T * D));
  double* s_out = (double*)xalloc(sizeof(double) * (size_t)T);
  double* dgamma = (double*)xalloc(sizeof(double) * (size_t)D);
  double* abs_sum = (double*)xalloc(sizeof(double) * (size_t)D);
  for (int g = 0; g < 2; ++g)
    for (int mode = 0; mode < 2; ++mode)
      EXPECT(orc_mxnorm_bwd(x, ldx, g ? gamma : NULL, dy, lddy, inv, T, D, mode ? s_inj : NULL, dx,
                            s_out),
             0);
  EXPECT(orc_mxnorm_bwd_dgamma(x, ldx, dy, lddy, inv, T, D, dgamma, abs_sum), 0);
  EXPECT(orc_mxnorm_bwd_dgamma(x, ldx, dy, lddy, inv, T, D, dgamma, NULL), 0);
  free(x), free(dy), free(gamma), free(inv), free(s_inj), free(dx), free(s_out), free(dgamma);
  free(abs_sum);
}

static void gemm_ops(int64_t M, int64_t N, int64_t K) {
  for (int ea = 0; ea < 2; ++ea)
    for (int eb = 0; eb < 2; ++eb) {
      const int64_t lda = (ea == ORC_E2M1 ? K / 2 : K) + 16, ldb = (eb == ORC_E2M1 ? K / 2 : K);
      const int64_t ldsa = K / 32 + 4, ldsb = K / 32;
      uint8_t* a = (uint8_t*)xalloc((size_t)(M * lda));
      uint8_t* b = (uint8_t*)xalloc((size_t)(N * ldb));
      uint8_t* sa = (uint8_t*)xalloc((size_t)(M * ldsa));
      uint8_t* sb = (uint8_t*)xalloc((size_t)(N * ldsb));
      for (int64_t i = 0; i < M * lda; ++i) a[i] = (uint8_t)next_u32();
      for (int64_t i = 0; i < N * ldb; ++i) b[i] = (uint8_t)next_u32();
      for (int64_t i = 0; i < M * ldsa; ++i) sa[i] = (uint8_t)(120 + next_u32() % 16);
      for (int64_t i = 0; i < N * ldsb; ++i) sb[i] = (uint8_t)(i == 1 ? 0xFF : 120 + next_u32() % 16);
      double* c = (double*)xalloc(sizeof(double) * (size_t)(M * N));
      double* ab = (double*)xalloc(sizeof(double) * (size_t)(M * N));
      EXPECT(orc_mx_gemm(a, lda, sa, ldsa, ea, b, ldb, sb, ldsb, eb, M, N, K, c, ab), 0);
      EXPECT(orc_mx_gemm(a, lda, sa, ldsa, ea, b, ldb, sb, ldsb, eb, M, N, K, c, NULL), 0);
      free(a), free(b), free(sa), free(sb), free(c), free(ab);
    }
}

static void invalid_arguments(void) {
  uint16_t x[64] = {0};
  uint8_t codes[64], scales[4];
  double inv[2], c[4], dg[32];
  float f[2] = {1.0f, 1.0f};
  uint16_t dx[64];
  EXPECT(orc_mxcast(x, 32, -1, 32, ORC_E4M3, ORC_RNE, 0, 0, 0, 0, codes, scales), 2);
  EXPECT(orc_mxcast(x, 48, 1, 48, ORC_E4M3, ORC_RNE, 0, 0, 0, 0, codes, scales), 2);
  EXPECT(orc_mxcast(x, 32, 1, 32, 7, ORC_RNE, 0, 0, 0, 0, codes, scales), 4);
  EXPECT(orc_mxcast(x, 32, 1, 32, ORC_E4M3, 9, 0, 0, 0, 0, codes, scales), 4);
  EXPECT(orc_mxcast(x, 32, 1, 32, ORC_E4M3, ORC_RNE, 5, 0, 0, 0, codes, scales), 4);
  EXPECT(orc_mxcast(x, 32, 1, 32, ORC_E4M3, ORC_RNE, 0, 0, 0, -1, codes, scales), 2);
  EXPECT(orc_mxnorm(x, 32, NULL, 1, 32, 0.0, ORC_E4M3, ORC_RNE, 0, 0, 0, 0, NULL, codes, scales,
                    inv),
         5);
  EXPECT(orc_mxnorm(x, 32, NULL, 1, 32, NAN, ORC_E4M3, ORC_RNE, 0, 0, 0, 0, NULL, codes, scales,
                    inv),
         5);
  EXPECT(orc_rmsnorm_mxcast(x, 32, NULL, 1, 32, -1.0, ORC_E4M3, ORC_RNE, 0, 0, 0, 0, NULL, dx,
                            codes, scales, inv),
         5);
  EXPECT(orc_nvfp4_cast(x, 32, 1, 32, 1e-12, codes, scales), 4);
  EXPECT(orc_nvfp4_cast(x, 32, 1, 40, 1.0, codes, scales), 2);
  EXPECT(orc_mxnorm_bwd(x, 32, NULL, x, 32, f, -1, 32, NULL, dx, inv), 2);
  EXPECT(orc_mx_gemm(codes, 32, scales, 1, ORC_E4M3, codes, 32, scales, 1, ORC_E4M3, 1, 1, 48, c,
                     NULL),
         2);
  /* empty batches are valid and touch no row */
  EXPECT(orc_mxcast(x, 32, 0, 32, ORC_E2M1, ORC_SR, 0, 1, 2, 0, codes, scales), 0);
  EXPECT(orc_mxnorm(x, 32, NULL, 0, 32, 2.0, ORC_E4M3, ORC_RNE, 0, 0, 0, 0, NULL, codes, scales,
                    inv),
         0);
  EXPECT(orc_mxnorm_bwd_dgamma(x, 32, x, 32, f, 0, 32, dg, NULL), 0);
}

int main(void) {
  scalars();
  forward_ops(3, 32, 32);
  forward_ops(2, 96, 104);
  forward_ops(4, 64, 72);
  forward_ops(1, 1056, 1056);
  nvfp4_ops(3, 32, 32);
  nvfp4_ops(2, 96, 112);
  backward_ops(3, 64, 64, 72);
  backward_ops(2, 1056, 1064, 1056);
  gemm_ops(3, 2, 64);
  gemm_ops(2, 5, 128);
  invalid_arguments();
  if (g_failures) {
    fprintf(stderr, "%d unexpected statuses\n", g_failures);
    return 1;
  }
  printf("oracle sanitizer drive: ok\n");
  return 0;
}
