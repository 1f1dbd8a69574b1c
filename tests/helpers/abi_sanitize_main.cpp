// Drives the host side of libmxq's C ABI (argument validation, status codes,
// empty calls) for a build with AddressSanitizer and UndefinedBehaviorSanitizer
// of the library's host code. Every call here returns before the library makes
// any HIP call: invalid arguments, empty batches and the pure queries; so it
// runs without a GPU. Exits 0 when every call returned the status the header
// gives for it. Test infrastructure only.

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mxq.h"

static int g_failures = 0;

#define EXPECT(expr, want)                                                                 \
  do {                                                                                     \
    const long rc_ = (long)(expr);                                                         \
    if (rc_ != (long)(want)) {                                                             \
      fprintf(stderr, "%s:%d: %s returned %ld, expected %ld\n", __FILE__, __LINE__, #expr, \
              rc_, (long)(want));                                                          \
      ++g_failures;                                                                        \
    }                                                                                      \
  } while (0)

int main() {
  // small, 256-byte aligned buffers; the calls below never read them
  const size_t n = 1 << 16;
  uint8_t* buf = static_cast<uint8_t*>(aligned_alloc(256, n));
  uint8_t* buf2 = static_cast<uint8_t*>(aligned_alloc(256, n));
  uint8_t* buf3 = static_cast<uint8_t*>(aligned_alloc(256, n));
  memset(buf, 0, n), memset(buf2, 0, n), memset(buf3, 0, n);
  const uint16_t* x = reinterpret_cast<const uint16_t*>(buf);
  const uint16_t* xmis = reinterpret_cast<const uint16_t*>(buf + 2);
  uint8_t* codes = buf2;
  uint8_t* scales = buf3;
  float* inv = reinterpret_cast<float*>(buf3 + 4096);
  uint16_t* y = reinterpret_cast<uint16_t*>(buf3 + 8192);
  const mxq_rng rng = {1, 2};
  const float inf = INFINITY, nan = NAN;

  // ---- mxnorm_fwd
  EXPECT(mxnorm_fwd(nullptr, 64, nullptr, 4, 64, 2.f, MXQ_E4M3, MXQ_RNE, nullptr, 0, codes, scales,
                    inv, nullptr), MXQ_ERR_NULL);
  EXPECT(mxnorm_fwd(x, 64, nullptr, 4, 48, 2.f, MXQ_E4M3, MXQ_RNE, nullptr, 0, codes, scales, inv,
                    nullptr), MXQ_ERR_SHAPE);
  EXPECT(mxnorm_fwd(x, 32, nullptr, 4, 64, 2.f, MXQ_E4M3, MXQ_RNE, nullptr, 0, codes, scales, inv,
                    nullptr), MXQ_ERR_SHAPE);
  EXPECT(mxnorm_fwd(x, 64, nullptr, -1, 64, 2.f, MXQ_E4M3, MXQ_RNE, nullptr, 0, codes, scales, inv,
                    nullptr), MXQ_ERR_SHAPE);
  EXPECT(mxnorm_fwd(xmis, 64, nullptr, 4, 64, 2.f, MXQ_E4M3, MXQ_RNE, nullptr, 0, codes, scales,
                    inv, nullptr), MXQ_ERR_ALIGN);
  EXPECT(mxnorm_fwd(x, 68, nullptr, 4, 64, 2.f, MXQ_E4M3, MXQ_RNE, nullptr, 0, codes, scales, inv,
                    nullptr), MXQ_ERR_ALIGN);
  EXPECT(mxnorm_fwd(x, 64, nullptr, 4, 64, 0.f, MXQ_E4M3, MXQ_RNE, nullptr, 0, codes, scales, inv,
                    nullptr), MXQ_ERR_ARG);
  EXPECT(mxnorm_fwd(x, 64, nullptr, 4, 64, nan, MXQ_E4M3, MXQ_RNE, nullptr, 0, codes, scales, inv,
                    nullptr), MXQ_ERR_ARG);
  EXPECT(mxnorm_fwd(x, 64, nullptr, 4, 64, 2.f, (mxq_elem)7, MXQ_RNE, nullptr, 0, codes, scales,
                    inv, nullptr), MXQ_ERR_ARG);
  EXPECT(mxnorm_fwd(x, 64, nullptr, 4, 64, 2.f, MXQ_E4M3, MXQ_SR, nullptr, 0, codes, scales, inv,
                    nullptr), MXQ_ERR_ARG);
  EXPECT(mxnorm_fwd(x, 64, nullptr, 4, 64, 2.f, MXQ_E4M3, MXQ_RNE, nullptr, 0x100, codes, scales,
                    inv, nullptr), MXQ_ERR_ARG);
  EXPECT(mxnorm_fwd(x, 65536, nullptr, 4, 65536, 2.f, MXQ_E4M3, MXQ_RNE, nullptr, 0, codes, scales,
                    inv, nullptr), MXQ_ERR_UNSUPPORTED);
  EXPECT(mxnorm_fwd(x, 64, nullptr, 0, 64, inf, MXQ_E2M1, MXQ_SR, &rng, 0, codes, scales, inv,
                    nullptr), MXQ_OK);
  EXPECT(mxnorm_fwd(nullptr, 64, nullptr, 0, 64, 2.f, MXQ_E4M3, MXQ_RNE, nullptr, 0, nullptr,
                    nullptr, nullptr, nullptr), MXQ_OK);

  // ---- rmsnorm_mxcast_fwd (two-pass) and the single-pass comparator
  EXPECT(rmsnorm_mxcast_fwd(x, 64, nullptr, 4, 64, 1e-5f, MXQ_E4M3, MXQ_RNE, nullptr, 0, nullptr,
                            codes, scales, inv, nullptr), MXQ_ERR_NULL);
  EXPECT(rmsnorm_mxcast_fwd(x, 64, nullptr, 4, 64, -1.f, MXQ_E4M3, MXQ_RNE, nullptr, 0, y, codes,
                            scales, inv, nullptr), MXQ_ERR_ARG);
  EXPECT(rmsnorm_mxcast_fwd(x, 64, nullptr, 4, 96 + 8, 1e-5f, MXQ_E4M3, MXQ_RNE, nullptr, 0, y,
                            codes, scales, inv, nullptr), MXQ_ERR_SHAPE);
  EXPECT(rmsnorm_mxcast_fwd(x, 64, nullptr, 0, 64, 1e-5f, MXQ_E4M3, MXQ_RNE, nullptr, 0, y, codes,
                            scales, inv, nullptr), MXQ_OK);
  EXPECT(rmsnorm_mxcast_fused_fwd(x, 64, nullptr, 4, 64, inf, MXQ_E4M3, MXQ_RNE, nullptr, 0, codes,
                                  scales, inv, nullptr), MXQ_ERR_ARG);
  EXPECT(rmsnorm_mxcast_fused_fwd(x, 64, nullptr, 4, 64, 1e-5f, MXQ_E4M3, MXQ_RNE, nullptr, 0,
                                  nullptr, scales, inv, nullptr), MXQ_ERR_NULL);
  EXPECT(rmsnorm_mxcast_fused_fwd(x, 64, nullptr, 0, 64, 1e-5f, MXQ_E2M1, MXQ_RNE, nullptr, 0,
                                  codes, scales, inv, nullptr), MXQ_OK);

  // ---- mxcast_fwd
  EXPECT(mxcast_fwd(x, 64, 4, 64, MXQ_E4M3, MXQ_RNE, nullptr, 0, codes, nullptr, nullptr),
         MXQ_ERR_NULL);
  EXPECT(mxcast_fwd(x, 64, 4, 64, MXQ_E4M3, (mxq_round)3, nullptr, 0, codes, scales, nullptr),
         MXQ_ERR_ARG);
  EXPECT(mxcast_fwd(x, 64, 4, 64, MXQ_E4M3, MXQ_RNE, nullptr, MXQ_FLAG_FORCE_LDS, codes, scales,
                    nullptr), MXQ_ERR_ARG);
  EXPECT(mxcast_fwd(x, 64, 0, 64, MXQ_E4M3, MXQ_SR, &rng, MXQ_FLAG_SCALE_CEIL, codes, scales,
                    nullptr), MXQ_OK);

  // ---- NVFP4
  EXPECT(nvfp4_cast_fwd(x, 64, 4, 64, 0.f, codes, scales, nullptr), MXQ_ERR_ARG);
  EXPECT(nvfp4_cast_fwd(x, 64, 4, 64, nan, codes, scales, nullptr), MXQ_ERR_ARG);
  EXPECT(nvfp4_cast_fwd(nullptr, 64, 4, 64, 1.f, codes, scales, nullptr), MXQ_ERR_NULL);
  EXPECT(nvfp4_cast_fwd(x, 64, 0, 64, 1.f, codes, scales, nullptr), MXQ_OK);
  EXPECT(mxnorm_nvfp4_fwd(x, 64, nullptr, 4, 64, -2.f, 1.f, codes, scales, inv, nullptr),
         MXQ_ERR_ARG);
  EXPECT(mxnorm_nvfp4_fwd(x, 64, nullptr, 4, 16384, 2.f, 1.f, codes, scales, inv, nullptr),
         MXQ_ERR_SHAPE);
  EXPECT(mxnorm_nvfp4_fwd(x, 16384, nullptr, 4, 16384, 2.f, 1.f, codes, scales, inv, nullptr),
         MXQ_ERR_UNSUPPORTED);
  EXPECT(mxnorm_nvfp4_fwd(x, 64, nullptr, 0, 64, inf, 1.f, codes, scales, inv, nullptr), MXQ_OK);

  // ---- backward (an empty call with dgamma would launch the column sum: not made here)
  const uint16_t* dy = reinterpret_cast<const uint16_t*>(buf + 32768);
  uint16_t* dx = reinterpret_cast<uint16_t*>(buf2 + 32768);
  float* dgamma = reinterpret_cast<float*>(buf3 + 16384);
  void* ws = buf3 + 32768;
  EXPECT(mxnorm_bwd(nullptr, 64, nullptr, dy, 64, inv, 4, 64, dx, nullptr, nullptr, nullptr, 0,
                    nullptr), MXQ_ERR_NULL);
  EXPECT(mxnorm_bwd(x, 64, nullptr, dy, 64, inv, 4, 16384, dx, nullptr, nullptr, nullptr, 0,
                    nullptr), MXQ_ERR_SHAPE);
  EXPECT(mxnorm_bwd(x, 16384, nullptr, dy, 16384, inv, 4, 16384, dx, nullptr, nullptr, nullptr, 0,
                    nullptr), MXQ_ERR_UNSUPPORTED);
  EXPECT(mxnorm_bwd(x, 64, nullptr, dy, 64, inv, 4, 64, dx, nullptr, dgamma, nullptr, 0, nullptr),
         MXQ_ERR_NULL);
  EXPECT(mxnorm_bwd(x, 64, nullptr, dy, 64, inv, 4, 64, dx, nullptr, dgamma, ws, 16, nullptr),
         MXQ_ERR_ARG);
  EXPECT(mxnorm_bwd(xmis, 64, nullptr, dy, 64, inv, 4, 64, dx, nullptr, nullptr, nullptr, 0,
                    nullptr), MXQ_ERR_ALIGN);
  EXPECT(mxnorm_bwd(x, 64, nullptr, dy, 64, inv, 0, 64, dx, nullptr, nullptr, nullptr, 0, nullptr),
         MXQ_OK);
  EXPECT(mxnorm_bwd_noalloc(nullptr, 64, nullptr, dy, 64, inv, 4, 64, dx, nullptr, dgamma,
                            nullptr), MXQ_ERR_NULL);
  EXPECT(mxnorm_bwd_noalloc(x, 64, nullptr, dy, 64, inv, 4, 40, dx, nullptr, dgamma, nullptr),
         MXQ_ERR_SHAPE);
  EXPECT(mxnorm_bwd_noalloc(x, 64, nullptr, dy, 64, inv, 0, 64, dx, nullptr, nullptr, nullptr),
         MXQ_OK);
  EXPECT(mxnorm_bwd_workspace_size(-1, 64), 0);
  EXPECT(mxnorm_bwd_workspace_size(4, 40), 0);
  EXPECT(mxnorm_bwd_workspace_size(4, 64) >= 64 * sizeof(float), 1);
  EXPECT(mxnorm_bwd_workspace_size(1 << 20, 8192) <= (size_t)512 * 8192 * sizeof(float), 1);

  // ---- MX GEMM
  EXPECT(mx_gemm(codes, 128, scales, 4, codes, 128, scales, 4, 4, 4, 96, MXQ_E4M3, MXQ_E4M3, buf,
                 4, MXQ_OUT_F32, nullptr), MXQ_ERR_UNSUPPORTED);   // K % 128
  EXPECT(mx_gemm(codes, 128, scales, 4, codes, 128, scales, 4, 4, 4, 100, MXQ_E4M3, MXQ_E4M3, buf,
                 4, MXQ_OUT_F32, nullptr), MXQ_ERR_SHAPE);
  EXPECT(mx_gemm(codes, 128, scales, 4, codes, 128, scales, 4, 4, 4, 128, (mxq_elem)5, MXQ_E4M3,
                 buf, 4, MXQ_OUT_F32, nullptr), MXQ_ERR_ARG);
  EXPECT(mx_gemm(codes, 128, scales, 4, codes, 128, scales, 4, 4, 4, 128, MXQ_E4M3, MXQ_E4M3, buf,
                 4, (mxq_out_type)9, nullptr), MXQ_ERR_ARG);
  EXPECT(mx_gemm(codes, 128, scales, 4, codes, 64, scales, 4, 4, 4, 128, MXQ_E4M3, MXQ_E4M3, buf,
                 4, MXQ_OUT_F32, nullptr), MXQ_ERR_SHAPE);         // ldb < K
  EXPECT(mx_gemm(nullptr, 128, scales, 4, codes, 128, scales, 4, 4, 4, 128, MXQ_E4M3, MXQ_E4M3,
                 buf, 4, MXQ_OUT_F32, nullptr), MXQ_ERR_NULL);
  EXPECT(mx_gemm(codes + 1, 128, scales, 4, codes, 128, scales, 4, 4, 4, 128, MXQ_E4M3, MXQ_E4M3,
                 buf, 4, MXQ_OUT_F32, nullptr), MXQ_ERR_ALIGN);
  EXPECT(mx_gemm(codes, 128, scales, 4, codes, 128, scales, 4, 0, 4, 128, MXQ_E4M3, MXQ_E4M3, buf,
                 4, MXQ_OUT_BF16, nullptr), MXQ_OK);

  // ---- messages and version
  for (int s = -2; s <= 9; ++s) EXPECT(mxq_strerror((mxq_status)s) != nullptr, 1);
  EXPECT(mxq_abi_version(), MXQ_ABI_VERSION);

  free(buf), free(buf2), free(buf3);
  if (g_failures) {
    fprintf(stderr, "%d unexpected statuses\n", g_failures);
    return 1;
  }
  printf("abi sanitizer drive: ok\n");
  return 0;
}
