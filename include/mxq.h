/*
 * mxq.h - C ABI of libmxq: MXNorm fused with the MX cast, the two-pass
 * RMSNorm -> MXCast comparison path, and MXCast on its own, for AMD MI355X
 * (gfx950).
 *
 * What the operations compute is defined on the page "MXNorm: Reusing MXFP
 * block scales for efficient tensor normalisation" (gist.science technical
 * summary):
 *   §1.1  RMSNorm computes its statistic over the hidden dimension;
 *   §1.2  RMSNorm and the cast to MXFP (MXCast) normally run as separate
 *         steps, both aggregating statistics along the hidden dimension;
 *   §2.1  MX formats split a tensor into blocks of size B, each with one
 *         E8M0 scale derived from the block absmax; MXNorm takes the block
 *         absmaxes m_k, forms the power mean G = ((1/K) sum_k m_k^p)^(1/p)
 *         as the stand-in for the RMS, normalises by it and casts to MXFP in
 *         the same pass;
 *   §2.3  the gain gamma may be folded into the next linear layer's weights
 *         (pass gamma = NULL);
 *   §4    a drop-in for pre-norm RMSNorm whose only new knob is p.
 * The element formats follow the page "Recipes for Pre-training LLMs with
 * MXFP8" (E4M3 elements) and its related entries "FP8 Formats for Deep
 * Learning" (E4M3 without infinities, one NaN pattern) and "Microscaling Data
 * Formats for Deep Learning" (per-block scale with narrow elements); FP4 is the
 * E2M1 element. Stochastic rounding follows the aibr.jp stochastic-rounding
 * explainer (a neighbour chosen with probability by distance, unbiased).
 *
 * Fixed conventions (the pages leave these open):
 *   - bf16 input x [T, D] row-major with row stride ldx (elements); B = 32
 *     contiguous elements along D; K = D / 32; D must be a multiple of 32.
 *   - E8M0 scale of a block with absmax a: s = floor(log2 a) - emax clamped
 *     to [-127, 127], stored as s + 127 (emax 8 for E4M3, 2 for E2M1);
 *     a == 0 stores 0; a block holding NaN/Inf stores 0xFF and all its codes
 *     are 0x7F (E4M3) or 0x7 (E2M1).
 *   - elements are x / 2^s rounded to nearest-even (or stochastically),
 *     saturating at 448 (E4M3) or 6 (E2M1); the sign of zero is kept.
 *   - E2M1 codes are packed two per byte, element 2j in bits 3:0.
 *   - MXNorm normaliser: inv = RN32(1 / G) with G computed in fp32 from the
 *     exact block maxima (no epsilon, no c(p,B) factor); G == 0 gives inv = 0;
 *     a row holding NaN/Inf gives inv = NaN. y = RN32(RN32(x * gamma) * inv).
 *     When 1/G exceeds the fp32 range (a finite row whose block maxima are all
 *     below about 2^-128), inv_norm reports +Inf and y applies the same fp32
 *     mantissa at its true exponent: y = RN32(RN32(x * gamma) * 2^64 *
 *     (RN32(1/G) * 2^-64)), both power-of-two scalings exact.
 *   - A NaN in the bf16 y of the two-pass path has no defined sign or payload.
 *   - RMSNorm: inv = 1 / sqrt(sum(x^2) / D + eps) in fp32 and
 *     y = bf16_rne(RN32(RN32(x * gamma) * inv)).
 *   - Stochastic rounding: element n = t * D + d draws word r = word (n & 3)
 *     of Philox4x32-10 (Salmon et al., SC'11) with key = seed (low word first)
 *     and counter = (n >> 2 as two words, offset as two words); with frac the
 *     distance above the lower neighbour in units of the local quantum, it
 *     rounds up iff r < 2^(32-B) * floor(frac * 2^B): the top B bits of r
 *     against the top B bits of frac, B = 20 for E4M3 and 22 for E2M1 (the
 *     fp32 mantissa bits the format drops).
 *
 * Memory and execution:
 *   - every pointer is a device pointer owned by the caller; the library
 *     never allocates, frees, or keeps a pointer after returning.
 *   - outputs are contiguous: codes [T, D] bytes (E4M3) or [T, D/2] bytes
 *     (E2M1), scales [T, D/32] bytes, per-row normalisers [T] fp32.
 *   - alignment: x, gamma, codes and y_workspace 16 bytes; ldx % 8 == 0 and
 *     ldx >= D; scales and the normaliser arrays need none beyond their type.
 *   - calls enqueue work on `stream` (a hipStream_t; NULL is the default
 *     stream) and return without waiting. Arguments are validated before any
 *     HIP call; a launch failure returns MXQ_ERR_HIP; a device fault shows at
 *     the caller's next synchronisation.
 *   - T == 0 is a valid empty call (pointers are not read).
 *   - no global mutable state (except the scratch array of
 *     mxnorm_bwd_noalloc, described there): calls are thread-safe.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXQ_ABI_VERSION 4

/* The enumerations below are passed by value and checked by the library, so a
 * caller may hand it any int (an unknown element type, say, is rejected with
 * MXQ_ERR_ARG). Compiled as C++ (the library itself), each gets int as its
 * fixed underlying type: every int is then a value of the type, so checking an
 * out-of-range argument is defined behaviour, and the type keeps the size and
 * calling convention of a C enum. */
#ifdef __cplusplus
#define MXQ_ENUM_INT : int
#else
#define MXQ_ENUM_INT
#endif

typedef enum MXQ_ENUM_INT {
  MXQ_OK = 0,
  MXQ_ERR_NULL = 1,        /* a required pointer is NULL                         */
  MXQ_ERR_SHAPE = 2,       /* T < 0, D <= 0, D % 32 != 0, or ldx < D             */
  MXQ_ERR_ALIGN = 3,       /* a pointer or ldx breaks the alignment rules above  */
  MXQ_ERR_ARG = 4,         /* bad p / eps / element / rounding / flags / rng     */
  MXQ_ERR_UNSUPPORTED = 5, /* a size beyond what the kernels take (see each call) */
  MXQ_ERR_HIP = 6          /* the HIP runtime refused the launch                 */
} mxq_status;

typedef enum MXQ_ENUM_INT { MXQ_E4M3 = 0, MXQ_E2M1 = 1 } mxq_elem;
typedef enum MXQ_ENUM_INT { MXQ_RNE = 0, MXQ_SR = 1 } mxq_round;

/* Stochastic-rounding stream: read only when rnd == MXQ_SR. The same
 * (seed, offset) reproduces the same bits; callers advance offset per call. */
typedef struct {
  uint64_t seed;
  uint64_t offset;
} mxq_rng;

/* Forward flags. FORCE_REG / FORCE_LDS / FORCE_SPLIT select the variant of the
 * single-pass entry points (0 = automatic by D: one wavefront per row up to
 * 4096, rows split over several wavefronts above; all variants give
 * bit-identical results). SCALE_CEIL, accepted by every forward
 * entry point, replaces the OCP floor rule for the E8M0 block scale,
 * s = floor(log2 amax) - emax, by the round-up rule: the smallest s with
 * amax <= maxval * 2^s (maxval 448 for E4M3, 6 for E2M1), so no element of
 * the block saturates. The MXFP8 recipes page names a scale conversion of its
 * own without printing it; this is the reading that rounds the scale up. */
enum {
  MXQ_FLAG_FORCE_REG = 1u,   /* row held in one wavefront's registers (D <= 8192) */
  MXQ_FLAG_FORCE_LDS = 2u,   /* row staged in LDS (D <= MXQ_MAX_D)                */
  MXQ_FLAG_SCALE_CEIL = 4u,  /* round-up E8M0 scale rule                          */
  MXQ_FLAG_FORCE_SPLIT = 8u  /* row split over wavefronts' registers (D <= MXQ_MAX_D) */
};

/* Largest D of the register-resident MXNorm path and of any path. */
#define MXQ_MAX_D_REG 8192
#define MXQ_MAX_D 32768

/*
 * Fused MXNorm -> MX cast (MXNorm page, §2.1 and §2.3).
 *   x        [T, D] bf16 bits, row stride ldx.
 *   gamma    [D] bf16 bits, or NULL for gamma == 1 (folded into the next layer).
 *   p        power of the mean: > 0, or +INFINITY for the block-max maximum.
 *   elem     MXQ_E4M3 (codes [T, D]) or MXQ_E2M1 (codes [T, D/2]).
 *   rnd      MXQ_RNE, or MXQ_SR with rng != NULL.
 *   flags    0 (automatic), or one of MXQ_FLAG_FORCE_REG, MXQ_FLAG_FORCE_LDS,
 *            MXQ_FLAG_FORCE_SPLIT (all variants give bit-identical results),
 *            optionally or-ed with MXQ_FLAG_SCALE_CEIL.
 *   codes, scales  outputs; inv_norm [T] fp32 output, may be NULL.
 * Errors: NULL (x, codes, scales), SHAPE, ALIGN, ARG (p <= 0 or NaN, unknown
 * elem/rnd/flags, SR without rng), UNSUPPORTED (D too large for the path,
 * T * D >= 2^40, or more than 2^31 - 1 workgroups of rows), HIP.
 */
mxq_status mxnorm_fwd(const uint16_t* x, int64_t ldx, const uint16_t* gamma, int64_t T,
                      int64_t D, float p, mxq_elem elem, mxq_round rnd, const mxq_rng* rng,
                      uint32_t flags, uint8_t* codes, uint8_t* scales, float* inv_norm,
                      void* stream);

/*
 * Two-pass comparison path (MXNorm page, §1.1 and §1.2): RMSNorm writes bf16
 * y to y_workspace [T, D] (contiguous, caller-owned), then MXCast reads it.
 *   eps      >= 0 and finite.
 *   flags    0 or MXQ_FLAG_SCALE_CEIL (the scale rule of the cast).
 *   inv_rms  [T] fp32 output, may be NULL.
 * Other arguments and errors as for mxnorm_fwd (y_workspace NULL -> NULL;
 * also UNSUPPORTED when T * ceil(D / 512) >= 2^32 - 256, the cast pass's
 * 32-bit count of 512-element chunks).
 */
mxq_status rmsnorm_mxcast_fwd(const uint16_t* x, int64_t ldx, const uint16_t* gamma,
                              int64_t T, int64_t D, float eps, mxq_elem elem, mxq_round rnd,
                              const mxq_rng* rng, uint32_t flags, uint16_t* y_workspace,
                              uint8_t* codes, uint8_t* scales, float* inv_rms, void* stream);

/*
 * Single-pass exact-RMS comparator: RMSNorm's statistic (MXNorm page, §1.1),
 * inv = 1 / sqrt(sum(x^2) / D + eps) in fp32 summed in the same order as
 * rmsnorm_mxcast_fwd (so inv_rms is bit-identical to its), applied as in
 * mxnorm_fwd, y = RN32(RN32(x * gamma) * inv), and cast to MX in the same pass
 * (§2.1) without rounding y to bf16. It differs from mxnorm_fwd only in the
 * statistic (D squares instead of K block maxima) and from the two-pass path
 * only in keeping the row on chip. Arguments, flags and errors as for
 * mxnorm_fwd with eps (>= 0, finite) in place of p; inv_rms [T] may be NULL.
 */
mxq_status rmsnorm_mxcast_fused_fwd(const uint16_t* x, int64_t ldx, const uint16_t* gamma,
                                    int64_t T, int64_t D, float eps, mxq_elem elem,
                                    mxq_round rnd, const mxq_rng* rng, uint32_t flags,
                                    uint8_t* codes, uint8_t* scales, float* inv_rms,
                                    void* stream);

/*
 * MXCast of a bf16 activation (MXNorm page, §1.2 and §2.1): block absmax,
 * E8M0 scale and element cast, with no normalisation.
 *   flags    0 or MXQ_FLAG_SCALE_CEIL (the scale rule).
 * Other arguments and errors as for mxnorm_fwd (no gamma, p or inv_norm;
 * UNSUPPORTED when T * ceil(D / 512) >= 2^32 - 256, its 32-bit chunk count).
 */
mxq_status mxcast_fwd(const uint16_t* x, int64_t ldx, int64_t T, int64_t D, mxq_elem elem,
                      mxq_round rnd, const mxq_rng* rng, uint32_t flags, uint8_t* codes,
                      uint8_t* scales, void* stream);

/*
 * Straight-through backward of the normalisation (MXNorm page, §2.3, gradient
 * paragraph: RMSNorm's gradient computation is reused as a straight-through
 * estimator). The cast counts as the identity, and the forward's exported
 * normaliser inv_norm (1/G from mxnorm_fwd, or any per-row normaliser) stands
 * where RMSNorm has 1/rms. Per row t, with g = gamma * dy:
 *   s_t      = sum_i g_i * x_i
 *   dx_ti    = inv_t * g_i - inv_t^3 * (s_t / D) * x_ti      (rounded to bf16)
 *   dgamma_i = sum_t dy_ti * x_ti * inv_t                      (fp32)
 * fp32 order: g and dy * x are exact; s sums each lane's 512-element chunks
 * in order and then the wave, as the RMS paths do, except for rows of 2, 4, 6
 * or 8 chunks, where each half of the chunks is summed that way and the two
 * half sums add (the same order with and without dgamma); k = (inv*inv)*inv,
 * c = k * (s/D), dx = bf16(inv*g - c*x). dgamma sums rows in a fixed order
 * (bit-reproducible from run to run).
 *   x [T, D] bf16, row stride ldx; dy [T, D] bf16, row stride lddy.
 *   gamma [D] bf16 or NULL (gamma == 1).  inv_norm [T] fp32.
 *   dx [T, D] bf16 contiguous output.  row_dot [T] fp32 output (s), may be NULL.
 *   dgamma [D] fp32 output (16-byte aligned), may be NULL; it then needs a
 *   caller-owned workspace of at least mxnorm_bwd_workspace_size(T, D) bytes
 *   (16-byte aligned), which the call overwrites. For T == 0, dgamma is zeroed.
 * Errors: SHAPE (T < 0, D <= 0, D % 32, ldx or lddy < D), UNSUPPORTED
 * (D > MXQ_MAX_D_REG), NULL (x, dy, inv_norm, dx; workspace with dgamma), ARG
 * (workspace too small), ALIGN (16-byte x, dy, dx, gamma, dgamma, workspace;
 * ldx, lddy % 8), HIP.
 */
mxq_status mxnorm_bwd(const uint16_t* x, int64_t ldx, const uint16_t* gamma, const uint16_t* dy,
                      int64_t lddy, const float* inv_norm, int64_t T, int64_t D, uint16_t* dx,
                      float* row_dot, float* dgamma, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Workspace bytes mxnorm_bwd needs to produce dgamma (0 for a bad shape). */
size_t mxnorm_bwd_workspace_size(int64_t T, int64_t D);

/*
 * mxnorm_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). It computes exactly what mxnorm_bwd computes, with
 * the same kernels and summation order (bit-identical results), and allocates
 * nothing: the dgamma partial sums live in a 16 MiB array that the library
 * holds on each GPU it runs on until the process ends (every shape this entry
 * point accepts fits it; a larger one would return UNSUPPORTED). That array is
 * shared by every call on the GPU, so calls that overlap on one GPU (two
 * streams, two threads) race on it and must be serialised by the caller. The
 * current device must be the stream's device. The first call on a device
 * looks up the array's address on it.
 * Arguments and errors as for mxnorm_bwd without workspace and
 * workspace_bytes (HIP also when the array's address cannot be looked up).
 */
mxq_status mxnorm_bwd_noalloc(const uint16_t* x, int64_t ldx, const uint16_t* gamma,
                              const uint16_t* dy, int64_t lddy, const float* inv_norm, int64_t T,
                              int64_t D, uint16_t* dx, float* row_dot, float* dgamma,
                              void* stream);

/* Element type of a GEMM result. */
typedef enum MXQ_ENUM_INT { MXQ_OUT_F32 = 0, MXQ_OUT_BF16 = 1 } mxq_out_type;

/*
 * MX GEMM, the consumer of the MX output (MXNorm page, §2.3: the gain is
 * folded into the next linear layer's weight, which is MX-cast; §3.2 times the
 * layer around it):
 *   C[m][n] = sum_k A[m][k] * B[n][k],
 * with A[m][k] = dec(a[m][k]) * 2^(a_scales[m][k/32] - 127) (the MX output of
 * mxnorm_fwd / mxcast_fwd, [M, K]) and B likewise from the weight [N, K] MX-cast
 * along K (mxcast_fwd of W). The products run on the gfx950 block-scaled matrix
 * cores with fp32 accumulation (order not specified); C is fp32 or bf16
 * (round to nearest even) [M, N] with row stride ldc elements. A NaN code or a
 * 0xFF scale makes the outputs it reaches NaN.
 *   a, b       codes, lda / ldb bytes per row (>= K for E4M3, >= K/2 for packed
 *              E2M1, element 2j in the low nibble of byte j), 16-byte aligned rows.
 *   a_scales, b_scales  E8M0 bytes, ldsa / ldsb per row (>= K/32, % 4 == 0),
 *              4-byte aligned.
 *   elem_a, elem_b  MXQ_E4M3 or MXQ_E2M1, each operand its own (mixed pairs
 *              allowed).
 *   c          aligned to its element; 16-byte (fp32) or 8-byte (bf16) aligned
 *              rows with ldc % 4 == 0 take vector stores.
 * Errors: SHAPE (M, N < 0, K <= 0, K % 32, a leading dimension too small), ARG
 * (unknown element or output type), UNSUPPORTED (K % 128 != 0, sizes of
 * 2^31 or more), NULL, ALIGN, HIP. M == 0 or N == 0 is a no-op.
 */
mxq_status mx_gemm(const uint8_t* a, int64_t lda, const uint8_t* a_scales, int64_t ldsa,
                   const uint8_t* b, int64_t ldb, const uint8_t* b_scales, int64_t ldsb,
                   int64_t M, int64_t N, int64_t K, mxq_elem elem_a, mxq_elem elem_b, void* c,
                   int64_t ldc, mxq_out_type c_type, void* stream);

/*
 * NVFP4 (MXNorm page, §3.2, names the format for its layer-level result; the
 * pages do not define it, so the library takes the published two-level format
 * as a reading): E2M1 elements packed two per byte as for MXQ_E2M1, blocks of
 * 16 consecutive elements along a row, one E4M3 scale byte per block, and one
 * fp32 tensor scale s_t from the caller; value = e2m1 * e4m3(scale) * s_t.
 * Per block with a = max |y|: the scale byte is the E4M3 encoding (round to
 * nearest even, saturating at 448) of RN32(a * RN32(1 / (6 s_t))); with Sd its
 * value, each element is the E2M1 encoding (RNE, saturating) of
 * RN32(y * RN32(1 / RN32(Sd * s_t))), or a signed zero when Sd == 0. A block
 * holding NaN or Inf gets scale 0x7F (the E4M3 NaN) and element codes 0x7.
 *   x            [T, D] bf16 bits, row stride ldx (D % 32 == 0, D <= 8192).
 *   tensor_scale s_t, in [2^-32, 2^32] (1 for MXNorm's normalised output).
 *   codes        [T, D/2] packed E2M1, contiguous; scales [T, D/16] E4M3 bytes.
 * Errors: SHAPE, ARG (tensor_scale outside its range or NaN; p <= 0 or NaN),
 * UNSUPPORTED (D > 8192, T * D >= 2^40), NULL, ALIGN (x, codes: 16 bytes;
 * gamma: 16; inv_norm: 4), HIP.
 *
 * nvfp4_cast_fwd: the cast of x itself (y = x).
 */
mxq_status nvfp4_cast_fwd(const uint16_t* x, int64_t ldx, int64_t T, int64_t D,
                          float tensor_scale, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * MXNorm over NVFP4 blocks (MXNorm page, §2.1 with the blocks of the format
 * being cast to): G is the power mean of the 16-element block maxima of |x|
 * (K = D / 16), inv = RN32(1/G) as for mxnorm_fwd (reported in inv_norm, which
 * may be NULL), y = RN32(RN32(x * gamma) * inv), then the NVFP4 encoding above.
 * gamma may be NULL (gamma == 1); p > 0 or +INFINITY.
 */
mxq_status mxnorm_nvfp4_fwd(const uint16_t* x, int64_t ldx, const uint16_t* gamma, int64_t T,
                            int64_t D, float p, float tensor_scale, uint8_t* codes,
                            uint8_t* scales, float* inv_norm, void* stream);

/* Static message for a status code (never NULL). */
const char* mxq_strerror(mxq_status status);

/* MXQ_ABI_VERSION of the built library. */
int mxq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
