// mxq.hip - gfx950 kernels and the C ABI of libmxq (see include/mxq.h).
//
// Operations (page "MXNorm: Reusing MXFP block scales for efficient tensor
// normalisation", gist.science technical summary):
//   * mxnorm_fwd         §2.1: block absmax m_k, power mean G of the m_k,
//                        y = x * gamma / G, E8M0 scale per 32-block and the
//                        element cast, in one read of x and one write;
//   * rmsnorm_mxcast_fwd §1.1/§1.2: RMSNorm to a bf16 tensor, then MXCast
//                        (two kernels, the comparison path);
//   * mxcast_fwd         §1.2/§2.1: MXCast alone.
//
// Work layout (one wavefront = 64 lanes; one "chunk" = 512 contiguous
// elements of a row, one 16-byte load per lane; a 32-element MX block is the
// 4 lanes of a quad):
//   * MXNorm / RMSNorm: one wavefront per row, 4 rows per 256-thread
//     workgroup. Block maxima come from packed-u16 max on the bf16 bit
//     patterns plus two DPP quad steps; the row statistic is a butterfly
//     over the 16 quads; nothing crosses waves, so there is no barrier.
//     The register variant keeps the row in VGPRs (D <= 8192); the LDS
//     variant stages it with direct-to-LDS 16-byte loads and uses the same
//     reduction order, so both give identical bits.
//   * MXCast: every chunk is independent; each wavefront handles 4 chunks.
//   * Element casts use the gfx950 scaled converts (the E8M0 code is the
//     exponent field of the fp32 scale operand, which divides). The FP8
//     convert does not saturate, so values are clamped to +-448 * 2^s first;
//     the FP4 convert saturates by itself. Stochastic rounding is integer
//     code on Philox4x32-10 words.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mxq.h"

namespace {

#include "mxq_device.h"

constexpr int kCastChunksPerWave = 4; // MXCast chunks per wavefront

enum PMode { P_ONE = 0, P_TWO = 1, P_INF = 2, P_GEN = 3 };

// Row statistic of the single-pass normalise-and-cast kernels: the power mean
// of the block maxima (MXNorm), or the exact RMS over all D elements (RMSNorm's
// statistic, the single-pass comparator).
enum Stat { S_PMEAN = 0, S_RMS = 1 };

typedef short short2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ p-mean

// Term of the power mean for one block maximum m (m >= 0).
__device__ __forceinline__ float pmean_add(float s, float m, int pmode, float p) {
  if (pmode == P_ONE) return s + m;
  if (pmode == P_TWO) return __builtin_fmaf(m, m, s);
  return s + exp2f(p * log2f(m));  // m == 0 -> exp2(-inf) == 0
}

__device__ __forceinline__ float pmean_finish(float s, int pmode, float p, float K) {
  float q = s / K;
  if (pmode == P_ONE) return q;
  if (pmode == P_TWO) return sqrtf(q);
  return exp2f(log2f(q) / p);
}

// Sum of the power-mean terms of this lane's chunks, in chunk order, of the
// block maxima scaled by 2^shift. NCT > 0 gives a compile-time (unrolled)
// chunk count, NCT == 0 the runtime count.
template <int NCT, int PM, class BlockMax>
__device__ __forceinline__ float lane_terms_p(int nchunks, BlockMax mb, int shift, float p) {
  float s = 0.0f;
  if constexpr (NCT > 0) {
#pragma unroll
    for (int c = 0; c < NCT; ++c) s = pmean_add(s, ldexpf(__uint_as_float(mb(c) << 16), shift), PM, p);
  } else {
    for (int c = 0; c < nchunks; ++c)
      s = pmean_add(s, ldexpf(__uint_as_float(mb(c) << 16), shift), PM, p);
  }
  return s;
}

// The power mode is tested once, outside the term loop.
template <int NCT, class BlockMax>
__device__ __forceinline__ float lane_terms(int nchunks, BlockMax mb, int shift, int pmode, float p) {
  if (pmode == P_TWO) return lane_terms_p<NCT, P_TWO>(nchunks, mb, shift, p);
  if (pmode == P_ONE) return lane_terms_p<NCT, P_ONE>(nchunks, mb, shift, p);
  return lane_terms_p<NCT, P_GEN>(nchunks, mb, shift, p);
}

// Normaliser 1/G of a row from its block maxima (bf16 bit patterns, one per
// chunk for this lane's quad, zero for blocks past the row end). lane_max()
// gives this lane's maximum of the patterns. Terms are added chunk by chunk in
// each lane, then over the quads; every variant uses exactly this order.
// A sum inside [2^-96, 2^96] is finite and nonzero, so the row holds no NaN
// or Inf (either would make the sum non-finite) and is not all zero: the row
// maximum is only needed outside that range, and for p = inf.
template <int NCT, class BlockMax, class LaneMax>
__device__ __forceinline__ float row_normaliser(int nchunks, BlockMax mb, LaneMax lane_max,
                                                int pmode, float p, float K) {
  if (pmode != P_INF) {
    const float s = sum_over_quads(lane_terms<NCT>(nchunks, mb, 0, pmode, p));
    if (s >= 0x1p-96f && s <= 0x1p96f) return 1.0f / pmean_finish(s, pmode, p, K);
  }
  const uint32_t rmax = max_over_quads(lane_max());
  if (rmax >= 0x7F80u) return __builtin_nanf("");  // the row holds NaN or Inf
  if (rmax == 0u) return 0.0f;                      // all-zero row
  if (pmode == P_INF) return 1.0f / __uint_as_float(rmax << 16);
  // The p-th powers left the range where fp32 holds them accurately (an
  // underflowing or overflowing sum): rescale the maxima by 2^-E, E the
  // exponent of the row maximum, and undo it on G.
  int E = (int)((rmax >> 7) & 0xFFu) - 127;
  if (E < -126) E = -126;
  const float s = sum_over_quads(lane_terms<NCT>(nchunks, mb, -E, pmode, p));
  return 1.0f / ldexpf(pmean_finish(s, pmode, p, K), E);
}

// ------------------------------------------------------------------ scales

// Floor rule: s = floor(log2 a) - emax, read from the fp32 exponent field.
// Round-up rule: the smallest s with a <= maxval * 2^s. With maxval = 1.M * 2^emax
// (1.75 * 2^8 for E4M3, 1.5 * 2^2 for E2M1) that is the floor rule plus one
// exactly when a's mantissa exceeds M; adding 0x7FFFFF - M to the bits carries
// into the exponent field in exactly those cases (a finite a stays below
// 0x7F800000 + 0x7FFFFF, so the carry never reaches the sign). adj is 0 for
// the floor rule and scale_adjust<ELEM>() for the round-up rule. The code is
// s + 127 clamped at 0; NaN / Inf give 0xFF.
template <int ELEM>
__host__ __device__ constexpr uint32_t scale_adjust() {
  return 0x7FFFFFu - ((ELEM == MXQ_E4M3) ? 0x600000u : 0x400000u);
}

// A block's E8M0 byte (the low byte of code), and whether the block holds NaN
// or Inf (then code is all ones, so the byte is 0xFF, and every element of
// the block is encoded as NaN).
struct BlockScale {
  uint32_t code;
  bool bad;
};

// a is the block's absolute maximum: +0 or more, or NaN (a NaN with its sign
// bit set also counts as bad). Taking emax (and the round-up adjustment) off
// the bits in one clamped unsigned subtract, ahead of the shift, gives the
// biased exponent less emax, saturated at 0.
template <int ELEM>
__device__ __forceinline__ BlockScale e8m0_scale(float amax, uint32_t adj) {
  constexpr uint32_t kEmax = (ELEM == MXQ_E4M3) ? 8u : 2u;
  const uint32_t b = __float_as_uint(amax);
  const bool bad = b >= 0x7F800000u;
  const uint32_t code = __builtin_elementwise_sub_sat(b, (kEmax << 23) - adj) >> 23;
  return {bad ? ~0u : code, bad};  // all ones is an inline constant: no literal move
}

// ------------------------------------------------------------------ Philox

// a ^ b ^ c as one gfx950 three-input bitwise operation (0x96 is the truth
// table of the three-way parity, the same for any order of the inputs).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): multipliers 0xD2511F53
// and 0xCD9E8D57, key increments 0x9E3779B9 and 0xBB67AE85.
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    // one 32x32 -> 64-bit multiply each (v_mad_u64_u32 gives both halves)
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    c0 = xor3((uint32_t)(p1 >> 32), c1, k0);
    c1 = (uint32_t)p1;
    c2 = xor3((uint32_t)(p0 >> 32), c3, k1);
    c3 = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return make_uint4(c0, c1, c2, c3);
}

struct SrStream {
  uint32_t k0, k1, o0, o1;
  // Words for logical elements n0 .. n0+7 (n0 % 8 == 0).
  __device__ __forceinline__ void words8(uint64_t n0, uint32_t r[8]) const {
    const uint64_t b = n0 >> 2;
    const uint4 a = philox4x32_10((uint32_t)b, (uint32_t)(b >> 32), o0, o1, k0, k1);
    const uint4 c = philox4x32_10((uint32_t)(b + 1), (uint32_t)((b + 1) >> 32), o0, o1, k0, k1);
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
    r[4] = c.x; r[5] = c.y; r[6] = c.z; r[7] = c.w;
  }
};

// ------------------------------------------------------------------ encode

// 8 values y (not yet divided by the scale) -> 8 E4M3 codes, RNE, saturating.
// A non-finite block is encoded like any other (its scale and limit are then
// meaningless values that fault nothing) and its codes are replaced by NaN
// with a select, so the common path has no branch.
__device__ __forceinline__ uint2 encode8_e4m3_rne(const float y[8], BlockScale s) {
  const uint32_t code = s.code;
  const bool bad = s.bad;
  const float scale = __uint_as_float(code << 23);                  // 2^(code-127)
  const float lim = __uint_as_float(((code + 8u) << 23) | 0x00600000u); // 448 * 2^(code-127)
  float w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = __builtin_amdgcn_fmed3f(y[j], -lim, lim);
  // each convert writes one half of its destination and keeps the other, so
  // the starting value is irrelevant (both halves are written): reuse w bits
  short2_t a = __builtin_bit_cast(short2_t, w[0]), b = __builtin_bit_cast(short2_t, w[4]);
  a = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(a, w[0], w[1], scale, false);
  a = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(a, w[2], w[3], scale, true);
  b = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(b, w[4], w[5], scale, false);
  b = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(b, w[6], w[7], scale, true);
  const uint32_t lo = __builtin_bit_cast(uint32_t, a), hi = __builtin_bit_cast(uint32_t, b);
  return make_uint2(bad ? 0x7F7F7F7Fu : lo, bad ? 0x7F7F7F7Fu : hi);
}

// 8 values -> 8 E2M1 codes packed in one word (element 2j in the low nibble).
__device__ __forceinline__ uint32_t encode8_e2m1_rne(const float y[8], BlockScale s) {
  const bool bad = s.bad;  // as for E4M3: select, no branch
  const float scale = __uint_as_float(s.code << 23);
  uint32_t q = __float_as_uint(y[0]);  // all four bytes are written below
  q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, y[0], y[1], scale, 0);
  q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, y[2], y[3], scale, 1);
  q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, y[4], y[5], scale, 2);
  q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, y[6], y[7], scale, 3);
  return bad ? 0x77777777u : q;
}

// Stochastic rounding of v (already divided by the scale, |v| < 2^(emax+1)):
// with n the magnitude in units of the local quantum, truncated, and frac32 =
// floor(frac * 2^32) the part below it, round up iff r < frac32; saturating.
//   normal binades: n and the exponent form the code directly, (a >> sh) - bias,
//     and the discarded mantissa bits shifted to the top are frac32;
//   below the smallest normal the quantum is fixed (2^-9, E2M1 2^-1): q = |v| /
//     quantum is exact, n = trunc(q), and (q - n) * 2^32 is exact as well.
//   The magnitude goes through abs source modifiers and a bit-field extract
//   (no masking instruction); q - n is the hardware fraction of q (exact for
//   q >= 0). The sign is left to the caller.
template <int ELEM>
__device__ __forceinline__ uint32_t sr_mag_code(float v, uint32_t r) {
  constexpr int kSh = (ELEM == MXQ_E4M3) ? 20 : 22;                // fp32 mantissa bits dropped
  constexpr uint32_t kBias = (ELEM == MXQ_E4M3) ? 960u : 252u;     // (120 << 3), (126 << 1)
  constexpr float kMinNormal = (ELEM == MXQ_E4M3) ? 0x1p-6f : 1.0f;
  constexpr float kInvQuantum = (ELEM == MXQ_E4M3) ? 512.0f : 2.0f;
  constexpr uint32_t kMaxCode = (ELEM == MXQ_E4M3) ? 0x7Eu : 0x7u;
  const uint32_t u = __float_as_uint(v);
  // both forms, then a select per lane (no divergent branch); q < 2^18 always
  const float q = fabsf(v) * kInvQuantum;
  const uint32_t n_sub = (uint32_t)q;
  const uint32_t f_sub = (uint32_t)(__builtin_amdgcn_fractf(q) * 4294967296.0f);
  const bool normal = fabsf(v) >= kMinNormal;
  const uint32_t code = normal ? __builtin_amdgcn_ubfe(u, kSh, 31 - kSh) - kBias : n_sub;
  const uint32_t frac = normal ? u << (32 - kSh) : f_sub;  // the sign bit shifts out
  return min(code + (r < frac ? 1u : 0u), kMaxCode);
}

// The top bytes of four values (a in byte 0 ... d in byte 3), so each sign
// is bit 7 of its byte: three byte permutes.
__device__ __forceinline__ uint32_t top_bytes4(float a, float b, float c, float d) {
  const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x0C0C0703u);
  const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(d), __float_as_uint(c), 0x07030C0Cu);
  return __builtin_amdgcn_perm(hi, lo, 0x07060100u);
}

// Four E4M3 magnitudes packed in bytes (bit 7 clear) with the signs of the
// four values merged in by one and-or.
__device__ __forceinline__ uint32_t with_signs4(uint32_t mags, float a, float b, float c, float d) {
  return (top_bytes4(a, b, c, d) & 0x80808080u) | mags;
}

__device__ __forceinline__ uint2 encode8_e4m3_sr(const float y[8], BlockScale s, const uint32_t r[8]) {
  if (s.bad) return make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
  const float inv_scale = __uint_as_float((254u - s.code) << 23);  // 2^-(code-127), a normal float
  uint32_t c[8];
  float w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    w[j] = y[j] * inv_scale;
    c[j] = sr_mag_code<MXQ_E4M3>(w[j], r[j]);
  }
  return make_uint2(with_signs4(c[0] | c[1] << 8 | c[2] << 16 | c[3] << 24, w[0], w[1], w[2], w[3]),
                    with_signs4(c[4] | c[5] << 8 | c[6] << 16 | c[7] << 24, w[4], w[5], w[6], w[7]));
}

__device__ __forceinline__ uint32_t encode8_e2m1_sr(const float y[8], BlockScale s, const uint32_t r[8]) {
  if (s.bad) return 0x77777777u;
  const float inv_scale = __uint_as_float((254u - s.code) << 23);
  uint32_t q = 0;
  float w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    w[j] = y[j] * inv_scale;
    q |= sr_mag_code<MXQ_E2M1>(w[j], r[j]) << (4 * j);
  }
  // sign of element j is bit 3 of its nibble: bit 7 of byte j / 2 for odd j,
  // bit 3 of that byte for even j (the even top bytes shifted down a nibble)
  const uint32_t odd = top_bytes4(w[1], w[3], w[5], w[7]) & 0x80808080u;
  const uint32_t even = (top_bytes4(w[0], w[2], w[4], w[6]) >> 4) & 0x08080808u;
  return q | odd | even;
}

// ------------------------------------------------------------------ memory

__device__ __forceinline__ void store8_stream(uint8_t* p, uint2 v) {
  const u32x2 w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p));
}

__device__ __forceinline__ void store4_stream(uint8_t* p, uint32_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}

// Encodes the 8 elements at column d of a row and stores them. codes_row is
// the row's first code byte (uniform across the wave, so the store takes a
// scalar base and a 32-bit lane offset); n = row * D + d is the logical
// element index that keys the stochastic-rounding stream.
template <int ELEM, int RND>
__device__ __forceinline__ void encode_store8(uint8_t* codes_row, uint32_t d, uint64_t n,
                                              const float y[8], BlockScale code,
                                              const SrStream& rng) {
  if (RND == MXQ_SR) {
    uint32_t r[8];
    rng.words8(n, r);
    if (ELEM == MXQ_E4M3)
      store8_stream(codes_row + d, encode8_e4m3_sr(y, code, r));
    else
      store4_stream(codes_row + (d >> 1), encode8_e2m1_sr(y, code, r));
  } else {
    if (ELEM == MXQ_E4M3)
      store8_stream(codes_row + d, encode8_e4m3_rne(y, code));
    else
      store4_stream(codes_row + (d >> 1), encode8_e2m1_rne(y, code));
  }
}

// First code byte of row t (E2M1 packs two codes per byte; D is even).
template <int ELEM>
__device__ __forceinline__ uint8_t* code_row(uint8_t* codes, uint64_t nrow) {
  return codes + (ELEM == MXQ_E4M3 ? nrow : nrow >> 1);
}

// Make one lane's LDS writes visible to the other lanes of its wavefront.
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Scale bytes are gathered per wavefront in LDS (one byte per quad and chunk)
// and leave in dword stores, one per lane, instead of one byte store per
// block. vec: dst is 4-byte aligned and nbytes % 4 == 0; else bytes.
__device__ __forceinline__ void flush_scales(const uint32_t* sc, uint8_t* dst, int nbytes, bool vec,
                                             int lane) {
  wave_sync_lds();
  if (vec) {
    for (int j = lane; j * 4 < nbytes; j += kWave) reinterpret_cast<uint32_t*>(dst)[j] = sc[j];
  } else {
    const uint8_t* b = reinterpret_cast<const uint8_t*>(sc);
    for (int j = lane; j < nbytes; j += kWave) dst[j] = b[j];
  }
}

__device__ __forceinline__ void put_scale(uint32_t* sc, int idx, uint32_t code) {
  reinterpret_cast<uint8_t*>(sc)[idx] = (uint8_t)code;
}

// ------------------------------------------------------------------ MXNorm

struct NormArgs {
  const uint16_t* x;
  const uint16_t* gamma;
  uint8_t* codes;
  uint8_t* scales;
  float* inv_out;
  int64_t ldx;
  int64_t T;
  int D;
  int K;
  float Kf;
  float p;
  int pmode;
  float Df;    // D, for the RMS statistic
  float eps;   // RMS statistic only
  int sc_vec;  // scales rows can be written in dwords
  int ceil_rule;  // E8M0 round-up rule instead of the floor rule
  SrStream rng;
};

// How the block maximum of |x * gamma| is taken:
//   G_NONE  no gamma: the block maximum of |x| is reused (rounding is monotone);
//   G_GAIN  gains: fp32 max with abs modifiers over the products. A NaN
//           product can only come from a non-finite gain (a non-finite x
//           already makes the row's normaliser NaN), and the staging of the
//           gains turns every lane-group of 8 gains holding a NaN or Inf into
//           8 NaNs, so that group's products are all NaN, the fp32 max is NaN
//           and the block is flagged non-finite, as it must be.
enum GMode { G_NONE = 0, G_GAIN = 1 };

// First half of a chunk, needing no normaliser: v = x * gamma (exact: two
// bf16 factors) and the quad's block maximum of |v| as a bit pattern (for
// G_NONE, v = x and the maximum is the block maximum of |x|, mbits).
template <int GM>
__device__ __forceinline__ uint32_t chunk_products(const uint4& xb, const float g[8], uint32_t mbits,
                                                   float v[8]) {
  unpack8(xb, v);
  if (GM == G_NONE) return mbits << 16;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = v[j] * g[j];
  float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fabsf(v[2]));
  m = fmaxf(fmaxf(m, fabsf(v[3])), fabsf(v[4]));
  m = fmaxf(fmaxf(m, fabsf(v[5])), fabsf(v[6]));
  m = fmaxf(m, fabsf(v[7]));
  // integer max of non-negative floats: NaN bits exceed every other value
  return quad_max_u32(__float_as_uint(m));
}

// Second half: y = RN(v * inv), E8M0 code from max |y| = RN(max |v| * inv)
// (rounding is monotone), codes stored. Returns the code of the lane's block.
// vmax_bits has its sign bit clear and inv is +0 or more, or NaN, so the
// maximum is +0 or more, or NaN, as e8m0_scale expects.
template <int ELEM, int RND>
__device__ __forceinline__ uint32_t chunk_finish(const NormArgs& A, uint8_t* codes_row,
                                                 uint64_t nrow, uint32_t d, float v[8],
                                                 uint32_t vmax_bits, float inv) {
  const float amax = __uint_as_float(vmax_bits) * inv;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = v[j] * inv;
  const BlockScale s = e8m0_scale<ELEM>(amax, A.ceil_rule ? scale_adjust<ELEM>() : 0u);
  encode_store8<ELEM, RND>(codes_row, d, nrow + d, v, s, A.rng);
  return s.code;
}

// Both halves of the chunk at column d of row nrow / D.
template <int ELEM, int RND, int GM>
__device__ __forceinline__ uint32_t mxnorm_chunk(const NormArgs& A, uint8_t* codes_row,
                                                 uint64_t nrow, uint32_t d, const uint4& xb,
                                                 const float g[8], uint32_t mbits, float inv) {
  float v[8];
  const uint32_t vm = chunk_products<GM>(xb, g, mbits, v);
  return chunk_finish<ELEM, RND>(A, codes_row, nrow, d, v, vm, inv);
}

// 8 bf16 quiet NaNs.
__device__ __forceinline__ uint4 nan_group() {
  return make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
}

// Whether any of 8 bf16 values is NaN or Inf (exponent field all ones): the
// exponent fields alone, as 16-bit lanes, reach their largest value 0x7F80
// exactly then.
__device__ __forceinline__ bool nonfinite_bf16x8(const uint4& r) {
  const uint32_t k = 0x7F807F80u;
  const u16x2 a = __builtin_bit_cast(u16x2, r.x & k), b = __builtin_bit_cast(u16x2, r.y & k);
  const u16x2 c = __builtin_bit_cast(u16x2, r.z & k), d = __builtin_bit_cast(u16x2, r.w & k);
  const uint32_t m = __builtin_bit_cast(
      uint32_t, __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                          __builtin_elementwise_max(c, d)));
  const u16x2 h = __builtin_bit_cast(u16x2, m);
  return __builtin_elementwise_max(h.x, h.y) == 0x7F80u;
}

// gamma [D] goes to LDS as fp32, laid out [chunk][half][lane] (float4 each),
// so each lane reads its 8 gains of a chunk as two conflict-free 16-byte LDS
// reads. Staging is split in two: the global loads are issued first, ahead of
// the row loads (the memory counter retires loads in order, so gains loaded
// after the row could only be used once the whole row had arrived), and
// written to LDS after the row loads are in flight. Item i = c * 64 + lane;
// each of the workgroup's NT threads handles items tid, tid + NT, ...
template <int NC, int NT>
struct GammaStage {
  static constexpr int kItems = (NC * kWave + NT - 1) / NT;
  uint4 r[kItems];

  __device__ __forceinline__ void load(const uint16_t* gamma, int D) {
    const RangeLoader g(gamma, D);
#pragma unroll
    for (int k = 0; k < kItems; ++k) r[k] = g.load8(((int)threadIdx.x + k * NT) * 8);
  }

  // Writes the gains to LDS (a group of 8 holding a NaN or Inf becomes 8
  // NaNs, see G_GAIN; the replacement is skipped by the whole wavefront when
  // none of its groups needs it) and waits for the whole workgroup. Items
  // past the row end read zeros; the chunks they belong to are never
  // encoded, so their gains are never read.
  __device__ __forceinline__ void store(float4* g_lds) {
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
      const int i = (int)threadIdx.x + k * NT;
      if (i < NC * kWave) {
        uint4 q = r[k];
        const bool bad = nonfinite_bf16x8(q);
        if (__builtin_amdgcn_ballot_w64(bad) != 0) q = bad ? nan_group() : q;
        float v[8];
        unpack8(q, v);
        const int c = i / kWave, l = i % kWave;
        g_lds[(2 * c) * kWave + l] = make_float4(v[0], v[1], v[2], v[3]);
        g_lds[(2 * c + 1) * kWave + l] = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
    __syncthreads();
  }
};


// The rest of a register-resident row once its chunks are loaded: block
// maxima and the normaliser, then each chunk's products, scale, cast and
// stores.
template <int NC, int ELEM, int RND, int GM, int STAT>
__device__ __forceinline__ void mxnorm_row_reg(const NormArgs& A, uint4 (&raw)[NC],
                                               const float4* g_lds, int64_t row, int lane,
                                               uint32_t* sc) {
  const int dl = lane * 8;
  uint32_t mb[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    // every lane computes (the loads are clamped in bounds), then masks: no branch
    const uint32_t valid = 0u - (uint32_t)(c * kChunk + dl < A.D);
    mb[c] = quad_max_u32(absmax_bits8(raw[c]) & valid);
  }
  float inv;
  if constexpr (STAT == S_RMS) {
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      if (c * kChunk + dl < A.D) s = sumsq8(raw[c], s);
    inv = rms_normaliser(s, A.Df, A.eps);
  } else {
    auto lane_max = [&]() {
      uint32_t m = 0;
#pragma unroll
      for (int c = 0; c < NC; ++c) m = max(m, mb[c]);
      return m;
    };
    inv = row_normaliser<NC>(NC, [&](int c) { return mb[c]; }, lane_max, A.pmode, A.p, A.Kf);
  }
  if (lane == 0 && A.inv_out) A.inv_out[row] = inv;
  // The empty asm claims to rewrite the packed row, so the compiler widens
  // each chunk to fp32 where it is used below instead of ahead of the row
  // reduction, where all widened chunks would be live at once.
#pragma unroll
  for (int c = 0; c < NC; ++c)
    asm volatile("" : "+v"(raw[c].x), "+v"(raw[c].y), "+v"(raw[c].z), "+v"(raw[c].w));

  const uint64_t nrow = (uint64_t)row * (uint64_t)A.D;
  uint8_t* crow = code_row<ELEM>(A.codes, nrow);
  float g[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int d = c * kChunk + dl;
    if (d < A.D) {
      if (GM != G_NONE) gains(g_lds, c, lane, g);
      const uint32_t code = mxnorm_chunk<ELEM, RND, GM>(A, crow, nrow, d, raw[c], g, mb[c], inv);
      // block d / 32 = 16 c + lane / 4: the chunk's part is an immediate offset
      if ((lane & 3) == 0) put_scale(sc, c * 16 + (lane >> 2), code);
    }
  }
  flush_scales(sc, A.scales + (uint64_t)row * (uint64_t)A.K, A.K, A.sc_vec != 0, lane);
}

// Register-resident row: NC chunks of 512 elements held in VGPRs. The
// workgroup's rows share one LDS copy of gamma.

template <int NC, int ELEM, int RND, bool GAMMA, int STAT>
__global__ __launch_bounds__(kThreads) void mxnorm_reg_kernel(NormArgs A) {
  __shared__ float4 g_lds[GAMMA ? NC * kWave * 2 : 1];
  __shared__ uint32_t sc_lds[kRowsPerBlock][NC * 4];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // wave-uniform
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + wave;
  const bool live = row < A.T;
  const uint16_t* xr = A.x + (live ? row : A.T - 1) * A.ldx;  // a dead wave reads the last row
  const int dl = lane * 8;

  GammaStage<GAMMA ? NC : 1, kThreads> gs;
  if (GAMMA) gs.load(A.gamma, A.D);
  __builtin_amdgcn_sched_barrier(0);  // keep the gain loads ahead of the row loads
  uint4 raw[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) raw[c] = load_chunk(xr, c, dl, A.D);
  __builtin_amdgcn_sched_barrier(0);
  if (GAMMA) gs.store(g_lds);  // the row loads stay in flight meanwhile
  if (!live) return;
  uint32_t* sc = sc_lds[wave];
  if (!GAMMA)
    mxnorm_row_reg<NC, ELEM, RND, G_NONE, STAT>(A, raw, g_lds, row, lane, sc);
  else
    mxnorm_row_reg<NC, ELEM, RND, G_GAIN, STAT>(A, raw, g_lds, row, lane, sc);
}

constexpr int kMaxLdsRows = 16;  // wavefronts (rows) per workgroup of the LDS-staged variant

// LDS-staged row: each wavefront copies its row into its own LDS slice with
// direct-to-LDS loads (no VGPR staging), then runs the same two halves
// reading chunks back from LDS. The chunk loop is not unrolled, so rows up to
// MXQ_MAX_D fit; a lane only ever reads back the 16 bytes it loaded. gamma
// stays bf16 in LDS here (it is widened per use, to the same fp32 values).
// Dynamic LDS: [rows][nchunks * 64] uint4 row slices, gamma [nchunks * 64]
// uint4, then [rows][nchunks * 4] dwords of scales.
template <int ELEM, int RND, bool GAMMA, int STAT>
__global__ __launch_bounds__(kMaxLdsRows * kWave) void mxnorm_lds_kernel(NormArgs A, int nchunks, int rows) {
  extern __shared__ uint4 lds_rows[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // wave-uniform
  const int64_t row = (int64_t)blockIdx.x * rows + wave;
  const bool live = row < A.T;
  const uint16_t* xr = A.x + (live ? row : 0) * A.ldx;
  const int dl = lane * 8;
  uint4* slice = lds_rows + (size_t)wave * nchunks * kWave;
  uint4* g_lds = lds_rows + (size_t)rows * nchunks * kWave;
  uint32_t* sc = reinterpret_cast<uint32_t*>(g_lds + (GAMMA ? nchunks * kWave : 0)) +
                 (size_t)wave * nchunks * 4;

  // gamma first: the memory counter retires loads in order (see GammaStage)
  if (GAMMA) {
    for (int i = threadIdx.x; i < nchunks * kWave; i += rows * kWave) {
      const uint4 r = (i * 8 < A.D) ? load16(A.gamma + i * 8) : make_uint4(0, 0, 0, 0);
      g_lds[i] = nonfinite_bf16x8(r) ? nan_group() : r;  // see G_GAIN
    }
  }
  if (live) {
    for (int c = 0; c < nchunks; ++c) {
      if (c * kChunk + dl < A.D)
        __builtin_amdgcn_global_load_lds((const void*)(xr + c * kChunk + dl),
                                         (lds_void*)(slice + c * kWave), 16, 0, 0);
      else
        slice[c * kWave + lane] = make_uint4(0, 0, 0, 0);
    }
  }
  if (GAMMA) __syncthreads();
  if (!live) return;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  auto mb = [&](int c) { return quad_max_u32(absmax_bits8(slice[c * kWave + lane])); };
  float inv;
  if constexpr (STAT == S_RMS) {
    float s = 0.0f;
    for (int c = 0; c < nchunks; ++c)
      if (c * kChunk + dl < A.D) s = sumsq8(slice[c * kWave + lane], s);
    inv = rms_normaliser(s, A.Df, A.eps);
  } else {
    auto lane_max = [&]() {
      uint32_t m = 0;
      for (int c = 0; c < nchunks; ++c) m = max(m, mb(c));
      return m;
    };
    inv = row_normaliser<0>(nchunks, mb, lane_max, A.pmode, A.p, A.Kf);
  }
  if (lane == 0 && A.inv_out) A.inv_out[row] = inv;

  const uint64_t nrow = (uint64_t)row * (uint64_t)A.D;
  uint8_t* crow = code_row<ELEM>(A.codes, nrow);
  float g[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int c = 0; c < nchunks; ++c) {
    const int d = c * kChunk + dl;
    if (d < A.D) {
      const uint4 xb = slice[c * kWave + lane];
      uint32_t code;
      if (!GAMMA) {
        code = mxnorm_chunk<ELEM, RND, G_NONE>(A, crow, nrow, d, xb, g, mb(c), inv);
      } else {
        unpack8(g_lds[c * kWave + lane], g);
        code = mxnorm_chunk<ELEM, RND, G_GAIN>(A, crow, nrow, d, xb, g, 0u, inv);
      }
      if ((lane & 3) == 0) put_scale(sc, d >> 5, code);
    }
  }
  flush_scales(sc, A.scales + (uint64_t)row * (uint64_t)A.K, A.K, A.sc_vec != 0, lane);
}

// ------------------------------------------------------------------ RMSNorm

struct RmsArgs {
  const uint16_t* x;
  const uint16_t* gamma;
  uint16_t* y;
  float* inv_out;
  int64_t ldx;
  int64_t T;
  int D;
  float Df;
  float eps;
};


template <bool GAMMA>
__device__ __forceinline__ void rms_chunk_out(const RmsArgs& A, int64_t row, int d, const uint4& xb,
                                              float inv) {
  float v[8];
  unpack8(xb, v);
  if (GAMMA) {
    float g[8];
    unpack8(load16(A.gamma + d), g);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = v[j] * g[j];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = v[j] * inv;
  uint4 o;
  o.x = pack_bf16x2(v[0], v[1]);
  o.y = pack_bf16x2(v[2], v[3]);
  o.z = pack_bf16x2(v[4], v[5]);
  o.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(A.y + (uint64_t)row * (uint64_t)A.D + (uint64_t)d) = o;
}

// Row in registers (D <= NC * 512).
template <int NC, bool GAMMA>
__global__ __launch_bounds__(kThreads) void rmsnorm_reg_kernel(RmsArgs A) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= A.T) return;
  const uint16_t* xr = A.x + row * A.ldx;
  const int dl = lane * 8;
  uint4 raw[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) raw[c] = load_chunk(xr, c, dl, A.D);
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (c * kChunk + dl < A.D) s = sumsq8(raw[c], s);
  const float inv = rms_normaliser(s, A.Df, A.eps);
  if (lane == 0 && A.inv_out) A.inv_out[row] = inv;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int d = c * kChunk + dl;
    if (d < A.D) rms_chunk_out<GAMMA>(A, row, d, raw[c], inv);
  }
}

// Wide rows: the second half reads x again (from cache or HBM).
template <bool GAMMA>
__global__ __launch_bounds__(kThreads) void rmsnorm_wide_kernel(RmsArgs A, int nchunks) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= A.T) return;
  const uint16_t* xr = A.x + row * A.ldx;
  const int dl = lane * 8;
  float s = 0.0f;
  for (int c = 0; c < nchunks; ++c)
    if (c * kChunk + dl < A.D) s = sumsq8(load16(xr + c * kChunk + dl), s);
  const float inv = rms_normaliser(s, A.Df, A.eps);
  if (lane == 0 && A.inv_out) A.inv_out[row] = inv;
  for (int c = 0; c < nchunks; ++c) {
    const int d = c * kChunk + dl;
    if (d < A.D) rms_chunk_out<GAMMA>(A, row, d, load16(xr + d), inv);
  }
}

// ------------------------------------------------------------------ MXCast

struct CastArgs {
  const uint16_t* x;
  uint8_t* codes;
  uint8_t* scales;
  int64_t ldx;
  uint32_t total_chunks;  // T * chunks_per_row
  uint32_t chunks_per_row;
  int D;
  int K;
  int sc_vec;  // every chunk holds 16 blocks (D % 512 == 0) and scales take dword stores
  int ceil_rule;  // E8M0 round-up rule instead of the floor rule
  SrStream rng;
};

template <int ELEM, int RND>
__global__ __launch_bounds__(kThreads) void mxcast_kernel(CastArgs A) {
  __shared__ uint32_t sc_lds[kRowsPerBlock][kCastChunksPerWave * 4];
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const uint32_t g0 = (blockIdx.x * kRowsPerBlock + wave) * kCastChunksPerWave;
  const int dl = lane * 8;
  uint4 raw[kCastChunksPerWave];
  uint32_t rows[kCastChunksPerWave];
  int ds[kCastChunksPerWave];
#pragma unroll
  for (int u = 0; u < kCastChunksPerWave; ++u) {
    const uint32_t g = min(g0 + u, A.total_chunks - 1);  // past the end: re-read the last chunk
    const uint32_t r = g / A.chunks_per_row;
    rows[u] = r;
    const int c = (int)(g - r * A.chunks_per_row);
    ds[u] = c * kChunk + dl;
    raw[u] = load_chunk(A.x + (int64_t)r * A.ldx, c, dl, A.D);
  }
  uint32_t* sc = sc_lds[wave];
#pragma unroll
  for (int u = 0; u < kCastChunksPerWave; ++u) {
    if (g0 + u < A.total_chunks && ds[u] < A.D) {
      const uint32_t mbits = quad_max_u32(absmax_bits8(raw[u]));
      const BlockScale s = e8m0_scale<ELEM>(__uint_as_float(mbits << 16),
                                            A.ceil_rule ? scale_adjust<ELEM>() : 0u);
      const uint32_t code = s.code;
      float v[8];
      unpack8(raw[u], v);
      const uint64_t nrow = (uint64_t)rows[u] * (uint64_t)A.D;
      encode_store8<ELEM, RND>(code_row<ELEM>(A.codes, nrow), (uint32_t)ds[u], nrow + ds[u], v,
                               s, A.rng);
      if ((lane & 3) == 0) {
        if (A.sc_vec)
          put_scale(sc, u * 16 + (lane >> 2), code);
        else
          A.scales[(uint64_t)rows[u] * (uint64_t)A.K + (uint64_t)(ds[u] >> 5)] = (uint8_t)code;
      }
    }
  }
  if (A.sc_vec && g0 < A.total_chunks) {
    // with 16 blocks per chunk, block q of chunk g sits at scale index 16 g + q
    const uint32_t nvalid = min((uint32_t)kCastChunksPerWave, A.total_chunks - g0);
    flush_scales(sc, A.scales + (uint64_t)g0 * 16u, (int)(16 * nvalid), true, lane);
  }
}

// ------------------------------------------------------------------ launch helpers



// Workgroup counts above this are refused (the x dimension of a grid).
constexpr int64_t kMaxGrid = 0x7FFFFFFF;

template <int NC, int ELEM, int RND, bool GAMMA, int STAT>
mxq_status launch_mxnorm_reg(const NormArgs& A, hipStream_t s) {
  if ((A.T + kRowsPerBlock - 1) / kRowsPerBlock > kMaxGrid) return MXQ_ERR_UNSUPPORTED;
  const unsigned grid = (unsigned)((A.T + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL((mxnorm_reg_kernel<NC, ELEM, RND, GAMMA, STAT>), dim3(grid), dim3(kThreads), 0, s, A);
  MXQ_LAUNCH_CHECK();
  return MXQ_OK;
}

template <int ELEM, int RND, bool GAMMA, int STAT>
mxq_status dispatch_mxnorm_reg(const NormArgs& A, int nc, hipStream_t s) {
  switch (nc) {
#define MXQ_CASE(N) \
  case N:           \
    return launch_mxnorm_reg<N, ELEM, RND, GAMMA, STAT>(A, s);
    MXQ_CASE(1) MXQ_CASE(2) MXQ_CASE(3) MXQ_CASE(4) MXQ_CASE(5) MXQ_CASE(6) MXQ_CASE(7)
    MXQ_CASE(8) MXQ_CASE(9) MXQ_CASE(10) MXQ_CASE(11) MXQ_CASE(12) MXQ_CASE(13) MXQ_CASE(14)
    MXQ_CASE(15) MXQ_CASE(16)
#undef MXQ_CASE
    default:
      return MXQ_ERR_UNSUPPORTED;
  }
}

constexpr size_t kLdsPerBlockMax = 160 * 1024;  // gfx950 LDS per workgroup

template <int ELEM, int RND, bool GAMMA, int STAT>
mxq_status launch_mxnorm_lds(const NormArgs& A, int nc, hipStream_t s) {
  // per row: the bf16 row and its scale bytes; per workgroup: bf16 gamma.
  // Rows per workgroup: the count that keeps the most rows resident per CU
  // (LDS is the limit), the smaller one on ties.
  const size_t per_row = (size_t)nc * kWave * sizeof(uint4) + (size_t)nc * 16;
  const size_t g_bytes = GAMMA ? (size_t)nc * kWave * sizeof(uint4) : 0;
  if (per_row + g_bytes > kLdsPerBlockMax) return MXQ_ERR_UNSUPPORTED;
  int rows = 1;
  size_t best = 0;
  for (int r = 1; r <= kMaxLdsRows; ++r) {
    const size_t b = per_row * r + g_bytes;
    if (b > kLdsPerBlockMax) break;
    const size_t resident = (size_t)r * (kLdsPerBlockMax / b);
    if (resident > best) {
      best = resident;
      rows = r;
    }
  }
  const size_t bytes = per_row * rows + g_bytes;
  if ((A.T + rows - 1) / rows > kMaxGrid) return MXQ_ERR_UNSUPPORTED;
  auto kern = mxnorm_lds_kernel<ELEM, RND, GAMMA, STAT>;
  if (bytes > 64 * 1024 &&
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)bytes) != hipSuccess)
    return MXQ_ERR_HIP;
  const unsigned grid = (unsigned)((A.T + rows - 1) / rows);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kWave * rows), bytes, s, A, nc, rows);
  MXQ_LAUNCH_CHECK();
  return MXQ_OK;
}

template <int ELEM, int RND, int STAT>
mxq_status dispatch_mxnorm(const NormArgs& A, bool gamma, bool lds, int nc, hipStream_t s) {
  if (lds)
    return gamma ? launch_mxnorm_lds<ELEM, RND, true, STAT>(A, nc, s)
                 : launch_mxnorm_lds<ELEM, RND, false, STAT>(A, nc, s);
  return gamma ? dispatch_mxnorm_reg<ELEM, RND, true, STAT>(A, nc, s)
               : dispatch_mxnorm_reg<ELEM, RND, false, STAT>(A, nc, s);
}

template <int STAT>
mxq_status dispatch_norm_cast(const NormArgs& A, mxq_elem elem, mxq_round rnd, bool gamma,
                              bool lds, int nc, hipStream_t s) {
  if (elem == MXQ_E4M3)
    return rnd == MXQ_SR ? dispatch_mxnorm<MXQ_E4M3, MXQ_SR, STAT>(A, gamma, lds, nc, s)
                         : dispatch_mxnorm<MXQ_E4M3, MXQ_RNE, STAT>(A, gamma, lds, nc, s);
  return rnd == MXQ_SR ? dispatch_mxnorm<MXQ_E2M1, MXQ_SR, STAT>(A, gamma, lds, nc, s)
                       : dispatch_mxnorm<MXQ_E2M1, MXQ_RNE, STAT>(A, gamma, lds, nc, s);
}

template <int NC, bool GAMMA>
mxq_status launch_rms_reg(const RmsArgs& A, hipStream_t s) {
  if ((A.T + kRowsPerBlock - 1) / kRowsPerBlock > kMaxGrid) return MXQ_ERR_UNSUPPORTED;
  const unsigned grid = (unsigned)((A.T + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL((rmsnorm_reg_kernel<NC, GAMMA>), dim3(grid), dim3(kThreads), 0, s, A);
  MXQ_LAUNCH_CHECK();
  return MXQ_OK;
}

template <bool GAMMA>
mxq_status dispatch_rms(const RmsArgs& A, int nc, hipStream_t s) {
  switch (nc) {
#define MXQ_CASE(N) \
  case N:           \
    return launch_rms_reg<N, GAMMA>(A, s);
    MXQ_CASE(1) MXQ_CASE(2) MXQ_CASE(3) MXQ_CASE(4) MXQ_CASE(5) MXQ_CASE(6) MXQ_CASE(7)
    MXQ_CASE(8) MXQ_CASE(9) MXQ_CASE(10) MXQ_CASE(11) MXQ_CASE(12) MXQ_CASE(13) MXQ_CASE(14)
    MXQ_CASE(15) MXQ_CASE(16)
#undef MXQ_CASE
    default: {
      if ((A.T + kRowsPerBlock - 1) / kRowsPerBlock > kMaxGrid) return MXQ_ERR_UNSUPPORTED;
      const unsigned grid = (unsigned)((A.T + kRowsPerBlock - 1) / kRowsPerBlock);
      hipLaunchKernelGGL((rmsnorm_wide_kernel<GAMMA>), dim3(grid), dim3(kThreads), 0, s, A, nc);
      MXQ_LAUNCH_CHECK();
      return MXQ_OK;
    }
  }
}

template <int ELEM, int RND>
mxq_status launch_cast(const CastArgs& A, hipStream_t s) {
  const uint32_t per_block = kRowsPerBlock * kCastChunksPerWave;
  const unsigned grid = (A.total_chunks + per_block - 1) / per_block;
  hipLaunchKernelGGL((mxcast_kernel<ELEM, RND>), dim3(grid), dim3(kThreads), 0, s, A);
  MXQ_LAUNCH_CHECK();
  return MXQ_OK;
}

mxq_status dispatch_cast(const CastArgs& A, mxq_elem elem, mxq_round rnd, hipStream_t s) {
  if (elem == MXQ_E4M3)
    return rnd == MXQ_SR ? launch_cast<MXQ_E4M3, MXQ_SR>(A, s) : launch_cast<MXQ_E4M3, MXQ_RNE>(A, s);
  return rnd == MXQ_SR ? launch_cast<MXQ_E2M1, MXQ_SR>(A, s) : launch_cast<MXQ_E2M1, MXQ_RNE>(A, s);
}


// ------------------------------------------------------------------ validation

mxq_status check_common(const uint16_t* x, int64_t ldx, int64_t T, int64_t D, mxq_elem elem,
                        mxq_round rnd, const mxq_rng* rng, const uint8_t* codes,
                        const uint8_t* scales) {
  if (T < 0 || D <= 0 || D % 32 != 0 || ldx < D) return MXQ_ERR_SHAPE;
  if (elem != MXQ_E4M3 && elem != MXQ_E2M1) return MXQ_ERR_ARG;
  if (rnd != MXQ_RNE && rnd != MXQ_SR) return MXQ_ERR_ARG;
  if (rnd == MXQ_SR && rng == nullptr) return MXQ_ERR_ARG;
  if (T == 0) return MXQ_OK;
  if (x == nullptr || codes == nullptr || scales == nullptr) return MXQ_ERR_NULL;
  if (!aligned(x, 16) || ldx % 8 != 0 || !aligned(codes, 16)) return MXQ_ERR_ALIGN;
  if ((uint64_t)T * (uint64_t)D >= (1ull << 40)) return MXQ_ERR_UNSUPPORTED;
  return MXQ_OK;
}

SrStream make_stream(const mxq_rng* rng) {
  SrStream s{0, 0, 0, 0};
  if (rng) {
    s.k0 = (uint32_t)rng->seed;
    s.k1 = (uint32_t)(rng->seed >> 32);
    s.o0 = (uint32_t)rng->offset;
    s.o1 = (uint32_t)(rng->offset >> 32);
  }
  return s;
}

// Validation and launch shared by the single-pass normalise-and-cast entry
// points; the statistic's own argument (p or eps) is checked by the caller.
template <int STAT>
mxq_status norm_cast(const uint16_t* x, int64_t ldx, const uint16_t* gamma, int64_t T, int64_t D,
                     float p, float eps, mxq_elem elem, mxq_round rnd, const mxq_rng* rng,
                     uint32_t flags, uint8_t* codes, uint8_t* scales, float* inv_out,
                     void* stream) {
  if (flags & ~(uint32_t)(MXQ_FLAG_FORCE_REG | MXQ_FLAG_FORCE_LDS | MXQ_FLAG_SCALE_CEIL))
    return MXQ_ERR_ARG;
  if ((flags & MXQ_FLAG_FORCE_REG) && (flags & MXQ_FLAG_FORCE_LDS)) return MXQ_ERR_ARG;
  if (D > MXQ_MAX_D) return MXQ_ERR_UNSUPPORTED;
  if ((flags & MXQ_FLAG_FORCE_REG) && D > MXQ_MAX_D_REG) return MXQ_ERR_UNSUPPORTED;
  if (T == 0) return MXQ_OK;
  if (gamma != nullptr && !aligned(gamma, 16)) return MXQ_ERR_ALIGN;
  if (inv_out != nullptr && !aligned(inv_out, 4)) return MXQ_ERR_ALIGN;

  NormArgs A;
  A.x = x;
  A.gamma = gamma;
  A.codes = codes;
  A.scales = scales;
  A.inv_out = inv_out;
  A.ldx = ldx;
  A.T = T;
  A.D = (int)D;
  A.K = (int)(D / 32);
  A.Kf = (float)(D / 32);
  A.p = p;
  A.pmode = isinf(p) ? P_INF : (p == 1.0f ? P_ONE : (p == 2.0f ? P_TWO : P_GEN));
  A.Df = (float)D;
  A.eps = eps;
  A.sc_vec = (A.K % 4 == 0) && aligned(scales, 4);
  A.ceil_rule = (flags & MXQ_FLAG_SCALE_CEIL) != 0;
  A.rng = make_stream(rng);
  const int nc = (int)((D + kChunk - 1) / kChunk);
  const bool lds = (flags & MXQ_FLAG_FORCE_LDS) || (!(flags & MXQ_FLAG_FORCE_REG) && D > MXQ_MAX_D_REG);
  return dispatch_norm_cast<STAT>(A, elem, rnd, gamma != nullptr, lds, nc, (hipStream_t)stream);
}

}  // namespace

// ------------------------------------------------------------------ C ABI

extern "C" {

mxq_status mxnorm_fwd(const uint16_t* x, int64_t ldx, const uint16_t* gamma, int64_t T,
                      int64_t D, float p, mxq_elem elem, mxq_round rnd, const mxq_rng* rng,
                      uint32_t flags, uint8_t* codes, uint8_t* scales, float* inv_norm,
                      void* stream) {
  mxq_status st = check_common(x, ldx, T, D, elem, rnd, rng, codes, scales);
  if (st != MXQ_OK) return st;
  if (!(p > 0.0f)) return MXQ_ERR_ARG;  // also rejects NaN
  return norm_cast<S_PMEAN>(x, ldx, gamma, T, D, p, 0.0f, elem, rnd, rng, flags, codes, scales,
                            inv_norm, stream);
}

mxq_status rmsnorm_mxcast_fused_fwd(const uint16_t* x, int64_t ldx, const uint16_t* gamma,
                                    int64_t T, int64_t D, float eps, mxq_elem elem,
                                    mxq_round rnd, const mxq_rng* rng, uint32_t flags,
                                    uint8_t* codes, uint8_t* scales, float* inv_rms,
                                    void* stream) {
  mxq_status st = check_common(x, ldx, T, D, elem, rnd, rng, codes, scales);
  if (st != MXQ_OK) return st;
  if (!(eps >= 0.0f) || isinf(eps)) return MXQ_ERR_ARG;
  return norm_cast<S_RMS>(x, ldx, gamma, T, D, 2.0f, eps, elem, rnd, rng, flags, codes, scales,
                          inv_rms, stream);
}

mxq_status rmsnorm_mxcast_fwd(const uint16_t* x, int64_t ldx, const uint16_t* gamma,
                              int64_t T, int64_t D, float eps, mxq_elem elem, mxq_round rnd,
                              const mxq_rng* rng, uint32_t flags, uint16_t* y_workspace,
                              uint8_t* codes, uint8_t* scales, float* inv_rms, void* stream) {
  mxq_status st = check_common(x, ldx, T, D, elem, rnd, rng, codes, scales);
  if (st != MXQ_OK) return st;
  if (!(eps >= 0.0f) || isinf(eps)) return MXQ_ERR_ARG;
  if (flags & ~(uint32_t)MXQ_FLAG_SCALE_CEIL) return MXQ_ERR_ARG;
  if (D > MXQ_MAX_D) return MXQ_ERR_UNSUPPORTED;
  if (T == 0) return MXQ_OK;
  // the cast pass counts 512-element chunks in 32 bits, as mxcast_fwd does
  if ((uint64_t)T * (uint64_t)((D + kChunk - 1) / kChunk) >= (1ull << 32) - kThreads)
    return MXQ_ERR_UNSUPPORTED;
  if (y_workspace == nullptr) return MXQ_ERR_NULL;
  if (!aligned(y_workspace, 16)) return MXQ_ERR_ALIGN;
  if (gamma != nullptr && !aligned(gamma, 16)) return MXQ_ERR_ALIGN;
  if (inv_rms != nullptr && !aligned(inv_rms, 4)) return MXQ_ERR_ALIGN;

  hipStream_t s = (hipStream_t)stream;
  RmsArgs R;
  R.x = x;
  R.gamma = gamma;
  R.y = y_workspace;
  R.inv_out = inv_rms;
  R.ldx = ldx;
  R.T = T;
  R.D = (int)D;
  R.Df = (float)D;
  R.eps = eps;
  const int nc = (int)((D + kChunk - 1) / kChunk);
  st = gamma ? dispatch_rms<true>(R, nc, s) : dispatch_rms<false>(R, nc, s);
  if (st != MXQ_OK) return st;

  CastArgs C;
  C.x = y_workspace;
  C.codes = codes;
  C.scales = scales;
  C.ldx = D;
  C.chunks_per_row = (uint32_t)nc;
  C.total_chunks = (uint32_t)(T * nc);
  C.D = (int)D;
  C.K = (int)(D / 32);
  C.sc_vec = (D % kChunk == 0) && aligned(scales, 4);
  C.ceil_rule = (flags & MXQ_FLAG_SCALE_CEIL) != 0;
  C.rng = make_stream(rng);
  return dispatch_cast(C, elem, rnd, s);
}

mxq_status mxcast_fwd(const uint16_t* x, int64_t ldx, int64_t T, int64_t D, mxq_elem elem,
                      mxq_round rnd, const mxq_rng* rng, uint32_t flags, uint8_t* codes,
                      uint8_t* scales, void* stream) {
  mxq_status st = check_common(x, ldx, T, D, elem, rnd, rng, codes, scales);
  if (st != MXQ_OK) return st;
  if (flags & ~(uint32_t)MXQ_FLAG_SCALE_CEIL) return MXQ_ERR_ARG;
  if (T == 0) return MXQ_OK;
  const uint64_t nc = (uint64_t)((D + kChunk - 1) / kChunk);
  if ((uint64_t)T * nc >= (1ull << 32) - kThreads) return MXQ_ERR_UNSUPPORTED;
  CastArgs C;
  C.x = x;
  C.codes = codes;
  C.scales = scales;
  C.ldx = ldx;
  C.chunks_per_row = (uint32_t)nc;
  C.total_chunks = (uint32_t)(T * nc);
  C.D = (int)D;
  C.K = (int)(D / 32);
  C.sc_vec = (D % kChunk == 0) && aligned(scales, 4);
  C.ceil_rule = (flags & MXQ_FLAG_SCALE_CEIL) != 0;
  C.rng = make_stream(rng);
  return dispatch_cast(C, elem, rnd, (hipStream_t)stream);
}

const char* mxq_strerror(mxq_status status) {
  switch (status) {
    case MXQ_OK: return "ok";
    case MXQ_ERR_NULL: return "a required pointer is NULL";
    case MXQ_ERR_SHAPE: return "bad shape: need T >= 0, D > 0, D % 32 == 0, ldx >= D";
    case MXQ_ERR_ALIGN: return "misaligned pointer or row stride (16-byte rows and buffers)";
    case MXQ_ERR_ARG: return "bad argument (p, eps, element format, rounding, flags or rng)";
    case MXQ_ERR_UNSUPPORTED: return "unsupported size for this path";
    case MXQ_ERR_HIP: return "HIP runtime refused the kernel launch";
  }
  return "unknown status";
}

int mxq_abi_version(void) { return MXQ_ABI_VERSION; }

}  // extern "C"
