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
//     the FP4 convert saturates by itself. Stochastic rounding uses the
//     gfx950 stochastic-rounding converts fed the complement of each
//     element's Philox4x32-10 word (see encode8_e4m3_sr).
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

// Every kernel adds a row's statistic in one canonical order, whatever its
// work layout: the row is cut into groups of kGroupChunks chunks (2048
// elements); within a group each lane adds its chunks' terms in chunk order,
// the group total is the sum over the quads (or the wave, for the RMS) of
// those lane sums, and the group totals are added in group order. Register,
// LDS and split-row kernels therefore produce the same bits.
constexpr int kGroupChunks = 4;

// Term of the power mean for one block maximum m (m >= 0).
__device__ __forceinline__ float pmean_add(float s, float m, int pmode, float p) {
  if (pmode == P_ONE) return s + m;
  if (pmode == P_TWO) return __builtin_fmaf(m, m, s);
  return s + exp2f(p * log2f(m));  // m == 0 -> exp2(-inf) == 0
}

// (s / K)^(1/p). Kinv is 1/K when K is a power of two (then s * Kinv is s / K
// exactly) and 0 otherwise.
__device__ __forceinline__ float pmean_finish(float s, int pmode, float p, float K, float Kinv) {
  const float q = Kinv != 0.0f ? s * Kinv : s / K;
  if (pmode == P_ONE) return q;
  if (pmode == P_TWO) return sqrtf(q);
  return exp2f(log2f(q) / p);
}

// One lane's sum of the power-mean terms of chunks [c0, c1) in chunk order, of
// the block maxima scaled by 2^shift (mb(c): the lane's quad's maximum of chunk
// c as bf16 bits, 0 past the row end). UNROLL > 0: c1 - c0 <= UNROLL, unrolled.
template <int UNROLL, int PM, class BlockMax>
__device__ __forceinline__ float lane_terms_p(int c0, int c1, BlockMax mb, int shift, float p) {
  float s = 0.0f;
  if constexpr (UNROLL > 0) {
#pragma unroll
    for (int k = 0; k < UNROLL; ++k)
      if (c0 + k < c1) s = pmean_add(s, ldexpf(__uint_as_float(mb(c0 + k) << 16), shift), PM, p);
  } else {
    for (int c = c0; c < c1; ++c) s = pmean_add(s, ldexpf(__uint_as_float(mb(c) << 16), shift), PM, p);
  }
  return s;
}

// Group total of chunks [c0, c1) (one group): lane sums, then over the quads.
// The power mode is tested once, outside the term loop.
template <int UNROLL, class BlockMax>
__device__ __forceinline__ float group_terms(int c0, int c1, BlockMax mb, int shift, int pmode,
                                             float p) {
  float t;
  if (pmode == P_TWO)
    t = lane_terms_p<UNROLL, P_TWO>(c0, c1, mb, shift, p);
  else if (pmode == P_ONE)
    t = lane_terms_p<UNROLL, P_ONE>(c0, c1, mb, shift, p);
  else
    t = lane_terms_p<UNROLL, P_GEN>(c0, c1, mb, shift, p);
  return sum_over_quads(t);
}

// The canonical total over a whole row held by one wave (nchunks chunks; NCT > 0
// a compile-time count, unrolled).
template <int NCT, class BlockMax>
__device__ __forceinline__ float row_terms(int nchunks, BlockMax mb, int shift, int pmode, float p) {
  float total = 0.0f;
  if constexpr (NCT > 0) {
#pragma unroll
    for (int g0 = 0; g0 < NCT; g0 += kGroupChunks)
      total += group_terms<kGroupChunks>(g0, min(g0 + kGroupChunks, NCT), mb, shift, pmode, p);
  } else {
    for (int g0 = 0; g0 < nchunks; g0 += kGroupChunks)
      total += group_terms<kGroupChunks>(g0, min(g0 + kGroupChunks, nchunks), mb, shift, pmode, p);
  }
  return total;
}

// floor(log2) of a nonzero finite bf16 magnitude given as bits 0x0001 .. 0x7F7F:
// the unbiased exponent, or for a subnormal the position of its leading
// mantissa bit (value = mantissa * 2^-133).
__device__ __forceinline__ int bf16_exponent(uint32_t m) {
  const int ef = (int)(m >> 7);
  return ef ? ef - 127 : -133 + (31 - __builtin_clz(m));
}

// Whether a row whose direct total is s is finished without the rescaled total
// (p = inf never needs a total). For p = 1 and 2 a total inside [2^-96, 2^96]
// always gives G >= 2^-106 (K <= 1024), so only other p compute G here.
__device__ __forceinline__ bool direct_total_suffices(float s, int pmode, float p, float K,
                                                      float Kinv) {
  return pmode != P_INF && s >= 0x1p-96f && s <= 0x1p96f &&
         (pmode == P_ONE || pmode == P_TWO || pmean_finish(s, pmode, p, K, Kinv) >= 0x1p-126f);
}

// A row's normaliser. The products v = x * gamma are multiplied by `apply`
// after an exact power-of-two pre-scaling by `pre`: y = RN32((v * pre) * apply).
// `inv` is RN32(1/G), the value reported per row. While 1/G fits fp32, pre = 1
// and apply = inv, so y = RN32(v * inv). When 1/G exceeds the fp32 range (a
// finite row whose block maxima are all below about 2^-128), inv is +Inf,
// pre = 2^64 and apply = RN32(1/G) * 2^-64: the same fp32 mantissa applied at
// an exponent fp32 can hold, so y is what RN32(v * RN32(1/G)) would be with an
// unbounded exponent.
struct Normaliser {
  float inv;
  float apply;
  float pre;
};

__device__ __forceinline__ Normaliser plain_normaliser(float inv) { return {inv, inv, 1.0f}; }

// Normaliser 1/G of a row from its statistic. total(shift) gives the row's
// canonical total of the terms of the block maxima scaled by 2^shift;
// row_max() the row's largest block maximum as bf16 bits. A direct total
// inside [2^-96, 2^96] is finite and nonzero, so the row holds no NaN or Inf
// (either would make it non-finite) and is not all zero; if G is also a normal
// fp32 value, inv = 1/G. Otherwise the row maximum decides: NaN or Inf in the
// row gives NaN, an all-zero row 0; else the maxima are rescaled by 2^-E,
// E = floor(log2 of the row maximum), so the largest lies in [1, 2), and
// G = G' * 2^E. p = inf takes this path always.
template <class Total, class RowMax>
__device__ __forceinline__ Normaliser row_normaliser(Total total, RowMax row_max, int pmode, float p,
                                                     float K, float Kinv) {
  if (pmode != P_INF) {
    const float s = total(0);
    if (s >= 0x1p-96f && s <= 0x1p96f) {
      const float G = pmean_finish(s, pmode, p, K, Kinv);
      if (G >= 0x1p-126f) return plain_normaliser(1.0f / G);
    }
  }
  const uint32_t rmax = row_max();
  if (rmax >= 0x7F80u) return plain_normaliser(__builtin_nanf(""));  // the row holds NaN or Inf
  if (rmax == 0u) return plain_normaliser(0.0f);                      // all-zero row
  const int E = bf16_exponent(rmax);
  const float Gs = (pmode == P_INF) ? ldexpf(__uint_as_float(rmax << 16), -E)
                                    : pmean_finish(total(-E), pmode, p, K, Kinv);
  const float G = ldexpf(Gs, E);
  if (G >= 0x1p-126f) return plain_normaliser(1.0f / G);
  // G below the normal range: scale RN32(1/G') instead of forming a subnormal G
  const float r = 1.0f / Gs;
  const float inv = ldexpf(r, -E);  // exact, or +Inf past the fp32 range
  if (inv <= 0x1.fffffep127f) return plain_normaliser(inv);
  return {inv, ldexpf(r, -E - 64), 0x1p64f};
}

// ------------------------------------------------------------------ RMS

// The RMS statistic's group total of chunks [c0, c1): each lane adds the
// squares of its chunks in chunk order, then the wave adds the lane sums.
template <int UNROLL, class Chunk>
__device__ __forceinline__ float group_sumsq(int c0, int c1, Chunk chunk) {
  float s = 0.0f;
  if constexpr (UNROLL > 0) {
#pragma unroll
    for (int k = 0; k < UNROLL; ++k)
      if (c0 + k < c1) s = chunk(c0 + k, s);
  } else {
    for (int c = c0; c < c1; ++c) s = chunk(c, s);
  }
  return sum_over_wave(s);
}

// The canonical sum of squares of a row held by one wave. chunk(c, s) adds
// chunk c's squares (zero for lanes past the row end) to the lane sum s.
template <int NCT, class Chunk>
__device__ __forceinline__ float row_sumsq(int nchunks, Chunk chunk) {
  float total = 0.0f;
  if constexpr (NCT > 0) {
#pragma unroll
    for (int g0 = 0; g0 < NCT; g0 += kGroupChunks)
      total += group_sumsq<kGroupChunks>(g0, min(g0 + kGroupChunks, NCT), chunk);
  } else {
    for (int g0 = 0; g0 < nchunks; g0 += kGroupChunks)
      total += group_sumsq<kGroupChunks>(g0, min(g0 + kGroupChunks, nchunks), chunk);
  }
  return total;
}

// RMSNorm's normaliser from the canonical sum of squares.
__device__ __forceinline__ float rms_inv(float total, float Df, float eps) {
  return 1.0f / sqrtf(total / Df + eps);
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
// and 0xCD9E8D57, key increments 0x9E3779B9 and 0xBB67AE85. Returns the
// bitwise complement of the four output words (what the stochastic-rounding
// converts take, see encode8_e4m3_sr): the last round's xors become xnors
// (truth table 0x69) and its two low products are inverted.
__device__ __forceinline__ uint4 philox4x32_10_not(uint32_t c0, uint32_t c1, uint32_t c2,
                                                   uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 9; ++i) {
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
  const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
  return make_uint4(__builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x69), ~(uint32_t)p1,
                    __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x69), ~(uint32_t)p0);
}

struct SrStream {
  uint32_t k0, k1, o0, o1;
  // Complemented words for logical elements n0 .. n0+7 (n0 % 8 == 0).
  __device__ __forceinline__ void words8_not(uint64_t n0, uint32_t r[8]) const {
    const uint64_t b = n0 >> 2;
    const uint4 a = philox4x32_10_not((uint32_t)b, (uint32_t)(b >> 32), o0, o1, k0, k1);
    const uint4 c = philox4x32_10_not((uint32_t)(b + 1), (uint32_t)((b + 1) >> 32), o0, o1, k0, k1);
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
    r[4] = c.x; r[5] = c.y; r[6] = c.z; r[7] = c.w;
  }
};

// ------------------------------------------------------------------ encode

// 8 values y (not yet divided by the scale) -> 8 E4M3 codes, RNE, saturating.
// A non-finite block is encoded like any other (its scale and limit are then
// meaningless values that fault nothing) and its codes are then replaced by
// NaN, behind a branch that a wavefront with no such block skips.
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
  uint32_t lo = __builtin_bit_cast(uint32_t, a), hi = __builtin_bit_cast(uint32_t, b);
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(bad) != 0, 0)) {  // rare, wavefront-uniform
    // kept a branch (the empty asm cannot be speculated): as selects the fix-up cost every
    // chunk three VALU instructions, 1% of the Llama-3 shape's time
    asm volatile("");
    lo = bad ? 0x7F7F7F7Fu : lo;
    hi = bad ? 0x7F7F7F7Fu : hi;
  }
  return make_uint2(lo, hi);
}

// 8 values -> 8 E2M1 codes packed in one word (element 2j in the low nibble).
__device__ __forceinline__ uint32_t encode8_e2m1_rne(const float y[8], BlockScale s) {
  const bool bad = s.bad;  // replaced after a wave-wide test, which compiles to selects here
  const float scale = __uint_as_float(s.code << 23);
  uint32_t q = __float_as_uint(y[0]);  // all four bytes are written below
  q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, y[0], y[1], scale, 0);
  q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, y[2], y[3], scale, 1);
  q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, y[4], y[5], scale, 2);
  q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, y[6], y[7], scale, 3);
  if (__builtin_amdgcn_ballot_w64(bad) != 0) q = bad ? 0x77777777u : q;
  return q;
}

// Stochastic rounding: with q = |y| / 2^s in units of the local quantum,
// n = floor(q) and f = q - n, round up iff r < 2^(32-B) * floor(f * 2^B), where
// r is the element's Philox word and B = 23 - (stored mantissa bits) is the
// number of fp32 mantissa bits the format drops (20 for E4M3, 22 for E2M1);
// saturating. The gfx950 stochastic-rounding converts take exactly this
// decision when fed ~r: they add the top B bits of their random operand to the
// top B bits of the fraction and round up on the carry, and
// f_B + (2^B - 1 - r_B) >= 2^B  <=>  r_B < f_B  (r_B, f_B the top B bits).
// Probed on the device against the rule over random values from 2^-45 to the
// format maximum (subnormal targets included) and at every threshold +- 1 and
// +- one step of the low bits; the FP4 convert is given one value per
// instruction (its pair partner zero), because it draws the second value's
// bits differently. Both converts are clamped first, like the FP8 RNE path
// (the FP8 convert does not saturate; 448 and 6 are on the grid, so a clamped
// value's fraction is zero and it stays put).
__device__ __forceinline__ uint2 encode8_e4m3_sr(const float y[8], BlockScale s, const uint32_t nr[8]) {
  const uint32_t code = s.code;
  const float scale = __uint_as_float(code << 23);
  const float lim = __uint_as_float(((code + 8u) << 23) | 0x00600000u);  // 448 * 2^(code-127)
  float w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = __builtin_amdgcn_fmed3f(y[j], -lim, lim);
  int lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(lo, w[0], nr[0], scale, 0);
  lo = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(lo, w[1], nr[1], scale, 1);
  lo = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(lo, w[2], nr[2], scale, 2);
  lo = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(lo, w[3], nr[3], scale, 3);
  hi = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(hi, w[4], nr[4], scale, 0);
  hi = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(hi, w[5], nr[5], scale, 1);
  hi = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(hi, w[6], nr[6], scale, 2);
  hi = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(hi, w[7], nr[7], scale, 3);
  return make_uint2(s.bad ? 0x7F7F7F7Fu : (uint32_t)lo, s.bad ? 0x7F7F7F7Fu : (uint32_t)hi);
}

typedef float float2_t __attribute__((ext_vector_type(2)));

// One value through the FP4 stochastic-rounding convert into byte SEL of acc
// (low nibble; the pair partner is zero, so the high nibble is 0). Written as
// assembly because the compiler does not carry the destination's other bytes
// from one call of this convert's builtin to the next; here the destination
// is an input and output of every instruction, as the hardware treats it.
template <int SEL>
__device__ __forceinline__ void cvt_sr_fp4_into(uint32_t& acc, float w, uint32_t nr, float scale) {
  const float2_t pair = {w, 0.0f};
  if constexpr (SEL == 0)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3" : "+v"(acc) : "v"(pair), "v"(nr), "v"(scale));
  else if constexpr (SEL == 1)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,0]"
        : "+v"(acc) : "v"(pair), "v"(nr), "v"(scale));
  else if constexpr (SEL == 2)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,0,1]"
        : "+v"(acc) : "v"(pair), "v"(nr), "v"(scale));
  else
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,1]"
        : "+v"(acc) : "v"(pair), "v"(nr), "v"(scale));
}

__device__ __forceinline__ uint32_t encode8_e2m1_sr(const float y[8], BlockScale s, const uint32_t nr[8]) {
  const uint32_t code = s.code;
  const float scale = __uint_as_float(code << 23);
  const float lim = __uint_as_float(((code + 2u) << 23) | 0x00400000u);  // 6 * 2^(code-127)
  float w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = __builtin_amdgcn_fmed3f(y[j], -lim, lim);
  // byte j of `even` holds element 2j in its low nibble, of `odd` element 2j+1
  uint32_t even = 0, odd = 0;
  cvt_sr_fp4_into<0>(even, w[0], nr[0], scale);
  cvt_sr_fp4_into<1>(even, w[2], nr[2], scale);
  cvt_sr_fp4_into<2>(even, w[4], nr[4], scale);
  cvt_sr_fp4_into<3>(even, w[6], nr[6], scale);
  cvt_sr_fp4_into<0>(odd, w[1], nr[1], scale);
  cvt_sr_fp4_into<1>(odd, w[3], nr[3], scale);
  cvt_sr_fp4_into<2>(odd, w[5], nr[5], scale);
  cvt_sr_fp4_into<3>(odd, w[7], nr[7], scale);
  return s.bad ? 0x77777777u : (even | (odd << 4));
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
    rng.words8_not(n, r);
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
  float Kinv;  // 1/K when K is a power of two, else 0
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
//   G_GAIN  gains: the IEEE-2019 maximum (gfx950 v_maximum3_f32, which returns
//           NaN when any input is NaN) with abs modifiers over the products, so
//           a product made NaN or Inf by a non-finite gain (a non-finite x
//           already makes the row's normaliser NaN) flags its block
//           non-finite, as it must.
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
  auto mx = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
  float m = mx(mx(fabsf(v[0]), fabsf(v[1])), fabsf(v[2]));
  m = mx(mx(m, fabsf(v[3])), fabsf(v[4]));
  m = mx(mx(m, fabsf(v[5])), fabsf(v[6]));
  m = mx(m, fabsf(v[7]));
  // integer max of non-negative floats (or NaN): NaN bits exceed every other value
  return quad_max_u32(__float_as_uint(m));
}

// Second half: y = RN(v * inv), E8M0 code from max |y| = RN(max |v| * inv)
// (rounding is monotone), codes stored. Returns the code of the lane's block.
// vmax_bits has its sign bit clear and inv is +0 or more, or NaN, so the
// maximum is +0 or more, or NaN, as e8m0_scale expects. A normaliser past the
// fp32 range first scales v and its maximum by N.pre (exact; the branch is
// uniform over the wavefront and taken only by such rows).
template <int ELEM, int RND>
__device__ __forceinline__ uint32_t chunk_finish(const NormArgs& A, uint8_t* codes_row,
                                                 uint64_t nrow, uint32_t d, float v[8],
                                                 uint32_t vmax_bits, const Normaliser& N) {
  float vmax = __uint_as_float(vmax_bits);
  if (N.pre != 1.0f) {
    vmax = vmax * N.pre;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = v[j] * N.pre;
  }
  const float inv = N.apply;
  const float amax = vmax * inv;
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
                                                 const float g[8], uint32_t mbits,
                                                 const Normaliser& N) {
  float v[8];
  const uint32_t vm = chunk_products<GM>(xb, g, mbits, v);
  return chunk_finish<ELEM, RND>(A, codes_row, nrow, d, v, vm, N);
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

  // Writes the gains to LDS and waits for the whole workgroup. Items past the
  // row end read zeros; the chunks they belong to are never encoded, so their
  // gains are never read.
  __device__ __forceinline__ void store(float4* g_lds) {
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
      const int i = (int)threadIdx.x + k * NT;
      if (i < NC * kWave) {
        float v[8];
        unpack8(r[k], v);
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
  // chunks 0 .. NC-2 are whole (NC = ceil(D / 512)); only the last can end
  // inside the row, and its lanes past the end are masked
  const bool last_in = (NC - 1) * kChunk + dl < A.D;
  uint32_t mb[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t m = absmax_bits8(raw[c]);
    mb[c] = quad_max_u32(c < NC - 1 ? m : (last_in ? m : 0u));
  }
  Normaliser N;
  if constexpr (STAT == S_RMS) {
    const float s = row_sumsq<NC>(NC, [&](int c, float t) {
      return (c < NC - 1 || last_in) ? sumsq8(raw[c], t) : t;
    });
    N = plain_normaliser(rms_inv(s, A.Df, A.eps));
  } else {
    auto mbf = [&](int c) { return mb[c]; };
    auto row_max = [&]() {
      uint32_t m = 0;
#pragma unroll
      for (int c = 0; c < NC; ++c) m = max(m, mb[c]);
      return max_over_quads(m);
    };
    N = row_normaliser([&](int shift) { return row_terms<NC>(NC, mbf, shift, A.pmode, A.p); },
                       row_max, A.pmode, A.p, A.Kf, A.Kinv);
  }
  if (lane == 0 && A.inv_out) A.inv_out[row] = N.inv;
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
    if (c < NC - 1 || last_in) {
      if (GM != G_NONE) gains(g_lds, c, lane, g);
      const uint32_t code = mxnorm_chunk<ELEM, RND, GM>(A, crow, nrow, d, raw[c], g, mb[c], N);
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
  for (int c = 0; c < NC - 1; ++c) raw[c] = load16_stream(xr + c * kChunk + dl);
  raw[NC - 1] = load_chunk(xr, NC - 1, dl, A.D);  // the only chunk that can pass the row end
  __builtin_amdgcn_sched_barrier(0);
  if (GAMMA) gs.store(g_lds);  // the row loads stay in flight meanwhile
  if (!live) return;
  uint32_t* sc = sc_lds[wave];
  if (!GAMMA)
    mxnorm_row_reg<NC, ELEM, RND, G_NONE, STAT>(A, raw, g_lds, row, lane, sc);
  else
    mxnorm_row_reg<NC, ELEM, RND, G_GAIN, STAT>(A, raw, g_lds, row, lane, sc);
}

// ------------------------------------------------------------------ split rows

constexpr int kSplitMaxWaves = 16;  // wavefronts per workgroup of the split-row kernel

// A row split over W wavefronts of one workgroup: wave w holds statistic group
// w, chunks [4w, 4w + 4) of the row, in VGPRs, with the gains of those chunks.
// When the row's chunk count is not a multiple of 4, the last wave's spare
// slots hold copies of the row's last chunk: they are left out of the
// statistic, and they encode to the same codes the real last chunk does (same
// data, gains, scale and random words), written to the same place again; so
// the loads and the encode need no chunk tests. The row's last chunk may end
// inside the row (D % 512 != 0): its lanes past the end count nothing and
// store nothing, as in the one-wave kernel.
// Each wave's group total meets the others in LDS and every wave adds all of
// them in group order, so the statistic has exactly the bits of the one-wave
// kernels. Every wave then encodes its own chunks: the work after the row's
// last byte arrives is spread over W wavefronts (and the CU's SIMDs) instead
// of one, and a wave needs 16 KB of loads in flight at most, so the kernel
// keeps the occupancy of the short rows at any D.
template <int ELEM, int RND, bool GAMMA, int STAT, bool RAGGED>
__global__ __launch_bounds__(kSplitMaxWaves * kWave) void mxnorm_split_kernel(NormArgs A, int nchunks) {
  constexpr int CPW = kGroupChunks;  // chunks per wave: one statistic group
  __shared__ __align__(16) float part[kSplitMaxWaves];
  __shared__ __align__(16) float part2[kSplitMaxWaves];
  __shared__ __align__(16) uint32_t pmax[kSplitMaxWaves];
  __shared__ uint32_t sc_lds[kSplitMaxWaves][CPW * 4];
  const int W = (nchunks + CPW - 1) / CPW;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // wave-uniform
  const int64_t row = blockIdx.x;
  const uint16_t* xr = A.x + row * A.ldx;
  const int dl = lane * 8;
  const int c0 = w * CPW;
  const int ncw = min(CPW, nchunks - c0);  // this wave's real chunks, >= 1
  // Chunk slot c of this wave is row chunk min(c0 + c, nchunks - 1); loads are
  // unconditional (a predicated load makes the compiler wait for the loads
  // before it). Only the row's last chunk can end inside the row; a lane's 8
  // elements lie wholly inside or past the end (D % 32 == 0), and a lane past
  // it re-reads the row's last 16 bytes and stores nothing.
  // (RAGGED: D % 512 != 0; otherwise every lane is inside and nothing is tested)
  auto chunk_of = [&](int c) { return min(c0 + c, nchunks - 1); };
  const bool last_in = !RAGGED || (nchunks - 1) * kChunk + dl < A.D;
  auto lane_in = [&](int c) { return !RAGGED || c0 + c < nchunks - 1 || last_in; };
  auto elem_of = [&](int c) {
    return RAGGED ? min(chunk_of(c) * kChunk + dl, A.D - 8) : chunk_of(c) * kChunk + dl;
  };

  uint4 graw[CPW];
  if (GAMMA) {
#pragma unroll
    for (int c = 0; c < CPW; ++c) graw[c] = load16(A.gamma + elem_of(c));
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the gain loads ahead of the row loads
  uint4 raw[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) raw[c] = load16_stream(xr + elem_of(c));
  __builtin_amdgcn_sched_barrier(0);

  uint32_t mb[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) mb[c] = quad_max_u32(lane_in(c) ? absmax_bits8(raw[c]) : 0u);
  auto mb_stat = [&](int c) { return c < ncw ? mb[c] : 0u; };  // spare slots add nothing
  auto wave_group = [&](float* dst, int shift) {  // this wave's group total -> dst[w]
    float t;
    if constexpr (STAT == S_RMS)
      t = group_sumsq<CPW>(0, CPW, [&](int c, float u) {
        return c < ncw && lane_in(c) ? sumsq8(raw[c], u) : u;
      });
    else
      t = group_terms<CPW>(0, CPW, mb_stat, shift, A.pmode, A.p);
    if (lane == 0) dst[w] = t;
  };
  if (STAT == S_RMS || A.pmode != P_INF) wave_group(part, 0);
  if (STAT == S_PMEAN) {
    uint32_t m = 0;
#pragma unroll
    for (int c = 0; c < CPW; ++c) m = max(m, mb[c]);  // copies of the last chunk change no maximum
    m = max_over_quads(m);
    if (lane == 0) pmax[w] = m;
  }
  __syncthreads();

  // 16-byte LDS reads; the group totals are added in group order
  auto row_total = [&](const float* src) {
    float t = 0.0f;
#pragma unroll
    for (int k4 = 0; k4 < kSplitMaxWaves; k4 += 4) {
      if (k4 >= W) break;
      const float4 q = *reinterpret_cast<const float4*>(src + k4);
      t = k4 == 0 ? q.x : t + q.x;
      if (k4 + 1 < W) t += q.y;
      if (k4 + 2 < W) t += q.z;
      if (k4 + 3 < W) t += q.w;
    }
    return t;
  };
  auto row_max = [&]() {
    uint32_t m = 0;
#pragma unroll
    for (int j4 = 0; j4 < kSplitMaxWaves; j4 += 4) {
      if (j4 >= W) break;
      const uint4 q = *reinterpret_cast<const uint4*>(pmax + j4);
      m = max(m, q.x);
      if (j4 + 1 < W) m = max(m, q.y);
      if (j4 + 2 < W) m = max(m, q.z);
      if (j4 + 3 < W) m = max(m, q.w);
    }
    return m;
  };
  Normaliser N;
  if constexpr (STAT == S_RMS) {
    N = plain_normaliser(rms_inv(row_total(part), A.Df, A.eps));
  } else {
    const bool pinf = A.pmode == P_INF;
    const float s = pinf ? 0.0f : row_total(part);
    const uint32_t rmax = row_max();
    const bool finite_nonzero = rmax != 0u && rmax < 0x7F80u;
    float s2 = 0.0f;
    // the rescaled totals: a workgroup-uniform decision, so every wave
    // reaches the barrier
    if (!pinf && finite_nonzero && !direct_total_suffices(s, A.pmode, A.p, A.Kf, A.Kinv)) {
      wave_group(part2, -bf16_exponent(rmax));
      __syncthreads();
      s2 = row_total(part2);
    }
    N = row_normaliser([&](int shift) { return shift == 0 ? s : s2; }, [&]() { return rmax; },
                       A.pmode, A.p, A.Kf, A.Kinv);
  }
  if (w == 0 && lane == 0 && A.inv_out) A.inv_out[row] = N.inv;
#pragma unroll
  for (int c = 0; c < CPW; ++c)  // widen each chunk where it is used (see mxnorm_row_reg)
    asm volatile("" : "+v"(raw[c].x), "+v"(raw[c].y), "+v"(raw[c].z), "+v"(raw[c].w));

  const uint64_t nrow = (uint64_t)row * (uint64_t)A.D;
  uint8_t* crow = code_row<ELEM>(A.codes, nrow);
  uint32_t* sc = sc_lds[w];
  float g[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    if (lane_in(c)) {  // a whole quad (one block) is in or out
      const int d = chunk_of(c) * kChunk + dl;
      uint32_t code;
      if (!GAMMA) {
        code = mxnorm_chunk<ELEM, RND, G_NONE>(A, crow, nrow, d, raw[c], g, mb[c], N);
      } else {
        unpack8(graw[c], g);
        code = mxnorm_chunk<ELEM, RND, G_GAIN>(A, crow, nrow, d, raw[c], g, 0u, N);
      }
      if ((lane & 3) == 0) put_scale(sc, c * 16 + (lane >> 2), code);  // spare slots: not flushed
    }
  }
  // this wave's blocks: 16 per real chunk, fewer in a last chunk that ends
  // inside the row
  flush_scales(sc, A.scales + (uint64_t)row * (uint64_t)A.K + (uint64_t)(c0 * 16),
               min(ncw * 16, A.K - c0 * 16), A.sc_vec != 0, lane);
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
      g_lds[i] = r;
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

  // lanes past the row end hold zeros (above), which add nothing
  auto mb = [&](int c) { return quad_max_u32(absmax_bits8(slice[c * kWave + lane])); };
  Normaliser N;
  if constexpr (STAT == S_RMS) {
    const float s = row_sumsq<0>(nchunks, [&](int c, float t) { return sumsq8(slice[c * kWave + lane], t); });
    N = plain_normaliser(rms_inv(s, A.Df, A.eps));
  } else {
    auto row_max = [&]() {
      uint32_t m = 0;
      for (int c = 0; c < nchunks; ++c) m = max(m, mb(c));
      return max_over_quads(m);
    };
    N = row_normaliser([&](int shift) { return row_terms<0>(nchunks, mb, shift, A.pmode, A.p); },
                       row_max, A.pmode, A.p, A.Kf, A.Kinv);
  }
  if (lane == 0 && A.inv_out) A.inv_out[row] = N.inv;

  const uint64_t nrow = (uint64_t)row * (uint64_t)A.D;
  uint8_t* crow = code_row<ELEM>(A.codes, nrow);
  float g[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int c = 0; c < nchunks; ++c) {
    const int d = c * kChunk + dl;
    if (d < A.D) {
      const uint4 xb = slice[c * kWave + lane];
      uint32_t code;
      if (!GAMMA) {
        code = mxnorm_chunk<ELEM, RND, G_NONE>(A, crow, nrow, d, xb, g, mb(c), N);
      } else {
        unpack8(g_lds[c * kWave + lane], g);
        code = mxnorm_chunk<ELEM, RND, G_GAIN>(A, crow, nrow, d, xb, g, 0u, N);
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


// y for one chunk; g holds the chunk's 8 gains when GAMMA.
template <bool GAMMA>
__device__ __forceinline__ void rms_chunk_out(const RmsArgs& A, int64_t row, int d, const uint4& xb,
                                              float inv, const float g[8]) {
  float v[8];
  unpack8(xb, v);
  if (GAMMA) {
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
// The workgroup's 4 rows share one LDS copy of gamma, staged as in
// mxnorm_reg_kernel (gain loads first, the row loads in flight across the
// staging barrier).
__global__ __launch_bounds__(kThreads) void rmsnorm_reg_kernel(RmsArgs A) {
  __shared__ float4 g_lds[GAMMA ? NC * kWave * 2 : 1];
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
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
  if (GAMMA) gs.store(g_lds);
  if (!live) return;
  const float s = row_sumsq<NC>(NC, [&](int c, float t) {
    return c * kChunk + dl < A.D ? sumsq8(raw[c], t) : t;
  });
  const float inv = rms_inv(s, A.Df, A.eps);
  if (lane == 0 && A.inv_out) A.inv_out[row] = inv;
  // widen each chunk again where it is used (see mxnorm_row_reg)
#pragma unroll
  for (int c = 0; c < NC; ++c)
    asm volatile("" : "+v"(raw[c].x), "+v"(raw[c].y), "+v"(raw[c].z), "+v"(raw[c].w));
  float g[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int d = c * kChunk + dl;
    if (d < A.D) {
      if (GAMMA) gains(g_lds, c, lane, g);
      rms_chunk_out<GAMMA>(A, row, d, raw[c], inv, g);
    }
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
  const float s = row_sumsq<0>(nchunks, [&](int c, float t) {
    return c * kChunk + dl < A.D ? sumsq8(load16(xr + c * kChunk + dl), t) : t;
  });
  const float inv = rms_inv(s, A.Df, A.eps);
  if (lane == 0 && A.inv_out) A.inv_out[row] = inv;
  float g[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int c = 0; c < nchunks; ++c) {
    const int d = c * kChunk + dl;
    if (d < A.D) {
      if (GAMMA) unpack8(load16(A.gamma + d), g);
      rms_chunk_out<GAMMA>(A, row, d, load16(xr + d), inv, g);
    }
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

// Split rows: 4 chunks per wavefront, one row per workgroup of up to 16
// wavefronts.
template <int ELEM, int RND, bool GAMMA, int STAT>
mxq_status launch_mxnorm_split(const NormArgs& A, int nc, hipStream_t s) {
  const int W = (nc + kGroupChunks - 1) / kGroupChunks;
  if (W > kSplitMaxWaves) return MXQ_ERR_UNSUPPORTED;
  if (A.T > kMaxGrid) return MXQ_ERR_UNSUPPORTED;
  if (A.D % kChunk != 0)
    hipLaunchKernelGGL((mxnorm_split_kernel<ELEM, RND, GAMMA, STAT, true>), dim3((unsigned)A.T),
                       dim3(kWave * W), 0, s, A, nc);
  else
    hipLaunchKernelGGL((mxnorm_split_kernel<ELEM, RND, GAMMA, STAT, false>), dim3((unsigned)A.T),
                       dim3(kWave * W), 0, s, A, nc);
  MXQ_LAUNCH_CHECK();
  return MXQ_OK;
}

enum Variant { V_REG = 0, V_LDS = 1, V_SPLIT = 2 };

template <int ELEM, int RND, int STAT>
mxq_status dispatch_mxnorm(const NormArgs& A, bool gamma, int variant, int nc, hipStream_t s) {
  if (variant == V_LDS)
    return gamma ? launch_mxnorm_lds<ELEM, RND, true, STAT>(A, nc, s)
                 : launch_mxnorm_lds<ELEM, RND, false, STAT>(A, nc, s);
  if (variant == V_SPLIT)
    return gamma ? launch_mxnorm_split<ELEM, RND, true, STAT>(A, nc, s)
                 : launch_mxnorm_split<ELEM, RND, false, STAT>(A, nc, s);
  return gamma ? dispatch_mxnorm_reg<ELEM, RND, true, STAT>(A, nc, s)
               : dispatch_mxnorm_reg<ELEM, RND, false, STAT>(A, nc, s);
}

template <int STAT>
mxq_status dispatch_norm_cast(const NormArgs& A, mxq_elem elem, mxq_round rnd, bool gamma,
                              int variant, int nc, hipStream_t s) {
  if (elem == MXQ_E4M3)
    return rnd == MXQ_SR ? dispatch_mxnorm<MXQ_E4M3, MXQ_SR, STAT>(A, gamma, variant, nc, s)
                         : dispatch_mxnorm<MXQ_E4M3, MXQ_RNE, STAT>(A, gamma, variant, nc, s);
  return rnd == MXQ_SR ? dispatch_mxnorm<MXQ_E2M1, MXQ_SR, STAT>(A, gamma, variant, nc, s)
                       : dispatch_mxnorm<MXQ_E2M1, MXQ_RNE, STAT>(A, gamma, variant, nc, s);
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
  constexpr uint32_t kForce = MXQ_FLAG_FORCE_REG | MXQ_FLAG_FORCE_LDS | MXQ_FLAG_FORCE_SPLIT;
  if (flags & ~(kForce | (uint32_t)MXQ_FLAG_SCALE_CEIL)) return MXQ_ERR_ARG;
  if (__builtin_popcount(flags & kForce) > 1) return MXQ_ERR_ARG;
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
  A.Kinv = ((D / 32) & (D / 32 - 1)) == 0 ? 1.0f / (float)(D / 32) : 0.0f;
  A.p = p;
  A.pmode = isinf(p) ? P_INF : (p == 1.0f ? P_ONE : (p == 2.0f ? P_TWO : P_GEN));
  A.Df = (float)D;
  A.eps = eps;
  A.sc_vec = (A.K % 4 == 0) && aligned(scales, 4);
  A.ceil_rule = (flags & MXQ_FLAG_SCALE_CEIL) != 0;
  A.rng = make_stream(rng);
  const int nc = (int)((D + kChunk - 1) / kChunk);
  // automatic: rows longer than 4096 elements split over several
  // wavefronts, shorter ones take one wavefront per row. At 4096 elements the
  // two measure the same within a few percent either way over 2048..32768
  // rows; from 8192 the split rows are faster (shorter per-wave work after
  // the row lands, fewer VGPRs). The LDS-staged variant only when forced.
  const int variant = (flags & MXQ_FLAG_FORCE_LDS)     ? V_LDS
                      : (flags & MXQ_FLAG_FORCE_REG)   ? V_REG
                      : (flags & MXQ_FLAG_FORCE_SPLIT) ? V_SPLIT
                      : nc > 2 * kGroupChunks          ? V_SPLIT
                                                       : V_REG;
  return dispatch_norm_cast<STAT>(A, elem, rnd, gamma != nullptr, variant, nc, (hipStream_t)stream);
}

// ------------------------------------------------------------------ NVFP4

// NVFP4 (a reading: the MXNorm page names the format in §3.2 without defining
// it): E2M1 elements packed as for MXFP4, blocks of 16 consecutive elements,
// one E4M3 scale byte per block, one fp32 tensor scale s_t from the caller.
// Per block with a = max |y|: scale byte = E4M3 RNE (saturating at 448) of
// RN32(a * k), k = RN32(1 / (6 s_t)); with Sd its value, element code = E2M1
// RNE (saturating) of RN32(y * r), r = RN32(1 / RN32(Sd * s_t)), or r = 0 when
// Sd == 0 (signed zeros); a block holding NaN or Inf gets scale 0x7F and codes
// 0x7. MXNorm over NVFP4 takes G from the same 16-element blocks (K = D / 16)
// and y = RN32(RN32(x * gamma) * inv) as for MX.
//
// One wavefront per row (D <= 8192), 4 rows per workgroup, the gains staged in
// LDS. A block is one lane pair (8 elements each), so its maximum is one DPP step; the statistic adds
// each lane's pair terms in chunk order, then the two pairs of a quad, then the
// quads as the MX kernels do.
struct Nvfp4Args {
  const uint16_t* x;
  const uint16_t* gamma;
  uint8_t* codes;
  uint8_t* scales;
  float* inv_out;
  int64_t ldx;
  int64_t T;
  int D;
  float Kf;
  float Kinv;  // 1/K when K is a power of two, else 0
  float p;
  int pmode;
  float k;     // RN32(1 / (6 s_t))
  float s_t;
};

template <int NC, bool NORM, bool GAMMA>
__global__ __launch_bounds__(kThreads) void nvfp4_kernel(Nvfp4Args A) {
  // r for every finite scale byte: RN32(1 / RN32(Sd * s_t)), 0 for Sd == 0,
  // computed once per workgroup (a correctly rounded division each); the
  // gains staged as fp32 in LDS, as in mxnorm_reg_kernel
  __shared__ float rtab[128];
  __shared__ float4 g_lds[GAMMA ? NC * kWave * 2 : 1];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
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
  if (threadIdx.x < 128) {
    const float Sd = __builtin_amdgcn_cvt_f32_fp8((int)threadIdx.x, 0);
    rtab[threadIdx.x] = (threadIdx.x == 0 || threadIdx.x == 0x7F) ? 0.0f : 1.0f / (Sd * A.s_t);
  }
  if (GAMMA)
    gs.store(g_lds);  // includes the workgroup barrier
  else
    __syncthreads();
  if (!live) return;  // no barriers below
  // only the last chunk can end inside the row; its lanes past the end
  // re-read the row's last 16 bytes and are left out of statistic and stores
  auto in_row = [&](int c) { return c < NC - 1 || c * kChunk + dl < A.D; };

  Normaliser N = plain_normaliser(1.0f);
  if constexpr (NORM) {
    uint32_t mb[NC];  // the lane pair's block maximum of |x| as bf16 bits
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint32_t m = in_row(c) ? absmax_bits8(raw[c]) : 0u;
      mb[c] = max(m, dpp<kDppQuadSwap1>(m));
    }
    auto total = [&](int shift) {
      float t;
      auto blk = [&](int c) { return mb[c]; };
      if (A.pmode == P_TWO)
        t = lane_terms_p<NC, P_TWO>(0, NC, blk, shift, A.p);
      else if (A.pmode == P_ONE)
        t = lane_terms_p<NC, P_ONE>(0, NC, blk, shift, A.p);
      else
        t = lane_terms_p<NC, P_GEN>(0, NC, blk, shift, A.p);
      // both lanes of a pair hold the pair's terms: the quad's two pairs, then the quads
      const uint32_t u = __float_as_uint(t);
      return sum_over_quads(__uint_as_float(f32_add_bits(u, dpp<kDppQuadSwap2>(u))));
    };
    auto row_max = [&]() {
      uint32_t m = 0;
#pragma unroll
      for (int c = 0; c < NC; ++c) m = max(m, mb[c]);
      return max_over_quads(max(m, dpp<kDppQuadSwap2>(m)));
    };
    N = row_normaliser(total, row_max, A.pmode, A.p, A.Kf, A.Kinv);
    if (lane == 0 && A.inv_out) A.inv_out[row] = N.inv;
  }

  const uint64_t crow = (uint64_t)row * (uint64_t)(A.D / 2);
  const uint64_t srow = (uint64_t)row * (uint64_t)(A.D / 16);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float v[8];
    unpack8(raw[c], v);
    if (GAMMA) {
      float g[8];
      gains(g_lds, c, lane, g);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] *= g[j];  // exact: two bf16 values
    }
    // the block's maximum of |v| (NaN-propagating), then of |y| by monotone rounding
    float am = __builtin_fabsf(v[0]);
#pragma unroll
    for (int j = 1; j < 8; ++j) am = __builtin_elementwise_maximum(am, __builtin_fabsf(v[j]));
    am = __builtin_elementwise_maximum(am, __uint_as_float(dpp<kDppQuadSwap1>(__float_as_uint(am))));
    float y[8];
    float a;
    if constexpr (NORM) {
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = (v[j] * N.pre) * N.apply;
      a = (am * N.pre) * N.apply;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = v[j];
      a = am;
    }
    const bool bad = !(a <= 0x1.fffffep127f);  // NaN or Inf in the block
    // scale byte: E4M3 RNE of min(RN32(a k), 448) (the convert does not saturate)
    const float q = __builtin_fminf(a * A.k, 448.0f);
    short2_t sp = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(short2_t{0, 0}, q, q, 1.0f, false);
    uint32_t sc = (uint32_t)__builtin_bit_cast(uint32_t, sp) & 0x7Fu;  // q >= 0 (or NaN: bad)
    const float r = rtab[sc];
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] *= r;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
    if (bad) {
      w = 0x77777777u;
      sc = 0x7Fu;
    }
    if (in_row(c)) {
      const int d = c * kChunk + dl;
      store4_stream(A.codes + crow + (uint64_t)(d >> 1), w);
      if ((lane & 1) == 0) A.scales[srow + (uint64_t)(d >> 4)] = (uint8_t)sc;
    }
  }
}

template <bool NORM, bool GAMMA>
mxq_status dispatch_nvfp4(const Nvfp4Args& A, int nc, hipStream_t s) {
  const unsigned grid = (unsigned)((A.T + kRowsPerBlock - 1) / kRowsPerBlock);
  switch (nc) {
#define MXQ_CASE(N)                                                                     \
  case N:                                                                               \
    hipLaunchKernelGGL((nvfp4_kernel<N, NORM, GAMMA>), dim3(grid), dim3(kThreads), 0, s, A); \
    break;
    MXQ_CASE(1) MXQ_CASE(2) MXQ_CASE(3) MXQ_CASE(4) MXQ_CASE(5) MXQ_CASE(6) MXQ_CASE(7)
    MXQ_CASE(8) MXQ_CASE(9) MXQ_CASE(10) MXQ_CASE(11) MXQ_CASE(12) MXQ_CASE(13) MXQ_CASE(14)
    MXQ_CASE(15) MXQ_CASE(16)
#undef MXQ_CASE
    default:
      return MXQ_ERR_UNSUPPORTED;
  }
  MXQ_LAUNCH_CHECK();
  return MXQ_OK;
}

// Validation and launch shared by the two NVFP4 entry points.
mxq_status nvfp4_run(const uint16_t* x, int64_t ldx, const uint16_t* gamma, int64_t T, int64_t D,
                     bool norm, float p, float tensor_scale, uint8_t* codes, uint8_t* scales,
                     float* inv_out, void* stream) {
  if (T < 0 || D <= 0 || D % 32 != 0 || ldx < D) return MXQ_ERR_SHAPE;
  if (!(tensor_scale >= 0x1p-32f && tensor_scale <= 0x1p32f)) return MXQ_ERR_ARG;  // also NaN
  if (norm && !(p > 0.0f)) return MXQ_ERR_ARG;
  if (D > MXQ_MAX_D_REG) return MXQ_ERR_UNSUPPORTED;
  if (T == 0) return MXQ_OK;
  if (x == nullptr || codes == nullptr || scales == nullptr) return MXQ_ERR_NULL;
  if (!aligned(x, 16) || ldx % 8 != 0 || !aligned(codes, 16)) return MXQ_ERR_ALIGN;
  if (gamma != nullptr && !aligned(gamma, 16)) return MXQ_ERR_ALIGN;
  if (inv_out != nullptr && !aligned(inv_out, 4)) return MXQ_ERR_ALIGN;
  if ((uint64_t)T * (uint64_t)D >= (1ull << 40)) return MXQ_ERR_UNSUPPORTED;
  if ((T + kRowsPerBlock - 1) / kRowsPerBlock > kMaxGrid) return MXQ_ERR_UNSUPPORTED;
  Nvfp4Args A;
  A.x = x;
  A.gamma = gamma;
  A.codes = codes;
  A.scales = scales;
  A.inv_out = inv_out;
  A.ldx = ldx;
  A.T = T;
  A.D = (int)D;
  const int64_t K = D / 16;
  A.Kf = (float)K;
  A.Kinv = (K & (K - 1)) == 0 ? 1.0f / (float)K : 0.0f;
  A.p = p;
  A.pmode = isinf(p) ? P_INF : (p == 1.0f ? P_ONE : (p == 2.0f ? P_TWO : P_GEN));
  A.k = (float)(1.0 / (6.0 * (double)tensor_scale));
  A.s_t = tensor_scale;
  const int nc = (int)((D + kChunk - 1) / kChunk);
  hipStream_t s = (hipStream_t)stream;
  if (!norm) return dispatch_nvfp4<false, false>(A, nc, s);
  return gamma ? dispatch_nvfp4<true, true>(A, nc, s) : dispatch_nvfp4<true, false>(A, nc, s);
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

mxq_status nvfp4_cast_fwd(const uint16_t* x, int64_t ldx, int64_t T, int64_t D,
                          float tensor_scale, uint8_t* codes, uint8_t* scales, void* stream) {
  return nvfp4_run(x, ldx, nullptr, T, D, false, 2.0f, tensor_scale, codes, scales, nullptr,
                   stream);
}

mxq_status mxnorm_nvfp4_fwd(const uint16_t* x, int64_t ldx, const uint16_t* gamma, int64_t T,
                            int64_t D, float p, float tensor_scale, uint8_t* codes,
                            uint8_t* scales, float* inv_norm, void* stream) {
  return nvfp4_run(x, ldx, gamma, T, D, true, p, tensor_scale, codes, scales, inv_norm, stream);
}

}  // extern "C"
