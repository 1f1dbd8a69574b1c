// mx_gemm.hip - the MX GEMM that consumes MXNorm's output on MI355X (gfx950).
//
// C[m][n] = sum_k A[m][k] * B[n][k] over MX operands: A is the activation's
// E4M3 codes [M, K] with E8M0 scales [M, K/32] (MXNorm's output, page "MXNorm:
// Reusing MXFP block scales for efficient tensor normalisation", §2.1), B the
// next linear layer's weight [N, K], gain folded and MX-cast along K (§2.3,
// MXNormLinear). The products run on the gfx950 block-scaled matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4), which apply both operands' E8M0 scales
// and accumulate in fp32. (With register operands it and its 16 x 16 x 128
// sibling both issue at about 4.5 PFLOP/s with 8-bit operands; the 32 x 32 x
// 64 form needs a quarter of the accumulators and half the instructions and
// scale operands for a 128 x 64 wave tile.)
//
// Either operand may be E2M1 (FP4, packed two to a byte, element 2j in the
// low nibble): the same instruction with format code 4 runs FP4 operands at
// nearly twice its 8-bit rate.
//
// Operand layout of that instruction for 8-bit data (probed on the device):
// lane l carries row l % 32 of its 32 x 64 operand; its 32 bytes are K
// [16 g, 16 g + 16) then [32 + 16 g, 32 + 16 g + 16), g = l / 32; the scale
// of K block b (32 columns) of row r is the byte of lane r + 32 b's scale
// register that the instruction's op_sel value (0-3) names; the other bytes
// are ignored. Result element v of lane l is
// row 8 (v / 4) + 4 (l / 32) + v % 4 (of the first operand) and column l % 32
// (of the second). Here the instruction takes B as its first operand and A
// as its second, so each lane's 16 results are C row l % 32 at 4 groups of 4
// consecutive columns. For FP4 data (probed too) lane l carries K
// [32 g, 32 g + 32) of row l % 32 as 32 nibbles in its first 16 bytes, even K
// in the low nibble: exactly 16 consecutive bytes of a packed E2M1 row.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "mxq.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWave = 64;
// 8 waves, 2 x 4 over the tile, 128 x 64 each: two waves per SIMD, so one
// wave's MFMAs run while the other waits on its LDS reads. (Four waves of
// 128 x 128, one per SIMD with all 256 accumulation registers, left the
// matrix pipe idle at every such wait: 8-9% slower on MXFP8, 3-4% on MXFP4.)
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = 256;        // tile rows (A)
constexpr int kBN = 256;        // tile columns (B rows)
constexpr int kBK = 128;        // K per step: 4 MX blocks, two MFMAs deep (FP4 x FP4: 256, see below)
constexpr int kChunks = kBK / 16;   // 16-byte chunks per row and step (8-bit codes)

// MFMA format codes of the element types, and the 16-byte chunks a row of
// that type holds per K step (8 for E4M3, 4 for packed E2M1).
constexpr int kFmtE4M3 = 0, kFmtE2M1 = 4;
template <int F> constexpr int chunks_of() { return F == kFmtE2M1 ? 4 : 8; }

// Chunk c of row r sits at position c ^ swz(r). gfx950's LDS serves a
// 16-byte read 16 lanes at a time over 64 banks (256 bytes), so the 16
// consecutive rows such a group reads must land on 16 distinct 16-byte bank
// slots: rows of 128 bytes fill 2 rows per 256 bytes, and (r >> 1) & 7 sets
// rows of equal parity apart; rows of 64 bytes fill 4, and (r >> 2) & 3 sets
// rows of equal r % 4 apart. (The r & 7 pattern, conflict-free on a 32-bank
// LDS, measures 4 conflict cycles per read here.)
template <int CH> __device__ __forceinline__ int swz(int r) {
  return CH == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}

struct GemmArgs {
  const uint8_t* a;
  const uint8_t* sa;
  const uint8_t* b;
  const uint8_t* sb;
  void* c;
  int64_t lda, ldsa, ldb, ldsb, ldc;  // code bytes, scale bytes, C elements per row
  int M, N, K;
  int tiles_m, tiles_n;
  int vec;    // C rows allow 4-element vector stores (aligned base, ldc % 4 == 0)
  int vec16;  // bf16 C rows allow 16-byte stores (16-byte aligned base, ldc % 8 == 0)
};

// One K step of both operands in LDS. Code rows hold 8 (E4M3) or 4 (E2M1)
// chunks of 16 bytes, swizzled as swz above.
// sa / sb serve the loop that loads scales step by step (the grouped loop
// reads ScaleGroup below): the step's scale words (its 4 E8M0 bytes of a
// row), stored in the order the MFMA lanes consume them: position
// h * 128 + rl * 4 + blk holds row h * 128 + blk * 32 + rl, so a lane's 4
// words are contiguous.
struct Stage {
  uint4 a[kBM * kChunks];
  uint4 b[kBN * kChunks];
  uint32_t sa[kBM];
  uint32_t sb[kBN];
};
// the bf16 epilogue stages 8 KB per wave across a stage's a and b arrays
static_assert(offsetof(Stage, b) == sizeof(uint4) * kBM * kChunks &&
                  sizeof(uint4) * (kBM + kBN) * kChunks >= kWaves * 8192,
              "a stage's code arrays hold the epilogue's slots");

__device__ __forceinline__ int scale_row(int p) {
  return (p >> 7) * 128 + (p & 3) * 32 + ((p >> 2) & 31);
}

// The scales of kScaleSteps consecutive 128-deep K steps: 16 E8M0 bytes of
// each row, moved by one 16-byte DMA per row (entry r holds tile row r; word
// s of it is step s's 4 blocks; a 256-deep FP4 step takes words 2 s and
// 2 s + 1, so a group holds two of those). One request per row brings four
// steps' scales, where loading them step by step costs a whole L2 request for
// 4 bytes.
constexpr int kScaleSteps = 4;
struct ScaleGroup {
  uint4 a[kBM];
  uint4 b[kBN];
};

// Pieces to spread one step's code DMA over (the first sub-step's 4 blocks of
// MFMAs, one 32-row A block each), so that the wave does not stall issuing it
// all at once.
constexpr int kSpread = 4;

// Direct-to-LDS loads of one operand's K step, CH chunks per row: a wave
// instruction moves 64 x 16 bytes = 64 / CH rows; lane i lands at position
// i, i.e. row i / CH, physical chunk i % CH, so it fetches logical chunk
// (i % CH) ^ swz(row). Each of the 8 waves moves CH / 2 such instructions
// (256 rows in all). Rows past the matrix end re-read its last row (their
// results are never stored).
template <int CH>
__device__ __forceinline__ void load_one(const uint8_t* base, int64_t ld, int rows_valid,
                                         uint4* dst, int r0, int ks, int wave, int lane, int q) {
  constexpr int kRows = kWave / CH;
  const int blk = wave * (CH / 2) + q;
  const int r = blk * kRows + lane / CH;
  const int c = (lane % CH) ^ swz<CH>(r);
  __builtin_amdgcn_global_load_lds(
      (const void*)(base + (int64_t)min(r0 + r, rows_valid - 1) * ld + ks * (16 * CH) + c * 16),
      (lds_void*)&dst[blk * kWave], 16, 0, 0);
}

template <int CH>
__device__ __forceinline__ void load_operand(const uint8_t* base, int64_t ld, int rows_valid,
                                             uint4* dst, int r0, int ks, int wave, int lane) {
#pragma unroll
  for (int q = 0; q < CH / 2; ++q) load_one<CH>(base, ld, rows_valid, dst, r0, ks, wave, lane, q);
}

// Piece `piece` (of kSpread) of a step's code DMA: its share of the A then
// B instructions.
template <int CHA, int CHB>
__device__ __forceinline__ void load_codes_piece(const GemmArgs& G, Stage* S, int m0, int n0,
                                                 int ks, int wave, int lane, int piece) {
  constexpr int CA = CHA / 2, CB = CHB / 2;
#pragma unroll
  for (int t = 0; t < CA + CB; ++t) {
    if (t * kSpread / (CA + CB) != piece) continue;
    if (t < CA)
      load_one<2 * CA>(G.a, G.lda, G.M, S->a, m0, ks, wave, lane, t);
    else
      load_one<2 * CB>(G.b, G.ldb, G.N, S->b, n0, ks, wave, lane, t - CA);
  }
}

// Scale group gk (K steps kScaleSteps gk ...) of the tile's rows: lane i of
// wave w < 4 moves A row w * 64 + i's 16 bytes, of wave w >= 4 B row
// (w - 4) * 64 + i's. Needs 16-byte aligned scale rows with at least
// 16 (gk + 1) bytes.
__device__ __forceinline__ void load_scale_group(const GemmArgs& G, ScaleGroup* SG, int m0, int n0,
                                                 int gk, int wave, int lane) {
  if (wave < 4) {
    const int r = wave * kWave + lane;
    __builtin_amdgcn_global_load_lds((const void*)(G.sa + (int64_t)min(m0 + r, G.M - 1) * G.ldsa + gk * 16),
                                     (lds_void*)&SG->a[wave * kWave], 16, 0, 0);
  } else {
    const int r = (wave - 4) * kWave + lane;
    __builtin_amdgcn_global_load_lds((const void*)(G.sb + (int64_t)min(n0 + r, G.N - 1) * G.ldsb + gk * 16),
                                     (lds_void*)&SG->b[(wave - 4) * kWave], 16, 0, 0);
  }
}

// A whole step's codes and, step by step (GROUPED false), its scales: 4
// bytes (the step's 4 blocks) per row; lane i of wave w fills position
// (w % 4) * 64 + i of A's scales (w < 4) or B's (w >= 4).
template <int FA, int FB, bool GROUPED, bool WIDE = false>
__device__ __forceinline__ void load_stage(const GemmArgs& G, Stage* S, int m0, int n0, int ks,
                                           int wave, int lane) {
  load_operand<WIDE ? 8 : chunks_of<FA>()>(G.a, G.lda, G.M, S->a, m0, ks, wave, lane);
  load_operand<WIDE ? 8 : chunks_of<FB>()>(G.b, G.ldb, G.N, S->b, n0, ks, wave, lane);
  if (GROUPED) return;
  const int w4 = wave & 3;
  const int rs = scale_row(w4 * kWave + lane);
  if (wave < 4)
    __builtin_amdgcn_global_load_lds((const void*)(G.sa + (int64_t)min(m0 + rs, G.M - 1) * G.ldsa + ks * 4),
                                     (lds_void*)&S->sa[w4 * kWave], 4, 0, 0);
  else
    __builtin_amdgcn_global_load_lds((const void*)(G.sb + (int64_t)min(n0 + rs, G.N - 1) * G.ldsb + ks * 4),
                                     (lds_void*)&S->sb[w4 * kWave], 4, 0, 0);
}

// The MFMA operand of lane (row r, half g) for the 64-deep sub-step kk of
// the step. 8-bit rows: chunks 4 kk + g and 4 kk + 2 + g (32 bytes). Packed
// FP4 rows (CH chunks per step: 4, or 8 for a 256-deep step): chunk 2 kk + g
// (16 bytes; the upper half of the register block is unused).
template <int F, int CH>
__device__ __forceinline__ v8i operand(const uint4* rows, int r, int kk, int g) {
  if (F != kFmtE2M1) {
    const uint4 lo = rows[r * CH + ((4 * kk + g) ^ swz<CH>(r))];
    const uint4 hi = rows[r * CH + ((4 * kk + 2 + g) ^ swz<CH>(r))];
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  const uint4 lo = rows[r * CH + ((2 * kk + g) ^ swz<CH>(r))];
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
}

// The scale words of the lane's 4 operand rows h * 128 + blk * 32 + rl
// (blk = 0..3).
__device__ __forceinline__ uint4 scale_words(const uint32_t* sc, int h, int rl) {
  return *reinterpret_cast<const uint4*>(sc + h * 128 + rl * 4);
}

// The scaled MFMA takes each operand's E8M0 scale from one byte of a 32-bit
// register, the byte chosen by the instruction's op_sel field (an immediate,
// the same for every lane). A scale word holds a row's 4 blocks of one
// 128-deep K step, block b in byte b; the lanes of half g = 0 need blocks 0
// and 2 (sub-steps 0 and 1), those of half g = 1 blocks 1 and 3. Shifting a
// half-1 lane's word right by one byte puts its blocks in bytes 0 and 2 as
// well, so one shift per word and step replaces a byte extraction per MFMA,
// and sub-step kk selects byte 2 (kk & 1).
template <int FB, int FA, int SEL>
__device__ __forceinline__ v16f mfma_scaled(v8i b, v8i a, v16f c, uint32_t sb, uint32_t sa) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, FB, FA, SEL, (int)sb, SEL,
                                                          (int)sa);
}

// One K step of the wave's 128 x 64 eighth: the next step's DMA into
// `fill`, then this step's operands from `use` into the MFMAs, in sub-steps
// of 64 (the MX blocks 2 kk and 2 kk + 1 of the step): two for a 128-deep
// step, four for the 256-deep steps of FP4 x FP4 (WIDE), whose scales take
// two words per row and step. Per sub-step, the 2 B operands are read first
// and the A operand one 32-row block ahead of the 2 MFMAs that use it, so the
// reads overlap the MFMAs. That `use` has landed is the caller's wait and
// barrier.
//
// GROUPED: `fill` and `use` are two distinct LDS objects known at compile
// time, so the compiler's alias analysis tells the DMA's writes from these
// reads and the reads overlap the DMA in flight; the code DMA is spread over
// the first K half's 4 blocks of MFMAs. The step's scales are word `sstep`
// of the scale group `sg`; when `sg_fill` is set, the next group (group sgk
// of the tile at sm0, sn0) goes out right after those reads.
// Otherwise (stages chosen at run time) the whole DMA, scales included, goes
// out first and the compiler waits for it before the first LDS read.
template <int FA, int FB, bool GROUPED, bool WIDE>
__device__ __forceinline__ void k_step(const GemmArgs& G, Stage* fill, const Stage* use, int fm0,
                                       int fn0, int fks, int wave, int lane, int wm, int wn,
                                       v16f (&acc)[4][2], const ScaleGroup* sg, int sstep,
                                       ScaleGroup* sg_fill, int sm0, int sn0, int sgk) {
  constexpr int CA = WIDE ? 8 : chunks_of<FA>(), CB = WIDE ? 8 : chunks_of<FB>();
  constexpr int KK = WIDE ? 4 : 2;  // 64-deep sub-steps
  if (!GROUPED) {
    load_stage<FA, FB, false>(G, fill, fm0, fn0, fks, wave, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
  const int g = lane >> 5, rl = lane & 31;
  // WIDE: 8 scale bytes per row and step, words 2 sstep and 2 sstep + 1
  uint32_t sbw4[4], saw4[4], sbw4h[4], saw4h[4];
  if (GROUPED) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t* wb = reinterpret_cast<const uint32_t*>(&sg->b[wn * 64 + (j & 1) * 32 + rl]);
      const uint32_t* wa = reinterpret_cast<const uint32_t*>(&sg->a[wm * 128 + j * 32 + rl]);
      if (WIDE) {
        if (j < 2) sbw4[j] = wb[2 * sstep], sbw4h[j] = wb[2 * sstep + 1];
        saw4[j] = wa[2 * sstep], saw4h[j] = wa[2 * sstep + 1];
      } else {
        if (j < 2) sbw4[j] = wb[sstep];
        saw4[j] = wa[sstep];
      }
    }
    if (sg_fill) load_scale_group(G, sg_fill, sm0, sn0, sgk, wave, lane);
  } else {
    const uint2 sbw = *reinterpret_cast<const uint2*>(use->sb + (wn >> 1) * 128 + rl * 4 + (wn & 1) * 2);
    const uint4 saw = scale_words(use->sa, wm, rl);
    sbw4[0] = sbw.x, sbw4[1] = sbw.y, sbw4[2] = 0, sbw4[3] = 0;
    saw4[0] = saw.x, saw4[1] = saw.y, saw4[2] = saw.z, saw4[3] = saw.w;
  }
  const uint32_t shift = 8u * (uint32_t)g;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j < 2) sbw4[j] >>= shift;
    saw4[j] >>= shift;
    if (WIDE) {
      if (j < 2) sbw4h[j] >>= shift;
      saw4h[j] >>= shift;
    }
  }
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    // the sub-step's MX block of the lane's half: byte 2 (kk & 1) of its shifted word
    v8i bo[2];
    uint32_t sbv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bo[j] = operand<FB, CB>(use->b, wn * 64 + j * 32 + rl, kk, g);
      sbv[j] = kk < 2 ? sbw4[j] : sbw4h[j];
    }
    v8i ao = operand<FA, CA>(use->a, wm * 128 + rl, kk, g);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v8i ao_next;
      if (i + 1 < 4) ao_next = operand<FA, CA>(use->a, wm * 128 + (i + 1) * 32 + rl, kk, g);
      if (GROUPED && kk == 0) load_codes_piece<CA, CB>(G, fill, fm0, fn0, fks, wave, lane, i);
      const uint32_t sav = kk < 2 ? saw4[i] : saw4h[i];
      // B is the first operand, so each lane's results are consecutive columns of C
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = (kk & 1) ? mfma_scaled<FB, FA, 2>(bo[j], ao, acc[i][j], sbv[j], sav)
                             : mfma_scaled<FB, FA, 0>(bo[j], ao, acc[i][j], sbv[j], sav);
      if (i + 1 < 4) ao = ao_next;
      // keep the next block's reads ahead of this block's MFMAs (the
      // scheduler would otherwise sink them to their use and wait on each)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The start of a step: this wave's DMA has landed and its LDS reads of the
// previous step are complete (s_waitcnt vmcnt(0) lgkmcnt(0): encoding 0x0070,
// expcnt left at its maximum), then a barrier. After it every wave's share of
// this step is visible, and no wave still reads the stage this step's DMA
// refills. The wait is the intrinsic, not inline assembly, so the compiler's
// own wait insertion knows the DMA is complete. The barrier carries no memory
// fence (__syncthreads() would also wait for loads the compiler still thinks
// in flight).
__device__ __forceinline__ void step_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0070);
  __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Four consecutive elements of C at element offset off: one 8-byte (bf16) or
// 16-byte (fp32) store. Ordinary (write-back) stores: L2 merges the partial
// lines of a tile's rows before they go to memory.
template <bool OUT_BF16>
__device__ __forceinline__ void store4(void* c, int64_t off, const v4f& v) {
  if (OUT_BF16) {
    const u32x2 w = {(uint32_t)bf16_rne(v[0]) | ((uint32_t)bf16_rne(v[1]) << 16),
                     (uint32_t)bf16_rne(v[2]) | ((uint32_t)bf16_rne(v[3]) << 16)};
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(c) + off) = w;
  } else {
    *reinterpret_cast<v4f*>(static_cast<float*>(c) + off) = v;
  }
}

// Epilogue of a tile. acc[i][j] element 4 q + t holds C[row i*32 + rl]
// [column j*32 + 8 q + 4 g + t] (rl = lane % 32, g = lane / 32): each lane
// stores 4 groups of 4 consecutive elements, each as one 8-byte (bf16) or
// 16-byte (fp32) store. A tile wholly inside C (a wave-uniform test) takes
// straight-line stores; an edge tile checks each element. The accumulators
// are cleared for the next tile.
template <bool OUT_BF16>
__device__ __forceinline__ void store_tile(const GemmArgs& G, int m0, int n0, int wm, int wn,
                                           int lane, v16f (&acc)[4][2]) {
  const int g = lane >> 5, rl = lane & 31;
  if (G.vec && m0 + kBM <= G.M && n0 + kBN <= G.N) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = m0 + wm * 128 + i * 32 + rl;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v16f& a = acc[i][j];
          store4<OUT_BF16>(G.c, row * G.ldc + n0 + wn * 64 + j * 32 + 8 * q + 4 * g,
                           v4f{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]});
        }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + wm * 128 + i * 32 + rl;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + wn * 64 + j * 32 + 8 * q + 4 * g;
          const v16f& a = acc[i][j];
          const v4f v = v4f{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
          if (G.vec && row < G.M && col + 3 < G.N) {
            store4<OUT_BF16>(G.c, (int64_t)row * G.ldc + col, v);
          } else if (row < G.M) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (col + e < G.N) {
                if (OUT_BF16)
                  static_cast<uint16_t*>(G.c)[(int64_t)row * G.ldc + col + e] = bf16_rne(v[e]);
                else
                  static_cast<float*>(G.c)[(int64_t)row * G.ldc + col + e] = v[e];
              }
            }
          }
        }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};
}

// Epilogue of a whole bf16 tile through LDS. Stored straight from the
// accumulators, each store instruction writes 8 bytes to each of 32 rows, so
// every 128-byte line of C is assembled from 8 partial writes. Instead each
// wave writes its 128 x 64 eighth, 64 rows at a time, into its own 8 KB slot
// of a stage no wave reads any more (128 bytes per row; 16-byte group c of
// slot row r at c ^ (r & 7), which spreads rows of equal parity over the
// banks), then reads it back 16 contiguous bytes per lane and stores whole
// lines: 8 rows of 128 bytes per instruction, non-temporal (C is written
// once; streaming it keeps the operand panels in L2). A wave reads back only
// what it wrote, and its LDS accesses complete in order.
__device__ __forceinline__ void store_tile_bf16_lds(const GemmArgs& G, int m0, int n0, int wm,
                                                    int wn, int wave, int lane, v16f (&acc)[4][2],
                                                    uint4* stage) {
  uint8_t* slot = reinterpret_cast<uint8_t*>(stage) + wave * 8192;
  const int g = lane >> 5, rl = lane & 31;
  uint16_t* C = static_cast<uint16_t*>(G.c);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int r = ii * 32 + rl;  // slot row; wave-tile row 64 h + r
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v16f& a = acc[2 * h + ii][j];
          const u32x2 w = {(uint32_t)bf16_rne(a[4 * q]) | ((uint32_t)bf16_rne(a[4 * q + 1]) << 16),
                           (uint32_t)bf16_rne(a[4 * q + 2]) | ((uint32_t)bf16_rne(a[4 * q + 3]) << 16)};
          *reinterpret_cast<u32x2*>(slot + r * 128 + (((4 * j + q) ^ (r & 7)) << 4) + g * 8) = w;
        }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = 8 * k + (lane >> 3), c16 = lane & 7;
      const uint4 v = *reinterpret_cast<const uint4*>(slot + r * 128 + ((c16 ^ (r & 7)) << 4));
      const int64_t row = m0 + wm * 128 + h * 64 + r;
      __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w},
                                  reinterpret_cast<u32x4*>(C + row * G.ldc + n0 + wn * 64 + c16 * 8));
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};
}

// Tile order: the 8 XCDs take workgroup ids round robin, so tile t is first
// mapped to slot (t % 8) * (n / 8) + t / 8, giving each XCD (and its L2) a
// contiguous run of the sequence (tiles b + j G stay on b's XCD); the
// sequence walks groups of 4 tile rows column by column, so neighbours share
// A rows or B rows.
__device__ __forceinline__ void tile_origin(const GemmArgs& G, int t, int& m0, int& n0) {
  const int nb = G.tiles_m * G.tiles_n;
  int pid = t;
  if (nb % 8 == 0) pid = (pid % 8) * (nb / 8) + pid / 8;
  constexpr int kGroup = 4;
  const int group = pid / (kGroup * G.tiles_n);
  const int first = group * kGroup;
  const int gsz = min(G.tiles_m - first, kGroup);
  const int in_group = pid % (kGroup * G.tiles_n);
  m0 = (first + in_group % gsz) * kBM;
  n0 = (in_group / gsz) * kBN;
}

// Persistent kernel: workgroup b takes tiles b, b + G, b + 2G, ... (G = grid
// size, a multiple of 8), as one sequence of (tile, K step) pairs, so the
// next tile's first DMA streams during this tile's last step. Two LDS
// stages. Each step waits for its own DMA (the only loads in flight); a
// barrier then makes every wave's share visible and orders the refill of the
// other stage after every wave's reads of it in the previous step. The step
// issues the next step's DMA, then computes.
//
// GROUPED (K a multiple of kScaleSteps steps, 16-byte aligned scale rows):
// the loop body is two steps, the first reading S0 and filling S1, the
// second the reverse, so both stages are named at compile time and the LDS
// reads overlap the DMA in flight. The scales come in groups of kScaleSteps
// steps, double-buffered in SG0 / SG1 (group number, counted across tiles,
// even: SG0): a group's first step issues the next group's DMA into the
// other buffer, whose last reads (the previous group's) the step's barrier
// has ordered before it, and the next step's wait and barrier see it landed.
// Otherwise the stage alternates at run time, scales come step by step, and
// each step's reads wait for the DMA it issued (correct, slower).
template <bool OUT_BF16, bool GROUPED, int FA, int FB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mx_gemm_kernel(GemmArgs G) {
  __shared__ Stage S0, S1;
  __shared__ ScaleGroup SG0, SG1;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = wave >> 2, wn = wave & 3;   // wave's 128 x 64 eighth of the tile
  const int nb = G.tiles_m * G.tiles_n;
  // FP4 x FP4 on the grouped loop takes 256-deep steps (128 bytes of each
  // row, as an 8-bit step), half as many steps and barriers per tile: 8%
  // faster than 128-deep steps on the MXFP4 projections (same box)
  constexpr bool WIDE = GROUPED && FA == kFmtE2M1 && FB == kFmtE2M1;
  constexpr int SGS = WIDE ? 2 : kScaleSteps;  // steps per scale group
  const int nk = G.K / (WIDE ? 2 * kBK : kBK);
  const int my_tiles = (nb - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  if (my_tiles <= 0) return;

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

  int m0, n0;
  tile_origin(G, blockIdx.x, m0, n0);
  load_stage<FA, FB, GROUPED, WIDE>(G, &S0, m0, n0, 0, wave, lane);
  if (GROUPED) load_scale_group(G, &SG0, m0, n0, 0, wave, lane);
  for (int jt = 0; jt < my_tiles; ++jt) {
    // the tile after this one (past the last: this one again; its DMA then
    // fills a stage no later step reads)
    int nm0 = m0, nn0 = n0;
    if (jt + 1 < my_tiles) tile_origin(G, blockIdx.x + (jt + 1) * gridDim.x, nm0, nn0);
    if (GROUPED) {
      const int ng = nk / SGS;
      for (int ks = 0; ks < nk; ks += 2) {
        const int gi = jt * ng + ks / SGS;
        const ScaleGroup* sg = (gi & 1) ? &SG1 : &SG0;
        ScaleGroup* sg_next = (gi & 1) ? &SG0 : &SG1;
        const bool gstart = ks % SGS == 0;
        const bool glast = ks + SGS >= nk;   // next group: the next tile's first
        step_barrier();
        k_step<FA, FB, true, WIDE>(G, &S1, &S0, m0, n0, ks + 1, wave, lane, wm, wn, acc, sg,
                                   ks % SGS, gstart ? sg_next : nullptr, glast ? nm0 : m0,
                                   glast ? nn0 : n0, glast ? 0 : ks / SGS + 1);
        const bool last = ks + 2 == nk;
        step_barrier();
        k_step<FA, FB, true, WIDE>(G, &S0, &S1, last ? nm0 : m0, last ? nn0 : n0,
                                   last ? 0 : ks + 2, wave, lane, wm, wn, acc, sg,
                                   (ks + 1) % SGS, nullptr, 0, 0, 0);
      }
    } else {
      for (int ks = 0; ks < nk; ++ks) {
        const int step = jt * nk + ks;
        const bool last = ks + 1 == nk;
        step_barrier();
        Stage* fill = (step & 1) ? &S0 : &S1;
        const Stage* use = (step & 1) ? &S1 : &S0;
        k_step<FA, FB, false, false>(G, fill, use, last ? nm0 : m0, last ? nn0 : n0, last ? 0 : ks + 1,
                              wave, lane, wm, wn, acc, nullptr, 0, nullptr, 0, 0, 0);
      }
    }
    if (GROUPED && OUT_BF16 && G.vec16 && m0 + kBM <= G.M && n0 + kBN <= G.N) {
      // the tile's last step read S1 (the next tile's first DMA fills S0):
      // once every wave's reads of it are complete, S1 stages the epilogue
      // (8 slots of 8 KB over its a and b arrays, which are contiguous);
      // the next tile's first wait and barrier order its refill after
      // every wave's epilogue reads (s_waitcnt lgkmcnt(0) alone: 0xC07F)
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_s_barrier();
      store_tile_bf16_lds(G, m0, n0, wm, wn, wave, lane, acc, S1.a);
    } else {
      store_tile<OUT_BF16>(G, m0, n0, wm, wn, lane, acc);
    }
    m0 = nm0;
    n0 = nn0;
  }
  // the last (repeated) DMA lands before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Compute units of the current device, cached per device (one workgroup per
// CU: the kernel's registers and LDS allow no more).
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace

template <int FA, int FB>
void launch_gemm(const GemmArgs& G, bool bf16, bool grouped, unsigned grid, hipStream_t s) {
  if (bf16) {
    if (grouped)
      hipLaunchKernelGGL((mx_gemm_kernel<true, true, FA, FB>), dim3(grid), dim3(kThreads), 0, s, G);
    else
      hipLaunchKernelGGL((mx_gemm_kernel<true, false, FA, FB>), dim3(grid), dim3(kThreads), 0, s, G);
  } else {
    if (grouped)
      hipLaunchKernelGGL((mx_gemm_kernel<false, true, FA, FB>), dim3(grid), dim3(kThreads), 0, s, G);
    else
      hipLaunchKernelGGL((mx_gemm_kernel<false, false, FA, FB>), dim3(grid), dim3(kThreads), 0, s, G);
  }
}

extern "C" mxq_status mx_gemm(const uint8_t* a, int64_t lda, const uint8_t* a_scales, int64_t ldsa,
                              const uint8_t* b, int64_t ldb, const uint8_t* b_scales, int64_t ldsb,
                              int64_t M, int64_t N, int64_t K, mxq_elem elem_a, mxq_elem elem_b,
                              void* c, int64_t ldc, mxq_out_type c_type, void* stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 32 != 0) return MXQ_ERR_SHAPE;
  if (elem_a != MXQ_E4M3 && elem_a != MXQ_E2M1) return MXQ_ERR_ARG;
  if (elem_b != MXQ_E4M3 && elem_b != MXQ_E2M1) return MXQ_ERR_ARG;
  if (c_type != MXQ_OUT_F32 && c_type != MXQ_OUT_BF16) return MXQ_ERR_ARG;
  // code bytes per row: K for E4M3, K / 2 for packed E2M1
  const int64_t row_a = elem_a == MXQ_E2M1 ? K / 2 : K, row_b = elem_b == MXQ_E2M1 ? K / 2 : K;
  if (lda < row_a || ldb < row_b || ldsa < K / 32 || ldsb < K / 32 || ldc < N) return MXQ_ERR_SHAPE;
  if (K % kBK != 0 || M >= (1ll << 31) || N >= (1ll << 31) || K >= (1ll << 31))
    return MXQ_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return MXQ_OK;
  if (!a || !a_scales || !b || !b_scales || !c) return MXQ_ERR_NULL;
  if (!aligned(a, 16) || !aligned(b, 16) || lda % 16 || ldb % 16 || !aligned(a_scales, 4) ||
      !aligned(b_scales, 4) || ldsa % 4 || ldsb % 4 ||
      !aligned(c, c_type == MXQ_OUT_BF16 ? 2 : 4))
    return MXQ_ERR_ALIGN;
  GemmArgs G;
  G.a = a;
  G.sa = a_scales;
  G.b = b;
  G.sb = b_scales;
  G.c = c;
  G.lda = lda;
  G.ldsa = ldsa;
  G.ldb = ldb;
  G.ldsb = ldsb;
  G.ldc = ldc;
  G.M = (int)M;
  G.N = (int)N;
  G.K = (int)K;
  G.tiles_m = (int)((M + kBM - 1) / kBM);
  G.tiles_n = (int)((N + kBN - 1) / kBN);
  G.vec = (ldc % 4 == 0) && aligned(c, c_type == MXQ_OUT_BF16 ? 8 : 16);
  G.vec16 = c_type == MXQ_OUT_BF16 && ldc % 8 == 0 && aligned(c, 16);
  // persistent grid: one workgroup per CU, a multiple of 8 (one per XCD
  // round-robin slot), at most one per tile
  const int nb = G.tiles_m * G.tiles_n;
  const int cus = cu_count();
  if (cus <= 0) return MXQ_ERR_HIP;
  int grid_i = nb < cus ? nb : cus;
  if (grid_i >= 8) grid_i -= grid_i % 8;
  const unsigned grid = (unsigned)grid_i;
  hipStream_t s = (hipStream_t)stream;
  // the fast loop: whole scale groups (16 bytes of each scale row per
  // kScaleSteps steps, so 16-byte aligned rows) and an even step count
  const bool grouped = K % (kBK * kScaleSteps) == 0 && aligned(a_scales, 16) &&
                       aligned(b_scales, 16) && ldsa % 16 == 0 && ldsb % 16 == 0;
  const bool bf16 = c_type == MXQ_OUT_BF16;
  if (elem_a == MXQ_E4M3 && elem_b == MXQ_E4M3)
    launch_gemm<kFmtE4M3, kFmtE4M3>(G, bf16, grouped, grid, s);
  else if (elem_a == MXQ_E4M3)
    launch_gemm<kFmtE4M3, kFmtE2M1>(G, bf16, grouped, grid, s);
  else if (elem_b == MXQ_E4M3)
    launch_gemm<kFmtE2M1, kFmtE4M3>(G, bf16, grouped, grid, s);
  else
    launch_gemm<kFmtE2M1, kFmtE2M1>(G, bf16, grouped, grid, s);
  if (hipGetLastError() != hipSuccess) return MXQ_ERR_HIP;
  return MXQ_OK;
}
