// mxq_bwd.hip - the straight-through backward of the normalisation on MI355X
// (gfx950), and its C-ABI entry points. What it computes is described on the
// page "MXNorm: Reusing MXFP block scales for efficient tensor normalisation",
// §2.3 (gradient paragraph); the declarations in mxq.h give the contract.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "mxq.h"

namespace {

#include "mxq_device.h"

// ------------------------------------------------------------------ backward

// Straight-through backward (MXNorm page, §2.3, gradient paragraph): the cast
// counts as the identity and RMSNorm's gradient is taken with the forward's
// normaliser inv = 1/G:  g = gamma * dy,  s = sum_i g_i x_i,
// dx_i = inv * g_i - inv^3 * (s / D) * x_i,  dgamma_i = sum_t dy_ti x_ti inv_t.
// fp32 order: g and dy * x are exact products of two bf16 values; s sums in
// chunk order per lane, then over the wave as every RMS path does, except for
// rows of 2, 4, 6 or 8 chunks (split_dot below), where each half of the
// row's chunks is summed that way and the two half sums add; k = (inv * inv)
// * inv, c = k * (s / D), dx = bf16(inv * g - c * x).
struct BwdArgs {
  const uint16_t* x;
  const uint16_t* dy;
  const uint16_t* gamma;
  const float* inv;
  uint16_t* dx;
  float* row_dot;
  float* partial;   // [groups][D] fp32 dgamma partials, or null
  int64_t ldx;
  int64_t lddy;
  int64_t T;
  int D;
  float Df;
  int rows_per_group;  // rows per workgroup, a multiple of kRowsPerBlock
};

// Rows of NC chunks whose dgamma backward splits each row over two
// wavefronts (mxnorm_bwd_pair_kernel); every backward kernel then sums the row
// dot by halves, so that dx and the row dot do not depend on whether dgamma
// is wanted.
constexpr bool split_dot(int nc) { return nc % 2 == 0 && nc <= 8; }

// One workgroup of 4 waves takes rows [g R, g R + R); wave w takes rows
// g R + w, g R + w + 4, ... in order and keeps its dgamma sums in registers
// (chunk c, element j of lane l is column 512 c + 8 l + j). The 4 waves'
// sums are combined as (w0 + w2) + (w1 + w3) through LDS into the group's
// partial row. KEEP holds the row's x and dy in registers between the two
// passes (D <= 4096); otherwise the second pass loads them again (from L2).
// NT: dx leaves through non-temporal stores.
template <int NC, bool GAMMA, bool DGAMMA, bool KEEP, bool NT>
__global__ __launch_bounds__(kThreads) void mxnorm_bwd_kernel(BwdArgs A) {
  __shared__ float4 g_lds[GAMMA ? NC * kWave * 2 : 1];
  __shared__ float red[DGAMMA ? 2 * NC * 8 * kWave : 1];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int dl = lane * 8;
  const int64_t row0 = (int64_t)blockIdx.x * A.rows_per_group;
  const int64_t row_end = min(A.T, row0 + A.rows_per_group);

  // Gains and the wave's first row go out before the gains are staged to
  // LDS: gains first (loads retire in order, so staging waits for them
  // alone), then the row, whose loads stay in flight across the staging and
  // its barrier. Item i of the gains is chunk i / 64, lane i % 64; a load past
  // the row end is clamped in bounds and its item never read.
  constexpr int kGItems = (NC * kWave + kThreads - 1) / kThreads;
  uint4 gr[GAMMA ? kGItems : 1];
  if (GAMMA) {
#pragma unroll
    for (int k = 0; k < kGItems; ++k) {
      const int i = min((int)threadIdx.x + k * kThreads, NC * kWave - 1);
      gr[k] = load16(A.gamma + min(i * 8, A.D - 8));
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // KEEP: the row's packed x and dy in registers. The next row goes into
  // xn / dn: the first one here, later ones (with dgamma a wave walks
  // several rows) while the current row is processed; without dgamma each
  // wave has one row.
  constexpr bool PREFETCH = KEEP && DGAMMA;
  uint4 xk[KEEP ? NC : 1], dk[KEEP ? NC : 1], xn[KEEP ? NC : 1], dn[KEEP ? NC : 1];
  if (KEEP && row0 + wave < row_end) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      xn[c] = load_chunk(A.x + (row0 + wave) * A.ldx, c, dl, A.D);
      dn[c] = load_chunk(A.dy + (row0 + wave) * A.lddy, c, dl, A.D);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  if (GAMMA) {
#pragma unroll
    for (int k = 0; k < kGItems; ++k) {
      const int i = (int)threadIdx.x + k * kThreads;
      if (i < NC * kWave) {
        float v[8];
        unpack8(gr[k], v);
        const int c = i / kWave, l = i % kWave;
        g_lds[(2 * c) * kWave + l] = make_float4(v[0], v[1], v[2], v[3]);
        g_lds[(2 * c + 1) * kWave + l] = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
    __syncthreads();
  }

  float acc[DGAMMA ? NC : 1][8];
  if (DGAMMA) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[c][j] = 0.0f;
  }

  for (int64_t row = row0 + wave; row < row_end; row += kRowsPerBlock) {
    const uint16_t* xr = A.x + row * A.ldx;
    const uint16_t* dr = A.dy + row * A.lddy;
    float s = 0.0f, s_hi = 0.0f;  // s_hi: the second half's chunks (split_dot)
    float g[8] = {1, 1, 1, 1, 1, 1, 1, 1};
    const int64_t next = row + kRowsPerBlock;
    if (KEEP) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        xk[c] = xn[c];
        dk[c] = dn[c];
      }
      if (PREFETCH && next < row_end) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          xn[c] = load_chunk(A.x + next * A.ldx, c, dl, A.D);
          dn[c] = load_chunk(A.dy + next * A.lddy, c, dl, A.D);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c * kChunk + dl < A.D) {
        float xv[8], dv[8];
        unpack8(KEEP ? xk[c] : load16(xr + c * kChunk + dl), xv);
        unpack8(KEEP ? dk[c] : load16(dr + c * kChunk + dl), dv);
        if (GAMMA) gains(g_lds, c, lane, g);
        float& t = (split_dot(NC) && c >= NC / 2) ? s_hi : s;
#pragma unroll
        for (int j = 0; j < 8; ++j) t = __builtin_fmaf(g[j] * dv[j], xv[j], t);
      }
    }
    if (KEEP) {
      // keep the packed row: widen again in the second pass rather than hold
      // both passes' fp32 copies (see mxnorm_row_reg)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        asm volatile("" : "+v"(xk[c].x), "+v"(xk[c].y), "+v"(xk[c].z), "+v"(xk[c].w));
        asm volatile("" : "+v"(dk[c].x), "+v"(dk[c].y), "+v"(dk[c].z), "+v"(dk[c].w));
      }
    }
    s = split_dot(NC) ? sum_over_wave(s) + sum_over_wave(s_hi) : sum_over_wave(s);
    const float a = A.inv[row];
    if (lane == 0 && A.row_dot) A.row_dot[row] = s;
    const float k = (a * a) * a;
    const float cf = k * (s / A.Df);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int d = c * kChunk + dl;
      if (d < A.D) {
        float xv[8], dv[8], o[8];
        unpack8(KEEP ? xk[c] : load16(xr + d), xv);
        unpack8(KEEP ? dk[c] : load16(dr + d), dv);
        if (GAMMA) gains(g_lds, c, lane, g);
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = a * (g[j] * dv[j]) - cf * xv[j];
        const u32x4 w = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                         pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
        u32x4* dst = reinterpret_cast<u32x4*>(A.dx + (uint64_t)row * (uint64_t)A.D + (uint64_t)d);
        if constexpr (NT)
          __builtin_nontemporal_store(w, dst);
        else
          *dst = w;
        if (DGAMMA) {
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[c][j] += (dv[j] * xv[j]) * a;
        }
      }
    }
    // a wave with several rows and no prefetch loads its next row once this
    // one is done with (the current plan gives such waves a single row)
    if (KEEP && !PREFETCH && next < row_end) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        xn[c] = load_chunk(A.x + next * A.ldx, c, dl, A.D);
        dn[c] = load_chunk(A.dy + next * A.lddy, c, dl, A.D);
      }
    }
  }

  if (DGAMMA) {
    // red: two slots of [chunk][element][lane] floats
    auto slot = [&](int sl, int c, int j) -> float& { return red[((sl * NC + c) * 8 + j) * kWave + lane]; };
    if (wave >= 2) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j) slot(wave - 2, c, j) = acc[c][j];
    }
    __syncthreads();
    if (wave < 2) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[c][j] += slot(wave, c, j);
    }
    __syncthreads();
    if (wave == 1) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j) slot(0, c, j) = acc[c][j];
    }
    __syncthreads();
    if (wave == 0) {
      float* out = A.partial + (uint64_t)blockIdx.x * (uint64_t)A.D;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int d = c * kChunk + dl;
        if (d < A.D) {
          float r[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) r[j] = acc[c][j] + slot(0, c, j);
          *reinterpret_cast<float4*>(out + d) = make_float4(r[0], r[1], r[2], r[3]);
          *reinterpret_cast<float4*>(out + d + 4) = make_float4(r[4], r[5], r[6], r[7]);
        }
      }
    }
  }
}

// dx and the dgamma partial rows with each row split over two wavefronts
// (rows of NC = 2 H chunks, H <= 4). A workgroup of 8 waves takes rows
// [g R, g R + R); wave w takes column half h = w & 1 (chunks [h H, h H + H))
// of rows g R + r, g R + r + 4, ... (r = w >> 1), so a wave holds half the
// registers of a whole-row wave and the workgroup keeps 4 waves per SIMD
// where the whole-row kernel keeps 2. Each half's row dot (chunk order per
// lane, then over the wave) meets its partner's in LDS at a barrier per step,
// s = s_0 + s_1. Every wave runs the same number of steps, so the barriers
// match; a step past a slot's last row does no work. The next row's half is
// loaded once the current one is done with: holding both would take the wave
// past 128 VGPRs, and with it the workgroup's 4 waves per SIMD (a form that
// kept the column sums in LDS to make room for the next half measured 3-6%
// slower: 47.6-48.9 against 45.9 us per call on [8192, 4096]; reloading each
// chunk's registers with the next row's chunk as soon as its dx is stored
// measured 47.4-47.8 against 45.4-46.3 us, the same on [32768, 4096]). dgamma adds
// the same terms in the same order as mxnorm_bwd_kernel (a slot's rows in
// order, then (r0 + r2) + (r1 + r3) per column), so the partial rows are
// bit-identical. dx leaves through non-temporal stores (measured faster on
// [8192, 4096] and [32768, 4096]: 45.7-46.3 against 46.2-47.1 us per call,
// 155.5 against 161.6-162.5 us).
constexpr int kPairWaves = 8;
constexpr int kPairThreads = kPairWaves * kWave;

template <int H, bool GAMMA>
__global__ __launch_bounds__(kPairThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void mxnorm_bwd_pair_kernel(BwdArgs A) {
  constexpr int NC = 2 * H;
  constexpr int kGFloat4 = GAMMA ? NC * kWave * 2 : 0;      // gains, as float4
  constexpr int kRedFloat4 = 2 * 2 * H * 8 * kWave / 4;    // [half][slot][c][j][lane] floats
  constexpr int kLds = kGFloat4 > kRedFloat4 ? kGFloat4 : kRedFloat4;
  __shared__ float4 lds[kLds];   // the gains, then (after the last step) the dgamma combine
  __shared__ float s_lds[2][4][2];  // [step parity][slot][half]
  float4* g_lds = lds;
  float* red = reinterpret_cast<float*>(lds);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int h = wave & 1, r = wave >> 1;
  const int dl = lane * 8;
  const int64_t row0 = (int64_t)blockIdx.x * A.rows_per_group;
  const int64_t row_end = min(A.T, row0 + A.rows_per_group);
  const int steps = (int)((row_end - row0 + kRowsPerBlock - 1) / kRowsPerBlock);  // uniform

  constexpr int kGItems = (NC * kWave + kPairThreads - 1) / kPairThreads;
  uint4 gr[GAMMA ? kGItems : 1];
  if (GAMMA) {
#pragma unroll
    for (int k = 0; k < kGItems; ++k) {
      const int i = min((int)threadIdx.x + k * kPairThreads, NC * kWave - 1);
      gr[k] = load16(A.gamma + min(i * 8, A.D - 8));
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // The wave's chunks are h H + c, c < H; the last can end inside the row.
  uint4 xk[H], dk[H];
  auto load_half = [&](int64_t row, uint4 (&xb)[H], uint4 (&db)[H]) {
#pragma unroll
    for (int c = 0; c < H; ++c) {
      xb[c] = load_chunk(A.x + row * A.ldx, h * H + c, dl, A.D);
      db[c] = load_chunk(A.dy + row * A.lddy, h * H + c, dl, A.D);
    }
  };
  if (row0 + r < row_end) load_half(row0 + r, xk, dk);
  __builtin_amdgcn_sched_barrier(0);

  if (GAMMA) {
#pragma unroll
    for (int k = 0; k < kGItems; ++k) {
      const int i = (int)threadIdx.x + k * kPairThreads;
      if (i < NC * kWave) {
        float v[8];
        unpack8(gr[k], v);
        const int c = i / kWave, l = i % kWave;
        g_lds[(2 * c) * kWave + l] = make_float4(v[0], v[1], v[2], v[3]);
        g_lds[(2 * c + 1) * kWave + l] = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
  }
  __syncthreads();

  float acc[H][8];
#pragma unroll
  for (int c = 0; c < H; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[c][j] = 0.0f;

  for (int step = 0; step < steps; ++step) {
    const int64_t row = row0 + r + (int64_t)step * kRowsPerBlock;
    const int64_t next = row + kRowsPerBlock;
    const bool live = row < row_end;  // uniform over the wave
    float s = 0.0f;
    float g[8] = {1, 1, 1, 1, 1, 1, 1, 1};
    if (live) {
#pragma unroll
      for (int c = 0; c < H; ++c) {
        const int cc = h * H + c;
        if (cc * kChunk + dl < A.D) {
          float xv[8], dv[8];
          unpack8(xk[c], xv);
          unpack8(dk[c], dv);
          if (GAMMA) gains(g_lds, cc, lane, g);
#pragma unroll
          for (int j = 0; j < 8; ++j) s = __builtin_fmaf(g[j] * dv[j], xv[j], s);
        }
      }
#pragma unroll
      for (int c = 0; c < H; ++c) {
        asm volatile("" : "+v"(xk[c].x), "+v"(xk[c].y), "+v"(xk[c].z), "+v"(xk[c].w));
        asm volatile("" : "+v"(dk[c].x), "+v"(dk[c].y), "+v"(dk[c].z), "+v"(dk[c].w));
      }
      s = sum_over_wave(s);
      if (lane == 0) s_lds[step & 1][r][h] = s;
    }
    // Both halves' sums are in LDS after this barrier. The slot written at
    // step + 2 is this step's again; no wave gets there before every wave has
    // passed the barrier of step + 1, so after its read here. (A handshake
    // between the two waves of a row alone, through per-slot step flags in
    // LDS, measured no faster: 46.0-47.2 against 45.5-45.8 us per call on
    // [8192, 4096].)
    __syncthreads();
    if (live) {
      s = s_lds[step & 1][r][0] + s_lds[step & 1][r][1];
      const float a = A.inv[row];
      if (h == 0 && lane == 0 && A.row_dot) A.row_dot[row] = s;
      const float k = (a * a) * a;
      const float cf = k * (s / A.Df);
#pragma unroll
      for (int c = 0; c < H; ++c) {
        const int cc = h * H + c;
        const int d = cc * kChunk + dl;
        if (d < A.D) {
          float xv[8], dv[8], o[8];
          unpack8(xk[c], xv);
          unpack8(dk[c], dv);
          if (GAMMA) gains(g_lds, cc, lane, g);
#pragma unroll
          for (int j = 0; j < 8; ++j) o[j] = a * (g[j] * dv[j]) - cf * xv[j];
          const u32x4 w = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                           pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
          u32x4* dst = reinterpret_cast<u32x4*>(A.dx + (uint64_t)row * (uint64_t)A.D + (uint64_t)d);
          __builtin_nontemporal_store(w, dst);
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[c][j] += (dv[j] * xv[j]) * a;
        }
      }
    }
    if (next < row_end) load_half(next, xk, dk);
  }

  // The slots' sums per column: (r0 + r2) + (r1 + r3), through LDS (the gains
  // are dead: the barrier below follows every wave's last read of them).
  auto slot = [&](int sl, int c, int j) -> float& {
    return red[(((h * 2 + sl) * H + c) * 8 + j) * kWave + lane];
  };
  __syncthreads();
  if (r >= 2) {
#pragma unroll
    for (int c = 0; c < H; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) slot(r - 2, c, j) = acc[c][j];
  }
  __syncthreads();
  if (r < 2) {
#pragma unroll
    for (int c = 0; c < H; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[c][j] += slot(r, c, j);
  }
  __syncthreads();
  if (r == 1) {
#pragma unroll
    for (int c = 0; c < H; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) slot(0, c, j) = acc[c][j];
  }
  __syncthreads();
  if (r == 0) {
    float* out = A.partial + (uint64_t)blockIdx.x * (uint64_t)A.D;
#pragma unroll
    for (int c = 0; c < H; ++c) {
      const int d = (h * H + c) * kChunk + dl;
      if (d < A.D) {
        float o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = acc[c][j] + slot(0, c, j);
        *reinterpret_cast<float4*>(out + d) = make_float4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<float4*>(out + d + 4) = make_float4(o[4], o[5], o[6], o[7]);
      }
    }
  }
}

// dgamma[d] = sum of in[r][d] over the rows r < rows (rows <= kBwdMaxGroups;
// rows == 0 writes zeros and reads nothing). A workgroup covers 8 float4
// columns, one whole 128-byte line of each row, so that no line is fetched by
// two workgroups (neighbouring workgroups usually run on different XCDs,
// whose L2s do not share lines). Wave w adds rows [w q, w q + q)
// (q = ceil(rows / 4)): lane l takes float4 column l % 8 of rows
// w q + l / 8 + 8 k, k = 0..15, in that order, so that one load instruction
// reads 8 whole lines and the sixteen loads go out together (one memory round
// trip). The 8 lanes of a column then combine by a butterfly over lane bits
// 3..5 (every lane ends with the same sum), and the four wave sums as
// (w0 + w1) + (w2 + w3).
constexpr int kColLoads = 16;  // loads per lane: 8 rows each, 128 rows per wave
__global__ __launch_bounds__(kThreads) void col_sum_kernel(const float* in, int rows, int D4,
                                                           float* out) {
  __shared__ float4 part[3][8];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int c = lane & 7, rs = lane >> 3;
  const int q = blockIdx.x * 8 + c;  // float4 column, < D4 (D4 % 8 == 0)
  float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (rows > 0) {
    const int per = (rows + 3) / 4;
    const int r0 = wave * per;
    const int r1 = min(rows, r0 + per);
    const float4* src = reinterpret_cast<const float4*>(in);
    float4 v[kColLoads];
#pragma unroll
    for (int k = 0; k < kColLoads; ++k) v[k] = src[(size_t)min(r0 + rs + 8 * k, rows - 1) * D4 + q];
#pragma unroll
    for (int k = 0; k < kColLoads; ++k)
      if (r0 + rs + 8 * k < r1) {
        a.x += v[k].x; a.y += v[k].y; a.z += v[k].z; a.w += v[k].w;
      }
  }
#pragma unroll
  for (int m = 8; m < kWave; m <<= 1) {
    a.x += __shfl_xor(a.x, m);
    a.y += __shfl_xor(a.y, m);
    a.z += __shfl_xor(a.z, m);
    a.w += __shfl_xor(a.w, m);
  }
  if (wave > 0 && rs == 0) part[wave - 1][c] = a;
  __syncthreads();
  if (wave == 0 && rs == 0) {
    const float4 b = part[0][c], d = part[1][c], e = part[2][c];
    float4 o;
    o.x = (a.x + b.x) + (d.x + e.x);
    o.y = (a.y + b.y) + (d.y + e.y);
    o.z = (a.z + b.z) + (d.z + e.z);
    o.w = (a.w + b.w) + (d.w + e.w);
    reinterpret_cast<float4*>(out)[q] = o;
  }
}

// Backward launch geometry: rows per workgroup, a multiple of 4, so that at
// most kBwdMaxGroups partial rows are written; one column-sum launch then
// adds them (each wave of it covers at most 128 rows: 8 per load, 16 loads).
constexpr int64_t kBwdMaxGroups = 512;
static_assert(kBwdMaxGroups <= 4 * 8 * kColLoads, "the column sum reads at most 512 rows");

struct BwdPlan {
  int64_t rows_per_group, groups;
  size_t workspace_bytes;
};

BwdPlan bwd_plan(int64_t T, int64_t D, bool dgamma = true) {
  BwdPlan p;
  // without dgamma there are no partials: one row per wave, as in the forward
  int64_t r = dgamma ? (T + kBwdMaxGroups - 1) / kBwdMaxGroups : kRowsPerBlock;
  r = ((r + kRowsPerBlock - 1) / kRowsPerBlock) * kRowsPerBlock;
  p.rows_per_group = r < kRowsPerBlock ? kRowsPerBlock : r;
  p.groups = (T + p.rows_per_group - 1) / p.rows_per_group;
  p.workspace_bytes = (size_t)p.groups * (size_t)D * sizeof(float);
  return p;
}

// With dgamma, rows of 2, 4, 6 or 8 chunks go to the pair kernel (on
// [8192, 4096] 45.7-46.3 against 47.8-47.9 us per call for the whole-row
// kernel, on [32768, 4096] 155.5 against 159 us). In the whole-row kernel,
// non-temporal dx stores measured faster without dgamma (34.6 against 34.8 us
// on [8192, 4096], 128 against 136 us on [32768, 4096]) and with it at 64
// rows per workgroup ([32768, 4096]: 157 against 163 us), but slower at 16
// rows per workgroup ([8192, 4096]: 45.7 against 43.4 us); its dgamma form
// takes them from 32 rows per workgroup on.
template <int NC, bool GAMMA, bool DGAMMA>
mxq_status launch_bwd(const BwdArgs& A, unsigned groups, hipStream_t s) {
  constexpr bool kKeep = NC <= 8;
  if constexpr (DGAMMA && split_dot(NC)) {
    hipLaunchKernelGGL((mxnorm_bwd_pair_kernel<NC / 2, GAMMA>),
                       dim3(groups), dim3(kPairThreads), 0, s, A);
    MXQ_LAUNCH_CHECK();
    return MXQ_OK;
  }
  if (!DGAMMA || A.rows_per_group >= 32)
    hipLaunchKernelGGL((mxnorm_bwd_kernel<NC, GAMMA, DGAMMA, kKeep, true>), dim3(groups),
                       dim3(kThreads), 0, s, A);
  else
    hipLaunchKernelGGL((mxnorm_bwd_kernel<NC, GAMMA, true, kKeep, false>), dim3(groups),
                       dim3(kThreads), 0, s, A);
  MXQ_LAUNCH_CHECK();
  return MXQ_OK;
}

template <bool GAMMA, bool DGAMMA>
mxq_status dispatch_bwd(const BwdArgs& A, int nc, unsigned groups, hipStream_t s) {
  switch (nc) {
#define MXQ_CASE(N) \
  case N:           \
    return launch_bwd<N, GAMMA, DGAMMA>(A, groups, s);
    MXQ_CASE(1) MXQ_CASE(2) MXQ_CASE(3) MXQ_CASE(4) MXQ_CASE(5) MXQ_CASE(6) MXQ_CASE(7)
    MXQ_CASE(8) MXQ_CASE(9) MXQ_CASE(10) MXQ_CASE(11) MXQ_CASE(12) MXQ_CASE(13) MXQ_CASE(14)
    MXQ_CASE(15) MXQ_CASE(16)
#undef MXQ_CASE
    default:
      return MXQ_ERR_UNSUPPORTED;
  }
}

mxq_status launch_col_sum(const float* in, int rows, int D, float* out, hipStream_t s) {
  const int D4 = D / 4;  // a multiple of 8 (D % 32 == 0)
  hipLaunchKernelGGL(col_sum_kernel, dim3(D4 / 8), dim3(kThreads), 0, s, in, rows, D4, out);
  MXQ_LAUNCH_CHECK();
  return MXQ_OK;
}

// Argument checks shared by both entry points (the workspace is checked by
// the caller).
mxq_status check_bwd(const uint16_t* x, int64_t ldx, const uint16_t* gamma, const uint16_t* dy,
                     int64_t lddy, const float* inv_norm, int64_t T, int64_t D, uint16_t* dx,
                     const float* row_dot, const float* dgamma) {
  if (T < 0 || D <= 0 || D % 32 != 0 || ldx < D || lddy < D) return MXQ_ERR_SHAPE;
  if (D > MXQ_MAX_D_REG) return MXQ_ERR_UNSUPPORTED;
  if ((uint64_t)T * (uint64_t)D >= (1ull << 40)) return MXQ_ERR_UNSUPPORTED;
  if (dgamma != nullptr && !aligned(dgamma, 16)) return MXQ_ERR_ALIGN;
  if (T == 0) return MXQ_OK;
  if (x == nullptr || dy == nullptr || inv_norm == nullptr || dx == nullptr) return MXQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(dy, 16) || !aligned(dx, 16) || ldx % 8 != 0 || lddy % 8 != 0)
    return MXQ_ERR_ALIGN;
  if (gamma != nullptr && !aligned(gamma, 16)) return MXQ_ERR_ALIGN;
  if (!aligned(inv_norm, 4) || (row_dot != nullptr && !aligned(row_dot, 4))) return MXQ_ERR_ALIGN;
  return MXQ_OK;
}

// Launches after validation; partial holds the dgamma partial rows (at least
// bwd_plan(T, D).workspace_bytes) when dgamma is wanted.
mxq_status run_bwd(const uint16_t* x, int64_t ldx, const uint16_t* gamma, const uint16_t* dy,
                   int64_t lddy, const float* inv_norm, int64_t T, int64_t D, uint16_t* dx,
                   float* row_dot, float* dgamma, float* partial, hipStream_t s) {
  if (T == 0) {
    // nothing to read; the gain's gradient of an empty batch is zero
    return dgamma ? launch_col_sum(nullptr, 0, (int)D, dgamma, s) : MXQ_OK;
  }
  const BwdPlan plan = bwd_plan(T, D, dgamma != nullptr);
  BwdArgs A;
  A.x = x;
  A.dy = dy;
  A.gamma = gamma;
  A.inv = inv_norm;
  A.dx = dx;
  A.row_dot = row_dot;
  A.partial = dgamma ? partial : nullptr;
  A.ldx = ldx;
  A.lddy = lddy;
  A.T = T;
  A.D = (int)D;
  A.Df = (float)D;
  A.rows_per_group = (int)plan.rows_per_group;
  const int nc = (int)((D + kChunk - 1) / kChunk);
  const unsigned groups = (unsigned)plan.groups;
  const bool g = gamma != nullptr;
  mxq_status st;
  if (dgamma)
    st = g ? dispatch_bwd<true, true>(A, nc, groups, s) : dispatch_bwd<false, true>(A, nc, groups, s);
  else
    st = g ? dispatch_bwd<true, false>(A, nc, groups, s) : dispatch_bwd<false, false>(A, nc, groups, s);
  if (st != MXQ_OK || dgamma == nullptr) return st;
  // partials [groups][D] -> dgamma [D]
  return launch_col_sum(A.partial, (int)plan.groups, (int)D, dgamma, s);
}

// ------------------------------------------------------------------ allocation-free variant

// The dgamma partial rows of mxnorm_bwd_noalloc: every partial row the
// backward can write (at most kBwdMaxGroups rows of MXQ_MAX_D_REG floats,
// 16 MiB), in one array per GPU that the library holds until the process
// ends. Each call writes every partial row it later reads, so nothing needs
// clearing between calls; calls that overlap on one GPU race on it.
constexpr size_t kScratchBytes = (size_t)kBwdMaxGroups * MXQ_MAX_D_REG * sizeof(float);

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// The array's device address on the current device. In host code `scratch`
// is only a handle for the runtime, never an address a kernel may use: the
// address is looked up once per device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

mxq_status device_scratch(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MXQ_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MXQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return MXQ_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = static_cast<float*>(g_scratch[dev]);
  return MXQ_OK;
}

}  // namespace

extern "C" {

size_t mxnorm_bwd_workspace_size(int64_t T, int64_t D) {
  if (T < 0 || D <= 0 || D % 32 != 0) return 0;
  return bwd_plan(T, D).workspace_bytes;
}

mxq_status mxnorm_bwd(const uint16_t* x, int64_t ldx, const uint16_t* gamma, const uint16_t* dy,
                      int64_t lddy, const float* inv_norm, int64_t T, int64_t D, uint16_t* dx,
                      float* row_dot, float* dgamma, void* workspace, size_t workspace_bytes,
                      void* stream) {
  mxq_status st = check_bwd(x, ldx, gamma, dy, lddy, inv_norm, T, D, dx, row_dot, dgamma);
  if (st != MXQ_OK) return st;
  if (dgamma != nullptr) {
    if (workspace == nullptr) return MXQ_ERR_NULL;
    if (workspace_bytes < bwd_plan(T, D).workspace_bytes) return MXQ_ERR_ARG;
    if (!aligned(workspace, 16)) return MXQ_ERR_ALIGN;
  }
  return run_bwd(x, ldx, gamma, dy, lddy, inv_norm, T, D, dx, row_dot, dgamma,
                 static_cast<float*>(workspace), (hipStream_t)stream);
}

mxq_status mxnorm_bwd_noalloc(const uint16_t* x, int64_t ldx, const uint16_t* gamma,
                              const uint16_t* dy, int64_t lddy, const float* inv_norm, int64_t T,
                              int64_t D, uint16_t* dx, float* row_dot, float* dgamma,
                              void* stream) {
  mxq_status st = check_bwd(x, ldx, gamma, dy, lddy, inv_norm, T, D, dx, row_dot, dgamma);
  if (st != MXQ_OK) return st;
  float* partial = nullptr;
  if (dgamma != nullptr) {
    if (bwd_plan(T, D).workspace_bytes > kScratchBytes) return MXQ_ERR_UNSUPPORTED;
    st = device_scratch(&partial);
    if (st != MXQ_OK) return st;
  }
  return run_bwd(x, ldx, gamma, dy, lddy, inv_norm, T, D, dx, row_dot, dgamma, partial,
                 (hipStream_t)stream);
}

}  // extern "C"
