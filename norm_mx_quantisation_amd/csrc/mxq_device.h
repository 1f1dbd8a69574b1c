// mxq_device.h - device helpers shared by the library's kernel sources
// (constants of the wavefront-per-row layout, bf16 widening, cross-lane
// reductions, row loads, gain staging reads). Included inside each source's
// anonymous namespace; the oracle never includes it.
#pragma once

constexpr int kWave = 64;
constexpr int kChunk = 512;           // elements per wave-wide chunk
constexpr int kRowsPerBlock = 4;      // wavefronts (rows) per workgroup
constexpr int kThreads = kWave * kRowsPerBlock;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ void unpack8(const uint4& r, float v[8]) {
  v[0] = bf16_lo(r.x); v[1] = bf16_hi(r.x);
  v[2] = bf16_lo(r.y); v[3] = bf16_hi(r.y);
  v[4] = bf16_lo(r.z); v[5] = bf16_hi(r.z);
  v[6] = bf16_lo(r.w); v[7] = bf16_hi(r.w);
}

// Largest |x| of 8 bf16 values as a bit pattern with the sign cleared. For
// non-negative bf16 the integer order is the magnitude order, with +Inf
// (0x7F80) below every NaN, so a non-finite element always surfaces.
__device__ __forceinline__ uint32_t absmax_bits8(const uint4& r) {
  const uint32_t k = 0x7FFF7FFFu;
  u16x2 a = __builtin_bit_cast(u16x2, r.x & k);
  u16x2 b = __builtin_bit_cast(u16x2, r.y & k);
  u16x2 c = __builtin_bit_cast(u16x2, r.z & k);
  u16x2 d = __builtin_bit_cast(u16x2, r.w & k);
  u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                      __builtin_elementwise_max(c, d));
  return (uint32_t)__builtin_elementwise_max(m.x, m.y);  // one 16-bit max of the halves
}

// Cross-lane moves that stay in the VALU (no LDS round trip): DPP within a
// quad and within a row of 16 lanes; across rows, lane reads into scalar
// registers (over_quads below).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppRowMirror = 0x140;    // lane i <-> 15 - i within a row of 16
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7 - i within 8 lanes

// Max over the 4 lanes of a quad (one MX block); exact, so any order is fine.
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  v = max(v, dpp<kDppQuadSwap1>(v));
  v = max(v, dpp<kDppQuadSwap2>(v));
  return v;
}

__device__ __forceinline__ uint32_t f32_add_bits(uint32_t a, uint32_t b) {
  return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
}

// Butterfly over the 16 quads of a wave for a value each quad holds in all 4
// lanes, with a commutative op: quad q meets q ^ 1 (half mirror), then pairs
// meet pairs (row mirror), so every lane of a row of 16 holds its row's
// value; the four row values are read into scalar registers and combined as
// (row0 op row1) op (row2 op row3). The result is wave-uniform, and the
// combining tree is the one an XOR butterfly over lane distances 4, 8, 16, 32
// builds.
template <class Op>
__device__ __forceinline__ uint32_t over_quads(uint32_t v, Op op) {
  v = op(v, dpp<kDppHalfMirror>(v));
  v = op(v, dpp<kDppRowMirror>(v));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)op(op(r0, r1), op(r2, r3)));
}

// Sum over the 16 quads of a value held identically by each quad's 4 lanes.
__device__ __forceinline__ float sum_over_quads(float v) {
  return __uint_as_float(over_quads(__float_as_uint(v), f32_add_bits));
}

__device__ __forceinline__ uint32_t max_over_quads(uint32_t v) {
  return over_quads(v, [](uint32_t a, uint32_t b) { return max(a, b); });
}

// Sum over all 64 lanes: lane pairs, then pairs of pairs within each quad,
// then over the quads.
__device__ __forceinline__ float sum_over_wave(float v) {
  uint32_t u = __float_as_uint(v);
  u = f32_add_bits(u, dpp<kDppQuadSwap1>(u));
  u = f32_add_bits(u, dpp<kDppQuadSwap2>(u));
  return sum_over_quads(__uint_as_float(u));
}

// Adds the squares of 8 bf16 values to s, in element order.
__device__ __forceinline__ float sumsq8(const uint4& r, float s) {
  float v[8];
  unpack8(r, v);
#pragma unroll
  for (int j = 0; j < 8; ++j) s = __builtin_fmaf(v[j], v[j], s);
  return s;
}

// ------------------------------------------------------------------ memory

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// The activation is read exactly once and the codes are written once: both
// go through non-temporal accesses.
__device__ __forceinline__ uint4 load16_stream(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Chunk c of a row, 16 bytes per lane. A lane whose 8 elements lie past the
// row end reads the row's last 16 bytes instead, so every load is
// unconditional and in bounds (a predicated load would make the compiler wait
// for earlier loads); callers mask such lanes where the data is used.
__device__ __forceinline__ uint4 load_chunk(const uint16_t* xr, int c, int dl, int D) {
  return load16_stream(xr + min(c * kChunk + dl, D - 8));
}

// Loads from one wave-uniform range (gamma) through a buffer resource whose
// size is the range's bytes: a lane's 16 bytes past the end read as zeros
// (the resource's range check), so the loads need no clamp. Word 3 is the
// gfx9 raw-buffer format.
struct RangeLoader {
  __amdgpu_buffer_rsrc_t rsrc;
  __device__ __forceinline__ RangeLoader(const uint16_t* base, int elems)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, elems * 2,
                                               0x00020000)) {}
  // 8 elements from element e
  __device__ __forceinline__ uint4 load8(int e) const {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, e * 2, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
  }
};

// Gains of chunk c for this lane, from the fp32 LDS copy laid out
// [chunk][half][lane] (two conflict-free 16-byte reads).
__device__ __forceinline__ void gains(const float4* g_lds, int c, int lane, float g[8]) {
  const float4 a = g_lds[(2 * c) * kWave + lane];
  const float4 b = g_lds[(2 * c + 1) * kWave + lane];
  g[0] = a.x; g[1] = a.y; g[2] = a.z; g[3] = a.w;
  g[4] = b.x; g[5] = b.y; g[6] = b.z; g[7] = b.w;
}

// Two fp32 values to a bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const uint16_t ua = __builtin_bit_cast(uint16_t, (__bf16)a);  // round to nearest even
  const uint16_t ub = __builtin_bit_cast(uint16_t, (__bf16)b);
  return (uint32_t)ua | ((uint32_t)ub << 16);
}

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

#define MXQ_LAUNCH_CHECK()                                   \
  do {                                                       \
    if (hipGetLastError() != hipSuccess) return MXQ_ERR_HIP; \
  } while (0)
