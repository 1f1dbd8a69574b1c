// stream_floor.hip - bytes-only reference kernels with the traffic of the fused
// MXNorm -> MXFP8 call (libmxq_floor.so).
//
// These kernels are not part of the MX path and compute nothing of the method.
// Each moves exactly the bytes the fused call must move (read 2D bytes of a bf16
// row, write D code bytes and D/32 scale bytes) in the fused kernel's layout (one
// wavefront per row, 4 rows per 256-thread workgroup, 16-byte loads per lane,
// 8-byte code stores per lane, scale bytes gathered per wavefront and written in
// dwords). The timing module runs them beside the fused kernel on the same
// buffers to show what a kernel that only moves those bytes reaches on MI355X,
// with and without the dependencies the method adds:
//   bit 0  non-temporal loads
//   bit 1  non-temporal stores
//   bit 2  stores wait for a wavefront-wide reduction over the whole row (the
//          row normaliser's dependency)
//   bit 3  a workgroup first stages a D-element bf16 vector from L2 into LDS as
//          fp32 behind a barrier, and every chunk reads its 8 values back (the
//          gain staging)
// The "codes" are the high bytes of the bf16 inputs and each block's "scale" is
// one of its bytes: cheap byte moves that keep the stores live.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

#include "mxq_device.h"

template <bool NTL>
__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  if (NTL) return load16_stream(p);
  return load16(p);
}

template <bool NTS>
__device__ __forceinline__ void st8(uint8_t* p, uint2 v) {
  if (NTS) {
    const u32x2 w = {v.x, v.y};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p));
  } else {
    *reinterpret_cast<uint2*>(p) = v;
  }
}

struct FloorArgs {
  const uint16_t* x;
  const uint16_t* vec;  // D bf16 values staged to LDS (variant bit 3)
  uint8_t* codes;
  uint8_t* scales;
  int64_t T;
  int D;
};

template <int NC, bool NTL, bool NTS, bool GATE, bool STAGE>
__global__ __launch_bounds__(kThreads) void floor_kernel(FloorArgs A) {
  __shared__ float4 v_lds[STAGE ? NC * kWave * 2 : 1];
  __shared__ uint32_t sc_lds[kRowsPerBlock][NC * 4];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + wave;
  const bool live = row < A.T;
  const uint16_t* xr = A.x + (live ? row : A.T - 1) * (int64_t)A.D;
  const int dl = lane * 8;

  uint4 st[STAGE ? (NC * kWave + kThreads - 1) / kThreads : 1];
  if (STAGE) {
    const RangeLoader g(A.vec, A.D);
#pragma unroll
    for (int k = 0; k < (NC * kWave + kThreads - 1) / kThreads; ++k)
      st[k] = g.load8(((int)threadIdx.x + k * kThreads) * 8);
  }
  __builtin_amdgcn_sched_barrier(0);
  uint4 raw[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) raw[c] = ld16<NTL>(xr + min(c * kChunk + dl, A.D - 8));
  __builtin_amdgcn_sched_barrier(0);
  if (STAGE) {
#pragma unroll
    for (int k = 0; k < (NC * kWave + kThreads - 1) / kThreads; ++k) {
      const int i = (int)threadIdx.x + k * kThreads;
      if (i < NC * kWave) {
        float v[8];
        unpack8(st[k], v);
        const int c = i / kWave, l = i % kWave;
        v_lds[(2 * c) * kWave + l] = make_float4(v[0], v[1], v[2], v[3]);
        v_lds[(2 * c + 1) * kWave + l] = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
    __syncthreads();
  }
  if (!live) return;

  uint32_t flip = 0;
  if (GATE) {
    uint32_t m = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c) m = max(m, absmax_bits8(raw[c]));
    m = max_over_quads(quad_max_u32(m));
    flip = (m >> 31) ? 0x01010101u : 0u;  // never set (sign bits are cleared), unknown to the compiler
  }
  uint8_t* crow = A.codes + (uint64_t)row * (uint64_t)A.D;
  uint32_t* sc = sc_lds[wave];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int d = c * kChunk + dl;
    if (d < A.D) {
      uint2 code = make_uint2(__builtin_amdgcn_perm(raw[c].y, raw[c].x, 0x07050301u),
                              __builtin_amdgcn_perm(raw[c].w, raw[c].z, 0x07050301u));
      if (STAGE) {
        const float4 a = v_lds[(2 * c) * kWave + lane];
        code.x ^= (__float_as_uint(a.x) >> 31);
      }
      code.x ^= flip;
      st8<NTS>(crow + d, code);
      if ((lane & 3) == 0) reinterpret_cast<uint8_t*>(sc)[c * 16 + (lane >> 2)] = (uint8_t)code.x;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int K = A.D / 32;
  uint32_t* srow = reinterpret_cast<uint32_t*>(A.scales + (uint64_t)row * (uint64_t)K);
  for (int j = lane; j * 4 < K; j += kWave) srow[j] = sc[j];
}

template <int NC, int V>
int launch_v(const FloorArgs& A, hipStream_t s) {
  const unsigned grid = (unsigned)((A.T + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL((floor_kernel<NC, (V & 1) != 0, (V & 2) != 0, (V & 4) != 0, (V & 8) != 0>),
                     dim3(grid), dim3(kThreads), 0, s, A);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

template <int NC>
int launch_nc(const FloorArgs& A, int v, hipStream_t s) {
  switch (v) {
#define FLOOR_CASE(V) \
  case V:             \
    return launch_v<NC, V>(A, s);
    FLOOR_CASE(0) FLOOR_CASE(1) FLOOR_CASE(2) FLOOR_CASE(3) FLOOR_CASE(4) FLOOR_CASE(5)
    FLOOR_CASE(6) FLOOR_CASE(7) FLOOR_CASE(8) FLOOR_CASE(9) FLOOR_CASE(10) FLOOR_CASE(11)
    FLOOR_CASE(12) FLOOR_CASE(13) FLOOR_CASE(14) FLOOR_CASE(15)
#undef FLOOR_CASE
    default:
      return 2;
  }
}

}  // namespace

extern "C" {

// Bytes-only reference launch: x [T, D] bf16 contiguous, vec [D] bf16 (read
// only with variant bit 3), codes [T, D] bytes, scales [T, D/32] bytes, all
// device pointers, 16-byte aligned (scales 4-byte). D is 4096 or 8192.
// Returns 0 on success, 1 for a bad pointer or alignment, 2 for an unsupported
// size or variant, 3 when the launch fails.
int mxq_floor_stream(const uint16_t* x, const uint16_t* vec, int64_t T, int64_t D,
                     uint8_t* codes, uint8_t* scales, int variant, void* stream) {
  if (T <= 0 || (D != 4096 && D != 8192)) return 2;
  if (x == nullptr || codes == nullptr || scales == nullptr) return 1;
  if ((variant & 8) && vec == nullptr) return 1;
  if (((uintptr_t)x & 15) || ((uintptr_t)codes & 15) || ((uintptr_t)scales & 3) ||
      (vec && ((uintptr_t)vec & 15)))
    return 1;
  if ((T + kRowsPerBlock - 1) / kRowsPerBlock > 0x7FFFFFFF) return 2;
  FloorArgs A{x, vec, codes, scales, T, (int)D};
  return D == 4096 ? launch_nc<8>(A, variant, (hipStream_t)stream)
                   : launch_nc<16>(A, variant, (hipStream_t)stream);
}

}  // extern "C"
