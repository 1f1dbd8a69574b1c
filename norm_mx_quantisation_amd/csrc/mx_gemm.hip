// mx_gemm.hip - the MX GEMM that consumes MXNorm's output on MI355X (gfx950).
//
// C[m][n] = sum_k A[m][k] * B[n][k] over MX operands: A is the activation's
// E4M3 codes [M, K] with E8M0 scales [M, K/32] (MXNorm's output, page "MXNorm:
// Reusing MXFP block scales for efficient tensor normalisation", §2.1), B the
// next linear layer's weight [N, K], gain folded and MX-cast along K (§2.3,
// MXNormLinear). The products run on the gfx950 block-scaled matrix cores
// (v_mfma_scale_f32_16x16x128_f8f6f4), which apply both operands' E8M0 scales
// and accumulate in fp32.
//
// Operand layout of that instruction for 8-bit data (probed on the device):
// lane l carries row l % 16 of its 16 x 128 operand; its 32 bytes are K
// [16 g, 16 g + 16) then [64 + 16 g, 64 + 16 g + 16), g = l / 16; the scale of
// K block b (32 columns) of row r is the low byte of lane r + 16 b's scale
// register, whose other bytes must be zero. The result's
// lane l holds column l % 16, rows 4 (l / 16) + i in its 4 registers.
// Here the instruction takes B as its row operand and A as its column
// operand, so each lane's 4 registers are 4 consecutive columns of C.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "mxq.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWave = 64;
constexpr int kThreads = 256;   // 4 waves, 2 x 2 over the tile
constexpr int kBM = 256;        // tile rows (A)
constexpr int kBN = 256;        // tile columns (B rows)
constexpr int kBK = 128;        // K per step: 4 MX blocks, one MFMA deep
constexpr int kChunks = kBK / 16;   // 16-byte chunks per row and step

struct GemmArgs {
  const uint8_t* a;
  const uint8_t* sa;
  const uint8_t* b;
  const uint8_t* sb;
  void* c;
  int64_t lda, ldsa, ldb, ldsb, ldc;  // code bytes, scale bytes, C elements per row
  int M, N, K;
  int tiles_m, tiles_n;
  int vec;  // C rows allow 4-element vector stores (aligned base, ldc % 4 == 0)
};

// One K step of both operands in LDS. Code rows hold 8 chunks of 16 bytes;
// chunk c of row r sits at position c ^ (r & 7), so the 8 lanes that read one
// 128-byte stretch of a row group touch all 32 banks once.
struct Stage {
  uint4 a[kBM * kChunks];
  uint4 b[kBN * kChunks];
  uint32_t sa[kBM];   // the step's 4 scale bytes of each row
  uint32_t sb[kBN];
};

// Direct-to-LDS loads of one K step. A wave instruction moves 64 x 16 bytes
// = 8 rows; lane i lands at position i, i.e. row i / 8, physical chunk i % 8,
// so it fetches logical chunk (i % 8) ^ (row & 7). Rows past the matrix end
// re-read its last row (their results are never stored).
__device__ __forceinline__ void load_stage(const GemmArgs& G, Stage& S, int m0, int n0, int ks,
                                           int wave, int lane) {
  const int k0 = ks * kBK;
#pragma unroll
  for (int q = 0; q < kBM / 8 / 4; ++q) {
    const int blk = wave * (kBM / 8 / 4) + q;
    const int r = blk * 8 + (lane >> 3);
    const int c = (lane & 7) ^ (r & 7);
    const int ra = min(m0 + r, G.M - 1);
    __builtin_amdgcn_global_load_lds((const void*)(G.a + (int64_t)ra * G.lda + k0 + c * 16),
                                     (lds_void*)&S.a[blk * kWave], 16, 0, 0);
  }
#pragma unroll
  for (int q = 0; q < kBN / 8 / 4; ++q) {
    const int blk = wave * (kBN / 8 / 4) + q;
    const int r = blk * 8 + (lane >> 3);
    const int c = (lane & 7) ^ (r & 7);
    const int rb = min(n0 + r, G.N - 1);
    __builtin_amdgcn_global_load_lds((const void*)(G.b + (int64_t)rb * G.ldb + k0 + c * 16),
                                     (lds_void*)&S.b[blk * kWave], 16, 0, 0);
  }
  // scales: 4 bytes (the step's 4 blocks) per row, 64 rows per wave
  const int rs = wave * kWave + lane;
  __builtin_amdgcn_global_load_lds((const void*)(G.sa + (int64_t)min(m0 + rs, G.M - 1) * G.ldsa + ks * 4),
                                   (lds_void*)&S.sa[wave * kWave], 4, 0, 0);
  __builtin_amdgcn_global_load_lds((const void*)(G.sb + (int64_t)min(n0 + rs, G.N - 1) * G.ldsb + ks * 4),
                                   (lds_void*)&S.sb[wave * kWave], 4, 0, 0);
}
// The 32-byte MFMA operand of lane (row r, group g): chunks g and 4 + g.
__device__ __forceinline__ v8i operand(const uint4* rows, int r, int g) {
  const uint4 lo = rows[r * kChunks + (g ^ (r & 7))];
  const uint4 hi = rows[r * kChunks + ((4 + g) ^ (r & 7))];
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Workgroup barrier without the memory fence __syncthreads() carries (that
// fence waits for every load in flight, including the next step's prefetch).
// LDS hazards are handled by the explicit waits around it.
__device__ __forceinline__ void barrier() { __builtin_amdgcn_s_barrier(); }

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mx_gemm_e4m3_kernel(GemmArgs G) {
  __shared__ Stage S[2];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = wave >> 1, wn = wave & 1;   // wave's 128 x 128 quarter of the tile

  // Persistent: workgroup b takes tiles b, b + G, b + 2G, ... (G = grid
  // size, a multiple of 8), walked as one flattened sequence of (tile, K
  // step) pairs, so the next tile's first DMA streams during this tile's last
  // step and the epilogue's stores drain while the next tile computes.
  const int nb = G.tiles_m * G.tiles_n;
  const int nk = G.K / kBK;
  const int my_tiles = (nb - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int total = my_tiles * nk;
  const int g = lane >> 4;
  const int rl = lane & 15;

  // Tile order: the 8 XCDs take workgroup ids round robin, so tile t is first
  // mapped to slot (t % 8) * (n / 8) + t / 8, giving each XCD (and its L2) a
  // contiguous run of the sequence (tiles b + j G stay on b's XCD); the
  // sequence walks groups of 4 tile rows column by column, so neighbours
  // share A rows or B rows.
  auto tile_origin = [&](int t, int& m0, int& n0) {
    int pid = t;
    if (nb % 8 == 0) pid = (pid % 8) * (nb / 8) + pid / 8;
    constexpr int kGroup = 4;
    const int group = pid / (kGroup * G.tiles_n);
    const int first = group * kGroup;
    const int gsz = min(G.tiles_m - first, kGroup);
    const int in_group = pid % (kGroup * G.tiles_n);
    m0 = (first + in_group % gsz) * kBM;
    n0 = (in_group / gsz) * kBN;
  };

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // Two LDS stages. Per step: wait for the step's DMA (the only memory
  // loads in flight), barrier, issue every LDS read of the step's operands
  // and scales, then the next step's DMA into the other stage, then the 64
  // MFMAs, which consume the reads as they land. No LDS read follows a DMA in
  // program order within the step, so the compiler's wait before LDS reads
  // (any read may alias an LDS DMA in flight) never fires; the DMA overlaps
  // the MFMAs and the reads overlap the first MFMAs. The barrier also orders
  // the refill of a stage after every wave's reads of it, two steps earlier.
  int m0, n0;
  tile_origin(blockIdx.x, m0, n0);
  if (total > 0) load_stage(G, S[0], m0, n0, 0, wave, lane);
  for (int jt = 0; jt < my_tiles; ++jt) {
  for (int ks = 0; ks < nk; ++ks) {
    const int step = jt * nk + ks;
    Stage& cur = S[step & 1];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    barrier();  // every wave's share of this step is in LDS
    v8i ao[8], bo[8];
    int sav[8], sbv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rb = wn * 128 + i * 16 + rl;
      bo[i] = operand(cur.b, rb, g);
      sbv[i] = (int)((cur.sb[rb] >> (8 * g)) & 0xFFu);  // the other bytes must be zero
      const int ra = wm * 128 + i * 16 + rl;
      ao[i] = operand(cur.a, ra, g);
      sav[i] = (int)((cur.sa[ra] >> (8 * g)) & 0xFFu);
    }
    if (step + 1 < total) {
      int nm0 = m0, nn0 = n0;
      if (ks + 1 == nk) tile_origin(blockIdx.x + (jt + 1) * gridDim.x, nm0, nn0);
      load_stage(G, S[(step + 1) & 1], nm0, nn0, ks + 1 == nk ? 0 : ks + 1, wave, lane);
    }
    // the instruction computes B A^T here (B as its row operand), so that each
    // lane ends with 4 consecutive columns of C for the epilogue
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bo[j], ao[i], acc[i][j], 0, 0, 0,
                                                                     sbv[j], 0, sav[i]);
  }

    // Epilogue of the tile. acc[i][j] holds (B A^T) for B rows j*16 + 4g .. +3
    // and A row i*16 + rl: lane (rl, g) has C[row i*16 + rl][columns
    // j*16 + 4g .. +3], stored as one 8-byte (bf16) or 16-byte (fp32) store; a
    // tile wholly inside C stores without per-element checks.
    const bool full = G.vec && m0 + kBM <= G.M && n0 + kBN <= G.N;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = m0 + wm * 128 + i * 16 + rl;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col = n0 + wn * 128 + j * 16 + 4 * g;
        const v4f v = acc[i][j];
        acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        if (full || (G.vec && row < G.M && col + 3 < G.N)) {
          if (OUT_BF16) {
            const uint2 w = make_uint2((uint32_t)bf16_rne(v[0]) | ((uint32_t)bf16_rne(v[1]) << 16),
                                       (uint32_t)bf16_rne(v[2]) | ((uint32_t)bf16_rne(v[3]) << 16));
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(G.c) + (int64_t)row * G.ldc + col) = w;
          } else {
            *reinterpret_cast<float4*>(static_cast<float*>(G.c) + (int64_t)row * G.ldc + col) =
                make_float4(v[0], v[1], v[2], v[3]);
          }
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
    if (jt + 1 < my_tiles) tile_origin(blockIdx.x + (jt + 1) * gridDim.x, m0, n0);
  }
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

extern "C" mxq_status mx_gemm(const uint8_t* a, int64_t lda, const uint8_t* a_scales, int64_t ldsa,
                              const uint8_t* b, int64_t ldb, const uint8_t* b_scales, int64_t ldsb,
                              int64_t M, int64_t N, int64_t K, mxq_elem elem_a, mxq_elem elem_b,
                              void* c, int64_t ldc, mxq_out_type c_type, void* stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 32 != 0) return MXQ_ERR_SHAPE;
  if (elem_a != MXQ_E4M3 && elem_a != MXQ_E2M1) return MXQ_ERR_ARG;
  if (elem_b != MXQ_E4M3 && elem_b != MXQ_E2M1) return MXQ_ERR_ARG;
  if (c_type != MXQ_OUT_F32 && c_type != MXQ_OUT_BF16) return MXQ_ERR_ARG;
  if (lda < K || ldb < K || ldsa < K / 32 || ldsb < K / 32 || ldc < N) return MXQ_ERR_SHAPE;
  if (elem_a != MXQ_E4M3 || elem_b != MXQ_E4M3) return MXQ_ERR_UNSUPPORTED;
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
  // persistent grid: one workgroup per CU, a multiple of 8 (one per XCD
  // round-robin slot), at most one per tile
  const int nb = G.tiles_m * G.tiles_n;
  const int cus = cu_count();
  if (cus <= 0) return MXQ_ERR_HIP;
  int grid_i = nb < cus ? nb : cus;
  if (grid_i >= 8) grid_i -= grid_i % 8;
  const unsigned grid = (unsigned)grid_i;
  hipStream_t s = (hipStream_t)stream;
  if (c_type == MXQ_OUT_BF16)
    hipLaunchKernelGGL(mx_gemm_e4m3_kernel<true>, dim3(grid), dim3(kThreads), 0, s, G);
  else
    hipLaunchKernelGGL(mx_gemm_e4m3_kernel<false>, dim3(grid), dim3(kThreads), 0, s, G);
  if (hipGetLastError() != hipSuccess) return MXQ_ERR_HIP;
  return MXQ_OK;
}
