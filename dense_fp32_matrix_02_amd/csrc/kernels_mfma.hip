// FP32 matrix-core GEMM kernels for gfx950 (CDNA4): C = A.B, row-major,
// alpha = 1, beta = 0.
//
// The structure follows the pages' progression, rebuilt for 64-lane
// wavefronts and matrix cores:
//  * a workgroup owns a BM x BN tile of C and marches K in BK-deep slabs of A
//    and B (CUDA Handbook section 17.3, Figure 17-2);
//  * each slab is loaded once from global memory with coalesced 128-bit loads
//    and reused from LDS by every wave of the workgroup (ratcatcher.ru
//    "Matrix multiplication: naive and tiled", section 2; GPU Parallel Book
//    ch. 9, section 9.4), double-buffered so one barrier per slab suffices
//    where the pages need two per phase (ratcatcher page, section 2);
//  * each wave owns a register tile of (BM/WM) x (BN/WN) outputs held as
//    32x32 FP32 matrix-instruction accumulators, the wave-level analogue of
//    the per-thread register microtile (GPU Parallel Book section 9.5, and the
//    warp-level tiling and matrix instructions its section 9.7 points to);
//  * the LDS row stride of the A slab is padded by 4 floats so the rows that
//    the 32 lanes of a half-wave read fall in distinct bank groups while
//    128-bit accesses stay 16-byte aligned (the padding idea of GPU Parallel
//    Book section 9.4, re-derived for 128-bit reads).
//
// Operand layout of v_mfma_f32_32x32x2_f32 (wave64): lane l supplies
// A[m = l % 32][k = l / 32] and B[k = l / 32][n = l % 32]; accumulator
// register r of lane l holds D[m = 8*(r/4) + 4*(l/32) + r%4][n = l % 32].
// Lane l reads four consecutive k of its A row with one 128-bit LDS read, so
// four instructions u = 0..3 cover k = kk + u (lanes 0-31) and kk + 4 + u
// (lanes 32-63): eight k per group of four instructions, each B element taken
// at the same k as the A element it multiplies.
//
// Edges: rows of A beyond M are clamped to row M-1 (they only feed rows of C
// that are not stored); columns of B beyond N are loaded as zero; in the last
// slab, k >= K is loaded as zero in both operands; stores are masked to
// i < M, j < N. Global loads need only 4-byte alignment, so any leading
// dimension works.

#include "sgemm_internal.h"

namespace sgemm_impl {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// 16-byte global load that needs only 4-byte alignment (gfx950 runs in
// unaligned-access mode for global memory).
__device__ __forceinline__ f32x4 ldg4(const float* p) {
  f32x4 v;
  __builtin_memcpy(&v, p, sizeof(v));
  return v;
}

template <int BM_, int BN_, int BK_, int WM_, int WN_, int PADA_, int PADB_, int GROUP_M_>
struct MfmaCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WM = WM_, WN = WN_;          // waves along M and N
  static constexpr int PADA = PADA_, PADB = PADB_;  // LDS row padding (floats)
  static constexpr int GROUP_M = GROUP_M_;
  static constexpr int NT = 64 * WM * WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;  // 32x32 blocks per wave
  static constexpr int SA = BK + PADA;                // A slab: [BM][SA]
  static constexpr int SB = BN + PADB;                // B slab: [BK][SB]
  static constexpr int A_TPR = BK / 4;                // float4 loads per A row
  static constexpr int A_RPP = NT / A_TPR;            // A rows per pass
  static constexpr int A_PASSES = BM / A_RPP;
  static constexpr int B_TPR = BN / 4;
  static constexpr int B_RPP = NT / B_TPR;
  static constexpr int B_PASSES = BK / B_RPP;
  static constexpr int LDS_BYTES = 4 * 2 * (BM * SA + BK * SB);

  static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "wave tile must be 32x32 blocks");
  static_assert(BK % 8 == 0, "slab depth is a multiple of 8");
  static_assert(PADA % 4 == 0 && PADB % 4 == 0, "padding keeps 16-byte alignment");
  static_assert(NT % A_TPR == 0 && BM % A_RPP == 0, "A slab load shape");
  static_assert(NT % B_TPR == 0 && B_RPP <= BK && BK % B_RPP == 0, "B slab load shape");
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per CU");
};

template <class Cfg>
__global__ void __launch_bounds__(Cfg::NT) mfma_gemm_kernel(GemmArgs g) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
  constexpr int SA = Cfg::SA, SB = Cfg::SB;
  constexpr int FM = Cfg::FM, FN = Cfg::FN;
  constexpr int AP = Cfg::A_PASSES, BP = Cfg::B_PASSES;

  __shared__ __attribute__((aligned(16))) float As[2 * BM * SA];
  __shared__ __attribute__((aligned(16))) float Bs[2 * BK * SB];

  const int M = g.M, N = g.N, K = g.K;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, Cfg::GROUP_M, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x;

  // ---- global -> register loader geometry (fixed per thread) -------------
  const int a_c = t % Cfg::A_TPR;   // float4 column of the A slab row
  const int a_r = t / Cfg::A_TPR;   // first A slab row of this thread
  const float* a_src[AP];
#pragma unroll
  for (int p = 0; p < AP; ++p) {
    int row = m0 + a_r + p * Cfg::A_RPP;
    row = row < M ? row : M - 1;
    a_src[p] = g.A + (int64_t)row * g.lda + 4 * a_c;
  }
  const int b_c = t % Cfg::B_TPR;
  const int b_r = t / Cfg::B_TPR;
  const int bcol = n0 + 4 * b_c;
  const int b_valid = N - bcol;  // valid columns in this thread's float4 chunk
  const float* b_src[BP];
#pragma unroll
  for (int p = 0; p < BP; ++p)
    b_src[p] = g.B + (int64_t)(b_r + p * Cfg::B_RPP) * g.ldb + (b_valid > 0 ? bcol : 0);
  const int64_t b_step = (int64_t)BK * g.ldb;

  f32x4 ra[AP], rb[BP];

  // Load slab k0 into registers. `tail` is set only for the last slab when K
  // is not a multiple of BK: then k >= K is loaded as zero in both operands.
  auto load_slab = [&](int k0, int64_t b_off, bool tail) {
#pragma unroll
    for (int p = 0; p < AP; ++p) {
      const float* src = a_src[p] + k0;
      const int kc = k0 + 4 * a_c;
      if (!tail || kc + 3 < K) {
        ra[p] = ldg4(src);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) ra[p][e] = (kc + e < K) ? src[e] : 0.0f;
      }
    }
#pragma unroll
    for (int p = 0; p < BP; ++p) {
      const float* src = b_src[p] + b_off;
      const int kr = k0 + b_r + p * Cfg::B_RPP;
      if (tail && kr >= K) {
        rb[p] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      } else if (b_valid >= 4) {
        rb[p] = ldg4(src);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) rb[p][e] = (e < b_valid) ? src[e] : 0.0f;
      }
    }
  };

  auto store_slab = [&](int buf) {
    float* as = As + buf * (BM * SA);
    float* bs = Bs + buf * (BK * SB);
#pragma unroll
    for (int p = 0; p < AP; ++p)
      *reinterpret_cast<f32x4*>(as + (a_r + p * Cfg::A_RPP) * SA + 4 * a_c) = ra[p];
#pragma unroll
    for (int p = 0; p < BP; ++p)
      *reinterpret_cast<f32x4*>(bs + (b_r + p * Cfg::B_RPP) * SB + 4 * b_c) = rb[p];
  };

  // ---- wave tile ----------------------------------------------------------
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave % Cfg::WM, wn = wave / Cfg::WM;
  const int l32 = lane & 31, h = lane >> 5;
  const int a_frag = (wm * Cfg::WTM + l32) * SA + 4 * h;
  const int b_frag = (4 * h) * SB + wn * Cfg::WTN + l32;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto compute_slab = [&](int buf) {
    const float* as = As + buf * (BM * SA) + a_frag;
    const float* bs = Bs + buf * (BK * SB) + b_frag;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 8) {
      f32x4 af[FM];
      float bf[FN][4];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const f32x4*>(as + i * 32 * SA + kk);
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int u = 0; u < 4; ++u) bf[j][u] = bs[(kk + u) * SB + 32 * j];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][u], bf[j][u], acc[i][j], 0, 0, 0);
    }
  };

  // ---- K loop: one barrier per slab with two LDS buffers -------------------
  const int nk = (K + BK - 1) / BK;
  const bool ktail = (K % BK) != 0;
  load_slab(0, 0, ktail && nk == 1);
  store_slab(0);
  __syncthreads();
  int64_t b_off = 0;
  for (int s = 0; s < nk; ++s) {
    const bool more = s + 1 < nk;
    if (more) {
      b_off += b_step;
      load_slab((s + 1) * BK, b_off, ktail && s + 2 == nk);
    }
    compute_slab(s & 1);
    if (more) store_slab((s + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: masked stores, C is never read ----------------------------
  const int row0 = m0 + wm * Cfg::WTM + 4 * h;
  const int col0 = n0 + wn * Cfg::WTN + l32;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = col0 + 32 * j;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + 32 * i + 8 * (r >> 2) + (r & 3);
        if (row < M && col < N) g.C[(int64_t)row * g.ldc + col] = acc[i][j][r];
      }
    }
}

template <class Cfg>
hipError_t launch_mfma(const GemmArgs& g, hipStream_t stream) {
  const int64_t tiles = (int64_t)((g.M + Cfg::BM - 1) / Cfg::BM) * ((g.N + Cfg::BN - 1) / Cfg::BN);
  GemmArgs a = g;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mfma_gemm_kernel<Cfg>),
                         dim3((unsigned)tiles), dim3(Cfg::NT), args, 0, stream);
}

}  // namespace

#define SGEMM_MFMA_CFG(BM, BN, BK, WM, WN, PA, PB, G)                                     \
  {"mfma32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN, KIND_MFMA, BM, BN, BK, 64 * WM * WN, \
   &launch_mfma<MfmaCfg<BM, BN, BK, WM, WN, PA, PB, G>>}

KernelConfig kMfmaConfigs[] = {
    SGEMM_MFMA_CFG(256, 256, 16, 2, 2, 4, 4, 4),
    SGEMM_MFMA_CFG(256, 256, 32, 2, 2, 4, 4, 4),
    SGEMM_MFMA_CFG(256, 256, 16, 2, 4, 4, 4, 4),
    SGEMM_MFMA_CFG(256, 128, 16, 2, 2, 4, 4, 4),
    SGEMM_MFMA_CFG(128, 128, 16, 2, 2, 4, 4, 4),
    SGEMM_MFMA_CFG(128, 128, 32, 2, 2, 4, 4, 4),
    SGEMM_MFMA_CFG(128, 64, 16, 2, 2, 4, 4, 4),
    SGEMM_MFMA_CFG(64, 64, 16, 2, 2, 4, 4, 4),
};
const int kNumMfmaConfigs = sizeof(kMfmaConfigs) / sizeof(kMfmaConfigs[0]);

}  // namespace sgemm_impl
