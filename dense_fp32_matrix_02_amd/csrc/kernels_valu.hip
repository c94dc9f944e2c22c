// Vector-FMA comparison GEMM kernel for gfx950:
//   C_b = alpha * A_b . B_b + beta * C_b   (row-major FP32, b = blockIdx.y),
// computed with plain FP32 fused multiply-adds on the vector ALUs instead of
// the matrix cores.
//
// It is the register-tiled kernel of the pages rebuilt for 64-lane waves:
// each thread owns a TM x 8 microtile of C in registers (the 8x8 microtile
// the CUDA Handbook section 17.3 found best; the RM x RN register tile of GPU
// Parallel Book ch. 9, section 9.5) and the workgroup stages BK-deep slabs of
// A and B through double-buffered LDS (ratcatcher.ru "Matrix multiplication:
// naive and tiled", section 2; GPU Parallel Book section 9.4). Per k a thread
// reads TM values of A and 8 of B with 128-bit LDS reads and performs TM*8
// FMAs from registers. A is stored k-major in LDS ([BK][BM+4]) so a thread's
// rows are contiguous; the thread's rows are split in groups of four spread
// across the tile, and so are its columns, which keeps every 128-bit LDS read
// either a broadcast or part of a contiguous run. The FMAs are the VOP2
// accumulate form v_fmac_f32 with vector operands, which gfx950 issues at
// the full FP32 vector rate.
//
// Edge rules are those of the matrix-core kernels: rows of A beyond M are
// clamped, columns of B beyond N and k >= K in the last slab load as zero,
// stores are masked to i < M, j < N; the last slab's load is peeled out of
// the main loop.

#include <type_traits>

#include "sgemm_internal.h"

namespace sgemm_impl {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 ldg4(const float* p) {
  f32x4 v;
  __builtin_memcpy(&v, p, sizeof(v));
  return v;
}

template <int BM_, int BN_, int BK_, int TM_, int GROUP_M_, int WAVES_>
struct ValuCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, GROUP_M = GROUP_M_;
  // Minimum waves per SIMD the register allocation must allow (the occupancy
  // bound GPU Parallel Book section 9.6 sweeps with __launch_bounds__).
  static constexpr int WAVES = WAVES_;
  static constexpr int TM = TM_, TN = 8;         // microtile per thread
  static constexpr int RG = TM / 4, CG = TN / 4;  // groups of four rows / columns
  static constexpr int TX = BN / TN, TY = BM / TM;
  static constexpr int NT = TX * TY;
  static constexpr int SA = BM + 4;              // A slab, k-major: [BK][SA]
  static constexpr int SB = BN + 4;              // B slab: [BK][SB]
  static constexpr int A_TPR = BK / 4;
  static constexpr int A_RPP = NT / A_TPR;
  static constexpr int A_PASSES = BM / A_RPP;
  static constexpr int B_TPR = BN / 4;
  static constexpr int B_RPP = NT / B_TPR;
  static constexpr int B_PASSES = BK / B_RPP;
  static_assert(TM % 4 == 0 && NT % 64 == 0, "whole wavefronts, rows in groups of four");
  static_assert(NT % A_TPR == 0 && BM % A_RPP == 0, "A slab load shape");
  static_assert(NT % B_TPR == 0 && B_RPP <= BK && BK % B_RPP == 0, "B slab load shape");
  static_assert(4 * 2 * BK * (SA + SB) <= 160 * 1024, "LDS budget");
};

template <class Cfg>
__global__ void __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(Cfg::WAVES)))
valu_gemm_kernel(GemmArgs g) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
  constexpr int SA = Cfg::SA, SB = Cfg::SB;
  constexpr int AP = Cfg::A_PASSES, BP = Cfg::B_PASSES;
  constexpr int TM = Cfg::TM, TN = Cfg::TN, RG = Cfg::RG, CG = Cfg::CG;

  __shared__ __attribute__((aligned(16))) float As[2 * BK * SA];
  __shared__ __attribute__((aligned(16))) float Bs[2 * BK * SB];

  const int M = g.M, N = g.N;
  const int K = (blockIdx.y == gridDim.y - 1) ? g.k_last : g.K;  // last split-K chunk may be short
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, Cfg::GROUP_M, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x;
  const int b = blockIdx.y;  // batch entry (the host launches at most kMaxGridY per grid)
  const float* A = g.A + (int64_t)b * g.strideA;
  const float* B = g.B + (int64_t)b * g.strideB;
  float* C = g.C + (int64_t)b * g.strideC;

  // ---- global -> register loader geometry --------------------------------
  const int a_c = t % Cfg::A_TPR, a_r = t / Cfg::A_TPR;
  const float* a_src[AP];
#pragma unroll
  for (int p = 0; p < AP; ++p) {
    int row = m0 + a_r + p * Cfg::A_RPP;
    row = row < M ? row : M - 1;
    a_src[p] = A + (int64_t)row * g.lda + 4 * a_c;
  }
  const int b_c = t % Cfg::B_TPR, b_r = t / Cfg::B_TPR;
  const int bcol = n0 + 4 * b_c;
  const int b_valid = N - bcol;
  const float* b_src[BP];
#pragma unroll
  for (int p = 0; p < BP; ++p)
    b_src[p] = B + (int64_t)(b_r + p * Cfg::B_RPP) * g.ldb + (b_valid > 0 ? bcol : 0);
  f32x4 ra[AP], rb[BP];

  auto load_slab = [&](int k0, auto tail_tag) {
    constexpr bool TAIL = decltype(tail_tag)::value;
#pragma unroll
    for (int p = 0; p < AP; ++p) {
      const float* src = a_src[p] + k0;
      const int kc = k0 + 4 * a_c;
      if (!TAIL || kc + 3 < K) {
        ra[p] = ldg4(src);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) ra[p][e] = (kc + e < K) ? src[e] : 0.0f;
      }
    }
    const int64_t b_off = (int64_t)k0 * g.ldb;
#pragma unroll
    for (int p = 0; p < BP; ++p) {
      const float* src = b_src[p] + b_off;
      const int kr = k0 + b_r + p * Cfg::B_RPP;
      if (TAIL && kr >= K) {
        rb[p] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      } else if (b_valid >= 4) {
        rb[p] = ldg4(src);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) rb[p][e] = (e < b_valid) ? src[e] : 0.0f;
      }
    }
  };
  using Full = std::integral_constant<bool, false>;
  using Tail = std::integral_constant<bool, true>;

  auto store_slab = [&](int buf) {
    float* as = As + buf * (BK * SA);
    float* bs = Bs + buf * (BK * SB);
#pragma unroll
    for (int p = 0; p < AP; ++p)
#pragma unroll
      for (int e = 0; e < 4; ++e) as[(4 * a_c + e) * SA + a_r + p * Cfg::A_RPP] = ra[p][e];
#pragma unroll
    for (int p = 0; p < BP; ++p)
      *reinterpret_cast<f32x4*>(bs + (b_r + p * Cfg::B_RPP) * SB + 4 * b_c) = rb[p];
  };

  // ---- microtile: rows 4*ty + (BM/RG)*rg + 0..3, columns 4*tx + (BN/CG)*cg + 0..3
  const int tx = t % Cfg::TX, ty = t / Cfg::TX;
  float acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;

  auto compute_slab = [&](int buf) {
    const float* as = As + buf * (BK * SA) + 4 * ty;
    const float* bs = Bs + buf * (BK * SB) + 4 * tx;
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float a[TM], bb[TN];
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(as + k * SA + rg * (BM / RG));
#pragma unroll
        for (int e = 0; e < 4; ++e) a[4 * rg + e] = v[e];
      }
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(bs + k * SB + cg * (BN / CG));
#pragma unroll
        for (int e = 0; e < 4; ++e) bb[4 * cg + e] = v[e];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_fmaf(a[i], bb[j], acc[i][j]);
    }
  };

  // ---- K loop (same structure as the matrix-core kernels) -----------------
  const int nk = (K + BK - 1) / BK;
  const bool ktail = (K % BK) != 0;
  if (ktail && nk == 1) load_slab(0, Tail{}); else load_slab(0, Full{});
  store_slab(0);
  __syncthreads();
  int s = 0;
  for (; s + 2 < nk; ++s) {
    load_slab((s + 1) * BK, Full{});
    __builtin_amdgcn_sched_barrier(0);  // keep the next slab's loads ahead of the FMAs
    compute_slab(s & 1);
    store_slab((s + 1) & 1);
    __syncthreads();
  }
  if (s + 1 < nk) {
    if (ktail) load_slab((s + 1) * BK, Tail{}); else load_slab((s + 1) * BK, Full{});
    __builtin_amdgcn_sched_barrier(0);
    compute_slab(s & 1);
    store_slab((s + 1) & 1);
    __syncthreads();
    ++s;
  }
  compute_slab(s & 1);

  // ---- epilogue --------------------------------------------------------------
  const float alpha = g.alpha, beta = g.beta;
  auto store_tile = [&](auto op) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = m0 + 4 * ty + (i / 4) * (BM / RG) + (i % 4);
      if (row >= M) continue;
      float* crow = C + (int64_t)row * g.ldc;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = n0 + 4 * tx + (j / 4) * (BN / CG) + (j % 4);
        if (col < N) op(crow + col, acc[i][j]);
      }
    }
  };
  if (alpha == 1.0f && beta == 0.0f)
    store_tile([](float* p, float v) { *p = v; });
  else if (beta == 0.0f)
    store_tile([alpha](float* p, float v) { *p = alpha * v; });
  else
    store_tile([alpha, beta](float* p, float v) { *p = __builtin_fmaf(beta, *p, alpha * v); });
}

template <class Cfg>
hipError_t launch_valu(const GemmArgs& g, hipStream_t stream) {
  const int64_t tiles = (int64_t)((g.M + Cfg::BM - 1) / Cfg::BM) * ((g.N + Cfg::BN - 1) / Cfg::BN);
  GemmArgs a = g;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&valu_gemm_kernel<Cfg>),
                         dim3((unsigned)tiles, (unsigned)g.batch), dim3(Cfg::NT), args, 0, stream);
}

}  // namespace

// Name: valu<TM>x8_<BM>x<BN>x<BK>[_o<W>]: microtile TM x 8 per thread, block
// tile BM x BN, registers bounded for at least W waves per SIMD (default 1).
#define SGEMM_VALU_CFG(BM, BN, BK, TM, W, SUFFIX)                                                        \
  {"valu" #TM "x8_" #BM "x" #BN "x" #BK SUFFIX, KIND_VALU, BM, BN, BK, (BM / TM) * (BN / 8), 0, 0, \
   &launch_valu<ValuCfg<BM, BN, BK, TM, 4, W>>,                                                        \
   reinterpret_cast<const void*>(&valu_gemm_kernel<ValuCfg<BM, BN, BK, TM, 4, W>>), 1}

KernelConfig kValuConfigs[] = {
    SGEMM_VALU_CFG(128, 128, 8, 8, 1, ""),
    SGEMM_VALU_CFG(128, 128, 8, 8, 5, "_o5"),
    SGEMM_VALU_CFG(128, 128, 16, 8, 1, ""),
    SGEMM_VALU_CFG(128, 128, 16, 8, 4, "_o4"),
    SGEMM_VALU_CFG(64, 64, 16, 8, 1, ""),
    SGEMM_VALU_CFG(256, 128, 8, 16, 1, ""),
    SGEMM_VALU_CFG(256, 128, 8, 16, 3, "_o3"),
};
const int kNumValuConfigs = sizeof(kValuConfigs) / sizeof(kValuConfigs[0]);

}  // namespace sgemm_impl
