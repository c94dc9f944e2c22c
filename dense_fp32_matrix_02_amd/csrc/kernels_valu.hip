// Vector-FMA comparison GEMM kernel for gfx950: C = A.B, row-major FP32,
// alpha = 1, beta = 0, computed with plain FP32 fused multiply-adds on the
// vector ALUs instead of the matrix cores.
//
// It is the register-tiled kernel of the pages rebuilt for 64-lane waves:
// each thread owns an 8x8 microtile of C in registers (the 8x8 microtile the
// CUDA Handbook section 17.3 found best; the RM x RN register tile of GPU
// Parallel Book ch. 9, section 9.5) and the workgroup stages BK-deep slabs of
// A and B through double-buffered LDS (ratcatcher.ru "Matrix multiplication:
// naive and tiled", section 2; GPU Parallel Book section 9.4). Per k a thread
// reads 8 values of A and 8 of B (four 128-bit LDS reads) and performs 64
// FMAs from registers. A is stored k-major in LDS ([BK][BM+4]) so a thread's
// rows are contiguous; the thread's rows are split in two groups of four,
// half a tile apart, and so are its columns, which keeps every 128-bit LDS
// read either a broadcast or part of a contiguous run.
//
// Edge rules are those of the matrix-core kernels: rows of A beyond M are
// clamped, columns of B beyond N and k >= K in the last slab load as zero,
// stores are masked to i < M, j < N.

#include "sgemm_internal.h"

namespace sgemm_impl {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 ldg4(const float* p) {
  f32x4 v;
  __builtin_memcpy(&v, p, sizeof(v));
  return v;
}

template <int BM_, int BN_, int BK_, int GROUP_M_>
struct ValuCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, GROUP_M = GROUP_M_;
  static constexpr int TM = 8, TN = 8;           // microtile per thread
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
  static_assert(NT % 64 == 0, "whole wavefronts");
  static_assert(NT % A_TPR == 0 && BM % A_RPP == 0, "A slab load shape");
  static_assert(NT % B_TPR == 0 && B_RPP <= BK && BK % B_RPP == 0, "B slab load shape");
  static_assert(4 * 2 * BK * (SA + SB) <= 160 * 1024, "LDS budget");
};

template <class Cfg>
__global__ void __launch_bounds__(Cfg::NT) valu_gemm_kernel(GemmArgs g) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
  constexpr int SA = Cfg::SA, SB = Cfg::SB;
  constexpr int AP = Cfg::A_PASSES, BP = Cfg::B_PASSES;

  __shared__ __attribute__((aligned(16))) float As[2 * BK * SA];
  __shared__ __attribute__((aligned(16))) float Bs[2 * BK * SB];

  const int M = g.M, N = g.N, K = g.K;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, Cfg::GROUP_M, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x;

  {
  const int bb = blockIdx.y;  // batch entry (the host launches at most kMaxGridY per grid)
  const float* A = g.A + (int64_t)bb * g.strideA;
  const float* B = g.B + (int64_t)bb * g.strideB;
  float* C = g.C + (int64_t)bb * g.strideC;
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
  const int64_t b_step = (int64_t)BK * g.ldb;
  f32x4 ra[AP], rb[BP];

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

  const int tx = t % Cfg::TX, ty = t / Cfg::TX;
  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

  auto compute_slab = [&](int buf) {
    const float* as = As + buf * (BK * SA) + 4 * ty;
    const float* bs = Bs + buf * (BK * SB) + 4 * tx;
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(as + k * SA);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(as + k * SA + BM / 2);
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(bs + k * SB);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(bs + k * SB + BN / 2);
      const float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      const float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
  };

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

  const float alpha = g.alpha, beta = g.beta;
  const bool plain = (alpha == 1.0f && beta == 0.0f);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = m0 + (i < 4 ? 4 * ty + i : BM / 2 + 4 * ty + (i - 4));
    if (row >= M) continue;
    float* crow = C + (int64_t)row * g.ldc;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = n0 + (j < 4 ? 4 * tx + j : BN / 2 + 4 * tx + (j - 4));
      if (col < N) {
        if (plain) {
          crow[col] = acc[i][j];
        } else {
          const float v = alpha * acc[i][j];
          crow[col] = (beta != 0.0f) ? __builtin_fmaf(beta, crow[col], v) : v;
        }
      }
    }
  }
  }
}

template <class Cfg>
hipError_t launch_valu(const GemmArgs& g, hipStream_t stream) {
  const int64_t tiles = (int64_t)((g.M + Cfg::BM - 1) / Cfg::BM) * ((g.N + Cfg::BN - 1) / Cfg::BN);
  GemmArgs a = g;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&valu_gemm_kernel<Cfg>),
                         dim3((unsigned)tiles, (unsigned)g.batch), dim3(Cfg::NT), args, 0, stream);
}

// C_b = beta * C_b over the M x N block of every batch entry: the result
// when K == 0 (the empty sum) or alpha == 0. beta == 0 writes +0 without
// reading C. A plain kernel rather than a memset so the call stays safe
// inside captured graphs.
__global__ void __launch_bounds__(256) scale_c_kernel(GemmArgs g) {
  const int64_t total = (int64_t)g.M * g.N;
  {
  const int bb = blockIdx.y;  // batch entry (the host launches at most kMaxGridY per grid)
    float* C = g.C + (int64_t)bb * g.strideC;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
      const int64_t i = e / g.N, j = e - i * g.N;
      float* p = C + i * g.ldc + j;
      *p = (g.beta != 0.0f) ? g.beta * *p : 0.0f;
    }
  }
}

}  // namespace

hipError_t launch_scale_c(const GemmArgs& g, hipStream_t stream) {
  const int64_t total = (int64_t)g.M * g.N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  GemmArgs a = g;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&scale_c_kernel), dim3((unsigned)blocks, (unsigned)g.batch),
                         dim3(256), args, 0, stream);
}

#define SGEMM_VALU_CFG(BM, BN, BK, G)                                                  \
  {"valu8x8_" #BM "x" #BN "x" #BK, KIND_VALU, BM, BN, BK, (BM / 8) * (BN / 8), 0, 0, \
   &launch_valu<ValuCfg<BM, BN, BK, G>>}

KernelConfig kValuConfigs[] = {
    SGEMM_VALU_CFG(128, 128, 8, 4),
    SGEMM_VALU_CFG(128, 128, 16, 4),
    SGEMM_VALU_CFG(64, 64, 16, 4),
};
const int kNumValuConfigs = sizeof(kValuConfigs) / sizeof(kValuConfigs[0]);

}  // namespace sgemm_impl
