// FP32 matrix-core GEMM kernels for gfx950 (CDNA4): C = A.B, row-major,
// alpha = 1, beta = 0.
//
// The structure follows the pages' progression, rebuilt for 64-lane
// wavefronts and matrix cores:
//  * a workgroup owns a BM x BN tile of C and marches K in BK-deep slabs of A
//    and B (CUDA Handbook section 17.3, Figure 17-2);
//  * each slab is loaded once from global memory with coalesced loads and
//    reused from LDS by every wave of the workgroup (ratcatcher.ru "Matrix
//    multiplication: naive and tiled", section 2; GPU Parallel Book ch. 9,
//    section 9.4), double-buffered so one barrier per slab suffices where the
//    pages need two per phase (ratcatcher page, section 2);
//  * each wave owns a register tile of (BM/WM) x (BN/WN) outputs held as
//    32x32 FP32 matrix-instruction accumulators, the wave-level analogue of
//    the per-thread register microtile (GPU Parallel Book section 9.5, and the
//    warp-level tiling and matrix instructions its section 9.7 points to);
//  * LDS rows are padded by 4 floats so the rows that the 32 lanes of a
//    half-wave read fall in distinct bank groups while 128-bit accesses stay
//    16-byte aligned (the padding idea of GPU Parallel Book section 9.4,
//    re-derived for 128-bit reads).
//
// Operand layout of v_mfma_f32_32x32x2_f32 (wave64): lane l supplies
// A[m = l % 32][k = l / 32] and B[k = l / 32][n = l % 32]; accumulator
// register r of lane l holds D[m = 8*(r/4) + 4*(l/32) + r%4][n = l % 32].
// Lane l reads four consecutive k of its A row with one 128-bit LDS read, so
// four instructions u = 0..3 cover k = kk + u (lanes 0-31) and kk + 4 + u
// (lanes 32-63): eight k per group of four instructions. Each B element is
// taken at the same k as the A element it multiplies, so the group sums
// exactly the eight products of k = kk..kk+7.
//
// Two LDS layouts of the B slab:
//  * n-major [BK][BN+4] (BKM = false): the slab is stored as it lies in
//    memory (128-bit global loads along n); a lane reads its four k values
//    with four 32-bit LDS reads of consecutive columns;
//  * k-major [BN][BK+4] (BKM = true): each lane loads four consecutive k of
//    one column with four 32-bit global loads (consecutive lanes take
//    consecutive columns, so every load instruction is one contiguous run)
//    and stores them with one 128-bit LDS write; fragments are then read
//    exactly like A's, one 128-bit LDS read per 32 columns per eight k.
//
// Edges: rows of A beyond M are clamped to row M-1 and columns of B beyond N
// are loaded as zero (n-major) or clamped to column N-1 (k-major): either way
// they only feed outputs that are not stored. In the last slab, k >= K is
// loaded as zero in both operands; that slab's load is peeled out of the main
// loop so the steady state has no K checks. Stores are masked to i < M,
// j < N. Global loads need only 4-byte alignment, so any leading dimension
// works.

#include <type_traits>

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

template <int BM_, int BN_, int BK_, int WM_, int WN_, bool BKM_, int GROUP_M_>
struct MfmaCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WM = WM_, WN = WN_;    // waves along M and N
  static constexpr bool BKM = BKM_;           // B slab k-major in LDS
  static constexpr int GROUP_M = GROUP_M_;
  static constexpr int NT = 64 * WM * WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;  // 32x32 blocks per wave
  static constexpr int SA = BK + 4;                   // A slab: [BM][SA]
  // B slab: [BK][BN+4] (n-major) or [BN][BK+4] (k-major)
  static constexpr int SB = BKM ? BK + 4 : BN + 4;
  static constexpr int B_FLOATS = BKM ? BN * SB : BK * SB;
  static constexpr int A_TPR = BK / 4;                // float4 loads per A row
  static constexpr int A_RPP = NT / A_TPR;            // A rows per pass
  static constexpr int A_PASSES = BM / A_RPP;
  // n-major B: float4 chunks along n
  static constexpr int B_TPR = BN / 4;
  static constexpr int B_RPP = NT / B_TPR;
  static constexpr int B_PASSES_N = BKM ? 1 : BK / B_RPP;
  // k-major B: each thread owns a column and groups of four k
  static constexpr int B_QPP = NT / BN;               // k-quads per pass
  static constexpr int B_PASSES_K = BKM ? (BK / 4) / B_QPP : 1;
  static constexpr int B_PASSES = BKM ? B_PASSES_K : B_PASSES_N;
  static constexpr int LDS_BYTES = 4 * 2 * (BM * SA + B_FLOATS);

  static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "wave tile must be 32x32 blocks");
  static_assert(BK % 8 == 0, "slab depth is a multiple of 8");
  static_assert(NT % A_TPR == 0 && BM % A_RPP == 0, "A slab load shape");
  static_assert(BKM || (NT % B_TPR == 0 && B_RPP <= BK && BK % B_RPP == 0), "n-major B load shape");
  static_assert(!BKM || (NT % BN == 0 && (BK / 4) % B_QPP == 0), "k-major B load shape");
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per CU");
};

template <class Cfg>
__global__ void __launch_bounds__(Cfg::NT) mfma_gemm_kernel(GemmArgs g) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
  constexpr int SA = Cfg::SA, SB = Cfg::SB;
  constexpr int FM = Cfg::FM, FN = Cfg::FN;
  constexpr int AP = Cfg::A_PASSES, BP = Cfg::B_PASSES;
  constexpr bool BKM = Cfg::BKM;

  __shared__ __attribute__((aligned(16))) float As[2 * BM * SA];
  __shared__ __attribute__((aligned(16))) float Bs[2 * Cfg::B_FLOATS];

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
  // n-major B: thread owns float4 column chunk b_c of rows b_r + p*B_RPP.
  // k-major B: thread owns column b_c = t % BN and k-quads b_r + p*B_QPP; a
  // column beyond N is clamped to N-1 (it only feeds columns of C that are
  // not stored), so the k-major loader has no per-lane branch.
  const int b_c = BKM ? t % BN : t % Cfg::B_TPR;
  const int b_r = BKM ? t / BN : t / Cfg::B_TPR;
  const int bcol = n0 + (BKM ? b_c : 4 * b_c);
  const int b_valid = N - bcol;  // n-major: valid columns of the chunk
  const int64_t ldb = g.ldb;
  const float* b_src[BP];
#pragma unroll
  for (int p = 0; p < BP; ++p) {
    const int64_t row = BKM ? 4 * (b_r + p * Cfg::B_QPP) : b_r + p * Cfg::B_RPP;
    const int col = BKM ? (bcol < N ? bcol : N - 1) : (b_valid > 0 ? bcol : 0);
    b_src[p] = g.B + row * ldb + col;
  }
  const int64_t b_step = (int64_t)BK * ldb;

  f32x4 ra[AP], rb[BP];

  // Load slab k0 into registers. The tail variant (TAIL = true) is used only
  // for the last slab when K is not a multiple of BK: k >= K then loads as
  // zero in both operands. The full variant has no K checks at all.
  auto load_slab = [&](int k0, int64_t b_off, auto tail_tag) {
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
#pragma unroll
    for (int p = 0; p < BP; ++p) {
      const float* src = b_src[p] + b_off;
      if constexpr (BKM) {
        const int kr = k0 + 4 * (b_r + p * Cfg::B_QPP);
#pragma unroll
        for (int e = 0; e < 4; ++e) rb[p][e] = (!TAIL || kr + e < K) ? src[e * ldb] : 0.0f;
      } else {
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
    }
  };
  using Full = std::integral_constant<bool, false>;
  using Tail = std::integral_constant<bool, true>;

  auto store_slab = [&](int buf) {
    float* as = As + buf * (BM * SA);
    float* bs = Bs + buf * Cfg::B_FLOATS;
#pragma unroll
    for (int p = 0; p < AP; ++p)
      *reinterpret_cast<f32x4*>(as + (a_r + p * Cfg::A_RPP) * SA + 4 * a_c) = ra[p];
#pragma unroll
    for (int p = 0; p < BP; ++p) {
      if constexpr (BKM)
        *reinterpret_cast<f32x4*>(bs + b_c * SB + 4 * (b_r + p * Cfg::B_QPP)) = rb[p];
      else
        *reinterpret_cast<f32x4*>(bs + (b_r + p * Cfg::B_RPP) * SB + 4 * b_c) = rb[p];
    }
  };

  // ---- wave tile ----------------------------------------------------------
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave % Cfg::WM, wn = wave / Cfg::WM;
  const int l32 = lane & 31, h = lane >> 5;
  const int a_frag = (wm * Cfg::WTM + l32) * SA + 4 * h;
  const int b_frag = BKM ? (wn * Cfg::WTN + l32) * SB + 4 * h : (4 * h) * SB + wn * Cfg::WTN + l32;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto compute_slab = [&](int buf) {
    const float* as = As + buf * (BM * SA) + a_frag;
    const float* bs = Bs + buf * Cfg::B_FLOATS + b_frag;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 8) {
      f32x4 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const f32x4*>(as + i * 32 * SA + kk);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (BKM) {
          bf[j] = *reinterpret_cast<const f32x4*>(bs + j * 32 * SB + kk);
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) bf[j][u] = bs[(kk + u) * SB + 32 * j];
        }
      }
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
  // Slab s+1 is loaded into registers while slab s is multiplied from LDS.
  // The last slab's load is peeled out of the loop so the steady state runs
  // the full loader only.
  const int nk = (K + BK - 1) / BK;
  const bool ktail = (K % BK) != 0;
  if (ktail && nk == 1) load_slab(0, 0, Tail{}); else load_slab(0, 0, Full{});
  store_slab(0);
  __syncthreads();
  int64_t b_off = 0;
  int s = 0;
  for (; s + 2 < nk; ++s) {
    b_off += b_step;
    load_slab((s + 1) * BK, b_off, Full{});
    // Keep the global loads ahead of the matrix instructions: without this
    // fence the scheduler may sink them next to the LDS stores that consume
    // them, exposing the whole memory latency once per slab.
    __builtin_amdgcn_sched_barrier(0);
    compute_slab(s & 1);
    store_slab((s + 1) & 1);
    __syncthreads();
  }
  if (s + 1 < nk) {
    b_off += b_step;
    if (ktail) load_slab((s + 1) * BK, b_off, Tail{}); else load_slab((s + 1) * BK, b_off, Full{});
    __builtin_amdgcn_sched_barrier(0);
    compute_slab(s & 1);
    store_slab((s + 1) & 1);
    __syncthreads();
    ++s;
  }
  compute_slab(s & 1);

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

// Name: mfma32_<BM>x<BN>x<BK>_w<WM>x<WN>, with suffix _bk when the B slab is
// stored k-major in LDS.
#define SGEMM_MFMA_CFG(BM, BN, BK, WM, WN, BKM, SUFFIX, G)                                 \
  {"mfma32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN SUFFIX, KIND_MFMA, BM, BN, BK, 64 * WM * WN, \
   &launch_mfma<MfmaCfg<BM, BN, BK, WM, WN, BKM, G>>}
#define SGEMM_MFMA_N(BM, BN, BK, WM, WN) SGEMM_MFMA_CFG(BM, BN, BK, WM, WN, false, "", 4)
#define SGEMM_MFMA_K(BM, BN, BK, WM, WN) SGEMM_MFMA_CFG(BM, BN, BK, WM, WN, true, "_bk", 4)

KernelConfig kMfmaConfigs[] = {
    // large block tiles: compute-bound squares
    SGEMM_MFMA_N(256, 256, 16, 2, 2),
    SGEMM_MFMA_N(256, 256, 32, 2, 2),
    SGEMM_MFMA_N(256, 256, 16, 2, 4),
    SGEMM_MFMA_N(256, 256, 32, 2, 4),
    SGEMM_MFMA_N(256, 256, 16, 4, 4),
    SGEMM_MFMA_N(256, 256, 32, 4, 4),
    SGEMM_MFMA_K(256, 256, 16, 2, 2),
    SGEMM_MFMA_K(256, 256, 32, 2, 2),
    SGEMM_MFMA_K(256, 256, 16, 2, 4),
    SGEMM_MFMA_N(256, 128, 16, 2, 2),
    SGEMM_MFMA_N(256, 128, 16, 2, 4),
    SGEMM_MFMA_N(256, 128, 32, 2, 4),
    SGEMM_MFMA_K(256, 128, 32, 2, 4),
    SGEMM_MFMA_N(256, 128, 16, 4, 2),
    SGEMM_MFMA_N(256, 128, 32, 4, 2),
    // medium tiles: grid fill on mid-sized and ragged problems
    SGEMM_MFMA_N(128, 128, 16, 2, 2),
    SGEMM_MFMA_N(128, 128, 32, 2, 2),
    SGEMM_MFMA_N(128, 128, 16, 2, 4),
    SGEMM_MFMA_K(128, 128, 32, 2, 2),
    SGEMM_MFMA_N(128, 64, 16, 2, 2),
    SGEMM_MFMA_N(128, 64, 32, 2, 2),
    SGEMM_MFMA_K(128, 64, 16, 2, 2),
    SGEMM_MFMA_K(128, 64, 32, 2, 2),
    // small tiles and deep slabs: few serial slab steps for small problems
    SGEMM_MFMA_N(64, 64, 16, 2, 2),
    SGEMM_MFMA_N(64, 64, 32, 2, 2),
    SGEMM_MFMA_N(64, 64, 64, 2, 2),
    SGEMM_MFMA_K(64, 64, 64, 2, 2),
    SGEMM_MFMA_N(32, 32, 32, 1, 1),
    SGEMM_MFMA_N(32, 32, 64, 1, 1),
};
const int kNumMfmaConfigs = sizeof(kMfmaConfigs) / sizeof(kMfmaConfigs[0]);

}  // namespace sgemm_impl
