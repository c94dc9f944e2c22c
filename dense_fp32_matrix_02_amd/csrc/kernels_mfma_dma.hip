// FP32 matrix-core GEMM kernels for gfx950 that stage the A and B slabs with
// direct global-to-LDS loads (global_load_lds_dwordx4): each lane's 16 bytes
// go from memory straight into LDS, with no register staging and no LDS store
// instructions, which frees registers and issue slots in the K loop and lets
// a third LDS stage fit next to a second workgroup on the compute unit.
//
// Computation and block structure are those of the register-staged kernels
// (a workgroup owns a BM x BN tile of C and marches K in BK-deep slabs; each
// wave owns a register tile of 32x32 matrix-instruction accumulators; CUDA
// Handbook section 17.3, GPU Parallel Book ch. 9 sections 9.4-9.7). Plain
// product only: C = alpha * A.B + beta * C, A k-contiguous, B line-contiguous.
//
// LDS layouts (unpadded):
//  * A slab [BM][BK]: row r holds k = 0..BK-1 in 16-byte chunks; chunk c is
//    stored at position c ^ swz(r), which keeps the 128-bit fragment reads of
//    eight consecutive rows in distinct banks;
//  * B slab [BK][BN]: k-row by k-row, as in memory.
// A direct load writes 64 lanes x 16 bytes to consecutive LDS addresses, so
// the lane order is chosen to fill one 1 KiB region of the layout per
// instruction; each lane fetches whichever global chunk belongs in its slot.
//
// Direct loads need 16-byte aligned global chunks that lie wholly inside the
// matrices, and cannot zero k >= K. Problems whose N or K is not a multiple
// of the tile, or whose operands are not 16-byte aligned, run a second
// instantiation that stages every slab through registers instead (same
// layouts, K tail zeroed in registers).

#include <type_traits>

#include "sgemm_internal.h"

namespace sgemm_impl {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

__device__ __forceinline__ f32x4 load16(const float* p) {
  f32x4 v;
  __builtin_memcpy(&v, p, sizeof(v));
  return v;
}

// 16-byte global -> LDS copy for one lane; `lds` must be the same for every
// lane of the wave (the hardware adds 16 * lane).
__device__ __forceinline__ void copy16_to_lds(const float* g, float* lds) {
  __builtin_amdgcn_global_load_lds((global_void*)g, (lds_void*)lds, 16, 0, 0);
}

// Wait until every vector memory load of this wave has completed (the
// direct loads count there too). Encoded s_waitcnt: vmcnt = 0, the other
// counters at their maximum (no wait).
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int BM_, int BN_, int BK_, int WM_, int WN_, int STAGES_>
struct DmaCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, STAGES = STAGES_;
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static constexpr int WTM = BM / WM, WTN = BN / WN, FM = WTM / 32, FN = WTN / 32;
  static constexpr int CPR = BK / 4;                 // 16-byte chunks per A row
  static constexpr int A_FLOATS = BM * BK, B_FLOATS = BK * BN;
  static constexpr int A_REGIONS = A_FLOATS / 256;   // 1 KiB regions per slab
  static constexpr int B_REGIONS = B_FLOATS / 256;
  static constexpr int A_PER_WAVE = A_REGIONS / NW, B_PER_WAVE = B_REGIONS / NW;
  static constexpr int A_CHUNKS = A_FLOATS / 4 / NT, B_CHUNKS = B_FLOATS / 4 / NT;  // per thread
  static constexpr int LDS_BYTES = 4 * STAGES * (A_FLOATS + B_FLOATS);
  static_assert(BK == 16 || BK == 32, "A swizzle is defined for 16- and 32-deep slabs");
  static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "wave tile must be 32x32 blocks");
  static_assert(A_REGIONS % NW == 0 && B_REGIONS % NW == 0, "whole 1 KiB regions per wave");
  static_assert((A_FLOATS / 4) % NT == 0 && (B_FLOATS / 4) % NT == 0, "whole chunks per thread");
  static_assert(BN % 4 == 0 && STAGES >= 2, "slab shape");
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per CU");
};

// Position of chunk c of A row r: rows two (BK = 16) or one (BK = 32) 128-byte
// bank spans apart get different chunk permutations.
template <int BK>
__device__ __forceinline__ int swz(int r) {
  return BK == 16 ? (r >> 1) & 3 : r & 7;
}

// DIRECT: every slab by direct loads (the launcher guarantees 16-byte aligned
// chunks, N a multiple of BN and K a multiple of BK); otherwise every slab
// through registers. Two kernels rather than a branch, so each gets the registers it
// needs.
template <class Cfg, bool DIRECT>
__global__ void __launch_bounds__(Cfg::NT) mfma_dma_kernel(GemmArgs g) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, FM = Cfg::FM, FN = Cfg::FN;
  constexpr int ST = Cfg::STAGES, CPR = Cfg::CPR;
  // One array per stage, selected at compile time: the compiler can then see
  // that a direct load into one stage does not alias reads of another, and
  // does not make those reads wait for the load.
  __shared__ __attribute__((aligned(1024))) float As0[Cfg::A_FLOATS];
  __shared__ __attribute__((aligned(1024))) float As1[Cfg::A_FLOATS];
  __shared__ __attribute__((aligned(1024))) float As2[ST > 2 ? Cfg::A_FLOATS : 4];
  __shared__ __attribute__((aligned(1024))) float Bs0[Cfg::B_FLOATS];
  __shared__ __attribute__((aligned(1024))) float Bs1[Cfg::B_FLOATS];
  __shared__ __attribute__((aligned(1024))) float Bs2[ST > 2 ? Cfg::B_FLOATS : 4];
  auto stage_a = [&](auto st) -> float* {
    if constexpr (decltype(st)::value == 0) return As0;
    else if constexpr (decltype(st)::value == 1) return As1;
    else return As2;
  };
  auto stage_b = [&](auto st) -> float* {
    if constexpr (decltype(st)::value == 0) return Bs0;
    else if constexpr (decltype(st)::value == 1) return Bs1;
    else return Bs2;
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;

  const int M = g.M, N = g.N;
  const int K = (blockIdx.y == gridDim.y - 1) ? g.k_last : g.K;  // last split-K chunk may be short
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, 4, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave % Cfg::WM, wn = wave / Cfg::WM;
  const int l32 = lane & 31, h = lane >> 5;
  const float* A = g.A + (int64_t)blockIdx.y * g.strideA;
  const float* B = g.B + (int64_t)blockIdx.y * g.strideB;


  // ---- direct-load geometry: lane slot -> global chunk --------------------
  // A region q (q = p*NW + wave) holds rows 256/BK*q ... of the slab; slot s
  // of the region is row s / CPR, stored chunk s % CPR, loaded chunk
  // (s % CPR) ^ swz(row). Rows beyond M are clamped (they feed no output).
  const float* a_src[Cfg::A_PER_WAVE];
#pragma unroll
  for (int p = 0; p < Cfg::A_PER_WAVE; ++p) {
    const int slot = (p * Cfg::NW + wave) * 64 + lane;
    const int row = slot / CPR;
    const int chunk = (slot % CPR) ^ swz<BK>(row);
    int grow = m0 + row;
    grow = grow < M ? grow : M - 1;
    a_src[p] = A + (int64_t)grow * g.lda + 4 * chunk;
  }
  // B region q holds k-rows 256/BN*q ...; slot s is k-row s / (BN/4), chunk s % (BN/4).
  const float* b_src[Cfg::B_PER_WAVE];
#pragma unroll
  for (int p = 0; p < Cfg::B_PER_WAVE; ++p) {
    const int slot = (p * Cfg::NW + wave) * 64 + lane;
    b_src[p] = B + (int64_t)(slot / (BN / 4)) * g.ldb + n0 + 4 * (slot % (BN / 4));
  }
  auto issue_direct = [&](int k0, auto stage) {
    float* as = stage_a(stage);
    float* bs = stage_b(stage);
#pragma unroll
    for (int p = 0; p < Cfg::A_PER_WAVE; ++p)
      copy16_to_lds(a_src[p] + k0, as + (p * Cfg::NW + wave) * 256);
#pragma unroll
    for (int p = 0; p < Cfg::B_PER_WAVE; ++p)
      copy16_to_lds(b_src[p] + (int64_t)k0 * g.ldb, bs + (p * Cfg::NW + wave) * 256);
  };

  // ---- register staging (edge tiles, unaligned operands, the K tail) ------
  f32x4 ra[Cfg::A_CHUNKS], rb[Cfg::B_CHUNKS];
  auto load_regs = [&](int k0, bool tail) {
#pragma unroll
    for (int c = 0; c < Cfg::A_CHUNKS; ++c) {
      const int idx = c * Cfg::NT + t;  // row idx / CPR, logical chunk idx % CPR
      int grow = m0 + idx / CPR;
      grow = grow < M ? grow : M - 1;
      const int kc = k0 + 4 * (idx % CPR);
      const float* s = A + (int64_t)grow * g.lda + kc;
      if (!tail || kc + 3 < K) {
        ra[c] = load16(s);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) ra[c][e] = (kc + e < K) ? s[e] : 0.0f;
      }
    }
#pragma unroll
    for (int c = 0; c < Cfg::B_CHUNKS; ++c) {
      const int idx = c * Cfg::NT + t;  // k-row idx / (BN/4), chunk idx % (BN/4)
      const int kr = k0 + idx / (BN / 4);
      const int col = n0 + 4 * (idx % (BN / 4));
      const int valid = N - col;
      const float* s = B + (int64_t)kr * g.ldb + (valid > 0 ? col : 0);
      if (tail && kr >= K) {
        rb[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      } else if (valid >= 4) {
        rb[c] = load16(s);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) rb[c][e] = (e < valid) ? s[e] : 0.0f;
      }
    }
  };
  auto store_regs = [&](auto stage) {
    float* as = stage_a(stage);
    float* bs = stage_b(stage);
#pragma unroll
    for (int c = 0; c < Cfg::A_CHUNKS; ++c) {
      const int idx = c * Cfg::NT + t;
      const int row = idx / CPR;
      *reinterpret_cast<f32x4*>(as + row * BK + 4 * ((idx % CPR) ^ swz<BK>(row))) = ra[c];
    }
#pragma unroll
    for (int c = 0; c < Cfg::B_CHUNKS; ++c) {
      const int idx = c * Cfg::NT + t;
      *reinterpret_cast<f32x4*>(bs + (idx / (BN / 4)) * BN + 4 * (idx % (BN / 4))) = rb[c];
    }
  };

  // ---- fragments and the inner product ------------------------------------
  // Lane (l32, h) of block row i reads A row r = wm*WTM + 32i + l32 at logical
  // chunk kk/4 + h, stored at chunk (kk/4 + h) ^ swz(r); swz(r) = swz(l32)
  // because 32i and wm*WTM are multiples of 32. kk/4 is even, so
  // (kk/4 + h) ^ swz = (kk/4) ^ (h ^ swz) and the float offset is kk ^ akey.
  const int a_row = wm * Cfg::WTM + l32;
  const int akey = 4 * (h ^ swz<BK>(l32));
  const int b_col = wn * Cfg::WTN + l32;
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto compute = [&](auto stage) {
    const float* as = stage_a(stage) + a_row * BK;
    const float* bs = stage_b(stage) + (4 * h) * BN + b_col;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 8) {
      f32x4 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const f32x4*>(as + 32 * i * BK + (kk ^ akey));
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int u = 0; u < 4; ++u) bf[j][u] = bs[(kk + u) * BN + 32 * j];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][u], bf[j][u], acc[i][j], 0, 0, 0);
    }
  };

  // ---- K loop ---------------------------------------------------------------
  const int nfull = K / BK;               // slabs with no k >= K
  const bool tail = (K % BK) != 0;
  if constexpr (DIRECT) {
    // STAGES-deep pipeline of direct loads over the full slabs: slab s+ST-1 is
    // in flight while slab s is multiplied (slab s lives in stage s % ST).
    // Each wave waits for its own loads of the next slab, then the barrier
    // publishes them to the workgroup. The loop is unrolled by ST so every
    // stage index is a constant.
    issue_direct(0, S0{});
    if (ST > 2 && nfull > 1) issue_direct(BK, S1{});
    wait_loads();
    __syncthreads();
    auto step = [&](auto cur, int s) {
      constexpr int CUR = decltype(cur)::value;
      using Next = std::integral_constant<int, (CUR + ST - 1) % ST>;
      const bool more = s + ST - 1 < nfull;
      if (more) issue_direct((s + ST - 1) * BK, Next{});
      __builtin_amdgcn_sched_barrier(0);
      compute(cur);
      if constexpr (ST == 3) {
        // Slab s+1 must have landed; slab s+2's loads may stay in flight.
        constexpr int per_slab = Cfg::A_PER_WAVE + Cfg::B_PER_WAVE;
        static_assert(per_slab <= 15, "vmcnt field");
        if (more) __builtin_amdgcn_s_waitcnt(0x0F70 | per_slab);
        else wait_loads();
      } else {
        wait_loads();
      }
      __syncthreads();
    };
    // Whole groups of ST slabs, then the remaining nfull % ST (no exit from
    // the middle of the unrolled body, so the accumulators stay in place).
    int s = 0;
    for (; s + ST <= nfull; s += ST) {
      step(S0{}, s);
      step(S1{}, s + 1);
      if constexpr (ST > 2) step(S2{}, s + 2);
    }
    if (s < nfull) step(S0{}, s);
    if (s + 1 < nfull) step(S1{}, s + 1);
  } else {
    // Register staging through stages 0 and 1, last slab peeled.
    const int nk = nfull + (tail ? 1 : 0);
    load_regs(0, tail && nk == 1);
    store_regs(S0{});
    __syncthreads();
    auto rstep = [&](auto cur, int s) {
      using Other = std::integral_constant<int, 1 - decltype(cur)::value>;
      if (s + 1 < nk) load_regs((s + 1) * BK, tail && s + 2 == nk);
      __builtin_amdgcn_sched_barrier(0);
      compute(cur);
      if (s + 1 < nk) store_regs(Other{});
      __syncthreads();
    };
    int s = 0;
    for (; s + 2 <= nk; s += 2) {
      rstep(S0{}, s);
      rstep(S1{}, s + 1);
    }
    if (s < nk) rstep(S0{}, s);
  }

  // ---- epilogue: masked stores; C is read only when beta != 0 ------------
  float* C = g.C + (int64_t)blockIdx.y * g.strideC;
  const int row0 = m0 + wm * Cfg::WTM + 4 * h;
  const int col0 = n0 + wn * Cfg::WTN + l32;
  const float alpha = g.alpha, beta = g.beta;
  auto store_tile = [&](auto op) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = col0 + 32 * j;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + 32 * i + 8 * (r >> 2) + (r & 3);
          if (row < M && col < N) op(C + (int64_t)row * g.ldc + col, acc[i][j][r]);
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

// Direct loads need every 16-byte chunk they fetch to be aligned and inside
// the matrices: A and B (and each batch entry) 16-byte aligned, leading
// dimensions multiples of 4, and no tile crossing the right edge of C. The
// direct kernel also takes K (and a short last split-K chunk) in whole slabs,
// which keeps the K tail, and its registers, out of it.
template <class Cfg>
hipError_t launch_mfma_dma(const GemmArgs& g, hipStream_t stream) {
  const int64_t tiles = (int64_t)((g.M + Cfg::BM - 1) / Cfg::BM) * ((g.N + Cfg::BN - 1) / Cfg::BN);
  const bool direct = ((reinterpret_cast<uintptr_t>(g.A) | reinterpret_cast<uintptr_t>(g.B)) & 15) == 0 &&
                      ((g.lda | g.ldb) & 3) == 0 && (g.batch <= 1 || ((g.strideA | g.strideB) & 3) == 0) &&
                      g.N % Cfg::BN == 0 && g.K % Cfg::BK == 0 && g.k_last % Cfg::BK == 0;
  GemmArgs a = g;
  void* args[] = {&a};
  const void* kernel = direct ? reinterpret_cast<const void*>(&mfma_dma_kernel<Cfg, true>)
                              : reinterpret_cast<const void*>(&mfma_dma_kernel<Cfg, false>);
  return hipLaunchKernel(kernel, dim3((unsigned)tiles, (unsigned)g.batch), dim3(Cfg::NT), args, 0, stream);
}

}  // namespace

// Name: mfma32_<BM>x<BN>x<BK>_w<WM>x<WN>_lds<STAGES>: direct global-to-LDS
// staging with STAGES LDS buffers; plain product only.
#define SGEMM_MFMA_DMA(BM, BN, BK, WM, WN, ST)                                                       \
  {"mfma32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_lds" #ST, KIND_MFMA, BM, BN, BK, 64 * WM * WN, 0, \
   0, &launch_mfma_dma<DmaCfg<BM, BN, BK, WM, WN, ST>>}

KernelConfig kMfmaDmaConfigs[] = {
    // 256x256 block tile, 16 waves of 64x64, two stages: one workgroup per CU
    SGEMM_MFMA_DMA(256, 256, 16, 4, 4, 2),
};
const int kNumMfmaDmaConfigs = sizeof(kMfmaDmaConfigs) / sizeof(kMfmaDmaConfigs[0]);

}  // namespace sgemm_impl
