// FP32 matrix-core GEMM kernels for gfx950 (CDNA4):
//   C_b = alpha * op(A_b) . op(B_b) + beta * C_b   (row-major, b < batch),
// the plain product C = A.B being alpha = 1, beta = 0, batch = 1.
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
// Each lane fetches four values u = 0..3 of its row (A) or column (B) at
// k = kk + 4*(l/32) + u, so four instructions cover k = kk..kk+7, every
// product pairing A and B at the same k.
//
// Each operand is a block of ROWS lines (BM rows of op(A), BN columns of
// op(B)) by BK values of k per slab, read from memory in one of three ways:
//  * KC, k contiguous in memory (A, or B transposed): 128-bit global loads
//    along k, LDS [ROWS][BK+4], fragments read with one 128-bit LDS read;
//  * MC, lines contiguous in memory (B, or A transposed): 128-bit global
//    loads along the lines, LDS [BK][ROWS+4], fragments read with four
//    32-bit LDS reads of consecutive lines;
//  * KM, lines contiguous in memory but staged k-major: four 32-bit global
//    loads along k (consecutive lanes take consecutive lines, so every load
//    instruction is one contiguous run), LDS [ROWS][BK+4], 128-bit fragment
//    reads.
//
// Edges: lines beyond M (or N) are clamped to the last line (KC, KM) or
// loaded as zero (MC); either way they only feed outputs that are not stored.
// In the last slab k >= K loads as zero in both operands; that slab's load is
// peeled out of the main loop so the steady state has no K checks. Stores
// are masked to i < M, j < N. Global loads need only 4-byte alignment, so any
// leading dimension works.

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

enum Layout { KC = 0, MC = 1, KM = 2 };

// A line-contiguous chunk that crosses the end of its line (valid < 4 of its
// values inside the matrix) is read as the line's last whole chunk, which ends
// at the same place, so every lane issues the same 16-byte load. This moves
// the lane's `valid` values from the end of that chunk to the front and zeroes
// the rest; valid >= 4 keeps v, valid <= 0 gives zeros. It runs when the chunk
// is stored to LDS, not after the load, so the load stays in flight during
// the slab's MFMAs.
__device__ __forceinline__ f32x4 line_end_chunk(f32x4 v, int valid) {
  f32x4 r;
  r[0] = valid >= 4 ? v[0] : valid == 3 ? v[1] : valid == 2 ? v[2] : valid == 1 ? v[3] : 0.0f;
  r[1] = valid >= 4 ? v[1] : valid == 3 ? v[2] : valid == 2 ? v[3] : 0.0f;
  r[2] = valid >= 4 ? v[2] : valid == 3 ? v[3] : 0.0f;
  r[3] = valid >= 4 ? v[3] : 0.0f;
  return r;
}

// One operand of the block tile: ROWS lines by BK values of k per slab,
// loaded by NT threads. A "line" of the loader is a row of the KC source, a
// k-row of the MC source, or a group of four k of the KM source.
template <int ROWS, int BK, int NT, int L>
struct Operand {
  static constexpr bool KMAJ = (L != MC);            // LDS [ROWS][BK+4]
  static constexpr int S = KMAJ ? BK + 4 : ROWS + 4;  // LDS row stride (floats)
  static constexpr int FLOATS = KMAJ ? ROWS * S : BK * S;
  static constexpr int TPL = (L == KC) ? BK / 4 : (L == MC ? ROWS / 4 : ROWS);  // threads per line
  static constexpr int LPP = NT / TPL;                                          // lines per pass
  static constexpr int LINES = (L == KC) ? ROWS : (L == MC ? BK : BK / 4);
  static constexpr int PASSES = (LINES + LPP - 1) / LPP;
  // When the threads do not divide the lines evenly, the last pass is partial.
  static constexpr bool PARTIAL = (LINES % LPP) != 0;
  static_assert(NT % TPL == 0 && LPP >= 1 && PASSES >= 1, "operand load shape");
  static_assert(ROWS % 32 == 0 && BK % 8 == 0, "operand tile shape");

  const float* src[PASSES];
  int64_t ld;
  int line0;  // first line of this thread
  int col;    // KC: float4 index along k; MC: float4 index along lines; KM: line
  int valid;  // MC: lines of this thread's float4 chunk that lie inside the matrix
  // MC, uniform over the workgroup: 0 when every chunk of the tile lies inside
  // the matrix, 1 when some cross its end and R >= 4 (read as the line's last
  // whole chunk), 2 when R < 4 (read value by value).
  int edge;
  f32x4 reg[PASSES];

  // base: the operand of this batch entry; r0: first line of the block tile;
  // R: number of lines of the matrix (M for A, N for B).
  __device__ __forceinline__ void init(const float* base, int64_t ld_, int r0, int R, int t) {
    ld = ld_;
    col = t % TPL;
    line0 = t / TPL;
    valid = R - (r0 + 4 * col);
    edge = r0 + ROWS <= R ? 0 : (R >= 4 ? 1 : 2);
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      int line = line0 + p * LPP;
      if (PARTIAL && line >= LINES) line = LINES - 1;  // unused slot of a partial pass
      if constexpr (L == KC) {
        int row = r0 + line;
        row = row < R ? row : R - 1;
        src[p] = base + (int64_t)row * ld + 4 * col;
      } else if constexpr (L == MC) {
        int c0 = r0 + 4 * col;
        if (valid < 4) c0 = R >= 4 ? R - 4 : (valid > 0 ? c0 : 0);
        src[p] = base + (int64_t)line * ld + c0;
      } else {
        const int c = r0 + col < R ? r0 + col : R - 1;
        src[p] = base + (int64_t)(4 * line) * ld + c;
      }
    }
  }

  // Load slab k0 into registers; TAIL zeroes k >= K (last slab only).
  template <bool TAIL>
  __device__ __forceinline__ void load(int k0, int K) {
    const int64_t koff = (L == KC) ? (int64_t)k0 : (int64_t)k0 * ld;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const float* s = src[p] + koff;
      const int line = line0 + p * LPP;
      if (PARTIAL && p == PASSES - 1 && line >= LINES) break;
      if constexpr (L == KC) {
        const int kc = k0 + 4 * col;
        if (!TAIL || kc + 3 < K) {
          reg[p] = ldg4(s);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) reg[p][e] = (kc + e < K) ? s[e] : 0.0f;
        }
      } else if constexpr (L == MC) {
        const int kr = k0 + line;
        if (TAIL && kr >= K) {
          reg[p] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        } else if (edge != 2) {
          reg[p] = ldg4(s);  // put in place by store() when edge == 1
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) reg[p][e] = (e < valid) ? s[e] : 0.0f;
        }
      } else {
        const int kr = k0 + 4 * line;
#pragma unroll
        for (int e = 0; e < 4; ++e) reg[p][e] = (!TAIL || kr + e < K) ? s[e * ld] : 0.0f;
      }
    }
  }

  __device__ __forceinline__ void store(float* lds) const {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int line = line0 + p * LPP;
      if (PARTIAL && p == PASSES - 1 && line >= LINES) break;
      float* d = (L == KM) ? lds + col * S + 4 * line : lds + line * S + 4 * col;
      if (L == MC && edge == 1) *reinterpret_cast<f32x4*>(d) = line_end_chunk(reg[p], valid);
      else *reinterpret_cast<f32x4*>(d) = reg[p];
    }
  }

  // LDS offset of the fragment of line `row` (within the tile) for lane half h.
  __device__ __forceinline__ static int frag_offset(int row, int h) {
    return KMAJ ? row * S + 4 * h : (4 * h) * S + row;
  }
  // Four k values (kk + 4h + u, u = 0..3) of one line.
  __device__ __forceinline__ static f32x4 frag(const float* lds, int kk) {
    if constexpr (KMAJ) {
      return *reinterpret_cast<const f32x4*>(lds + kk);
    } else {
      f32x4 v;
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = lds[(kk + u) * S];
      return v;
    }
  }
};

// KG > 1 splits every slab's k range among KG groups of WM x WN waves: group
// g multiplies k = g*BK/KG .. (g+1)*BK/KG - 1 of each slab into its own
// accumulators, and the groups' sums are added in ascending g through LDS at
// the end. All KG*WM*WN waves load the slabs. This keeps several waves per
// SIMD busy when the tile grid alone gives too few (small and mid-sized
// problems) without a second pass over C.
template <int BM_, int BN_, int BK_, int WM_, int WN_, int LA_, int LB_, int GROUP_M_, int KG_ = 1>
struct MfmaCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WM = WM_, WN = WN_;  // waves along M and N
  static constexpr int KG = KG_;            // wave groups sharing each slab's k range
  static constexpr int KS = BK / KG;        // k values per group per slab
  static constexpr int GROUP_M = GROUP_M_;
  static constexpr int NT = 64 * WM * WN * KG;
  static constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;  // 32x32 blocks per wave
  using OpA = Operand<BM, BK, NT, LA_>;
  using OpB = Operand<BN, BK, NT, LB_>;
  static constexpr int SLAB_FLOATS = 2 * (OpA::FLOATS + OpB::FLOATS);
  static constexpr int RED_FLOATS = (KG - 1) * BM * BN;  // partial sums of groups 1..KG-1
  static constexpr int LDS_FLOATS = SLAB_FLOATS > RED_FLOATS ? SLAB_FLOATS : RED_FLOATS;
  static constexpr int LDS_BYTES = 4 * LDS_FLOATS;
  static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "wave tile must be 32x32 blocks");
  static_assert(KS % 8 == 0 && KS * KG == BK, "each group takes whole 8-deep k steps");
  static_assert(NT <= 1024, "at most 1024 threads per workgroup");
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per CU");
};

template <class Cfg>
__global__ void __launch_bounds__(Cfg::NT) mfma_gemm_kernel(GemmArgs g) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
  constexpr int FM = Cfg::FM, FN = Cfg::FN;
  using OpA = typename Cfg::OpA;
  using OpB = typename Cfg::OpB;

  // Two slab buffers of each operand; with KG > 1 the same memory holds the
  // groups' partial sums after the last slab.
  __shared__ __attribute__((aligned(16))) float smem[Cfg::LDS_FLOATS];
  float* const As = smem;
  float* const Bs = smem + 2 * OpA::FLOATS;

  const int M = g.M, N = g.N;
  const int K = (blockIdx.y == gridDim.y - 1) ? g.k_last : g.K;  // last split-K chunk may be short
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, Cfg::GROUP_M, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int kg = Cfg::KG == 1 ? 0 : wave / (Cfg::WM * Cfg::WN);  // k group
  const int wg = wave - kg * (Cfg::WM * Cfg::WN);
  const int wm = wg % Cfg::WM, wn = wg / Cfg::WM;
  const int l32 = lane & 31, h = lane >> 5;
  // Fragment offsets include the group's first k of the slab.
  const int a_frag = OpA::frag_offset(wm * Cfg::WTM + l32, h) + kg * Cfg::KS * (OpA::KMAJ ? 1 : OpA::S);
  const int b_frag = OpB::frag_offset(wn * Cfg::WTN + l32, h) + kg * Cfg::KS * (OpB::KMAJ ? 1 : OpB::S);
  constexpr int A_BLOCK = OpA::KMAJ ? 32 * OpA::S : 32;  // offset between 32-line blocks
  constexpr int B_BLOCK = OpB::KMAJ ? 32 * OpB::S : 32;
  using Full = std::integral_constant<bool, false>;
  using Tail = std::integral_constant<bool, true>;

  {
    const int b = blockIdx.y;  // batch entry (the host launches at most kMaxGridY per grid)
    OpA opa;
    OpB opb;
    opa.init(g.A + (int64_t)b * g.strideA, g.lda, m0, M, t);
    opb.init(g.B + (int64_t)b * g.strideB, g.ldb, n0, N, t);

    auto load_slab = [&](int k0, auto tail_tag) {
      constexpr bool TAIL = decltype(tail_tag)::value;
      opa.template load<TAIL>(k0, K);
      opb.template load<TAIL>(k0, K);
    };
    auto store_slab = [&](int buf) {
      opa.store(As + buf * OpA::FLOATS);
      opb.store(Bs + buf * OpB::FLOATS);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto compute_slab = [&](int buf) {
      const float* as = As + buf * OpA::FLOATS + a_frag;
      const float* bs = Bs + buf * OpB::FLOATS + b_frag;
#pragma unroll
      for (int kk = 0; kk < Cfg::KS; kk += 8) {
        f32x4 af[FM], bf[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = OpA::frag(as + i * A_BLOCK, kk);
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[j] = OpB::frag(bs + j * B_BLOCK, kk);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][u], bf[j][u], acc[i][j], 0, 0, 0);
      }
    };

    // ---- K loop: one barrier per slab with two LDS buffers -----------------
    // Slab s+1 is loaded into registers while slab s is multiplied from LDS.
    // The last slab's load is peeled out of the loop so the steady state runs
    // the full loader only.
    const int nk = (K + BK - 1) / BK;
    const bool ktail = (K % BK) != 0;
    if (ktail && nk == 1) load_slab(0, Tail{}); else load_slab(0, Full{});
    store_slab(0);
    __syncthreads();
    int s = 0;
    for (; s + 2 < nk; ++s) {
      load_slab((s + 1) * BK, Full{});
      // Keep the global loads ahead of the matrix instructions: without this
      // fence the scheduler may sink them next to the LDS stores that consume
      // them, exposing the whole memory latency once per slab.
      __builtin_amdgcn_sched_barrier(0);
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

    // ---- k groups: add the groups' sums in ascending group order ----------
    if constexpr (Cfg::KG > 1) {
      constexpr int WAVE_FLOATS = FM * FN * 16 * 64;  // one wave's accumulators
      __syncthreads();  // every group has finished reading the slab buffers
      if (kg > 0) {
        float* red = smem + ((kg - 1) * Cfg::WM * Cfg::WN + wg) * WAVE_FLOATS + lane;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) red[((i * FN + j) * 16 + r) * 64] = acc[i][j][r];
      }
      __syncthreads();
      if (kg > 0) return;
#pragma unroll
      for (int q = 1; q < Cfg::KG; ++q) {
        const float* red = smem + ((q - 1) * Cfg::WM * Cfg::WN + wg) * WAVE_FLOATS + lane;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] += red[((i * FN + j) * 16 + r) * 64];
      }
    }

    // ---- epilogue: masked stores; C is read only when beta != 0 ------------
    float* C = g.C + (int64_t)b * g.strideC;
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
}

template <class Cfg>
hipError_t launch_mfma(const GemmArgs& g, hipStream_t stream) {
  const int64_t tiles = (int64_t)((g.M + Cfg::BM - 1) / Cfg::BM) * ((g.N + Cfg::BN - 1) / Cfg::BN);
  GemmArgs a = g;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mfma_gemm_kernel<Cfg>),
                         dim3((unsigned)tiles, (unsigned)g.batch), dim3(Cfg::NT), args, 0, stream);
}

}  // namespace

// Name: mfma32_<BM>x<BN>x<BK>_w<WM>x<WN>[_bk][_kg<KG>][_<ops>]: _bk stages B
// (read line-contiguous) k-major; _kg<KG> splits each slab's k range among KG wave
// groups (see MfmaCfg); <ops> = tn, nt or tt names transposed operands (first
// letter A, second B); no ops suffix is the plain product.
#define SGEMM_MFMA_CFG(BM, BN, BK, WM, WN, KG, GM, LA, LB, TA, TB, SUFFIX)                       \
  {"mfma32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN SUFFIX, KIND_MFMA, BM, BN, BK,                \
   64 * WM * WN * KG, TA, TB, &launch_mfma<MfmaCfg<BM, BN, BK, WM, WN, LA, LB, GM, KG>>,        \
   reinterpret_cast<const void*>(&mfma_gemm_kernel<MfmaCfg<BM, BN, BK, WM, WN, LA, LB, GM, KG>>), KG}
#define SGEMM_MFMA_N(BM, BN, BK, WM, WN) SGEMM_MFMA_CFG(BM, BN, BK, WM, WN, 1, 4, KC, MC, 0, 0, "")
#define SGEMM_MFMA_K(BM, BN, BK, WM, WN) SGEMM_MFMA_CFG(BM, BN, BK, WM, WN, 1, 4, KC, KM, 0, 0, "_bk")
#define SGEMM_MFMA_KG(BM, BN, BK, WM, WN, KG) \
  SGEMM_MFMA_CFG(BM, BN, BK, WM, WN, KG, 4, KC, MC, 0, 0, "_kg" #KG)
#define SGEMM_MFMA_OPS_SFX(BM, BN, BK, WM, WN, KG, SFX)                          \
  SGEMM_MFMA_CFG(BM, BN, BK, WM, WN, KG, 4, MC, MC, 1, 0, SFX "_tn"),            \
      SGEMM_MFMA_CFG(BM, BN, BK, WM, WN, KG, 4, KC, KC, 0, 1, SFX "_nt"),        \
      SGEMM_MFMA_CFG(BM, BN, BK, WM, WN, KG, 4, MC, KC, 1, 1, SFX "_tt")
#define SGEMM_MFMA_OPS(BM, BN, BK, WM, WN) SGEMM_MFMA_OPS_SFX(BM, BN, BK, WM, WN, 1, "")
#define SGEMM_MFMA_OPS_KG(BM, BN, BK, WM, WN, KG) SGEMM_MFMA_OPS_SFX(BM, BN, BK, WM, WN, KG, "_kg" #KG)

KernelConfig kMfmaConfigs[] = {
    // large block tiles: compute-bound squares
    SGEMM_MFMA_N(256, 256, 16, 2, 2),
    SGEMM_MFMA_N(256, 256, 16, 2, 4),
    SGEMM_MFMA_N(256, 256, 32, 2, 4),
    SGEMM_MFMA_N(256, 256, 16, 4, 4),
    SGEMM_MFMA_N(256, 256, 32, 4, 4),
    SGEMM_MFMA_K(256, 256, 16, 2, 2),
    SGEMM_MFMA_K(256, 256, 16, 2, 4),
    SGEMM_MFMA_N(256, 128, 16, 2, 2),
    SGEMM_MFMA_N(256, 128, 16, 2, 4),
    SGEMM_MFMA_N(256, 128, 32, 2, 4),
    SGEMM_MFMA_K(256, 128, 32, 2, 4),
    SGEMM_MFMA_N(256, 128, 16, 4, 2),
    SGEMM_MFMA_N(256, 128, 32, 4, 2),
    // B staged k-major with 16 waves: 128-bit fragment reads for both operands
    SGEMM_MFMA_K(256, 256, 16, 4, 4),
    SGEMM_MFMA_K(256, 128, 16, 4, 2),
    SGEMM_MFMA_K(256, 128, 32, 4, 2),
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
    // k groups: more waves per tile for grids too small to fill the chip
    SGEMM_MFMA_KG(128, 128, 32, 2, 2, 2),
    SGEMM_MFMA_KG(128, 64, 32, 2, 2, 2),
    SGEMM_MFMA_KG(64, 64, 32, 2, 2, 2),
    SGEMM_MFMA_KG(64, 64, 64, 2, 2, 2),
    SGEMM_MFMA_KG(64, 64, 64, 2, 2, 4),
    SGEMM_MFMA_KG(32, 32, 64, 1, 1, 4),
    SGEMM_MFMA_KG(32, 32, 128, 1, 1, 4),
    SGEMM_MFMA_KG(32, 32, 128, 1, 1, 8),
    SGEMM_MFMA_KG(32, 32, 64, 1, 1, 8),
    SGEMM_MFMA_KG(32, 32, 256, 1, 1, 16),
    SGEMM_MFMA_KG(64, 64, 128, 2, 2, 4),
    SGEMM_MFMA_KG(128, 64, 64, 2, 2, 4),
    // 192-row tiles: one tile per compute unit for M near 3000-3072
    SGEMM_MFMA_N(192, 128, 16, 3, 2),
    SGEMM_MFMA_KG(192, 128, 16, 3, 2, 2),
    SGEMM_MFMA_KG(192, 128, 32, 3, 2, 2),
    SGEMM_MFMA_KG(128, 192, 16, 2, 3, 2),
    SGEMM_MFMA_N(192, 64, 16, 3, 2),
    // transposed operands (op(A) = A^T and/or op(B) = B^T)
    SGEMM_MFMA_OPS(256, 128, 16, 4, 2),
    SGEMM_MFMA_OPS(128, 64, 16, 2, 2),
    // more layouts for the transposed forms: _ak stages op(A) = A^T k-major
    // (b128 fragment reads), 32-deep slabs read whole 128-byte lines of a
    // k-contiguous operand, and 256x256 tiles halve the panel re-reads
    SGEMM_MFMA_CFG(256, 128, 16, 4, 2, 1, 4, KM, MC, 1, 0, "_ak_tn"),
    SGEMM_MFMA_CFG(256, 256, 16, 4, 4, 1, 4, MC, MC, 1, 0, "_tn"),
    SGEMM_MFMA_CFG(256, 256, 16, 4, 4, 1, 4, KM, MC, 1, 0, "_ak_tn"),
    SGEMM_MFMA_CFG(256, 128, 32, 4, 2, 1, 4, KC, KC, 0, 1, "_nt"),
    SGEMM_MFMA_CFG(256, 256, 16, 4, 4, 1, 4, KC, KC, 0, 1, "_nt"),
    SGEMM_MFMA_CFG(256, 256, 32, 4, 4, 1, 4, KC, KC, 0, 1, "_nt"),
    SGEMM_MFMA_CFG(256, 128, 16, 4, 2, 1, 4, KM, KC, 1, 1, "_ak_tt"),
    SGEMM_MFMA_CFG(256, 256, 16, 4, 4, 1, 4, MC, KC, 1, 1, "_tt"),
    SGEMM_MFMA_CFG(256, 256, 16, 4, 4, 1, 4, KM, KC, 1, 1, "_ak_tt"),
    SGEMM_MFMA_CFG(256, 256, 16, 4, 4, 1, 4, KM, KM, 1, 0, "_ak_bk_tn"),
    SGEMM_MFMA_OPS_KG(64, 64, 64, 2, 2, 2),
    SGEMM_MFMA_OPS_KG(32, 32, 128, 1, 1, 4),
    SGEMM_MFMA_OPS_KG(32, 32, 256, 1, 1, 16),
};
const int kNumMfmaConfigs = sizeof(kMfmaConfigs) / sizeof(kMfmaConfigs[0]);

}  // namespace sgemm_impl
