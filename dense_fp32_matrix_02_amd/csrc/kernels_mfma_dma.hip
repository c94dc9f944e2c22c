// FP32 matrix-core GEMM kernels for gfx950 that stage the A and B slabs with
// direct global-to-LDS loads (global_load_lds_dwordx4): each lane's 16 bytes
// go from memory straight into LDS, with no register staging and no LDS store
// instructions, which frees registers and issue slots in the K loop.
//
// Computation and block structure are those of the register-staged kernels
// (a workgroup owns a BM x BN tile of C and marches K in BK-deep slabs; each
// wave owns a register tile of 32x32 matrix-instruction accumulators; CUDA
// Handbook section 17.3, GPU Parallel Book ch. 9 sections 9.4-9.7), for
// C = alpha * op(A).op(B) + beta * C with op(X) = X or X^T.
//
// Each operand's slab has one of two LDS layouts, fixed by how the operand
// lies in memory. Its "lines" are the rows of op(A) or the columns of op(B):
//  * k-contiguous lines (A, and B^T): slab [ROWS][BK], 16-byte chunk c of
//    line r stored at chunk position c ^ swz(r), which keeps the 128-bit
//    fragment reads of eight consecutive lines in distinct banks;
//  * line-contiguous k-rows (B, and A^T): slab [BK][ROWS], as in memory;
//    fragments are four 32-bit reads of consecutive lines.
// A direct load writes 64 lanes x 16 bytes to consecutive LDS addresses, so
// the lane order is chosen to fill one 1 KiB region of the layout per
// instruction; each lane fetches whichever global chunk belongs in its slot.
//
// Direct loads need 16-byte aligned global chunks that lie wholly inside the
// matrices, and cannot zero k >= K. Lines past the edge of C are clamped to
// the last line (or the last whole chunk of lines), which feeds only outputs
// that are never stored. When K is not a whole number of slabs, a third
// instantiation loads the whole slabs directly and stages only the last,
// partial one through registers. Misaligned operands run an instantiation
// that stages every slab through registers (same layouts, edges and K tail
// zeroed in registers).

#include <type_traits>
#include <utility>

#include "sgemm_internal.h"

namespace sgemm_impl {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// A line-contiguous chunk that crosses the end of its line (valid < 4 of its
// values inside the matrix) is read as the line's last whole chunk, which ends
// at the same place. This moves the lane's `valid` values from the end of that
// chunk to the front and zeroes the rest; valid >= 4 keeps v, valid <= 0
// gives zeros. It runs when the chunk is stored to LDS, so the load stays in
// flight until then.
// Written as single selects of plain values: nested conditionals on vector
// elements compiled to divergent branches.
__device__ __forceinline__ f32x4 line_end_chunk(f32x4 v, int valid) {
  const float v0 = v[0], v1 = v[1], v2 = v[2], v3 = v[3];
  float r0 = 0.0f, r1 = 0.0f, r2 = 0.0f, r3 = 0.0f;
  r0 = valid == 1 ? v3 : r0;
  r0 = valid == 2 ? v2 : r0;
  r1 = valid == 2 ? v3 : r1;
  r0 = valid == 3 ? v1 : r0;
  r1 = valid == 3 ? v2 : r1;
  r2 = valid == 3 ? v3 : r2;
  r0 = valid >= 4 ? v0 : r0;
  r1 = valid >= 4 ? v1 : r1;
  r2 = valid >= 4 ? v2 : r2;
  r3 = valid >= 4 ? v3 : r3;
  return f32x4{r0, r1, r2, r3};
}

// f(std::integral_constant<int, i>{}) for i = 0 .. N-1, unrolled at compile time.
template <class F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

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
// The s_waitcnt immediate that waits until at most n (< 64) vector memory
// loads of this wave are in flight: vmcnt's low four bits sit in bits 3:0 of
// the immediate and its high two in bits 15:14.
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Position of chunk c of a k-contiguous line r is c ^ swz(r). gfx950's LDS
// has 64 four-byte banks and serves a 128-bit read 16 lanes at a time, so
// the 16 consecutive lines that 16 lanes read at one logical chunk must fall
// in 16 different four-bank groups. A line of BK floats starts at bank
// (r * BK) mod 64: with BK = 16 lines r and r + 4 start at the same bank, so
// the chunk permutation changes with r / 4; with BK = 32, with r / 2; with
// BK >= 64 every line starts at bank 0, so it changes with r. (Counter probe
// of these read patterns: 4 LDS cycles per 64-lane 128-bit read with these
// permutations, 8 with the permutation of every second line.)
template <int BK>
__device__ __forceinline__ int swz(int r) {
  return BK == 16 ? (r >> 2) & 3 : BK == 32 ? (r >> 1) & 7 : r & 15;
}

// One operand's slab: ROWS lines by BK k values, staged by NW waves.
// KCONTIG: the operand's lines are k-contiguous in memory (layout [ROWS][BK],
// swizzled); otherwise its k-rows are line-contiguous (layout [BK][ROWS]).
// X, ld: the stored matrix and its leading dimension; line0: first line of
// the tile; extent: lines that exist (M for op(A), N for op(B)).
template <int ROWS, int BK, bool KCONTIG, int NW>
struct Slab {
  static constexpr int NT = 64 * NW;
  static constexpr int FLOATS = ROWS * BK;
  static constexpr int REGIONS = FLOATS / 256;         // 1 KiB regions per slab
  static constexpr int PER_WAVE = REGIONS / NW;        // direct loads per wave per slab
  static constexpr int CHUNKS = FLOATS / 4 / NT;       // register-staged chunks per thread
  static constexpr int CPL = KCONTIG ? BK / 4 : ROWS / 4;  // 16-byte chunks per LDS row
  static constexpr bool KC = KCONTIG;
  static_assert(!KCONTIG || BK == 16 || BK % 32 == 0, "swizzle is defined for 16-deep and 32k-deep slabs");
  static_assert(ROWS % 32 == 0 && REGIONS % NW == 0, "whole 1 KiB regions per wave");
  static_assert((FLOATS / 4) % NT == 0, "whole chunks per thread");

  // Global chunk that fills LDS slot `slot` (of 16 bytes) of the slab at k = 0.
  // Direct loads only: the launcher guarantees 16-byte aligned chunks and, for
  // line-contiguous operands, extent a multiple of 4.
  __device__ static const float* direct_src(const float* X, int64_t ld, int line0, int extent, int slot) {
    if constexpr (KCONTIG) {
      const int r = slot / CPL;
      const int chunk = (slot % CPL) ^ swz<BK>(r);
      int line = line0 + r;
      line = line < extent ? line : extent - 1;
      return X + (int64_t)line * ld + 4 * chunk;
    } else {
      int col = line0 + 4 * (slot % CPL);
      col = col <= extent - 4 ? col : extent - 4;
      return X + (int64_t)(slot / CPL) * ld + col;
    }
  }
  // Register staging without branches, for the hand-ordered loop (whole
  // slabs; a line-contiguous operand's lines at least 4 values long). Chunk
  // idx of the slab at k = 0 is read from chunk_src: k-contiguous lines past
  // the extent repeat the last line, and a line-contiguous chunk that crosses
  // the end of the lines is read as the line's last whole chunk, which ends
  // where the lines end. store_chunk writes every chunk to its own slot with
  // one 128-bit write, so in a slot whose chunk crossed the end, line c of the
  // tile sits read_fix(c) floats after c; the fragment reads add that offset
  // (the slot's other floats feed only outputs that are never stored). The
  // LDS layout is otherwise that of store().
  __device__ static const float* chunk_src(const float* X, int64_t ld, int line0, int extent, int idx) {
    if constexpr (KCONTIG) {
      int line = line0 + idx / CPL;
      line = line < extent ? line : extent - 1;
      return X + (int64_t)line * ld + 4 * (idx % CPL);
    } else {
      const int col = line0 + 4 * (idx % CPL);
      return X + (int64_t)(idx / CPL) * ld + (col <= extent - 4 ? col : extent - 4);
    }
  }
  // Where line c of the tile (0 <= c < ROWS) sits in the slot chunk_src
  // filled, relative to c: a chunk with 1 to 3 lines left before the extent
  // was read starting 4 - valid lines early. Lines past the extent keep 0,
  // so every read stays inside its own slot.
  __device__ static int read_fix(int line0, int extent, int c) {
    if constexpr (KCONTIG) return 0;
    const int valid = extent - (line0 + (c & ~3));
    return valid >= 1 && valid <= 3 && (c & 3) < valid ? 4 - valid : 0;
  }
  __device__ static void store_chunk(float* lds, f32x4 v, int idx) {
    if constexpr (KCONTIG) {
      const int line = idx / CPL;
      *reinterpret_cast<f32x4*>(lds + line * BK + 4 * ((idx % CPL) ^ swz<BK>(line))) = v;
    } else {
      *reinterpret_cast<f32x4*>(lds + (idx / CPL) * ROWS + 4 * (idx % CPL)) = v;
    }
  }
  // Offset of the slab at k0 from the slab at k = 0.
  __device__ static int64_t k_offset(int k0, int64_t ld) {
    if constexpr (KCONTIG) return k0;
    else return (int64_t)k0 * ld;
  }

  // Register staging: this thread's chunks of the slab at k0; with `tail`,
  // k >= K reads as zero. Lines past the extent read as zero or repeat the
  // last line (outputs that are never stored).
  __device__ static void load(f32x4 (&r)[CHUNKS], const float* X, int64_t ld, int line0, int extent,
                              int K, int k0, bool tail, int t) {
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
      const int idx = c * NT + t;
      if constexpr (KCONTIG) {  // line idx / CPL, logical chunk idx % CPL
        int line = line0 + idx / CPL;
        line = line < extent ? line : extent - 1;
        const int kc = k0 + 4 * (idx % CPL);
        const float* s = X + (int64_t)line * ld + kc;
        if (!tail || kc + 3 < K) {
          r[c] = load16(s);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) r[c][e] = (kc + e < K) ? s[e] : 0.0f;
        }
      } else {  // k-row idx / CPL, chunk idx % CPL
        const int kr = k0 + idx / CPL;
        const int col = line0 + 4 * (idx % CPL);
        const int valid = extent - col;
        // In a tile that crosses the end of the lines (and lines of at least
        // 4 values), a chunk that crosses it is read as the line's last whole
        // chunk, so every lane issues one 16-byte load; store() puts the
        // lane's values in place.
        const bool inside = line0 + ROWS <= extent;
        const int c0 = (valid >= 4 || inside) ? col : (extent >= 4 ? extent - 4 : (valid > 0 ? col : 0));
        const float* s = X + (int64_t)kr * ld + c0;
        if (tail && kr >= K) {
          r[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        } else if (inside || extent >= 4) {
          r[c] = load16(s);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) r[c][e] = (e < valid) ? s[e] : 0.0f;
        }
      }
    }
  }
  // line0 and extent as given to load().
  __device__ static void store(float* lds, const f32x4 (&r)[CHUNKS], int line0, int extent, int t) {
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
      const int idx = c * NT + t;
      if constexpr (KCONTIG) {
        const int line = idx / CPL;
        *reinterpret_cast<f32x4*>(lds + line * BK + 4 * ((idx % CPL) ^ swz<BK>(line))) = r[c];
      } else {
        float* d = lds + (idx / CPL) * ROWS + 4 * (idx % CPL);
        if (line0 + ROWS > extent && extent >= 4)
          *reinterpret_cast<f32x4*>(d) = line_end_chunk(r[c], extent - (line0 + 4 * (idx % CPL)));
        else
          *reinterpret_cast<f32x4*>(d) = r[c];
      }
    }
  }

  // Fragments. Lane (l32, h) of line block i reads line `line_w + 32 i + l32`
  // at k = kk + 4h + u, u = 0..3. For k-contiguous lines that is logical chunk
  // kk/4 + h, stored at (kk/4 + h) ^ swz(l32) (line_w and 32 i are multiples
  // of 32, and swz depends on the line modulo 32); kk/4 is even, so the float
  // offset is kk ^ key, key = 4 (h ^ swz). A k group's first k of the slab,
  // a multiple of 32 that kk never reaches, is XORed into the key the same way.
  __device__ static const float* frag_base(const float* lds, int line_w, int l32, int h) {
    if constexpr (KCONTIG) return lds + (line_w + l32) * BK;
    else return lds + 4 * h * ROWS + line_w + l32;
  }
  __device__ static int frag_key(int l32, int h) { return KCONTIG ? 4 * (h ^ swz<BK>(l32)) : 0; }
  // fix: read_fix of the lane's line in block i, for slabs stored by store_chunk.
  __device__ static f32x4 frag(const float* base, int i, int kk, int key, int fix = 0) {
    if constexpr (KCONTIG) {
      return *reinterpret_cast<const f32x4*>(base + 32 * i * BK + (kk ^ key));
    } else {
      f32x4 v;
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = base[(kk + u) * ROWS + 32 * i + fix];
      return v;
    }
  }
};

// KG > 1 splits each slab's k range among KG groups of WM x WN waves (every
// wave still takes part in the loads); after the last slab the groups' sums
// are added in ascending group order through the then idle stage buffers.
template <int BM_, int BN_, int BK_, int WM_, int WN_, int STAGES_, int TA_ = 0, int TB_ = 0, int KG_ = 1>
struct DmaCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, STAGES = STAGES_;
  static constexpr int TA = TA_, TB = TB_, KG = KG_;
  static constexpr int NW = WM * WN * KG, NT = 64 * NW;
  static constexpr int WTM = BM / WM, WTN = BN / WN, FM = WTM / 32, FN = WTN / 32;
  static constexpr int KSUB = BK / KG;  // k values of each slab per group
  // op(A) = A has k-contiguous rows; op(B) = B^T has k-contiguous columns.
  using SlabA = Slab<BM, BK, TA == 0, NW>;
  using SlabB = Slab<BN, BK, TB != 0, NW>;
  static constexpr int LDS_BYTES = 4 * STAGES * (SlabA::FLOATS + SlabB::FLOATS);
  // partial sums of groups 1..KG-1, BM*BN floats each, packed into the stage arrays
  static constexpr int RED_PER_ARRAY =
      (SlabA::FLOATS < SlabB::FLOATS ? SlabA::FLOATS : SlabB::FLOATS) / (BM * BN);
  static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "wave tile must be 32x32 blocks");
  static_assert(STAGES >= 2 && STAGES <= 4, "two to four LDS stages");
  static_assert(NT <= 1024, "at most 16 waves per workgroup");
  static_assert(KG == 1 || (KSUB % 32 == 0 && KSUB * KG == BK), "each group takes whole 32-deep k ranges");
  static_assert(KG == 1 || KG - 1 <= RED_PER_ARRAY * 2 * STAGES, "group sums fit in the stage arrays");
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per CU");
  // Waves per SIMD the direct kernel's registers must allow: four, or as many
  // as the workgroups that fit in LDS can bring (the unused stage arrays of a
  // two-stage kernel take up to 2 KiB more), and no more than leave room for
  // the wave's accumulators (FM x FN blocks of 16 registers) next to its
  // fragments and addresses in the 512 registers a SIMD lane holds: 128
  // each for four waves, 256 for two, all 512 for one (accumulators then in
  // AGPRs).
  static constexpr int LDS_WGS = (160 * 1024) / (LDS_BYTES + 2048);
  static constexpr int LDS_WAVES = LDS_WGS * NW / 4 < 4 ? (LDS_WGS * NW / 4 > 1 ? LDS_WGS * NW / 4 : 1) : 4;
  static constexpr int ACC_REGS = FM * FN * 16;
  static constexpr int REG_WAVES = ACC_REGS <= 64 ? 4 : ACC_REGS <= 160 ? 2 : 1;
  static constexpr int WAVES_EU = LDS_WAVES < REG_WAVES ? LDS_WAVES : REG_WAVES;
  static constexpr bool SCHED = false;
};

// One wave per SIMD (2 x 2 waves of 128 x 128) with a hand-ordered slab loop
// (see the SCHED branch of the kernel).
template <int BM_, int BN_, int BK_, int WM_, int WN_, int TA_ = 0, int TB_ = 0, int ST_ = 2>
struct DmaSchedCfg : DmaCfg<BM_, BN_, BK_, WM_, WN_, ST_, TA_, TB_, 1> {
  static constexpr bool SCHED = true;
};

// DIRECT: every slab by direct loads (the launcher guarantees 16-byte aligned
// chunks inside the matrices and K a multiple of BK); otherwise every slab
// through registers. Two kernels rather than a branch, so each gets the
// registers it needs. The direct kernels are held to the registers of
// WAVES_EU waves per SIMD (128 VGPRs for four), so small tiles keep several
// workgroups per compute unit instead of spending the register file on one.
// KTAIL (with DIRECT, for K >= BK not a multiple of BK): the whole slabs by
// direct loads, then the last, partial slab through registers with k >= K
// zeroed, unpipelined, after the direct loop has freed the stage arrays.
template <class Cfg, bool DIRECT, bool KTAIL = false>
__global__ void __launch_bounds__(Cfg::NT, DIRECT ? Cfg::WAVES_EU : 1) mfma_dma_kernel(GemmArgs g) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, FM = Cfg::FM, FN = Cfg::FN;
  constexpr int ST = Cfg::STAGES, NW = Cfg::NW;
  using SA = typename Cfg::SlabA;
  using SB = typename Cfg::SlabB;
  // One array per stage, selected at compile time: the compiler can then see
  // that a direct load into one stage does not alias reads of another, and
  // does not make those reads wait for the load.
  __shared__ __attribute__((aligned(1024))) float As0[SA::FLOATS];
  __shared__ __attribute__((aligned(1024))) float As1[SA::FLOATS];
  __shared__ __attribute__((aligned(1024))) float As2[ST > 2 ? SA::FLOATS : 4];
  __shared__ __attribute__((aligned(1024))) float As3[ST > 3 ? SA::FLOATS : 4];
  __shared__ __attribute__((aligned(1024))) float Bs0[SB::FLOATS];
  __shared__ __attribute__((aligned(1024))) float Bs1[SB::FLOATS];
  __shared__ __attribute__((aligned(1024))) float Bs2[ST > 2 ? SB::FLOATS : 4];
  __shared__ __attribute__((aligned(1024))) float Bs3[ST > 3 ? SB::FLOATS : 4];
  auto stage_a = [&](auto st) -> float* {
    if constexpr (decltype(st)::value == 0) return As0;
    else if constexpr (decltype(st)::value == 1) return As1;
    else if constexpr (decltype(st)::value == 2) return As2;
    else return As3;
  };
  auto stage_b = [&](auto st) -> float* {
    if constexpr (decltype(st)::value == 0) return Bs0;
    else if constexpr (decltype(st)::value == 1) return Bs1;
    else if constexpr (decltype(st)::value == 2) return Bs2;
    else return Bs3;
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;

  const int M = g.M, N = g.N;
  const int K = (blockIdx.y == gridDim.y - 1) ? g.k_last : g.K;  // last split-K chunk may be short
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, 4, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int kg = Cfg::KG == 1 ? 0 : wave / (Cfg::WM * Cfg::WN);  // k group
  const int wt = Cfg::KG == 1 ? wave : wave % (Cfg::WM * Cfg::WN);  // wave tile within the group
  const int wm = wt % Cfg::WM, wn = wt / Cfg::WM;
  const int l32 = lane & 31, h = lane >> 5;
  const float* A = g.A + (int64_t)blockIdx.y * g.strideA;
  const float* B = g.B + (int64_t)blockIdx.y * g.strideB;

  // ---- direct loads: region q = p*NW + wave of each slab is this wave's ----
  const float* a_src[SA::PER_WAVE];
#pragma unroll
  for (int p = 0; p < SA::PER_WAVE; ++p) a_src[p] = SA::direct_src(A, g.lda, m0, M, (p * NW + wave) * 64 + lane);
  const float* b_src[SB::PER_WAVE];
#pragma unroll
  for (int p = 0; p < SB::PER_WAVE; ++p) b_src[p] = SB::direct_src(B, g.ldb, n0, N, (p * NW + wave) * 64 + lane);
  auto issue_direct = [&](int k0, auto stage) {
    float* as = stage_a(stage);
    float* bs = stage_b(stage);
    const int64_t oa = SA::k_offset(k0, g.lda), ob = SB::k_offset(k0, g.ldb);
#pragma unroll
    for (int p = 0; p < SA::PER_WAVE; ++p) copy16_to_lds(a_src[p] + oa, as + (p * NW + wave) * 256);
#pragma unroll
    for (int p = 0; p < SB::PER_WAVE; ++p) copy16_to_lds(b_src[p] + ob, bs + (p * NW + wave) * 256);
  };

  // ---- register staging (edge tiles, unaligned operands, the K tail) ------
  f32x4 ra[SA::CHUNKS], rb[SB::CHUNKS];
  auto load_regs = [&](int k0, bool tail) __attribute__((always_inline)) {
    SA::load(ra, A, g.lda, m0, M, K, k0, tail, t);
    SB::load(rb, B, g.ldb, n0, N, K, k0, tail, t);
  };
  auto store_regs = [&](auto stage) __attribute__((always_inline)) {
    SA::store(stage_a(stage), ra, m0, M, t);
    SB::store(stage_b(stage), rb, n0, N, t);
  };

  // ---- fragments and the inner product ------------------------------------
  // Group kg multiplies k = kg*KSUB .. (kg+1)*KSUB - 1 of each slab: for a
  // k-contiguous slab the offset goes into the fragment key (KSUB is a
  // multiple of 32), for a line-contiguous one into the base address.
  const int kbase = kg * Cfg::KSUB;
  const int akey = SA::frag_key(l32, h) ^ (SA::KC ? kbase : 0);
  const int bkey = SB::frag_key(l32, h) ^ (SB::KC ? kbase : 0);
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto compute = [&](auto stage) __attribute__((always_inline)) {
    const float* as = SA::frag_base(stage_a(stage), wm * Cfg::WTM, l32, h) + (SA::KC ? 0 : SA::k_offset(kbase, BM));
    const float* bs = SB::frag_base(stage_b(stage), wn * Cfg::WTN, l32, h) + (SB::KC ? 0 : SB::k_offset(kbase, BN));
#pragma unroll
    for (int kk = 0; kk < Cfg::KSUB; kk += 8) {
      f32x4 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = SA::frag(as, i, kk, akey);
#pragma unroll
      for (int j = 0; j < FN; ++j) bf[j] = SB::frag(bs, j, kk, bkey);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][u], bf[j][u], acc[i][j], 0, 0, 0);
    }
  };
  // The same over a partial slab whose first r < KSUB values are all that is
  // left (the rest zeroed): MFMA step u of fragment set kk multiplies
  // k = kk + u and kk + 4 + u, so only the steps with kk + u < r run.
  auto compute_partial = [&](auto stage, int r) __attribute__((always_inline)) {
    const float* as = SA::frag_base(stage_a(stage), wm * Cfg::WTM, l32, h) + (SA::KC ? 0 : SA::k_offset(kbase, BM));
    const float* bs = SB::frag_base(stage_b(stage), wn * Cfg::WTN, l32, h) + (SB::KC ? 0 : SB::k_offset(kbase, BN));
#pragma unroll
    for (int kk = 0; kk < Cfg::KSUB; kk += 8) {
      if (kk < r) {
        f32x4 af[FM], bf[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = SA::frag(as, i, kk, akey);
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[j] = SB::frag(bs, j, kk, bkey);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (kk + u < r) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
              for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][u], bf[j][u], acc[i][j], 0, 0, 0);
          }
      }
    }
  };

  // ---- K loop ---------------------------------------------------------------
  const int nfull = K / BK;               // slabs with no k >= K
  const bool tail = (K % BK) != 0;
  // Register staging through stages 0 and 1, last slab peeled.
  auto register_loop = [&]() __attribute__((always_inline)) {
    const int nk = nfull + (tail ? 1 : 0);
    load_regs(0, tail && nk == 1);
    store_regs(S0{});
    __syncthreads();
    auto rstep = [&](auto cur, int s) __attribute__((always_inline)) {
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
  };
  if constexpr (Cfg::SCHED) {
    // One wave per SIMD, so nothing else fills the matrix pipe while this
    // wave waits: slab s is multiplied in G groups of FM x FN MFMAs, and
    // between groups the wave issues the loads of a later slab (spread over
    // the first quarter of the slab: with direct loads measured 0.7% faster
    // than over the first half, and faster than two or all-at-once groups)
    // and the next fragment set's LDS reads (double-buffered in registers).
    // The barrier that publishes slab s+1 comes two groups before the end of
    // slab s (its last LDS reads were issued earlier), and slab s+1's first
    // fragments are read while those two groups run (four when a group is a
    // single MFMA). sched_barrier keeps this order.
    // Direct loads (DIRECT): with ST stages the loads go ST - 1 slabs ahead,
    // into the stage slab s - 1 has just left, and the barrier waits only for
    // slab s + 1.
    // Register staging (operands of any alignment): two LDS stages and one
    // slab in registers. In step s the registers hold slab s + 1; each
    // group that loads first writes its chunks of them to the stage slab
    // s - 1 has left, then reloads them with slab s + 2 (the compiler waits
    // for each chunk's load, issued a whole step before). The barrier
    // publishes slab s + 1. A partial last slab follows the loop, staged on
    // its own. It needs a whole slab and, for a line-contiguous operand,
    // lines of at least 4 values (the whole-chunk reads of its last chunk);
    // smaller problems take the plain register loop.
    // In both, a load past the last slab reloads the last slab instead, so
    // every wave issues the same loads in every step (the vmcnt waits count
    // them) and the loop has no branch (a branch makes the compiler wait for
    // every LDS read at the join); those loads complete before a barrier like
    // any other. A wave with a single 32 x 32 block keeps two accumulator
    // chains (even and odd k steps), so that no MFMA waits for the one
    // before it; they are added after the loop.
    const bool sched = DIRECT || (nfull >= 1 && (SA::KC || M >= 4) && (SB::KC || N >= 4));
    if (sched) {
      static_assert(Cfg::KG == 1 && (BK / 8) % 2 == 0, "scheduled loop: no k groups, an even number of fragment sets");
      constexpr int KK = BK / 8;                 // fragment sets per slab, 8 k each
      constexpr int G = 4 * KK;                  // MFMA groups per slab
      constexpr int SST = DIRECT ? ST : 2;       // LDS stages the loop cycles through
      constexpr int AHEAD = DIRECT ? ST - 1 : 2;  // step s loads slab s + AHEAD
      // per slab: this wave's direct loads, or this thread's register chunks
      constexpr int NA = DIRECT ? SA::PER_WAVE : SA::CHUNKS;
      constexpr int NL = NA + (DIRECT ? SB::PER_WAVE : SB::CHUNKS);
      constexpr int LG = G / 4;                  // groups that issue them
      // The barrier group: after the slab's last LDS reads (issued in group
      // G - 7) and while the set the next slab's first reads go to is free
      // (from group G - 4 on); with one MFMA per group, four groups leave
      // time for those reads to land.
      constexpr int BAR_G = FM * FN >= 4 ? G - 2 : G - 4;
      constexpr int PER_G = (NL + LG - 1) / LG;
      constexpr int NACC = FM * FN == 1 ? 2 : 1;
      f32x16 acc2[NACC == 2 ? FM : 1][NACC == 2 ? FN : 1];
      if constexpr (NACC == 2) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc2[i][j][r] = 0.0f;
      }
      // register staging: where each of this lane's fragment lines sits in its slot
      int afix[DIRECT ? 1 : FM], bfix[DIRECT ? 1 : FN];
      if constexpr (!DIRECT) {
#pragma unroll
        for (int i = 0; i < FM; ++i) afix[i] = SA::read_fix(m0, M, wm * Cfg::WTM + 32 * i + l32);
#pragma unroll
        for (int j = 0; j < FN; ++j) bfix[j] = SB::read_fix(n0, N, wn * Cfg::WTN + 32 * j + l32);
      }
      f32x4 af[2][FM], bf[2][FN];
      auto read_set = [&](auto stage, auto set, int kk) __attribute__((always_inline)) {
        constexpr int SET = decltype(set)::value;
        const float* as = SA::frag_base(stage_a(stage), wm * Cfg::WTM, l32, h);
        const float* bs = SB::frag_base(stage_b(stage), wn * Cfg::WTN, l32, h);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          if constexpr (DIRECT) af[SET][i] = SA::frag(as, i, kk, akey);
          else af[SET][i] = SA::frag(as, i, kk, akey, afix[i]);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if constexpr (DIRECT) bf[SET][j] = SB::frag(bs, j, kk, bkey);
          else bf[SET][j] = SB::frag(bs, j, kk, bkey, bfix[j]);
        }
      };
      // register staging: each chunk's source at k = 0
      constexpr int RA = DIRECT ? 1 : SA::CHUNKS, RB = DIRECT ? 1 : SB::CHUNKS;
      const float* pa[RA];
      const float* pb[RB];
      if constexpr (!DIRECT) {
#pragma unroll
        for (int c = 0; c < RA; ++c) pa[c] = SA::chunk_src(A, g.lda, m0, M, c * Cfg::NT + t);
#pragma unroll
        for (int c = 0; c < RB; ++c) pb[c] = SB::chunk_src(B, g.ldb, n0, N, c * Cfg::NT + t);
      }
      // load q of the slab at k0: a direct load into `stage`, or chunk q into registers
      auto load_one = [&](int q, int k0, auto stage) __attribute__((always_inline)) {
        if constexpr (DIRECT) {
          if (q < NA)
            copy16_to_lds(a_src[q] + SA::k_offset(k0, g.lda), stage_a(stage) + (q * NW + wave) * 256);
          else
            copy16_to_lds(b_src[q - NA] + SB::k_offset(k0, g.ldb), stage_b(stage) + ((q - NA) * NW + wave) * 256);
        } else {
          if (q < NA)
            ra[q] = load16(pa[q] + SA::k_offset(k0, g.lda));
          else
            rb[q - NA] = load16(pb[q - NA] + SB::k_offset(k0, g.ldb));
        }
      };
      // register chunk q to `stage`
      auto store_one = [&](int q, auto stage) __attribute__((always_inline)) {
        if (q < NA)
          SA::store_chunk(stage_a(stage), ra[q], q * Cfg::NT + t);
        else
          SB::store_chunk(stage_b(stage), rb[q - NA], (q - NA) * Cfg::NT + t);
      };
      using Z = std::integral_constant<int, 0>;
      auto group = [&](auto cur, auto gi_c, int k1) __attribute__((always_inline)) {
        constexpr int gi = decltype(gi_c)::value;
        constexpr int kk = gi / 4, u = gi % 4, set = kk & 1;
        constexpr int CUR = decltype(cur)::value;
        using Next = std::integral_constant<int, (CUR + SST - 1) % SST>;   // where slab s + ST - 1 goes
        using Following = std::integral_constant<int, (CUR + 1) % SST>;    // where slab s + 1 is
        // The next set is read one group into this one: the compiler waits for
        // every outstanding LDS read before the next group that uses a set, so
        // reads issued right before such a group would stall it.
        if constexpr (u == 1 && kk + 1 < KK) read_set(cur, std::integral_constant<int, (kk + 1) & 1>{}, (kk + 1) * 8);
        if constexpr (gi < LG) {
#pragma unroll
          for (int q = gi * PER_G; q < (gi + 1) * PER_G && q < NL; ++q) {
            if constexpr (DIRECT) {
              load_one(q, k1, Next{});
            } else {  // the reload reuses the chunk's registers once the write has them
              store_one(q, Following{});
              __builtin_amdgcn_sched_barrier(0);
              load_one(q, k1, Z{});
            }
          }
        }
        if constexpr (gi == BAR_G) {
          if constexpr (DIRECT) __builtin_amdgcn_s_waitcnt(vmcnt_imm((ST - 2) * NL));  // slab s + 1 has landed
          __syncthreads();
          read_set(Following{}, Z{}, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            if constexpr (NACC == 2 && (u & 1))
              acc2[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[set][i][u], bf[set][j][u], acc2[i][j], 0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[set][i][u], bf[set][j][u], acc[i][j], 0, 0, 0);
          }
        __builtin_amdgcn_sched_barrier(0);
      };
      auto sched_step = [&](auto cur, int s) __attribute__((always_inline)) {
        const int k1 = (s + AHEAD < nfull ? s + AHEAD : nfull - 1) * BK;
        static_for<G>([&](auto gi_c) __attribute__((always_inline)) { group(cur, gi_c, k1); });
      };
      static_assert(!DIRECT || (ST - 2) * NL < 64, "vmcnt field");
      if constexpr (DIRECT) {
        // slabs 0 .. ST-2 (a slab past the last reloads the last one)
        static_for<ST - 1>([&](auto i_c) __attribute__((always_inline)) {
          constexpr int i = decltype(i_c)::value;
          const int k0 = (i < nfull ? i : nfull - 1) * BK;
#pragma unroll
          for (int q = 0; q < NL; ++q) load_one(q, k0, std::integral_constant<int, i>{});
        });
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((ST - 2) * NL));  // slab 0 has landed
      } else {
        // slab 0 to stage 0, slab 1 into the registers
#pragma unroll
        for (int q = 0; q < NL; ++q) load_one(q, 0, Z{});
#pragma unroll
        for (int q = 0; q < NL; ++q) store_one(q, S0{});
        const int k1 = (nfull > 1 ? 1 : 0) * BK;
#pragma unroll
        for (int q = 0; q < NL; ++q) load_one(q, k1, Z{});
      }
      __syncthreads();
      read_set(S0{}, Z{}, 0);
      int s = 0;
      for (; s + SST <= nfull; s += SST) {
        sched_step(S0{}, s);
        sched_step(S1{}, s + 1);
        if constexpr (SST > 2) sched_step(S2{}, s + 2);
        if constexpr (SST > 3) sched_step(S3{}, s + 3);
      }
      if (s < nfull) sched_step(S0{}, s);
      if constexpr (SST > 2) {
        if (s + 1 < nfull) sched_step(S1{}, s + 1);
      }
      if constexpr (SST > 3) {
        if (s + 2 < nfull) sched_step(S2{}, s + 2);
      }
      if constexpr (NACC == 2) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] += acc2[i][j];
      }
      // With more than two stages the last step's reloads may still be in
      // flight past its barrier: they land before the stage arrays are reused
      // or the wave ends.
      if constexpr (DIRECT && ST > 2) wait_loads();
      // A partial last slab (k >= K zeroed), staged through registers after
      // every wave has left the stage arrays.
      if constexpr (KTAIL || !DIRECT) {
        if (tail) {
          load_regs(nfull * BK, true);
          __syncthreads();
          store_regs(S0{});
          __syncthreads();
          compute_partial(S0{}, K - nfull * BK);
        }
      }
    } else {
      register_loop();
    }
  } else if constexpr (DIRECT) {
    // STAGES-deep pipeline of direct loads over the full slabs: slab s+ST-1 is
    // in flight while slab s is multiplied (slab s lives in stage s % ST).
    // Each wave waits for its own loads of the next slab, then the barrier
    // publishes them to the workgroup. The loop is unrolled by ST so every
    // stage index is a constant.
    // Each wave has per_slab direct loads in flight per slab; the wait
    // before a barrier lets the loads of the slabs after the next one stay in
    // flight (vmcnt takes an immediate, hence the cases).
    constexpr int per_slab = SA::PER_WAVE + SB::PER_WAVE;
    static_assert((ST - 2) * per_slab <= 15, "vmcnt field");
    auto wait_slabs_ahead = [&](int ahead) {  // until at most `ahead` later slabs are in flight
      if (ST > 3 && ahead >= 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * per_slab));
      else if (ST > 2 && ahead >= 1) __builtin_amdgcn_s_waitcnt(0x0F70 | per_slab);
      else wait_loads();
    };
    issue_direct(0, S0{});
    if (ST > 2 && nfull > 1) issue_direct(BK, S1{});
    if (ST > 3 && nfull > 2) issue_direct(2 * BK, S2{});
    wait_slabs_ahead((nfull < ST - 1 ? nfull : ST - 1) - 1);
    __syncthreads();
    auto step = [&](auto cur, int s) {
      constexpr int CUR = decltype(cur)::value;
      using Next = std::integral_constant<int, (CUR + ST - 1) % ST>;
      const bool more = s + ST - 1 < nfull;
      if (more) issue_direct((s + ST - 1) * BK, Next{});
      __builtin_amdgcn_sched_barrier(0);
      compute(cur);
      // Slab s+1 must have landed; the slabs issued after it may stay in flight.
      const int issued = (s + ST - 1 < nfull ? s + ST - 1 : nfull - 1);  // last slab issued
      wait_slabs_ahead(issued - (s + 1));
      __syncthreads();
    };
    // Whole groups of ST slabs, then the remaining nfull % ST (no exit from
    // the middle of the unrolled body, so the accumulators stay in place).
    int s = 0;
    for (; s + ST <= nfull; s += ST) {
      step(S0{}, s);
      step(S1{}, s + 1);
      if constexpr (ST > 2) step(S2{}, s + 2);
      if constexpr (ST > 3) step(S3{}, s + 3);
    }
    if (s < nfull) step(S0{}, s);
    if (s + 1 < nfull) step(S1{}, s + 1);
    if constexpr (ST > 3) {
      if (s + 2 < nfull) step(S2{}, s + 2);
    }
    if constexpr (KTAIL) {
      if (tail) {
        load_regs(nfull * BK, true);
        store_regs(S0{});
        __syncthreads();
        compute(S0{});
        if constexpr (Cfg::KG > 1) __syncthreads();  // the groups' sums reuse the stage arrays
      }
    }
  } else {
    register_loop();
  }

  // ---- k groups: add the groups' sums in ascending group order ----------
  if constexpr (Cfg::KG > 1) {
    constexpr int WAVE_FLOATS = FM * FN * 16 * 64;  // one wave's accumulators
    // Partial sums of group q (1..KG-1) go to block q-1 of the stage arrays
    // As0, Bs0, As1, Bs1, ... (RED_PER_ARRAY blocks of BM*BN floats each).
    auto red_block = [&](int q) -> float* {
      const int a = (q - 1) / Cfg::RED_PER_ARRAY, off = ((q - 1) % Cfg::RED_PER_ARRAY) * BM * BN;
      float* base = a == 0   ? As0
                    : a == 1 ? Bs0
                    : a == 2 ? As1
                    : a == 3 ? Bs1
                    : a == 4 ? As2
                    : a == 5 ? Bs2
                    : a == 6 ? As3
                             : Bs3;
      return base + off + wt * WAVE_FLOATS + lane;
    };
    // The K loop ends with a barrier, so no wave still reads a slab.
    if (kg > 0) {
      float* red = red_block(kg);
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
      const float* red = red_block(q);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] += red[((i * FN + j) * 16 + r) * 64];
    }
  }

  // ---- epilogue: C is read only when beta != 0 ----------------------------
  // Element r of block (i, j) belongs to row row0 + 32 i + 8 (r / 4) + r % 4
  // and column col0 + 32 j. A tile wholly inside C stores without masks: the
  // wave's first row and column give a uniform base, each element adds a
  // uniform offset, and a lane adds its own (its row within four and its
  // column), the same for every element and 32-bit while 4 ldc is; with
  // beta != 0 a block's 16 values of C are all read before any is written.
  // Edge tiles mask every element.
  float* C = g.C + (int64_t)blockIdx.y * g.strideC;
  const int row0 = m0 + wm * Cfg::WTM + 4 * h;
  const int col0 = n0 + wn * Cfg::WTN + l32;
  const float alpha = g.alpha, beta = g.beta;
  if (m0 + BM <= M && n0 + BN <= N && g.ldc < (1 << 27)) {
    float* cw = C + (int64_t)(m0 + wm * Cfg::WTM) * g.ldc + (n0 + wn * Cfg::WTN);
    const uint32_t lane_off = (uint32_t)(4 * h) * (uint32_t)g.ldc + (uint32_t)l32;
    auto at = [&](int i, int j, int r) __attribute__((always_inline)) -> float* {
      return cw + ((int64_t)(32 * i + 8 * (r >> 2) + (r & 3)) * g.ldc + 32 * j) + lane_off;
    };
    auto each = [&](auto op) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) op(at(i, j, r), acc[i][j][r]);
    };
    if (alpha == 1.0f && beta == 0.0f) {
      each([](float* p, float v) { *p = v; });
    } else if (beta == 0.0f) {
      each([alpha](float* p, float v) { *p = alpha * v; });
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          float old[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) old[r] = *at(i, j, r);
#pragma unroll
          for (int r = 0; r < 16; ++r) *at(i, j, r) = __builtin_fmaf(beta, old[r], alpha * acc[i][j][r]);
        }
    }
    return;
  }
  auto store_tile = [&](auto op) __attribute__((always_inline)) {
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

// The LDS stage arrays of a kernel. Each stage is its own __shared__ array,
// and code picks one with a compile-time index: the compiler then sees that a
// direct load into one stage does not alias reads of another, and does not
// make those reads wait for the load.
struct Stages {
  float* a[3];
  float* b[3];
};

#define SGEMM_DMA_DECLARE_STAGES(Cfg, st)                                                     \
  __shared__ __attribute__((aligned(1024))) float As0[Cfg::SlabA::FLOATS];                    \
  __shared__ __attribute__((aligned(1024))) float As1[Cfg::SlabA::FLOATS];                    \
  __shared__ __attribute__((aligned(1024))) float As2[Cfg::STAGES > 2 ? Cfg::SlabA::FLOATS : 4]; \
  __shared__ __attribute__((aligned(1024))) float Bs0[Cfg::SlabB::FLOATS];                    \
  __shared__ __attribute__((aligned(1024))) float Bs1[Cfg::SlabB::FLOATS];                    \
  __shared__ __attribute__((aligned(1024))) float Bs2[Cfg::STAGES > 2 ? Cfg::SlabB::FLOATS : 4]; \
  const Stages st{{As0, As1, As2}, {Bs0, Bs1, Bs2}}

// tile_product: the per-tile K loop of mfma_dma_kernel above, as a function the
// stream-K kernel calls once per piece of work (DIRECT and the register
// budget as there). The plain kernel keeps its own copy of the loop: written
// through this function it compiled to a slightly different K loop (one more
// 64-bit address add per two slabs) that ran 0.75% slower at 8192^3 and
// 4096^3, timed alternately against the original in one process.
//
// Unlike the plain kernel it has no direct variant with a register-staged last
// slab: in the stream-K kernel that variant spilled 150 to 290 VGPRs. The
// stream-K kernel adds a partial last slab in its epilogue instead.
//
// It computes the workgroup's BM x BN tile of op(A).op(B) at rows m0.., columns
// n0.., over k = 0 .. K-1 of the operands whose k = 0 lies at A and B. It hands
// the accumulators to epi(acc, row0, col0) (with k groups, group 0 only, after the
// groups' sums are added), where accumulator element r of block (i, j) belongs to
// row row0 + 32 i + 8 (r / 4) + r % 4 and column col0 + 32 j. Every slab step
// ends with a barrier, so when it returns no wave still reads the stage arrays.
template <class Cfg, bool DIRECT, class Epi>
__device__ __forceinline__ void tile_product(const GemmArgs& g, const Stages& st, const float* A, const float* B,
                                             int K, int m0, int n0, Epi&& epi) {
  constexpr int BK = Cfg::BK, FM = Cfg::FM, FN = Cfg::FN;
  constexpr int ST = Cfg::STAGES, NW = Cfg::NW;
  static_assert(ST <= 3, "the stream-K kernel keeps three stage arrays");
  using SA = typename Cfg::SlabA;
  using SB = typename Cfg::SlabB;
  auto stage_a = [&](auto s) -> float* { return st.a[decltype(s)::value]; };
  auto stage_b = [&](auto s) -> float* { return st.b[decltype(s)::value]; };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;

  const int M = g.M, N = g.N;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int kg = Cfg::KG == 1 ? 0 : wave / (Cfg::WM * Cfg::WN);  // k group
  const int wt = Cfg::KG == 1 ? wave : wave % (Cfg::WM * Cfg::WN);  // wave tile within the group
  const int wm = wt % Cfg::WM, wn = wt / Cfg::WM;
  const int l32 = lane & 31, h = lane >> 5;

  // ---- direct loads: region q = p*NW + wave of each slab is this wave's ----
  const float* a_src[SA::PER_WAVE];
#pragma unroll
  for (int p = 0; p < SA::PER_WAVE; ++p) a_src[p] = SA::direct_src(A, g.lda, m0, M, (p * NW + wave) * 64 + lane);
  const float* b_src[SB::PER_WAVE];
#pragma unroll
  for (int p = 0; p < SB::PER_WAVE; ++p) b_src[p] = SB::direct_src(B, g.ldb, n0, N, (p * NW + wave) * 64 + lane);
  auto issue_direct = [&](int k0, auto stage) {
    float* as = stage_a(stage);
    float* bs = stage_b(stage);
    const int64_t oa = SA::k_offset(k0, g.lda), ob = SB::k_offset(k0, g.ldb);
#pragma unroll
    for (int p = 0; p < SA::PER_WAVE; ++p) copy16_to_lds(a_src[p] + oa, as + (p * NW + wave) * 256);
#pragma unroll
    for (int p = 0; p < SB::PER_WAVE; ++p) copy16_to_lds(b_src[p] + ob, bs + (p * NW + wave) * 256);
  };

  // ---- register staging (edge tiles, unaligned operands, the K tail) ------
  f32x4 ra[SA::CHUNKS], rb[SB::CHUNKS];
  auto load_regs = [&](int k0, bool tail) {
    SA::load(ra, A, g.lda, m0, M, K, k0, tail, t);
    SB::load(rb, B, g.ldb, n0, N, K, k0, tail, t);
  };
  auto store_regs = [&](auto stage) {
    SA::store(stage_a(stage), ra, m0, M, t);
    SB::store(stage_b(stage), rb, n0, N, t);
  };

  // ---- fragments and the inner product ------------------------------------
  // Group kg's first k of each slab: in the fragment key for a k-contiguous
  // slab, in the base address for a line-contiguous one.
  const int kbase = kg * Cfg::KSUB;
  const int akey = SA::frag_key(l32, h) ^ (SA::KC ? kbase : 0);
  const int bkey = SB::frag_key(l32, h) ^ (SB::KC ? kbase : 0);
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto compute = [&](auto stage) {
    const float* as =
        SA::frag_base(stage_a(stage), wm * Cfg::WTM, l32, h) + (SA::KC ? 0 : SA::k_offset(kbase, Cfg::BM));
    const float* bs =
        SB::frag_base(stage_b(stage), wn * Cfg::WTN, l32, h) + (SB::KC ? 0 : SB::k_offset(kbase, Cfg::BN));
#pragma unroll
    for (int kk = 0; kk < Cfg::KSUB; kk += 8) {
      f32x4 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = SA::frag(as, i, kk, akey);
#pragma unroll
      for (int j = 0; j < FN; ++j) bf[j] = SB::frag(bs, j, kk, bkey);
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
        constexpr int per_slab = SA::PER_WAVE + SB::PER_WAVE;
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

  // ---- k groups: add the groups' sums in ascending group order ----------
  if constexpr (Cfg::KG > 1) {
    constexpr int WAVE_FLOATS = FM * FN * 16 * 64;  // one wave's accumulators
    // Partial sums of group q (1..KG-1) go to block q-1 of the stage arrays
    // a0, b0, a1, b1, ... (RED_PER_ARRAY blocks of BM*BN floats each).
    auto red_block = [&](int q) -> float* {
      const int a = (q - 1) / Cfg::RED_PER_ARRAY, off = ((q - 1) % Cfg::RED_PER_ARRAY) * Cfg::BM * Cfg::BN;
      float* base = a == 0   ? st.a[0]
                    : a == 1 ? st.b[0]
                    : a == 2 ? st.a[1]
                    : a == 3 ? st.b[1]
                    : a == 4 ? st.a[2]
                             : st.b[2];
      return base + off + wt * WAVE_FLOATS + lane;
    };
    // The K loop ends with a barrier, so no wave still reads a slab.
    if (kg > 0) {
      float* red = red_block(kg);
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
      const float* red = red_block(q);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] += red[((i * FN + j) * 16 + r) * 64];
    }
  }
  epi(acc, m0 + wm * Cfg::WTM + 4 * h, n0 + wn * Cfg::WTN + l32);
}

// C = alpha * acc + beta * C over the accumulators of one wave (rows and
// columns as tile_product hands them over), masked to the M x N matrix; C is
// read only when beta != 0.
template <int FM, int FN>
__device__ __forceinline__ void store_c(const f32x16 (&acc)[FM][FN], int row0, int col0, float* C, int64_t ldc,
                                        int M, int N, float alpha, float beta) {
  auto store_tile = [&](auto op) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = col0 + 32 * j;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + 32 * i + 8 * (r >> 2) + (r & 3);
          if (row < M && col < N) op(C + (int64_t)row * ldc + col, acc[i][j][r]);
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

// acc += the products of k = kt .. K-1 (fewer than a slab) for one wave's
// accumulators, with rows and columns as tile_product hands them over: plain
// FMAs on operand elements read straight from memory, zero for rows past M
// and columns past N. The stream-K kernel adds a partial last slab this way
// in the epilogue, since staging it through registers there spilled.
template <class Cfg>
__device__ __forceinline__ void add_k_tail(f32x16 (&acc)[Cfg::FM][Cfg::FN], const GemmArgs& g, int kt, int row0,
                                           int col0) {
  constexpr int T = Cfg::BK - 1;  // at most this many k values remain
  // op(B) values of the tail for this lane's columns, then each row in turn
  // with k innermost, so no per-row address stays live across rows
  float bv[T][Cfg::FN];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int k = kt + t, col = col0 + 32 * j;
      bv[t][j] = (k < g.K && col < g.N) ? (Cfg::TB ? g.B[(int64_t)col * g.ldb + k] : g.B[(int64_t)k * g.ldb + col])
                                        : 0.0f;
    }
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = row0 + 32 * i + 8 * (r >> 2) + (r & 3);
      if (row >= g.M) continue;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int k = kt + t;
        if (k >= g.K) break;
        const float av = Cfg::TA ? g.A[(int64_t)k * g.lda + row] : g.A[(int64_t)row * g.lda + k];
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) acc[i][j][r] = __builtin_fmaf(av, bv[t][j], acc[i][j][r]);
      }
    }
}

// Stream-K (Osama et al., "Stream-K: Work-centric Parallel Decomposition for
// Dense Matrix-Matrix Multiplication on the GPU", PPoPP 2023): a persistent
// grid of G workgroups, about one per resident slot of the device. The first
// dp_tiles tiles of the tile order run whole, tile j on workgroup j % G. The
// remaining sk_tiles tiles are cut into their iters BK-deep slabs, and the
// sk_tiles * iters slabs (in tile order, k ascending within a tile) are dealt
// out as G contiguous ranges: workgroup w takes slabs [w U / G, (w+1) U / G),
// U = sk_tiles * iters. A range crosses tile boundaries; each piece of a tile
// it holds is a segment. A segment that spans its whole tile is stored to C;
// any other is a partial sum, stored as a dense row-major BM x BN block in
// slot 2w (the range's first segment) or 2w+1 (its last) of the workspace
// (StreamKPlan). A second kernel then adds each split tile's partials in
// ascending k order. Every workgroup's loop ends after its own range, so the
// grid drains whether or not all of it is resident at once.
// KTAIL (direct loads, K not a whole number of slabs): the iters slabs are
// the whole ones, and the piece that ends a tile adds the k >= iters * BK
// products in its epilogue (add_k_tail).
template <class Cfg, bool DIRECT, bool KTAIL = false>
__global__ void __launch_bounds__(Cfg::NT, DIRECT ? Cfg::WAVES_EU : 1)
    mfma_dma_streamk_kernel(GemmArgs g, StreamKPlan p) {
  static_assert(Cfg::KG == 1, "stream-K runs tiles without k groups");
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
  SGEMM_DMA_DECLARE_STAGES(Cfg, st);
  using SA = typename Cfg::SlabA;
  using SB = typename Cfg::SlabB;
  const int G = gridDim.x, w = blockIdx.x;
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int n_dp = w < p.dp_tiles ? (p.dp_tiles - 1 - w) / G + 1 : 0;
  const int64_t begin = (int64_t)w * p.sk_iters / G, end = (int64_t)(w + 1) * p.sk_iters / G;
  int64_t it = begin;
  for (int item = 0;; ++item) {
    int tile, kb, ke;
    if (item < n_dp) {
      tile = w + item * G;
      kb = 0;
      ke = p.iters;
    } else {
      if (it >= end) break;
      const int u = (int)(it / p.iters);
      kb = (int)(it - (int64_t)u * p.iters);
      ke = (end - it) < (int64_t)(p.iters - kb) ? kb + (int)(end - it) : p.iters;
      tile = p.dp_tiles + u;
    }
    const bool whole = kb == 0 && ke == p.iters;
    float* slot = p.partials + (size_t)(2 * w + (it == begin ? 0 : 1)) * (BM * BN);
    if (item >= n_dp) it += ke - kb;
    int tm, tn;
    tile_coords(tile, tiles_m, tiles_n, 4, tm, tn);
    const int k0 = kb * BK;
    const int klen = ((int64_t)ke * BK < (int64_t)g.K ? ke * BK : g.K) - k0;
    const int m0 = tm * BM, n0 = tn * BN;
    tile_product<Cfg, DIRECT>(
        g, st, g.A + SA::k_offset(k0, g.lda), g.B + SB::k_offset(k0, g.ldb), klen, m0, n0,
        [&](f32x16(&acc)[Cfg::FM][Cfg::FN], int row0, int col0) {
          if constexpr (KTAIL) {
            if (ke == p.iters) add_k_tail<Cfg>(acc, g, p.iters * BK, row0, col0);
          }
          if (whole) {
            store_c(acc, row0, col0, g.C, g.ldc, g.M, g.N, g.alpha, g.beta);
          } else {
            // the whole block, edges included (the fixup masks them)
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
              for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                  slot[(row0 - m0 + 32 * i + 8 * (r >> 2) + (r & 3)) * BN + col0 - n0 + 32 * j] = acc[i][j][r];
          }
        });
  }
}

// Adds the partial sums of the stream-K tiles that were split: tile
// dp_tiles + blockIdx.y, 1024 consecutive elements of its row-major BM x BN
// block per workgroup (4 columns per thread). The workgroups holding pieces of
// the tile are those whose slab ranges meet [u iters, (u+1) iters); their
// blocks are added in ascending workgroup order, which is ascending k, so
// repeated calls give identical bits. C = alpha * sum + beta * C, masked to
// the M x N matrix; C is read only when beta != 0.
__global__ void __launch_bounds__(256) streamk_fixup_kernel(GemmArgs g, StreamKPlan p, int bm, int bn, int grid) {
  const int u = blockIdx.y;
  const int64_t it0 = (int64_t)u * p.iters, it1 = it0 + p.iters - 1;
  const int64_t U = p.sk_iters;
  // the workgroup whose range holds slab `it`: the last w with w U / G <= it
  auto owner = [&](int64_t it) { return (int)(((it + 1) * grid - 1) / U); };
  const int wa = owner(it0), wb = owner(it1);
  if (wa == wb) return;  // the whole tile lay in one range and went straight to C
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= bm * bn) return;
  f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int w = wa; w <= wb; ++w) {
    const int64_t b = (int64_t)w * U / grid, en = (int64_t)(w + 1) * U / grid;
    if (b == en) continue;  // a workgroup with no slabs
    const int block = 2 * w + (b >= it0 ? 0 : 1);
    s += *reinterpret_cast<const f32x4*>(p.partials + (size_t)block * bm * bn + e);
  }
  const int tiles_m = (g.M + bm - 1) / bm, tiles_n = (g.N + bn - 1) / bn;
  int tm, tn;
  tile_coords(p.dp_tiles + u, tiles_m, tiles_n, 4, tm, tn);
  const int row = tm * bm + e / bn, col = tn * bn + e % bn;
  if (row >= g.M) return;
  float* c = g.C + (int64_t)row * g.ldc + col;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (col + q < g.N) {
      const float v = g.alpha * s[q];
      c[q] = (g.beta != 0.0f) ? __builtin_fmaf(g.beta, c[q], v) : v;
    }
  }
}

// Direct loads need every 16-byte chunk they fetch to be aligned and inside
// the matrices: A and B (and each batch entry) 16-byte aligned, leading
// dimensions multiples of 4, and the extent of a line-contiguous operand (M
// for A^T, N for B) a multiple of 4 so the last chunk of lines is whole. The
// direct kernel also takes K (and a short last split-K chunk) in whole slabs,
// which keeps the K tail, and its registers, out of it.
template <class Cfg>
bool direct_ok(const GemmArgs& g) {
  const bool aligned = ((reinterpret_cast<uintptr_t>(g.A) | reinterpret_cast<uintptr_t>(g.B)) & 15) == 0 &&
                       ((g.lda | g.ldb) & 3) == 0 && (g.batch <= 1 || ((g.strideA | g.strideB) & 3) == 0);
  const bool lines = (Cfg::TA == 0 || g.M % 4 == 0) && (Cfg::TB != 0 || g.N % 4 == 0);
  return g.M > 0 && g.N > 0 && aligned && lines && g.K % Cfg::BK == 0 && g.k_last % Cfg::BK == 0;
}

// The direct kernel with a register-staged last slab: the same alignment, K
// (and a short last split-K chunk) at least one slab but not all multiples of
// BK. Its direct loads stop at the last whole slab of each batch entry.
template <class Cfg>
bool direct_tail_ok(const GemmArgs& g) {
  const bool aligned = ((reinterpret_cast<uintptr_t>(g.A) | reinterpret_cast<uintptr_t>(g.B)) & 15) == 0 &&
                       ((g.lda | g.ldb) & 3) == 0 && (g.batch <= 1 || ((g.strideA | g.strideB) & 3) == 0);
  const bool lines = (Cfg::TA == 0 || g.M % 4 == 0) && (Cfg::TB != 0 || g.N % 4 == 0);
  return g.M > 0 && g.N > 0 && aligned && lines && g.K >= Cfg::BK && g.k_last >= Cfg::BK &&
         (g.K % Cfg::BK != 0 || g.k_last % Cfg::BK != 0);
}

template <class Cfg>
hipError_t launch_mfma_dma(const GemmArgs& g, hipStream_t stream) {
  const int64_t tiles = (int64_t)((g.M + Cfg::BM - 1) / Cfg::BM) * ((g.N + Cfg::BN - 1) / Cfg::BN);
  GemmArgs a = g;
  void* args[] = {&a};
  const void* kernel = direct_ok<Cfg>(g)        ? reinterpret_cast<const void*>(&mfma_dma_kernel<Cfg, true>)
                       : direct_tail_ok<Cfg>(g) ? reinterpret_cast<const void*>(&mfma_dma_kernel<Cfg, true, true>)
                                                : reinterpret_cast<const void*>(&mfma_dma_kernel<Cfg, false>);
  return hipLaunchKernel(kernel, dim3((unsigned)tiles, (unsigned)g.batch), dim3(Cfg::NT), args, 0, stream);
}

// The hand-ordered loop staged through registers: operands of any alignment.
template <class Cfg>
hipError_t launch_mfma_rs(const GemmArgs& g, hipStream_t stream) {
  const int64_t tiles = (int64_t)((g.M + Cfg::BM - 1) / Cfg::BM) * ((g.N + Cfg::BN - 1) / Cfg::BN);
  GemmArgs a = g;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mfma_dma_kernel<Cfg, false>),
                         dim3((unsigned)tiles, (unsigned)g.batch), dim3(Cfg::NT), args, 0, stream);
}

template <class Cfg>
hipError_t launch_mfma_dma_streamk(const GemmArgs& g, const StreamKPlan& plan, int grid, bool direct,
                                   hipStream_t stream) {
  // the direct kernel only where its loads stay aligned and inside the matrices
  // with direct loads a K that is not a whole number of slabs takes the KTAIL
  // kernel, whose plan counts only the whole slabs
  const bool ktail = direct && g.K % Cfg::BK != 0;
  if (direct && !direct_ok<Cfg>(g) && !direct_tail_ok<Cfg>(g)) return hipErrorInvalidValue;
  if (plan.iters != (ktail ? g.K / Cfg::BK : (g.K + Cfg::BK - 1) / Cfg::BK)) return hipErrorInvalidValue;
  if (grid <= 0 || plan.iters <= 0 || (plan.sk_tiles > 0 && plan.partials == nullptr)) return hipErrorInvalidValue;
  GemmArgs a = g;
  StreamKPlan pl = plan;
  void* args[] = {&a, &pl};
  const void* kernel = !direct ? reinterpret_cast<const void*>(&mfma_dma_streamk_kernel<Cfg, false>)
                       : ktail ? reinterpret_cast<const void*>(&mfma_dma_streamk_kernel<Cfg, true, true>)
                               : reinterpret_cast<const void*>(&mfma_dma_streamk_kernel<Cfg, true>);
  hipError_t err = hipLaunchKernel(kernel, dim3((unsigned)grid), dim3(Cfg::NT), args, 0, stream);
  if (err != hipSuccess || plan.sk_tiles == 0) return err;
  int bm = Cfg::BM, bn = Cfg::BN, gr = grid;
  void* fargs[] = {&a, &pl, &bm, &bn, &gr};
  const unsigned parts = (unsigned)((Cfg::BM * Cfg::BN + 1023) / 1024);
  return hipLaunchKernel(reinterpret_cast<const void*>(&streamk_fixup_kernel), dim3(parts, (unsigned)plan.sk_tiles),
                         dim3(256), fargs, 0, stream);
}

}  // namespace

// Name: mfma32_<BM>x<BN>x<BK>_w<WM>x<WN>[_kg<KG>]_lds<STAGES>[_<ops>]: direct
// global-to-LDS staging with STAGES LDS buffers; _kg<KG> splits each slab's k
// range among KG wave groups; <ops> = tn, nt or tt names transposed operands
// (first letter A, second B), none the plain product.
#define SGEMM_MFMA_DMA_CFG(BM, BN, BK, WM, WN, KG, ST, TA, TB, SFX)                                      \
  {"mfma32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN SFX, KIND_MFMA, BM, BN, BK, 64 * WM * WN * KG, TA, TB,  \
   &launch_mfma_dma<DmaCfg<BM, BN, BK, WM, WN, ST, TA, TB, KG>>,                                         \
   reinterpret_cast<const void*>(&mfma_dma_kernel<DmaCfg<BM, BN, BK, WM, WN, ST, TA, TB, KG>, true>), KG, \
   nullptr, {nullptr, nullptr}}
// The one-wave-per-SIMD tile with the hand-ordered slab loop.
#define SGEMM_MFMA_DMA_SCHED_CFG(BM, BN, BK, WM, WN, TA, TB, SFX)                                          \
  {"mfma32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_lds2_sched" SFX, KIND_MFMA, BM, BN, BK, 64 * WM * WN, TA, TB, \
   &launch_mfma_dma<DmaSchedCfg<BM, BN, BK, WM, WN, TA, TB>>,                                              \
   reinterpret_cast<const void*>(&mfma_dma_kernel<DmaSchedCfg<BM, BN, BK, WM, WN, TA, TB>, true>), 1,      \
   nullptr, {nullptr, nullptr}}
#define SGEMM_MFMA_DMA_SCHED(BM, BN, BK, WM, WN) SGEMM_MFMA_DMA_SCHED_CFG(BM, BN, BK, WM, WN, 0, 0, "")
// ST stages (the name then reads _lds<ST>_sched), for each op pair.
#define SGEMM_MFMA_DMA_SCHED_ST_CFG(BM, BN, BK, WM, WN, ST, TA, TB, SFX)                                     \
  {"mfma32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_lds" #ST "_sched" SFX, KIND_MFMA, BM, BN, BK, 64 * WM * WN, \
   TA, TB, &launch_mfma_dma<DmaSchedCfg<BM, BN, BK, WM, WN, TA, TB, ST>>,                                     \
   reinterpret_cast<const void*>(&mfma_dma_kernel<DmaSchedCfg<BM, BN, BK, WM, WN, TA, TB, ST>, true>), 1,     \
   nullptr, {nullptr, nullptr}}
#define SGEMM_MFMA_DMA_SCHED_ST(BM, BN, BK, WM, WN, ST) SGEMM_MFMA_DMA_SCHED_ST_CFG(BM, BN, BK, WM, WN, ST, 0, 0, "")
#define SGEMM_MFMA_DMA_SCHED_ST_OPS(BM, BN, BK, WM, WN, ST)                  \
  SGEMM_MFMA_DMA_SCHED_ST_CFG(BM, BN, BK, WM, WN, ST, 1, 0, "_tn"),          \
      SGEMM_MFMA_DMA_SCHED_ST_CFG(BM, BN, BK, WM, WN, ST, 0, 1, "_nt"),      \
      SGEMM_MFMA_DMA_SCHED_ST_CFG(BM, BN, BK, WM, WN, ST, 1, 1, "_tt")
#define SGEMM_MFMA_DMA_SCHED_OPS(BM, BN, BK, WM, WN)                  \
  SGEMM_MFMA_DMA_SCHED_CFG(BM, BN, BK, WM, WN, 1, 0, "_tn"),          \
      SGEMM_MFMA_DMA_SCHED_CFG(BM, BN, BK, WM, WN, 0, 1, "_nt"),      \
      SGEMM_MFMA_DMA_SCHED_CFG(BM, BN, BK, WM, WN, 1, 1, "_tt")
// The hand-ordered loop staged through registers (_rs): no direct loads, so
// operands of any alignment; every slab and the K tail through registers.
#define SGEMM_MFMA_RS_SCHED_CFG(BM, BN, BK, WM, WN, TA, TB, SFX)                                               \
  {"mfma32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_rs_sched" SFX, KIND_MFMA, BM, BN, BK, 64 * WM * WN, TA, TB,    \
   &launch_mfma_rs<DmaSchedCfg<BM, BN, BK, WM, WN, TA, TB>>,                                                     \
   reinterpret_cast<const void*>(&mfma_dma_kernel<DmaSchedCfg<BM, BN, BK, WM, WN, TA, TB>, false>), 1, nullptr,   \
   {nullptr, nullptr}, 1}
#define SGEMM_MFMA_RS_SCHED(BM, BN, BK, WM, WN) SGEMM_MFMA_RS_SCHED_CFG(BM, BN, BK, WM, WN, 0, 0, "")
#define SGEMM_MFMA_RS_SCHED_OPS(BM, BN, BK, WM, WN)                  \
  SGEMM_MFMA_RS_SCHED_CFG(BM, BN, BK, WM, WN, 1, 0, "_tn"),          \
      SGEMM_MFMA_RS_SCHED_CFG(BM, BN, BK, WM, WN, 0, 1, "_nt"),      \
      SGEMM_MFMA_RS_SCHED_CFG(BM, BN, BK, WM, WN, 1, 1, "_tt")
// The same with a stream-K form (configurations without k groups).
#define SGEMM_MFMA_DMA_SK_CFG(BM, BN, BK, WM, WN, ST, TA, TB, SFX)                                         \
  {"mfma32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN SFX, KIND_MFMA, BM, BN, BK, 64 * WM * WN, TA, TB,        \
   &launch_mfma_dma<DmaCfg<BM, BN, BK, WM, WN, ST, TA, TB, 1>>,                                           \
   reinterpret_cast<const void*>(&mfma_dma_kernel<DmaCfg<BM, BN, BK, WM, WN, ST, TA, TB, 1>, true>), 1,    \
   &launch_mfma_dma_streamk<DmaCfg<BM, BN, BK, WM, WN, ST, TA, TB, 1>>,                                   \
   {reinterpret_cast<const void*>(&mfma_dma_streamk_kernel<DmaCfg<BM, BN, BK, WM, WN, ST, TA, TB, 1>, false>), \
    reinterpret_cast<const void*>(&mfma_dma_streamk_kernel<DmaCfg<BM, BN, BK, WM, WN, ST, TA, TB, 1>, true>)}}
#define SGEMM_MFMA_DMA(BM, BN, BK, WM, WN, ST) SGEMM_MFMA_DMA_SK_CFG(BM, BN, BK, WM, WN, ST, 0, 0, "_lds" #ST)
#define SGEMM_MFMA_DMA_OPS(BM, BN, BK, WM, WN, ST)                                  \
  SGEMM_MFMA_DMA_SK_CFG(BM, BN, BK, WM, WN, ST, 1, 0, "_lds" #ST "_tn"),            \
      SGEMM_MFMA_DMA_SK_CFG(BM, BN, BK, WM, WN, ST, 0, 1, "_lds" #ST "_nt"),        \
      SGEMM_MFMA_DMA_SK_CFG(BM, BN, BK, WM, WN, ST, 1, 1, "_lds" #ST "_tt")
#define SGEMM_MFMA_DMA_KG(BM, BN, BK, WM, WN, KG, ST) \
  SGEMM_MFMA_DMA_CFG(BM, BN, BK, WM, WN, KG, ST, 0, 0, "_kg" #KG "_lds" #ST)
#define SGEMM_MFMA_DMA_KG_OPS(BM, BN, BK, WM, WN, KG, ST)                                  \
  SGEMM_MFMA_DMA_CFG(BM, BN, BK, WM, WN, KG, ST, 1, 0, "_kg" #KG "_lds" #ST "_tn"),        \
      SGEMM_MFMA_DMA_CFG(BM, BN, BK, WM, WN, KG, ST, 0, 1, "_kg" #KG "_lds" #ST "_nt"),    \
      SGEMM_MFMA_DMA_CFG(BM, BN, BK, WM, WN, KG, ST, 1, 1, "_kg" #KG "_lds" #ST "_tt")

KernelConfig kMfmaDmaConfigs[] = {
    // 256x256 block tile, 16 waves of 64x64, two stages: one workgroup per CU
    SGEMM_MFMA_DMA(256, 256, 16, 4, 4, 2),
    SGEMM_MFMA_DMA_OPS(256, 256, 16, 4, 4, 2),
    // smaller tiles of 64x64 wave tiles, several workgroups per CU: mid-size
    // shapes whose 256x256 grid leaves compute units idle or a last wave thin
    SGEMM_MFMA_DMA(128, 128, 16, 2, 2, 2),
    SGEMM_MFMA_DMA_OPS(128, 128, 16, 2, 2, 2),
    SGEMM_MFMA_DMA(256, 128, 16, 4, 2, 2),
    SGEMM_MFMA_DMA_OPS(256, 128, 16, 4, 2, 2),
    SGEMM_MFMA_DMA(128, 256, 16, 2, 4, 2),
    SGEMM_MFMA_DMA_OPS(128, 256, 16, 2, 4, 2),
    // k groups: more waves on the small tiles of long-K shapes
    SGEMM_MFMA_DMA_KG(64, 64, 64, 2, 2, 2, 2),
    SGEMM_MFMA_DMA_KG(32, 32, 128, 1, 1, 4, 2),
    SGEMM_MFMA_DMA_KG_OPS(32, 32, 128, 1, 1, 4, 2),
    SGEMM_MFMA_DMA_KG(32, 32, 256, 1, 1, 8, 2),
    SGEMM_MFMA_DMA_KG_OPS(32, 32, 256, 1, 1, 8, 2),
    // deeper pipelines: loads two or three slabs ahead
    SGEMM_MFMA_DMA_CFG(256, 256, 16, 4, 4, 1, 4, 0, 0, "_lds4"),
    SGEMM_MFMA_DMA_CFG(64, 64, 32, 2, 2, 1, 4, 0, 0, "_lds4"),
    SGEMM_MFMA_DMA_CFG(64, 64, 64, 2, 2, 1, 3, 0, 0, "_lds3"),
    SGEMM_MFMA_DMA_SCHED(256, 256, 32, 2, 2),
    SGEMM_MFMA_DMA_SCHED_OPS(256, 256, 32, 2, 2),
    SGEMM_MFMA_DMA_SCHED_ST(64, 64, 32, 2, 2, 4),
    SGEMM_MFMA_DMA_SCHED_ST_OPS(64, 64, 32, 2, 2, 4),
    SGEMM_MFMA_DMA_SCHED_ST(64, 64, 64, 2, 2, 3),
    SGEMM_MFMA_DMA_SCHED_ST_OPS(64, 64, 64, 2, 2, 3),
    // 128x128 tiles of four 64x64 waves: mid-size products (2048^3: 256 tiles)
    SGEMM_MFMA_DMA_SCHED_ST(128, 128, 32, 2, 2, 4),
    SGEMM_MFMA_DMA_SCHED_ST(128, 128, 64, 2, 2, 2),
    SGEMM_MFMA_DMA_SCHED_ST_OPS(128, 128, 64, 2, 2, 2),
    // 256x128 tiles of four 128x64 waves
    SGEMM_MFMA_DMA_SCHED_ST(256, 128, 32, 2, 2, 2),
    SGEMM_MFMA_DMA_SCHED_ST(192, 128, 32, 2, 2, 2),
    SGEMM_MFMA_DMA_SCHED_ST(192, 128, 32, 2, 2, 3),
    // hand-ordered tiles staged through registers: any alignment
    SGEMM_MFMA_RS_SCHED(192, 128, 32, 2, 2),
    SGEMM_MFMA_RS_SCHED_OPS(192, 128, 32, 2, 2),
};
const int kNumMfmaDmaConfigs = sizeof(kMfmaDmaConfigs) / sizeof(kMfmaDmaConfigs[0]);

}  // namespace sgemm_impl
