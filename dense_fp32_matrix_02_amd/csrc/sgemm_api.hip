// Host side of the C ABI declared in include/sgemm_mi355.h: argument
// validation (pure host code, before any HIP call), tile-configuration
// selection and the kernel launch on the caller's stream. No allocation, no
// synchronisation, no mutable global state.

#include "sgemm_mi355.h"

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "sgemm_internal.h"

namespace sgemm_impl {
namespace {

// The measured tile table (tile_table.inc, written by tune.py): per op pair,
// the candidate configurations with their occupancy, the measured shapes,
// and each candidate's median time at each shape (0: not a candidate there).
struct TableConfig {
  const char* name;
  int occupancy;  // workgroups one compute unit holds at once
};
struct TableShape {
  int M, N, K;
};
struct TableNorm {
  const char* name;
  int occupancy;
  float us_per_busy;  // median over the measured shapes of time / busy_time
};
struct TableBlock {
  int opA, opB;
  int ncand, nshapes;
  const TableConfig* cand;
  const TableShape* shapes;
  const float* times_us;  // nshapes x ncand, row-major
  int nnorm;
  const TableNorm* norms;  // every configuration of the op pair
  // stream-K forms: microseconds per slab of the evenly dealt work (beyond
  // kStreamKOverheadUs, the store of C counted as kStoreDepth / BK slabs per
  // tile), median over the stream-K grid
  int nstreamk;
  const TableNorm* streamk;
};
struct SplitShape {
  int M, N, K;
  int splits;  // the fastest split count measured there
};
#include "tile_table.inc"
constexpr int kNumTableBlocks = sizeof(kTableBlocks) / sizeof(kTableBlocks[0]);
constexpr int kNumSplitShapes = sizeof(kSplitShapes) / sizeof(kSplitShapes[0]) - 1;  // without the sentinel

// Index of the shape nearest (M, N, K) in (log M, log N, log K), summed
// absolute distance, among those within a factor of two in every dimension
// (the first on a tie); -1 when none qualifies.
template <class Shape>
int nearest_shape(const Shape* shapes, int count, int M, int N, int K) {
  int near = -1;
  double near_d = 1e30;
  for (int s = 0; s < count; ++s) {
    const Shape& e = shapes[s];
    // within a factor of two in every dimension (integer test before any log)
    if ((int64_t)M > 2LL * e.M || (int64_t)e.M > 2LL * M || (int64_t)N > 2LL * e.N ||
        (int64_t)e.N > 2LL * N || (int64_t)K > 2LL * e.K || (int64_t)e.K > 2LL * K)
      continue;
    const double d = std::fabs(std::log2((double)M / e.M)) + std::fabs(std::log2((double)N / e.N)) +
                     std::fabs(std::log2((double)K / e.K));
    if (d < near_d) {
      near_d = d;
      near = s;
    }
  }
  return near;
}

constexpr int kCompute = 256;  // compute units on MI355X

// Block tiles of the selection rule, per operand pair (plain, op(A) = A^T,
// op(B) = B^T, both), largest first, each with the fewest workgroups
// (counting batch entries) it needs to be chosen. The rule picks the tile of
// split-K chunk products, and stands in for the measured table only if that
// has nothing for an op pair. A tile is also skipped when the matrix would
// fill less than kRuleMinFill of its padded tile grid (a batch of 64x64
// products in 256x128 tiles computes 8 times the useful work). Below the last
// threshold, a 32x32 tile with its slabs split among wave groups keeps the
// SIMDs busy; long K takes the deeper one. The thresholds were fitted to the
// measured grid (about 2% slower than the best configuration there,
// geometric mean) and to strided batches of 64^3 to 1024^3 products.
struct RuleTile {
  const char* config;
  int min_wgs;
};
const RuleTile kRulePlain[] = {{"mfma32_256x128x16_w4x2", 256},
                               {"mfma32_128x64x16_w2x2", 768},
                               {"mfma32_64x64x32_w2x2", 1024},
                               {"mfma32_64x64x64_w2x2_kg2", 256}};
const RuleTile kRuleTN[] = {{"mfma32_256x256x16_w4x4_ak_tn", 256},
                            {"mfma32_256x128x16_w4x2_tn", 256},
                            {"mfma32_128x64x16_w2x2_tn", 512},
                            {"mfma32_64x64x64_w2x2_kg2_tn", 256}};
const RuleTile kRuleNT[] = {{"mfma32_256x256x32_w4x4_nt", 256},
                            {"mfma32_256x128x16_w4x2_nt", 256},
                            {"mfma32_128x64x16_w2x2_nt", 512},
                            {"mfma32_64x64x64_w2x2_kg2_nt", 256}};
const RuleTile kRuleTT[] = {{"mfma32_256x256x16_w4x4_tt", 256},
                            {"mfma32_256x128x16_w4x2_tt", 256},
                            {"mfma32_128x64x16_w2x2_tt", 512},
                            {"mfma32_64x64x64_w2x2_kg2_tt", 256}};
const RuleTile* const kRuleTiles[2][2] = {{kRulePlain, kRuleNT}, {kRuleTN, kRuleTT}};
constexpr int kRuleTileCount = 4;
const char* const kRuleSmall = "32x32x128_w1x1_kg4";
const char* const kRuleSmallLongK = "32x32x256_w1x1_kg16";
constexpr int kRuleLongK = 4096;
constexpr double kRuleMinFill = 0.75;

// Configuration ids: the register-staged matrix-core kernels, then the
// direct-to-LDS ones, then the vector kernels.
int num_configs() { return kNumMfmaConfigs + kNumMfmaDmaConfigs + kNumValuConfigs; }

const KernelConfig* config_at(int id) {
  if (id < 0) return nullptr;
  if (id < kNumMfmaConfigs) return &kMfmaConfigs[id];
  id -= kNumMfmaConfigs;
  if (id < kNumMfmaDmaConfigs) return &kMfmaDmaConfigs[id];
  id -= kNumMfmaDmaConfigs;
  if (id < kNumValuConfigs) return &kValuConfigs[id];
  return nullptr;
}

int config_id(const char* name) {
  for (int i = 0; i < num_configs(); ++i)
    if (std::strcmp(config_at(i)->name, name) == 0) return i;
  return -1;
}

int64_t tiles_for(const KernelConfig& c, int M, int N) {
  return ((int64_t)M + c.bm - 1) / c.bm * (((int64_t)N + c.bn - 1) / c.bn);
}

const char* ops_suffix(int opA, int opB) {
  static const char* const s[2][2] = {{"", "_nt"}, {"_tn", "_tt"}};
  return s[opA][opB];
}

// The selection's data, resolved once per process (a function-local static:
// initialised on first use, thread-safe, never written afterwards), so a call
// costs no string comparisons: the rule's configuration ids and, per op pair,
// the table's candidates (id, occupancy, and each measured time divided by
// the busy time at its own shape, 0 where not a candidate) and every
// configuration's id, occupancy and median time per busy unit.
struct ResolvedBlock {
  const TableBlock* src = nullptr;
  int ids[64];
  int occ[64];
  std::vector<double> norm;  // nshapes x ncand
  // every configuration of the op pair: id, occupancy, median time per busy unit
  std::vector<int> gid, gocc;
  std::vector<double> gnorm;
  // stream-K forms: id, occupancy, microseconds per slab
  std::vector<int> skid, skocc;
  std::vector<double> sknorm;
};

struct Resolved {
  int rule[2][2][kRuleTileCount];  // -1 where a configuration is not built
  int small[2][2][2];              // [opA][opB][long K]
  ResolvedBlock block[2][2];
};

bool is_direct_config(int id) {
  return id >= kNumMfmaConfigs && id < kNumMfmaConfigs + kNumMfmaDmaConfigs &&
         !kMfmaDmaConfigs[id - kNumMfmaConfigs].staged;
}

// Fill model of a launch of configuration c on an M x N x K problem (batch
// entries in grid.y): workgroups are dealt round-robin over the XCDs and
// their compute units, so the busiest CU gets n = ceil(workgroups / 256) of
// them. It runs them `occ` at a time, at full rate only while at least
// kSatChains independent 32x32 accumulator blocks are resident (two per
// SIMD, so one block's matrix instructions, or its wave's loads, overlap
// another's); with b < kSatChains resident, a workgroup takes kSatChains / b
// times as long. A workgroup holds kgroups * (BM/32) * (BN/32) blocks. Its
// store of C counts as kStoreDepth more steps of k: with every CU storing,
// a CU's share of the 8 TB/s writes a BM x BN tile of 4-byte values in the
// time its share of the 157.3 TFLOP/s peak spends on 2 * BM * BN * 39 flops.
// The busy time, in units of one workgroup slab step at full rate, is
//   n * max(1, kSatChains / (min(n, occ) * blocks per workgroup))
//     * (ceil(K / BK) + kStoreDepth / BK).
constexpr int kSatChains = 8;
constexpr double kStoreDepth = 40.0;

// Evaluated in double: the workgroup count (up to 2^52 tiles of 32 x 32 times
// 65535 batch entries) can exceed int64 for shapes the selection is asked
// about before validation.
double busy_time(const KernelConfig& c, int occ, int M, int N, int K, int batch) {
  const double wgs = (double)tiles_for(c, M, N) * (double)(batch < kMaxGridY ? batch : kMaxGridY);
  const double n = std::ceil(wgs / kCompute);
  if (!(n > 0.0)) return 0.0;
  const double blocks = (double)(c.kgroups > 0 ? c.kgroups : 1) * (c.bm / 32) * (c.bn / 32);
  const double resident = (n < occ ? n : (double)occ) * blocks;
  const double stretch = resident >= kSatChains ? 1.0 : (double)kSatChains / resident;
  return n * stretch * ((double)(((int64_t)K + c.bk - 1) / c.bk) + kStoreDepth / c.bk);
}

const Resolved& resolved() {
  static const Resolved r = [] {
    Resolved x;
    for (int a = 0; a < 2; ++a)
      for (int b = 0; b < 2; ++b) {
        for (int i = 0; i < kRuleTileCount; ++i) x.rule[a][b][i] = config_id(kRuleTiles[a][b][i].config);
        for (int l = 0; l < 2; ++l) {
          char name[64];
          std::snprintf(name, sizeof(name), "mfma32_%s%s", l ? kRuleSmallLongK : kRuleSmall, ops_suffix(a, b));
          x.small[a][b][l] = config_id(name);
        }
      }
    for (int t = 0; t < kNumTableBlocks; ++t) {
      const TableBlock& tb = kTableBlocks[t];
      if (tb.opA < 0 || tb.opA > 1 || tb.opB < 0 || tb.opB > 1 || tb.ncand > 64) continue;
      ResolvedBlock& rb = x.block[tb.opA][tb.opB];
      rb.src = &tb;
      for (int c = 0; c < tb.ncand; ++c) {
        int id = config_id(tb.cand[c].name);
        const KernelConfig* cfg = config_at(id);
        if (cfg && (cfg->transA != tb.opA || cfg->transB != tb.opB || cfg->kind != KIND_MFMA)) id = -1;
        rb.ids[c] = id;
        rb.occ[c] = tb.cand[c].occupancy > 0 ? tb.cand[c].occupancy : 1;
      }
      for (int c = 0; c < tb.nnorm; ++c) {
        const int id = config_id(tb.norms[c].name);
        const KernelConfig* cfg = config_at(id);
        if (!cfg || cfg->transA != tb.opA || cfg->transB != tb.opB || cfg->kind != KIND_MFMA ||
            !(tb.norms[c].us_per_busy > 0.0f))
          continue;
        rb.gid.push_back(id);
        rb.gocc.push_back(tb.norms[c].occupancy > 0 ? tb.norms[c].occupancy : 1);
        rb.gnorm.push_back(tb.norms[c].us_per_busy);
      }
      for (int c = 0; c < tb.nstreamk && tb.streamk; ++c) {
        const int id = config_id(tb.streamk[c].name);
        const KernelConfig* cfg = config_at(id);
        if (!cfg || cfg->transA != tb.opA || cfg->transB != tb.opB || cfg->streamk == nullptr ||
            !(tb.streamk[c].us_per_busy > 0.0f))
          continue;
        rb.skid.push_back(id);
        rb.skocc.push_back(tb.streamk[c].occupancy > 0 ? tb.streamk[c].occupancy : 1);
        rb.sknorm.push_back(tb.streamk[c].us_per_busy);
      }
      rb.norm.assign((size_t)tb.nshapes * tb.ncand, 0.0);
      for (int s = 0; s < tb.nshapes; ++s) {
        const TableShape& e = tb.shapes[s];
        for (int c = 0; c < tb.ncand; ++c) {
          const float t_us = tb.times_us[(size_t)s * tb.ncand + c];
          const KernelConfig* cfg = config_at(rb.ids[c]);
          if (cfg && t_us > 0.0f)
            rb.norm[(size_t)s * tb.ncand + c] = t_us / busy_time(*cfg, rb.occ[c], e.M, e.N, e.K, 1);
        }
      }
    }
    return x;
  }();
  return r;
}

// The first rule tile whose grid reaches its workgroup threshold, else the
// small k-group tile for this K.
int rule_select(int opA, int opB, int M, int N, int K, int batch) {
  const int64_t gy = batch < kMaxGridY ? batch : kMaxGridY;
  const Resolved& rs = resolved();
  for (int i = 0; i < kRuleTileCount; ++i) {
    const int id = rs.rule[opA][opB][i];
    if (id < 0) continue;
    const KernelConfig& c = *config_at(id);
    const int64_t n = tiles_for(c, M, N);
    const double fill = n > 0 ? (double)M * N / ((double)n * c.bm * c.bn) : 1.0;
    if ((double)n * (double)gy >= kRuleTiles[opA][opB][i].min_wgs && fill >= kRuleMinFill) return id;
  }
  return rs.small[opA][opB][K >= kRuleLongK ? 1 : 0];
}

// Whether direct-to-LDS configuration c takes its direct path on this
// problem (its launcher's condition, with `aligned` standing for the pointer,
// leading-dimension and stride alignment): K of at least one slab (a last,
// partial slab goes through registers at the end), and for a line-contiguous
// operand an extent that is a multiple of 4. Otherwise it stages every slab
// through registers, which its measured times do not describe.
bool direct_path(const KernelConfig& c, int M, int N, int K, bool aligned) {
  return aligned && M > 0 && N > 0 && K >= c.bk && (!c.transA || M % 4 == 0) && (c.transB || N % 4 == 0);
}


// Model selection for a single product: the measured shape of this op pair
// nearest (M, N, K) in (log M, log N, log K), among those within a factor of
// two in every dimension (the first on a tie); then the candidate with the
// least predicted time, each candidate's measured time there scaled by the
// ratio of busy_time at (M, N, K) to busy_time at the measured shape (the
// first on a tie). -1 when no measured shape qualifies.
int model_select(int opA, int opB, int M, int N, int K, bool aligned, double* predicted_us = nullptr) {
  if (M <= 0 || N <= 0 || K <= 0) return -1;
  const ResolvedBlock& rb = resolved().block[opA][opB];
  if (!rb.src) return -1;
  const TableBlock& tb = *rb.src;
  const int near = nearest_shape(tb.shapes, tb.nshapes, M, N, K);
  if (near < 0) return -1;
  int best = -1;
  double best_t = 0.0;
  for (int c = 0; c < tb.ncand; ++c) {
    const double norm = rb.norm[(size_t)near * tb.ncand + c];
    if (norm <= 0.0) continue;
    const int id = rb.ids[c];
    const KernelConfig& cfg = *config_at(id);
    if (is_direct_config(id) && !direct_path(cfg, M, N, K, aligned)) continue;
    const double t = norm * busy_time(cfg, rb.occ[c], M, N, K, 1);
    if (best < 0 || t < best_t) {
      best = id;
      best_t = t;
    }
  }
  if (predicted_us) *predicted_us = best_t;
  return best;
}

// Selection for batches, and for single products with no measured shape
// nearby: every configuration of the op pair, each predicted as its median
// time per unit of busy time over the measured shapes times busy_time for
// this problem (batch entries included); the least predicted time wins (the
// first on a tie). Direct-to-LDS configurations count only when the problem
// takes their direct path. -1 when the table has no configuration for the
// op pair. Over 26 measured batches (2 x 2048^3 to 4096 x 16x16x64) it
// picks a configuration within 0.945 of the best (geometric mean), against
// 0.836 for the rule.
int global_select(int opA, int opB, int M, int N, int K, int batch, bool aligned,
                  double* predicted_us = nullptr) {
  if (M <= 0 || N <= 0 || K <= 0 || batch <= 0) return -1;
  const ResolvedBlock& rb = resolved().block[opA][opB];
  int best = -1;
  double best_t = 0.0;
  for (size_t c = 0; c < rb.gid.size(); ++c) {
    const int id = rb.gid[c];
    const KernelConfig& cfg = *config_at(id);
    if (is_direct_config(id) && !direct_path(cfg, M, N, K, aligned)) continue;
    const double t = rb.gnorm[c] * busy_time(cfg, rb.gocc[c], M, N, K, batch);
    if (best < 0 || t < best_t) {
      best = id;
      best_t = t;
    }
  }
  if (predicted_us) *predicted_us = best_t;
  return best;
}

// Single products near a measured shape take the model selection; batches,
// and shapes with no measured shape nearby, the median-time model; the rule
// only if the table has nothing for the op pair (or the problem is empty).
int select_mfma(int opA, int opB, int M, int N, int K, int batch, bool aligned = true) {
  int id = batch == 1 ? model_select(opA, opB, M, N, K, aligned) : -1;
  if (id < 0) id = global_select(opA, opB, M, N, K, batch, aligned);
  return id >= 0 ? id : rule_select(opA, opB, M, N, K, batch);
}

// Vector-kernel configurations the selection considers, largest block tile
// first (the fastest measured configuration of each tile size): the largest
// that still gives one workgroup per compute unit, else the smallest.
const char* const kValuRuleTiles[] = {"valu8x8_128x128x8", "valu8x8_64x64x16"};

int select_valu(int M, int N) {
  static const int ids[2] = {config_id(kValuRuleTiles[0]), config_id(kValuRuleTiles[1])};
  int last = -1;
  for (const int id : ids) {
    if (id < 0) continue;
    last = id;
    if (tiles_for(*config_at(id), M, N) >= kCompute) return id;
  }
  return last;
}

bool overlaps(const void* p, unsigned __int128 pbytes, const void* q, unsigned __int128 qbytes) {
  const unsigned __int128 a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + qbytes && b < a + pbytes;
}

struct Problem {
  int opA, opB, M, N, K;
  float alpha;
  const float* A;
  int lda;
  long long strideA;
  const float* B;
  int ldb;
  long long strideB;
  float beta;
  const float* C;
  int ldc;
  long long strideC;
  int batch;
};

int validate(const Problem& p) {
  if ((p.opA != 0 && p.opA != 1) || (p.opB != 0 && p.opB != 1)) return SGEMM_MI355_ERR_OP;
  if (p.M < 0 || p.N < 0 || p.K < 0 || p.batch < 0) return SGEMM_MI355_ERR_DIM;
  // Rows of the stored matrices: A is M x K (opA = N) or K x M (opA = T).
  const int a_cols = p.opA ? p.M : p.K, a_rows = p.opA ? p.K : p.M;
  const int b_cols = p.opB ? p.K : p.N, b_rows = p.opB ? p.N : p.K;
  if (p.lda < (a_cols > 1 ? a_cols : 1) || p.ldb < (b_cols > 1 ? b_cols : 1) ||
      p.ldc < (p.N > 1 ? p.N : 1))
    return SGEMM_MI355_ERR_LD;
  if (p.strideA < 0 || p.strideB < 0 || p.strideC < 0) return SGEMM_MI355_ERR_STRIDE;
  const unsigned __int128 c_elems =
      (p.M > 0 && p.N > 0) ? (unsigned __int128)(p.M - 1) * (unsigned)p.ldc + (unsigned)p.N : 0;
  if (p.batch > 1 && (unsigned __int128)p.strideC < c_elems) return SGEMM_MI355_ERR_STRIDE;
  if (p.M == 0 || p.N == 0 || p.batch == 0) return SGEMM_MI355_OK;
  const bool uses_ab = p.alpha != 0.0f && p.K > 0;
  if (p.C == nullptr) return SGEMM_MI355_ERR_NULL;
  if (uses_ab && (p.A == nullptr || p.B == nullptr)) return SGEMM_MI355_ERR_NULL;
  if (((uintptr_t)p.C & 3) != 0) return SGEMM_MI355_ERR_ALIGN;
  if (uses_ab && ((((uintptr_t)p.A) | ((uintptr_t)p.B)) & 3) != 0) return SGEMM_MI355_ERR_ALIGN;
  // Row and column numbers stay 32-bit ints inside the kernels with one
  // block tile of headroom; byte extents must fit the address space.
  if (p.M > INT_MAX - 1024 || p.N > INT_MAX - 1024 || p.K > INT_MAX - 1024)
    return SGEMM_MI355_ERR_EXTENT;
  const unsigned __int128 nb = (unsigned __int128)(p.batch - 1);
  const unsigned __int128 c_bytes = 4 * (nb * (unsigned long long)p.strideC + c_elems);
  const unsigned __int128 limit = (unsigned __int128)1 << 62;
  if (c_bytes > limit) return SGEMM_MI355_ERR_EXTENT;
  if (uses_ab) {
    const unsigned __int128 a_elems = (unsigned __int128)(a_rows - 1) * (unsigned)p.lda + (unsigned)a_cols;
    const unsigned __int128 b_elems = (unsigned __int128)(b_rows - 1) * (unsigned)p.ldb + (unsigned)b_cols;
    const unsigned __int128 a_bytes = 4 * (nb * (unsigned long long)p.strideA + a_elems);
    const unsigned __int128 b_bytes = 4 * (nb * (unsigned long long)p.strideB + b_elems);
    if (a_bytes > limit || b_bytes > limit) return SGEMM_MI355_ERR_EXTENT;
    if (overlaps(p.C, c_bytes, p.A, a_bytes) || overlaps(p.C, c_bytes, p.B, b_bytes))
      return SGEMM_MI355_ERR_ALIAS;
  }
  return SGEMM_MI355_OK;
}

// Launch `cfg` (or the C = beta*C kernel) over all batch entries of g, one
// launch per kMaxGridY entries; the last entry of the whole batch has
// K = g.k_last.
hipError_t launch_batches(const KernelConfig* cfg, const GemmArgs& g, bool scale_only,
                          hipStream_t stream) {
  for (int b0 = 0; b0 < g.batch; b0 += kMaxGridY) {
    GemmArgs gc = g;
    gc.batch = (g.batch - b0) < kMaxGridY ? (g.batch - b0) : kMaxGridY;
    gc.C = g.C + (int64_t)b0 * g.strideC;
    gc.k_last = (b0 + gc.batch == g.batch) ? g.k_last : g.K;
    if (!scale_only) {
      gc.A = g.A + (int64_t)b0 * g.strideA;
      gc.B = g.B + (int64_t)b0 * g.strideB;
    }
    const hipError_t err = scale_only ? launch_scale_c(gc, stream) : cfg->launch(gc, stream);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

int run(const Problem& p, float* C, hipStream_t stream, int config) {
  const int v = validate(p);
  if (v != SGEMM_MI355_OK) return v;
  const KernelConfig* cfg = config_at(config);
  if (cfg == nullptr || cfg->transA != p.opA || cfg->transB != p.opB) return SGEMM_MI355_ERR_CONFIG;
  if (p.M == 0 || p.N == 0 || p.batch == 0) return SGEMM_MI355_OK;
  const GemmArgs g{p.M,     p.N,       p.K,       p.A,       p.lda,     p.B,      p.ldb,
                   C,       p.ldc,     p.alpha,   p.beta,    p.strideA, p.strideB, p.strideC,
                   p.batch, p.K};
  const bool scale_only = (p.K == 0 || p.alpha == 0.0f);
  if (!scale_only && tiles_for(*cfg, p.M, p.N) * cfg->threads > (int64_t)UINT32_MAX)
    return SGEMM_MI355_ERR_EXTENT;
  return launch_batches(cfg, g, scale_only, stream) == hipSuccess ? SGEMM_MI355_OK
                                                                  : SGEMM_MI355_ERR_LAUNCH;
}

// ---- split-K -----------------------------------------------------------------
// K is cut into `splits` chunks of kchunk values (a multiple of 32; the last
// chunk takes the rest). Chunk s multiplies op(A)[:, s*kchunk ...] by
// op(B)[s*kchunk ..., :] into the dense M x N partial W_s of the caller's
// workspace (one strided-batched launch, batch entry = chunk), then one
// reduction kernel forms C = alpha * (W_0 + W_1 + ...) + beta * C, adding the
// partials in ascending order so repeated calls give identical bits.

constexpr int kMaxSplits = 256;

struct SplitPlan {
  int splits;  // effective number of chunks (<= requested)
  int kchunk;
  int k_last;
};

SplitPlan plan_splits(int K, int splits) {
  if (splits < 1) splits = 1;
  if (K <= 0) return SplitPlan{1, K, K};
  int64_t kc = ((int64_t)K + splits - 1) / splits;
  kc = (kc + 31) / 32 * 32;
  const int eff = (int)(((int64_t)K + kc - 1) / kc);
  if (eff <= 1) return SplitPlan{1, K, K};
  return SplitPlan{eff, (int)kc, (int)(K - (int64_t)(eff - 1) * kc)};
}

uint64_t splitk_bytes(int M, int N, int splits) {
  return (M > 0 && N > 0 && splits > 1) ? 4ull * (uint64_t)splits * (uint64_t)M * (uint64_t)N : 0;
}

int run_splitk(const Problem& p, float* C, int splits, float* W, size_t w_bytes, hipStream_t stream,
               int config) {
  if (splits < 1 || splits > kMaxSplits) return SGEMM_MI355_ERR_DIM;
  const int v = validate(p);
  if (v != SGEMM_MI355_OK) return v;
  const SplitPlan sp = plan_splits(p.K, splits);
  const bool uses_ab = p.alpha != 0.0f && p.K > 0 && p.M > 0 && p.N > 0;
  if (!uses_ab || sp.splits == 1) return run(p, C, stream, config);
  const KernelConfig* cfg = config_at(config);
  if (cfg == nullptr || cfg->transA != p.opA || cfg->transB != p.opB) return SGEMM_MI355_ERR_CONFIG;
  const uint64_t need = splitk_bytes(p.M, p.N, sp.splits);
  if (W == nullptr) return SGEMM_MI355_ERR_NULL;
  if (((uintptr_t)W & 3) != 0) return SGEMM_MI355_ERR_ALIGN;
  if ((uint64_t)w_bytes < need) return SGEMM_MI355_ERR_WORKSPACE;
  // The workspace may not overlap A, B or C.
  const unsigned __int128 a_bytes =
      4 * ((unsigned __int128)((p.opA ? p.K : p.M) - 1) * (unsigned)p.lda + (unsigned)(p.opA ? p.M : p.K));
  const unsigned __int128 b_bytes =
      4 * ((unsigned __int128)((p.opB ? p.N : p.K) - 1) * (unsigned)p.ldb + (unsigned)(p.opB ? p.K : p.N));
  const unsigned __int128 c_bytes = 4 * ((unsigned __int128)(p.M - 1) * (unsigned)p.ldc + (unsigned)p.N);
  if (overlaps(W, need, p.A, a_bytes) || overlaps(W, need, p.B, b_bytes) || overlaps(W, need, C, c_bytes))
    return SGEMM_MI355_ERR_ALIAS;
  if (tiles_for(*cfg, p.M, p.N) * cfg->threads > (int64_t)UINT32_MAX) return SGEMM_MI355_ERR_EXTENT;
  const int64_t plane = (int64_t)p.M * p.N;
  const GemmArgs g{p.M,
                   p.N,
                   sp.kchunk,
                   p.A,
                   p.lda,
                   p.B,
                   p.ldb,
                   W,
                   p.N,
                   1.0f,
                   0.0f,
                   p.opA ? (int64_t)sp.kchunk * p.lda : (int64_t)sp.kchunk,
                   p.opB ? (int64_t)sp.kchunk : (int64_t)sp.kchunk * p.ldb,
                   plane,
                   sp.splits,
                   sp.k_last};
  if (launch_batches(cfg, g, false, stream) != hipSuccess) return SGEMM_MI355_ERR_LAUNCH;
  if (launch_splitk_reduce(W, sp.splits, p.M, p.N, p.alpha, p.beta, C, p.ldc, stream) != hipSuccess)
    return SGEMM_MI355_ERR_LAUNCH;
  return SGEMM_MI355_OK;
}

// Split count and tile for a problem. Near the measured split-K grid (M, N
// up to 2048 and K from 1024 to 65536, within a factor of two of a grid
// shape in every dimension), the fastest split count measured at the
// nearest grid shape: splitting pays where the tile grid leaves compute units
// idle or a thin last wave, in proportion to K (on the grid, from 4 splits of
// 64x64x1024 to 32 of 64x64x65536, none for 1024^2 at K <= 4096). Elsewhere a
// rule: split only when the unsplit grid has fewer than two workgroups per CU,
// into chunks of about kSplitChunk values of k (a power-of-two count). The
// grid was measured for the plain product; the transposed forms use it too.
// The chunk products take the rule's tile for the chunk shape.
constexpr int kSplitChunk = 1024;

void select_splitk(int opA, int opB, int M, int N, int K, int* splits, int* config) {
  const int single = select_mfma(opA, opB, M, N, K, 1);
  int s = 1;
  const int near = (M > 0 && N > 0 && K > 0) ? nearest_shape(kSplitShapes, kNumSplitShapes, M, N, K) : -1;
  if (near >= 0) {
    s = kSplitShapes[near].splits;
  } else if (tiles_for(*config_at(single), M, N) < 2 * kCompute) {
    while (2 * s <= kMaxSplits && (int64_t)K >= 2LL * s * kSplitChunk) s *= 2;
  }
  const SplitPlan sp = plan_splits(K, s);
  *splits = sp.splits;
  *config = sp.splits == 1 ? single : rule_select(opA, opB, M, N, sp.kchunk, sp.splits);
}

// ---- stream-K -----------------------------------------------------------------
// A persistent grid of (compute units x the stream-K kernel's occupancy)
// workgroups. The tiles of the whole rounds run whole; the slabs of the
// tiles of the last, partial round are dealt evenly to the grid, and a
// second kernel adds the partial sums of every tile split between
// workgroups (StreamKPlan in sgemm_internal.h). The workspace holds two
// BM x BN blocks per workgroup.

// Compute units of the current device (0 if the runtime cannot say).
int device_compute_units() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

// Workgroups of c's stream-K kernel (direct loads or register staging) one
// compute unit holds at once (0 if the runtime cannot say).
int streamk_occupancy(const KernelConfig& c, bool direct) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, c.streamk_kernel[direct ? 1 : 0], c.threads, 0) !=
      hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

// With direct loads and K not a whole number of slabs (ktail), the slabs dealt
// out are the whole ones; the kernel adds the rest of K in each tile's last
// piece.
StreamKPlan streamk_plan(const KernelConfig& c, int M, int N, int K, int grid, bool ktail) {
  const int64_t tiles = tiles_for(c, M, N);
  const int64_t dp = tiles / grid * grid;
  const int iters = ktail ? K / c.bk : (int)(((int64_t)K + c.bk - 1) / c.bk);
  return StreamKPlan{(int)dp, (int)(tiles - dp), iters, (tiles - dp) * iters, nullptr};
}

uint64_t streamk_bytes(const KernelConfig& c, int grid) { return 8ull * (uint64_t)grid * c.bm * c.bn; }

// Workspace c's stream-K form needs for an M x N x K product: the larger of
// its two kernels' needs, since alignment decides which one runs.
uint64_t streamk_need(const KernelConfig& c, int M, int N, int K) {
  if (tiles_for(c, M, N) > INT_MAX / 2) return 0;  // run_streamk rejects these (ERR_EXTENT)
  const int cus = device_compute_units();
  uint64_t need = 0;
  for (int d = 0; d < 2 && cus > 0 && M > 0 && N > 0 && K > 0; ++d) {
    const int occ = streamk_occupancy(c, d != 0);
    if (occ <= 0) continue;
    const int grid = cus * occ;
    const bool ktail = d != 0 && K >= c.bk && K % c.bk != 0;
    if (streamk_plan(c, M, N, K, grid, ktail).sk_tiles > 0 && streamk_bytes(c, grid) > need)
      need = streamk_bytes(c, grid);
  }
  return need;
}

bool operands_aligned(const Problem& p) {
  return ((reinterpret_cast<uintptr_t>(p.A) | reinterpret_cast<uintptr_t>(p.B)) & 15) == 0 &&
         ((p.lda | p.ldb) & 3) == 0 && (p.batch <= 1 || ((p.strideA | p.strideB) & 3) == 0);
}

// Whether a caller workspace of `need` bytes at W overlaps A, B or C of a
// single product.
bool workspace_overlaps(const Problem& p, const float* C, const float* W, uint64_t need) {
  const unsigned __int128 a_bytes =
      4 * ((unsigned __int128)((p.opA ? p.K : p.M) - 1) * (unsigned)p.lda + (unsigned)(p.opA ? p.M : p.K));
  const unsigned __int128 b_bytes =
      4 * ((unsigned __int128)((p.opB ? p.N : p.K) - 1) * (unsigned)p.ldb + (unsigned)(p.opB ? p.K : p.N));
  const unsigned __int128 c_bytes = 4 * ((unsigned __int128)(p.M - 1) * (unsigned)p.ldc + (unsigned)p.N);
  return overlaps(W, need, p.A, a_bytes) || overlaps(W, need, p.B, b_bytes) || overlaps(W, need, C, c_bytes);
}

int run_streamk(const Problem& p, float* C, float* W, size_t w_bytes, hipStream_t stream, int config) {
  const int v = validate(p);
  if (v != SGEMM_MI355_OK) return v;
  const KernelConfig* cfg = config_at(config);
  if (cfg == nullptr || cfg->transA != p.opA || cfg->transB != p.opB || cfg->streamk == nullptr)
    return SGEMM_MI355_ERR_CONFIG;
  if (p.M == 0 || p.N == 0) return SGEMM_MI355_OK;
  if (p.K == 0 || p.alpha == 0.0f) return run(p, C, stream, config);  // C = beta * C
  const bool direct = direct_path(*cfg, p.M, p.N, p.K, operands_aligned(p));
  const int cus = device_compute_units(), occ = streamk_occupancy(*cfg, direct);
  if (cus <= 0 || occ <= 0) return SGEMM_MI355_ERR_LAUNCH;
  if (tiles_for(*cfg, p.M, p.N) > INT_MAX / 2) return SGEMM_MI355_ERR_EXTENT;
  const int grid = cus * occ;
  StreamKPlan plan = streamk_plan(*cfg, p.M, p.N, p.K, grid, direct && p.K % cfg->bk != 0);
  if (plan.sk_tiles == 0) return run(p, C, stream, config);  // whole rounds only: the plain launch
  const uint64_t need = streamk_bytes(*cfg, grid);
  if (W == nullptr) return SGEMM_MI355_ERR_NULL;
  if (((uintptr_t)W & 15) != 0) return SGEMM_MI355_ERR_ALIGN;
  if ((uint64_t)w_bytes < need) return SGEMM_MI355_ERR_WORKSPACE;
  if (workspace_overlaps(p, C, W, need)) return SGEMM_MI355_ERR_ALIAS;
  plan.partials = W;
  const GemmArgs g{p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, C, p.ldc, p.alpha, p.beta, 0, 0, 0, 1, p.K};
  return cfg->streamk(g, plan, grid, direct, stream) == hipSuccess ? SGEMM_MI355_OK : SGEMM_MI355_ERR_LAUNCH;
}

// Stream-K selection. Each stream-K configuration of the op pair whose direct
// kernel would run (the register-staged stream-K kernels were slower than the
// plain path on every shape measured) and that leaves a partial last round is
// predicted as its measured time per slab (the table's stream-K block) times
// tiles * (slabs + kStoreDepth / BK) / kCompute (every tile's store of C
// counted as in busy_time), plus kStreamKOverheadUs: the partial sums, two
// BM x BN blocks per workgroup of the grid (occupancy x BM x BN is the same
// for every stream-K tile, 128 MiB on 256 compute units), the fixup kernel
// and its launch. The plain path's time is the larger of the nearest-shape
// and the median estimates for the configuration it would run: rescaled from
// a measured shape with a different fill, the first can be optimistic
// (1280 x 1280 x 32768: 0.71 ms predicted, 1.13 ms measured). Stream-K is
// chosen when it is predicted below kStreamKGain of that; otherwise -1.
// The time per slab was measured with K from 2048 up; like the nearest-shape
// lookup, the model is not carried beyond a factor of two of that, so K below
// kStreamKMinK keeps the plain path (at two slabs per tile, 10000 x 10000 x 30
// would take stream-K on a median estimate of 160 us where the plain path
// runs in 109).
constexpr double kStreamKOverheadUs = 40.0;
constexpr double kStreamKGain = 0.97;
constexpr int kStreamKMinK = 1024;

// The median model's estimate for configuration `id` (0 if the table has none).
double global_estimate(int opA, int opB, int id, int M, int N, int K) {
  const ResolvedBlock& rb = resolved().block[opA][opB];
  for (size_t c = 0; c < rb.gid.size(); ++c)
    if (rb.gid[c] == id) return rb.gnorm[c] * busy_time(*config_at(id), rb.gocc[c], M, N, K, 1);
  return 0.0;
}

int select_streamk(int opA, int opB, int M, int N, int K, bool aligned) {
  if (M <= 0 || N <= 0 || K < kStreamKMinK) return -1;
  double plain_us = 0.0;
  int plain = model_select(opA, opB, M, N, K, aligned, &plain_us);
  if (plain >= 0) {
    const double g = global_estimate(opA, opB, plain, M, N, K);
    if (g > plain_us) plain_us = g;
  } else {
    plain = global_select(opA, opB, M, N, K, 1, aligned, &plain_us);
  }
  if (plain < 0) return -1;
  const ResolvedBlock& rb = resolved().block[opA][opB];
  int best = -1;
  double best_t = 0.0;
  for (size_t c = 0; c < rb.skid.size(); ++c) {
    const int id = rb.skid[c];
    const KernelConfig& cfg = *config_at(id);
    if (!direct_path(cfg, M, N, K, aligned)) continue;
    const int64_t tiles = tiles_for(cfg, M, N);
    if (tiles % ((int64_t)kCompute * rb.skocc[c]) == 0) continue;  // whole rounds: nothing to split
    const double slabs =
        (double)tiles * ((double)(((int64_t)K + cfg.bk - 1) / cfg.bk) + kStoreDepth / cfg.bk) / kCompute;
    const double t = rb.sknorm[c] * slabs + kStreamKOverheadUs;
    if (best < 0 || t < best_t) {
      best = id;
      best_t = t;
    }
  }
  return (best >= 0 && best_t < kStreamKGain * plain_us) ? best : -1;
}

Problem plain(int M, int N, int K, const float* A, int lda, const float* B, int ldb, const float* C,
              int ldc) {
  return Problem{0, 0, M, N, K, 1.0f, A, lda, 0, B, ldb, 0, 0.0f, C, ldc, 0, 1};
}

int select_for(const Problem& p) {
  if (p.opA < 0 || p.opA > 1 || p.opB < 0 || p.opB > 1) return 0;
  const bool aligned = ((reinterpret_cast<uintptr_t>(p.A) | reinterpret_cast<uintptr_t>(p.B)) & 15) == 0 &&
                       ((p.lda | p.ldb) & 3) == 0 && (p.batch <= 1 || ((p.strideA | p.strideB) & 3) == 0);
  return select_mfma(p.opA, p.opB, p.M < 0 ? 0 : p.M, p.N < 0 ? 0 : p.N, p.K, p.batch < 1 ? 1 : p.batch,
                     aligned);
}

// ---- split-K without allocation -------------------------------------------
// The partial sums of sgemm_mi355_splitk_noalloc live in this file-scope
// device array instead of a caller workspace: every device the library runs
// on holds one copy of SGEMM_MI355_SCRATCH_BYTES until the process ends. In
// host code `scratch` names a host-side stand-in, not device memory; the
// device address of each device's copy comes from hipGetSymbolAddress, taken
// once per device with that device current and kept in scratch_ptr.
static __device__ __align__(256) float scratch[SGEMM_MI355_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
float* scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (device address), or an error code.
int current_scratch(float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return SGEMM_MI355_ERR_LAUNCH;
  }
  if (dev < 0 || dev >= kMaxDevices) return SGEMM_MI355_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return SGEMM_MI355_ERR_LAUNCH;
    }
    scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = scratch_ptr[dev];
  return SGEMM_MI355_OK;
}

}  // namespace
}  // namespace sgemm_impl

using namespace sgemm_impl;

extern "C" {

int sgemm_mi355(int M, int N, int K, const float* A, int lda, const float* B, int ldb, float* C,
                int ldc, hipStream_t stream) {
  const Problem p = plain(M, N, K, A, lda, B, ldb, C, ldc);
  return run(p, C, stream, select_for(p));
}

int sgemm_mi355_valu(int M, int N, int K, const float* A, int lda, const float* B, int ldb,
                     float* C, int ldc, hipStream_t stream) {
  const Problem p = plain(M, N, K, A, lda, B, ldb, C, ldc);
  return run(p, C, stream, select_valu(M < 0 ? 0 : M, N < 0 ? 0 : N));
}

int sgemm_mi355_with_config(int M, int N, int K, const float* A, int lda, const float* B, int ldb,
                            float* C, int ldc, hipStream_t stream, int config) {
  return run(plain(M, N, K, A, lda, B, ldb, C, ldc), C, stream, config);
}

int sgemm_mi355_ex(int opA, int opB, int M, int N, int K, float alpha, const float* A, int lda,
                   const float* B, int ldb, float beta, float* C, int ldc, hipStream_t stream) {
  const Problem p{opA, opB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1};
  return run(p, C, stream, select_for(p));
}

int sgemm_mi355_strided_batched(int opA, int opB, int M, int N, int K, float alpha,
                                const float* A, int lda, long long strideA, const float* B, int ldb,
                                long long strideB, float beta, float* C, int ldc,
                                long long strideC, int batch, hipStream_t stream) {
  const Problem p{opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC, batch};
  return run(p, C, stream, select_for(p));
}

int sgemm_mi355_strided_batched_with_config(int opA, int opB, int M, int N, int K, float alpha,
                                            const float* A, int lda, long long strideA,
                                            const float* B, int ldb, long long strideB, float beta,
                                            float* C, int ldc, long long strideC, int batch,
                                            hipStream_t stream, int config) {
  const Problem p{opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC, batch};
  return run(p, C, stream, config);
}

size_t sgemm_mi355_splitk_workspace_size(int M, int N, int K, int splits) {
  if (M <= 0 || N <= 0 || K <= 0 || splits < 1 || splits > kMaxSplits) return 0;
  return (size_t)splitk_bytes(M, N, plan_splits(K, splits).splits);
}

int sgemm_mi355_splitk(int opA, int opB, int M, int N, int K, float alpha, const float* A, int lda,
                       const float* B, int ldb, float beta, float* C, int ldc, int splits,
                       float* workspace, size_t workspace_bytes, hipStream_t stream) {
  const Problem p{opA, opB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1};
  if (validate(p) != SGEMM_MI355_OK) return validate(p);
  const SplitPlan sp = plan_splits(K, splits);
  const int config = sp.splits > 1 ? rule_select(opA, opB, M, N, sp.kchunk, sp.splits) : select_for(p);
  return run_splitk(p, C, splits, workspace, workspace_bytes, stream, config);
}

int sgemm_mi355_splitk_with_config(int opA, int opB, int M, int N, int K, float alpha,
                                   const float* A, int lda, const float* B, int ldb, float beta,
                                   float* C, int ldc, int splits, float* workspace,
                                   size_t workspace_bytes, hipStream_t stream, int config) {
  const Problem p{opA, opB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1};
  return run_splitk(p, C, splits, workspace, workspace_bytes, stream, config);
}

int sgemm_mi355_splitk_noalloc(int opA, int opB, int M, int N, int K, float alpha, const float* A, int lda,
                               const float* B, int ldb, float beta, float* C, int ldc, int splits,
                               hipStream_t stream) {
  const Problem p{opA, opB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1};
  const int v = validate(p);
  if (v != SGEMM_MI355_OK) return v;
  if (splits < 1 || splits > kMaxSplits) return SGEMM_MI355_ERR_DIM;
  const SplitPlan sp = plan_splits(K, splits);
  const int config = sp.splits > 1 ? rule_select(opA, opB, M, N, sp.kchunk, sp.splits) : select_for(p);
  const bool uses_ab = alpha != 0.0f && K > 0 && M > 0 && N > 0;
  const uint64_t need = uses_ab ? splitk_bytes(M, N, sp.splits) : 0;
  if (need == 0) return run_splitk(p, C, splits, nullptr, 0, stream, config);
  if (need > SGEMM_MI355_SCRATCH_BYTES) return SGEMM_MI355_ERR_SCRATCH;
  float* w = nullptr;
  const int e = current_scratch(&w);
  if (e != SGEMM_MI355_OK) return e;
  return run_splitk(p, C, splits, w, SGEMM_MI355_SCRATCH_BYTES, stream, config);
}

int sgemm_mi355_select_splitk(int opA, int opB, int M, int N, int K, int* splits, int* config) {
  if ((opA != 0 && opA != 1) || (opB != 0 && opB != 1)) return SGEMM_MI355_ERR_OP;
  if (M < 0 || N < 0 || K < 0) return SGEMM_MI355_ERR_DIM;
  if (!splits || !config) return SGEMM_MI355_ERR_NULL;
  select_splitk(opA, opB, M, N, K, splits, config);
  return SGEMM_MI355_OK;
}

size_t sgemm_mi355_streamk_workspace_size(int opA, int opB, int M, int N, int K, int config) {
  if ((opA != 0 && opA != 1) || (opB != 0 && opB != 1) || M <= 0 || N <= 0 || K <= 0) return 0;
  uint64_t need = 0;
  if (config >= 0) {
    const KernelConfig* c = config_at(config);
    if (c && c->streamk && c->transA == opA && c->transB == opB) need = streamk_need(*c, M, N, K);
  } else {
    for (int aligned = 0; aligned < 2; ++aligned) {  // the choice may depend on alignment
      const int id = select_streamk(opA, opB, M, N, K, aligned != 0);
      if (id >= 0) {
        const uint64_t n = streamk_need(*config_at(id), M, N, K);
        if (n > need) need = n;
      }
    }
  }
  return (size_t)need;
}

int sgemm_mi355_streamk(int opA, int opB, int M, int N, int K, float alpha, const float* A, int lda,
                        const float* B, int ldb, float beta, float* C, int ldc, float* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  const Problem p{opA, opB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1};
  const int v = validate(p);
  if (v != SGEMM_MI355_OK) return v;
  const int id = select_streamk(opA, opB, M, N, K, operands_aligned(p));
  return id >= 0 ? run_streamk(p, C, workspace, workspace_bytes, stream, id) : run(p, C, stream, select_for(p));
}

int sgemm_mi355_streamk_with_config(int opA, int opB, int M, int N, int K, float alpha,
                                    const float* A, int lda, const float* B, int ldb, float beta,
                                    float* C, int ldc, float* workspace, size_t workspace_bytes,
                                    hipStream_t stream, int config) {
  const Problem p{opA, opB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1};
  return run_streamk(p, C, workspace, workspace_bytes, stream, config);
}

int sgemm_mi355_select_streamk(int opA, int opB, int M, int N, int K, int* config) {
  if ((opA != 0 && opA != 1) || (opB != 0 && opB != 1)) return SGEMM_MI355_ERR_OP;
  if (M < 0 || N < 0 || K < 0) return SGEMM_MI355_ERR_DIM;
  if (!config) return SGEMM_MI355_ERR_NULL;
  *config = select_streamk(opA, opB, M, N, K, true);
  return SGEMM_MI355_OK;
}

int sgemm_mi355_config_streamk(int config) {
  const KernelConfig* c = config_at(config);
  if (!c) return SGEMM_MI355_ERR_CONFIG;
  return c->streamk != nullptr ? 1 : 0;
}

int sgemm_mi355_validate(int M, int N, int K, const float* A, int lda, const float* B, int ldb,
                         const float* C, int ldc) {
  return validate(plain(M, N, K, A, lda, B, ldb, C, ldc));
}

int sgemm_mi355_validate_ex(int opA, int opB, int M, int N, int K, float alpha, const float* A,
                            int lda, long long strideA, const float* B, int ldb, long long strideB,
                            float beta, const float* C, int ldc, long long strideC, int batch) {
  return validate(Problem{opA, opB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc,
                          strideC, batch});
}

int sgemm_mi355_select_config(int M, int N, int K) {
  if (M < 0 || N < 0 || K < 0) return SGEMM_MI355_ERR_DIM;
  return select_mfma(0, 0, M, N, K, 1);
}

int sgemm_mi355_config_staging(int config, int M, int N, int K, const float* A, int lda, const float* B,
                               int ldb) {
  const KernelConfig* c = config_at(config);
  if (!c) return SGEMM_MI355_ERR_CONFIG;
  if (M < 0 || N < 0 || K < 0) return SGEMM_MI355_ERR_DIM;
  if (!is_direct_config(config)) return 0;
  const Problem p{c->transA, c->transB, M, N, K, 1.0f, A, lda, 0, B, ldb, 0, 0.0f, nullptr, 0, 0, 1};
  if (!direct_path(*c, M, N, K, operands_aligned(p))) return 0;
  return K % c->bk == 0 ? 1 : 2;
}

int sgemm_mi355_selected_config(int M, int N, int K, const float* A, int lda, const float* B, int ldb) {
  if (M < 0 || N < 0 || K < 0) return SGEMM_MI355_ERR_DIM;
  return select_for(plain(M, N, K, A, lda, B, ldb, nullptr, 0));
}

int sgemm_mi355_select_config_valu(int M, int N, int K) {
  if (M < 0 || N < 0 || K < 0) return SGEMM_MI355_ERR_DIM;
  return select_valu(M, N);
}

int sgemm_mi355_select_config_ex(int opA, int opB, int M, int N, int K, int batch) {
  if ((opA != 0 && opA != 1) || (opB != 0 && opB != 1)) return SGEMM_MI355_ERR_OP;
  if (M < 0 || N < 0 || K < 0 || batch < 0) return SGEMM_MI355_ERR_DIM;
  return select_mfma(opA, opB, M, N, K, batch < 1 ? 1 : batch);
}

int sgemm_mi355_num_configs(void) { return num_configs(); }

const char* sgemm_mi355_config_name(int config) {
  const KernelConfig* c = config_at(config);
  return c ? c->name : nullptr;
}

int sgemm_mi355_config_info(int config, int* bm, int* bn, int* bk, int* threads) {
  const KernelConfig* c = config_at(config);
  if (!c) return SGEMM_MI355_ERR_CONFIG;
  if (bm) *bm = c->bm;
  if (bn) *bn = c->bn;
  if (bk) *bk = c->bk;
  if (threads) *threads = c->threads;
  return SGEMM_MI355_OK;
}

int sgemm_mi355_config_occupancy(int config, int* workgroups_per_cu) {
  const KernelConfig* c = config_at(config);
  if (!c) return SGEMM_MI355_ERR_CONFIG;
  if (!workgroups_per_cu) return SGEMM_MI355_ERR_NULL;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, c->kernel, c->threads, 0) != hipSuccess) {
    (void)hipGetLastError();  // leave no sticky error for the caller's next HIP call
    return SGEMM_MI355_ERR_LAUNCH;
  }
  *workgroups_per_cu = n;
  return SGEMM_MI355_OK;
}

int sgemm_mi355_config_ops(int config, int* opA, int* opB) {
  const KernelConfig* c = config_at(config);
  if (!c) return SGEMM_MI355_ERR_CONFIG;
  if (opA) *opA = c->transA;
  if (opB) *opB = c->transB;
  return SGEMM_MI355_OK;
}

int sgemm_mi355_tile_map(int bid, int tiles_m, int tiles_n, int group_m, int* tm, int* tn) {
  if (tiles_m <= 0 || tiles_n <= 0 || group_m <= 0 || bid < 0 ||
      (int64_t)tiles_m * tiles_n > INT_MAX || bid >= tiles_m * tiles_n || !tm || !tn)
    return SGEMM_MI355_ERR_DIM;
  tile_coords(bid, tiles_m, tiles_n, group_m, *tm, *tn);
  return SGEMM_MI355_OK;
}

const char* sgemm_mi355_strerror(int code) {
  switch (code) {
    case SGEMM_MI355_OK: return "success";
    case SGEMM_MI355_ERR_DIM: return "a matrix dimension or the batch count is negative";
    case SGEMM_MI355_ERR_LD: return "a leading dimension is smaller than its row length";
    case SGEMM_MI355_ERR_NULL: return "null pointer for a matrix with elements";
    case SGEMM_MI355_ERR_ALIAS: return "C overlaps A or B";
    case SGEMM_MI355_ERR_EXTENT: return "problem too large for one launch";
    case SGEMM_MI355_ERR_LAUNCH: return "the HIP runtime rejected the kernel launch";
    case SGEMM_MI355_ERR_CONFIG: return "unknown kernel configuration, or one built for other operand layouts";
    case SGEMM_MI355_ERR_ALIGN: return "a matrix pointer is not 4-byte aligned";
    case SGEMM_MI355_ERR_STRIDE: return "a batch stride is negative, or batch entries of C overlap";
    case SGEMM_MI355_ERR_OP: return "an operand op is neither SGEMM_MI355_OP_N nor SGEMM_MI355_OP_T";
    case SGEMM_MI355_ERR_SCRATCH:
      return "the split-K partial sums exceed the library's static scratch (SGEMM_MI355_SCRATCH_BYTES per device)";
    case SGEMM_MI355_ERR_WORKSPACE:
      return "the workspace is smaller than sgemm_mi355_splitk_workspace_size or sgemm_mi355_streamk_workspace_size";
    default: return "unknown error code";
  }
}

const char* sgemm_mi355_version(void) { return "0.6.1"; }

}  // extern "C"
