// Host side of the C ABI declared in include/sgemm_mi355.h: argument
// validation (pure host code, before any HIP call), tile-configuration
// selection and the kernel launch on the caller's stream. No allocation, no
// synchronisation, no mutable global state.

#include "sgemm_mi355.h"

#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "sgemm_internal.h"

namespace sgemm_impl {
namespace {

struct ShapeEntry {
  int M, N, K;
  const char* config;
};
#include "tile_table.inc"

constexpr int kCompute = 256;  // compute units on MI355X

// Block tiles the selection rule considers when the table has no entry,
// largest first (the fastest measured configuration of each tile size).
const char* const kRuleTiles[] = {"256x128x16_w4x2", "128x64x16_w2x2", "64x64x64_w2x2",
                                  "32x32x32_w1x1"};
const char* const kRuleTilesOps[] = {"256x128x16_w4x2", "128x64x16_w2x2", "64x64x32_w2x2",
                                     "32x32x32_w1x1"};

int num_configs() { return kNumMfmaConfigs + kNumValuConfigs; }

const KernelConfig* config_at(int id) {
  if (id < 0) return nullptr;
  if (id < kNumMfmaConfigs) return &kMfmaConfigs[id];
  if (id < kNumMfmaConfigs + kNumValuConfigs) return &kValuConfigs[id - kNumMfmaConfigs];
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

// The largest rule tile that still gives at least one workgroup per compute
// unit (counting batch entries), else the smallest.
int rule_select(int opA, int opB, int M, int N, int batch) {
  const char* const* tiles = (opA || opB) ? kRuleTilesOps : kRuleTiles;
  const int n = 4;
  const int64_t gy = batch < kMaxGridY ? batch : kMaxGridY;
  int last = -1;
  for (int i = 0; i < n; ++i) {
    char name[64];
    std::snprintf(name, sizeof(name), "mfma32_%s%s", tiles[i], ops_suffix(opA, opB));
    const int id = config_id(name);
    if (id < 0) continue;
    last = id;
    if (tiles_for(*config_at(id), M, N) * gy >= kCompute) return id;
  }
  return last;
}

int select_mfma(int opA, int opB, int M, int N, int K, int batch) {
  if (!opA && !opB && batch == 1)
    for (const ShapeEntry* e = kShapeTable; e->config; ++e)
      if (e->M == M && e->N == N && e->K == K) {
        const int id = config_id(e->config);
        if (id >= 0) return id;
      }
  return rule_select(opA, opB, M, N, batch);
}

// Vector-kernel configurations: largest tile with one workgroup per CU.
int select_valu(int M, int N) {
  int best = -1, smallest = -1;
  int64_t best_area = -1, small_area = INT64_MAX;
  for (int i = kNumMfmaConfigs; i < num_configs(); ++i) {
    const KernelConfig* c = config_at(i);
    const int64_t area = (int64_t)c->bm * c->bn;
    if (area < small_area) { small_area = area; smallest = i; }
    if (tiles_for(*c, M, N) >= kCompute && area > best_area) { best = i; best_area = area; }
  }
  return best >= 0 ? best : smallest;
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

int run(const Problem& p, float* C, hipStream_t stream, int config) {
  const int v = validate(p);
  if (v != SGEMM_MI355_OK) return v;
  const KernelConfig* cfg = config_at(config);
  if (cfg == nullptr || cfg->transA != p.opA || cfg->transB != p.opB) return SGEMM_MI355_ERR_CONFIG;
  if (p.M == 0 || p.N == 0 || p.batch == 0) return SGEMM_MI355_OK;
  const GemmArgs g{p.M,     p.N,       p.K,       p.A,       p.lda,     p.B,      p.ldb,
                   C,       p.ldc,     p.alpha,   p.beta,    p.strideA, p.strideB, p.strideC,
                   p.batch};
  const bool scale_only = (p.K == 0 || p.alpha == 0.0f);
  if (!scale_only && tiles_for(*cfg, p.M, p.N) * cfg->threads > (int64_t)UINT32_MAX)
    return SGEMM_MI355_ERR_EXTENT;
  // One launch per kMaxGridY batch entries (grid.y indexes the entry).
  for (int b0 = 0; b0 < p.batch; b0 += kMaxGridY) {
    GemmArgs gc = g;
    gc.batch = (p.batch - b0) < kMaxGridY ? (p.batch - b0) : kMaxGridY;
    gc.C = C + (int64_t)b0 * p.strideC;
    if (!scale_only) {
      gc.A = p.A + (int64_t)b0 * p.strideA;
      gc.B = p.B + (int64_t)b0 * p.strideB;
    }
    const hipError_t err = scale_only ? launch_scale_c(gc, stream) : cfg->launch(gc, stream);
    if (err != hipSuccess) return SGEMM_MI355_ERR_LAUNCH;
  }
  return SGEMM_MI355_OK;
}

Problem plain(int M, int N, int K, const float* A, int lda, const float* B, int ldb, const float* C,
              int ldc) {
  return Problem{0, 0, M, N, K, 1.0f, A, lda, 0, B, ldb, 0, 0.0f, C, ldc, 0, 1};
}

int select_for(const Problem& p) {
  if (p.opA < 0 || p.opA > 1 || p.opB < 0 || p.opB > 1) return 0;
  return select_mfma(p.opA, p.opB, p.M < 0 ? 0 : p.M, p.N < 0 ? 0 : p.N, p.K, p.batch < 1 ? 1 : p.batch);
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
    default: return "unknown error code";
  }
}

const char* sgemm_mi355_version(void) { return "0.2.0"; }

}  // extern "C"
