// Host side of the C ABI declared in include/sgemm_mi355.h: argument
// validation (pure host code, before any HIP call), tile-configuration
// selection and the kernel launch on the caller's stream. No allocation, no
// synchronisation, no mutable global state.

#include "sgemm_mi355.h"

#include <climits>
#include <cstdint>
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

// Largest block tile with at least one workgroup per compute unit; if even
// the smallest tile under-fills the chip, the smallest tile. Among configs of
// equal tile area the first listed wins.
int rule_select(int M, int N, int first, int count) {
  int best = -1;
  int64_t best_area = -1;
  int smallest = first;
  for (int i = first; i < first + count; ++i) {
    const KernelConfig* c = config_at(i);
    const int64_t area = (int64_t)c->bm * c->bn;
    const KernelConfig* s = config_at(smallest);
    if (area < (int64_t)s->bm * s->bn) smallest = i;
    if (tiles_for(*c, M, N) >= kCompute && area > best_area) {
      best = i;
      best_area = area;
    }
  }
  return best >= 0 ? best : smallest;
}

int select_mfma(int M, int N, int K) {
  for (const ShapeEntry* e = kShapeTable; e->config; ++e)
    if (e->M == M && e->N == N && e->K == K) {
      const int id = config_id(e->config);
      if (id >= 0) return id;
    }
  return rule_select(M, N, 0, kNumMfmaConfigs);
}

int select_valu(int M, int N) { return rule_select(M, N, kNumMfmaConfigs, kNumValuConfigs); }

bool overlaps(const void* p, uint64_t pbytes, const void* q, uint64_t qbytes) {
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + qbytes && b < a + pbytes;
}

int validate(int M, int N, int K, const float* A, int lda, const float* B, int ldb,
             const float* C, int ldc) {
  if (M < 0 || N < 0 || K < 0) return SGEMM_MI355_ERR_DIM;
  if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1))
    return SGEMM_MI355_ERR_LD;
  if (M == 0 || N == 0) return SGEMM_MI355_OK;
  if (C == nullptr) return SGEMM_MI355_ERR_NULL;
  if (K > 0 && (A == nullptr || B == nullptr)) return SGEMM_MI355_ERR_NULL;
  if (((uintptr_t)C & 3) != 0) return SGEMM_MI355_ERR_ALIGN;
  if (K > 0 && ((((uintptr_t)A) | ((uintptr_t)B)) & 3) != 0) return SGEMM_MI355_ERR_ALIGN;
  // Index arithmetic inside the kernels keeps row and column numbers in
  // 32-bit ints with up to one block tile of headroom.
  if (M > INT_MAX - 1024 || N > INT_MAX - 1024 || K > INT_MAX - 1024) return SGEMM_MI355_ERR_EXTENT;
  const uint64_t c_bytes = 4 * ((uint64_t)(M - 1) * (uint64_t)ldc + (uint64_t)N);
  if (K > 0) {
    const uint64_t a_bytes = 4 * ((uint64_t)(M - 1) * (uint64_t)lda + (uint64_t)K);
    const uint64_t b_bytes = 4 * ((uint64_t)(K - 1) * (uint64_t)ldb + (uint64_t)N);
    if (overlaps(C, c_bytes, A, a_bytes) || overlaps(C, c_bytes, B, b_bytes))
      return SGEMM_MI355_ERR_ALIAS;
  }
  return SGEMM_MI355_OK;
}

int run(int M, int N, int K, const float* A, int lda, const float* B, int ldb, float* C,
        int ldc, hipStream_t stream, int config) {
  const int v = validate(M, N, K, A, lda, B, ldb, C, ldc);
  if (v != SGEMM_MI355_OK) return v;
  const KernelConfig* cfg = config_at(config);
  if (cfg == nullptr) return SGEMM_MI355_ERR_CONFIG;
  if (M == 0 || N == 0) return SGEMM_MI355_OK;
  hipError_t err;
  if (K == 0) {
    err = launch_zero_fill(C, M, N, ldc, stream);
  } else {
    const int64_t tiles = tiles_for(*cfg, M, N);
    if (tiles * cfg->threads > (int64_t)UINT32_MAX) return SGEMM_MI355_ERR_EXTENT;
    const GemmArgs g{M, N, K, A, lda, B, ldb, C, ldc};
    err = cfg->launch(g, stream);
  }
  return err == hipSuccess ? SGEMM_MI355_OK : SGEMM_MI355_ERR_LAUNCH;
}

}  // namespace
}  // namespace sgemm_impl

using namespace sgemm_impl;

extern "C" {

int sgemm_mi355(int M, int N, int K, const float* A, int lda, const float* B, int ldb, float* C,
                int ldc, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0) return SGEMM_MI355_ERR_DIM;
  return run(M, N, K, A, lda, B, ldb, C, ldc, stream, select_mfma(M, N, K));
}

int sgemm_mi355_valu(int M, int N, int K, const float* A, int lda, const float* B, int ldb,
                     float* C, int ldc, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0) return SGEMM_MI355_ERR_DIM;
  return run(M, N, K, A, lda, B, ldb, C, ldc, stream, select_valu(M, N));
}

int sgemm_mi355_with_config(int M, int N, int K, const float* A, int lda, const float* B, int ldb,
                            float* C, int ldc, hipStream_t stream, int config) {
  return run(M, N, K, A, lda, B, ldb, C, ldc, stream, config);
}

int sgemm_mi355_validate(int M, int N, int K, const float* A, int lda, const float* B, int ldb,
                         const float* C, int ldc) {
  return validate(M, N, K, A, lda, B, ldb, C, ldc);
}

int sgemm_mi355_select_config(int M, int N, int K) {
  if (M < 0 || N < 0 || K < 0) return SGEMM_MI355_ERR_DIM;
  return select_mfma(M, N, K);
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
    case SGEMM_MI355_ERR_DIM: return "a matrix dimension is negative";
    case SGEMM_MI355_ERR_LD: return "a leading dimension is smaller than its row length";
    case SGEMM_MI355_ERR_NULL: return "null pointer for a matrix with elements";
    case SGEMM_MI355_ERR_ALIAS: return "C overlaps A or B";
    case SGEMM_MI355_ERR_EXTENT: return "problem too large for one launch";
    case SGEMM_MI355_ERR_LAUNCH: return "the HIP runtime rejected the kernel launch";
    case SGEMM_MI355_ERR_CONFIG: return "unknown kernel configuration id";
    case SGEMM_MI355_ERR_ALIGN: return "a matrix pointer is not 4-byte aligned";
    default: return "unknown error code";
  }
}

const char* sgemm_mi355_version(void) { return "0.1.0"; }

}  // extern "C"
