// Internal declarations shared by the kernels and the host dispatcher.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace sgemm_impl {

// Arguments of one launch, passed to the kernels by value. The operation is
//   C_b = alpha * op(A_b) . op(B_b) + beta * C_b,   b = 0 .. batch-1,
// with X_b = X + b * strideX. op(A) is M x K: A itself (row-major M x K,
// element (i, k) at A[i*lda + k]) or, with transA, the transpose of a
// row-major K x M matrix (element (i, k) at A[k*lda + i]); likewise op(B) is
// K x N from a K x N matrix or, with transB, from an N x K matrix. When
// beta == 0, C is not read. Offsets are computed in 64 bits.
struct GemmArgs {
  int M, N, K;
  const float* A;
  int64_t lda;
  const float* B;
  int64_t ldb;
  float* C;
  int64_t ldc;
  float alpha, beta;
  int64_t strideA, strideB, strideC;
  int batch;
  int k_last;  // K of the last batch entry of the launch (split-K chunks); K otherwise
};

using LaunchFn = hipError_t (*)(const GemmArgs&, hipStream_t);

// Stream-K schedule of one single-product launch on a persistent grid of G
// workgroups. Tiles are numbered in the order of tile_coords. Tiles
// [0, dp_tiles) run whole, tile j on workgroup j % G; the iters BK-deep slabs
// of each of the sk_tiles tiles after them, sk_iters = sk_tiles * iters in
// all, taken in tile order and ascending k, are dealt to the workgroups in
// contiguous ranges, workgroup w taking [w * sk_iters / G, (w+1) * sk_iters / G).
// A workgroup stores a piece of a tile that is not the whole tile as a dense
// row-major BM x BN block of partial sums: in block 2w of `partials` if the
// piece starts its range, else in block 2w + 1 (the piece that ends it).
struct StreamKPlan {
  int dp_tiles, sk_tiles;
  int iters;
  int64_t sk_iters;
  float* partials;  // 2 * G blocks of BM * BN floats, 16-byte aligned
};

// Runs the stream-K kernel (grid G, direct loads when `direct`) and then the
// kernel that adds the partial sums of every split tile into C.
using StreamKLaunchFn = hipError_t (*)(const GemmArgs&, const StreamKPlan&, int grid, bool direct,
                                       hipStream_t);

enum KernelKind { KIND_MFMA = 0, KIND_VALU = 1 };

struct KernelConfig {
  const char* name;
  int kind;
  int bm, bn, bk;
  int threads;
  int transA, transB;  // operand layouts the kernel reads
  LaunchFn launch;
  const void* kernel;  // the kernel launch() runs for 16-byte aligned operands (occupancy queries)
  int kgroups;         // wave groups that split each slab's k range (1: none)
  // Stream-K form (null where the configuration has none) and its two kernels,
  // staged through registers [0] and by direct loads [1] (occupancy queries).
  StreamKLaunchFn streamk;
  const void* streamk_kernel[2];
  // 1: a configuration of the direct-load kernel family that stages every slab
  // through registers (the hand-ordered tiles named _rs), so it has no direct
  // path and takes operands of any alignment.
  int staged;
};

// Host-only tables (not const: a const global would also be emitted for the
// device). Defined in kernels_mfma.hip, kernels_mfma_dma.hip and kernels_valu.hip.
extern KernelConfig kMfmaConfigs[];
extern const int kNumMfmaConfigs;
extern KernelConfig kMfmaDmaConfigs[];  // defined in kernels_mfma_dma.hip
extern const int kNumMfmaDmaConfigs;
extern KernelConfig kValuConfigs[];
extern const int kNumValuConfigs;

// C_b = beta * C_b over the M x N block of every batch entry of the launch
// (the K == 0 or alpha == 0 case); beta == 0 writes +0 without reading C.
// Defined in kernels_util.hip.
hipError_t launch_scale_c(const GemmArgs& g, hipStream_t s);

// C = alpha * sum_{s < splits} W_s + beta * C over M x N, the W_s dense M x N
// partial products (row stride N) at W + s*M*N, summed in ascending s.
// Defined in kernels_util.hip.
hipError_t launch_splitk_reduce(const float* W, int splits, int M, int N, float alpha, float beta,
                                float* C, int64_t ldc, hipStream_t s);

// Batch entries per launch: each launch covers one batch entry per grid.y
// index, and larger batches are split into several launches on the host.
constexpr int kMaxGridY = 65535;

// Workgroup -> C-tile map shared by all kernels. Workgroups are dispatched
// round-robin over the 8 XCDs (workgroup b runs on XCD b % 8), each XCD with
// its own L2. The map first renumbers workgroups so that consecutive logical
// ids run on the same XCD, then walks the tile grid in bands of `group_m`
// tile rows, column by column, so the tiles resident on one XCD at a time
// share a few A row panels and B column panels in that XCD's L2.
__host__ __device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int group_m,
                                                     int& tm, int& tn) {
  const int nwg = tiles_m * tiles_n;
  const int q = nwg >> 3, rem = nwg & 7;
  const int xcd = bid & 7, slot = bid >> 3;
  const int lid = xcd * q + (xcd < rem ? xcd : rem) + slot;
  const int band = group_m * tiles_n;
  const int first_m = (lid / band) * group_m;
  const int rows = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
  const int in_band = lid - (lid / band) * band;
  tm = first_m + in_band % rows;
  tn = in_band / rows;
}

}  // namespace sgemm_impl
