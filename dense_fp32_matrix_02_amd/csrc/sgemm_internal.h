// Internal declarations shared by the kernels and the host dispatcher.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace sgemm_impl {

// Arguments of one C = A.B call, passed to the kernels by value. Leading
// dimensions are 64-bit so every offset row*ld + col is computed in 64 bits.
struct GemmArgs {
  int M, N, K;
  const float* A;
  int64_t lda;
  const float* B;
  int64_t ldb;
  float* C;
  int64_t ldc;
};

using LaunchFn = hipError_t (*)(const GemmArgs&, hipStream_t);

enum KernelKind { KIND_MFMA = 0, KIND_VALU = 1 };

struct KernelConfig {
  const char* name;
  int kind;
  int bm, bn, bk;
  int threads;
  LaunchFn launch;
};

// Defined in kernels_mfma.hip and kernels_valu.hip.
extern KernelConfig kMfmaConfigs[];  // host-only tables (not const: a const
                                      // global would also be emitted on the device)
extern const int kNumMfmaConfigs;
extern KernelConfig kValuConfigs[];
extern const int kNumValuConfigs;

// C[0..M) x [0..N) = +0 (the K == 0 case). Defined in kernels_valu.hip.
hipError_t launch_zero_fill(float* C, int M, int N, int64_t ldc, hipStream_t s);

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
