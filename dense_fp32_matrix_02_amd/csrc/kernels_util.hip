// Element-wise helper kernels of the GEMM library: the C = beta*C update
// (K == 0 or alpha == 0) and the fixed-order split-K reduction. Both are
// bandwidth-bound passes over C; plain kernels rather than memsets so the
// calls stay safe inside captured graphs.

#include "sgemm_internal.h"

namespace sgemm_impl {
namespace {

// C_b = beta * C_b over the M x N block of batch entry blockIdx.y; beta == 0
// writes +0 without reading C (the empty sum for K == 0, or alpha == 0).
__global__ void __launch_bounds__(256) scale_c_kernel(GemmArgs g) {
  const int64_t total = (int64_t)g.M * g.N;
  float* C = g.C + (int64_t)blockIdx.y * g.strideC;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t i = e / g.N, j = e - i * g.N;
    float* p = C + i * g.ldc + j;
    *p = (g.beta != 0.0f) ? g.beta * *p : 0.0f;
  }
}

// C = alpha * sum_s W_s + beta * C, the partials W_s dense M x N at
// W + s*M*N, added in ascending s so the result does not depend on timing.
// One thread per element of C; each partial is read along rows (coalesced).
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* W, int splits, int M, int N,
                                                            float alpha, float beta, float* C,
                                                            int64_t ldc) {
  const int64_t total = (int64_t)M * N;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    float s = 0.0f;
    for (int p = 0; p < splits; ++p) s += W[p * total + e];
    const int64_t i = e / N, j = e - i * N;
    float* c = C + i * ldc + j;
    const float v = alpha * s;
    *c = (beta != 0.0f) ? __builtin_fmaf(beta, *c, v) : v;
  }
}

unsigned blocks_for(int64_t total, int64_t cap) {
  int64_t b = (total + 255) / 256;
  return (unsigned)(b < cap ? (b > 0 ? b : 1) : cap);
}

}  // namespace

hipError_t launch_scale_c(const GemmArgs& g, hipStream_t stream) {
  GemmArgs a = g;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&scale_c_kernel),
                         dim3(blocks_for((int64_t)g.M * g.N, 4096), (unsigned)g.batch), dim3(256), args,
                         0, stream);
}

hipError_t launch_splitk_reduce(const float* W, int splits, int M, int N, float alpha, float beta,
                                float* C, int64_t ldc, hipStream_t stream) {
  void* args[] = {&W, &splits, &M, &N, &alpha, &beta, &C, &ldc};
  return hipLaunchKernel(reinterpret_cast<const void*>(&splitk_reduce_kernel),
                         dim3(blocks_for((int64_t)M * N, 8192)), dim3(256), args, 0, stream);
}

}  // namespace sgemm_impl
