// A native caller of the C ABI in include/sgemm_mi355.h, with no Python and no
// torch: device memory from hipMalloc, a stream from hipStreamCreate, results
// checked bit for bit against the CPU oracle library (oracle/liboracle.so) on
// small-integer inputs, whose products and sums are exact in FP32.
//
// Run by tests/test_native_gpu.py; prints one line per case and exits 0 when
// every case passes. Built by __graft_entry__.build() with hipcc (host code
// only).

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "sgemm_mi355.h"

// The oracle's entry points (test infrastructure; see oracle/ref_sgemm.c).
extern "C" {
void ref_sgemm_f32(int M, int N, int K, const float* A, int lda, const float* B, int ldb, float* C,
                   int ldc);
void ref_sgemm_ex_f32(int opA, int opB, int M, int N, int K, float alpha, const float* A, int lda,
                      const float* B, int ldb, float beta, float* C, int ldc);
}

namespace {

int failures = 0;

#define HIP_OK(call)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess) {                                                            \
      std::printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      std::exit(2);                                                                    \
    }                                                                                  \
  } while (0)

// Integers in [-4, 4] from a 64-bit linear congruential generator (Knuth's
// MMIX constants): the same host values feed the library and the oracle.
struct Ints {
  unsigned long long s;
  explicit Ints(unsigned long long seed) : s(seed * 2654435761ull + 1) {}
  float next() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((int)((s >> 33) % 9) - 4);
  }
  std::vector<float> fill(size_t n) {
    std::vector<float> v(n);
    for (auto& x : v) x = next();
    return v;
  }
};

struct Dev {
  float* p = nullptr;
  size_t n = 0;
  explicit Dev(size_t count) : n(count) { HIP_OK(hipMalloc(&p, (n ? n : 1) * sizeof(float))); }
  Dev(const std::vector<float>& h) : Dev(h.size()) { put(h); }
  ~Dev() { (void)hipFree(p); }
  void put(const std::vector<float>& h) {
    HIP_OK(hipMemcpy(p, h.data(), h.size() * sizeof(float), hipMemcpyHostToDevice));
  }
  std::vector<float> get() const {
    std::vector<float> h(n);
    HIP_OK(hipMemcpy(h.data(), p, n * sizeof(float), hipMemcpyDeviceToHost));
    return h;
  }
};

void check(const char* name, int rc, const std::vector<float>& got, const std::vector<float>& want) {
  size_t bad = 0, first = 0;
  for (size_t i = 0; i < want.size(); ++i)
    if (!(got[i] == want[i]) && !(got[i] != got[i] && want[i] != want[i])) {  // NaN padding matches NaN
      if (!bad) first = i;
      ++bad;
    }
  const bool ok = rc == SGEMM_MI355_OK && bad == 0;
  if (!ok) ++failures;
  if (bad)
    std::printf("%s %s: rc=%d, %zu mismatches (first at %zu: %g vs %g)\n", ok ? "PASS" : "FAIL", name,
                rc, bad, first, got[first], want[first]);
  else
    std::printf("%s %s: rc=%d (%s)\n", ok ? "PASS" : "FAIL", name, rc, sgemm_mi355_strerror(rc));
  std::fflush(stdout);
}

void expect_code(const char* name, int rc, int want) {
  const bool ok = rc == want;
  if (!ok) ++failures;
  std::printf("%s %s: rc=%d, expected %d (%s)\n", ok ? "PASS" : "FAIL", name, rc, want,
              sgemm_mi355_strerror(want));
  std::fflush(stdout);
}

}  // namespace

int main() {
  std::printf("library %s, %d configurations\n", sgemm_mi355_version(), sgemm_mi355_num_configs());
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  const float nan = __builtin_nanf("");

  {  // plain product with padded leading dimensions: padding of C stays untouched
    const int M = 301, N = 257, K = 203, lda = K + 3, ldb = N + 5, ldc = N + 7;
    Ints g(1);
    std::vector<float> A = g.fill((size_t)M * lda), B = g.fill((size_t)K * ldb);
    std::vector<float> C0((size_t)M * ldc, nan), want = C0;
    Dev dA(A), dB(B), dC(C0);
    const int rc = sgemm_mi355(M, N, K, dA.p, lda, dB.p, ldb, dC.p, ldc, stream);
    HIP_OK(hipStreamSynchronize(stream));
    ref_sgemm_f32(M, N, K, A.data(), lda, B.data(), ldb, want.data(), ldc);
    check("sgemm_mi355 301x257x203, padded ld", rc, dC.get(), want);
  }
  {  // general form: op(A) = A^T, alpha = 2, beta = -1 (C is read)
    const int M = 130, N = 97, K = 211, lda = M, ldb = N, ldc = N;
    Ints g(2);
    std::vector<float> A = g.fill((size_t)K * lda), B = g.fill((size_t)K * ldb);
    std::vector<float> C0 = g.fill((size_t)M * ldc), want = C0;
    Dev dA(A), dB(B), dC(C0);
    const int rc = sgemm_mi355_ex(SGEMM_MI355_OP_T, SGEMM_MI355_OP_N, M, N, K, 2.0f, dA.p, lda, dB.p,
                                  ldb, -1.0f, dC.p, ldc, stream);
    HIP_OK(hipStreamSynchronize(stream));
    ref_sgemm_ex_f32(1, 0, M, N, K, 2.0f, A.data(), lda, B.data(), ldb, -1.0f, want.data(), ldc);
    check("sgemm_mi355_ex tn alpha=2 beta=-1", rc, dC.get(), want);
  }
  {  // both operands transposed through a direct global-to-LDS configuration, forced by name
    const int M = 300, N = 260, K = 160, lda = M, ldb = K, ldc = N;
    int cid = -1;
    for (int i = 0; i < sgemm_mi355_num_configs(); ++i)
      if (std::strcmp(sgemm_mi355_config_name(i), "mfma32_256x256x16_w4x4_lds2_tt") == 0) cid = i;
    Ints g(5);
    std::vector<float> A = g.fill((size_t)K * lda), B = g.fill((size_t)N * ldb);
    std::vector<float> C0((size_t)M * ldc, nan), want = C0;
    Dev dA(A), dB(B), dC(C0);
    const int rc = cid < 0 ? SGEMM_MI355_ERR_CONFIG
                           : sgemm_mi355_strided_batched_with_config(SGEMM_MI355_OP_T, SGEMM_MI355_OP_T, M, N, K, 1.0f,
                                                                     dA.p, lda, 0, dB.p, ldb, 0, 0.0f, dC.p, ldc,
                                                                     0, 1, stream, cid);
    HIP_OK(hipStreamSynchronize(stream));
    ref_sgemm_ex_f32(1, 1, M, N, K, 1.0f, A.data(), lda, B.data(), ldb, 0.0f, want.data(), ldc);
    check("direct-LDS tt configuration 300x260x160", rc, dC.get(), want);
  }
  {  // K not a whole number of 16-deep slabs on aligned rows: the direct kernel with a
     // register-staged last slab, forced by name, then the library's own choice
    const int M = 300, N = 260, K = 164;
    int cid = -1;
    for (int i = 0; i < sgemm_mi355_num_configs(); ++i)
      if (std::strcmp(sgemm_mi355_config_name(i), "mfma32_256x256x16_w4x4_lds2") == 0) cid = i;
    Ints g(7);
    std::vector<float> A = g.fill((size_t)M * K), B = g.fill((size_t)K * N);
    std::vector<float> C0((size_t)M * N, nan), want = C0;
    Dev dA(A), dB(B), dC(C0);
    int rc = cid < 0 ? SGEMM_MI355_ERR_CONFIG
                     : sgemm_mi355_with_config(M, N, K, dA.p, K, dB.p, N, dC.p, N, stream, cid);
    HIP_OK(hipStreamSynchronize(stream));
    ref_sgemm_f32(M, N, K, A.data(), K, B.data(), N, want.data(), N);
    check("direct-LDS 256x256 with a partial last slab, 300x260x164", rc, dC.get(), want);
    dC.put(C0);
    rc = sgemm_mi355(M, N, K, dA.p, K, dB.p, N, dC.p, N, stream);
    HIP_OK(hipStreamSynchronize(stream));
    check("sgemm_mi355 300x260x164", rc, dC.get(), want);
  }
  {  // strided batch with a shared B (strideB = 0)
    const int batch = 5, M = 70, N = 45, K = 33;
    Ints g(3);
    std::vector<float> A = g.fill((size_t)batch * M * K), B = g.fill((size_t)K * N);
    std::vector<float> C0((size_t)batch * M * N, nan), want = C0;
    Dev dA(A), dB(B), dC(C0);
    const int rc = sgemm_mi355_strided_batched(0, 0, M, N, K, 1.0f, dA.p, K, (long long)M * K, dB.p, N, 0,
                                               0.0f, dC.p, N, (long long)M * N, batch, stream);
    HIP_OK(hipStreamSynchronize(stream));
    for (int b = 0; b < batch; ++b)
      ref_sgemm_f32(M, N, K, A.data() + (size_t)b * M * K, K, B.data(), N, want.data() + (size_t)b * M * N, N);
    check("sgemm_mi355_strided_batched x5, shared B", rc, dC.get(), want);
  }
  {  // split-K with a caller-owned workspace, deterministic across calls
    const int M = 96, N = 80, K = 5000, splits = 4;
    Ints g(4);
    std::vector<float> A = g.fill((size_t)M * K), B = g.fill((size_t)K * N);
    std::vector<float> want((size_t)M * N, 0.0f);
    const size_t ws = sgemm_mi355_splitk_workspace_size(M, N, K, splits);
    Dev dA(A), dB(B), dC((size_t)M * N), dW(ws / sizeof(float));
    int rc = sgemm_mi355_splitk(0, 0, M, N, K, 1.0f, dA.p, K, dB.p, N, 0.0f, dC.p, N, splits, dW.p, ws,
                                stream);
    HIP_OK(hipStreamSynchronize(stream));
    const std::vector<float> first = dC.get();
    ref_sgemm_f32(M, N, K, A.data(), K, B.data(), N, want.data(), N);
    check("sgemm_mi355_splitk 96x80x5000, 4 chunks", rc, first, want);
    rc = sgemm_mi355_splitk(0, 0, M, N, K, 1.0f, dA.p, K, dB.p, N, 0.0f, dC.p, N, splits, dW.p, ws,
                            stream);
    HIP_OK(hipStreamSynchronize(stream));
    check("sgemm_mi355_splitk repeated call, same bits", rc, dC.get(), first);
    expect_code("sgemm_mi355_splitk short workspace",
                sgemm_mi355_splitk(0, 0, M, N, K, 1.0f, dA.p, K, dB.p, N, 0.0f, dC.p, N, splits, dW.p,
                                   ws - 4, stream),
                SGEMM_MI355_ERR_WORKSPACE);
  }
  {  // stream-K in 256x256 tiles: 9 tiles whose slabs are dealt to the whole grid,
     // partial sums added by the fixup kernel; the same bits on a second call
    const int M = 600, N = 520, K = 1040;
    int cid = -1;
    for (int i = 0; i < sgemm_mi355_num_configs(); ++i)
      if (std::strcmp(sgemm_mi355_config_name(i), "mfma32_256x256x16_w4x4_lds2") == 0) cid = i;
    Ints g(6);
    std::vector<float> A = g.fill((size_t)M * K), B = g.fill((size_t)K * N);
    std::vector<float> C0 = g.fill((size_t)M * N), want = C0;
    const size_t ws = cid < 0 ? 0 : sgemm_mi355_streamk_workspace_size(0, 0, M, N, K, cid);
    Dev dA(A), dB(B), dC(C0), dW(ws / sizeof(float) + 4);
    int rc = cid < 0 || ws == 0 ? SGEMM_MI355_ERR_CONFIG
                                : sgemm_mi355_streamk_with_config(0, 0, M, N, K, 3.0f, dA.p, K, dB.p, N, 0.5f, dC.p,
                                                                  N, dW.p, ws, stream, cid);
    HIP_OK(hipStreamSynchronize(stream));
    ref_sgemm_ex_f32(0, 0, M, N, K, 3.0f, A.data(), K, B.data(), N, 0.5f, want.data(), N);
    check("sgemm_mi355_streamk_with_config 600x520x1040, alpha=3 beta=0.5", rc, dC.get(), want);
    dC.put(C0);
    rc = sgemm_mi355_streamk_with_config(0, 0, M, N, K, 3.0f, dA.p, K, dB.p, N, 0.5f, dC.p, N, dW.p, ws, stream,
                                         cid);
    HIP_OK(hipStreamSynchronize(stream));
    check("sgemm_mi355_streamk repeated call", rc, dC.get(), want);
    expect_code("sgemm_mi355_streamk short workspace",
                sgemm_mi355_streamk_with_config(0, 0, M, N, K, 3.0f, dA.p, K, dB.p, N, 0.5f, dC.p, N, dW.p,
                                                ws - 16, stream, cid),
                SGEMM_MI355_ERR_WORKSPACE);
  }
  {  // argument errors are reported before anything is enqueued
    Dev d(64 * 64);
    expect_code("negative M", sgemm_mi355(-1, 4, 4, d.p, 4, d.p, 4, d.p, 4, stream), SGEMM_MI355_ERR_DIM);
    expect_code("lda < K", sgemm_mi355(4, 4, 8, d.p, 7, d.p, 4, d.p + 2048, 4, stream), SGEMM_MI355_ERR_LD);
    expect_code("C overlaps A", sgemm_mi355(8, 8, 8, d.p, 8, d.p + 1024, 8, d.p + 32, 8, stream),
                SGEMM_MI355_ERR_ALIAS);
    expect_code("null B", sgemm_mi355(4, 4, 4, d.p, 4, nullptr, 4, d.p + 2048, 4, stream),
                SGEMM_MI355_ERR_NULL);
    expect_code("unknown op", sgemm_mi355_ex(2, 0, 4, 4, 4, 1.0f, d.p, 4, d.p + 1024, 4, 0.0f, d.p + 2048, 4,
                                             stream),
                SGEMM_MI355_ERR_OP);
  }
  HIP_OK(hipStreamDestroy(stream));
  std::printf("%s: %d failure(s)\n", failures ? "FAILED" : "ALL PASSED", failures);
  return failures ? 1 : 0;
}
