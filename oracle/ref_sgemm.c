/*
 * CPU oracle for single-precision GEMM, C = A.B on row-major matrices.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do. It shares no code, header or constant with the HIP library.
 *
 * What it computes (the plain definition, written out):
 *   Each output element is the dot product of row i of A with column j of B,
 *   one multiply and one add per term, 2*M*N*K operations in all
 *   (ratcatcher.ru "Matrix multiplication: naive and tiled", section 1;
 *   GPU Parallel Book ch. 9, section 9.1). The naive kernels on both pages
 *   start an FP32 accumulator at 0.0f and add the products A[i][k]*B[k][j]
 *   for k = 0, 1, ..., K-1 (ratcatcher page section 1, naive kernel; GPU
 *   Parallel Book section 9.2). General M, N, K with row-major offsets
 *   row*ld + col follow the CUDA Handbook, section 17.3 (sgemm_cache takes
 *   M, N, K; A is indexed (row)*K + k and B k*N + col) and the ratcatcher page
 *   section 1 (element (row, col) at offset row*N + col); the leading
 *   dimensions lda, ldb, ldc generalise those strides.
 *
 * Readings where the pages are silent:
 *   - The product and the add are rounded separately (round to nearest even),
 *     i.e. no fused multiply-add: this file must be compiled with
 *     -ffp-contract=off. Each term is one FP32 multiply then one FP32 add.
 *   - k runs in ascending order, so the result is one fixed, reproducible
 *     FP32 value per element.
 *   - The loops run in i-k-j order with a row of accumulators, and OpenMP
 *     splits the rows i. Every C[i][j] still sees exactly the same ordered
 *     sequence of adds as the i-j-k triple loop, so results are bitwise those
 *     of the triple loop and independent of the thread count.
 *   - K == 0 gives C = +0 (the empty sum); M == 0 or N == 0 does nothing.
 *
 * ref_sgemm_f64_abs: the same sum accumulated in FP64 (products of two FP32
 * values are exact in FP64), plus S[i][j] = sum_k |A[i][k]*B[k][j]| in FP64.
 * C64 is the "FP64-accumulated reference" for error bounds; S scales the
 * per-element bound |C - C64| <= c*K*2^-23*S.
 *
 * ref_sgemm_ex_f32 / ref_sgemm_ex_f64_abs: the general form
 * C = alpha*op(A).op(B) + beta*C with op(X) = X or X^T on row-major storage
 * (the BLAS interface around the same product). The pages define only the
 * product; the reading taken for the rest: the product t is the FP32 sum
 * above, then C = fl(fl(alpha*t) + fl(beta*c)), each operation rounded
 * separately; C is not read when beta == 0 (the beta term is absent), and A
 * and B are not read when alpha == 0 or K == 0 (the alpha term is absent).
 *
 * Pinned by tests/test_oracle_cpu.py against brute force in exact rational
 * arithmetic, identity and all-ones closed forms, the transpose identity,
 * K = 1 products, exact small-integer results and a BLAS FP64 product.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#if defined(__FP_FAST_FMAF) || defined(__FAST_MATH__)
#error "the oracle must be built without fast-math and without FMA contraction"
#endif

/* Number of OpenMP threads the next call will use (1 without OpenMP). */
int ref_max_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void ref_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* C[i*ldc + j] = sum_{k<K} A[i*lda + k] * B[k*ldb + j], FP32, k ascending. */
void ref_sgemm_f32(int M, int N, int K,
                   const float *A, int lda,
                   const float *B, int ldb,
                   float *C, int ldc)
{
    if (M <= 0 || N <= 0) return;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < M; ++i) {
        float *c = C + (size_t)i * (size_t)ldc;
        const float *a = A + (size_t)i * (size_t)lda;
        for (int j = 0; j < N; ++j) c[j] = 0.0f;
        for (int k = 0; k < K; ++k) {
            const float aik = a[k];
            const float *b = B + (size_t)k * (size_t)ldb;
            for (int j = 0; j < N; ++j) {
                float p = aik * b[j];
                c[j] = c[j] + p;
            }
        }
    }
}

/* C64[i*N + j] = sum_k A[i][k]*B[k][j] and S[i*N + j] = sum_k |A[i][k]*B[k][j]|,
 * both in FP64, k ascending. C64 and S are dense M x N (row stride N). */
void ref_sgemm_f64_abs(int M, int N, int K,
                       const float *A, int lda,
                       const float *B, int ldb,
                       double *C64, double *S)
{
    if (M <= 0 || N <= 0) return;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < M; ++i) {
        double *c = C64 + (size_t)i * (size_t)N;
        double *s = S + (size_t)i * (size_t)N;
        const float *a = A + (size_t)i * (size_t)lda;
        for (int j = 0; j < N; ++j) { c[j] = 0.0; s[j] = 0.0; }
        for (int k = 0; k < K; ++k) {
            const double aik = (double)a[k];
            const float *b = B + (size_t)k * (size_t)ldb;
            for (int j = 0; j < N; ++j) {
                double p = aik * (double)b[j];
                c[j] = c[j] + p;
                s[j] = s[j] + fabs(p);
            }
        }
    }
}

/* op(A)(i, k) and op(B)(k, j) on row-major storage. */
static inline float op_a(int opA, const float *A, int lda, int i, int k)
{
    return opA ? A[(size_t)k * (size_t)lda + i] : A[(size_t)i * (size_t)lda + k];
}

static inline float op_b(int opB, const float *B, int ldb, int k, int j)
{
    return opB ? B[(size_t)j * (size_t)ldb + k] : B[(size_t)k * (size_t)ldb + j];
}

/* C = alpha*op(A).op(B) + beta*C in FP32; the product term is the FP32 sum
 * from +0 with k ascending, then fl(fl(alpha*t) + fl(beta*c)). */
void ref_sgemm_ex_f32(int opA, int opB, int M, int N, int K, float alpha,
                      const float *A, int lda, const float *B, int ldb,
                      float beta, float *C, int ldc)
{
    if (M <= 0 || N <= 0) return;
    const int use_ab = (alpha != 0.0f) && K > 0;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < M; ++i) {
        float *c = C + (size_t)i * (size_t)ldc;
        for (int j = 0; j < N; ++j) {
            float t = 0.0f;
            if (use_ab) {
                for (int k = 0; k < K; ++k) {
                    float p = op_a(opA, A, lda, i, k) * op_b(opB, B, ldb, k, j);
                    t = t + p;
                }
            }
            float out;
            if (use_ab && beta != 0.0f) {
                float at = alpha * t;
                float bc = beta * c[j];
                out = at + bc;
            } else if (use_ab) {
                out = alpha * t;
            } else if (beta != 0.0f) {
                out = beta * c[j];
            } else {
                out = 0.0f;
            }
            c[j] = out;
        }
    }
}

/* P64 = op(A).op(B) and S = sum_k |op(A)(i,k)*op(B)(k,j)| in FP64, dense
 * M x N (row stride N), k ascending. */
void ref_sgemm_ex_f64_abs(int opA, int opB, int M, int N, int K,
                          const float *A, int lda, const float *B, int ldb,
                          double *P64, double *S)
{
    if (M <= 0 || N <= 0) return;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < M; ++i) {
        for (int j = 0; j < N; ++j) {
            double t = 0.0, s = 0.0;
            for (int k = 0; k < K; ++k) {
                double p = (double)op_a(opA, A, lda, i, k) * (double)op_b(opB, B, ldb, k, j);
                t = t + p;
                s = s + fabs(p);
            }
            P64[(size_t)i * (size_t)N + j] = t;
            S[(size_t)i * (size_t)N + j] = s;
        }
    }
}
