/*
 * gemm_oracle.c -- CPU oracle for the dense GEMM  C = alpha*A*B + beta*C.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file; only the tests, the smoke check and the CPU
 * baseline leg of the bench do.  It shares no code with the HIP library.
 *
 * What it computes (the definition, written out, nothing more):
 *
 *   C(i,j) = sum_k A(i,k) * B(k,j)                 -- element formula: the
 *       dot product of row i of A with column j of B (dilfish.github.io
 *       section 5.2 snippet; chongfengling.github.io section 1; elainafan.one
 *       "稠密矩阵乘法").
 *   C <- alpha * A*B + beta * C                     -- the BLAS GEMM form:
 *       alpha scales the product and beta accumulates into the existing C
 *       in the same call (elainafan.one "稠密矩阵乘法", after the element
 *       formula).  The display formula is lost in the extraction; this is
 *       the reading the surrounding text supports.
 *   Row-major storage: X(r,c) = X[r*ld + c] with the column index
 *       contiguous (chongfengling.github.io section 2.2; elainafan.one
 *       "行主序" and the matmul_cpu listing).
 *   Transposed operands: C <- alpha * op(A)*op(B) + beta * C, where op(X) is
 *       X or its transpose, op(X)(r,c) = X(c,r).  A linear layer keeps its
 *       input X as [batch, in] and its weight W as [out, in], and both of
 *       its backward products are GEMMs (elainafan.one "全连接层"); with
 *       that storage the forward product is X * W^T, the weight gradient
 *       G^T * X and the input gradient G * W.  The page's formulas are lost
 *       in the extraction; these are the products its shapes admit.
 *       oracle_op forms op(X) explicitly before the product.
 *   Bias: the linear layer adds its bias vector b to every output row
 *       (elainafan.one "全连接层": X * W^T + b), so with a bias
 *       C(i,j) <- alpha * (op(A) op(B))(i,j) + beta * C(i,j) + b(j): added
 *       after the BLAS form, unscaled.  A batch of problems is a loop over
 *       independent problems (in the Python wrapper).
 *
 * Precision: every input is first widened EXACTLY to fp64 (fp32 values and
 * bf16 and IEEE binary16 bit patterns are all exact in fp64), so the oracle
 * consumes the already-rounded inputs.  The sum runs over k in ascending order and
 * accumulates in fp64.  Each product of two fp32 (24-bit significand) values
 * is exact in fp64 (48 <= 53 bits), so only the additions round.  The page's
 * own CPU loop (elainafan.one "CPU 实现") accumulates in float; the oracle
 * uses fp64 instead so that its own error (about K * 2^-53 relative) sits far
 * below the fp32 accumulation error of the device kernels it judges.
 *
 * Readings of points the pages leave open (each is also listed with the rest
 * of the readings in the design notes):
 *   - beta == 0: C is not read (BLAS convention), so NaN/Inf already in C
 *     cannot reach the result.
 *   - alpha == 0 or K == 0: the empty/zero product contributes exactly 0, so
 *     C <- beta*C (zeros when beta == 0 as well).
 *   - M == 0 or N == 0: nothing to compute.
 *
 * Two loop orders are provided.  oracle_gemm_ijk is the literal triple loop
 * (i, j, then k), one thread.  oracle_gemm is the same arithmetic in i-k-j
 * order with a row of fp64 accumulators, rows spread over OpenMP threads;
 * every element still sees its products added in ascending k, so the two are
 * bit-identical (the page notes that loop order changes cache behaviour, not
 * the operations: elainafan.one, paragraph after the matmul_cpu listing).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- op(X): the operand as used by the product ------------------------ */

/* out (rows x cols, packed) = op(X), where X is stored row-major with leading
 * dimension ld: X itself (rows x cols stored) when trans == 0, or the
 * transpose of X (X stored cols x rows) when trans == 1. */
void oracle_op(const double* X, int64_t rows, int64_t cols, int64_t ld, int trans,
               double* out) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = trans ? X[c * ld + r] : X[r * ld + c];
}

/* ---- exact widening of the inputs to fp64 ------------------------------ */

/* fp32 -> fp64: exact. dst is packed rows x cols. */
void oracle_widen_f32(const float* src, int64_t rows, int64_t cols, int64_t ld,
                      double* dst) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            dst[r * cols + c] = (double)src[r * ld + c];
}

/* bf16 bit pattern -> fp32 (the bits are the upper half) -> fp64: exact. */
static double bf16_bits_value(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

void oracle_widen_bf16(const uint16_t* src, int64_t rows, int64_t cols,
                       int64_t ld, double* dst) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            dst[r * cols + c] = bf16_bits_value(src[r * ld + c]);
}

/* IEEE 754 binary16 bit pattern -> fp64, from the format's definition:
 * sign bit 15, biased exponent bits 14..10 (bias 15), fraction bits 9..0.
 * Exponent 0: subnormal, fraction * 2^-24.  Exponent 31: infinity (fraction
 * 0) or NaN.  Otherwise (1024 + fraction) * 2^(exponent - 25).  Exact. */
static double f16_bits_value(uint16_t h) {
    const int sign = h >> 15, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)f, -24);
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

void oracle_widen_f16(const uint16_t* src, int64_t rows, int64_t cols,
                      int64_t ld, double* dst) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            dst[r * cols + c] = f16_bits_value(src[r * ld + c]);
}

/* ---- the definition ---------------------------------------------------- */

/* Epilogue of the BLAS form for one element: alpha*acc + beta*c0, with the
 * beta == 0 reading: c0 is not read then, even when the caller passed C0.
 * When beta != 0 the caller must pass C0. */
static double combine(double alpha, double acc, double beta, const double* c0) {
    double r = alpha * acc;
    if (beta != 0.0) r += beta * (*c0);
    return r;
}

/* The linear layer's bias: b(j) added to every row after the BLAS form
 * (bias == NULL: none). */
static double add_bias(double r, const double* bias, int64_t j) {
    return bias ? r + bias[j] : r;
}

/* Literal triple loop: for each (i, j), acc = sum over ascending k. */
void oracle_gemm_ijk(int64_t M, int64_t N, int64_t K, double alpha,
                     const double* A, int64_t lda, const double* B, int64_t ldb,
                     double beta, const double* C0, int64_t ldc0, const double* bias,
                     double* R, int64_t ldr) {
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += A[i * lda + k] * B[k * ldb + j];
            R[i * ldr + j] = add_bias(combine(alpha, acc, beta,
                                              C0 ? &C0[i * ldc0 + j] : NULL), bias, j);
        }
    }
}

/* Same arithmetic, i-k-j order: row i keeps N fp64 accumulators, and for
 * k = 0, 1, ... adds A(i,k)*B(k,j) into accumulator j.  Rows are independent
 * and are shared among threads; no sum is ever split across threads. */
void oracle_gemm(int64_t M, int64_t N, int64_t K, double alpha,
                 const double* A, int64_t lda, const double* B, int64_t ldb,
                 double beta, const double* C0, int64_t ldc0, const double* bias,
                 double* R, int64_t ldr) {
#pragma omp parallel
    {
        double* acc = (double*)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < M; ++i) {
            for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double a = A[i * lda + k];
                const double* brow = &B[k * ldb];
                for (int64_t j = 0; j < N; ++j) acc[j] += a * brow[j];
            }
            for (int64_t j = 0; j < N; ++j)
                R[i * ldr + j] = add_bias(combine(alpha, acc[j], beta,
                                                  C0 ? &C0[i * ldc0 + j] : NULL), bias, j);
        }
        free(acc);
    }
}

/* Round fp64 results to fp32, nearest-even (C's conversion under the default
 * rounding mode). */
void oracle_round_f32(const double* src, int64_t n, float* dst) {
    for (int64_t i = 0; i < n; ++i) dst[i] = (float)src[i];
}

/* Threads oracle_gemm will use (1 when built without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
