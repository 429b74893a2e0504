/*
 * gemm_oracle.c -- CPU reference ("oracle") for the bf16 GEMM with fp32
 * accumulation and fused alpha/beta/bias/GELU epilogue.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link
 * or call this file: only the test-suite, the package's smoke check and the
 * CPU-baseline leg of the benchmark use it.  It shares no code, header or
 * constant with the HIP library.
 *
 * What it computes is the plain definition, evaluated slowly and exactly up
 * to one final rounding:
 *
 *   C_out[m,n] = bf16_rne( epi( alpha * sum_k A[m,k]*B[k,n]
 *                               + beta * C_in[m,n]      (only if beta != 0)
 *                               + bias[n] ) )           (only if bias given)
 *
 * Sources (web pages on the subject):
 *  - "Outperforming cuBLAS on H100: a worklog" (P. Shankhdhar), section
 *    "Recap of Simon's blog": the product C[m,n] = A[m,k] x B[k,n];
 *    section "Experimental setup": bf16 matrices, A row-major, B and C
 *    column-major.
 *  - DeepGEMM kernel-set article (demingchina.com), sections 1.2 and 6.3:
 *    low-precision FP8 inputs; the fp8 product below takes OCP FP8 E4M3
 *    operands (4 exponent bits, bias 7, 3 mantissa bits, no infinities,
 *    S.1111.111 = NaN) with optional per-row scales of A and per-column
 *    scales of B.
 *  - The same DeepGEMM article, section 1.1: the BLAS
 *    form C = alpha*A*B + beta*C; section 3.1: low-precision inputs with
 *    high-precision accumulation; section 6.1: bias is added first, then the
 *    activation (ReLU/GELU) is applied, then the result is written;
 *    section 6.2: an int8 output quantized per token (per row of C),
 *    y = round(x * scale + zero_point), with x the fp32 GEMM output.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - GELU is the tanh form 0.5*y*(1+tanh(sqrt(2/pi)*(y+0.044715*y^3))),
 *    applied to the whole pre-activation sum (alpha*AB + beta*C + bias).
 *  - ReLU is y < 0 ? 0 : y (NaN passes through).
 *  - Quantization: x is the epilogue value rounded once to fp32 (the page's
 *    "FP32 output"); the code is decided in fp32 as the page's formula
 *    reads, t = fma(x, scale[m], zero_point) (one rounding), then rounded to
 *    the nearest integer with ties to even, then saturated to [-128, 127];
 *    a NaN t gives 0.  "Per token" is read as one scale per row m of C.
 *  - bias is indexed by the output column n (length N).
 *  - beta == 0 means C_in is not read at all (BLAS convention).
 *  - Accumulation is in double; every bf16*bf16 product is exact in double
 *    (8+8 significant bits), and each output element sums its products in
 *    ascending k.  The result is rounded to bf16 ONCE, round-to-nearest-even,
 *    directly from double (no intermediate float rounding).
 *
 * Layout (same meaning as the library's arguments):
 *   A: row-major M x K,     element (m,k) at A[m*lda + k], lda >= K
 *   B: column-major K x N,  element (k,n) at B[k + n*ldb], ldb >= K
 *   C: column-major M x N,  element (m,n) at C[m + n*ldc], ldc >= M
 *
 * Parallelism: output elements are independent and each one is computed by a
 * single thread in a fixed order, so the result does not depend on the
 * thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <omp.h>

#define ORACLE_EPI_NONE 0
#define ORACLE_EPI_GELU_TANH 1
#define ORACLE_EPI_RELU 2
#define ORACLE_PI 3.14159265358979323846264338327950288

/* Exact decode: bf16 is the upper half of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Round a double to the nearest bf16 (8 significant bits, binary32 exponent
 * range, subnormals down to 2^-133), ties to even, in one step.
 *
 * Method: find the binade exponent e = floor(log2|x|) (clamped to -126, below
 * which the spacing stays 2^-133), the spacing q = 2^(e-7) of bf16 values in
 * that binade, and round |x|/q to an integer with rint() (the default
 * round-to-nearest-even mode).  |x|/q and r*q are exact (scaling by a power
 * of two).  A result of 2^128 or more is an overflow and becomes infinity,
 * which is also where IEEE round-to-nearest sends it.
 */
uint16_t oracle_bf16_from_f64(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    double ax = fabs(x);
    if (isinf(ax))
        return (uint16_t)(sign | 0x7F80u);
    if (ax == 0.0)
        return sign;
    int E;
    (void)frexp(ax, &E);           /* ax = f * 2^E with f in [0.5, 1) */
    int e = E - 1;                 /* floor(log2(ax)) */
    if (e < -126)
        e = -126;
    double q = ldexp(1.0, e - 7);  /* spacing of bf16 values near ax */
    double r = rint(ax / q) * q;
    if (r >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80u);
    float f = (float)r;            /* exact: r has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)(u >> 16));
}

/* GELU, tanh form (Hendrycks & Gimpel), evaluated in double with libm tanh. */
double oracle_gelu_tanh(double y)
{
    const double c = sqrt(2.0 / ORACLE_PI);
    return 0.5 * y * (1.0 + tanh(c * (y + 0.044715 * y * y * y)));
}

/* ReLU: negative values to 0, everything else (NaN included) unchanged. */
double oracle_relu(double y)
{
    return y < 0.0 ? 0.0 : y;
}

/*
 * The int8 code of one epilogue value y for a row with scale s and zero
 * point zp, decided in fp32: x = (float)y, t = fmaf(x, s, zp), round half to
 * even (rintf in the default rounding mode), saturate.  *t_exact (if not
 * NULL) receives y*s + zp in double, the value the decision approximates.
 */
int oracle_quantize_i8(double y, float s, int32_t zp, double *t_exact)
{
    if (t_exact)
        *t_exact = y * (double)s + (double)zp;
    float x = (float)y;
    float t = fmaf(x, s, (float)zp);
    if (isnan(t))
        return 0;
    float r = rintf(t);
    if (r < -128.0f)
        return -128;
    if (r > 127.0f)
        return 127;
    return (int)r;
}

/* oracle_quantize_i8 over n values with their own scales (for sampled
 * elements); t_exact may be NULL. */
void oracle_quantize_i8_array(const double *y, const float *s, int32_t zp, int8_t *q, double *t_exact,
                              int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        q[i] = (int8_t)oracle_quantize_i8(y[i], s[i], zp, t_exact ? &t_exact[i] : NULL);
}

/*
 * Exact decode of an OCP FP8 E4M3 value: (-1)^s * 2^(e-7) * (1 + m/8) for
 * exponent field e >= 1, (-1)^s * 2^-6 * m/8 for e == 0, NaN for e == 15 and
 * m == 7 (the format has no infinities).
 */
double oracle_fp8_e4m3_to_f64(uint8_t bits)
{
    int s = (bits >> 7) & 1, e = (bits >> 3) & 15, m = bits & 7;
    if (e == 15 && m == 7)
        return NAN;
    double mag = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
    return s ? -mag : mag;
}

void oracle_fp8_e4m3_to_f64_array(const uint8_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_fp8_e4m3_to_f64(in[i]);
}

/* Element-wise array forms of the two conversions (n elements). */
void oracle_bf16_to_f64_array(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_to_f64(in[i]);
}

void oracle_bf16_from_f64_array(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_from_f64(in[i]);
}

void oracle_gelu_tanh_array(const double *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_gelu_tanh(in[i]);
}

/* sum_k A[m,k] * B[k,n] in double, k ascending. */
static double dot_row_col(const uint16_t *a_row, const uint16_t *b_col, int64_t K)
{
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k)
        s += oracle_bf16_to_f64(a_row[k]) * oracle_bf16_to_f64(b_col[k]);
    return s;
}

/* The epilogue on one element, in double: alpha*s (+ beta*c0) (+ bias), act. */
static double epilogue(double s, double alpha, double beta, const uint16_t *c_in,
                       const uint16_t *bias, int64_t n, int epi)
{
    double y = alpha * s;
    if (beta != 0.0)
        y += beta * oracle_bf16_to_f64(*c_in);
    if (bias)
        y += oracle_bf16_to_f64(bias[n]);
    if (epi == ORACLE_EPI_GELU_TANH)
        y = oracle_gelu_tanh(y);
    else if (epi == ORACLE_EPI_RELU)
        y = oracle_relu(y);
    return y;
}

static int epi_ok(int epi)
{
    return epi == ORACLE_EPI_NONE || epi == ORACLE_EPI_GELU_TANH || epi == ORACLE_EPI_RELU;
}

/*
 * Full product.  C_in (may be NULL when beta == 0) and C_out are separate
 * buffers with the same leading dimension ldc.  If `pre` is not NULL it
 * receives the double value before the final rounding, column-major with
 * leading dimension M.  Returns 0, or -1 on a bad argument.
 */
int oracle_gemm(int64_t M, int64_t N, int64_t K,
                const uint16_t *A, int64_t lda,
                const uint16_t *B, int64_t ldb,
                const uint16_t *C_in, int64_t ldc,
                double alpha, double beta,
                const uint16_t *bias, int epi,
                uint16_t *C_out, double *pre, int nthreads)
{
    if (M < 0 || N < 0 || K < 0)
        return -1;
    if (lda < (K > 1 ? K : 1) || ldb < (K > 1 ? K : 1) || ldc < (M > 1 ? M : 1))
        return -1;
    if (!epi_ok(epi))
        return -1;
    if (beta != 0.0 && !C_in)
        return -1;
    if (nthreads < 1)
        nthreads = omp_get_max_threads();
    int64_t total = M * N;
#pragma omp parallel for schedule(dynamic, 64) num_threads(nthreads)
    for (int64_t idx = 0; idx < total; ++idx) {
        int64_t n = idx / M, m = idx % M;
        double s = dot_row_col(A + m * lda, B + n * ldb, K);
        double y = epilogue(s, alpha, beta, C_in ? C_in + m + n * ldc : NULL, bias, n, epi);
        if (pre)
            pre[m + n * M] = y;
        C_out[m + n * ldc] = oracle_bf16_from_f64(y);
    }
    return 0;
}

/*
 * The same definition on a list of output coordinates (m[i], n[i]) only, for
 * checking sampled elements of products too large to evaluate in full.
 */
int oracle_gemm_elems(int64_t M, int64_t N, int64_t K,
                      const uint16_t *A, int64_t lda,
                      const uint16_t *B, int64_t ldb,
                      const uint16_t *C_in, int64_t ldc,
                      double alpha, double beta,
                      const uint16_t *bias, int epi,
                      int64_t count, const int64_t *ms, const int64_t *ns,
                      uint16_t *out, double *pre, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || count < 0)
        return -1;
    if (lda < (K > 1 ? K : 1) || ldb < (K > 1 ? K : 1) || ldc < (M > 1 ? M : 1))
        return -1;
    if (!epi_ok(epi))
        return -1;
    if (beta != 0.0 && !C_in)
        return -1;
    for (int64_t i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N)
            return -1;
    if (nthreads < 1)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i];
        double s = dot_row_col(A + m * lda, B + n * ldb, K);
        double y = epilogue(s, alpha, beta, C_in ? C_in + m + n * ldc : NULL, bias, n, epi);
        if (pre)
            pre[i] = y;
        out[i] = oracle_bf16_from_f64(y);
    }
    return 0;
}

/*
 * The quantizing product: Q[m + n*ldq] = oracle_quantize_i8(y[m,n], scale[m],
 * zp) with y the epilogue value of oracle_gemm (before any bf16 rounding).
 * C_in is read only when beta != 0.  If `t_exact` is not NULL it receives
 * y*scale[m] + zp in double, column-major with leading dimension M.
 */
int oracle_gemm_q8(int64_t M, int64_t N, int64_t K,
                   const uint16_t *A, int64_t lda,
                   const uint16_t *B, int64_t ldb,
                   const uint16_t *C_in, int64_t ldc,
                   double alpha, double beta,
                   const uint16_t *bias, int epi,
                   const float *scale, int32_t zp,
                   int8_t *Q, int64_t ldq, double *t_exact, int nthreads)
{
    if (M < 0 || N < 0 || K < 0)
        return -1;
    if (lda < (K > 1 ? K : 1) || ldb < (K > 1 ? K : 1) || ldq < (M > 1 ? M : 1))
        return -1;
    if (beta != 0.0 && (!C_in || ldc < (M > 1 ? M : 1)))
        return -1;
    if (!epi_ok(epi) || (M > 0 && !scale))
        return -1;
    if (nthreads < 1)
        nthreads = omp_get_max_threads();
    int64_t total = M * N;
#pragma omp parallel for schedule(dynamic, 64) num_threads(nthreads)
    for (int64_t idx = 0; idx < total; ++idx) {
        int64_t n = idx / M, m = idx % M;
        double s = dot_row_col(A + m * lda, B + n * ldb, K);
        double y = epilogue(s, alpha, beta, beta != 0.0 ? C_in + m + n * ldc : NULL, bias, n, epi);
        Q[m + n * ldq] = (int8_t)oracle_quantize_i8(y, scale[m], zp, t_exact ? &t_exact[m + n * M] : NULL);
    }
    return 0;
}

/*
 * The fp8-input product: C_out[m,n] = bf16_rne(epi(alpha * sa[m] * sb[n] *
 * sum_k A[m,k]*B[k,n] + beta*C_in[m,n] + bias[n])), A and B OCP FP8 E4M3
 * bytes in the same layouts as the bf16 product (A[m*lda + k], B[k + n*ldb]),
 * sa / sb per-row / per-column fp32 scales or NULL (1).  Products of two
 * E4M3 values are exact in double and summed with k ascending; the scale
 * factors multiply the exact sum in double.  `pre` (if not NULL) receives
 * the value before rounding, column-major with leading dimension M.
 */
int oracle_gemm_fp8(int64_t M, int64_t N, int64_t K,
                    const uint8_t *A, int64_t lda,
                    const uint8_t *B, int64_t ldb,
                    const uint16_t *C_in, int64_t ldc,
                    double alpha, double beta,
                    const float *sa, const float *sb,
                    const uint16_t *bias, int epi,
                    uint16_t *C_out, double *pre, int nthreads)
{
    if (M < 0 || N < 0 || K < 0)
        return -1;
    if (lda < (K > 1 ? K : 1) || ldb < (K > 1 ? K : 1) || ldc < (M > 1 ? M : 1))
        return -1;
    if (!epi_ok(epi) || (beta != 0.0 && !C_in))
        return -1;
    if (nthreads < 1)
        nthreads = omp_get_max_threads();
    int64_t total = M * N;
#pragma omp parallel for schedule(dynamic, 64) num_threads(nthreads)
    for (int64_t idx = 0; idx < total; ++idx) {
        int64_t n = idx / M, m = idx % M;
        const uint8_t *a = A + m * lda, *b = B + n * ldb;
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += oracle_fp8_e4m3_to_f64(a[k]) * oracle_fp8_e4m3_to_f64(b[k]);
        if (sa)
            s *= (double)sa[m];
        if (sb)
            s *= (double)sb[n];
        double y = epilogue(s, alpha, beta, beta != 0.0 ? C_in + m + n * ldc : NULL, bias, n, epi);
        if (pre)
            pre[m + n * M] = y;
        C_out[m + n * ldc] = oracle_bf16_from_f64(y);
    }
    return 0;
}

/* The fp8 definition above on a list of output coordinates only. */
int oracle_gemm_fp8_elems(int64_t M, int64_t N, int64_t K,
                          const uint8_t *A, int64_t lda,
                          const uint8_t *B, int64_t ldb,
                          const uint16_t *C_in, int64_t ldc,
                          double alpha, double beta,
                          const float *sa, const float *sb,
                          const uint16_t *bias, int epi,
                          int64_t count, const int64_t *ms, const int64_t *ns,
                          uint16_t *out, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || count < 0)
        return -1;
    if (lda < (K > 1 ? K : 1) || ldb < (K > 1 ? K : 1) || ldc < (M > 1 ? M : 1))
        return -1;
    if (!epi_ok(epi) || (beta != 0.0 && !C_in))
        return -1;
    for (int64_t i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N)
            return -1;
    if (nthreads < 1)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i];
        const uint8_t *a = A + m * lda, *b = B + n * ldb;
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += oracle_fp8_e4m3_to_f64(a[k]) * oracle_fp8_e4m3_to_f64(b[k]);
        if (sa)
            s *= (double)sa[m];
        if (sb)
            s *= (double)sb[n];
        double y = epilogue(s, alpha, beta, beta != 0.0 ? C_in + m + n * ldc : NULL, bias, n, epi);
        out[i] = oracle_bf16_from_f64(y);
    }
    return 0;
}
