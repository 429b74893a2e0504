/*
 * gemm_bf16.h -- C ABI of the MI355X (gfx950) bf16 GEMM library.
 *
 *   C[m,n] <- epi( alpha * sum_k A[m,k] * B[k,n] + beta * C[m,n] + bias[n] )
 *
 * The product and the layouts (bf16 matrices, A row-major, B and C
 * column-major) follow "Outperforming cuBLAS on H100: a worklog", sections
 * "Recap of Simon's blog" and "Experimental setup".  The BLAS form with alpha
 * and beta, fp32 accumulation of bf16 inputs, and the fused epilogue (bias
 * first, then the activation, then the write) follow the DeepGEMM kernel-set
 * article on demingchina.com, sections 1.1, 3.1 and 6.1.
 *
 * Numerics: products of bf16 inputs are accumulated in fp32 on the MFMA
 * units; alpha, beta*C, bias and the activation are applied in fp32; the
 * result is rounded once to bf16, round-to-nearest-even.
 *
 * gemm_bf16_q8 writes int8 instead: the same fp32 epilogue value, then a
 * per-row quantization (section 6.2 of the same article).
 *
 * Every function is thread-safe.  The library keeps no pointer to caller
 * buffers after a call returns.  Its one device allocation is the split-K
 * workspace (fp32 partial sums, and per-strip arrival counters or handoff
 * records for the short-product kernel, whose splits pass their partials
 * within one XCD where the strips allow it), used by shapes of two kinds:
 * 3 <= M <= 64 with few columns, and products, bf16 or FP8, whose 128x128
 * tiles would leave most compute units idle and whose K is long enough to
 * pay for the split (for example 512 x 512 x 8192; with tails the partials
 * are padded to whole tiles).  It is one buffer per
 * (device, stream) of a fixed size -- 64 KiB of counters plus 64 KiB per
 * compute unit (16 MiB + 64 KiB on a 256-CU device) -- allocated with
 * hipMalloc by the first call on that stream that splits K (its counters
 * zeroed by a fill kernel on the stream), never grown or freed, and kept
 * until the process ends; no split plan needs more, so no later call
 * allocates, frees or synchronises.  Calls whose shape needs no split
 * allocate nothing.  A first split call made under HIP graph capture fails
 * with GEMM_ERR_HIP when the runtime refuses hipMalloc during capture:
 * callers that capture use gemm_bf16_noalloc.
 */
#ifndef GEMM_BF16_H
#define GEMM_BF16_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Raw bf16 bits (sign, 8-bit exponent, 7-bit mantissa). */
typedef uint16_t gemm_bf16_t;

/* Raw OCP FP8 E4M3 bits (sign, 4-bit exponent with bias 7, 3-bit mantissa;
 * no infinities, S.1111.111 is NaN). */
typedef uint8_t gemm_fp8_t;

/* Epilogue activation, applied last to alpha*AB + beta*C + bias (the
 * DeepGEMM article, section 6.1: bias first, then ReLU or GELU). */
enum gemm_bf16_epilogue {
    GEMM_EPI_NONE = 0,
    /* GELU, tanh form: 0.5x(1 + tanh(sqrt(2/pi)(x + 0.044715x^3))) */
    GEMM_EPI_GELU_TANH = 1,
    /* ReLU: x < 0 ? 0 : x (NaN passes through) */
    GEMM_EPI_RELU = 2
};

/* Status codes.  Argument errors are detected on the host, in this order,
 * before any HIP call is made. */
enum gemm_bf16_status {
    GEMM_OK = 0,
    GEMM_ERR_DIM = -1,       /* M, N or K negative */
    GEMM_ERR_LD = -2,        /* lda < max(1,K), ldb < max(1,K) or ldc < max(1,M) */
    GEMM_ERR_NULL = -3,      /* NULL A (M*K>0), NULL B (K*N>0) or NULL C (M*N>0) */
    GEMM_ERR_EPILOGUE = -4,  /* epilogue not in enum gemm_bf16_epilogue */
    GEMM_ERR_HIP = -5        /* the HIP runtime reported an error; see
                                gemm_bf16_last_hip_error() */
};

/*
 * gemm_bf16 -- enqueue C <- epi(alpha*A*B + beta*C + bias) on `stream`.
 *
 *   M, N, K  problem size (any value >= 0).
 *   A        device pointer, row-major M x K: element (m,k) at A[m*lda + k].
 *   B        device pointer, column-major K x N: element (k,n) at B[k + n*ldb].
 *   C        device pointer, column-major M x N: element (m,n) at C[m + n*ldc].
 *            In/out: holds the initial C when beta != 0.  When beta == 0 it
 *            is write-only and is never read (NaN in it cannot propagate).
 *   alpha, beta  fp32 scalars.
 *   bias     NULL, or a device pointer to N bf16 values added to column n.
 *   epilogue one of enum gemm_bf16_epilogue.
 *   stream   HIP stream (0 = the null stream).  The call is asynchronous: it
 *            enqueues the work and returns without synchronising.
 *
 * Quick returns: M == 0 or N == 0 enqueues nothing.  K == 0 computes
 * C <- epi(beta*C + bias) (the empty sum contributes nothing).
 *
 * Any alignment of the pointers (2-byte bf16 alignment) and any leading
 * dimensions are accepted.  The fast kernels need K, lda and ldb multiples
 * of 8 and A, B 16-byte aligned (the large-grid ones also C aligned and
 * ldc % 8 == 0; the 128x128 kernel for shapes with tails takes any C);
 * other inputs take a bounds-checked path that computes the same result
 * more slowly.
 *
 * Ownership: all buffers belong to the caller and must stay valid until the
 * enqueued work has completed.  A, B and bias must not overlap C.  The
 * split-K workspace (see above) is shared by the calls on one stream, which
 * run in order; calls on different streams use different workspaces.
 *
 * Returns GEMM_OK or a negative gemm_bf16_status.
 */
int gemm_bf16(int64_t M, int64_t N, int64_t K,
              const gemm_bf16_t *A, int64_t lda,
              const gemm_bf16_t *B, int64_t ldb,
              gemm_bf16_t *C, int64_t ldc,
              float alpha, float beta,
              const gemm_bf16_t *bias,
              int epilogue, hipStream_t stream);

/*
 * gemm_bf16_noalloc -- gemm_bf16 for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, result, kernels and errors as
 * gemm_bf16; it never calls hipMalloc, hipFree or any allocating routine.
 *
 * Its split-K scratch is a static device array inside the library (64 KiB
 * of counters and 16 MiB of fp32 partials, sized for 256 compute units),
 * one copy per GPU, held until the process ends.  Split plans are capped to
 * fit it (on a device with more than 256 compute units a shape may split
 * less than under gemm_bf16); a plan that would not fit is refused with
 * GEMM_ERR_HIP (hipErrorInvalidValue) before anything is enqueued -- by
 * construction no shape reaches that.  The first call on a device looks up
 * the array and enqueues one small kernel that zeroes its counters; every
 * later call enqueues only the product's kernels.
 *
 * All gemm_bf16_noalloc calls on one GPU share that one array, and it
 * keeps the last call's contents: calls that may overlap on one GPU (on
 * different streams, or from several threads without ordering) race on it
 * and give undefined results.  Calls ordered on one stream are safe.
 */
int gemm_bf16_noalloc(int64_t M, int64_t N, int64_t K,
                      const gemm_bf16_t *A, int64_t lda,
                      const gemm_bf16_t *B, int64_t ldb,
                      gemm_bf16_t *C, int64_t ldc,
                      float alpha, float beta,
                      const gemm_bf16_t *bias,
                      int epilogue, hipStream_t stream);

/*
 * gemm_bf16_q8 -- enqueue the same product and epilogue with an int8 output
 * quantized per row (per token): the DeepGEMM article (demingchina.com),
 * section 6.2, y = round(x * scale + zero_point) with one scale per row.
 *
 *   Q[m + n*ldq] = sat8( rne( fma( v[m,n], scale[m], zero_point ) ) )
 *   v[m,n]       = epi( alpha * sum_k A[m,k]*B[k,n] + beta*C[m,n] + bias[n] )
 *
 * v is the fp32 value gemm_bf16 would round to bf16; the multiply-add is one
 * fp32 fused operation, rne rounds to the nearest integer with ties to even,
 * sat8 clamps to [-128, 127], and a NaN v gives 0.
 *
 *   A, lda, B, ldb, alpha, beta, bias, epilogue, stream: as in gemm_bf16.
 *   C        device pointer, column-major M x N bf16 input C0 (element (m,n)
 *            at C[m + n*ldc]), read only when beta != 0; may be NULL (and
 *            ldc anything) when beta == 0.  Never written.
 *   Q        device pointer, column-major M x N int8 output, element (m,n)
 *            at Q[m + n*ldq], ldq >= max(1, M).  Rows M..ldq-1 untouched.
 *   scale    device pointer to M fp32 scales, one per row m.
 *   zero_point  added after the scaling (converted to fp32).
 *
 * Errors as gemm_bf16, with these differences: GEMM_ERR_LD also when
 * ldq < max(1,M), and ldc is only checked when beta != 0; GEMM_ERR_NULL also
 * for a NULL Q or scale (M*N > 0), and for a NULL C only when beta != 0.
 * Q must not overlap A, B, C, bias or scale.
 *
 * Kernels: 1 <= M <= 64 (K, lda, ldb multiples of 8, A and B 16-byte
 * aligned; any ldc, ldq and Q alignment) the streaming kernel, splitting K
 * through the split-K workspace when the strips are few; large grids the
 * 256x256 ring kernel (Q, scale 16-byte aligned, ldq % 8 == 0); small grids
 * of 128x128 tiles split-K with a quantizing reduction; else the
 * bounds-checked kernel.  All give the same result.
 */
int gemm_bf16_q8(int64_t M, int64_t N, int64_t K,
                 const gemm_bf16_t *A, int64_t lda,
                 const gemm_bf16_t *B, int64_t ldb,
                 const gemm_bf16_t *C, int64_t ldc,
                 int8_t *Q, int64_t ldq,
                 float alpha, float beta,
                 const gemm_bf16_t *bias, int epilogue,
                 const float *scale, int32_t zero_point,
                 hipStream_t stream);

/*
 * gemm_fp8 -- enqueue the product of FP8 operands, the FP8 input path of the
 * DeepGEMM article (demingchina.com), sections 1.2 and 6.3:
 *
 *   C[m,n] <- epi( alpha * sa[m] * sb[n] * sum_k A[m,k]*B[k,n]
 *                  + beta * C[m,n] + bias[n] )
 *
 * with A and B OCP FP8 E4M3 values (exact products, fp32 accumulation), the
 * scales, alpha, beta*C, bias and the activation in fp32, one RNE to bf16.
 *
 *   A        device pointer, row-major M x K bytes: A[m*lda + k], lda >= K.
 *   B        device pointer, column-major K x N bytes: B[k + n*ldb], ldb >= K.
 *   C, ldc, alpha, beta, bias, epilogue, stream: as in gemm_bf16.
 *   scale_a  NULL (all 1), or a device pointer to M fp32 per-row scales.
 *   scale_b  NULL (all 1), or a device pointer to N fp32 per-column scales.
 *
 * Errors and quick returns as gemm_bf16.  With K, lda and ldb multiples of
 * 16 and A, B 16-byte aligned: 1 <= M <= 2 (and 3 <= M <= 4 when
 * N * K < 2^26) takes a matrix-vector kernel and the other M <= 64 a
 * streaming FP8 MFMA kernel (any ldc); larger M the 256x256 FP8 MFMA
 * kernel, or where its tiles would fill less than half of the compute
 * units the 128x128 one (any M and N: tails are masked; exact tile
 * multiples with C 16-byte aligned and ldc % 8 == 0 run unmasked, anything
 * else accesses C element by element where it must).  On those small grids
 * K is split over several ranges when it is long enough (fp32 partial tiles
 * in the split-K workspace, then an ordered reduction that applies the
 * scales and the epilogue).  Other inputs take the bounds-checked path
 * (same result).
 */
int gemm_fp8(int64_t M, int64_t N, int64_t K,
             const gemm_fp8_t *A, int64_t lda,
             const gemm_fp8_t *B, int64_t ldb,
             gemm_bf16_t *C, int64_t ldc,
             float alpha, float beta,
             const float *scale_a, const float *scale_b,
             const gemm_bf16_t *bias, int epilogue,
             hipStream_t stream);

/* Human-readable text for a status code (static storage, never NULL). */
const char *gemm_bf16_status_string(int status);

/* The hipError_t of the calling thread's most recent GEMM_ERR_HIP, else 0. */
int gemm_bf16_last_hip_error(void);

/*
 * gemm_bf16_kernel_name -- name of the kernel configuration gemm_bf16 would
 * launch for these arguments (static storage), e.g. "ring256x256x64",
 * or "none" when nothing would be launched or the arguments are invalid.
 * Makes no HIP call apart from querying the current device's compute-unit
 * count.  Pointers are only inspected for their alignment.
 */
const char *gemm_bf16_kernel_name(int64_t M, int64_t N, int64_t K,
                                  const gemm_bf16_t *A, int64_t lda,
                                  const gemm_bf16_t *B, int64_t ldb,
                                  const gemm_bf16_t *C, int64_t ldc,
                                  float beta, const gemm_bf16_t *bias,
                                  int epilogue);

/* The kernel configuration gemm_bf16_q8 would launch (as
 * gemm_bf16_kernel_name). */
const char *gemm_bf16_q8_kernel_name(int64_t M, int64_t N, int64_t K,
                                     const gemm_bf16_t *A, int64_t lda,
                                     const gemm_bf16_t *B, int64_t ldb,
                                     const gemm_bf16_t *C, int64_t ldc,
                                     const int8_t *Q, int64_t ldq,
                                     float beta, const float *scale,
                                     int epilogue);

/* The kernel configuration gemm_fp8 would launch (as gemm_bf16_kernel_name). */
const char *gemm_fp8_kernel_name(int64_t M, int64_t N, int64_t K,
                                 const gemm_fp8_t *A, int64_t lda,
                                 const gemm_fp8_t *B, int64_t ldb,
                                 const gemm_bf16_t *C, int64_t ldc,
                                 int epilogue);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_BF16_H */
