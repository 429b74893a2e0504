// gemm_bf16.hip -- host side of the library: argument validation, kernel
// selection and launch behind the C ABI declared in include/gemm_bf16.h.
#include "gemm_bf16.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "configs.h"
#include "device_common.h"
#include "kernel_generic.h"

namespace gb {

enum KernelKind {
    kNone = 0, kLarge, kMedium, kSkinny64, kSkinny32, kGeneric, kRing32, kRing, kRingMasked, kRingQ8, kNumKinds
};

static const char *const kKindNames[kNumKinds] = {"none",            "tile256x256x32_s5", "tile128x128x64_s4",
                                                  "skinny64x32x256", "skinny32x32x256",   "generic64x64x32",
                                                  "ring256x256x64_mfma32", "ring256x256x64",
                                                  "ring256x256x64_masked", "ring256x256x64_q8"};

static const char *kind_name(int k) { return (k >= 0 && k < kNumKinds) ? kKindNames[k] : "none"; }

static thread_local int t_last_hip_error = 0;

// Compute-unit count per device, filled on first use (benign race: every
// thread computes the same value).
static std::atomic<int> g_cu_count[64];

static int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    g_cu_count[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

static bool epilogue_ok(int epilogue) {
    return epilogue == GEMM_EPI_NONE || epilogue == GEMM_EPI_GELU_TANH || epilogue == GEMM_EPI_RELU;
}

static uint32_t epilogue_flags(float beta, const void *bias, int epilogue) {
    return (beta != 0.0f ? kEpiBeta : 0u) | (bias ? kEpiBias : 0u) |
           (epilogue == GEMM_EPI_GELU_TANH ? kEpiGelu : 0u) | (epilogue == GEMM_EPI_RELU ? kEpiRelu : 0u);
}

static int validate(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                    const void *C, int64_t ldc, int epilogue) {
    if (M < 0 || N < 0 || K < 0) return GEMM_ERR_DIM;
    const int64_t kmin = K > 1 ? K : 1, mmin = M > 1 ? M : 1;
    if (lda < kmin || ldb < kmin || ldc < mmin) return GEMM_ERR_LD;
    if ((M > 0 && K > 0 && !A) || (K > 0 && N > 0 && !B) || (M > 0 && N > 0 && !C)) return GEMM_ERR_NULL;
    if (!epilogue_ok(epilogue)) return GEMM_ERR_EPILOGUE;
    return GEMM_OK;
}

// The quantizing entry point: C (the bf16 C0) is only needed when beta != 0;
// Q (M x N int8, ldq >= M) and scale (M floats) always.
static int validate_q8(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                       const void *C, int64_t ldc, const void *Q, int64_t ldq, float beta, const void *scale,
                       int epilogue) {
    if (M < 0 || N < 0 || K < 0) return GEMM_ERR_DIM;
    const int64_t kmin = K > 1 ? K : 1, mmin = M > 1 ? M : 1;
    if (lda < kmin || ldb < kmin || ldq < mmin || (beta != 0.0f && ldc < mmin)) return GEMM_ERR_LD;
    const bool out = M > 0 && N > 0;
    if ((M > 0 && K > 0 && !A) || (K > 0 && N > 0 && !B) || (out && beta != 0.0f && !C) || (out && !Q) ||
        (out && !scale))
        return GEMM_ERR_NULL;
    if (!epilogue_ok(epilogue)) return GEMM_ERR_EPILOGUE;
    return GEMM_OK;
}

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <class Cfg>
static bool tile_path_ok(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                         int64_t ldb, const void *C, int64_t ldc) {
    if (K <= 0 || M % Cfg::BM || N % Cfg::BN || K % Cfg::BK) return false;
    if (lda % 8 || ldb % 8 || ldc % 8) return false;
    if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return false;
    // 32-bit buffer offsets inside a tile's rows
    const int64_t lim = (int64_t)1 << 31;
    if ((Cfg::BM * lda + K) * 2 >= lim || (Cfg::BN * ldb + K) * 2 >= lim) return false;
    // tile indices held in int
    if (M / Cfg::BM * (N / Cfg::BN) >= lim) return false;
    return true;
}

// The masked ring kernel: any M, N >= 1; K and the leading dimensions
// multiples of 8 (16-byte operand chunks and C columns), 16-byte aligned
// pointers, 32-bit buffer offsets within a tile's rows.
static bool ring_masked_ok(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                           int64_t ldb, const void *C, int64_t ldc) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 8) return false;
    if (lda % 8 || ldb % 8 || ldc % 8) return false;
    if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return false;
    const int64_t lim = (int64_t)1 << 31;
    if ((ShapeRing::BM * lda + K) * 2 >= lim || (ShapeRing::BN * ldb + K) * 2 >= lim) return false;
    if (K + ShapeRing::BK >= lim) return false;
    const int64_t tiles = ((M + ShapeRing::BM - 1) / ShapeRing::BM) * ((N + ShapeRing::BN - 1) / ShapeRing::BN);
    return tiles < lim;
}

static bool skinny_path_ok(int rows, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                           int64_t ldb, const void *C, int64_t ldc) {
    if (M != rows || K <= 0 || N % ShapeSkinny::BN || K % ShapeSkinny::KS) return false;
    if (lda % 8 || ldb % 8 || ldc % 8) return false;
    if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return false;
    const int64_t lim = (int64_t)1 << 31;
    if (((rows - 1) * lda + K) * 2 >= lim || ((ShapeSkinny::BN - 1) * ldb + K) * 2 >= lim) return false;
    if (N / ShapeSkinny::BN >= lim) return false;
    return true;
}

// Kernel for a shape.  GEMM_BF16_FORCE_KERNEL=<name> (a kKindNames entry)
// overrides the choice when that kernel can run the shape; it exists for
// testing and benchmarking the alternatives.
static int choose_kernel(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                         int64_t ldb, const void *C, int64_t ldc, int cus) {
    if (M == 0 || N == 0) return kNone;
    const bool okL = tile_path_ok<ShapeL>(M, N, K, A, lda, B, ldb, C, ldc);
    const bool okM = tile_path_ok<ShapeM>(M, N, K, A, lda, B, ldb, C, ldc);
    const bool okR = tile_path_ok<ShapeRing>(M, N, K, A, lda, B, ldb, C, ldc);
    const bool okRM = ring_masked_ok(M, N, K, A, lda, B, ldb, C, ldc);
    const bool okS64 = skinny_path_ok(64, M, N, K, A, lda, B, ldb, C, ldc);
    const bool okS32 = skinny_path_ok(32, M, N, K, A, lda, B, ldb, C, ldc);
    if (const char *force = std::getenv("GEMM_BF16_FORCE_KERNEL")) {
        if (!std::strcmp(force, kKindNames[kGeneric])) return kGeneric;
        if (!std::strcmp(force, kKindNames[kLarge]) && okL) return kLarge;
        if (!std::strcmp(force, kKindNames[kMedium]) && okM) return kMedium;
        if (!std::strcmp(force, kKindNames[kRing32]) && okR) return kRing32;
        if (!std::strcmp(force, kKindNames[kRing]) && okR) return kRing;
        if (!std::strcmp(force, kKindNames[kRingMasked]) && okRM) return kRingMasked;
        if (!std::strcmp(force, kKindNames[kSkinny64]) && okS64) return kSkinny64;
        if (!std::strcmp(force, kKindNames[kSkinny32]) && okS32) return kSkinny32;
    }
    // 256x256 tiles when they give at least half the compute units a tile:
    // exact multiples take the unmasked ring kernel, shapes with tails the
    // masked one.
    if (okRM) {
        const int64_t tiles = ((M + ShapeRing::BM - 1) / ShapeRing::BM) * ((N + ShapeRing::BN - 1) / ShapeRing::BN);
        if (tiles * 2 >= cus || (!okM && okR)) return okR ? kRing : kRingMasked;
    }
    if (okL) {
        const int64_t tiles = (M / ShapeL::BM) * (N / ShapeL::BN);
        if (tiles * 2 >= cus || !okM) return kLarge;
    }
    if (okM) return kMedium;
    if (okS64) return kSkinny64;
    if (okS32) return kSkinny32;
    return kGeneric;
}

// The quantizing path: the masked ring kernel when its requirements hold
// (also for Q, scale and ldq) and its 256x256 tiles give at least half the
// compute units a tile, else the bounds-checked kernel.
static int choose_kernel_q8(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                            int64_t ldb, const void *C, int64_t ldc, float beta, const void *Q, int64_t ldq,
                            const void *scale, int cus) {
    if (M == 0 || N == 0) return kNone;
    const void *c_probe = beta != 0.0f ? C : A;  // C is not read when beta == 0
    const int64_t ldc_probe = beta != 0.0f ? ldc : 8;
    const bool ok = ring_masked_ok(M, N, K, A, lda, B, ldb, c_probe, ldc_probe) && aligned16(Q) &&
                    aligned16(scale) && ldq % 8 == 0;
    if (ok) {
        const int64_t tiles = ((M + ShapeRing::BM - 1) / ShapeRing::BM) * ((N + ShapeRing::BN - 1) / ShapeRing::BN);
        const char *force = std::getenv("GEMM_BF16_FORCE_KERNEL");
        const bool forced = force && !std::strcmp(force, kKindNames[kRingQ8]);
        if (tiles * 2 >= cus || forced) return kRingQ8;
    }
    return kGeneric;
}

static hipError_t launch_generic(const GemmArgs &args, int cus, hipStream_t stream) {
    const int64_t tiles_m = (args.M + GenericConfig::BM - 1) / GenericConfig::BM;
    const int64_t tiles_n = (args.N + GenericConfig::BN - 1) / GenericConfig::BN;
    const int64_t tiles = tiles_m * tiles_n;
    const int64_t cap = (int64_t)cus * 8;
    const int grid = (int)(tiles < cap ? tiles : cap);
    hipLaunchKernelGGL(gemm_generic_kernel, dim3(grid), dim3(GenericConfig::kThreads), 0, stream, args, tiles_m,
                       tiles);
    return hipGetLastError();
}

}  // namespace gb

extern "C" {

int gemm_bf16(int64_t M, int64_t N, int64_t K, const gemm_bf16_t *A, int64_t lda, const gemm_bf16_t *B,
              int64_t ldb, gemm_bf16_t *C, int64_t ldc, float alpha, float beta, const gemm_bf16_t *bias,
              int epilogue, hipStream_t stream) {
    using namespace gb;
    const int st = validate(M, N, K, A, lda, B, ldb, C, ldc, epilogue);
    if (st != GEMM_OK) return st;
    if (M == 0 || N == 0) return GEMM_OK;

    GemmArgs args;
    args.M = M;
    args.N = N;
    args.K = K;
    args.A = A;
    args.lda = lda;
    args.B = B;
    args.ldb = ldb;
    args.C = C;
    args.ldc = ldc;
    args.alpha = alpha;
    args.beta = beta;
    args.bias = bias;
    args.flags = epilogue_flags(beta, bias, epilogue);
    args.Q = nullptr;
    args.ldq = 0;
    args.scale = nullptr;
    args.zp = 0.f;

    const int cus = device_cu_count();
    hipError_t err = hipSuccess;
    switch (choose_kernel(M, N, K, A, lda, B, ldb, C, ldc, cus)) {
    case kLarge: err = launch_tile_large(args, cus, stream); break;
    case kMedium: err = launch_tile_medium(args, cus, stream); break;
    case kRing32: err = launch_tile_ring_mfma32(args, cus, stream); break;
    case kRing: err = launch_tile_ring(args, cus, stream); break;
    case kRingMasked: err = launch_tile_ring_masked(args, cus, stream); break;
    case kSkinny64: err = launch_skinny_m64(args, cus, stream); break;
    case kSkinny32: err = launch_skinny_m32(args, cus, stream); break;
    default: err = launch_generic(args, cus, stream); break;
    }
    if (err != hipSuccess) {
        t_last_hip_error = (int)err;
        return GEMM_ERR_HIP;
    }
    return GEMM_OK;
}

int gemm_bf16_q8(int64_t M, int64_t N, int64_t K, const gemm_bf16_t *A, int64_t lda, const gemm_bf16_t *B,
                 int64_t ldb, const gemm_bf16_t *C, int64_t ldc, int8_t *Q, int64_t ldq, float alpha, float beta,
                 const gemm_bf16_t *bias, int epilogue, const float *scale, int32_t zero_point,
                 hipStream_t stream) {
    using namespace gb;
    const int st = validate_q8(M, N, K, A, lda, B, ldb, C, ldc, Q, ldq, beta, scale, epilogue);
    if (st != GEMM_OK) return st;
    if (M == 0 || N == 0) return GEMM_OK;

    GemmArgs args;
    args.M = M;
    args.N = N;
    args.K = K;
    args.A = A;
    args.lda = lda;
    args.B = B;
    args.ldb = ldb;
    args.C = const_cast<gemm_bf16_t *>(C);  // read only (beta != 0); never written on this path
    args.ldc = beta != 0.0f ? ldc : 1;
    args.alpha = alpha;
    args.beta = beta;
    args.bias = bias;
    args.flags = epilogue_flags(beta, bias, epilogue);
    args.Q = Q;
    args.ldq = ldq;
    args.scale = scale;
    args.zp = (float)zero_point;

    const int cus = device_cu_count();
    hipError_t err = hipSuccess;
    if (choose_kernel_q8(M, N, K, A, lda, B, ldb, C, ldc, beta, Q, ldq, scale, cus) == kRingQ8)
        err = launch_tile_ring_q8(args, cus, stream);
    else
        err = launch_generic(args, cus, stream);
    if (err != hipSuccess) {
        t_last_hip_error = (int)err;
        return GEMM_ERR_HIP;
    }
    return GEMM_OK;
}

const char *gemm_bf16_q8_kernel_name(int64_t M, int64_t N, int64_t K, const gemm_bf16_t *A, int64_t lda,
                                     const gemm_bf16_t *B, int64_t ldb, const gemm_bf16_t *C, int64_t ldc,
                                     const int8_t *Q, int64_t ldq, float beta, const float *scale,
                                     int epilogue) {
    if (gb::validate_q8(M, N, K, A, lda, B, ldb, C, ldc, Q, ldq, beta, scale, epilogue) != GEMM_OK) return "none";
    return gb::kind_name(
        gb::choose_kernel_q8(M, N, K, A, lda, B, ldb, C, ldc, beta, Q, ldq, scale, gb::device_cu_count()));
}

const char *gemm_bf16_status_string(int status) {
    switch (status) {
    case GEMM_OK: return "ok";
    case GEMM_ERR_DIM: return "negative dimension";
    case GEMM_ERR_LD: return "leading dimension too small";
    case GEMM_ERR_NULL: return "null pointer for a non-empty operand";
    case GEMM_ERR_EPILOGUE: return "unknown epilogue";
    case GEMM_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

int gemm_bf16_last_hip_error(void) { return gb::t_last_hip_error; }

const char *gemm_bf16_kernel_name(int64_t M, int64_t N, int64_t K, const gemm_bf16_t *A, int64_t lda,
                                  const gemm_bf16_t *B, int64_t ldb, const gemm_bf16_t *C, int64_t ldc,
                                  float beta, const gemm_bf16_t *bias, int epilogue) {
    (void)beta;
    (void)bias;
    if (gb::validate(M, N, K, A, lda, B, ldb, C, ldc, epilogue) != GEMM_OK) return "none";
    return gb::kind_name(gb::choose_kernel(M, N, K, A, lda, B, ldb, C, ldc, gb::device_cu_count()));
}

}  // extern "C"
