// gemm_bf16.hip -- host side of the library: argument validation, kernel
// selection and launch behind the C ABI declared in include/gemm_bf16.h.
#include "gemm_bf16.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "configs.h"
#include "device_common.h"
#include "kernel_generic.h"
#include "kernel_skinny.h"

namespace gb {

enum KernelKind {
    kNone = 0, kLarge, kMedium, kSkinny, kGeneric, kRing32, kRing, kRingMasked, kRingQ8, kFp8Mfma32, kSplitK, kGemv, kSplitKQ8, kFp8Masked, kGemvFp8, kSkinnyFp8, kFp8SplitK, kRingQ8Masked, kSkinnyQ8, kMediumMasked, kSplitKMasked, kFp8SplitKMasked, kFp8, kFp8Mfma16Masked, kRingW8, kFp8Medium, kFp8MediumMasked, kFp8SplitKMedium, kFp8SplitKMediumMasked, kSplitKQ8Masked, kSkinnyT, kSkinnyQ8T, kSkinnyFp8T, kTileQ8, kTileQ8Masked, kNumKinds
};

static const char *const kKindNames[kNumKinds] = {"none",            "tile256x256x32_s5", "tile128x128x64_s4",
                                                  "skinny",          "generic64x64x32",
                                                  "ring256x256x64_mfma32", "ring256x256x64",
                                                  "ring256x256x64_masked", "ring256x256x64_q8",
                                                  "fp8_256x256x128_mfma32", "splitk128x128x64", "gemv",
                                                  "splitk128x128x64_q8", "fp8_256x256x128_masked",
                                                  "gemv_fp8",          "skinny_fp8",
                                                  "splitk_fp8_256x256x128", "ring256x256x64_q8_masked",
                                                  "skinny_q8", "tile128x128x64_s4_masked",
                                                  "splitk128x128x64_masked", "splitk_fp8_256x256x128_masked",
                                                  "fp8_256x256x128", "fp8_256x256x128_mfma16_masked",
                                                  "ring256x256x64_w8", "fp8_128x128x128",
                                                  "fp8_128x128x128_masked", "splitk_fp8_128x128x128",
                                                  "splitk_fp8_128x128x128_masked", "splitk128x128x64_q8_masked",
                                                  "skinny_t", "skinny_q8_t", "skinny_fp8_t",
                                                  "tile128x128x64_q8", "tile128x128x64_q8_masked"};

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

// The masked ring kernel: any M, N >= 1; K, lda and ldb multiples of 8
// (16-byte operand chunks), A and B 16-byte aligned (C: any ldc and
// alignment, accessed element by element unless ldc % 8 == 0 and C is
// aligned), 32-bit buffer offsets within a tile's rows.
static bool ring_masked_ok(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                           int64_t ldb, const void *C, int64_t ldc) {
    (void)C;
    (void)ldc;
    if (M <= 0 || N <= 0 || K <= 0 || K % 8) return false;
    if (lda % 8 || ldb % 8) return false;
    if (!aligned16(A) || !aligned16(B)) return false;
    const int64_t lim = (int64_t)1 << 31;
    if ((ShapeRing::BM * lda + K) * 2 >= lim || (ShapeRing::BN * ldb + K) * 2 >= lim) return false;
    if (K + ShapeRing::BK >= lim) return false;
    const int64_t tiles = ((M + ShapeRing::BM - 1) / ShapeRing::BM) * ((N + ShapeRing::BN - 1) / ShapeRing::BN);
    return tiles < lim;
}

// The masked 128x128 tile kernel: any M, N >= 1; K, lda and ldb multiples
// of 8, A and B 16-byte aligned (C: any ldc and alignment, accessed element
// by element unless ldc % 8 == 0 and C is aligned), 32-bit buffer offsets
// within a tile's rows (K rounded up to a slice).
static bool medium_masked_ok(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                             int64_t ldb, const void *C, int64_t ldc) {
    (void)C;
    (void)ldc;
    if (M <= 0 || N <= 0 || K <= 0 || K % 8) return false;
    if (lda % 8 || ldb % 8) return false;
    if (!aligned16(A) || !aligned16(B)) return false;
    const int64_t lim = (int64_t)1 << 31;
    if ((ShapeM::BM * lda + K + ShapeM::BK) * 2 >= lim || (ShapeM::BN * ldb + K + ShapeM::BK) * 2 >= lim) return false;
    const int64_t tiles = ((M + ShapeM::BM - 1) / ShapeM::BM) * ((N + ShapeM::BN - 1) / ShapeM::BN);
    return tiles < lim / 64;
}

// The streaming kernel for short products: 1 <= M <= 64, K a multiple of 8,
// lda and ldb multiples of 8, A and B 16-byte aligned (C may have any ldc:
// its accesses go element by element unless C is aligned and ldc % 8 == 0),
// 32-bit buffer offsets within a strip's rows (strips are at most 128
// columns).
static bool skinny_path_ok(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                           int64_t ldb, const void *C, int64_t ldc) {
    (void)C;
    (void)ldc;
    if (M <= 0 || M > 64 || N <= 0 || K <= 0 || K % 8) return false;
    if (lda % 8 || ldb % 8) return false;
    if (!aligned16(A) || !aligned16(B)) return false;
    const int64_t lim = (int64_t)1 << 31;
    if ((64 * lda + K + 256) * 2 >= lim || (128 * ldb + K + 256) * 2 >= lim) return false;
    if (N / 32 + 1 >= lim / 64) return false;
    return true;
}

// The matrix-vector kernel: 1 <= M <= 4, K a multiple of 8, lda and ldb
// multiples of 8, A and B 16-byte aligned, 32-bit byte offsets within four
// rows of A and four columns of B (C may have any ldc).
static bool gemv_path_ok(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                         int64_t ldb) {
    if (M <= 0 || M > 4 || N <= 0 || K <= 0 || K % 8) return false;
    if (lda % 8 || ldb % 8) return false;
    if (!aligned16(A) || !aligned16(B)) return false;
    const int64_t lim = (int64_t)1 << 31;
    if ((4 * lda + K) * 2 >= lim || (4 * ldb + K) * 2 >= lim) return false;
    return true;
}

// Split-K scratch.  Every split path stores fp32 partials, and the
// streaming kernel also keeps one uint32 arrival counter per strip; both
// live in one buffer laid out as [counters | partials].  Its size is fixed:
// kScratchCounters counters and kScratchFloatsPerCu floats (one 128x128
// fp32 tile) per compute unit.  The plans below never split further than
// that holds, so no call ever needs more.
constexpr size_t kScratchCounters = 16384;
constexpr size_t kScratchCounterBytes = kScratchCounters * 4;
constexpr size_t kScratchFloatsPerCu = 128 * 128;

// How the streaming kernel covers a short product: its row block (32 or
// 64), strip width, and the K split.
//  * 32-column strips by default.  K is split only when the strips alone
//    would leave more than half of the compute units idle, or exactly half
//    when the split colocates: then up to one unit per compute unit, each
//    split keeping at least 8 K-slices (4 where K is too short for 4 such
//    splits) so the rings have something to overlap: interleaved, cold B,
//    64 x 512 x 16384 takes 15.5 us in 8
//    splits against 18.2 us in 16, 32 x 1024 x 8192 11.3 us in 4 against
//    12.4 us in 8, while 64 x 2048 x 4096 keeps 4 splits of 4 slices
//    (11.9 us; 2 splits 12.7 us).  The split colocates (handoff.h) when
//    the strips are a multiple of 8 and every unit has its own workgroup;
//    else the partials cross XCDs through device-wide atomics.  Colocated
//    against crossing, interleaved in one process (cold B): 64 x 2048 x 4096
//    11.8 against 16.7 us, 64 x 1024 x 16384 18.3 against 21.3 us,
//    64 x 512 x 16384 17.7 against 24.2 us.
//  * Where 32-column strips would leave compute units idle without a split
//    (N from 4096 to 8191 on 256 CUs) and the N / 64 strips of 64 columns
//    are a multiple of 8, bf16 products take 64-column strips with K split
//    (at least 8 slices of 256) so that the units fill the CUs, colocated:
//    64 x 4096 x 8192 21.1 against 28.6 us, 64 x 6144 x 8192 27.1 against
//    29.3 us, 32 x 4096 x 8192 19.2 against 22.4 us.  Where the 32-column
//    strips split or fill the CUs, 64-column strips are slower (their rings
//    keep fewer B slices in flight): 64 x 8192 x 8192 unsplit 39.1 against
//    29.2 us, split in two 35.2 us.
// cap_floats bounds the partials (strips x splits x rows x columns floats)
// and the strips must fit the counters (records, when colocated).
struct SkinnyPlan {
    int rows, cols, strips, splits, spp, colocate;
};

static SkinnyPlan plan_skinny_width(int64_t M, int64_t N, int64_t K, int cus, size_t cap_floats, bool fp8,
                                    int width, int coloc_ok) {
    SkinnyPlan p{};
    p.rows = M <= 32 ? 32 : 64;
    p.cols = width;
    const int ks = fp8 ? ShapeSkinny::KS_FP8
                       : (width == 32 ? ShapeSkinny::KS_N32 : width == 64 ? ShapeSkinny::KS_N64 : ShapeSkinny::KS_N128);
    const int64_t nk = (K + ks - 1) / ks;
    const int64_t strips = (N + width - 1) / width;
    p.strips = (int)strips;
    // 32-column strips filling exactly half of the compute units split in
    // two when the halves colocate and keep 8 slices each: int8 output
    // 64 x 4096 x 8192 21.1 against 28.7 us unsplit, FP8 64 x 4096 x 16384
    // 20.1 against 25.1 us (FP8 32 x 4096 x 4096, 4 slices a half: 9.6
    // against 8.5 us, so it stays whole).
    const bool split = width == 64 ? strips * 2 <= cus
                                   : strips * 2 < cus ||
                                         (strips * 2 == cus && coloc_ok && strips % kNumXcds == 0 && nk >= 16);
    int64_t splits = split ? cus / strips : 1;
    if (const char *env = std::getenv("GEMM_BF16_SKINNY_SPLITS")) {  // tuning knob
        const int s = std::atoi(env);
        if (s >= 1) splits = s;
    }
    // At least 8 K-slices per split, so the rings (3 and 4 slices deep) have
    // a loop to overlap, or 4 where K is too short for 4 such splits.
    int64_t max_splits = nk / 8;
    if (max_splits < 4) max_splits = nk / 4 < 4 ? nk / 4 : 4;
    if (max_splits < 1) max_splits = 1;
    if (splits > max_splits) splits = max_splits;
    const int64_t per_split = strips * (int64_t)p.cols * p.rows;
    if (splits > 1 && (strips > (int64_t)kScratchCounters || splits * per_split > (int64_t)cap_floats))
        splits = strips > (int64_t)kScratchCounters ? 1 : (int64_t)cap_floats / per_split;
    if (splits < 1) splits = 1;
    p.spp = (int)((nk + splits - 1) / splits);
    p.splits = (int)((nk + p.spp - 1) / p.spp);  // no empty split
    const bool coloc = coloc_ok && p.splits > 1 && p.splits < 256 && strips % kNumXcds == 0 &&
                       strips * p.splits <= cus && (size_t)strips * sizeof(HandoffRecord) <= kScratchCounterBytes;
    p.colocate = coloc ? coloc_ok : 0;
    return p;
}

static SkinnyPlan plan_skinny(int64_t M, int64_t N, int64_t K, int cus, size_t cap_floats, bool fp8 = false,
                              bool q8 = false) {
    int coloc_ok = 1;
    if (const char *env = std::getenv("GEMM_BF16_SKINNY_COLOCATE")) {
        // tuning knob: 0 = partials cross XCDs; testing knob: "fence" = colocated, always the fenced path
        if (env[0] == '0') coloc_ok = 0;
        if (!std::strcmp(env, "fence")) coloc_ok = 2;
    }
    if (fp8 || q8)  // the FP8 and int8-output instances are built for 32-column strips
        return plan_skinny_width(M, N, K, cus, cap_floats, fp8, 32, coloc_ok);
    if (const char *env = std::getenv("GEMM_BF16_SKINNY_COLS")) {  // tuning knob: 32, 64 or 128
        const int w = std::atoi(env);
        if (w == 32 || w == 64 || w == 128) return plan_skinny_width(M, N, K, cus, cap_floats, false, w, coloc_ok);
    }
    const int64_t strips32 = (N + 31) / 32, strips64 = (N + 63) / 64;
    if (coloc_ok && strips32 < cus && strips32 * 2 >= cus && strips64 % kNumXcds == 0 && strips64 * 2 <= cus) {
        const SkinnyPlan p = plan_skinny_width(M, N, K, cus, cap_floats, false, 64, coloc_ok);
        if (p.colocate) return p;
    }
    return plan_skinny_width(M, N, K, cus, cap_floats, false, 32, coloc_ok);
}

// Where a call's split-K scratch comes from.
//  * gemm_bf16 and the other allocating entry points: one buffer per
//    (device, stream), allocated by the first call on that stream that
//    splits, at its fixed size (counters + CUs x 64 KiB), with the counters
//    zeroed by a fill kernel on that stream; it is never grown, freed or
//    synchronized on afterwards and lives until the process ends.  Calls on
//    one stream are ordered, so they share it safely; calls on other streams
//    get their own.  (A stream handle that is destroyed and handed out again
//    by the runtime finds the old buffer: work on the destroyed stream must
//    have finished by then, as for any memory it used.)
//  * gemm_bf16_noalloc: the library's static device array (below), shared
//    by every such call on the device.
struct Scratch {
    char *fixed = nullptr;   // the static array's device address (no-allocation entry point)
    size_t cap_floats = 0;   // partial floats the buffer holds
};

static std::mutex g_ws_mutex;  // guards g_ws (a lookup, or one allocation per (device, stream))
static std::map<std::pair<int, hipStream_t>, char *> g_ws;

__global__ void zero_u32_kernel(uint32_t *p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

static hipError_t zero_counters(uint32_t *cnt, hipStream_t stream) {
    const int n = (int)kScratchCounters;
    hipLaunchKernelGGL(zero_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, cnt, n);
    return hipGetLastError();
}

static Scratch stream_scratch(int cus) {
    Scratch s;
    s.cap_floats = (size_t)cus * kScratchFloatsPerCu;
    return s;
}

static hipError_t get_scratch(const Scratch &src, hipStream_t stream, uint32_t **cnt, float **partials) {
    char *base = src.fixed;
    if (base == nullptr) {
        int dev = 0;
        hipError_t err = hipGetDevice(&dev);
        if (err != hipSuccess) return err;
        std::lock_guard<std::mutex> lock(g_ws_mutex);
        auto it = g_ws.find(std::make_pair(dev, stream));
        if (it != g_ws.end()) {
            base = it->second;
        } else {
            if ((err = hipMalloc(&base, kScratchCounterBytes + src.cap_floats * 4)) != hipSuccess) return err;
            if ((err = zero_counters(reinterpret_cast<uint32_t *>(base), stream)) != hipSuccess) {
                (void)hipFree(base);
                return err;
            }
            g_ws.emplace(std::make_pair(dev, stream), base);
        }
    }
    *cnt = reinterpret_cast<uint32_t *>(base);
    *partials = reinterpret_cast<float *>(base + kScratchCounterBytes);
    return hipSuccess;
}

// The transposed product C' = C^T for the streaming kernel's transposed
// output: M' = N, N' = M, A' = B^T (row-major, lda' = ldb), B' = A^T
// (column-major, ldb' = lda), the FP8 scales swapped (scale_a' indexes the
// rows of C', i.e. C's columns).  C, Q, bias and the int8 scales keep C's
// indexing; the kernel writes C' (and Q') back transposed.
static GemmArgs transposed(const GemmArgs &args) {
    GemmArgs t = args;
    t.M = args.N;
    t.N = args.M;
    t.A = args.B;
    t.lda = args.ldb;
    t.B = args.A;
    t.ldb = args.lda;
    t.scale_a = args.scale_b;
    t.scale_b = args.scale_a;
    return t;
}

static hipError_t launch_skinny_plan(const GemmArgs &args, int cus, const Scratch &scr, hipStream_t stream,
                                     bool fp8 = false, bool q8 = false, bool trans = false) {
    const SkinnyPlan p = plan_skinny(args.M, args.N, args.K, cus, scr.cap_floats, fp8, q8);
    SkinnyWork work{};
    work.num_strips = p.strips;
    work.splits = p.splits;
    work.spp = p.spp;
    work.c_vector = aligned16(args.C) && args.ldc % 8 == 0;
    work.q_vector = q8 && (reinterpret_cast<uintptr_t>(args.Q) & 7u) == 0 && args.ldq % 8 == 0;
    work.colocate = p.colocate;
    if (p.splits > 1) {
        const size_t floats = (size_t)p.strips * p.splits * p.cols * p.rows;
        if (floats > scr.cap_floats || (size_t)p.strips > kScratchCounters) return hipErrorInvalidValue;
        hipError_t err = get_scratch(scr, stream, &work.counters, &work.partials);
        if (err != hipSuccess) return err;
        work.records = reinterpret_cast<HandoffRecord *>(work.counters);
    }
    if (q8)
        return trans ? launch_skinny_q8_t(p.rows, args, work, cus, stream)
                     : launch_skinny_q8(p.rows, args, work, cus, stream);
    if (fp8)
        return trans ? launch_skinny_fp8_t(p.rows, args, work, cus, stream)
                     : launch_skinny_fp8(p.rows, args, work, cus, stream);
    return trans ? launch_skinny_t(p.rows, p.cols, args, work, cus, stream)
                 : launch_skinny(p.rows, p.cols, args, work, cus, stream);
}

// Split-K on the 128x128 tiles: used when those tiles alone would leave more
// than half of the compute units idle.  The K-slices (64 wide) are cut into
// ranges of at least kMinSlices slices each, so every range still runs a
// pipelined loop, and at most CUs / tiles of them.  How many: a split trades
// each unit's K loop (slices / splits) against the fp32 partials written and
// read back (splits x tiles whole tiles), and the count that balances the
// two is close to 3 sqrt(slices / tiles); it is raised to the count that
// gives at least half of the compute units a unit.  Measured interleaved in
// one process (the count that fills every compute unit in parentheses):
// 1024 x 1024 x 4096 3 ranges 18.8 us (4: 19.5 us; 24.2 against 20.6 us on
// a slower box), 1024 x 512 x 4096 4 ranges 15.7 us (8: 18.1 us),
// 512 x 512 x 8192 8 ranges 16.7 us (16: 18.4 us), 768 x 768 x 4096 4 ranges
// 18.1 us (7: 18.2 us; 3 ranges 17.3 us), 512 x 512 x 4096 8 ranges 12.9 us
// (the square-root rule alone would take 6, 13.7 us).  Partials take
// splits x (M x N padded to tiles) floats of scratch (at most CUs x 16K
// floats: splits * tiles <= CUs and a tile is 16K elements; forced split
// counts are capped by cap_floats).  Returns 1 when no split applies.
constexpr int kSplitMinSlices = 8;

// Shape: the 128x128 tiles' K-slice (ShapeM, 64 bf16 values; ShapeFp8M, 128
// FP8 values: the same 128-byte rows and MFMA time per slice).
template <class Shape = ShapeM>
static TileSplit plan_splitk(int64_t M, int64_t N, int64_t K, int cus, size_t cap_floats) {
    TileSplit p{};
    p.splits = 1;
    // tiles and slices rounded up: shapes with tails run the masked kernel
    const int64_t tiles = ((M + Shape::BM - 1) / Shape::BM) * ((N + Shape::BN - 1) / Shape::BN);
    const int64_t nk = (K + Shape::BK - 1) / Shape::BK;
    if (tiles <= 0 || tiles * 2 >= cus) return p;
    int64_t splits = std::llround(3.0 * std::sqrt((double)nk / (double)tiles));
    const int64_t half = (cus / 2 + tiles - 1) / tiles;
    if (splits < half) splits = half;
    if (splits > cus / tiles) splits = cus / tiles;
    if (const char *env = std::getenv("GEMM_BF16_SPLITK_SPLITS")) {  // tuning knob
        const int v = std::atoi(env);
        if (v >= 1) splits = v;
    }
    const int64_t max_splits = nk / kSplitMinSlices;
    if (splits > max_splits) splits = max_splits;
    // whole tiles are stored: the scratch is padded to tile multiples
    const int64_t ldp = (M + Shape::BM - 1) / Shape::BM * Shape::BM;
    const int64_t pstride = ldp * ((N + Shape::BN - 1) / Shape::BN * Shape::BN);
    if (splits > (int64_t)cap_floats / pstride) splits = (int64_t)cap_floats / pstride;
    if (splits < 2) return p;
    p.kper = (int)((nk + splits - 1) / splits);
    p.splits = (int)((nk + p.kper - 1) / p.kper);  // no empty range
    p.ldp = ldp;
    p.pstride = pstride;
    // A tile's ranges on one XCD when every unit has its own workgroup and
    // each XCD's share of them is whole tiles: the reduction then reads a
    // tile's partials on the XCD that wrote them.
    p.tile_major = tiles * p.splits <= cus && tiles % kNumXcds == 0;
    if (const char *env = std::getenv("GEMM_BF16_SPLITK_COLOCATE")) {  // tuning knob: 0 = range-major units
        if (env[0] == '0') p.tile_major = 0;
    }
    return p;
}

// Whether splitting K beats the unsplit 128x128 kernel on a small grid.
// Measured: the unsplit kernel takes about 4.3 us plus 0.31 us per 64-wide
// K-slice whatever the tile count (up to 64 tiles), while the split pays a
// reduction kernel and runs more, busier compute units; with the range
// counts of plan_splitk it wins from about 26 slices at 16 tiles, 32 at 32
// tiles and 45 at 64 tiles (interleaved: 1024 x 512 x 2048 12.7 us split
// against 14.6 us unsplit, FP8 1024 x 512 x 4096 13.1 against 15.5 us;
// 1024 x 1024 x 2048 14.9 against 14.8 us; 768 x 768 x 2048, 36 tiles,
// 15.9 against 14.6 us; 1024 x 1024 x 4096 20.1 against 25.6 us).  The
// quantizing output has no unsplit small-grid kernel and splits whenever
// the plan allows.
template <class Shape>
static bool splitk_pays_t(int64_t M, int64_t N, int64_t K) {
    const int64_t tiles = ((M + Shape::BM - 1) / Shape::BM) * ((N + Shape::BN - 1) / Shape::BN);
    const int64_t nk = (K + Shape::BK - 1) / Shape::BK;
    return 5 * nk >= 96 + 2 * tiles;
}
static bool splitk_pays(int64_t M, int64_t N, int64_t K) { return splitk_pays_t<ShapeM>(M, N, K); }

// Split-K over the 256x256 FP8 tiles, reached by GEMM_BF16_FORCE_KERNEL
// only (on the small grids where it applies the 128x128 tiles are faster):
// when those tiles fill less than half of the compute units, up to CUs /
// tiles ranges of at least 4 slices of 128, at most 8, and at most
// cap_floats floats of partials.  Returns 1 when no split applies.
static TileSplit plan_splitk_fp8(int64_t M, int64_t N, int64_t K, int cus, size_t cap_floats) {
    TileSplit p{};
    p.splits = 1;
    // tiles and slices rounded up (shapes with tails run the masked kernel,
    // whose partials are whole tiles in a padded workspace)
    const int64_t mp = (M + ShapeFp8::BM - 1) / ShapeFp8::BM * ShapeFp8::BM;
    const int64_t np = (N + ShapeFp8::BN - 1) / ShapeFp8::BN * ShapeFp8::BN;
    const int64_t tiles = (mp / ShapeFp8::BM) * (np / ShapeFp8::BN);
    const int64_t nk = (K + ShapeFp8::BK - 1) / ShapeFp8::BK;
    if (tiles <= 0 || tiles * 2 >= cus) return p;
    int64_t splits = cus / tiles;
    if (const char *env = std::getenv("GEMM_BF16_FP8_SPLITS")) {  // tuning knob
        const int v = std::atoi(env);
        if (v >= 1) splits = v;
    }
    if (splits > nk / 4) splits = nk / 4;
    if (splits > 8) splits = 8;
    const int64_t cap = (int64_t)cap_floats / (mp * np);
    if (splits > cap) splits = cap;
    if (splits < 2) return p;
    p.kper = (int)((nk + splits - 1) / splits);
    p.splits = (int)((nk + p.kper - 1) / p.kper);  // no empty range
    p.ldp = mp;
    p.pstride = mp * np;
    return p;
}

static hipError_t launch_fp8_splitk_plan(const GemmArgs &args, int cus, const Scratch &scr, hipStream_t stream,
                                         bool masked) {
    TileSplit p = plan_splitk_fp8(args.M, args.N, args.K, cus, scr.cap_floats);
    if (p.splits < 2) return masked ? launch_tile_fp8_mfma32_masked(args, cus, stream) : launch_tile_fp8(args, cus, stream);
    if ((size_t)p.splits * (size_t)p.pstride > scr.cap_floats) return hipErrorInvalidValue;
    uint32_t *unused = nullptr;
    hipError_t err = get_scratch(scr, stream, &unused, &p.P);
    if (err != hipSuccess) return err;
    return masked ? launch_tile_fp8_splitk_masked(args, p, cus, stream) : launch_tile_fp8_splitk(args, p, cus, stream);
}

// FP8 split-K on the 128x128 tiles (unsplit when the plan does not split).
static hipError_t launch_fp8_medium_splitk_plan(const GemmArgs &args, int cus, const Scratch &scr,
                                                hipStream_t stream, bool masked) {
    TileSplit p = plan_splitk<ShapeFp8M>(args.M, args.N, args.K, cus, scr.cap_floats);
    if (p.splits < 2)
        return masked ? launch_tile_fp8_medium_masked(args, cus, stream) : launch_tile_fp8_medium(args, cus, stream);
    if ((size_t)p.splits * (size_t)p.pstride > scr.cap_floats) return hipErrorInvalidValue;
    uint32_t *unused = nullptr;
    hipError_t err = get_scratch(scr, stream, &unused, &p.P);
    if (err != hipSuccess) return err;
    return masked ? launch_tile_fp8_medium_splitk_masked(args, p, cus, stream)
                  : launch_tile_fp8_medium_splitk(args, p, cus, stream);
}

// kQ8: the quantizing output (the host chose this path only when the plan
// splits).
static hipError_t launch_splitk_plan(const GemmArgs &args, int cus, const Scratch &scr, hipStream_t stream,
                                     bool q8 = false, bool masked = false) {
    TileSplit p = plan_splitk(args.M, args.N, args.K, cus, scr.cap_floats);
    if (p.splits < 2) {
        if (q8) return hipErrorInvalidValue;
        return masked ? launch_tile_medium_masked(args, cus, stream) : launch_tile_medium(args, cus, stream);
    }
    if ((size_t)p.splits * (size_t)p.pstride > scr.cap_floats) return hipErrorInvalidValue;
    uint32_t *unused = nullptr;
    hipError_t err = get_scratch(scr, stream, &unused, &p.P);
    if (err != hipSuccess) return err;
    if (q8) return masked ? launch_tile_medium_splitk_q8_masked(args, p, cus, stream)
                          : launch_tile_medium_splitk_q8(args, p, cus, stream);
    return masked ? launch_tile_medium_splitk_masked(args, p, cus, stream)
                  : launch_tile_medium_splitk(args, p, cus, stream);
}

// The int8 output on 128x128 tiles over the whole of K: the split kernels
// with a single K range -- the tile kernel stores each tile's fp32 sum to
// the workspace and the ordered reduction kernel runs the epilogue and
// quantizes (the unsplit tile kernel's epilogue writes bf16 only).  The
// workspace holds M x N floats rounded up to whole tiles.
static TileSplit plan_tile_q8(int64_t M, int64_t N, int64_t K) {
    TileSplit p{};
    p.splits = 1;
    p.kper = (int)((K + ShapeM::BK - 1) / ShapeM::BK);
    p.ldp = (M + ShapeM::BM - 1) / ShapeM::BM * ShapeM::BM;
    p.pstride = p.ldp * ((N + ShapeM::BN - 1) / ShapeM::BN * ShapeM::BN);
    p.tile_major = 0;
    return p;
}

static hipError_t launch_tile_q8_plan(const GemmArgs &args, int cus, const Scratch &scr, hipStream_t stream,
                                      bool masked) {
    TileSplit p = plan_tile_q8(args.M, args.N, args.K);
    if ((size_t)p.pstride > scr.cap_floats) return hipErrorInvalidValue;
    uint32_t *unused = nullptr;
    hipError_t err = get_scratch(scr, stream, &unused, &p.P);
    if (err != hipSuccess) return err;
    return masked ? launch_tile_medium_splitk_q8_masked(args, p, cus, stream)
                  : launch_tile_medium_splitk_q8(args, p, cus, stream);
}

// Kernel for a shape.  GEMM_BF16_FORCE_KERNEL=<name> (a kKindNames entry)
// overrides the choice when that kernel can run the shape; it exists for
// testing and benchmarking the alternatives.
static int choose_kernel(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                         int64_t ldb, const void *C, int64_t ldc, int cus, size_t cap_floats) {
    if (M == 0 || N == 0) return kNone;
    const bool okL = tile_path_ok<ShapeL>(M, N, K, A, lda, B, ldb, C, ldc);
    const bool okM = tile_path_ok<ShapeM>(M, N, K, A, lda, B, ldb, C, ldc);
    const bool okR = tile_path_ok<ShapeRing>(M, N, K, A, lda, B, ldb, C, ldc);
    const bool okRM = ring_masked_ok(M, N, K, A, lda, B, ldb, C, ldc);
    const bool okS = skinny_path_ok(M, N, K, A, lda, B, ldb, C, ldc);
    // the transposed product (N' = M, M' = N <= 64, A' = B^T, B' = A^T)
    const bool okST = skinny_path_ok(N, M, K, B, ldb, A, lda, C, ldc);
    const bool okV = gemv_path_ok(M, N, K, A, lda, B, ldb);
    const bool okMM = medium_masked_ok(M, N, K, A, lda, B, ldb, C, ldc);
    if (const char *force = std::getenv("GEMM_BF16_FORCE_KERNEL")) {
        if (!std::strcmp(force, kKindNames[kMediumMasked]) && okMM) return kMediumMasked;
        if (!std::strcmp(force, kKindNames[kSplitKMasked]) && okMM && plan_splitk(M, N, K, cus, cap_floats).splits >= 2)
            return kSplitKMasked;
        if (!std::strcmp(force, kKindNames[kGeneric])) return kGeneric;
        if (!std::strcmp(force, kKindNames[kLarge]) && okL) return kLarge;
        if (!std::strcmp(force, kKindNames[kMedium]) && okM) return kMedium;
        if (!std::strcmp(force, kKindNames[kSplitK]) && okM && plan_splitk(M, N, K, cus, cap_floats).splits >= 2)
            return kSplitK;
        if (!std::strcmp(force, kKindNames[kRing32]) && okR) return kRing32;
        if (!std::strcmp(force, kKindNames[kRing]) && okR) return kRing;
        if (!std::strcmp(force, kKindNames[kRingW8]) && okR) return kRingW8;
        if (!std::strcmp(force, kKindNames[kRingMasked]) && okRM) return kRingMasked;
        if (!std::strcmp(force, kKindNames[kSkinny]) && okS) return kSkinny;
        if (!std::strcmp(force, kKindNames[kSkinnyT]) && okST) return kSkinnyT;
        if (!std::strcmp(force, kKindNames[kGemv]) && okV) return kGemv;
    }
    // One to four rows: the matrix-vector kernel.  Each of its waves reads
    // every row of A for two columns of B, so at three and four rows on a
    // large B (N * K >= 2^26) the streaming kernel, which shares A across a
    // 32-column strip, is faster (8192 x 8192: 25.0 us against 27.8 us at
    // three rows and 29.2 us at four).
    // Where the streaming kernel's 32-column strips outnumber the compute
    // units, each unit fills and drains its rings: then the matrix-vector
    // kernel keeps three and four rows unless K is long (3 x 65536 x 2048:
    // 45.9 us against 57.2 us streaming, 4 x 32768 x 4096 49.0 against
    // 51.1 us; 4 x 16384 x 8192 52.3 against 47.8 us).
    const bool many_strips = (N + 31) / 32 > cus;
    if (okV && (M <= 2 || N * K < ((int64_t)1 << 26) || !okS || (many_strips && K >= 2048 && K < 8192)))
        return kGemv;
    // At most 64 rows: the streaming kernel (a 256-row tile would be mostly
    // empty) -- except with more strips than compute units over a short K
    // (fewer than 8 slices of 256), where the masked 128x128 tiles, which
    // overlap one another's loads, are faster (64 x 65536 x 512: 19.1 us
    // against 29.7 us, 28.6 us on the 256x256 ring; 4 x 65536 x 1024 30.8
    // against 39.2 us, 35.1 us on the matrix-vector kernel).
    if (okS) return (!many_strips || K >= 2048 || !okMM) ? kSkinny : kMediumMasked;
    // At most 64 columns: the streaming kernel on the transposed product,
    // writing C transposed (A, row-major, is then the streamed operand),
    // with the same exception over M's strips.
    if (okST) return ((M + 31) / 32 <= cus || K >= 2048 || !okMM) ? kSkinnyT : kMediumMasked;
    // 256x256 tiles when they give at least half the compute units a tile:
    // exact multiples take the unmasked ring kernel, shapes with tails the
    // masked one.
    // Exactly half: the 128x128 kernel gives every compute unit two tiles,
    // where the ring leaves half of them idle (2048 x 4096 x 4096: 66 us
    // against 72 us; from 144 ring tiles up the ring is faster, 72.9 us
    // against 93.7 us at 3072 x 3072 x 4096, when 128x128 tiles need a
    // third round).  The same with tails, masked: 2000 x 4000 x 4000 71.2
    // against 78.3 us, 2000 x 4000 x 2000 43.9 against 47.8 us; at 144 ring
    // tiles (2100 x 4000 x 4096) the masked ring, 85.8 against 99.9 us.
    // Just over one round (more ring tiles than compute units, at most 5/4
    // as many), the ring's second round leaves most compute units idle and
    // the 128x128 tiles balance better: 4096 x 4608 x 4096 (288 ring tiles)
    // 153.6 against 162.1 us, 5120 x 4096 x 4096 (320) 158.2 against
    // 177.0 us, 4096 x 4608 x 1024 46.2 against 51.2 us; from 352 ring tiles
    // (4096 x 5632 x 4096, 176.2 against 183.1 us) the ring is faster.  With
    // tails the masked ring stays faster (4000 x 4500 x 4000 173.4 against
    // 178.4 us).
    if (okRM) {
        const int64_t tiles = ((M + ShapeRing::BM - 1) / ShapeRing::BM) * ((N + ShapeRing::BN - 1) / ShapeRing::BN);
        if (tiles * 2 == cus && okM) return kMedium;
        if (tiles * 2 == cus && okMM) return kMediumMasked;
        if (tiles > cus && tiles * 4 <= (int64_t)cus * 5 && okM) return kMedium;
        if (tiles * 2 >= cus || (!okM && okR)) return okR ? kRing : kRingMasked;
    }
    if (okL) {
        const int64_t tiles = (M / ShapeL::BM) * (N / ShapeL::BN);
        if (tiles * 2 >= cus || !okM) return kLarge;
    }
    if (okM) return plan_splitk(M, N, K, cus, cap_floats).splits >= 2 && splitk_pays(M, N, K) ? kSplitK : kMedium;
    // Tails on small and mid-sized grids (and unaligned C or ldc % 8 != 0):
    // the masked 128x128 kernel, split by the same rule.  1000 x 1000 x 1000
    // runs in 11.5 us (1024^3 unmasked: 9.6 us; the bounds-checked kernel
    // 18.4 us), 1000 x 1000 x 4096 split in 21.8 us (bounds-checked 67 us).
    if (okMM) return plan_splitk(M, N, K, cus, cap_floats).splits >= 2 && splitk_pays(M, N, K) ? kSplitKMasked : kMediumMasked;
    return kGeneric;
}

// The quantizing path: the masked ring kernel when its requirements hold
// (also for Q, scale and ldq) and its 256x256 tiles give at least half the
// compute units a tile; on smaller grids split-K on 128x128 tiles when the
// shape allows it (its reduction quantizes), else whole-K 128x128 tiles
// through the same reduction when the workspace holds every tile; else the
// ring with idle compute units or the bounds-checked kernel.
static int choose_kernel_q8(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                            int64_t ldb, const void *C, int64_t ldc, float beta, const void *Q, int64_t ldq,
                            const void *scale, int cus, size_t cap_floats) {
    if (M == 0 || N == 0) return kNone;
    // At most 64 rows: the streaming kernel with the int8 epilogue (any ldc
    // and ldq; 8-row chunks of Q go out as one store when Q allows it).
    {
        const char *force = std::getenv("GEMM_BF16_FORCE_KERNEL");
        const bool forced_other = force && (!std::strcmp(force, kKindNames[kGeneric]) ||
                                            !std::strcmp(force, kKindNames[kRingQ8]) ||
                                            !std::strcmp(force, kKindNames[kRingQ8Masked]));
        if (!forced_other && skinny_path_ok(M, N, K, A, lda, B, ldb, C, ldc)) return kSkinnyQ8;
        if (force && !std::strcmp(force, kKindNames[kGeneric])) return kGeneric;
        // At most 64 columns: the same on the transposed product (Q and C
        // transposed back), except, as for bf16, where its strips outnumber
        // the compute units over fewer than 8 slices of 256.
        const bool okST = skinny_path_ok(N, M, K, B, ldb, A, lda, C, ldc);
        if (force && !std::strcmp(force, kKindNames[kSkinnyQ8T]) && okST) return kSkinnyQ8T;
        if (!forced_other && okST && ((M + 31) / 32 <= cus || K >= 2048)) return kSkinnyQ8T;
    }
    const void *c_probe = beta != 0.0f ? C : A;  // C is not read when beta == 0
    const int64_t ldc_probe = beta != 0.0f ? ldc : 8;
    const bool ok = ring_masked_ok(M, N, K, A, lda, B, ldb, c_probe, ldc_probe) && aligned16(Q) &&
                    aligned16(scale) && ldq % 8 == 0;
    if (ok) {
        const int64_t tiles = ((M + ShapeRing::BM - 1) / ShapeRing::BM) * ((N + ShapeRing::BN - 1) / ShapeRing::BN);
        const char *force = std::getenv("GEMM_BF16_FORCE_KERNEL");
        // exact tile multiples take the unmasked instance (8192 x 14336 x
        // 4096: 670 us against 717 us masked)
        // (the unmasked instance reads C0 in 16-byte runs when beta != 0)
        const bool exact = M % ShapeRing::BM == 0 && N % ShapeRing::BN == 0 && K % ShapeRing::BK == 0 &&
                           (beta == 0.0f || (aligned16(C) && ldc % 8 == 0));
        if (force && !std::strcmp(force, kKindNames[kRingQ8Masked])) return kRingQ8Masked;
        const bool forced = force && !std::strcmp(force, kKindNames[kRingQ8]);
        if (tiles * 2 >= cus || forced) return exact ? kRingQ8 : kRingQ8Masked;
        const bool can_split = plan_splitk(M, N, K, cus, cap_floats).splits >= 2;
        if (tile_path_ok<ShapeM>(M, N, K, A, lda, B, ldb, c_probe, ldc_probe) && can_split) return kSplitKQ8;
        // with tails: the masked split (1000 x 1000 x 4096 in 20.3 us against
        // 66.0 us on the bounds-checked kernel, 504 x 504 x 8192 18.1 against
        // 125.2 us, 1000 x 1000 x 1000 13.3 against 20.4 us)
        if (medium_masked_ok(M, N, K, A, lda, B, ldb, c_probe, ldc_probe) && can_split) return kSplitKQ8Masked;
        // whole K on 128x128 tiles, the workspace holding every tile
        const bool fits = (size_t)plan_tile_q8(M, N, K).pstride <= cap_floats;
        const bool exact128 = tile_path_ok<ShapeM>(M, N, K, A, lda, B, ldb, c_probe, ldc_probe);
        const bool masked128 = medium_masked_ok(M, N, K, A, lda, B, ldb, c_probe, ldc_probe);
        if (force && !std::strcmp(force, kKindNames[kTileQ8]) && fits && exact128) return kTileQ8;
        if (force && !std::strcmp(force, kKindNames[kTileQ8Masked]) && fits && masked128) return kTileQ8Masked;
        // From 8 slices of K the fp32 round trip pays for itself against the
        // ring with idle compute units or the bounds-checked kernel (2048 x
        // 2048 x 4096: 47.8 us against 82.2 us on the ring; 2048 x 1024 x
        // 4096 42.8 against 87.2 us generic; 1504 x 1504 x 320, masked, 16.6
        // against 27.8 us); at 4 slices it does not (2048 x 2048 x 256: 20.6
        // against 18.3 us on the ring).
        if (fits && K >= 8 * ShapeM::BK && force == nullptr) {
            if (exact128) return kTileQ8;
            if (masked128) return kTileQ8Masked;
        }
        // Grids too large to split on 128x128 tiles and too small to fill
        // half of the compute units with ring tiles: from more than an
        // eighth of the compute units in ring tiles the ring, with idle
        // compute units, beats the bounds-checked kernel (2048 x 2048 x 4096,
        // 64 ring tiles: 76.7 against 95.7 us; 3072 x 2048 x 4096 79.8
        // against 121.4 us; 1536 x 1536 x 4096, 36 tiles, 76.2 against
        // 82.5 us); at 32 ring tiles or fewer it does not (2048 x 1024 x 4096
        // 76.5 against 74.9 us, 1000 x 1000 x 4096 84.5 against 67.4 us).
        if (tiles * 8 > cus && force == nullptr) return exact ? kRingQ8 : kRingQ8Masked;
    }
    return kGeneric;
}

static hipError_t launch_generic(const GemmArgs &args, int cus, hipStream_t stream, bool fp8 = false) {
    const int64_t tiles_m = (args.M + GenericConfig::BM - 1) / GenericConfig::BM;
    const int64_t tiles_n = (args.N + GenericConfig::BN - 1) / GenericConfig::BN;
    const int64_t tiles = tiles_m * tiles_n;
    const int64_t cap = (int64_t)cus * 8;
    const int grid = (int)(tiles < cap ? tiles : cap);
    if (fp8)
        hipLaunchKernelGGL(gemm_generic_kernel<true>, dim3(grid), dim3(GenericConfig::kThreads), 0, stream, args,
                           tiles_m, tiles);
    else
        hipLaunchKernelGGL(gemm_generic_kernel<false>, dim3(grid), dim3(GenericConfig::kThreads), 0, stream, args,
                           tiles_m, tiles);
    return hipGetLastError();
}

// The fp8 product: one to four rows on the matrix-vector kernel, up to 64
// on the streaming kernel; else, with 16-byte aligned rows (lda, ldb % 16,
// K % 16), the 256x256 FP8 tile kernel, or the 128x128 one (whole K or
// split) where the 256x256 tiles would fill less than half of the compute
// units -- each unmasked for exact tile multiples (and ldc % 8, aligned C),
// masked for anything else; else the bounds-checked kernel (which converts
// the bytes to bf16 on their way into LDS).
static int choose_kernel_fp8(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                             int64_t ldb, const void *C, int64_t ldc, int cus, size_t cap_floats) {
    if (M == 0 || N == 0) return kNone;
    const char *force = std::getenv("GEMM_BF16_FORCE_KERNEL");
    if (force && !std::strcmp(force, kKindNames[kGeneric])) return kGeneric;
    // One to four rows: the matrix-vector kernel (16-byte chunks of 16 values).
    const int64_t lim = (int64_t)1 << 31;
    const bool okV = M <= 4 && K > 0 && K % 16 == 0 && lda % 16 == 0 && ldb % 16 == 0 && aligned16(A) &&
                     aligned16(B) && 4 * lda + K < lim && 4 * ldb + K < lim;
    // Up to 64 rows: the streaming kernel (slices of 512 bytes; C any ldc).
    const bool okS = M <= 64 && K > 0 && K % 16 == 0 && lda % 16 == 0 && ldb % 16 == 0 && aligned16(A) &&
                     aligned16(B) && 64 * lda + K + ShapeSkinny::KS_FP8 < lim &&
                     128 * ldb + K + ShapeSkinny::KS_FP8 < lim && N / 32 + 1 < lim / 64;
    if (force && !std::strcmp(force, kKindNames[kSkinnyFp8]) && okS) return kSkinnyFp8;
    // Up to 64 columns (more than 64 rows): the same on the transposed
    // product, B's columns as its rows.
    const bool okST = M > 64 && N <= 64 && K > 0 && K % 16 == 0 && lda % 16 == 0 && ldb % 16 == 0 &&
                      aligned16(A) && aligned16(B) && 64 * ldb + K + ShapeSkinny::KS_FP8 < lim &&
                      128 * lda + K + ShapeSkinny::KS_FP8 < lim && M / 32 + 1 < lim / 64;
    if (force && !std::strcmp(force, kKindNames[kSkinnyFp8T]) && okST) return kSkinnyFp8T;
    // As for bf16: at three and four rows on a large B the streaming kernel,
    // sharing A across a strip, is faster (8192 x 8192: 15.9 us against
    // 18.7 us at three rows, 15.8 against 19.3 at four).
    if (okV && (M <= 2 || N * K < ((int64_t)1 << 26) || !okS)) return kGemvFp8;
    bool ok = K > 0 && K % 16 == 0;
    ok = ok && lda % 16 == 0 && ldb % 16 == 0 && aligned16(A) && aligned16(B);
    ok = ok && ShapeFp8::BM * lda + K + ShapeFp8::BK < lim && ShapeFp8::BN * ldb + K + ShapeFp8::BK < lim;
    ok = ok && ((M + 255) / 256) * ((N + 255) / 256) < lim;
    const bool ok128 = ((M + ShapeFp8M::BM - 1) / ShapeFp8M::BM) * ((N + ShapeFp8M::BN - 1) / ShapeFp8M::BN) < lim / 64;
    // As for bf16, more than two 32-wide strips per compute unit over a
    // short K (fewer than 8 slices of 512) run faster on the masked 128x128
    // tiles (65536 x 64 x 1024: 20.5 us against 29.9 us streaming; 32 x
    // 32768 x 2048 16.3 against 20.0 us; at two strips per compute unit the
    // streaming kernel is still faster: 64 x 16384 x 2048 12.6 against
    // 13.9 us).
    const bool tiles_pay = ok && ok128 && K < 8 * ShapeSkinny::KS_FP8;
    if (okS) return ((N + 31) / 32 > 2 * cus && tiles_pay) ? kFp8MediumMasked : kSkinnyFp8;
    if (okST && force == nullptr)  // (a forced tile kernel takes such shapes too)
        return ((M + 31) / 32 > 2 * cus && tiles_pay) ? kFp8MediumMasked : kSkinnyFp8T;
    if (!ok) return kGeneric;
    // the unmasked instance stores C in 16-byte runs; the masked one takes any
    // C (element by element where ldc % 8 != 0 or C is unaligned)
    const bool exact = M % ShapeFp8::BM == 0 && N % ShapeFp8::BN == 0 && K % ShapeFp8::BK == 0 && ldc % 8 == 0 &&
                       aligned16(C);
    if (force && !std::strcmp(force, kKindNames[kFp8Masked])) return kFp8Masked;
    if (force && !std::strcmp(force, kKindNames[kFp8])) return exact ? kFp8 : kFp8Masked;
    if (force && !std::strcmp(force, kKindNames[kFp8Mfma16Masked])) return kFp8Mfma16Masked;
    if (force && !std::strcmp(force, kKindNames[kFp8Mfma32])) return exact ? kFp8Mfma32 : kFp8Masked;
    // the 128x128 tiles: exact multiples of 128 (and C's alignment), or masked
    const bool exact128 = M % ShapeFp8M::BM == 0 && N % ShapeFp8M::BN == 0 && K % ShapeFp8M::BK == 0 &&
                          ldc % 8 == 0 && aligned16(C);
    const bool can_split128 = ok128 && plan_splitk<ShapeFp8M>(M, N, K, cus, cap_floats).splits >= 2;
    if (force && ok128 && !std::strcmp(force, kKindNames[kFp8MediumMasked])) return kFp8MediumMasked;
    if (force && ok128 && !std::strcmp(force, kKindNames[kFp8Medium])) return exact128 ? kFp8Medium : kFp8MediumMasked;
    if (force && can_split128 &&
        (!std::strcmp(force, kKindNames[kFp8SplitKMedium]) || !std::strcmp(force, kKindNames[kFp8SplitKMediumMasked])))
        return exact128 ? kFp8SplitKMedium : kFp8SplitKMediumMasked;
    const bool can_split = plan_splitk_fp8(M, N, K, cus, cap_floats).splits >= 2;
    if (force && can_split &&
        (!std::strcmp(force, kKindNames[kFp8SplitK]) || !std::strcmp(force, kKindNames[kFp8SplitKMasked])))
        return exact ? kFp8SplitK : kFp8SplitKMasked;
    // Small and mid-sized grids (the 256x256 tiles fill at most half of the
    // compute units): the 128x128 tiles, splitting K by the bf16 128x128
    // kernel's rule (an FP8 slice of 128 has its bytes and MFMA time).  The
    // reduction takes any C: it reads and writes a chunk element by element
    // where ldc % 8 != 0, C is unaligned or the chunk straddles M.
    // Measured against the 256x256 paths (split where they split): 1024 x
    // 1024 x 4096 16.4 us against 32.5, 512 x 512 x 8192 (split) 14.8 against
    // 26.8, 2048 x 2048 x 2048 13.0 against 24.8, 1000 x 1000 x 4096 22.1
    // against 31.6.  At exactly half (128 tiles of 256x256) the 128x128
    // tiles still win, as for bf16: 2048 x 4096 x 4096 35.3 against 39.0 us,
    // 2048 x 4096 x 8192 60.9 against 69.8 us; at 144 tiles of 256x256 the
    // large tiles do (3072 x 3072 x 2048 27.4 against 34.8 us, 3072 x 3072 x
    // 4096 39.0 against 50.2 us).
    const int64_t tiles256 = ((M + ShapeFp8::BM - 1) / ShapeFp8::BM) * ((N + ShapeFp8::BN - 1) / ShapeFp8::BN);
    if (ok128 && tiles256 * 2 <= cus) {
        if (can_split128 && splitk_pays_t<ShapeFp8M>(M, N, K))
            return exact128 ? kFp8SplitKMedium : kFp8SplitKMediumMasked;
        return exact128 ? kFp8Medium : kFp8MediumMasked;
    }
    return exact ? kFp8 : kFp8Masked;
}

// The no-allocation entry point's scratch: a file-scope device array of
// the fixed split-K layout sized for 256 compute units (64 KiB of counters
// and 16 MiB of partials).  Each GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in,
// so its device address is looked up once per device (noalloc_scratch) and
// only that address is handed to kernels.
constexpr size_t kNoAllocCus = 256;
constexpr size_t kNoAllocFloats = kNoAllocCus * kScratchFloatsPerCu;
constexpr size_t kNoAllocBytes = kScratchCounterBytes + kNoAllocFloats * 4;
static __device__ __align__(256) char scratch[kNoAllocBytes];

static std::mutex g_noalloc_mutex;
static char *g_noalloc_ptr[64];  // device address of `scratch`, per device, after set-up

// Set-up on a device's first no-allocation call (with that device
// current): look up the array's device address and zero its counters with
// a fill kernel on the caller's stream.  The streaming kernel's last unit
// of each strip resets that strip's counter, so they stay zero between
// calls.
static hipError_t noalloc_scratch(hipStream_t stream, Scratch *out) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_noalloc_mutex);
    if (g_noalloc_ptr[dev] == nullptr) {
        void *p = nullptr;
        if ((err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return err;
        if (p == nullptr) return hipErrorInvalidSymbol;
        if ((err = zero_counters(reinterpret_cast<uint32_t *>(p), stream)) != hipSuccess) return err;
        g_noalloc_ptr[dev] = static_cast<char *>(p);
    }
    out->fixed = g_noalloc_ptr[dev];
    out->cap_floats = kNoAllocFloats;
    return hipSuccess;
}

// The bf16 product behind gemm_bf16 and gemm_bf16_noalloc (arguments
// already validated, M, N > 0); scr says where split-K partials go.
static int run_bf16(int64_t M, int64_t N, int64_t K, const gemm_bf16_t *A, int64_t lda, const gemm_bf16_t *B,
                    int64_t ldb, gemm_bf16_t *C, int64_t ldc, float alpha, float beta, const gemm_bf16_t *bias,
                    int epilogue, const Scratch &scr, int cus, hipStream_t stream) {
    GemmArgs args{};
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

    hipError_t err = hipSuccess;
    switch (choose_kernel(M, N, K, A, lda, B, ldb, C, ldc, cus, scr.cap_floats)) {
    case kLarge: err = launch_tile_large(args, cus, stream); break;
    case kMedium: err = launch_tile_medium(args, cus, stream); break;
    case kSplitK: err = launch_splitk_plan(args, cus, scr, stream); break;
    case kMediumMasked: err = launch_tile_medium_masked(args, cus, stream); break;
    case kSplitKMasked: err = launch_splitk_plan(args, cus, scr, stream, false, true); break;
    case kGemv: err = launch_gemv(args, stream); break;
    case kRing32: err = launch_tile_ring_mfma32(args, cus, stream); break;
    case kRing: err = launch_tile_ring(args, cus, stream); break;
    case kRingW8: err = launch_tile_ring_w8(args, cus, stream); break;
    case kRingMasked: err = launch_tile_ring_masked(args, cus, stream); break;
    case kSkinny: err = launch_skinny_plan(args, cus, scr, stream); break;
    case kSkinnyT: err = launch_skinny_plan(transposed(args), cus, scr, stream, false, false, true); break;
    default: err = launch_generic(args, cus, stream); break;
    }
    if (err != hipSuccess) {
        t_last_hip_error = (int)err;
        return GEMM_ERR_HIP;
    }
    return GEMM_OK;
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
    const int cus = device_cu_count();
    return run_bf16(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, bias, epilogue, stream_scratch(cus), cus,
                    stream);
}

int gemm_bf16_noalloc(int64_t M, int64_t N, int64_t K, const gemm_bf16_t *A, int64_t lda, const gemm_bf16_t *B,
                      int64_t ldb, gemm_bf16_t *C, int64_t ldc, float alpha, float beta, const gemm_bf16_t *bias,
                      int epilogue, hipStream_t stream) {
    using namespace gb;
    const int st = validate(M, N, K, A, lda, B, ldb, C, ldc, epilogue);
    if (st != GEMM_OK) return st;
    if (M == 0 || N == 0) return GEMM_OK;
    Scratch scr;
    const hipError_t err = noalloc_scratch(stream, &scr);
    if (err != hipSuccess) {
        t_last_hip_error = (int)err;
        return GEMM_ERR_HIP;
    }
    return run_bf16(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, bias, epilogue, scr, device_cu_count(), stream);
}

int gemm_bf16_q8(int64_t M, int64_t N, int64_t K, const gemm_bf16_t *A, int64_t lda, const gemm_bf16_t *B,
                 int64_t ldb, const gemm_bf16_t *C, int64_t ldc, int8_t *Q, int64_t ldq, float alpha, float beta,
                 const gemm_bf16_t *bias, int epilogue, const float *scale, int32_t zero_point,
                 hipStream_t stream) {
    using namespace gb;
    const int st = validate_q8(M, N, K, A, lda, B, ldb, C, ldc, Q, ldq, beta, scale, epilogue);
    if (st != GEMM_OK) return st;
    if (M == 0 || N == 0) return GEMM_OK;

    GemmArgs args{};
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
    const Scratch scr = stream_scratch(cus);
    hipError_t err = hipSuccess;
    switch (choose_kernel_q8(M, N, K, A, lda, B, ldb, C, ldc, beta, Q, ldq, scale, cus, scr.cap_floats)) {
    case kRingQ8: err = launch_tile_ring_q8(args, cus, stream); break;
    case kRingQ8Masked: err = launch_tile_ring_q8_masked(args, cus, stream); break;
    case kSkinnyQ8: err = launch_skinny_plan(args, cus, scr, stream, false, true); break;
    case kSkinnyQ8T: err = launch_skinny_plan(transposed(args), cus, scr, stream, false, true, true); break;
    case kSplitKQ8: err = launch_splitk_plan(args, cus, scr, stream, true); break;
    case kSplitKQ8Masked: err = launch_splitk_plan(args, cus, scr, stream, true, true); break;
    case kTileQ8: err = launch_tile_q8_plan(args, cus, scr, stream, false); break;
    case kTileQ8Masked: err = launch_tile_q8_plan(args, cus, scr, stream, true); break;
    default: err = launch_generic(args, cus, stream); break;
    }
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
        gb::choose_kernel_q8(M, N, K, A, lda, B, ldb, C, ldc, beta, Q, ldq, scale, gb::device_cu_count(),
                             gb::stream_scratch(gb::device_cu_count()).cap_floats));
}

int gemm_fp8(int64_t M, int64_t N, int64_t K, const gemm_fp8_t *A, int64_t lda, const gemm_fp8_t *B,
             int64_t ldb, gemm_bf16_t *C, int64_t ldc, float alpha, float beta, const float *scale_a,
             const float *scale_b, const gemm_bf16_t *bias, int epilogue, hipStream_t stream) {
    using namespace gb;
    const int st = validate(M, N, K, A, lda, B, ldb, C, ldc, epilogue);
    if (st != GEMM_OK) return st;
    if (M == 0 || N == 0) return GEMM_OK;

    GemmArgs args{};
    args.M = M;
    args.N = N;
    args.K = K;
    args.A = reinterpret_cast<const uint16_t *>(A);  // bytes; the fp8 kernels read them as such
    args.lda = lda;
    args.B = reinterpret_cast<const uint16_t *>(B);
    args.ldb = ldb;
    args.C = C;
    args.ldc = ldc;
    args.alpha = alpha;
    args.beta = beta;
    args.bias = bias;
    args.flags = epilogue_flags(beta, bias, epilogue);
    args.scale_a = scale_a;
    args.scale_b = scale_b;

    const int cus = device_cu_count();
    const Scratch scr = stream_scratch(cus);
    hipError_t err = hipSuccess;
    switch (choose_kernel_fp8(M, N, K, A, lda, B, ldb, C, ldc, cus, scr.cap_floats)) {
    case kFp8: err = launch_tile_fp8(args, cus, stream); break;
    case kFp8SplitK: err = launch_fp8_splitk_plan(args, cus, scr, stream, false); break;
    case kFp8SplitKMasked: err = launch_fp8_splitk_plan(args, cus, scr, stream, true); break;
    case kFp8Masked: err = launch_tile_fp8_mfma32_masked(args, cus, stream); break;
    case kFp8Mfma32: err = launch_tile_fp8_mfma32(args, cus, stream); break;
    case kFp8Mfma16Masked: err = launch_tile_fp8_mfma16_masked(args, cus, stream); break;
    case kFp8Medium: err = launch_tile_fp8_medium(args, cus, stream); break;
    case kFp8MediumMasked: err = launch_tile_fp8_medium_masked(args, cus, stream); break;
    case kFp8SplitKMedium: err = launch_fp8_medium_splitk_plan(args, cus, scr, stream, false); break;
    case kFp8SplitKMediumMasked: err = launch_fp8_medium_splitk_plan(args, cus, scr, stream, true); break;
    case kGemvFp8: err = launch_gemv(args, stream, true); break;
    case kSkinnyFp8: err = launch_skinny_plan(args, cus, scr, stream, true); break;
    case kSkinnyFp8T: err = launch_skinny_plan(transposed(args), cus, scr, stream, true, false, true); break;
    default: err = launch_generic(args, cus, stream, true); break;
    }
    if (err != hipSuccess) {
        t_last_hip_error = (int)err;
        return GEMM_ERR_HIP;
    }
    return GEMM_OK;
}

const char *gemm_fp8_kernel_name(int64_t M, int64_t N, int64_t K, const gemm_fp8_t *A, int64_t lda,
                                 const gemm_fp8_t *B, int64_t ldb, const gemm_bf16_t *C, int64_t ldc,
                                 int epilogue) {
    if (gb::validate(M, N, K, A, lda, B, ldb, C, ldc, epilogue) != GEMM_OK) return "none";
    const int cus = gb::device_cu_count();
    return gb::kind_name(
        gb::choose_kernel_fp8(M, N, K, A, lda, B, ldb, C, ldc, cus, gb::stream_scratch(cus).cap_floats));
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
    const int cus = gb::device_cu_count();
    return gb::kind_name(gb::choose_kernel(M, N, K, A, lda, B, ldb, C, ldc, cus, gb::stream_scratch(cus).cap_floats));
}

}  // extern "C"
