// kernel_skinny.h -- streaming kernel for short-and-wide products (at most 64
// rows of C) whose cost is reading B once from HBM.
//
// With M this small the product is memory-bound: at M = 64, N = K = 8192 the
// kernel moves 136 MB for 8.6 GFLOP (63 flop/byte, against a machine balance
// of about 300), so what matters is streaming the K x N operand B at full
// HBM bandwidth (small M "lacks data reuse, memory loads become the
// bottleneck" -- DeepGEMM article, demingchina.com, section 5.1; small N is
// bandwidth-bound in "Outperforming cuBLAS on H100: a worklog", section
// "Conclusion").  Decode-sized products (M = 1..16) take the same path.
//
// Work split.  A work unit is one strip of BN columns of C over one range of
// K (split-K: the K-slices are divided into `splits` contiguous ranges).
// One workgroup (four waves) per unit, looping over units (persistent).  The
// unit's B columns (K-contiguous) and all rows of A are walked in K-slices
// of KS: each slice is DMA-loaded into LDS with 16 B/lane loads, and the
// four waves split the slice's MFMA k-steps, each keeping a private fp32
// accumulator of the whole strip.  The four partial strips are then summed
// through LDS.  With one split the fused epilogue writes bf16 C directly;
// otherwise the unit's fp32 partial goes to a workspace and the last unit of
// the strip to arrive (an atomic counter per strip) adds the partials in
// split order -- the same order whichever unit is last, so the result is
// deterministic -- and runs the epilogue.  When the host places a strip's
// splits on one XCD (colocate) the partials are plain stores that the last
// unit reads back through that XCD's L2 (handoff.h); otherwise they cross
// XCDs as device-wide atomics.
//
// Why split K.  Every unit reads all M rows of A for its K range, so without
// a split each of 256 compute units pulls the whole of A through its load
// path: at M = 64, N = 8192, K = 8192 that is twice the B traffic per unit,
// and it (not HBM) is what limits a 32-column strip.  Wider strips with a
// split keep the unit count while dividing the A traffic per unit.
//
// Tails.  Rows of A past M, columns of B past N and K-chunks past K are
// loaded from an out-of-range buffer offset, which the DMA turns into zeros
// (the zero-fill of the DeepGEMM article, sections 4.2-4.3); the epilogue
// masks its loads and stores.  K must be a multiple of 8 (whole 16-byte
// chunks).
//
// Rings.  A (BMr x KS per slice) is re-read from L2 by every unit and
// arrives quickly, B (BN x KS per slice) comes from HBM once, so B is
// prefetched further ahead: rings of SA and SB slices, with SA-1 and SB-1
// slices in flight.
//
// LDS rows are KS*2 bytes; chunk c of row r is stored at c ^ (r & 15) (r & 15
// limited to the row's chunk count), which keeps the 32-row fragment reads
// on distinct banks in every 8- and 16-lane group.
//
// kFp8: A and B hold OCP FP8 E4M3 bytes (the FP8 input path of the DeepGEMM
// article, sections 1.2 and 6.3).  The byte layout is unchanged -- a slice
// row is still KS*2 bytes, now 2*KS values, and a 16-byte chunk 16 values --
// and the k-steps run on 32x32x64 FP8 MFMAs: lane l's 32 bytes of a k-step
// are chunks 4s + l/32 and 4s + 2 + l/32 (the same for A and B, which is all
// the MFMA needs).  The epilogue scales the sum by scale_a[m] and
// scale_b[n].
#pragma once

#include "device_common.h"
#include "handoff.h"
#include "tile_schedule.h"

namespace gb {

template <int FM_, int FN_ = 1, int KS_ = 256, int SA_ = 3, int SB_ = 4>
struct SkinnyConfig {
    static constexpr int FM = FM_;                 // 32-row MFMA blocks: up to 32 * FM rows
    static constexpr int FN = FN_;                 // 32-column MFMA blocks per strip
    static constexpr int BMr = 32 * FM;            // rows of C
    static constexpr int BN = 32 * FN;             // columns per strip
    static constexpr int KS = KS_;                 // K per slice
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 256;
    static constexpr int kRowBytes = KS * 2;       // 512 for KS = 256
    static constexpr int kChunks = kRowBytes / 16; // 16-byte chunks per row
    static constexpr int kSwzMask = kChunks >= 16 ? 15 : kChunks - 1;
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;
    static constexpr int kABytes = BMr * kRowBytes;
    static constexpr int kBBytes = BN * kRowBytes;
    static constexpr int SA = SA_, SB = SB_;       // ring depths
    static constexpr int kLdsBytes = SA * kABytes + SB * kBBytes;
    static constexpr int kALoads = BMr / kRowsPerLoad / kWaves;  // 1 KiB wave loads
    static constexpr int kBLoads = BN / kRowsPerLoad / kWaves;
    static constexpr int kStepsPerWave = KS / 16 / kWaves;
    // partial-sum staging: fp32, column-major, columns padded by 16 bytes
    static constexpr int kColBytes = BMr * 4 + 16;
    static constexpr int kPartBytes = BN * kColBytes;
    static constexpr int kFlagOffset = kLdsBytes - 16;  // the "last unit" flag word
    static_assert(FM == 1 || FM == 2, "up to 32 or 64 rows");
    static_assert(FN == 1 || FN == 2 || FN == 4, "strips of 32, 64 or 128 columns");
    static_assert(KS == 128 || KS == 256, "rows of 256 or 512 bytes");
    static_assert(BMr % (kRowsPerLoad * kWaves) == 0 && BN % (kRowsPerLoad * kWaves) == 0, "loads split");
    static_assert((KS / 16) % kWaves == 0, "k-steps split over the waves");
    static_assert(kLdsBytes <= 160 * 1024, "gfx950 has 160 KiB of LDS per compute unit");
    static_assert(SA >= 2 && SB > SA, "B is prefetched further ahead than A");
    static_assert((SA - 1) * kALoads + (SB - 1) * kBLoads < 64, "vmcnt is a 6-bit counter");
    static_assert(kWaves * kPartBytes + 16 <= kLdsBytes, "partial sums and the flag reuse the rings");
};

// The unit decomposition and the split-K workspace (unused with splits == 1):
// partials[unit * BN * BMr + chunk * 8 + row % 8] in fp32 (unit = strip *
// splits + split, chunk = col * BMr / 8 + row / 8) and, per strip, one
// uint32 counter or (colocate) one handoff record, zero between calls.
// colocate: the grid is exactly one workgroup per unit, a multiple of 8 of
// them, and each XCD's run of slots holds whole strips; a strip's splits
// then hand their partials over within one XCD (handoff.h) -- with 2, always
// through the fenced path (for testing it).
struct SkinnyWork {
    int num_strips;
    int splits;
    int spp;       // K-slices per split (the last split may have fewer)
    int c_vector;  // C 16-byte aligned and ldc % 8 == 0: 8-row chunks move as one 16-byte access
    int q_vector;  // int8 output: Q 8-byte aligned and ldq % 8 == 0 (8-row chunks as one 8-byte store)
    int colocate;
    float *partials;
    uint32_t *counters;
    HandoffRecord *records;  // the same memory as counters, for colocate
};

// Requirements checked by the host: 1 <= M <= BMr, N >= 1, K a multiple of
// one 16-byte chunk (8 values, 16 with kFp8), A/B 16-byte aligned, lda/ldb
// multiples of a chunk (C: any ldc >= M, element-wise accesses unless
// work.c_vector), the byte offsets of one unit ((BMr-1)*lda + K + a slice,
// (BN-1)*ldb + K + a slice) below 2^31, and every split owning at least one
// K-slice.
// kQ8: the int8 output of the quantizing entry point -- the epilogue value
// of row m becomes sat8(rne(fma(v, scale[m], zp))) in Q (C is then only
// read, when beta != 0).
// kTrans: the kernel computes the transposed product C' = A' B' of a
// product with at most 64 columns (the host passes A' = B^T, B' = A^T,
// M' = N, N' = M, and the bias of C's columns as bias[m']) and writes C'
// transposed: element (m', n') of C' goes to C[n' + m' * ldc], so each
// output chunk is 8 consecutive n' of one row m', contiguous in C.  With
// kFp8 the host also swaps the scales (scale_a[m'] is C's column scale,
// scale_b[n'] its row scale); with kQ8, scale[n'] is the quantization
// scale of C's row n' and Q is written transposed like C.
template <class Cfg, uint32_t kFlags, bool kFp8 = false, bool kQ8 = false, bool kTrans = false>
__global__ void __launch_bounds__(Cfg::kThreads)
gemm_skinny_kernel(const GemmArgs args, const SkinnyWork work) {
    static_assert(!(kFp8 && kQ8), "int8 output is built for bf16 inputs");
    __shared__ __attribute__((aligned(1024))) char smem[Cfg::kLdsBytes];
    char *const ringA = smem;
    char *const ringB = smem + Cfg::SA * Cfg::kABytes;
    constexpr int kElem = kFp8 ? 1 : 2;                       // bytes per value
    constexpr int kSliceVals = Cfg::kRowBytes / kElem;        // values per slice row
    constexpr int kChunkVals = 16 / kElem;                    // values per 16-byte chunk

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lda_bytes = (uint32_t)(args.lda * kElem), ldb_bytes = (uint32_t)(args.ldb * kElem);

    // Load side: a wave load covers rows kRowsPerLoad*q ..; lane i takes row
    // kRowsPerLoad*q + i/kChunks and LDS chunk position i%kChunks, holding
    // logical chunk (i%kChunks) ^ (row & kSwzMask).
    const int lrow = lane / Cfg::kChunks, lpos = lane % Cfg::kChunks;
    // Fragment side: lane l reads row l%32 (+32i) at logical chunk 2s + l/32.
    const uint32_t fragRow = (uint32_t)(lane & 31) * Cfg::kRowBytes;
    const int fragSw = lane & Cfg::kSwzMask;

    // Per-lane row, chunk and byte offset (row * ld + chunk * 16) of each of
    // this wave's loads -- the same for every slice and unit, so a load only
    // adds the slice's K offset (one scalar).
    int rA_[Cfg::kALoads], rB_[Cfg::kBLoads], cA[Cfg::kALoads], cB[Cfg::kBLoads];
    uint32_t vA[Cfg::kALoads], vB[Cfg::kBLoads];
#pragma unroll
    for (int i = 0; i < Cfg::kALoads; ++i) {
        rA_[i] = Cfg::kRowsPerLoad * (wave * Cfg::kALoads + i) + lrow;
        cA[i] = lpos ^ (rA_[i] & Cfg::kSwzMask);
        vA[i] = (uint32_t)rA_[i] * lda_bytes + (uint32_t)cA[i] * 16;
    }
#pragma unroll
    for (int i = 0; i < Cfg::kBLoads; ++i) {
        rB_[i] = Cfg::kRowsPerLoad * (wave * Cfg::kBLoads + i) + lrow;
        cB[i] = lpos ^ (rB_[i] & Cfg::kSwzMask);
        vB[i] = (uint32_t)rB_[i] * ldb_bytes + (uint32_t)cB[i] * 16;
    }

    const int nk = (int)((args.K + kSliceVals - 1) / kSliceVals);
    const int rowsA = (int)(args.M < Cfg::BMr ? args.M : Cfg::BMr);
    const int kmax = (int)args.K;
    const int num_units = work.num_strips * work.splits;
    const char *A8 = reinterpret_cast<const char *>(args.A);
    const char *B8 = reinterpret_cast<const char *>(args.B);
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(A8, (uint32_t)(((rowsA - 1) * args.lda + args.K) * kElem));

    const bool coloc = work.colocate != 0;
    const int xcd = coloc ? xcd_id() : 0;
    for (int w = blockIdx.x; w < num_units; w += gridDim.x) {
        const int unit = coloc ? handoff_slot(w, gridDim.x) : w;
        const int strip = unit / work.splits;
        const int split = unit % work.splits;
        const int64_t n0 = (int64_t)strip * Cfg::BN;
        const int colsB = (int)(args.N - n0 < Cfg::BN ? args.N - n0 : Cfg::BN);
        const int s0 = split * work.spp;
        const int ns = (nk - s0 < work.spp ? nk - s0 : work.spp);  // >= 1, checked by the host
        const __amdgpu_buffer_rsrc_t rB =
            make_rsrc(B8 + n0 * args.ldb * kElem, (uint32_t)(((colsB - 1) * args.ldb + args.K) * kElem));

        // Slice j of this unit's order into its ring buffer.  Slices are
        // issued in order (A and B each), walking the unit's K range from a
        // rotated start (strip index within its XCD, so the workgroups
        // sharing an L2 do not all request the same A lines at once; a
        // colocated XCD holds a contiguous run of strips).  A
        // chunk outside the matrix (row past M or N, k past K) is loaded from
        // the out-of-range offset; slices of full strips take a branch-free
        // path.
        const bool allA = rowsA == Cfg::BMr, allB = colsB == Cfg::BN;
        const int s_end = s0 + ns;
        const int xcd_strip = coloc ? strip % (work.num_strips / kNumXcds) : strip / kNumXcds;
        int ksA = s0 + xcd_strip % ns, ksB = ksA;
        auto issueA = [&](int j) {
            char *dst = ringA + (j % Cfg::SA) * Cfg::kABytes;
            const int ks = ksA;
            ksA = ksA + 1 == s_end ? s0 : ksA + 1;
            const uint32_t soff = (uint32_t)ks * Cfg::kRowBytes;
            if (allA && (ks + 1) * kSliceVals <= kmax) {
#pragma unroll
                for (int i = 0; i < Cfg::kALoads; ++i)
                    buffer_load_lds16(rA, (GB_LDS void *)(dst + (wave * Cfg::kALoads + i) * 1024), vA[i], soff);
            } else {
#pragma unroll
                for (int i = 0; i < Cfg::kALoads; ++i) {
                    const bool ok = rA_[i] < rowsA && ks * kSliceVals + cA[i] * kChunkVals < kmax;
                    buffer_load_lds16(rA, (GB_LDS void *)(dst + (wave * Cfg::kALoads + i) * 1024),
                                      ok ? vA[i] : kOobOffset, soff);
                }
            }
        };
        auto issueB = [&](int j) {
            char *dst = ringB + (j % Cfg::SB) * Cfg::kBBytes;
            const int ks = ksB;
            ksB = ksB + 1 == s_end ? s0 : ksB + 1;
            const uint32_t soff = (uint32_t)ks * Cfg::kRowBytes;
            if (allB && (ks + 1) * kSliceVals <= kmax) {
#pragma unroll
                for (int i = 0; i < Cfg::kBLoads; ++i)
                    buffer_load_lds16(rB, (GB_LDS void *)(dst + (wave * Cfg::kBLoads + i) * 1024), vB[i], soff);
            } else {
#pragma unroll
                for (int i = 0; i < Cfg::kBLoads; ++i) {
                    const bool ok = rB_[i] < colsB && ks * kSliceVals + cB[i] * kChunkVals < kmax;
                    buffer_load_lds16(rB, (GB_LDS void *)(dst + (wave * Cfg::kBLoads + i) * 1024),
                                      ok ? vB[i] : kOobOffset, soff);
                }
            }
        };

        f32x16 acc[Cfg::FM][Cfg::FN];
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = f32x16{};

        if (coloc && threadIdx.x == 0) handoff_register(work.records + strip, xcd);
        // Previous unit's partial-sum reduction is done with LDS.
        lds_barrier();
        // Prologue: the steady state issues A(j + SA-1), then B(j + SB-1), at
        // slice j's barrier; the prologue replays that order for the virtual
        // barriers j = -(SB-1) .. -1, leaving A(0 .. SA-2) and B(0 .. SB-2)
        // in flight.
        for (int j = -(Cfg::SB - 1); j < 0; ++j) {
            const int a = j + Cfg::SA - 1, b = j + Cfg::SB - 1;
            if (a >= 0 && a < ns) issueA(a);
            if (b < ns) issueB(b);
        }

        for (int kt = 0; kt < ns; ++kt) {
            // Slice kt's A and B have landed once only the loads issued after
            // A(kt) are outstanding (B(kt) went out before A(kt) since SB >
            // SA): when every slice up to kt+SB-2 exists these are A(kt+1 ..
            // kt+SA-2) and B(kt+SB-SA .. kt+SB-2); near the end of the range
            // the pipeline simply drains.
            if (kt + Cfg::SB - 1 <= ns)
                wait_vmcnt<(Cfg::SA - 2) * Cfg::kALoads + (Cfg::SA - 1) * Cfg::kBLoads>();
            else
                wait_vmcnt<0>();
            lds_barrier();  // everyone's loads landed; slice kt-1 fully read
            if (kt + Cfg::SA - 1 < ns) issueA(kt + Cfg::SA - 1);
            if (kt + Cfg::SB - 1 < ns) issueB(kt + Cfg::SB - 1);

            const char *sA = ringA + (kt % Cfg::SA) * Cfg::kABytes;
            const char *sB = ringB + (kt % Cfg::SB) * Cfg::kBBytes;
            if constexpr (kFp8) {
                // 64-byte k-steps: Cfg::kStepsPerWave / 2 per wave
#pragma unroll
                for (int st = 0; st < Cfg::kStepsPerWave / 2; ++st) {
                    const int s = wave * (Cfg::kStepsPerWave / 2) + st;
                    const uint32_t clo = (uint32_t)(((4 * s + (lane >> 5)) ^ fragSw) << 4);
                    const uint32_t chi = (uint32_t)(((4 * s + 2 + (lane >> 5)) ^ fragSw) << 4);
                    i32x8 b[Cfg::FN];
#pragma unroll
                    for (int j = 0; j < Cfg::FN; ++j) {
                        b[j].lo = *(const GB_LDS i32x4 *)(sB + j * 32 * Cfg::kRowBytes + fragRow + clo);
                        b[j].hi = *(const GB_LDS i32x4 *)(sB + j * 32 * Cfg::kRowBytes + fragRow + chi);
                    }
#pragma unroll
                    for (int i = 0; i < Cfg::FM; ++i) {
                        i32x8 a;
                        a.lo = *(const GB_LDS i32x4 *)(sA + i * 32 * Cfg::kRowBytes + fragRow + clo);
                        a.hi = *(const GB_LDS i32x4 *)(sA + i * 32 * Cfg::kRowBytes + fragRow + chi);
#pragma unroll
                        for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = mfma_fp8_32x32x64(a, b[j], acc[i][j]);
                    }
                }
                continue;
            }
#pragma unroll
            for (int st = 0; st < Cfg::kStepsPerWave; ++st) {
                const int s = wave * Cfg::kStepsPerWave + st;
                const uint32_t coff = (uint32_t)(((2 * s + (lane >> 5)) ^ fragSw) << 4);
                bf16x8 b[Cfg::FN];
#pragma unroll
                for (int j = 0; j < Cfg::FN; ++j)
                    b[j] = *(const GB_LDS bf16x8 *)(sB + j * 32 * Cfg::kRowBytes + fragRow + coff);
#pragma unroll
                for (int i = 0; i < Cfg::FM; ++i) {
                    const bf16x8 a = *(const GB_LDS bf16x8 *)(sA + i * 32 * Cfg::kRowBytes + fragRow + coff);
#pragma unroll
                    for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = mfma_32x32x16(a, b[j], acc[i][j]);
                }
            }
        }

        // Sum the four waves' partial strips: wave w stores its strip as
        // fp32, column-major (column stride BMr*4 + 16 bytes), then each lane
        // sums 8 consecutive rows of one column over the four copies.
        lds_barrier();
        {
            char *part = smem + wave * Cfg::kPartBytes;
            const int h = lane >> 5;
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
                for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                         acc[i][j][4 * g + 3]};
                        *(GB_LDS f32x4 *)(part + (j * 32 + (lane & 31)) * Cfg::kColBytes +
                                          (i * 32 + g * 8 + h * 4) * 4) = v;
                    }
        }
        lds_barrier();
        constexpr int kChunksPerCol = Cfg::BMr / 8;
        constexpr int kChunks = Cfg::BN * kChunksPerCol;  // 8-row pieces of the strip
        constexpr int kChunksPerRow = Cfg::BN / 8;          // kTrans: 8-column pieces of a row
        static_assert(16 % kChunksPerRow == 0, "strips of 32, 64 or 128 columns");

        // The four waves' sum of one 8-row chunk (column idx / kChunksPerCol)
        // -- with kTrans, of one 8-column chunk (row idx / kChunksPerRow).
        auto wave_sum = [&](int idx, float (&x)[8]) {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = 0.f;
            if constexpr (kTrans) {
                // One float per column at the column stride: the 64 lanes of a
                // wave cover 64 / kChunksPerRow rows of kChunksPerRow chunks,
                // and chunks two apart would meet on the same banks, so lane
                // reads its 8 columns in the order e ^ rot (rot spreads the
                // chunks over the banks), then undoes the permutation with
                // conditional swaps of register pairs.
                const int r = idx / kChunksPerRow, q = idx % kChunksPerRow, c8 = q * 8;
                const int rot = ((q >> 1) * (16 / kChunksPerRow)) & 7;
#pragma unroll
                for (int w = 0; w < Cfg::kWaves; ++w)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        x[e] += *(const GB_LDS float *)(smem + w * Cfg::kPartBytes +
                                                        (c8 + (e ^ rot)) * Cfg::kColBytes + r * 4);
#pragma unroll
                for (int b = 1; b < 8; b <<= 1) {
                    const bool swap = (rot & b) != 0;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if ((e & b) == 0) {
                            const float lo = x[e], hi = x[e | b];
                            x[e] = swap ? hi : lo;
                            x[e | b] = swap ? lo : hi;
                        }
                }
                return;
            }
            const int col = idx / kChunksPerCol, q = idx % kChunksPerCol;
#pragma unroll
            for (int w = 0; w < Cfg::kWaves; ++w) {
                const char *p = smem + w * Cfg::kPartBytes + col * Cfg::kColBytes + q * 32;
                const f32x4 lo = *(const GB_LDS f32x4 *)p;
                const f32x4 hi = *(const GB_LDS f32x4 *)(p + 16);
                x[0] += lo.x; x[1] += lo.y; x[2] += lo.z; x[3] += lo.w;
                x[4] += hi.x; x[5] += hi.y; x[6] += hi.z; x[7] += hi.w;
            }
        };
        // The fused epilogue on one 8-row chunk of the strip's sum x: bf16 C
        // with a 16-byte store, element by element where the chunk straddles M.
        auto finish = [&](int idx, const float (&x)[8]) {
            if constexpr (kTrans) {
                // row m' of C', columns n0 + c8 .. + 7: C[n' + m' * ldc],
                // the bias of C's column m'
                const int r = idx / kChunksPerRow, c8 = (idx % kChunksPerRow) * 8;
                const int64_t n = n0 + c8;
                if (r >= args.M || n >= args.N) return;
                uint16_t *cp = args.C + (int64_t)r * args.ldc + n;
                const bool full = n + 8 <= args.N && work.c_vector;
                float xs[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) xs[e] = x[e];
                if constexpr (kFp8) {
                    // C's row scale, then its column scale, as the direct kernel multiplies
                    const float sc = args.scale_a ? args.scale_a[r] : 1.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float sr = (args.scale_b && n + e < args.N) ? args.scale_b[n + e] : 1.f;
                        xs[e] = x[e] * sr * sc;
                    }
                }
                float bias_v = 0.f;
                if constexpr ((kFlags & kEpiBias) != 0) bias_v = bf16_bits_to_f32(args.bias[r]);
                float cin[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                if constexpr ((kFlags & kEpiBeta) != 0) {
                    if (full) {
                        const u32x4 raw = *(const u32x4 *)cp;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            cin[2 * e] = bf16_bits_to_f32(raw[e] & 0xFFFFu);
                            cin[2 * e + 1] = bf16_bits_to_f32(raw[e] >> 16);
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) if (n + e < args.N) cin[e] = bf16_bits_to_f32(cp[e]);
                    }
                }
                if constexpr (kQ8) {
                    // columns past N' get scale 0 and are never stored
                    u32x2 qw = {0u, 0u};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float v = epilogue_value<kFlags>(xs[e], cin[e], bias_v, args.alpha, args.beta);
                        const float sc = n + e < args.N ? args.scale[n + e] : 0.f;
                        qw[e >> 2] |= ((uint32_t)quantize_i8(v, sc, args.zp) & 0xFFu) << ((e & 3) * 8);
                    }
                    int8_t *qp = args.Q + (int64_t)r * args.ldq + n;
                    if (n + 8 <= args.N && work.q_vector) {
                        __builtin_nontemporal_store(qw, (u32x2 *)qp);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (n + e < args.N) qp[e] = (int8_t)(qw[e >> 2] >> ((e & 3) * 8));
                    }
                    return;
                }
                u32x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    out[e] = pack_bf16x2(epilogue_value<kFlags>(xs[2 * e], cin[2 * e], bias_v, args.alpha, args.beta),
                                         epilogue_value<kFlags>(xs[2 * e + 1], cin[2 * e + 1], bias_v, args.alpha,
                                                                args.beta));
                if (full) {
                    __builtin_nontemporal_store(out, (u32x4 *)cp);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (n + e < args.N) cp[e] = (uint16_t)(out[e >> 1] >> ((e & 1) * 16));
                }
                return;
            }
            const int col = idx / kChunksPerCol, q = idx % kChunksPerCol;
            const int64_t n = n0 + col;
            const int64_t m = (int64_t)q * 8;
            if (n >= args.N || m >= args.M) return;
            uint16_t *cp = args.C + n * args.ldc + m;
            const bool full = m + 8 <= args.M && work.c_vector;
            float xs[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) xs[e] = x[e];
            if constexpr (kFp8) {
                const float sb = args.scale_b ? args.scale_b[n] : 1.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float sa = (args.scale_a && m + e < args.M) ? args.scale_a[m + e] : 1.f;
                    xs[e] = x[e] * sa * sb;
                }
            }
            float bias_v = 0.f;
            if constexpr ((kFlags & kEpiBias) != 0) bias_v = bf16_bits_to_f32(args.bias[n]);
            float cin[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if constexpr ((kFlags & kEpiBeta) != 0) {
                if (full) {
                    const u32x4 raw = *(const u32x4 *)cp;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        cin[2 * e] = bf16_bits_to_f32(raw[e] & 0xFFFFu);
                        cin[2 * e + 1] = bf16_bits_to_f32(raw[e] >> 16);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) if (m + e < args.M) cin[e] = bf16_bits_to_f32(cp[e]);
                }
            }
            if constexpr (kQ8) {
                // rows past M get scale 0 and are never stored
                u32x2 qw = {0u, 0u};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v = epilogue_value<kFlags>(xs[e], cin[e], bias_v, args.alpha, args.beta);
                    const float sc = m + e < args.M ? args.scale[m + e] : 0.f;
                    qw[e >> 2] |= ((uint32_t)quantize_i8(v, sc, args.zp) & 0xFFu) << ((e & 3) * 8);
                }
                int8_t *qp = args.Q + n * args.ldq + m;
                if (m + 8 <= args.M && work.q_vector) {
                    __builtin_nontemporal_store(qw, (u32x2 *)qp);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) if (m + e < args.M) qp[e] = (int8_t)(qw[e >> 2] >> ((e & 3) * 8));
                }
                return;
            }
            u32x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[e] = pack_bf16x2(epilogue_value<kFlags>(xs[2 * e], cin[2 * e], bias_v, args.alpha, args.beta),
                                     epilogue_value<kFlags>(xs[2 * e + 1], cin[2 * e + 1], bias_v, args.alpha,
                                                            args.beta));
            if (full) {
                __builtin_nontemporal_store(out, (u32x4 *)cp);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) if (m + e < args.M) cp[e] = (uint16_t)(out[e >> 1] >> ((e & 1) * 16));
            }
        };

        if (work.splits == 1) {
            for (int idx = threadIdx.x; idx < kChunks; idx += Cfg::kThreads) {
                float x[8];
                wave_sum(idx, x);
                finish(idx, x);
            }
            continue;
        }

        if (coloc) {
            // Split K within one XCD: plain stores of this unit's partial,
            // then the handoff; the last unit adds the partials in split
            // order (the same sum whichever unit is last), loading two
            // splits of every chunk it owns at a time.
            float *mine = work.partials + (int64_t)unit * (Cfg::BN * Cfg::BMr);
            for (int idx = threadIdx.x; idx < kChunks; idx += Cfg::kThreads) {
                float x[8];
                wave_sum(idx, x);
                *(f32x4 *)(mine + idx * 8) = f32x4{x[0], x[1], x[2], x[3]};
                *(f32x4 *)(mine + idx * 8 + 4) = f32x4{x[4], x[5], x[6], x[7]};
            }
            uint32_t *flag = (uint32_t *)(smem + Cfg::kFlagOffset);
            if (!handoff_arrive(work.records + strip, work.splits, xcd, work.colocate == 2, flag)) continue;
            constexpr int kCpt = (kChunks + Cfg::kThreads - 1) / Cfg::kThreads;
            constexpr int64_t kUnitFloats = Cfg::BN * Cfg::BMr;
            const float *base = work.partials + (int64_t)strip * work.splits * kUnitFloats;
            float x[kCpt][8];
#pragma unroll
            for (int c = 0; c < kCpt; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) x[c][e] = 0.f;
            auto add = [&](const f32x4 &lo, const f32x4 &hi, float (&y)[8]) {
                y[0] += lo.x; y[1] += lo.y; y[2] += lo.z; y[3] += lo.w;
                y[4] += hi.x; y[5] += hi.y; y[6] += hi.z; y[7] += hi.w;
            };
            int sp = 0;
            for (; sp + 2 <= work.splits; sp += 2) {
                f32x4 v[kCpt][4];
#pragma unroll
                for (int c = 0; c < kCpt; ++c) {
                    const int idx = threadIdx.x + c * Cfg::kThreads;
                    if (kChunks % Cfg::kThreads == 0 || idx < kChunks) {
                        const float *p = base + sp * kUnitFloats + idx * 8;
                        v[c][0] = *(const f32x4 *)p;
                        v[c][1] = *(const f32x4 *)(p + 4);
                        v[c][2] = *(const f32x4 *)(p + kUnitFloats);
                        v[c][3] = *(const f32x4 *)(p + kUnitFloats + 4);
                    }
                }
#pragma unroll
                for (int c = 0; c < kCpt; ++c) {
                    add(v[c][0], v[c][1], x[c]);
                    add(v[c][2], v[c][3], x[c]);
                }
            }
            if (sp < work.splits) {
#pragma unroll
                for (int c = 0; c < kCpt; ++c) {
                    const int idx = threadIdx.x + c * Cfg::kThreads;
                    if (kChunks % Cfg::kThreads == 0 || idx < kChunks) {
                        const float *p = base + sp * kUnitFloats + idx * 8;
                        add(*(const f32x4 *)p, *(const f32x4 *)(p + 4), x[c]);
                    }
                }
            }
#pragma unroll
            for (int c = 0; c < kCpt; ++c) {
                const int idx = threadIdx.x + c * Cfg::kThreads;
                if (kChunks % Cfg::kThreads == 0 || idx < kChunks) finish(idx, x[c]);
            }
            if (threadIdx.x == 0) handoff_reset(work.records + strip);
            continue;
        }

        // Split K across XCDs: publish this unit's partial, then count
        // arrivals per strip.  The XCDs' L2 caches are not coherent with
        // each other, and a cache-wide write-back / invalidate (an
        // agent-scope fence) costs tens of microseconds when every unit
        // issues one.  The partials are
        // small, so they move through agent-scope atomic read-modify-writes
        // instead, which the hardware performs coherently for the whole
        // device (as it does the arrival counter): each unit swaps its values
        // in, waits for those atomics to complete, then counts; the last unit
        // reads every partial back with an atomic OR of 0.
        unsigned long long *mine =
            (unsigned long long *)(work.partials + (int64_t)unit * (Cfg::BN * Cfg::BMr));
        for (int idx = threadIdx.x; idx < kChunks; idx += Cfg::kThreads) {
            float x[8];
            wave_sum(idx, x);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const unsigned long long bits = (unsigned long long)__builtin_bit_cast(uint32_t, x[2 * e]) |
                                                ((unsigned long long)__builtin_bit_cast(uint32_t, x[2 * e + 1]) << 32);
                __hip_atomic_exchange(mine + idx * 4 + e, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        wait_vmcnt<0>();
        __syncthreads();
        uint32_t *flag = (uint32_t *)(smem + Cfg::kFlagOffset);
        if (threadIdx.x == 0)
            *flag = atomicAdd(work.counters + strip, 1u) == (uint32_t)(work.splits - 1) ? 1u : 0u;
        __syncthreads();
        const bool last = *flag != 0u;
        if (!last) continue;
        unsigned long long *base =
            (unsigned long long *)(work.partials + (int64_t)strip * work.splits * (Cfg::BN * Cfg::BMr));
        for (int idx = threadIdx.x; idx < kChunks; idx += Cfg::kThreads) {
            float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int sp = 0; sp < work.splits; ++sp) {  // split order: the same sum whoever is last
                unsigned long long *src = base + (int64_t)sp * (Cfg::BN * Cfg::BMr / 2) + idx * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const unsigned long long bits =
                        __hip_atomic_fetch_or(src + e, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    x[2 * e] += __builtin_bit_cast(float, (uint32_t)bits);
                    x[2 * e + 1] += __builtin_bit_cast(float, (uint32_t)(bits >> 32));
                }
            }
            finish(idx, x);
        }
        // ready for the next call on this workspace (an atomic, like the adds)
        if (threadIdx.x == 0) atomicExch(work.counters + strip, 0u);
    }
}

// One workgroup per compute unit (at most one per work unit).
template <class Cfg, bool kFp8 = false, bool kQ8 = false, bool kTrans = false>
hipError_t launch_skinny(const GemmArgs &args, const SkinnyWork &work, int cus, hipStream_t stream) {
    const int units = work.num_strips * work.splits;
    const dim3 grid(units < cus ? units : cus), block(Cfg::kThreads);
    dispatch_flags(args.flags, [&](auto f) {
        hipLaunchKernelGGL((gemm_skinny_kernel<Cfg, decltype(f)::value, kFp8, kQ8, kTrans>), grid, block, 0, stream,
                           args, work);
    });
    return hipGetLastError();
}

// The configurations the host plans with: 32-column strips of 64 (or 32)
// rows, K-slices of 256 in A/B rings of 3 and 4 (6 for 32 rows) slices;
// 64-column strips (split K within an XCD), K-slices of 256 in rings of 2/3
// (2/4 for 32 rows); 128-column strips, K-slices of 128.
using SkinnyM64N32 = SkinnyConfig<2, 1, 256, 3, 4>;
using SkinnyM32N32 = SkinnyConfig<1, 1, 256, 3, 6>;
using SkinnyM64N64 = SkinnyConfig<2, 2, 256, 2, 3>;
using SkinnyM64N128 = SkinnyConfig<2, 4, 128, 2, 4>;
using SkinnyM32N64 = SkinnyConfig<1, 2, 256, 2, 4>;
using SkinnyM32N128 = SkinnyConfig<1, 4, 128, 2, 4>;

}  // namespace gb
