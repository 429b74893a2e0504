// kernel_tile.h -- the persistent MFMA GEMM kernel for tile-aligned shapes.
//
// One workgroup per compute unit loops over output tiles (tile_schedule.h).
// For each BM x BN tile of C it runs the K loop:
//
//   HBM/L2 --(buffer_load ... lds, 16 B per lane, coalesced)--> LDS ring of
//   STAGES buffers (XOR-swizzled rows) --(ds_read_b128)--> VGPR fragments
//   --(v_mfma_f32_32x32x16_bf16, or for FP8 E4M3 operands
//      v_mfma_scale_f32_32x32x64_f8f6f4)--> fp32 accumulators in AGPRs
//
// and then the fused epilogue stages the accumulators through LDS and writes
// bf16 C with 16-byte, column-contiguous stores.  FP8 operands (TileConfig's
// ELEM_ = 1) keep the byte layout: a slice of BK values is BK bytes per row,
// so a 128-value FP8 slice has the 128-byte rows of a 64-value bf16 slice.
//
// The decomposition into tiles, K-slices staged through on-chip memory and
// register accumulators is the one of "Outperforming cuBLAS on H100: a
// worklog", section "Recap of Simon's blog", and of the DeepGEMM article
// (demingchina.com), section 2.1; the multi-slice ring plays the role of its
// double buffer (section 3.3) and of the worklog's producer/consumer queue
// ("Kernel 4").  The pages' load path (TMA, mbarriers, producer warpgroups)
// does not exist on gfx950: every wave both issues loads and computes, the
// loads write LDS directly (no VGPR staging), and one workgroup barrier per
// K-slice orders the ring.
//
// Load pacing.  On gfx950 a vector-memory instruction that finds the
// address/data path busy stalls the issuing wave, and with it that wave's
// MFMA stream.  Issuing a slice's loads in a burst therefore costs far more
// than the bytes suggest; spreading them one per four MFMAs and giving each
// load more than two slices to land keeps the matrix cores busy.  So each
// slice's loads are split into two halves: the first half goes out right
// after the barrier that frees its buffer, the second half during the first
// k-step of the next slice, and data is consumed STAGES-1 slices later.
//
// Operand layout in LDS.  A (row-major) and B (column-major, i.e. rows of K
// per output column) are both K-contiguous, so both tiles are stored the
// same way: one row of BK values (kRowBytes bytes) per M (or N) index, split
// into 16-byte chunks.  Chunk c of row r is stored at position c ^ swz(r):
//   128-byte rows (8 chunks): swz(r) = (r & 7) ^ ((r >> 3) & 1)
//    64-byte rows (4 chunks): swz(r) = (r >> 2) & 3
// On gfx950 LDS has 64 four-byte banks and a ds_read_b128 is served in four
// phases of 16 lanes; lanes 0-31 fall into two phases by the parity of lane
// bits 2..4 ({0-3, 12-15, 20-27} and {4-11, 16-19, 28-31}), lanes 32-63 the
// same way (measured with the LDS bank-conflict counter).  A fragment read
// (32 consecutive rows, one logical chunk per half-wave) then touches 16
// distinct 16-byte bank groups in every phase -- the XOR swizzle the DeepGEMM
// article (section 3.2) uses against shared-memory bank conflicts, redone for
// these row widths and this lane-to-phase map.  The direct-to-LDS load
// writes a wave's 64 lanes to 1 KiB of consecutive LDS bytes, so the swizzle
// is applied on the global side: lane i fetches the chunk that belongs at
// its LDS position.
//
// Split-K.  When the tiles alone would leave most compute units idle (a
// 1024 x 1024 output is 64 tiles of 128x128 for 256 compute units), the
// K-slices are cut into `splits` contiguous ranges and a work unit is one
// (range, tile) pair.  When every unit has its own workgroup and each XCD's
// share of them is whole tiles, units are tile-major (u = t * splits + s):
// a tile's ranges then run on one XCD, and the reduction reads them there.
// Otherwise they are range-major (u = s * tiles + t), so the units of one
// range run side by side and share their A rows and B columns in L2.  A
// unit stores its fp32 partial tile to a workspace instead of running the
// epilogue; splitk_reduce_kernel then adds the partials of each element in
// range order (the same order on every run, so results are deterministic)
// and applies the fused epilogue.  It is a second kernel on the same stream:
// the kernel boundary makes the partials visible whichever XCDs wrote them
// (the XCDs' L2s are not coherent with each other).
#pragma once

#include "device_common.h"
#include "epilogue_tile.h"
#include "tile_schedule.h"

namespace gb {

// ELEM_: bytes per operand element, 2 (bf16 on v_mfma_f32_32x32x16_bf16) or
// 1 (FP8 E4M3 on v_mfma_scale_f32_32x32x64_f8f6f4).  BK counts elements, so
// an FP8 slice of 128 has the bytes, loads and LDS layout of a bf16 slice
// of 64 and twice its k.
template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int STAGES_, int ELEM_ = 2>
struct TileConfig {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, STAGES = STAGES_;
    static constexpr int kElem = ELEM_;
    static constexpr bool kFp8 = ELEM_ == 1;
    using Frag = std::conditional_t<kFp8, i32x8, bf16x8>;  // one lane's MFMA operand
    static constexpr int kWaves = WAVES_M * WAVES_N;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int WTM = BM / WAVES_M;  // wave tile
    static constexpr int WTN = BN / WAVES_N;
    static constexpr int FM = WTM / 32;       // 32x32 MFMA blocks per wave
    static constexpr int FN = WTN / 32;
    static constexpr int KSTEPS = BK / (kFp8 ? 64 : 16);  // MFMA k-steps per slice
    static constexpr int kRowBytes = BK * kElem;
    static constexpr int kSwzBK = kRowBytes / 2;           // the LDS swizzle is keyed on the row's bytes
    static constexpr int kChunks = kRowBytes / 16;         // 16-byte chunks per row
    static constexpr int kElemsPerChunk = 16 / kElem;
    static constexpr int kChunkSteps = kRowBytes / 32;     // 32-byte k groups of a row (chunk offsets)
    // ds_read_b128 per k-step: one per bf16 fragment, two per FP8 fragment
    static constexpr int kReadOps = (FM + FN) * (kFp8 ? 2 : 1);
    static constexpr int kReadsPerShadow = kReadOps <= FM * FN ? 1 : 2;
    static constexpr int kReadShadows = (kReadOps + kReadsPerShadow - 1) / kReadsPerShadow;
    static constexpr int kRowsPerLoad = 64 / kChunks;      // rows one 1 KiB wave load fills
    static constexpr int kABytes = BM * kRowBytes;
    static constexpr int kBBytes = BN * kRowBytes;
    static constexpr int kStageBytes = kABytes + kBBytes;
    static constexpr int kLdsBytes = STAGES * kStageBytes;
    static constexpr int kALoads = BM / kRowsPerLoad / kWaves;  // per wave per slice
    static constexpr int kBLoads = BN / kRowsPerLoad / kWaves;
    static constexpr int kLoads = kALoads + kBLoads;
    static constexpr int kHalf = kLoads / 2;
    // epilogue staging: per wave, 32 columns of WTM fp32 rows, padded by 16 B
    static constexpr int kEpiColBytes = WTM * 4 + 16;
    static constexpr int kEpiWaveBytes = 32 * kEpiColBytes;

    static_assert(kRowBytes == 64 || kRowBytes == 128, "swizzles exist for 64- and 128-byte rows");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must hold whole 32x32 blocks");
    static_assert(BM % (kRowsPerLoad * kWaves) == 0 && BN % (kRowsPerLoad * kWaves) == 0,
                  "tile rows must split evenly over the waves' loads");
    static_assert(kLoads % 2 == 0, "loads are issued in two halves");
    static_assert(STAGES >= 3, "a slice's loads land STAGES-1 slices after the first half is issued");
    static_assert((STAGES - 2) * kLoads + kHalf < 64, "vmcnt is a 6-bit counter");
    static_assert(kLdsBytes <= 160 * 1024, "gfx950 has 160 KiB of LDS per compute unit");
    static_assert(kWaves * kEpiWaveBytes <= kLdsBytes, "epilogue staging reuses the ring");
    static_assert(KSTEPS % 2 == 0, "fragment double-buffering alternates per k-step");
    static_assert(kReadShadows <= FM * FN && FM * FN >= kHalf, "MFMA count paces the reads and loads");
};

template <int BK>
__device__ __forceinline__ int lds_swizzle(int row) {
    if constexpr (BK == 64)
        return (row & 7) ^ ((row >> 3) & 1);
    else
        return (row >> 2) & 3;
}

// s_waitcnt vmcnt(n) for a run-time n that is a multiple of kStep, n < 64.
template <int kStep, int kN = 0>
__device__ __forceinline__ void wait_vmcnt_rt(int n) {
    if constexpr (kN + kStep < 64) {
        if (n > kN) {
            wait_vmcnt_rt<kStep, kN + kStep>(n);
            return;
        }
    }
    wait_vmcnt<kN>();
}

// kMasked: the shape has tails (M or N not a multiple of the tile, or K not
// a multiple of BK; K and the leading dimensions multiples of 8).  Every
// 16-byte operand chunk outside the matrix -- row or column past the end,
// or k at or past the unit's K -- is loaded from an out-of-range buffer
// offset, which the DMA turns into zeros (the zero-fill of the DeepGEMM
// article, sections 4.2-4.3), and the epilogue masks its accesses.
template <class Cfg, bool kMasked = false>
struct TileKernel {
    static constexpr int S = Cfg::STAGES;

    // Per-lane state that stays fixed for the whole launch (the masking
    // fields per tile).
    struct Lane {
        uint32_t vA[2], vB[2];            // load voffsets by parity of the row group
        uint32_t aRow, bRow;              // LDS row offsets of this lane's fragments
        uint32_t chunk_off[Cfg::kChunkSteps];  // swizzled chunk offset per 32-byte k group
        uint32_t lda_bytes, ldb_bytes;
        int wave;
        // masking only: this lane's row within a load's rows, its logical
        // chunk by parity of the row group, the tile's valid rows of A and
        // B and the unit's K; per unit, the voffset of each of this wave's
        // loads with rows past M or N already out of range (vAr, vBr), the
        // unit's last slice (klast) and, by parity, the out-of-range bit of
        // this lane's chunk in that slice (kx: 0 or kOobOffset)
        int lrow, lchunk[2];
        int rowsA, rowsB, kmax;
        uint32_t vAr[kMasked ? Cfg::kALoads : 1], vBr[kMasked ? Cfg::kBLoads : 1], kx[2];
        int klast;
    };

    // Per-unit masking state (kMasked): rows and the K tail.  Only the last
    // slice of a unit can hold chunks at or past its K, so a load's voffset
    // in the K loop is its row-masked one, with kx or-ed in when kt is that
    // slice: one vector instruction per load.
    __device__ __forceinline__ static void mask_unit(Lane &L, int nk) {
#pragma unroll
        for (int i = 0; i < Cfg::kALoads; ++i) {
            const int q = L.wave * Cfg::kALoads + i;
            L.vAr[i] = q * Cfg::kRowsPerLoad + L.lrow < L.rowsA ? L.vA[q & 1] : kOobOffset;
        }
#pragma unroll
        for (int i = 0; i < Cfg::kBLoads; ++i) {
            const int q = L.wave * Cfg::kBLoads + i;
            L.vBr[i] = q * Cfg::kRowsPerLoad + L.lrow < L.rowsB ? L.vB[q & 1] : kOobOffset;
        }
        L.klast = __builtin_amdgcn_readfirstlane(nk - 1);
#pragma unroll
        for (int p = 0; p < 2; ++p)
            L.kx[p] = (nk - 1) * Cfg::BK + L.lchunk[p] * Cfg::kElemsPerChunk < L.kmax ? 0u : kOobOffset;
    }

    // The voffset of this lane's chunk in load i of its operand (row group
    // q of the tile) in slice kt: the precomputed one, or (kMasked) an
    // out-of-range offset for rows past the matrix and chunks past the
    // unit's K.
    //
    // kK (masked instances): whether kt is the unit's last slice -- kKAny:
    // decided at run time; kKBefore: known to come before it (rows masked
    // only); kKLast: known to be it.
    enum : int { kKAny = 0, kKBefore = 1, kKLast = 2 };
    template <bool kIsA, int kK = kKAny>
    __device__ __forceinline__ static uint32_t voff(int i, int q, int kt, const Lane &L) {
        if constexpr (kMasked) {
            const uint32_t rows = kIsA ? L.vAr[i] : L.vBr[i];
            if constexpr (kK == kKBefore)
                return rows;
            else if constexpr (kK == kKLast)
                return L.kx[q & 1] | rows;
            else
                return (L.kx[q & 1] & (kt == L.klast ? 0xFFFFFFFFu : 0u)) | rows;
        } else {
            return kIsA ? L.vA[q & 1] : L.vB[q & 1];
        }
    }

    // Loads number LO .. HI-1 of K-slice kt into ring buffer buf.  Loads
    // 0 .. kALoads-1 fill this wave's row groups of A, the rest those of B.
    template <int LO, int HI, int kK = kKAny>
    __device__ __forceinline__ static void issue(char *smem, int buf, int kt, const Lane &L,
                                                 __amdgpu_buffer_rsrc_t rA, __amdgpu_buffer_rsrc_t rB) {
        char *sA = smem + buf * Cfg::kStageBytes;
        char *sB = sA + Cfg::kABytes;
        const uint32_t kbytes = (uint32_t)kt * Cfg::kRowBytes;
#pragma unroll
        for (int idx = LO; idx < HI; ++idx) {
            if (idx < Cfg::kALoads) {
                const int q = L.wave * Cfg::kALoads + idx;  // row group of the tile
                buffer_load_lds16(rA, (GB_LDS void *)(sA + q * 1024), voff<true, kK>(idx, q, kt, L),
                                  (uint32_t)(q * Cfg::kRowsPerLoad) * L.lda_bytes + kbytes);
            } else {
                const int q = L.wave * Cfg::kBLoads + (idx - Cfg::kALoads);
                buffer_load_lds16(rB, (GB_LDS void *)(sB + q * 1024), voff<false, kK>(idx - Cfg::kALoads, q, kt, L),
                                  (uint32_t)(q * Cfg::kRowsPerLoad) * L.ldb_bytes + kbytes);
            }
        }
    }

    using Frag = typename Cfg::Frag;

    __device__ __forceinline__ static f32x16 mfma(const Frag &a, const Frag &b, const f32x16 &c) {
        if constexpr (Cfg::kFp8)
            return mfma_fp8_32x32x64(a, b, c);
        else
            return mfma_32x32x16(a, b, c);
    }

    // Fragment read op r (0 .. kReadOps-1) of MFMA k-step kk of the slice at
    // (sA, sB).  A bf16 fragment (16 k) is one ds_read_b128: lane l takes
    // row l % 32 of its 32-row block and logical chunk 2kk + l/32.  An FP8
    // fragment (64 k) is two: its low 16 bytes from chunk 4kk + l/32 and its
    // high 16 bytes from chunk 4kk + 2 + l/32, the operand layout of the
    // 32x32x64 MFMA -- i.e. the chunks of bf16 k-steps 2kk and 2kk + 1.
    // Fragments go A0, B0, A1, B1, ... while both remain, then the rest of A.
    __device__ __forceinline__ static void read_op(const char *sA, const char *sB, int kk, int r, const Lane &L,
                                                   Frag (&a)[Cfg::FM], Frag (&b)[Cfg::FN]) {
        constexpr int kHalves = Cfg::kFp8 ? 2 : 1;
        const int fr = r / kHalves, half = r % kHalves;
        const bool is_a = fr < 2 * Cfg::FN ? (fr & 1) == 0 : true;
        const int f = fr < 2 * Cfg::FN ? fr >> 1 : fr - Cfg::FN;
        const uint32_t off = L.chunk_off[kHalves * kk + half];
        const char *src = is_a ? sA + L.aRow : sB + L.bRow;
        Frag &dst = is_a ? a[f] : b[f];
        if constexpr (Cfg::kFp8) {
            const i32x4 v = *(const GB_LDS i32x4 *)(src + f * 32 * Cfg::kRowBytes + off);
            if (half)
                dst.hi = v;
            else
                dst.lo = v;
        } else {
            dst = *(const GB_LDS bf16x8 *)(src + f * 32 * Cfg::kRowBytes + off);
        }
    }

    // All fragments of MFMA k-step kk of the slice in ring buffer buf.
    __device__ __forceinline__ static void read_frags(const char *smem, int buf, int kk, const Lane &L,
                                                      Frag (&a)[Cfg::FM], Frag (&b)[Cfg::FN]) {
        const char *sA = smem + buf * Cfg::kStageBytes;
        const char *sB = sA + Cfg::kABytes;
#pragma unroll
        for (int r = 0; r < Cfg::kReadOps; ++r) read_op(sA, sB, kk, r, L, a, b);
    }

    // One k-step: the FM x FN MFMAs on (a, b), issued one at a time, with the
    // other work of the k-step placed in the 32-cycle shadows between them:
    // after MFMA number s goes out (if kRead) fragment read s of k-step rkk of
    // ring buffer rbuf (A0, B0, A1, B1, ... into ra, rb: all reads in the
    // first FM + FN shadows, so they have landed long before the k-step
    // ends), and (if kLoad) the DMA loads LO .. LO + kHalf - 1 of slice lkt
    // into ring buffer lbuf, spread evenly over the remaining shadows.  A wave
    // has one MFMA in flight at a time, so an MFMA shadow that holds more
    // issue work than the MFMA's own 32 cycles leaves the matrix core idle;
    // one read or one load per shadow stays under that.  Hard scheduling
    // fences keep this order.
    template <bool kRead, bool kLoad, int LO, int kK = kKAny>
    __device__ __forceinline__ static void kstep(char *smem, const Frag (&a)[Cfg::FM], const Frag (&b)[Cfg::FN],
                                                 f32x16 (&acc)[Cfg::FM][Cfg::FN], int rbuf, int rkk,
                                                 Frag (&ra)[Cfg::FM], Frag (&rb)[Cfg::FN], int lbuf, int lkt,
                                                 const Lane &L, __amdgpu_buffer_rsrc_t rA,
                                                 __amdgpu_buffer_rsrc_t rB) {
        constexpr int kMf = Cfg::FM * Cfg::FN;
        constexpr int kLoadsHere = Cfg::kHalf;
        constexpr int kRps = Cfg::kReadsPerShadow;
        // first shadow of load l: after the reads if they leave room, else shared with them
        constexpr int kFree = kMf - Cfg::kReadShadows;
        const char *sA = smem + rbuf * Cfg::kStageBytes;
        const char *sB = sA + Cfg::kABytes;
#pragma unroll
        for (int s = 0; s < kMf; ++s) {
            const int p = s / Cfg::FN, j = s % Cfg::FN;
            acc[p][j] = mfma(a[p], b[j], acc[p][j]);
            __builtin_amdgcn_sched_barrier(0);
            if (kRead) {
#pragma unroll
                for (int u = 0; u < kRps; ++u)
                    if (s * kRps + u < Cfg::kReadOps) read_op(sA, sB, rkk, s * kRps + u, L, ra, rb);
            }
            if (kLoad) {
#pragma unroll
                for (int l = 0; l < kLoadsHere; ++l) {
                    const int slot = (kFree >= kLoadsHere) ? Cfg::kReadShadows + l * kFree / kLoadsHere
                                                           : l * kMf / kLoadsHere;
                    if (slot == s) issue_range<LO, kK>(smem, lbuf, lkt, L, rA, rB, l, 1);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // kCount loads starting at number LO + first (first is a compile-time
    // constant after unrolling).
    template <int LO, int kK = kKAny>
    __device__ __forceinline__ static void issue_range(char *smem, int buf, int kt, const Lane &L,
                                                       __amdgpu_buffer_rsrc_t rA, __amdgpu_buffer_rsrc_t rB,
                                                       int first, int count) {
        char *sA = smem + buf * Cfg::kStageBytes;
        char *sB = sA + Cfg::kABytes;
        const uint32_t kbytes = (uint32_t)kt * Cfg::kRowBytes;
#pragma unroll
        for (int r = 0; r < count; ++r) {
            const int idx = LO + first + r;
            if (idx < Cfg::kALoads) {
                const int q = L.wave * Cfg::kALoads + idx;
                buffer_load_lds16(rA, (GB_LDS void *)(sA + q * 1024), voff<true, kK>(idx, q, kt, L),
                                  (uint32_t)(q * Cfg::kRowsPerLoad) * L.lda_bytes + kbytes);
            } else {
                const int q = L.wave * Cfg::kBLoads + (idx - Cfg::kALoads);
                buffer_load_lds16(rB, (GB_LDS void *)(sB + q * 1024), voff<false, kK>(idx - Cfg::kALoads, q, kt, L),
                                  (uint32_t)(q * Cfg::kRowsPerLoad) * L.ldb_bytes + kbytes);
            }
        }
    }

    // One K-slice kt (in ring buffer cur) of the software pipeline.
    //   first:  issue the first half of slice kt+S's loads (into cur, once
    //           the barrier has freed it);
    //   second: issue the second half of slice kt+S-1's loads (into the
    //           buffer freed by the previous slice);
    //   ahead:  loads issued after slice kt+1's, still allowed in flight at
    //           the barrier;
    //   kNext:  a slice kt+1 exists.
    // kSteady: first = second = true and ahead = (S-2) * loads per slice, all
    // known at compile time; otherwise (the last few slices of a tile) they
    // are run-time values and the loads of those steps are issued in a burst.
    // While the MFMAs of k-step kk run, the fragments of kk+1 are read.
    // Before the last k-step every wave waits for slice kt+1, passes the
    // barrier (all waves have then finished reading slice kt) and reads
    // slice kt+1's first fragments during the last k-step's MFMAs.
    template <bool kSteady, bool kNext, int kK1 = kKAny, int kK2 = kKAny>
    __device__ __forceinline__ static void slice(char *smem, int kt, int cur, bool first, bool second, int ahead,
                                                 const Lane &L, __amdgpu_buffer_rsrc_t rA,
                                                 __amdgpu_buffer_rsrc_t rB, Frag (&fa)[2][Cfg::FM],
                                                 Frag (&fb)[2][Cfg::FN], f32x16 (&acc)[Cfg::FM][Cfg::FN]) {
        const int prev = (cur == 0) ? S - 1 : cur - 1;
        const int next = (cur + 1 == S) ? 0 : cur + 1;
        if (!kSteady && second) issue<Cfg::kHalf, Cfg::kLoads>(smem, prev, kt + S - 1, L, rA, rB);
#pragma unroll
        for (int kk = 0; kk < Cfg::KSTEPS - 1; ++kk) {
            if (kSteady && kk == 0)
                kstep<true, true, Cfg::kHalf, kK2>(smem, fa[0], fb[0], acc, cur, kk + 1, fa[1], fb[1], prev,
                                               kt + S - 1, L, rA, rB);
            else
                kstep<true, false, 0>(smem, fa[kk & 1], fb[kk & 1], acc, cur, kk + 1, fa[(kk + 1) & 1],
                                      fb[(kk + 1) & 1], 0, 0, L, rA, rB);
        }
        constexpr int kLast = (Cfg::KSTEPS - 1) & 1;
        if constexpr (kNext) {
            if constexpr (kSteady)
                wait_vmcnt<(S - 2) * Cfg::kLoads>();
            else
                wait_vmcnt_rt<Cfg::kHalf>(ahead);
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (kSteady) {
                kstep<true, true, 0, kK1>(smem, fa[kLast], fb[kLast], acc, next, 0, fa[0], fb[0], cur, kt + S, L, rA,
                                     rB);
            } else {
                if (first) issue<0, Cfg::kHalf>(smem, cur, kt + S, L, rA, rB);
                kstep<true, false, 0>(smem, fa[kLast], fb[kLast], acc, next, 0, fa[0], fb[0], 0, 0, L, rA, rB);
            }
        } else {
            kstep<false, false, 0>(smem, fa[kLast], fb[kLast], acc, 0, 0, fa[0], fb[0], 0, 0, L, rA, rB);
        }
    }
};

// Requirements checked by the host before launch: M % BM == 0, N % BN == 0,
// K % BK == 0, K > 0, A/B/C 16-byte aligned, lda/ldb/ldc multiples of 8, and
// BM*lda*2 + 2K, BN*ldb*2 + 2K below 2^31 (32-bit buffer offsets).
// Store a wave's accumulators as fp32 partial sums: a 32x32 MFMA result
// gives lane l column l % 32 and, in registers 4g..4g+3, rows
// 8g + 4(l/32) + 0..3, one 16-byte store each.
template <class Cfg>
__device__ __forceinline__ void tile_store_partial(const TileSplit &split, int s, int64_t m0, int64_t n0, int wm,
                                                   int wn, int lane, const f32x16 (&acc)[Cfg::FM][Cfg::FN]) {
    float *base = split.P + (int64_t)s * split.pstride;
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
        const int64_t n = n0 + wn * Cfg::WTN + j * 32 + (lane & 31);
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t m = m0 + wm * Cfg::WTM + i * 32 + g * 8 + (lane >> 5) * 4;
                const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                *(f32x4 *)(base + n * split.ldp + m) = v;
            }
    }
}

// kSplit: the units are (K range, tile) pairs and each stores its partial
// (kFlags is then unused: the reduction applies the epilogue).  kMasked:
// any M, N >= 1 and K % 8 == 0 (tails zero-filled and masked); a masked
// split stores whole tiles into a workspace padded to tile multiples
// (split.ldp, split.pstride), the rows and columns past the matrix holding
// zeros.
template <class Cfg, uint32_t kFlags, bool kSplit = false, bool kMasked = false>
__global__ void __launch_bounds__(Cfg::kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_tile_kernel(const GemmArgs args, const TileSchedule sched, const TileSplit split) {
    using TK = TileKernel<Cfg, kMasked>;
    constexpr int S = Cfg::STAGES;
    constexpr int L = Cfg::kLoads;
    constexpr int H = Cfg::kHalf;
    __shared__ __attribute__((aligned(1024))) char smem[Cfg::kLdsBytes];

    const int lane = threadIdx.x & 63;
    typename TK::Lane Ln;
    Ln.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = Ln.wave / Cfg::WAVES_N;
    const int wn = Ln.wave % Cfg::WAVES_N;
    Ln.lda_bytes = (uint32_t)(args.lda * Cfg::kElem);
    Ln.ldb_bytes = (uint32_t)(args.ldb * Cfg::kElem);

    // Load side: in row group q, lane i covers row q*kRowsPerLoad + i/kChunks
    // and LDS position i%kChunks, which holds logical chunk (i%kChunks) ^
    // swz(row).  swz only sees the row's low bits, which the parity of q and
    // the lane fix, so two offsets per operand suffice.
    const int lrow = lane / Cfg::kChunks, lpos = lane % Cfg::kChunks;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int c = lpos ^ lds_swizzle<Cfg::kSwzBK>(p * Cfg::kRowsPerLoad + lrow);
        Ln.vA[p] = lrow * Ln.lda_bytes + (uint32_t)(c << 4);
        Ln.vB[p] = lrow * Ln.ldb_bytes + (uint32_t)(c << 4);
        Ln.lchunk[p] = c;
    }
    Ln.lrow = lrow;
    Ln.rowsA = Ln.rowsB = Ln.kmax = 0;
    // Read side: MFMA operand lane l takes row l % 32 of its 32-row block;
    // in 32-byte k group kk its 16 bytes are logical chunk 2*kk + l/32
    // (read_op: one group per bf16 k-step, two per FP8 k-step).
    Ln.aRow = (uint32_t)(wm * Cfg::WTM + (lane & 31)) * Cfg::kRowBytes;
    Ln.bRow = (uint32_t)(wn * Cfg::WTN + (lane & 31)) * Cfg::kRowBytes;
#pragma unroll
    for (int kk = 0; kk < Cfg::kChunkSteps; ++kk)
        Ln.chunk_off[kk] = (uint32_t)(((2 * kk + (lane >> 5)) ^ lds_swizzle<Cfg::kSwzBK>(lane & 31)) << 4);

    const int nk_all = (int)((args.K + Cfg::BK - 1) / Cfg::BK);
    const int num_tiles = sched.num_tiles();
    const int num_units = kSplit ? num_tiles * split.splits : num_tiles;

    for (int u = sched.slot(blockIdx.x); u < num_units; u += sched.grid) {
        int t = u, s = 0, nk = nk_all;
        if constexpr (kSplit) {
            if (split.tile_major) {
                t = u / split.splits;
                s = u - t * split.splits;
            } else {
                s = u / num_tiles;
                t = u - s * num_tiles;
            }
            const int rest = nk_all - s * split.kper;
            nk = rest < split.kper ? rest : split.kper;
        }
        int tm, tn;
        sched.tile(t, tm, tn);
        const int64_t m0 = (int64_t)tm * Cfg::BM;
        const int64_t n0 = (int64_t)tn * Cfg::BN;
        const int64_t k0 = kSplit ? (int64_t)s * split.kper * Cfg::BK : 0;
        const int64_t kn = (int64_t)nk * Cfg::BK;
        if constexpr (kMasked) {
            Ln.rowsA = (int)(args.M - m0 < Cfg::BM ? args.M - m0 : Cfg::BM);
            Ln.rowsB = (int)(args.N - n0 < Cfg::BN ? args.N - n0 : Cfg::BN);
            Ln.kmax = (int)(args.K - k0);  // the unit's K: chunks at or past it are zeros
            TK::mask_unit(Ln, nk);
        }
        const char *A = reinterpret_cast<const char *>(args.A);
        const char *B = reinterpret_cast<const char *>(args.B);
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(A + (m0 * args.lda + k0) * Cfg::kElem,
                                                    (uint32_t)(((Cfg::BM - 1) * args.lda + kn) * Cfg::kElem));
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(B + (n0 * args.ldb + k0) * Cfg::kElem,
                                                    (uint32_t)(((Cfg::BN - 1) * args.ldb + kn) * Cfg::kElem));

        f32x16 acc[Cfg::FM][Cfg::FN];
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = f32x16{};

        // The previous tile's epilogue is done with LDS.
        lds_barrier();
        // Prologue: slices 0 .. S-2 and the first half of slice S-1 in
        // flight; once slice 0 has landed everywhere its first fragments are
        // read.
        typename Cfg::Frag fa[2][Cfg::FM], fb[2][Cfg::FN];
#pragma unroll
        for (int s = 0; s < S - 1; ++s)
            if (s < nk) TK::template issue<0, L>(smem, s, s, Ln, rA, rB);
        if (S - 1 < nk) TK::template issue<0, H>(smem, S - 1, S - 1, Ln, rA, rB);
        wait_vmcnt_rt<H>((nk - 1 < S - 2 ? nk - 1 : S - 2) * L + (S - 1 < nk ? H : 0));
        lds_barrier();
        TK::read_frags(smem, 0, 0, Ln, fa[0], fb[0]);
        // Drain every LGKM operation once per tile (a real s_waitcnt the
        // compiler sees), so at the loop head only the pipeline's own LDS
        // reads are pending and its waits stay exact.
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);

        int kt = 0, cur = 0;
        if constexpr (kMasked) {
            // Steady slices load slice kt + S (first half) and kt + S - 1
            // (second half): before the unit's last slice while
            // kt + S + 1 < nk, then one that loads the last one's first half.
            for (; kt + S + 1 < nk; ++kt) {
                TK::template slice<true, true, TK::kKBefore, TK::kKBefore>(smem, kt, cur, true, true, 0, Ln, rA,
                                                                            rB, fa, fb, acc);
                cur = (cur + 1 == S) ? 0 : cur + 1;
            }
            if (kt + S < nk) {
                TK::template slice<true, true, TK::kKLast, TK::kKBefore>(smem, kt, cur, true, true, 0, Ln, rA, rB,
                                                                          fa, fb, acc);
                ++kt;
                cur = (cur + 1 == S) ? 0 : cur + 1;
            }
        } else {
            for (; kt + S < nk; ++kt) {
                TK::template slice<true, true>(smem, kt, cur, true, true, 0, Ln, rA, rB, fa, fb, acc);
                cur = (cur + 1 == S) ? 0 : cur + 1;
            }
        }
        for (; kt + 1 < nk; ++kt) {
            // loads issued after slice kt+1's: slices kt+2 .. min(kt+S-1, nk-1)
            const int last = (kt + S - 1 < nk - 1) ? kt + S - 1 : nk - 1;
            TK::template slice<false, true>(smem, kt, cur, false, kt + S - 1 < nk, (last - (kt + 1)) * L, Ln, rA,
                                            rB, fa, fb, acc);
            cur = (cur + 1 == S) ? 0 : cur + 1;
        }
        TK::template slice<false, false>(smem, kt, cur, false, false, 0, Ln, rA, rB, fa, fb, acc);

        if constexpr (kSplit) {
            tile_store_partial<Cfg>(split, s, m0, n0, wm, wn, lane, acc);
        } else {
            // Every wave is done reading the ring (all loads landed at the
            // last wait): its memory now stages the epilogue.
            lds_barrier();
            tile_epilogue<Cfg, kFlags, kMasked>(smem, args, m0, n0, wm, wn, lane, Ln.wave, acc);
        }
    }
}

// The split-K reduction: thread i takes 8 consecutive rows of one column,
// adds the splits' partials in range order, multiplies by the fp8 scales
// when the call has them, applies alpha, beta*C, bias and
// the activation in fp32 and writes one 16-byte run of bf16 C -- or, with
// kQ8, quantizes the 8 values with their rows' scales and writes 8 bytes of
// int8 Q.  Requires M % 8 == 0, C 16-byte aligned and ldc % 8 == 0 (when C
// is read or written), and for kQ8 the scale 16-byte aligned (checked on
// the host) -- except that masked splits handle any M, C, ldc, Q and ldq.
//
// Which thread takes which chunk.  Without tile_major, chunk idx of the
// column-major chunk order (grid-stride).  With tile_major (kTileM x kTileN
// tiles, the split units of a tile consecutive, so on one XCD: the host
// launched one tile kernel workgroup per unit, a multiple of 8 of them, each
// XCD's share holding whole tiles), block b reduces part of a tile of the
// units on XCD b mod 8 -- the same XCD under the round-robin dispatch of
// workgroups to XCDs, so its partials are read from that XCD's L2 where they
// are still held.  Both mappings give the same sums in the same order.
template <uint32_t kFlags, bool kQ8 = false, int kTileM = 128, int kTileN = 128>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const GemmArgs args, const TileSplit split,
                                                            const TileSchedule sched) {
    constexpr int kTileChunks = kTileM / 8 * kTileN;  // 8-row chunks of a tile
    constexpr int kBlocksPerTile = kTileChunks / 256;
    static_assert(kTileChunks % 256 == 0, "whole blocks per tile");
    const int64_t chunks_m = (args.M + 7) / 8;
    int64_t total = chunks_m * args.N, step = (int64_t)gridDim.x * 256;
    int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    int64_t tm0 = 0, tn0 = 0;
    if (split.tile_major) {
        const int x = blockIdx.x % kNumXcds, j = blockIdx.x / kNumXcds;
        const int tiles_per_xcd = sched.grid / kNumXcds / split.splits;
        const int t = x * tiles_per_xcd + j / kBlocksPerTile;
        int tm, tn;
        sched.tile(t, tm, tn);
        tm0 = (int64_t)tm * kTileM;
        tn0 = (int64_t)tn * kTileN;
        idx = (int64_t)(j % kBlocksPerTile) * 256 + threadIdx.x;  // chunk within the tile
        total = idx + 1;  // one chunk per thread
        step = 1;
    }
    for (; idx < total; idx += step) {
        int64_t n, m;
        if (split.tile_major) {
            n = tn0 + idx / (kTileM / 8);
            m = tm0 + (idx % (kTileM / 8)) * 8;
            if (n >= args.N || m >= args.M) break;  // past the matrix in a tail tile
        } else {
            n = idx / chunks_m;
            m = (idx - n * chunks_m) * 8;
        }
        // Loads of four ranges go out before their sums, so the memory
        // latency is paid once per four ranges; the adds keep range order.
        const float *p = split.P + n * split.ldp + m;
        f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
        int s = 0;
        for (; s + 4 <= split.splits; s += 4) {
            f32x4 l[4], h[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                l[u] = *(const f32x4 *)(p + (int64_t)(s + u) * split.pstride);
                h[u] = *(const f32x4 *)(p + (int64_t)(s + u) * split.pstride + 4);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                lo += l[u];
                hi += h[u];
            }
        }
        for (; s < split.splits; ++s) {
            lo += *(const f32x4 *)(p + (int64_t)s * split.pstride);
            hi += *(const f32x4 *)(p + (int64_t)s * split.pstride + 4);
        }
        // a chunk that straddles M, or any chunk when ldc % 8 != 0 or C is
        // not 16-byte aligned (masked splits only), is read and written
        // element by element; partials past M are zeros in the padding
        const bool full = m + 8 <= args.M && (args.ldc & 7) == 0 && (reinterpret_cast<uintptr_t>(args.C) & 15) == 0;
        uint16_t *c = args.C + n * args.ldc + m;
        float bias_v = 0.f;
        if constexpr ((kFlags & kEpiBias) != 0) bias_v = bf16_bits_to_f32(args.bias[n]);
        float cin[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if constexpr ((kFlags & kEpiBeta) != 0) {
            if (full) {
                const u32x4 raw = *(const u32x4 *)c;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    cin[2 * e] = bf16_bits_to_f32(raw[e] & 0xFFFFu);
                    cin[2 * e + 1] = bf16_bits_to_f32(raw[e] >> 16);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) if (m + e < args.M) cin[e] = bf16_bits_to_f32(c[e]);
            }
        }
        float x[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        // fp8 inputs: the sum times scale_a[m] and scale_b[n] (NULL = 1), as
        // in the fp8 tile kernel's own epilogue
        if (args.scale_a) {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = x[e] * (m + e < args.M ? args.scale_a[m + e] : 0.f);
        }
        if (args.scale_b) {
            const float sb = args.scale_b[n];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = x[e] * sb;
        }
        if constexpr (kQ8) {
            // A chunk that straddles M (masked splits only) loads its rows'
            // scales one by one, 0 past M, and stores its bytes one by one,
            // as does every chunk when ldq % 8 != 0 or Q is not 8-byte
            // aligned; whole chunks load their 8 scales as two 16-byte loads.
            float sc[8];
            if (m + 8 <= args.M) {
                const f32x4 s_lo = *(const f32x4 *)(args.scale + m);
                const f32x4 s_hi = *(const f32x4 *)(args.scale + m + 4);
                sc[0] = s_lo.x; sc[1] = s_lo.y; sc[2] = s_lo.z; sc[3] = s_lo.w;
                sc[4] = s_hi.x; sc[5] = s_hi.y; sc[6] = s_hi.z; sc[7] = s_hi.w;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) sc[e] = m + e < args.M ? args.scale[m + e] : 0.f;
            }
            u32x2 qw = {0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = epilogue_value<kFlags>(x[e], cin[e], bias_v, args.alpha, args.beta);
                qw[e >> 2] |= ((uint32_t)quantize_i8(v, sc[e], args.zp) & 0xFFu) << ((e & 3) * 8);
            }
            int8_t *q = args.Q + n * args.ldq + m;
            if (m + 8 <= args.M && (args.ldq & 7) == 0 && (reinterpret_cast<uintptr_t>(args.Q) & 7) == 0) {
                __builtin_nontemporal_store(qw, (u32x2 *)q);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) if (m + e < args.M) q[e] = (int8_t)(qw[e >> 2] >> ((e & 3) * 8));
            }
        } else {
            u32x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[e] = pack_bf16x2(
                    epilogue_value<kFlags>(x[2 * e], cin[2 * e], bias_v, args.alpha, args.beta),
                    epilogue_value<kFlags>(x[2 * e + 1], cin[2 * e + 1], bias_v, args.alpha, args.beta));
            if (full) {
                __builtin_nontemporal_store(out, (u32x4 *)c);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) if (m + e < args.M) c[e] = (uint16_t)(out[e >> 1] >> ((e & 1) * 16));
            }
        }
    }
}

// Launch the tile kernel of configuration Cfg with the epilogue flags of
// args baked in.  The grid is min(tiles, compute units): one persistent
// workgroup per compute unit.
template <class Cfg, bool kMasked = false>
hipError_t launch_tile(const GemmArgs &args, int cus, hipStream_t stream) {
    TileSchedule s{};
    s.tiles_m = (int)((args.M + Cfg::BM - 1) / Cfg::BM);
    s.tiles_n = (int)((args.N + Cfg::BN - 1) / Cfg::BN);
    s.group_m = 4;
    const int tiles = s.num_tiles();
    s.grid = tiles < cus ? tiles : cus;
    const dim3 grid(s.grid), block(Cfg::kThreads);
    const TileSplit none{};
    dispatch_flags(args.flags, [&](auto f) {
        hipLaunchKernelGGL((gemm_tile_kernel<Cfg, decltype(f)::value, false, kMasked>), grid, block, 0, stream, args,
                           s, none);
    });
    return hipGetLastError();
}

// Split-K launch: the tile kernel over (range, tile) units into the
// workspace split.P, then the reduction with the epilogue flags baked in
// (kQ8: writing int8 Q).  The host has checked the tile-path requirements,
// split.splits >= 1 (one range: the int8 output over the whole of K, the
// reduction only running the epilogue), every range non-empty, and that
// split.P holds
// splits * pstride floats (ldp = M rounded up to BM, pstride = ldp times N
// rounded up to BN; exact shapes: M and M * N).
template <class Cfg, bool kQ8 = false, bool kMasked = false>
hipError_t launch_tile_splitk(const GemmArgs &args, const TileSplit &split, int cus, hipStream_t stream) {
    TileSchedule s{};
    s.tiles_m = (int)((args.M + Cfg::BM - 1) / Cfg::BM);
    s.tiles_n = (int)((args.N + Cfg::BN - 1) / Cfg::BN);
    s.group_m = 4;
    const int units = s.num_tiles() * split.splits;
    s.grid = units < cus ? units : cus;
    hipLaunchKernelGGL((gemm_tile_kernel<Cfg, 0u, true, kMasked>), dim3(s.grid), dim3(Cfg::kThreads), 0, stream, args,
                       s, split);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t threads = (args.M + 7) / 8 * args.N;
    const int64_t blocks = (threads + 255) / 256;
    const int64_t cap = (int64_t)cus * 8;
    // tile_major: one block per 256 chunks of every tile, in XCD order
    const int64_t tile_blocks = (int64_t)s.num_tiles() * (Cfg::BM / 8 * Cfg::BN / 256);
    const dim3 rgrid((unsigned)(split.tile_major ? tile_blocks : (blocks < cap ? blocks : cap)));
    dispatch_flags(args.flags, [&](auto f) {
        hipLaunchKernelGGL((splitk_reduce_kernel<decltype(f)::value, kQ8, Cfg::BM, Cfg::BN>), rgrid, dim3(256), 0,
                           stream, args, split, s);
    });
    return hipGetLastError();
}

}  // namespace gb
