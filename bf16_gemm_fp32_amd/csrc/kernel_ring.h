// kernel_ring.h -- persistent 256x256 MFMA tile kernel with K-slices of 64:
// every operand row of a slice is one full 128-byte line, LDS is a ring of
// five 32 KiB single-operand units, and the products run on
// v_mfma_f32_16x16x32_bf16.
//
// Why 128-byte rows.  Loading 64-byte row segments (K-slices of 32) makes
// the L2 deliver whole 128-byte lines for half-line requests: twice the
// L2->CU traffic, and on a power-limited chip that traffic costs clock.
//
// Why a ring of units.  One 64-wide slice of the 256x256 tile is 64 KiB, so
// 160 KiB of LDS holds two and a half slices.  Each slice is split into its
// A unit and its B unit (256 rows x 128 bytes each); A(j) of slice j lives in
// ring slot (2j) % 5, B(j) in (2j+1) % 5, so loads start as soon as any unit
// is free.  One barrier per slice, before its last k-step: every wave has
// then read its last fragments of slice j into registers (A(j)'s and B(j)'s
// slots are free) and slice j+1's units are published.  Between the barrier
// of slice j and that of slice j+1 a wave issues B(j+2) (during k-step 1 of
// slice j, into A(j)'s slot) and A(j+3) (during k-step 0 of slice j+1, into
// B(j)'s slot); at the barrier of slice j+1 only A(j+3)'s loads may still be
// in flight.
//
// Why 16x16x32 MFMAs.  Per flop the 16x16 form reads and writes half as many
// accumulator bytes as 32x32x16; on this power-limited part a pure-MFMA loop
// holds ~2.2 GHz with it against ~1.85 GHz with 32x32x16, and this kernel
// runs ~7% faster than the same ring on 32x32x16 (kernel_ring_mfma32.h).
//
//   HBM/L2 --(buffer_load_dwordx4 ... lds, direct DMA)--> LDS unit slots
//   LDS --(ds_read_b128, XOR-swizzled 128-byte rows)--> VGPR fragments
//   fragments --(v_mfma_f32_16x16x32_bf16)--> 256 fp32 accumulators (AGPRs)
//
// Per wave: a 128x128 tile = 8 x 8 blocks of 16x16, 64 accumulators of 4 fp32;
// a slice is two k-steps of 32, each 64 MFMAs fed by 8 A and 8 B fragments
// (ds_read_b128: row l % 16 of the block, k-chunk l / 16 of the k-step).
// Within a k-step the MFMAs go out one at a time; the 16-cycle shadow after
// MFMA s carries fragment read s for s < 16 (A0, B0, A1, B1, ...), and the
// unit's 8 DMA loads sit in shadows 16, 22, ..., 58.
//
// LDS rows (8 chunks of 16 bytes) store chunk c at c ^ swz(r) with
// swz(r) = (r >> 1) & 7.  On gfx950 a ds_read_b128 is served in four 16-lane
// phases (lanes 0-31 split by the parity of lane bits 2..4, lanes 32-63 the
// same way); with this swizzle a fragment read (16 rows x 4 chunks) touches
// 16 distinct 16-byte bank groups in every phase.  The DMA writes a wave's
// 64 lanes to 1 KiB of consecutive LDS bytes (8 rows of 128 bytes), so the
// swizzle is applied on the global side: lane i fetches the chunk that
// belongs at its LDS position.  This is the XOR swizzle of the DeepGEMM
// article (section 3.2), redone for this row width and lane-to-phase map.
#pragma once

#include <cstdlib>

#include "device_common.h"
#include "tile_schedule.h"

namespace gb {


// kWavesN: waves across the tile's columns (two down its rows).  2 gives
// four waves of 128x128, one per SIMD, 256 accumulators each; 4 gives eight
// waves of 128x64, two per SIMD, 128 accumulators each, so one wave's
// fragment reads, DMA issue and barrier waits can run under the other's
// MFMAs, at 1.5x the LDS fragment reads per slice.
template <int kWavesN>
struct RingConfigT {
    static constexpr int BM = 256, BN = 256, BK = 64;
    static constexpr int WAVES_M = 2, WAVES_N = kWavesN;
    static constexpr int kWaves = WAVES_M * WAVES_N;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // wave tile
    static constexpr int FM = WTM / 16, FN = WTN / 16;            // 16x16 MFMA blocks per wave
    static constexpr int KSTEPS = BK / 32;                        // MFMA k-steps per slice
    static constexpr int kMfmas = FM * FN;                        // MFMAs per wave per k-step
    static constexpr int kReads = FM + FN;                        // fragment reads per wave per k-step
    static constexpr int kRowBytes = BK * 2;                      // 128: one cache line
    static constexpr int kUnitBytes = BM * kRowBytes;             // one operand of one slice
    static constexpr int kSlots = 5;
    static constexpr int kLdsBytes = kSlots * kUnitBytes;
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;         // rows one wave DMA fills
    static constexpr int kUnitLoads = BM / kRowsPerLoad / kWaves; // DMA loads per wave per unit
    // The shadows (MFMA indices within a k-step) of a unit's DMA loads.
    static constexpr int kLoadStart = kWaves == 4 ? 16 : kReads + 1;
    static constexpr int kLoadStep = kWaves == 4 ? 6 : (kMfmas - kLoadStart) / kUnitLoads;
    static constexpr int kEpiColBytes = WTM * 4 + 16;
    static constexpr int kEpiWaveBytes = 32 * kEpiColBytes;
    // Epilogue staging in slots 0-2 leaves slots 3-4 for the next tile's
    // A(0), B(0); otherwise the staging takes the whole ring and the next
    // tile's loads wait for it.
    static constexpr bool kEpiInRing = kWaves * kEpiWaveBytes <= 3 * kUnitBytes;

    static_assert(BM == BN, "A and B units have the same size");
    static_assert(KSTEPS == 2, "the slice schedule below is written for 2 k-steps per slice");
    static_assert(FN <= FM && kReads <= kMfmas, "one fragment read per MFMA shadow");
    static_assert(kUnitLoads % 2 == 0 && kLoadStep >= 1 && kLoadStart >= kReads &&
                      kLoadStart + (kUnitLoads - 1) * kLoadStep < kMfmas,
                  "a unit's loads fit in the shadows after the reads, in row groups of both parities");
    static_assert(kLdsBytes <= 160 * 1024, "gfx950 has 160 KiB of LDS per compute unit");
    static_assert(kWaves * kEpiWaveBytes <= kLdsBytes, "epilogue staging fits in LDS");
};
using RingConfig = RingConfigT<2>;
using RingConfigW8 = RingConfigT<4>;
static_assert(RingConfig::kEpiInRing, "the four-wave ring stages its epilogue in slots 0-2");

__device__ __forceinline__ int ring_swizzle(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ int ring_slot(int s) { return s >= RingConfig::kSlots ? s - RingConfig::kSlots : s; }

__device__ __forceinline__ f32x4 mfma_16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// kMasked: the shape has tails (M or N not a multiple of 256, or K not a
// multiple of 64; K and the leading dimensions are multiples of 8).  Every
// 16-byte operand chunk outside the matrix -- row or column past the end,
// or k >= K -- is loaded from an out-of-range buffer offset, which the DMA
// turns into zeros (the zero-fill of the DeepGEMM article, sections 4.2-4.3),
// and the epilogue masks its loads and stores.  Unmasked instances carry no
// such code.
template <bool kMasked, class Cfg = RingConfig>
struct RingKernel {
    struct Lane {
        uint32_t vA[2], vB[2];    // load voffsets by parity of the 8-row group
        uint32_t aRow, bRow;      // LDS offsets (within a unit) of this lane's fragment rows
        uint32_t chunk_off[Cfg::KSTEPS];
        uint32_t lda_bytes, ldb_bytes;
        int wave;
        // masking only: this lane's row within a load's 8 rows, its logical
        // chunk by parity of the row group, and the tile's valid extents;
        // per tile, the voffset of each of this wave's loads of a unit with
        // rows past M or N already out of range (vAr, vBr); the last slice
        // (klast) and, by parity, the out-of-range bit of this lane's chunk
        // in that slice (kx: 0 or kOobOffset)
        int lrow, lchunk[2];
        int rowsA, rowsB, kmax;
        uint32_t vAr[kMasked ? Cfg::kUnitLoads : 1], vBr[kMasked ? Cfg::kUnitLoads : 1], kx[2];
        int klast;
    };

    // Masking state (kMasked): the K tail once per launch, the rows once per
    // tile.  Only the last slice can hold chunks at or past K, so a load's
    // voffset in the K loop is its row-masked one, with kx or-ed in when kt
    // is that slice: one vector instruction per load.
    __device__ __forceinline__ static void mask_k(Lane &L, int nk) {
        L.klast = __builtin_amdgcn_readfirstlane(nk - 1);
#pragma unroll
        for (int p = 0; p < 2; ++p) L.kx[p] = (nk - 1) * Cfg::BK + L.lchunk[p] * 8 < L.kmax ? 0u : kOobOffset;
    }
    __device__ __forceinline__ static void mask_rows(Lane &L) {
#pragma unroll
        for (int l = 0; l < Cfg::kUnitLoads; ++l) {
            const int q = L.wave * Cfg::kUnitLoads + l;
            const int row = q * Cfg::kRowsPerLoad + L.lrow;
            L.vAr[l] = row < L.rowsA ? L.vA[q & 1] : kOobOffset;
            L.vBr[l] = row < L.rowsB ? L.vB[q & 1] : kOobOffset;
        }
    }

    // DMA load number l (0 .. kUnitLoads-1) of this wave for one operand
    // unit: rows 8q .. 8q+7 of the tile, q = kUnitLoads * wave + l, K-slice
    // kt, into the slot.
    // kK (masked instances): whether kt is the last slice -- kKAny: decided
    // at run time; kKBefore: known to come before it (rows masked only, no
    // vector instruction); kKLast: known to be it.
    enum : int { kKAny = 0, kKBefore = 1, kKLast = 2 };
    template <bool kIsA, int kK = kKAny>
    __device__ __forceinline__ static void load(char *smem, int slot, int kt, int l, const Lane &L,
                                                __amdgpu_buffer_rsrc_t rsrc) {
        const int q = L.wave * Cfg::kUnitLoads + l;
        const uint32_t ld = kIsA ? L.lda_bytes : L.ldb_bytes;
        uint32_t voff = kIsA ? L.vA[q & 1] : L.vB[q & 1];
        if constexpr (kMasked) {
            const uint32_t rows = kIsA ? L.vAr[l] : L.vBr[l];
            if constexpr (kK == kKBefore)
                voff = rows;
            else if constexpr (kK == kKLast)
                voff = L.kx[q & 1] | rows;
            else
                voff = (L.kx[q & 1] & (kt == L.klast ? 0xFFFFFFFFu : 0u)) | rows;
        }
        buffer_load_lds16(rsrc, (GB_LDS void *)(smem + slot * Cfg::kUnitBytes + q * 1024), voff,
                          (uint32_t)(q * Cfg::kRowsPerLoad) * ld + (uint32_t)kt * Cfg::kRowBytes);
    }

    enum : int { kNoLoad = 0, kLoadA = 1, kLoadB = 2 };

    // Shadow schedule of a k-step: the fragment read (A0, B0, A1, B1, ...,
    // then the A fragments past the last B) and the DMA load (0 ..
    // kUnitLoads-1) that follow MFMA s, or -1.
    __host__ __device__ static constexpr int read_at(int s) { return s < Cfg::kReads ? s : -1; }
    __host__ __device__ static constexpr bool read_is_a(int r) { return r < 2 * Cfg::FN ? (r & 1) == 0 : true; }
    __host__ __device__ static constexpr int read_frag(int r) { return r < 2 * Cfg::FN ? r >> 1 : r - Cfg::FN; }
    __host__ __device__ static constexpr int load_at(int s) {
        return (s >= Cfg::kLoadStart && (s - Cfg::kLoadStart) % Cfg::kLoadStep == 0 &&
                (s - Cfg::kLoadStart) / Cfg::kLoadStep < Cfg::kUnitLoads)
                   ? (s - Cfg::kLoadStart) / Cfg::kLoadStep
                   : -1;
    }

    // One k-step: FM x FN MFMAs on (a, b), block (s / FN, s % FN) for MFMA s;
    // (if kRead) the FM + FN fragment reads of k-step rks from slots (rsa, rsb)
    // into (ra, rb) and (if kLoad) the DMA loads of the unit (kLoad's
    // operand) of slice lkt into slot lslot, each in the MFMA shadow that
    // read_at / load_at assign it.
    template <bool kRead, int kLoad, int kK = kKAny>
    __device__ __forceinline__ static void kstep(char *smem, const bf16x8 (&a)[Cfg::FM], const bf16x8 (&b)[Cfg::FN],
                                                 f32x4 (&acc)[Cfg::FM][Cfg::FN], int rsa, int rsb, int rks,
                                                 bf16x8 (&ra)[Cfg::FM], bf16x8 (&rb)[Cfg::FN], int lslot, int lkt,
                                                 const Lane &L, __amdgpu_buffer_rsrc_t rA, __amdgpu_buffer_rsrc_t rB) {
        const char *sA = smem + rsa * Cfg::kUnitBytes;
        const char *sB = smem + rsb * Cfg::kUnitBytes;
#pragma unroll
        for (int s = 0; s < Cfg::kMfmas; ++s) {
            const int p = s / Cfg::FN, q = s % Cfg::FN;
            acc[p][q] = mfma_16x16x32(a[p], b[q], acc[p][q]);
            __builtin_amdgcn_sched_barrier(0);
            const int r = read_at(s);
            if (kRead && r >= 0) {
                const int f = read_frag(r);
                if (read_is_a(r))
                    ra[f] = *(const GB_LDS bf16x8 *)(sA + L.aRow + f * 16 * Cfg::kRowBytes + L.chunk_off[rks]);
                else
                    rb[f] = *(const GB_LDS bf16x8 *)(sB + L.bRow + f * 16 * Cfg::kRowBytes + L.chunk_off[rks]);
            }
            const int l = load_at(s);
            if (kLoad != kNoLoad && l >= 0) {
                if (kLoad == kLoadA)
                    load<true, kK>(smem, lslot, lkt, l, L, rA);
                else
                    load<false, kK>(smem, lslot, lkt, l, L, rB);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Slice j with A(j) in slot sa.  kMode: 0 = steady (j + 2 < nk),
    // 1 = next to last (j + 2 == nk), 2 = last (mid() runs before its last
    // k-step).  On entry (fa[0], fb[0]) hold
    // k-step 0's fragments of slice j; on exit (modes 0, 1) those of j+1.
    //   k-step 0: reads k-step 1;          loads A(j+2) into B(j-1)'s slot (mode 0)
    //   wait for A(j+1), B(j+1); barrier   (modes 0, 1)
    //   k-step 1: reads slice j+1's k-step 0 (modes 0, 1);
    //             loads B(j+2) into A(j)'s slot (mode 0)
    template <int kMode, int kK = kKAny, class Mid>
    __device__ __forceinline__ static void slice(char *smem, int j, int sa, const Lane &L,
                                                 __amdgpu_buffer_rsrc_t rA, __amdgpu_buffer_rsrc_t rB,
                                                 bf16x8 (&fa)[2][Cfg::FM], bf16x8 (&fb)[2][Cfg::FN],
                                                 f32x4 (&acc)[Cfg::FM][Cfg::FN], Mid &&mid) {
        const int sb = ring_slot(sa + 1);   // B(j)
        const int san = ring_slot(sa + 2);  // A(j+1)
        const int sbn = ring_slot(sa + 3);  // B(j+1)
        const int sa2 = ring_slot(sa + 4);  // A(j+2)
        constexpr int kL0 = kMode == 0 ? kLoadA : kNoLoad;
        constexpr int kL1 = kMode == 0 ? kLoadB : kNoLoad;
        kstep<true, kL0, kK>(smem, fa[0], fb[0], acc, sa, sb, 1, fa[1], fb[1], sa2, j + 2, L, rA, rB);
        if constexpr (kMode <= 1) {
            if constexpr (kMode == 0)
                wait_vmcnt<Cfg::kUnitLoads>();
            else
                wait_vmcnt<0>();
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
            kstep<true, kL1, kK>(smem, fa[1], fb[1], acc, san, sbn, 0, fa[0], fb[0], sa, j + 2, L, rA, rB);
        } else {
            // k-step 0's fragments are dead: their registers take mid()'s loads
            mid();
            __builtin_amdgcn_sched_barrier(0);
            kstep<false, kNoLoad>(smem, fa[1], fb[1], acc, 0, 0, 0, fa[0], fb[0], 0, 0, L, rA, rB);
        }
    }
};

// The fused epilogue for the 16x16 accumulator layout: lane l of block
// (p, q) holds column 16q + l % 16, rows 16p + 4(l / 16) + 0..3.  Each wave
// works through its 128 columns in four groups of 32: it stages a group in
// LDS as fp32 (column-major, columns padded by 16 bytes), then every lane
// takes 8 consecutive rows of one column, 8 times, and writes each as one
// 16-byte store: alpha, beta*C, bias[n] and the activation in fp32, one RNE
// to bf16.  The C and bias values a group needs are loaded one group ahead
// (the first group's before the tile's last K-slice), so their latency hides
// behind the previous group's work instead of stalling every store.
struct RingEpiInputs {
    u32x4 c[8];    // C (beta != 0): 8 consecutive rows of one column per iteration
    uint32_t b[8]; // bias bits (bias != NULL), one column per iteration
    float s[8];    // kScaled: the column's scale_b[n] (1 without scale_b)
};

// Rows m .. m+7 of column n of C: full when m + 8 <= M; with masking, a
// chunk that straddles M -- or every chunk, when ldc % 8 != 0 or C is not
// 16-byte aligned -- is read and written element by element, and chunks
// past M or columns past N are skipped.  kScaled: also the column scales.
template <uint32_t kFlags, bool kMasked, bool kScaled = false, class Cfg = RingConfig>
__device__ __forceinline__ void ring_epi_load(RingEpiInputs &in, const GemmArgs &args, int64_t m0, int64_t n0,
                                              int wm, int wn, int lane, int jj) {
    constexpr int kColChunks = Cfg::WTM / 8;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int idx = t * 64 + lane;
        const int col = idx / kColChunks;
        const int q = idx % kColChunks;
        const int64_t n = n0 + wn * Cfg::WTN + jj * 32 + col;
        const int64_t m = m0 + wm * Cfg::WTM + q * 8;
        if constexpr (kScaled) in.s[t] = (args.scale_b && (!kMasked || n < args.N)) ? args.scale_b[n] : 1.f;
        if constexpr (kMasked) {
            in.c[t] = u32x4{0u, 0u, 0u, 0u};
            in.b[t] = 0u;
            if (n >= args.N) continue;
            if constexpr ((kFlags & kEpiBias) != 0) in.b[t] = args.bias[n];
            if constexpr ((kFlags & kEpiBeta) != 0) {
                const uint16_t *p = args.C + n * args.ldc + m;
                const bool cvec = (args.ldc & 7) == 0 && (reinterpret_cast<uintptr_t>(args.C) & 15) == 0;
                if (m + 8 <= args.M && cvec) {
                    in.c[t] = *(const u32x4 *)p;
                } else if (m < args.M) {
                    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                    for (int e = 0; e < 8; ++e) if (m + e < args.M) w[e >> 1] |= (uint32_t)p[e] << ((e & 1) * 16);
                    in.c[t] = u32x4{w[0], w[1], w[2], w[3]};
                }
            }
        } else {
            if constexpr ((kFlags & kEpiBeta) != 0) in.c[t] = *(const u32x4 *)(args.C + n * args.ldc + m);
            if constexpr ((kFlags & kEpiBias) != 0) in.b[t] = args.bias[n];
        }
    }
}

// kQ8: the quantizing output -- each value becomes one int8 byte of Q,
// sat8(rne(v * scale[m] + zp)); a lane's 8 rows are fixed for the whole tile
// (its 8-row chunk is lane % 16), so their scales are loaded once.
// kScaled: the FP8 input scales -- the product is acc * scale_a[m] *
// scale_b[n] (a missing scale is 1) before alpha, beta*C, bias and the
// activation; the row scales likewise load once per tile.
template <uint32_t kFlags, bool kMasked, bool kQ8, bool kScaled = false, class Cfg = RingConfig>
__device__ __forceinline__ void ring_epilogue(char *smem, const GemmArgs &args, int64_t m0, int64_t n0, int wm,
                                              int wn, int lane, int wave, const f32x4 (&acc)[Cfg::FM][Cfg::FN],
                                              RingEpiInputs &in) {
    char *stage = smem + wave * Cfg::kEpiWaveBytes;
    constexpr int kColChunks = Cfg::WTM / 8;      // 8-row chunks per column
    constexpr int kIters = 32 * kColChunks / 64;  // per lane per 32 columns
    static_assert(kIters == 8, "RingEpiInputs holds one group's 8 iterations");
    static_assert(64 % kColChunks == 0, "a lane's row chunk is the same in every iteration");
    const int c16 = lane & 15, r4 = (lane >> 4) * 4;
    float sc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if constexpr (kQ8) {
        const int64_t m = m0 + wm * Cfg::WTM + (lane % kColChunks) * 8;
        if (!kMasked || m + 8 <= args.M) {
            const f32x4 lo = *(const f32x4 *)(args.scale + m);
            const f32x4 hi = *(const f32x4 *)(args.scale + m + 4);
            sc[0] = lo.x; sc[1] = lo.y; sc[2] = lo.z; sc[3] = lo.w;
            sc[4] = hi.x; sc[5] = hi.y; sc[6] = hi.z; sc[7] = hi.w;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) if (m + e < args.M) sc[e] = args.scale[m + e];
        }
    }
    float sa[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
    if constexpr (kScaled) {
        const int64_t m = m0 + wm * Cfg::WTM + (lane % kColChunks) * 8;
        if (args.scale_a) {
            if (!kMasked || m + 8 <= args.M) {
#pragma unroll
                for (int e = 0; e < 8; ++e) sa[e] = args.scale_a[m + e];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (m + e < args.M) sa[e] = args.scale_a[m + e];
            }
        }
    }
    // The masked instances load a group's inputs at its start instead of
    // one group ahead: with their per-tile masks live, a second set of
    // inputs would not fit in the registers.
    constexpr bool kAhead = !kMasked;
#pragma unroll
    for (int jj = 0; jj < Cfg::FN / 2; ++jj) {
        RingEpiInputs next;
        if (kAhead && jj + 1 < Cfg::FN / 2)
            ring_epi_load<kFlags, kMasked, kScaled, Cfg>(next, args, m0, n0, wm, wn, lane, jj + 1);
        if (!kAhead && jj > 0) ring_epi_load<kFlags, kMasked, kScaled, Cfg>(in, args, m0, n0, wm, wn, lane, jj);
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
            for (int p = 0; p < Cfg::FM; ++p)
                *(GB_LDS f32x4 *)(stage + (qq * 16 + c16) * Cfg::kEpiColBytes + (p * 16 + r4) * 4) =
                    acc[p][2 * jj + qq];
#pragma unroll
        for (int t = 0; t < kIters; ++t) {
            const int idx = t * 64 + lane;
            const int col = idx / kColChunks;
            const int q = idx % kColChunks;
            const f32x4 lo = *(const GB_LDS f32x4 *)(stage + col * Cfg::kEpiColBytes + q * 32);
            const f32x4 hi = *(const GB_LDS f32x4 *)(stage + col * Cfg::kEpiColBytes + q * 32 + 16);
            const int64_t n = n0 + wn * Cfg::WTN + jj * 32 + col;
            const int64_t m = m0 + wm * Cfg::WTM + q * 8;
            float bias_v = 0.f;
            if constexpr ((kFlags & kEpiBias) != 0) bias_v = bf16_bits_to_f32(in.b[t]);
            float cin[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if constexpr ((kFlags & kEpiBeta) != 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    cin[2 * e] = bf16_bits_to_f32(in.c[t][e] & 0xFFFFu);
                    cin[2 * e + 1] = bf16_bits_to_f32(in.c[t][e] >> 16);
                }
            }
            float x[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            if constexpr (kScaled) {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = x[e] * sa[e] * in.s[t];
            }
            if constexpr (kQ8) {
                u32x2 qw = {0u, 0u};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v = epilogue_value<kFlags>(x[e], cin[e], bias_v, args.alpha, args.beta);
                    qw[e >> 2] |= ((uint32_t)quantize_i8(v, sc[e], args.zp) & 0xFFu) << ((e & 3) * 8);
                }
                int8_t *qp = args.Q + n * args.ldq + m;
                if (!kMasked || (n < args.N && m + 8 <= args.M)) {
                    __builtin_nontemporal_store(qw, (u32x2 *)qp);
                } else if (n < args.N) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) if (m + e < args.M) qp[e] = (int8_t)(qw[e >> 2] >> ((e & 3) * 8));
                }
                continue;
            }
            u32x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[e] = pack_bf16x2(
                    epilogue_value<kFlags>(x[2 * e], cin[2 * e], bias_v, args.alpha, args.beta),
                    epilogue_value<kFlags>(x[2 * e + 1], cin[2 * e + 1], bias_v, args.alpha, args.beta));
            uint16_t *p = args.C + n * args.ldc + m;
            if constexpr (kMasked) {
                if (n < args.N) {
                    if (m + 8 <= args.M && (args.ldc & 7) == 0 && (reinterpret_cast<uintptr_t>(args.C) & 15) == 0) {
                        __builtin_nontemporal_store(out, (u32x4 *)p);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) if (m + e < args.M)
                            p[e] = (uint16_t)(out[e >> 1] >> ((e & 1) * 16));
                    }
                }
            } else {
                __builtin_nontemporal_store(out, (u32x4 *)p);
            }
        }
        if (kAhead && jj + 1 < Cfg::FN / 2) in = next;
    }
}

// Requirements checked by the host before launch: M % 256 == 0,
// N % 256 == 0, K % 64 == 0 (masked: any M, N >= 1 and K % 8 == 0, any C
// alignment and ldc), K > 0, A/B (and unmasked C) 16-byte aligned,
// lda/ldb (and unmasked ldc) multiples of 8, and 256*lda*2 + 2K,
// 256*ldb*2 + 2K below 2^31; for kQ8 also Q and scale 16-byte aligned and
// ldq a multiple of 8.
template <uint32_t kFlags, bool kMasked, bool kQ8, class Cfg = RingConfig>
__global__ void __launch_bounds__(Cfg::kThreads)
gemm_ring_kernel(const GemmArgs args, const TileSchedule sched) {
    using RK = RingKernel<kMasked, Cfg>;
    __shared__ __attribute__((aligned(1024))) char smem[Cfg::kLdsBytes];

    const int lane = threadIdx.x & 63;
    typename RK::Lane Ln;
    Ln.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = Ln.wave / Cfg::WAVES_N;
    const int wn = Ln.wave % Cfg::WAVES_N;
    Ln.lda_bytes = (uint32_t)args.lda * 2u;
    Ln.ldb_bytes = (uint32_t)args.ldb * 2u;
    // Load side: lane i covers row 8q + i/8 of its row group q and LDS
    // position i%8, which holds logical chunk (i%8) ^ swz(row); swz sees row
    // bits 1..3, fixed by the lane and the parity of q.
    const int lrow = lane >> 3, lpos = lane & 7;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int c = lpos ^ ring_swizzle(p * Cfg::kRowsPerLoad + lrow);
        Ln.vA[p] = lrow * Ln.lda_bytes + (uint32_t)(c << 4);
        Ln.vB[p] = lrow * Ln.ldb_bytes + (uint32_t)(c << 4);
        Ln.lchunk[p] = c;
    }
    Ln.lrow = lrow;
    Ln.kmax = (int)args.K;
    // Read side: operand lane l takes row l % 16 of its 16-row block and 8
    // consecutive k from logical chunk 4*ks + l/16 (swz sees bits 1..3 of
    // the row, the same for every 16-row block).
    Ln.aRow = (uint32_t)(wm * Cfg::WTM + (lane & 15)) * Cfg::kRowBytes;
    Ln.bRow = (uint32_t)(wn * Cfg::WTN + (lane & 15)) * Cfg::kRowBytes;
#pragma unroll
    for (int ks = 0; ks < Cfg::KSTEPS; ++ks)
        Ln.chunk_off[ks] = (uint32_t)(((4 * ks + (lane >> 4)) ^ ring_swizzle(lane & 15)) << 4);

    const int nk = (int)((args.K + Cfg::BK - 1) / Cfg::BK);
    if constexpr (kMasked) RK::mask_k(Ln, nk);
    const int num_tiles = sched.num_tiles();

    // The tile a workgroup works on: its origin and operand buffers (and,
    // masked, its valid rows and columns).
    struct TileRef {
        int64_t m0, n0;
        __amdgpu_buffer_rsrc_t rA, rB;
    };
    auto tile_ref = [&](int t) {
        int tm, tn;
        sched.tile(t, tm, tn);
        TileRef r;
        r.m0 = (int64_t)tm * Cfg::BM;
        r.n0 = (int64_t)tn * Cfg::BN;
        r.rA = make_rsrc(args.A + r.m0 * args.lda, (uint32_t)(((Cfg::BM - 1) * args.lda + args.K) * 2));
        r.rB = make_rsrc(args.B + r.n0 * args.ldb, (uint32_t)(((Cfg::BN - 1) * args.ldb + args.K) * 2));
        if constexpr (kMasked) {
            Ln.rowsA = (int)(args.M - r.m0 < Cfg::BM ? args.M - r.m0 : Cfg::BM);
            Ln.rowsB = (int)(args.N - r.n0 < Cfg::BN ? args.N - r.n0 : Cfg::BN);
            RK::mask_rows(Ln);
        }
        return r;
    };
    // A(0) and B(0) of a tile into ring slots s0 and s0 + 1.
    auto load_first = [&](const TileRef &r, int s0) {
#pragma unroll
        for (int l = 0; l < Cfg::kUnitLoads; ++l) RK::template load<true>(smem, s0, 0, l, Ln, r.rA);
#pragma unroll
        for (int l = 0; l < Cfg::kUnitLoads; ++l) RK::template load<false>(smem, ring_slot(s0 + 1), 0, l, Ln, r.rB);
    };

    int t = sched.slot(blockIdx.x);
    if (t >= num_tiles) return;  // the host launches at most one workgroup per tile
    TileRef cur = tile_ref(t);
    // The first tile's ring starts at slot 0; every later tile's A(0) and
    // B(0) are loaded into slots 3 and 4 while the previous tile's epilogue
    // stages its results in the low slots (the persistent kernel's store of
    // tile i overlapping the loads of tile i+1, "Outperforming cuBLAS on H100:
    // a worklog", Kernel 6), so its ring starts at slot 3.
    int s0 = 0;
    load_first(cur, s0);

    for (;;) {
        f32x4 acc[Cfg::FM][Cfg::FN];
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        // Prologue: A(1), B(1) behind A(0), B(0).  Vector memory operations
        // complete in issue order, so once at most A(1) and B(1) are
        // outstanding, A(0) and B(0) -- and everything the previous
        // epilogue stored -- have landed.
        if (nk >= 2) {
#pragma unroll
            for (int l = 0; l < Cfg::kUnitLoads; ++l)
                RK::template load<true>(smem, ring_slot(s0 + 2), 1, l, Ln, cur.rA);
#pragma unroll
            for (int l = 0; l < Cfg::kUnitLoads; ++l)
                RK::template load<false>(smem, ring_slot(s0 + 3), 1, l, Ln, cur.rB);
            wait_vmcnt<2 * Cfg::kUnitLoads>();
        } else {
            wait_vmcnt<0>();
        }
        lds_barrier();
        bf16x8 fa[2][Cfg::FM], fb[2][Cfg::FN];
        {
            const char *sA = smem + s0 * Cfg::kUnitBytes;
            const char *sB = smem + ring_slot(s0 + 1) * Cfg::kUnitBytes;
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
                fa[0][i] = *(const GB_LDS bf16x8 *)(sA + Ln.aRow + i * 16 * Cfg::kRowBytes + Ln.chunk_off[0]);
#pragma unroll
            for (int i = 0; i < Cfg::FN; ++i)
                fb[0][i] = *(const GB_LDS bf16x8 *)(sB + Ln.bRow + i * 16 * Cfg::kRowBytes + Ln.chunk_off[0]);
        }
        // Drain every LGKM operation once per tile (a real s_waitcnt the
        // compiler sees), so the loop's LDS-read waits stay exact.
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);

        int j = 0, sa = s0;
        if constexpr (kMasked) {
            // the slices that load A(j+2), B(j+2) before the last one, then
            // the one that loads the last
            for (; j + 3 < nk; ++j) {
                RK::template slice<0, RK::kKBefore>(smem, j, sa, Ln, cur.rA, cur.rB, fa, fb, acc, [] {});
                sa = ring_slot(sa + 2);
            }
            if (j + 2 < nk) {
                RK::template slice<0, RK::kKLast>(smem, j, sa, Ln, cur.rA, cur.rB, fa, fb, acc, [] {});
                ++j;
                sa = ring_slot(sa + 2);
            }
        } else {
            for (; j + 2 < nk; ++j) {
                RK::template slice<0>(smem, j, sa, Ln, cur.rA, cur.rB, fa, fb, acc, [] {});
                sa = ring_slot(sa + 2);
            }
        }
        if (j + 1 < nk) {
            RK::template slice<1>(smem, j, sa, Ln, cur.rA, cur.rB, fa, fb, acc, [] {});
            ++j;
            sa = ring_slot(sa + 2);
        }
        // The epilogue's first C / bias values load during the last k-step.
        RingEpiInputs epi_in;
        RK::template slice<2>(smem, j, sa, Ln, cur.rA, cur.rB, fa, fb, acc, [&] {
            if constexpr ((kFlags & (kEpiBeta | kEpiBias)) != 0)
                ring_epi_load<kFlags, kMasked, false, Cfg>(epi_in, args, cur.m0, cur.n0, wm, wn, lane, 0);
        });

        // Every wave is done reading the ring (all loads landed at the last
        // wait): its low slots now stage the epilogue, and the next tile's
        // first units go into slots 3 and 4, which the staging leaves free
        // (kEpiInRing; else they load once the staging is done).
        lds_barrier();
        const int t_next = t + sched.grid;
        const bool more = t_next < num_tiles;
        TileRef next = cur;
        if (more) {
            next = tile_ref(t_next);
            if constexpr (Cfg::kEpiInRing) load_first(next, 3);
        }
        ring_epilogue<kFlags, kMasked, kQ8, false, Cfg>(smem, args, cur.m0, cur.n0, wm, wn, lane, Ln.wave, acc,
                                                        epi_in);
        if (!more) break;
        // The staging slots are free again before the next prologue loads
        // into them.
        lds_barrier();
        t = t_next;
        cur = next;
        if constexpr (Cfg::kEpiInRing) {
            s0 = 3;
        } else {
            s0 = 0;
            load_first(next, 0);
        }
    }
}

// Launch with the epilogue flags of args baked in; grid = min(tiles, CUs),
// one persistent workgroup per compute unit.  The masked instances run when
// the shape has tails.
template <bool kMasked, bool kQ8 = false, class Cfg = RingConfig>
hipError_t launch_ring_t(const GemmArgs &args, const TileSchedule &s, hipStream_t stream) {
    const dim3 grid(s.grid), block(Cfg::kThreads);
    dispatch_flags(args.flags, [&](auto f) {
        hipLaunchKernelGGL((gemm_ring_kernel<decltype(f)::value, kMasked, kQ8, Cfg>), grid, block, 0, stream, args,
                           s);
    });
    return hipGetLastError();
}

// The ring's schedule: grouped order with GROUP_M = 4 and the XCD slot
// remap.  GEMM_BF16_GROUP_M (1 .. 64) and GEMM_BF16_XCD_REMAP=0 override them;
// they exist to measure those two choices (the results stay correct under
// any order).
inline TileSchedule ring_schedule(const GemmArgs &args, int cus) {
    TileSchedule s{};
    s.tiles_m = (int)((args.M + RingConfig::BM - 1) / RingConfig::BM);
    s.tiles_n = (int)((args.N + RingConfig::BN - 1) / RingConfig::BN);
    s.group_m = 4;
    if (const char *env = std::getenv("GEMM_BF16_GROUP_M")) {
        const int g = std::atoi(env);
        if (g >= 1 && g <= 64) s.group_m = g;
    }
    if (const char *env = std::getenv("GEMM_BF16_XCD_REMAP")) s.no_xcd_remap = env[0] == '0';
    const int tiles = s.num_tiles();
    s.grid = tiles < cus ? tiles : cus;
    return s;
}

}  // namespace gb
