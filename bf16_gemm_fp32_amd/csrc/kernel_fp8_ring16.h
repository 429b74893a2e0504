// kernel_fp8_ring16.h -- persistent 256x256 tile kernel for OCP FP8 E4M3
// operands (the FP8 input path of the DeepGEMM article, sections 1.2 and
// 6.3) on v_mfma_scale_f32_16x16x128_f8f6f4: the byte layout, DMA loads,
// swizzle and epilogue of the bf16 ring kernel (kernel_ring.h), with one
// MFMA k-step per 128-byte K-slice.
//
// Why 16x16.  Per flop the 16x16 form reads and writes half the accumulator
// bytes of the 32x32 form; on this power-limited part that holds a higher
// clock (the bf16 ring runs about 7% faster on 16x16 than on 32x32).
//
// Fragments.  A 16x16x128 block takes 32 bytes per lane from each operand:
// lane l holds row (column) l % 16 of its 16-row block, and as its low and
// high 16 bytes the logical chunks l/16 and 4 + l/16 of the 128-byte row --
// the two reads the bf16 ring makes for that row in its two k-steps, so the
// same swizzle keeps them conflict-free.  Which k a byte holds is free as
// long as A and B agree, since the MFMA sums over k.
//
// Register schedule.  A slice is 64 MFMAs per wave (8 x 8 blocks of 16x16)
// in four quadrants of 4 x 4 blocks: rows 0-3 x columns 0-3, rows 0-3 x
// columns 4-7 (both column by column), rows 4-7 x columns 0-3, rows 4-7 x
// columns 4-7 (both row by row).  Every fragment then has one register set,
// 128 VGPRs in all: A_0..3 are dead after the second quadrant and B_0..3
// after the third, so the next slice's A_0..3 and B_0..3 are read in the
// third and fourth quadrants; B_4..7 are first needed in the second
// quadrant and A_4..7 in the third, so each slice reads its own B_4..7 in
// the first quadrant and its own A_4..7 in the second.
// One 16-byte read follows every even MFMA:
//   quadrant 0: B_4..B_7    1: A_4..A_7    2: A'_0..A'_3    3: B'_0..B'_3
// (A', B': the next slice's).
//
// LDS ring.  Five 32 KiB slots, A(j) in slot 2j % 5 and B(j) in 2j+1, as in
// the bf16 ring.  Slice j reads A(j), B(j) in its first half and A(j+1),
// B(j+1) in its second, so one barrier per slice, between the halves,
// publishes A(j+1), B(j+1) and frees the slots of A(j) and B(j).  A wave
// loads A(j+2) into B(j-1)'s slot in the first half (after MFMAs 1, 5, ...,
// 29) and B(j+2) into A(j)'s slot in the second (after MFMAs 33, ..., 61);
// at the barrier only A(j+2)'s loads may still be in flight.
//
// The end of K.  Every slice but the last runs the same schedule: a load of
// a slice past the end takes an out-of-range offset, so the DMA fetches
// nothing and writes zeros into a slot no later slice reads.  The last
// slice reads only its own fragments, loads nothing and needs no barrier;
// the epilogue's first loads go out in its second half.
//
// Tails (kMasked): rows past M or N and 16-byte chunks past K are loaded
// from an out-of-range buffer offset, which the DMA turns into zeros (the
// zero-fill of the DeepGEMM article, sections 4.2-4.3); the ring epilogue
// masks C.  K must be a multiple of 16.
#pragma once

#include "device_common.h"
#include "kernel_ring.h"
#include "tile_schedule.h"

namespace gb {

struct Fp8Ring16Config {
    static constexpr int BM = 256, BN = 256, BK = 128;  // BK in fp8 values = bytes
    static constexpr int WAVES_M = 2, WAVES_N = 2;
    static constexpr int kWaves = WAVES_M * WAVES_N;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // 128 x 128 wave tile
    static constexpr int FM = WTM / 16, FN = WTN / 16;            // 16x16 MFMA blocks per wave
    static constexpr int kRowBytes = BK;                          // 128: one cache line
    static constexpr int kUnitBytes = BM * kRowBytes;
    static constexpr int kSlots = 5;
    static constexpr int kLdsBytes = kSlots * kUnitBytes;
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;
    static constexpr int kUnitLoads = BM / kRowsPerLoad / kWaves;

    static_assert(FM == 8 && FN == 8 && kUnitLoads == 8,
                  "the slice schedule below is written for 8 x 8 blocks and 8 loads per unit");
    static_assert(kSlots == RingConfig::kSlots && kLdsBytes == RingConfig::kLdsBytes && WTM == RingConfig::WTM &&
                      FM == RingConfig::FM && FN == RingConfig::FN && kThreads == RingConfig::kThreads,
                  "the ring's slot arithmetic and epilogue apply unchanged");
};

// E4M3 x E4M3 16x16x128 block, fp32 accumulate: format selectors 0 / 0 and
// unit block scales (E8M0 exponent 127 = 2^0).
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(const i32x8 &a, const i32x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <bool kMasked>
struct Fp8Ring16Kernel {
    using Cfg = Fp8Ring16Config;

    struct Lane {
        uint32_t vA[2], vB[2];  // load voffsets by parity of the 8-row group
        uint32_t aRow, bRow;    // LDS offsets (within a unit) of this lane's fragment rows
        uint32_t lo_off, hi_off;
        uint32_t lda_bytes, ldb_bytes;
        int wave, nk;
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

    // Masking state (kMasked): the K tail (per launch, or per unit when K
    // is split) and the rows (per tile).  Only the last slice can hold
    // chunks at or past K, so a load's voffset in the K loop is its
    // row-masked one, with kx or-ed in when kt is that slice.
    __device__ __forceinline__ static void mask_k(Lane &L, int nk) {
        L.klast = __builtin_amdgcn_readfirstlane(nk - 1);
#pragma unroll
        for (int p = 0; p < 2; ++p) L.kx[p] = (nk - 1) * Cfg::BK + L.lchunk[p] * 16 < L.kmax ? 0u : kOobOffset;
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

    // DMA load number l (0..7) of this wave for one operand unit: rows
    // 8q .. 8q+7 of the tile, q = 8 * wave + l, K-slice kt, into the slot.
    // A slice past the end of K (kt >= nk) is loaded from the out-of-range
    // offset, which the buffer unit turns into zeros without touching
    // memory.  That offset goes into the per-lane voffset, which the range
    // check covers; the scalar offset stays the in-range row offset (its
    // sum with the out-of-range voffset stays below 2^32, so nothing wraps
    // back into range).
    //
    // kK: where kt lies -- kKAny: decided at run time (a slice past the end,
    // the last slice or one before it); kKBefore: known to come before the
    // last slice (no K test; rows masked only); kKLast: known to be it.
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
        const bool in_k = kK != kKAny || kt < L.nk;
        if (!in_k) voff = kOobOffset;
        buffer_load_lds16(rsrc, (GB_LDS void *)(smem + slot * Cfg::kUnitBytes + q * 1024), voff,
                          (uint32_t)(q * Cfg::kRowsPerLoad) * ld + (in_k ? (uint32_t)kt * Cfg::kRowBytes : 0u));
    }

    // One 16-byte half of fragment f (16-row block f of the wave's rows).
    __device__ __forceinline__ static i32x4 read(const char *unit, uint32_t row, int f, uint32_t off) {
        return *(const GB_LDS i32x4 *)(unit + row + f * 16 * Cfg::kRowBytes + off);
    }

    // Slice j with A(j) in slot sa.  kFull: the whole schedule above;
    // kLast: the tile's last slice, which reads only its own fragments and
    // runs mid() after MFMA 32, when A_0..3 are dead.
    enum : int { kLast = 0, kFull = 1 };

    // The block (row, column) of MFMA s.
    __host__ __device__ static constexpr int row_of(int s) {
        return ((s >> 4) >= 2 ? 4 : 0) + ((s >> 4) < 2 ? (s & 3) : ((s & 15) >> 2));
    }
    __host__ __device__ static constexpr int col_of(int s) {
        return (((s >> 4) & 1) ? 4 : 0) + ((s >> 4) < 2 ? ((s & 15) >> 2) : (s & 3));
    }

    template <int kMode, int kK, class Mid>
    __device__ __forceinline__ static void slice(char *smem, int j, int sa, const Lane &L,
                                                 __amdgpu_buffer_rsrc_t rA, __amdgpu_buffer_rsrc_t rB,
                                                 i32x8 (&fa)[Cfg::FM], i32x8 (&fb)[Cfg::FN],
                                                 f32x4 (&acc)[Cfg::FM][Cfg::FN], Mid &&mid) {
        const char *sA0 = smem + sa * Cfg::kUnitBytes;                 // A(j)
        const char *sB0 = smem + ring_slot(sa + 1) * Cfg::kUnitBytes;  // B(j)
        const char *sA1 = smem + ring_slot(sa + 2) * Cfg::kUnitBytes;  // A(j+1)
        const char *sB1 = smem + ring_slot(sa + 3) * Cfg::kUnitBytes;  // B(j+1)
        const int slotA2 = ring_slot(sa + 4);                          // B(j-1)'s slot takes A(j+2)
        const int slotB2 = sa;                                         // A(j)'s slot takes B(j+2)
#pragma unroll
        for (int s = 0; s < Cfg::FM * Cfg::FN; ++s) {
            if (kMode == kFull && s == 32) {
                // A(j+1), B(j+1) landed; every wave is done with A(j), B(j)
                wait_vmcnt<Cfg::kUnitLoads>();
                lds_barrier();
                __builtin_amdgcn_sched_barrier(0);
            }
            const int p = row_of(s), q = col_of(s);
            acc[p][q] = mfma_fp8_16x16x128(fa[p], fb[q], acc[p][q]);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (kMode == kLast) {
                if (s == 32) mid();
            }
            const int quad = s >> 4;
            if ((s & 1) == 0 && (kMode == kFull || quad < 2)) {
                const int f = 4 * (quad == 0 || quad == 1) + ((s & 15) >> 2);
                const uint32_t off = ((s >> 1) & 1) ? L.hi_off : L.lo_off;
                const bool isA = quad == 1 || quad == 2;
                const char *unit = quad == 0 ? sB0 : quad == 1 ? sA0 : quad == 2 ? sA1 : sB1;
                const i32x4 v = read(unit, isA ? L.aRow : L.bRow, f, off);
                i32x8 &d = isA ? fa[f] : fb[f];
                if ((s >> 1) & 1)
                    d.hi = v;
                else
                    d.lo = v;
            }
            if (kMode == kFull && (s & 3) == 1) {
                const int l = s >> 2;  // 0..15
                if (l < Cfg::kUnitLoads)
                    load<true, kK>(smem, slotA2, j + 2, l, L, rA);
                else
                    load<false, kK>(smem, slotB2, j + 2, l - Cfg::kUnitLoads, L, rB);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
};

// Requirements checked by the host before launch: M % 256 == 0,
// N % 256 == 0, K % 128 == 0 (masked: any M, N >= 1 and K % 16 == 0, any C
// alignment and ldc), K > 0, A/B (and unmasked C) 16-byte aligned, lda/ldb
// multiples of 16 (unmasked ldc a multiple of 8), and 256*lda + K + 128,
// 256*ldb + K + 128 (bytes) below 2^31.
template <uint32_t kFlags, bool kMasked>
__global__ void __launch_bounds__(Fp8Ring16Config::kThreads)
gemm_fp8_ring16_kernel(const GemmArgs args, const TileSchedule sched) {
    using Cfg = Fp8Ring16Config;
    using RK = Fp8Ring16Kernel<kMasked>;
    __shared__ __attribute__((aligned(1024))) char smem[Cfg::kLdsBytes];
    const uint8_t *A8 = reinterpret_cast<const uint8_t *>(args.A);
    const uint8_t *B8 = reinterpret_cast<const uint8_t *>(args.B);

    const int lane = threadIdx.x & 63;
    typename RK::Lane Ln;
    Ln.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = Ln.wave / Cfg::WAVES_N;
    const int wn = Ln.wave % Cfg::WAVES_N;
    Ln.lda_bytes = (uint32_t)args.lda;
    Ln.ldb_bytes = (uint32_t)args.ldb;
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
    Ln.nk = (int)((args.K + Cfg::BK - 1) / Cfg::BK);
    // Read side: lane l takes row l % 16 of its 16-row block; its fragment's
    // low 16 bytes are logical chunk l/16, its high 16 bytes chunk 4 + l/16.
    Ln.aRow = (uint32_t)(wm * Cfg::WTM + (lane & 15)) * Cfg::kRowBytes;
    Ln.bRow = (uint32_t)(wn * Cfg::WTN + (lane & 15)) * Cfg::kRowBytes;
    Ln.lo_off = (uint32_t)(((lane >> 4) ^ ring_swizzle(lane & 15)) << 4);
    Ln.hi_off = (uint32_t)(((4 + (lane >> 4)) ^ ring_swizzle(lane & 15)) << 4);

    const int nk = Ln.nk;
    if constexpr (kMasked) RK::mask_k(Ln, nk);
    const int num_tiles = sched.num_tiles();

    for (int t = sched.slot(blockIdx.x); t < num_tiles; t += sched.grid) {
        int tm, tn;
        sched.tile(t, tm, tn);
        const int64_t m0 = (int64_t)tm * Cfg::BM;
        const int64_t n0 = (int64_t)tn * Cfg::BN;
        if constexpr (kMasked) {
            Ln.rowsA = (int)(args.M - m0 < Cfg::BM ? args.M - m0 : Cfg::BM);
            Ln.rowsB = (int)(args.N - n0 < Cfg::BN ? args.N - n0 : Cfg::BN);
            RK::mask_rows(Ln);
        }
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(A8 + m0 * args.lda, (uint32_t)((Cfg::BM - 1) * args.lda + args.K));
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(B8 + n0 * args.ldb, (uint32_t)((Cfg::BN - 1) * args.ldb + args.K));

        f32x4 acc[Cfg::FM][Cfg::FN];
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        // The previous tile's epilogue is done with LDS.
        lds_barrier();
        // Prologue: A(0) -> slot 0, B(0) -> 1, A(1) -> 2, B(1) -> 3 (slices
        // past the end load nothing); then slice 0's A_0..3 and B_0..3.
#pragma unroll
        for (int l = 0; l < Cfg::kUnitLoads; ++l) RK::template load<true>(smem, 0, 0, l, Ln, rA);
#pragma unroll
        for (int l = 0; l < Cfg::kUnitLoads; ++l) RK::template load<false>(smem, 1, 0, l, Ln, rB);
#pragma unroll
        for (int l = 0; l < Cfg::kUnitLoads; ++l) RK::template load<true>(smem, 2, 1, l, Ln, rA);
#pragma unroll
        for (int l = 0; l < Cfg::kUnitLoads; ++l) RK::template load<false>(smem, 3, 1, l, Ln, rB);
        wait_vmcnt<2 * Cfg::kUnitLoads>();
        lds_barrier();
        i32x8 fa[Cfg::FM], fb[Cfg::FN];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            fa[i].lo = RK::read(smem, Ln.aRow, i, Ln.lo_off);
            fa[i].hi = RK::read(smem, Ln.aRow, i, Ln.hi_off);
            fb[i].lo = RK::read(smem + Cfg::kUnitBytes, Ln.bRow, i, Ln.lo_off);
            fb[i].hi = RK::read(smem + Cfg::kUnitBytes, Ln.bRow, i, Ln.hi_off);
        }
        // Drain every LGKM operation once per tile (a real s_waitcnt the
        // compiler sees), so the loop's LDS-read waits stay exact.
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);

        using K = RK;
        const auto none = [] {};
        // Slice j loads slice j + 2.  Masked: before the last one while
        // j + 3 < nk, then the last one, then (j = nk - 2) one past the end;
        // unmasked, one loop that tests for slices past the end.
        int sa = 0, j = 0;
        if constexpr (kMasked) {
            for (; j + 3 < nk; ++j) {
                RK::template slice<K::kFull, K::kKBefore>(smem, j, sa, Ln, rA, rB, fa, fb, acc, none);
                sa = ring_slot(sa + 2);
            }
            if (j + 2 < nk) {
                RK::template slice<K::kFull, K::kKLast>(smem, j, sa, Ln, rA, rB, fa, fb, acc, none);
                ++j;
                sa = ring_slot(sa + 2);
            }
        }
        for (; j + 1 < nk; ++j) {
            RK::template slice<K::kFull, K::kKAny>(smem, j, sa, Ln, rA, rB, fa, fb, acc, none);
            sa = ring_slot(sa + 2);
        }
        // The epilogue's first C / bias / scale values load during the last slice.
        RingEpiInputs epi_in;
        const auto mid = [&] { ring_epi_load<kFlags, kMasked, true>(epi_in, args, m0, n0, wm, wn, lane, 0); };
        RK::template slice<K::kLast, K::kKAny>(smem, nk - 1, sa, Ln, rA, rB, fa, fb, acc, mid);
        // With beta or masking, every MFMA of the tile completes here: the
        // compiler may not sink the last slice's MFMAs into the epilogue,
        // where their fragments would stay live beside the C loads and the
        // masked stores and spill.  (The plain epilogue is better without.)
        if constexpr (kMasked || (kFlags & kEpiBeta) != 0) {
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                for (int q = 0; q < Cfg::FN; ++q) asm volatile("" : "+a"(acc[i][q]));
        }
        // The out-of-range loads of the last full slices write zeros into
        // free slots: they land before the epilogue stages its values there.
        wait_vmcnt<0>();

        // Every wave is done reading the ring (all loads landed at the last
        // wait): its memory now stages the epilogue.
        lds_barrier();
        ring_epilogue<kFlags, kMasked, false, true>(smem, args, m0, n0, wm, wn, lane, Ln.wave, acc, epi_in);
    }
}

// Launch with the epilogue flags of args baked in; grid = min(tiles, CUs),
// one persistent workgroup per compute unit.
template <bool kMasked>
hipError_t launch_fp8_ring16(const GemmArgs &args, int cus, hipStream_t stream) {
    TileSchedule s{};
    s.tiles_m = (int)((args.M + Fp8Ring16Config::BM - 1) / Fp8Ring16Config::BM);
    s.tiles_n = (int)((args.N + Fp8Ring16Config::BN - 1) / Fp8Ring16Config::BN);
    s.group_m = 4;
    const int tiles = s.num_tiles();
    s.grid = tiles < cus ? tiles : cus;
    const dim3 grid(s.grid), block(Fp8Ring16Config::kThreads);
    dispatch_flags(args.flags, [&](auto f) {
        hipLaunchKernelGGL((gemm_fp8_ring16_kernel<decltype(f)::value, kMasked>), grid, block, 0, stream, args, s);
    });
    return hipGetLastError();
}

}  // namespace gb
