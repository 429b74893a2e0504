// kernel_fp8.h -- persistent 256x256 tile kernel for OCP FP8 E4M3 operands
// (the FP8 input path of the DeepGEMM article, sections 1.2 and 6.3) on
// v_mfma_f32_32x32x64_f8f6f4, with fp32 accumulation and the bf16 fused
// epilogue of the bf16 kernels plus per-row / per-column scales.
//
// Byte layout = the bf16 unit ring.  A K-slice is 128 fp8 values, so every
// operand row of a slice is again one full 128-byte line, a unit (one
// operand of one slice) is 256 rows x 128 bytes, and LDS holds a ring of
// five units: A(j) in slot (2j) % 5, B(j) in (2j+1) % 5, loaded by the same
// direct-to-LDS DMA.  One barrier per slice, before its last k-step; while
// slice j runs, A(j+2) is loaded into B(j-1)'s slot (k-step 0) and B(j+2)
// into A(j)'s (k-step 1).
//
// MFMAs.  The fp8 MFMA runs at twice the bf16 rate, so a 32x32x64 block takes
// the time of a 32x32x32 bf16 one: a k-step covers 64 of the slice's 128 k,
// and each wave (128 x 128 of the tile) issues 16 MFMAs per k-step, 64
// cycles each.  An operand fragment is 32 bytes per lane: lane l holds row
// (or column) l % 32 of its 32-row block and 32 of the k-step's 64 bytes.
// Which 32 bytes is free as long as A and B agree (the MFMA sums over k);
// lane half h = l / 32 takes logical chunks 4ks + h and 4ks + 2 + h, so each
// of a fragment's two ds_read_b128 touches one chunk per 32-row half -- the
// access pattern of the 32x32 bf16 kernel, conflict-free with the swizzle
// chunk c at c ^ ((r & 7) ^ ((r >> 3) & 1)).
//
// Shadows: after MFMA r of a k-step (r < 16) comes fragment read r of the
// next k-step (A0 lo, B0 lo, A0 hi, B0 hi, A1 lo, ...), after MFMA 2l+1 DMA
// load l of the unit the k-step loads.
//
// Tails (kMasked): rows past M or N and 16-byte chunks past K are loaded
// from an out-of-range buffer offset, which the DMA turns into zeros (the
// zero-fill of the DeepGEMM article, sections 4.2-4.3); the epilogue skips
// columns past N and 8-row chunks past M and writes a chunk that straddles
// M -- or every chunk, when ldc % 8 != 0 or C is unaligned -- element by
// element.  K must be a multiple of 16.
#pragma once

#include "device_common.h"
#include "kernel_tile.h"
#include "tile_schedule.h"

namespace gb {


struct Fp8Config {
    static constexpr int BM = 256, BN = 256, BK = 128;  // BK in fp8 elements = bytes
    static constexpr int WAVES_M = 2, WAVES_N = 2;
    static constexpr int kWaves = WAVES_M * WAVES_N;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // 128 x 128 wave tile
    static constexpr int FM = WTM / 32, FN = WTN / 32;            // 32x32 MFMA blocks per wave
    static constexpr int KSTEPS = BK / 64;                        // MFMA k-steps per slice
    static constexpr int kRowBytes = BK;                          // 128: one cache line
    static constexpr int kUnitBytes = BM * kRowBytes;
    static constexpr int kSlots = 5;
    static constexpr int kLdsBytes = kSlots * kUnitBytes;
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;
    static constexpr int kUnitLoads = BM / kRowsPerLoad / kWaves;
    static constexpr int kEpiColBytes = WTM * 4 + 16;
    static constexpr int kEpiWaveBytes = 32 * kEpiColBytes;

    static_assert(BM == BN, "A and B units have the same size");
    static_assert(KSTEPS == 2 && FM * FN == 16 && kUnitLoads == 8,
                  "the slice schedule below is written for 2 k-steps of 16 MFMAs and 8 loads per unit");
    static_assert(kLdsBytes <= 160 * 1024, "gfx950 has 160 KiB of LDS per compute unit");
    static_assert(kWaves * kEpiWaveBytes <= kLdsBytes, "epilogue staging reuses the ring");
};

__device__ __forceinline__ int fp8_swizzle(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ int fp8_slot(int s) { return s >= Fp8Config::kSlots ? s - Fp8Config::kSlots : s; }


template <bool kMasked>
struct Fp8Kernel {
    using Cfg = Fp8Config;

    struct Lane {
        uint32_t vA[2], vB[2];  // load voffsets by parity of the 8-row group
        uint32_t aRow, bRow;    // LDS offsets (within a unit) of this lane's fragment rows
        uint32_t lo_off[Cfg::KSTEPS], hi_off[Cfg::KSTEPS];
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
    // kK (masked instances): whether kt is the unit's last slice -- kKAny:
    // decided at run time; kKBefore: known to come before it (rows masked
    // only); kKLast: known to be it.
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

    // One k-step: 16 MFMAs on (a, b), block (s / FN, s % FN) for MFMA s;
    // (if kRead) after MFMA s one 16-byte half of a fragment of k-step rks
    // from slots (rsa, rsb) into (ra, rb); (if kLoad) after MFMA 2l+1 the
    // DMA load l of the unit (kLoad's operand) of slice lkt into slot lslot.
    template <bool kRead, int kLoad, int kK = kKAny>
    __device__ __forceinline__ static void kstep(char *smem, const i32x8 (&a)[Cfg::FM], const i32x8 (&b)[Cfg::FN],
                                                 f32x16 (&acc)[Cfg::FM][Cfg::FN], int rsa, int rsb, int rks,
                                                 i32x8 (&ra)[Cfg::FM], i32x8 (&rb)[Cfg::FN], int lslot, int lkt,
                                                 const Lane &L, __amdgpu_buffer_rsrc_t rA, __amdgpu_buffer_rsrc_t rB) {
        const char *sA = smem + rsa * Cfg::kUnitBytes;
        const char *sB = smem + rsb * Cfg::kUnitBytes;
#pragma unroll
        for (int s = 0; s < Cfg::FM * Cfg::FN; ++s) {
            const int p = s / Cfg::FN, q = s % Cfg::FN;
            acc[p][q] = mfma_fp8_32x32x64(a[p], b[q], acc[p][q]);
            __builtin_amdgcn_sched_barrier(0);
            if (kRead) {
                // read s = 4f + 2*hi + isB: the lo / hi half of A_f / B_f, so
                // A_f and B_f are complete after read 4f + 3
                const int f = s >> 2, hi = (s >> 1) & 1, isB = s & 1;
                const uint32_t off = hi ? L.hi_off[rks] : L.lo_off[rks];
                if (!isB) {
                    const i32x4 v = *(const GB_LDS i32x4 *)(sA + L.aRow + f * 32 * Cfg::kRowBytes + off);
                    if (hi)
                        ra[f].hi = v;
                    else
                        ra[f].lo = v;
                } else {
                    const i32x4 v = *(const GB_LDS i32x4 *)(sB + L.bRow + f * 32 * Cfg::kRowBytes + off);
                    if (hi)
                        rb[f].hi = v;
                    else
                        rb[f].lo = v;
                }
            }
            if (kLoad != kNoLoad && (s & 1) == 1) {
                const int l = s >> 1;
                if (kLoad == kLoadA)
                    load<true, kK>(smem, lslot, lkt, l, L, rA);
                else
                    load<false, kK>(smem, lslot, lkt, l, L, rB);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Slice j with A(j) in slot sa.  kMode: 0 = steady (j + 2 < nk),
    // 1 = next to last (j + 2 == nk), 2 = last.  On entry (fa[0], fb[0]) hold
    // k-step 0's fragments of slice j; on exit (modes 0, 1) those of j+1.
    //   k-step 0: reads k-step 1;          loads A(j+2) into B(j-1)'s slot (mode 0)
    //   wait for A(j+1), B(j+1); barrier   (modes 0, 1)
    //   k-step 1: reads slice j+1's k-step 0 (modes 0, 1);
    //             loads B(j+2) into A(j)'s slot (mode 0)
    template <int kMode, int kK = kKAny>
    __device__ __forceinline__ static void slice(char *smem, int j, int sa, const Lane &L,
                                                 __amdgpu_buffer_rsrc_t rA, __amdgpu_buffer_rsrc_t rB,
                                                 i32x8 (&fa)[2][Cfg::FM], i32x8 (&fb)[2][Cfg::FN],
                                                 f32x16 (&acc)[Cfg::FM][Cfg::FN]) {
        const int sb = fp8_slot(sa + 1);   // B(j)
        const int san = fp8_slot(sa + 2);  // A(j+1)
        const int sbn = fp8_slot(sa + 3);  // B(j+1)
        const int sa2 = fp8_slot(sa + 4);  // A(j+2)
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
            kstep<false, kNoLoad>(smem, fa[1], fb[1], acc, 0, 0, 0, fa[0], fb[0], 0, 0, L, rA, rB);
        }
    }
};

// The fused epilogue for the 32x32 accumulator layout (lane l: column l % 32,
// rows 8g + 4(l/32) + 0..3 in registers 4g..4g+3) with the fp8 scales: each
// wave stages 32 columns at a time in LDS as fp32, then every lane takes 8
// consecutive rows of one column -- the same rows throughout (its 8-row
// chunk is lane % 16), so their row scales load once -- and writes
// epi(alpha * sa[m] * sb[n] * acc + beta*C + bias[n]) as one 16-byte store.
template <uint32_t kFlags, bool kMasked>
__device__ __forceinline__ void fp8_epilogue(char *smem, const GemmArgs &args, int64_t m0, int64_t n0, int wm,
                                             int wn, int lane, int wave,
                                             const f32x16 (&acc)[Fp8Config::FM][Fp8Config::FN]) {
    using Cfg = Fp8Config;
    char *stage = smem + wave * Cfg::kEpiWaveBytes;
    constexpr int kColChunks = Cfg::WTM / 8;      // 8-row chunks per column
    constexpr int kIters = 32 * kColChunks / 64;  // per lane per 32 columns
    static_assert(64 % kColChunks == 0, "a lane's row chunk is the same in every iteration");
    const int h = lane >> 5;
    const bool cvec = !kMasked || ((args.ldc & 7) == 0 && (reinterpret_cast<uintptr_t>(args.C) & 15) == 0);
    const int64_t mrow = m0 + wm * Cfg::WTM + (lane % kColChunks) * 8;
    float sa[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
    if (args.scale_a) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (!kMasked || mrow + e < args.M) sa[e] = args.scale_a[mrow + e];
    }
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                const int row = i * 32 + g * 8 + h * 4;
                *(GB_LDS f32x4 *)(stage + (lane & 31) * Cfg::kEpiColBytes + row * 4) = v;
            }
#pragma unroll
        for (int t = 0; t < kIters; ++t) {
            const int idx = t * 64 + lane;
            const int col = idx / kColChunks;
            const int q = idx % kColChunks;
            const f32x4 lo = *(const GB_LDS f32x4 *)(stage + col * Cfg::kEpiColBytes + q * 32);
            const f32x4 hi = *(const GB_LDS f32x4 *)(stage + col * Cfg::kEpiColBytes + q * 32 + 16);
            const int64_t n = n0 + wn * Cfg::WTN + j * 32 + col;
            const int64_t m = m0 + wm * Cfg::WTM + q * 8;
            if (kMasked && (n >= args.N || m >= args.M)) continue;
            const bool full = !kMasked || (m + 8 <= args.M && cvec);
            uint16_t *p = args.C + n * args.ldc + m;
            const float sb = args.scale_b ? args.scale_b[n] : 1.f;
            float bias_v = 0.f;
            if constexpr ((kFlags & kEpiBias) != 0) bias_v = bf16_bits_to_f32(args.bias[n]);
            float cin[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if constexpr ((kFlags & kEpiBeta) != 0) {
                if (full) {
                    const u32x4 raw = *(const u32x4 *)p;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        cin[2 * e] = bf16_bits_to_f32(raw[e] & 0xFFFFu);
                        cin[2 * e + 1] = bf16_bits_to_f32(raw[e] >> 16);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) if (m + e < args.M) cin[e] = bf16_bits_to_f32(p[e]);
                }
            }
            const float x[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            u32x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[e] = pack_bf16x2(
                    epilogue_value<kFlags>(x[2 * e] * sa[2 * e] * sb, cin[2 * e], bias_v, args.alpha, args.beta),
                    epilogue_value<kFlags>(x[2 * e + 1] * sa[2 * e + 1] * sb, cin[2 * e + 1], bias_v, args.alpha,
                                           args.beta));
            if (full) {
                __builtin_nontemporal_store(out, (u32x4 *)p);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) if (m + e < args.M) p[e] = (uint16_t)(out[e >> 1] >> ((e & 1) * 16));
            }
        }
    }
}

// Requirements checked by the host before launch: M % 256 == 0,
// N % 256 == 0, K % 128 == 0 (masked: any M, N >= 1 and K % 16 == 0),
// K > 0, A/B/C 16-byte aligned, lda/ldb multiples of 16, ldc a multiple of
// 8, and 256*lda + K + 128, 256*ldb + K + 128 (bytes) below 2^31.
// kSplit: the units are (K range, tile) pairs -- unit u = s * tiles + t
// covers slices s * kper .. of tile t -- and each stores its unscaled fp32
// partial tile to split.P (padded to tile multiples when masked: rows and
// columns past the matrix hold zeros); splitk_reduce_kernel then adds them
// in range order and applies the scales and the epilogue (kFlags is
// unused).
template <uint32_t kFlags, bool kMasked, bool kSplit = false>
__global__ void __launch_bounds__(Fp8Config::kThreads)
gemm_fp8_kernel(const GemmArgs args, const TileSchedule sched, const TileSplit split) {
    using Cfg = Fp8Config;
    using RK = Fp8Kernel<kMasked>;
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
    // position i%8, which holds logical chunk (i%8) ^ swz(row); swz sees the
    // row's low 4 bits, fixed by the lane and the parity of q.
    const int lrow = lane >> 3, lpos = lane & 7;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int c = lpos ^ fp8_swizzle(p * Cfg::kRowsPerLoad + lrow);
        Ln.vA[p] = lrow * Ln.lda_bytes + (uint32_t)(c << 4);
        Ln.vB[p] = lrow * Ln.ldb_bytes + (uint32_t)(c << 4);
        Ln.lchunk[p] = c;
    }
    Ln.lrow = lrow;
    Ln.kmax = (int)args.K;
    // Read side: lane l takes row l % 32 of its 32-row block; in k-step ks its
    // fragment's low 16 bytes are logical chunk 4ks + l/32, its high 16 bytes
    // chunk 4ks + 2 + l/32.
    Ln.aRow = (uint32_t)(wm * Cfg::WTM + (lane & 31)) * Cfg::kRowBytes;
    Ln.bRow = (uint32_t)(wn * Cfg::WTN + (lane & 31)) * Cfg::kRowBytes;
    const int swz = fp8_swizzle(lane & 31), h = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < Cfg::KSTEPS; ++ks) {
        Ln.lo_off[ks] = (uint32_t)(((4 * ks + h) ^ swz) << 4);
        Ln.hi_off[ks] = (uint32_t)(((4 * ks + 2 + h) ^ swz) << 4);
    }

    const int nk_all = (int)((args.K + Cfg::BK - 1) / Cfg::BK);
    const int num_tiles = sched.num_tiles();
    const int num_units = kSplit ? num_tiles * split.splits : num_tiles;

    for (int u = sched.slot(blockIdx.x); u < num_units; u += sched.grid) {
        int t = u, sp = 0, nk = nk_all;
        if constexpr (kSplit) {
            sp = u / num_tiles;
            t = u - sp * num_tiles;
            const int rest = nk_all - sp * split.kper;
            nk = rest < split.kper ? rest : split.kper;
        }
        int tm, tn;
        sched.tile(t, tm, tn);
        const int64_t m0 = (int64_t)tm * Cfg::BM;
        const int64_t n0 = (int64_t)tn * Cfg::BN;
        // the unit's K range starts k0 bytes into every row (one byte per value)
        const int64_t k0 = kSplit ? (int64_t)sp * split.kper * Cfg::BK : 0;
        const int64_t kn = kSplit ? (int64_t)nk * Cfg::BK : args.K;
        if constexpr (kSplit && kMasked) Ln.kmax = (int)(args.K - k0);  // the unit's K
        if constexpr (kMasked) {
            Ln.rowsA = (int)(args.M - m0 < Cfg::BM ? args.M - m0 : Cfg::BM);
            Ln.rowsB = (int)(args.N - n0 < Cfg::BN ? args.N - n0 : Cfg::BN);
            RK::mask_rows(Ln);
            RK::mask_k(Ln, nk);
        }
        const __amdgpu_buffer_rsrc_t rA =
            make_rsrc(A8 + m0 * args.lda + k0, (uint32_t)((Cfg::BM - 1) * args.lda + kn));
        const __amdgpu_buffer_rsrc_t rB =
            make_rsrc(B8 + n0 * args.ldb + k0, (uint32_t)((Cfg::BN - 1) * args.ldb + kn));

        f32x16 acc[Cfg::FM][Cfg::FN];
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = f32x16{};

        // The previous tile's epilogue is done with LDS.
        lds_barrier();
        // Prologue: A(0) -> slot 0, B(0) -> 1, A(1) -> 2, B(1) -> 3.
#pragma unroll
        for (int l = 0; l < Cfg::kUnitLoads; ++l) RK::template load<true>(smem, 0, 0, l, Ln, rA);
#pragma unroll
        for (int l = 0; l < Cfg::kUnitLoads; ++l) RK::template load<false>(smem, 1, 0, l, Ln, rB);
        if (nk >= 2) {
#pragma unroll
            for (int l = 0; l < Cfg::kUnitLoads; ++l) RK::template load<true>(smem, 2, 1, l, Ln, rA);
#pragma unroll
            for (int l = 0; l < Cfg::kUnitLoads; ++l) RK::template load<false>(smem, 3, 1, l, Ln, rB);
            wait_vmcnt<2 * Cfg::kUnitLoads>();
        } else {
            wait_vmcnt<0>();
        }
        lds_barrier();
        i32x8 fa[2][Cfg::FM], fb[2][Cfg::FN];
        {
            const char *sA = smem;
            const char *sB = smem + Cfg::kUnitBytes;
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i) {
                fa[0][i].lo = *(const GB_LDS i32x4 *)(sA + Ln.aRow + i * 32 * Cfg::kRowBytes + Ln.lo_off[0]);
                fa[0][i].hi = *(const GB_LDS i32x4 *)(sA + Ln.aRow + i * 32 * Cfg::kRowBytes + Ln.hi_off[0]);
            }
#pragma unroll
            for (int i = 0; i < Cfg::FN; ++i) {
                fb[0][i].lo = *(const GB_LDS i32x4 *)(sB + Ln.bRow + i * 32 * Cfg::kRowBytes + Ln.lo_off[0]);
                fb[0][i].hi = *(const GB_LDS i32x4 *)(sB + Ln.bRow + i * 32 * Cfg::kRowBytes + Ln.hi_off[0]);
            }
        }
        // Drain every LGKM operation once per tile (a real s_waitcnt the
        // compiler sees), so the loop's LDS-read waits stay exact.
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);

        int j = 0, sa = 0;
        if constexpr (kMasked) {
            // the slices that load A(j+2), B(j+2) before the unit's last
            // one, then the one that loads the last
            for (; j + 3 < nk; ++j) {
                RK::template slice<0, RK::kKBefore>(smem, j, sa, Ln, rA, rB, fa, fb, acc);
                sa = fp8_slot(sa + 2);
            }
            if (j + 2 < nk) {
                RK::template slice<0, RK::kKLast>(smem, j, sa, Ln, rA, rB, fa, fb, acc);
                ++j;
                sa = fp8_slot(sa + 2);
            }
        } else {
            for (; j + 2 < nk; ++j) {
                RK::template slice<0>(smem, j, sa, Ln, rA, rB, fa, fb, acc);
                sa = fp8_slot(sa + 2);
            }
        }
        if (j + 1 < nk) {
            RK::template slice<1>(smem, j, sa, Ln, rA, rB, fa, fb, acc);
            ++j;
            sa = fp8_slot(sa + 2);
        }
        RK::template slice<2>(smem, j, sa, Ln, rA, rB, fa, fb, acc);

        if constexpr (kSplit) {
            // no LDS use: the next unit's first barrier orders the ring
            tile_store_partial<Cfg>(split, sp, m0, n0, wm, wn, lane, acc);
        } else {
            // Every wave is done reading the ring (all loads landed at the
            // last wait): its memory now stages the epilogue.
            lds_barrier();
            fp8_epilogue<kFlags, kMasked>(smem, args, m0, n0, wm, wn, lane, Ln.wave, acc);
        }
    }
}

template <bool kMasked>
hipError_t launch_fp8_ring(const GemmArgs &args, int cus, hipStream_t stream) {
    TileSchedule s{};
    s.tiles_m = (int)((args.M + Fp8Config::BM - 1) / Fp8Config::BM);
    s.tiles_n = (int)((args.N + Fp8Config::BN - 1) / Fp8Config::BN);
    s.group_m = 4;
    const int tiles = s.num_tiles();
    s.grid = tiles < cus ? tiles : cus;
    const dim3 grid(s.grid), block(Fp8Config::kThreads);
    const TileSplit none{};
    dispatch_flags(args.flags, [&](auto f) {
        hipLaunchKernelGGL((gemm_fp8_kernel<decltype(f)::value, kMasked>), grid, block, 0, stream, args, s, none);
    });
    return hipGetLastError();
}

// Split-K over these tiles (forced only; small grids take the 128x128 FP8
// tiles): the tile kernel over (range, tile) units into the workspace
// split.P, then the reduction (which applies the scales and the epilogue).  The host has checked the tile requirements (exact multiples,
// or the masked ones), split.splits >= 2, every range non-empty, and that
// split.P holds splits * pstride floats (ldp = M rounded up to 256, pstride
// = ldp times N rounded up to 256).
template <bool kMasked>
hipError_t launch_fp8_splitk(const GemmArgs &args, const TileSplit &split, int cus, hipStream_t stream) {
    TileSchedule s{};
    s.tiles_m = (int)((args.M + Fp8Config::BM - 1) / Fp8Config::BM);
    s.tiles_n = (int)((args.N + Fp8Config::BN - 1) / Fp8Config::BN);
    s.group_m = 4;
    const int units = s.num_tiles() * split.splits;
    s.grid = units < cus ? units : cus;
    // the FP8 units are range-major (split.tile_major is 0 on this path)
    hipLaunchKernelGGL((gemm_fp8_kernel<0u, kMasked, true>), dim3(s.grid), dim3(Fp8Config::kThreads), 0, stream,
                       args, s, split);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t threads = (args.M + 7) / 8 * args.N;
    const int64_t blocks = (threads + 255) / 256;
    const int64_t cap = (int64_t)cus * 8;
    const dim3 rgrid((unsigned)(blocks < cap ? blocks : cap));
    dispatch_flags(args.flags, [&](auto f) {
        hipLaunchKernelGGL((splitk_reduce_kernel<decltype(f)::value, false, Fp8Config::BM, Fp8Config::BN>), rgrid,
                           dim3(256), 0, stream, args, split, s);
    });
    return hipGetLastError();
}

}  // namespace gb
