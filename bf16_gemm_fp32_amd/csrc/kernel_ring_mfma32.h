// kernel_ring_mfma32.h -- the unit-ring 256x256x64 tile kernel of
// kernel_ring.h on v_mfma_f32_32x32x16_bf16 (FM x FN = 4 x 4 blocks of 32x32
// per wave, four k-steps of 16 per slice).  Kept as a measured alternative:
// it runs the same cycle count at a lower clock than the 16x16x32 kernel.
//
// Slice schedule (slots as in kernel_ring.h: A(j) in (2j) % 5, B(j) in
// (2j+1) % 5): while slice j runs, the second half of B(j+1), all of A(j+2)
// and the first half of B(j+2) are loaded into the slots that A(j-1), B(j-1)
// and A(j) free; one barrier per slice, before its last k-step.  Within a
// k-step the 16 MFMAs go out one at a time; the 32-cycle shadow of each
// carries at most one other instruction: the 8 fragment reads of the next
// k-step, then 4 DMA loads.
//
// LDS rows store chunk c at c ^ ((r & 7) ^ ((r >> 3) & 1)), conflict-free for
// the 32x32 fragment reads (32 rows x 2 chunks per instruction).
#pragma once

#include "device_common.h"
#include "epilogue_tile.h"
#include "tile_schedule.h"

namespace gb {

struct Ring32Config {
    static constexpr int BM = 256, BN = 256, BK = 64;
    static constexpr bool kFp8 = false;
    static constexpr int WAVES_M = 2, WAVES_N = 2;
    static constexpr int kWaves = WAVES_M * WAVES_N;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // 128 x 128 wave tile
    static constexpr int FM = WTM / 32, FN = WTN / 32;            // 32x32 MFMA blocks per wave
    static constexpr int KSTEPS = BK / 16;                        // MFMA k-steps per slice
    static constexpr int kRowBytes = BK * 2;                      // 128: one cache line
    static constexpr int kUnitBytes = BM * kRowBytes;             // one operand of one slice
    static constexpr int kSlots = 5;
    static constexpr int kLdsBytes = kSlots * kUnitBytes;
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;         // rows one wave DMA fills
    static constexpr int kUnitLoads = BM / kRowsPerLoad / kWaves; // DMA loads per wave per unit
    static constexpr int kEpiColBytes = WTM * 4 + 16;
    static constexpr int kEpiWaveBytes = 32 * kEpiColBytes;

    static_assert(BM == BN, "A and B units have the same size");
    static_assert(KSTEPS == 4 && FM * FN == 16 && kUnitLoads == 8,
                  "the slice schedule below is written for 4 k-steps of 16 MFMAs and 8 loads per unit");
    static_assert(kLdsBytes <= 160 * 1024, "gfx950 has 160 KiB of LDS per compute unit");
    static_assert(kWaves * kEpiWaveBytes <= kLdsBytes, "epilogue staging reuses the ring");
};

__device__ __forceinline__ int ring32_swizzle(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ int ring32_slot(int s) { return s >= Ring32Config::kSlots ? s - Ring32Config::kSlots : s; }

struct Ring32Kernel {
    using Cfg = Ring32Config;

    struct Lane {
        uint32_t vA[2], vB[2];    // load voffsets by parity of the 8-row group
        uint32_t aRow, bRow;      // LDS offsets (within a unit) of this lane's fragment rows
        uint32_t chunk_off[Cfg::KSTEPS];
        uint32_t lda_bytes, ldb_bytes;
        int wave;
    };

    // DMA load number l (0..7) of this wave for one operand unit: rows
    // 8q .. 8q+7 of the tile, q = 8 * wave + l, K-slice kt, into the unit
    // slot at LDS offset slot * kUnitBytes.
    template <bool kIsA>
    __device__ __forceinline__ static void load(char *smem, int slot, int kt, int l, const Lane &L,
                                                __amdgpu_buffer_rsrc_t rsrc) {
        const int q = L.wave * Cfg::kUnitLoads + l;
        const uint32_t ld = kIsA ? L.lda_bytes : L.ldb_bytes;
        buffer_load_lds16(rsrc, (GB_LDS void *)(smem + slot * Cfg::kUnitBytes + q * 1024),
                          kIsA ? L.vA[q & 1] : L.vB[q & 1],
                          (uint32_t)(q * Cfg::kRowsPerLoad) * ld + (uint32_t)kt * Cfg::kRowBytes);
    }

    // Loads l0 .. l0+3 of one unit, or none.
    enum : int { kNoLoad = 0, kLoadA = 1, kLoadB = 2 };

    // One k-step: MFMA s = 0..15 on block (s / FN, s % FN) with fragments
    // (a, b); after MFMA s, if kRead and s < 8, fragment read s of k-step
    // rkk from the units in slots (rsa, rsb) into (ra, rb), alternating
    // A0, B0, A1, B1, ...; after MFMAs 8, 10, 12, 14, if kLoad, DMA loads
    // l0 .. l0+3 of the unit (kLoad's operand) of slice lkt into slot lslot.
    template <bool kRead, int kLoad>
    __device__ __forceinline__ static void kstep(char *smem, const bf16x8 (&a)[Cfg::FM], const bf16x8 (&b)[Cfg::FN],
                                                 f32x16 (&acc)[Cfg::FM][Cfg::FN], int rsa, int rsb, int rkk,
                                                 bf16x8 (&ra)[Cfg::FM], bf16x8 (&rb)[Cfg::FN], int lslot, int lkt,
                                                 int l0, const Lane &L, __amdgpu_buffer_rsrc_t rA,
                                                 __amdgpu_buffer_rsrc_t rB) {
        const char *sA = smem + rsa * Cfg::kUnitBytes;
        const char *sB = smem + rsb * Cfg::kUnitBytes;
#pragma unroll
        for (int s = 0; s < Cfg::FM * Cfg::FN; ++s) {
            const int p = s / Cfg::FN, j = s % Cfg::FN;
            acc[p][j] = mfma_32x32x16(a[p], b[j], acc[p][j]);
            __builtin_amdgcn_sched_barrier(0);
            if (kRead && s < 2 * Cfg::FM) {
                const int f = s >> 1;
                if ((s & 1) == 0)
                    ra[f] = *(const GB_LDS bf16x8 *)(sA + L.aRow + f * 32 * Cfg::kRowBytes + L.chunk_off[rkk]);
                else
                    rb[f] = *(const GB_LDS bf16x8 *)(sB + L.bRow + f * 32 * Cfg::kRowBytes + L.chunk_off[rkk]);
            }
            if (kLoad != kNoLoad && s >= 8 && (s & 1) == 0) {
                const int l = l0 + ((s - 8) >> 1);
                if (kLoad == kLoadA)
                    load<true>(smem, lslot, lkt, l, L, rA);
                else
                    load<false>(smem, lslot, lkt, l, L, rB);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Slice j with A(j) in slot sa.  kMode: 0 = steady (j + 2 < nk),
    // 1 = next to last (j + 2 == nk), 2 = last.  On entry (fa[0], fb[0]) hold
    // k-step 0's fragments of slice j; on exit (modes 0, 1) they hold those
    // of slice j+1.
    //   k-step 0: reads k-step 1;  loads B(j+1) 4..7          (modes 0, 1)
    //   k-step 1: reads k-step 2;  loads A(j+2) 0..3          (mode 0)
    //   k-step 2: reads k-step 3;  loads A(j+2) 4..7          (mode 0)
    //   wait for A(j+1), B(j+1); barrier                      (modes 0, 1)
    //   k-step 3: reads slice j+1's k-step 0;                 (modes 0, 1)
    //             loads B(j+2) 0..3 into A(j)'s slot          (mode 0)
    template <int kMode>
    __device__ __forceinline__ static void slice(char *smem, int j, int sa, const Lane &L,
                                                 __amdgpu_buffer_rsrc_t rA, __amdgpu_buffer_rsrc_t rB,
                                                 bf16x8 (&fa)[2][Cfg::FM], bf16x8 (&fb)[2][Cfg::FN],
                                                 f32x16 (&acc)[Cfg::FM][Cfg::FN]) {
        const int sb = ring32_slot(sa + 1);   // B(j)
        const int san = ring32_slot(sa + 2);  // A(j+1)
        const int sbn = ring32_slot(sa + 3);  // B(j+1)
        const int sa2 = ring32_slot(sa + 4);  // A(j+2)
        constexpr int kL0 = kMode <= 1 ? kLoadB : kNoLoad;
        constexpr int kL12 = kMode == 0 ? kLoadA : kNoLoad;
        constexpr int kL3 = kMode == 0 ? kLoadB : kNoLoad;
        kstep<true, kL0>(smem, fa[0], fb[0], acc, sa, sb, 1, fa[1], fb[1], sbn, j + 1, 4, L, rA, rB);
        kstep<true, kL12>(smem, fa[1], fb[1], acc, sa, sb, 2, fa[0], fb[0], sa2, j + 2, 0, L, rA, rB);
        kstep<true, kL12>(smem, fa[0], fb[0], acc, sa, sb, 3, fa[1], fb[1], sa2, j + 2, 4, L, rA, rB);
        if constexpr (kMode <= 1) {
            // A(j+1) and B(j+1) landed; in mode 0 only A(j+2)'s 8 loads may remain
            if constexpr (kMode == 0)
                wait_vmcnt<8>();
            else
                wait_vmcnt<0>();
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
            kstep<true, kL3>(smem, fa[1], fb[1], acc, san, sbn, 0, fa[0], fb[0], sa, j + 2, 0, L, rA, rB);
        } else {
            kstep<false, kNoLoad>(smem, fa[1], fb[1], acc, 0, 0, 0, fa[0], fb[0], 0, 0, 0, L, rA, rB);
        }
    }
};

// Requirements checked by the host before launch: M % 256 == 0,
// N % 256 == 0, K % 64 == 0, K > 0, A/B/C 16-byte aligned, lda/ldb/ldc
// multiples of 8, and 256*lda*2 + 2K, 256*ldb*2 + 2K below 2^31.
template <uint32_t kFlags>
__global__ void __launch_bounds__(Ring32Config::kThreads)
gemm_ring32_kernel(const GemmArgs args, const TileSchedule sched) {
    using Cfg = Ring32Config;
    using RK = Ring32Kernel;
    __shared__ __attribute__((aligned(1024))) char smem[Cfg::kLdsBytes];

    const int lane = threadIdx.x & 63;
    RK::Lane Ln;
    Ln.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = Ln.wave / Cfg::WAVES_N;
    const int wn = Ln.wave % Cfg::WAVES_N;
    Ln.lda_bytes = (uint32_t)args.lda * 2u;
    Ln.ldb_bytes = (uint32_t)args.ldb * 2u;
    // Load side: lane i covers row 8q + i/8 of its row group q and LDS
    // position i%8, which holds logical chunk (i%8) ^ swz(row); swz sees the
    // row's low 4 bits, fixed by the lane and the parity of q.
    const int lrow = lane >> 3, lpos = lane & 7;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int c = lpos ^ ring32_swizzle(p * Cfg::kRowsPerLoad + lrow);
        Ln.vA[p] = lrow * Ln.lda_bytes + (uint32_t)(c << 4);
        Ln.vB[p] = lrow * Ln.ldb_bytes + (uint32_t)(c << 4);
    }
    // Read side: MFMA operand lane l takes row l % 32 of its 32-row block and
    // 8 consecutive k from logical chunk 2*kk + l/32.
    Ln.aRow = (uint32_t)(wm * Cfg::WTM + (lane & 31)) * Cfg::kRowBytes;
    Ln.bRow = (uint32_t)(wn * Cfg::WTN + (lane & 31)) * Cfg::kRowBytes;
#pragma unroll
    for (int kk = 0; kk < Cfg::KSTEPS; ++kk)
        Ln.chunk_off[kk] = (uint32_t)(((2 * kk + (lane >> 5)) ^ ring32_swizzle(lane & 31)) << 4);

    const int nk = (int)(args.K / Cfg::BK);
    const int num_tiles = sched.num_tiles();

    for (int t = sched.slot(blockIdx.x); t < num_tiles; t += sched.grid) {
        int tm, tn;
        sched.tile(t, tm, tn);
        const int64_t m0 = (int64_t)tm * Cfg::BM;
        const int64_t n0 = (int64_t)tn * Cfg::BN;
        const __amdgpu_buffer_rsrc_t rA =
            make_rsrc(args.A + m0 * args.lda, (uint32_t)(((Cfg::BM - 1) * args.lda + args.K) * 2));
        const __amdgpu_buffer_rsrc_t rB =
            make_rsrc(args.B + n0 * args.ldb, (uint32_t)(((Cfg::BN - 1) * args.ldb + args.K) * 2));

        f32x16 acc[Cfg::FM][Cfg::FN];
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = f32x16{};

        // The previous tile's epilogue is done with LDS.
        lds_barrier();
        // Prologue: A(0) -> slot 0, B(0) -> 1, A(1) -> 2, B(1) loads 0..3 -> 3
        // (slice 0 issues the rest of B(1)).
#pragma unroll
        for (int l = 0; l < Cfg::kUnitLoads; ++l) RK::load<true>(smem, 0, 0, l, Ln, rA);
#pragma unroll
        for (int l = 0; l < Cfg::kUnitLoads; ++l) RK::load<false>(smem, 1, 0, l, Ln, rB);
        if (nk >= 2) {
#pragma unroll
            for (int l = 0; l < Cfg::kUnitLoads; ++l) RK::load<true>(smem, 2, 1, l, Ln, rA);
#pragma unroll
            for (int l = 0; l < Cfg::kUnitLoads / 2; ++l) RK::load<false>(smem, 3, 1, l, Ln, rB);
            wait_vmcnt<Cfg::kUnitLoads + Cfg::kUnitLoads / 2>();
        } else {
            wait_vmcnt<0>();
        }
        lds_barrier();
        bf16x8 fa[2][Cfg::FM], fb[2][Cfg::FN];
        {
            const char *sA = smem;
            const char *sB = smem + Cfg::kUnitBytes;
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
                fa[0][i] = *(const GB_LDS bf16x8 *)(sA + Ln.aRow + i * 32 * Cfg::kRowBytes + Ln.chunk_off[0]);
#pragma unroll
            for (int i = 0; i < Cfg::FN; ++i)
                fb[0][i] = *(const GB_LDS bf16x8 *)(sB + Ln.bRow + i * 32 * Cfg::kRowBytes + Ln.chunk_off[0]);
        }
        // Drain every LGKM operation once per tile (a real s_waitcnt the
        // compiler sees), so the loop's LDS-read waits stay exact.
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);

        int j = 0, sa = 0;
        for (; j + 2 < nk; ++j) {
            RK::slice<0>(smem, j, sa, Ln, rA, rB, fa, fb, acc);
            sa = ring32_slot(sa + 2);
        }
        if (j + 1 < nk) {
            RK::slice<1>(smem, j, sa, Ln, rA, rB, fa, fb, acc);
            ++j;
            sa = ring32_slot(sa + 2);
        }
        RK::slice<2>(smem, j, sa, Ln, rA, rB, fa, fb, acc);

        // Every wave is done reading the ring (all loads landed at the last
        // wait): its memory now stages the epilogue.
        lds_barrier();
        tile_epilogue<Cfg, kFlags>(smem, args, m0, n0, wm, wn, lane, Ln.wave, acc);
    }
}

// Launch with the epilogue flags of args baked in; grid = min(tiles, CUs),
// one persistent workgroup per compute unit.
inline hipError_t launch_ring32(const GemmArgs &args, int cus, hipStream_t stream) {
    TileSchedule s{};
    s.tiles_m = (int)(args.M / Ring32Config::BM);
    s.tiles_n = (int)(args.N / Ring32Config::BN);
    s.group_m = 4;
    const int tiles = s.num_tiles();
    s.grid = tiles < cus ? tiles : cus;
    const dim3 grid(s.grid), block(Ring32Config::kThreads);
    dispatch_flags(args.flags, [&](auto f) {
        hipLaunchKernelGGL((gemm_ring32_kernel<decltype(f)::value>), grid, block, 0, stream, args, s);
    });
    return hipGetLastError();
}

}  // namespace gb
