// kernel_tile.h -- the persistent MFMA GEMM kernel for tile-aligned shapes.
//
// One workgroup per compute unit loops over output tiles (tile_schedule.h).
// For each BM x BN tile of C it runs the K loop:
//
//   HBM/L2 --(buffer_load ... lds, 16 B per lane, coalesced)--> LDS ring of
//   STAGES buffers (XOR-swizzled rows) --(ds_read_b128)--> VGPR fragments
//   --(v_mfma_f32_32x32x16_bf16)--> fp32 accumulators in AGPRs
//
// and then the fused epilogue writes bf16 C straight from the accumulators.
//
// The decomposition into tiles, K-slices staged through on-chip memory and
// register accumulators is the one of "Outperforming cuBLAS on H100: a
// worklog", section "Recap of Simon's blog", and of the DeepGEMM article
// (demingchina.com), section 2.1.  The pages' load path (TMA, mbarriers,
// producer/consumer warpgroups) does not exist on gfx950; here every wave
// both issues loads and computes, the loads write LDS directly (no VGPR
// staging), and one workgroup barrier per K-slice orders the ring.
//
// Operand layout in LDS.  A (row-major) and B (column-major, i.e. rows of
// K per output column) are both K-contiguous, so both tiles are stored the
// same way: one 128-byte row per M (or N) index holding BK = 64 bf16, split
// into eight 16-byte chunks.  Chunk c of row r is stored at position
// c ^ swz(r), swz(r) = (r & 7) ^ ((r >> 3) & 1).  A wave's fragment read
// (32 consecutive rows, one logical chunk) then hits 8 (or 16) distinct
// bank groups in every group of 8 (or 16) lanes -- the XOR swizzle the
// DeepGEMM article (section 3.2) uses against shared-memory bank conflicts,
// redone for 128-byte LDS rows.  The direct-to-LDS load writes a wave's 64
// lanes to 1 KiB of consecutive LDS bytes, so the swizzle is applied on the
// global side: lane i fetches the chunk that belongs at its LDS position.
#pragma once

#include "device_common.h"
#include "tile_schedule.h"

namespace gb {

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int STAGES_>
struct TileConfig {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, STAGES = STAGES_;
    static constexpr int kWaves = WAVES_M * WAVES_N;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int WTM = BM / WAVES_M;  // wave tile
    static constexpr int WTN = BN / WAVES_N;
    static constexpr int FM = WTM / 32;       // 32x32 MFMA blocks per wave
    static constexpr int FN = WTN / 32;
    static constexpr int KSTEPS = BK / 16;    // MFMA k-steps per slice
    static constexpr int kRowBytes = BK * 2;
    static constexpr int kRowsPerLoad = 8;    // one wave-wide 16 B/lane load = 8 rows
    static constexpr int kABytes = BM * kRowBytes;
    static constexpr int kBBytes = BN * kRowBytes;
    static constexpr int kStageBytes = kABytes + kBBytes;
    static constexpr int kLdsBytes = STAGES * kStageBytes;
    static constexpr int kALoads = BM / kRowsPerLoad / kWaves;  // per wave per slice
    static constexpr int kBLoads = BN / kRowsPerLoad / kWaves;
    static constexpr int kLoadsPerStage = kALoads + kBLoads;

    static_assert(BK == 64, "the swizzle is written for 128-byte LDS rows");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must hold whole 32x32 blocks");
    static_assert(BM % (kRowsPerLoad * kWaves) == 0 && BN % (kRowsPerLoad * kWaves) == 0,
                  "tile rows must split evenly over the waves' loads");
    static_assert(STAGES >= 2, "need at least double buffering");
    static_assert(kLdsBytes <= 160 * 1024, "gfx950 has 160 KiB of LDS per compute unit");
    static_assert(kLoadsPerStage * (STAGES - 2) < 64, "vmcnt limit");
};

__device__ __forceinline__ int lds_swizzle(int row) { return (row & 7) ^ ((row >> 3) & 1); }

template <class Cfg>
struct TileKernel {
    // Issue the loads of K-slice kt into ring buffer buf.  Wave-uniform
    // arguments only; per-lane offsets come precomputed.
    __device__ __forceinline__ static void issue_slice(char *smem, int buf, int kt, int wave,
                                                       __amdgpu_buffer_rsrc_t rA, __amdgpu_buffer_rsrc_t rB,
                                                       const uint32_t (&vA)[2], const uint32_t (&vB)[2],
                                                       uint32_t lda_bytes, uint32_t ldb_bytes) {
        char *sA = smem + buf * Cfg::kStageBytes;
        char *sB = sA + Cfg::kABytes;
        const uint32_t kbytes = (uint32_t)kt * Cfg::BK * 2;
#pragma unroll
        for (int j = 0; j < Cfg::kALoads; ++j) {
            const int q = wave * Cfg::kALoads + j;  // which 8-row group of the tile
            buffer_load_lds16(rA, (GB_LDS void *)(sA + q * 1024), vA[q & 1],
                              (uint32_t)(q * 8) * lda_bytes + kbytes);
        }
#pragma unroll
        for (int j = 0; j < Cfg::kBLoads; ++j) {
            const int q = wave * Cfg::kBLoads + j;
            buffer_load_lds16(rB, (GB_LDS void *)(sB + q * 1024), vB[q & 1],
                              (uint32_t)(q * 8) * ldb_bytes + kbytes);
        }
    }

    // MFMAs over one K-slice held in ring buffer buf.
    __device__ __forceinline__ static void compute_slice(const char *smem, int buf, uint32_t aRow, uint32_t bRow,
                                                         const uint32_t (&chunk_off)[Cfg::KSTEPS],
                                                         f32x16 (&acc)[Cfg::FM][Cfg::FN]) {
        const char *sA = smem + buf * Cfg::kStageBytes;
        const char *sB = sA + Cfg::kABytes;
#pragma unroll
        for (int kk = 0; kk < Cfg::KSTEPS; ++kk) {
            bf16x8 a[Cfg::FM], b[Cfg::FN];
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
                a[i] = *(const GB_LDS bf16x8 *)(sA + aRow + i * 32 * Cfg::kRowBytes + chunk_off[kk]);
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j)
                b[j] = *(const GB_LDS bf16x8 *)(sB + bRow + j * 32 * Cfg::kRowBytes + chunk_off[kk]);
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                for (int j = 0; j < Cfg::FN; ++j)
                    acc[i][j] = mfma_32x32x16(a[i], b[j], acc[i][j]);
        }
    }

    // Fused epilogue straight from the accumulators.  A 32x32 MFMA result
    // gives lane l the column j = l % 32 and, in registers 4g..4g+3, the four
    // consecutive rows 8g + 4(l / 32) + 0..3: with column-major C those are 8
    // contiguous bytes, written (and, with beta, read) as one 8-byte access.
    __device__ __forceinline__ static void epilogue(const GemmArgs &args, int64_t m0, int64_t n0, int wm, int wn,
                                                    int lane, const f32x16 (&acc)[Cfg::FM][Cfg::FN]) {
        const int h = lane >> 5;
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) {
            const int64_t n = n0 + wn * Cfg::WTN + j * 32 + (lane & 31);
            float bias_v = 0.f;
            if (args.flags & kEpiBias) bias_v = bf16_bits_to_f32(args.bias[n]);
            uint16_t *col = args.C + n * args.ldc;
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int64_t m = m0 + wm * Cfg::WTM + i * 32 + g * 8 + h * 4;
                    u32x2 *p = (u32x2 *)(col + m);
                    float cin[4] = {0.f, 0.f, 0.f, 0.f};
                    if (args.flags & kEpiBeta) {
                        const u32x2 raw = *p;
                        cin[0] = bf16_bits_to_f32(raw.x & 0xFFFFu);
                        cin[1] = bf16_bits_to_f32(raw.x >> 16);
                        cin[2] = bf16_bits_to_f32(raw.y & 0xFFFFu);
                        cin[3] = bf16_bits_to_f32(raw.y >> 16);
                    }
                    float v[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = epilogue_value(acc[i][j][g * 4 + q], cin[q], bias_v, args);
                    u32x2 out;
                    out.x = pack_bf16x2(v[0], v[1]);
                    out.y = pack_bf16x2(v[2], v[3]);
                    *p = out;
                }
            }
        }
    }
};

// Requirements checked by the host before launch: M % BM == 0, N % BN == 0,
// K % BK == 0, K > 0, A/B/C 16-byte aligned, lda/ldb/ldc multiples of 8, and
// BM*lda*2 + 2K, BN*ldb*2 + 2K below 2^31 (32-bit buffer offsets).
template <class Cfg>
__global__ void __launch_bounds__(Cfg::kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_tile_kernel(const GemmArgs args, const TileSchedule sched) {
    using TK = TileKernel<Cfg>;
    __shared__ __attribute__((aligned(1024))) char smem[Cfg::kLdsBytes];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / Cfg::WAVES_N;
    const int wn = wave % Cfg::WAVES_N;

    const uint32_t lda_bytes = (uint32_t)args.lda * 2u;
    const uint32_t ldb_bytes = (uint32_t)args.ldb * 2u;

    // Load side: in an 8-row group q, lane i covers row 8q + i/8 and LDS
    // position i%8, which holds logical chunk (i%8) ^ swz(row); swz depends
    // on the parity of q only, so two offsets per operand suffice.
    const int lrow = lane >> 3, lpos = lane & 7;
    const uint32_t vA[2] = {lrow * lda_bytes + (uint32_t)((lpos ^ lrow) << 4),
                            lrow * lda_bytes + (uint32_t)((lpos ^ lrow ^ 1) << 4)};
    const uint32_t vB[2] = {lrow * ldb_bytes + (uint32_t)((lpos ^ lrow) << 4),
                            lrow * ldb_bytes + (uint32_t)((lpos ^ lrow ^ 1) << 4)};

    // Read side: MFMA operand lane l takes row l % 32 of its 32-row block and
    // 8 consecutive k from logical chunk 2*kk + l/32.
    const uint32_t aRow = (uint32_t)(wm * Cfg::WTM + (lane & 31)) * Cfg::kRowBytes;
    const uint32_t bRow = (uint32_t)(wn * Cfg::WTN + (lane & 31)) * Cfg::kRowBytes;
    uint32_t chunk_off[Cfg::KSTEPS];
#pragma unroll
    for (int kk = 0; kk < Cfg::KSTEPS; ++kk)
        chunk_off[kk] = (uint32_t)(((2 * kk + (lane >> 5)) ^ lds_swizzle(lane & 31)) << 4);

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

        // Prologue: slices 0 .. STAGES-2 in flight.
#pragma unroll
        for (int s = 0; s < Cfg::STAGES - 1; ++s)
            if (s < nk) TK::issue_slice(smem, s, s, wave, rA, rB, vA, vB, lda_bytes, ldb_bytes);

        int buf = 0;
        for (int kt = 0; kt < nk; ++kt) {
            // Slice kt has landed once at most (STAGES-2) later slices are
            // still outstanding; near the end fewer were issued, so drain.
            if (kt + Cfg::STAGES - 2 < nk)
                wait_vmcnt<Cfg::kLoadsPerStage * (Cfg::STAGES - 2)>();
            else
                wait_vmcnt<0>();
            // Everyone's slice kt is in LDS, and everyone has finished
            // reading the buffer that the next load overwrites.
            lds_barrier();
            const int next = kt + Cfg::STAGES - 1;
            if (next < nk) {
                int nbuf = buf + Cfg::STAGES - 1;
                if (nbuf >= Cfg::STAGES) nbuf -= Cfg::STAGES;
                TK::issue_slice(smem, nbuf, next, wave, rA, rB, vA, vB, lda_bytes, ldb_bytes);
            }
            TK::compute_slice(smem, buf, aRow, bRow, chunk_off, acc);
            buf = (buf + 1 == Cfg::STAGES) ? 0 : buf + 1;
        }
        // LDS is reused by the next tile's loads.
        lds_barrier();
        TK::epilogue(args, m0, n0, wm, wn, lane, acc);
    }
}

}  // namespace gb
