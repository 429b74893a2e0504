// kernel_skinny.h -- streaming kernel for short-and-wide products (M = 32 or
// 64 rows of C) whose cost is reading B once from HBM.
//
// With M this small the product is memory-bound: at M = 64, N = K = 8192 the
// kernel moves 136 MB for 8.6 GFLOP (63 flop/byte, against a machine balance
// of about 300), so what matters is streaming the K x N operand B at full
// HBM bandwidth (small M "lacks data reuse, memory loads become the
// bottleneck" -- DeepGEMM article, demingchina.com, section 5.1; small N is
// bandwidth-bound in "Outperforming cuBLAS on H100: a worklog", section
// "Conclusion").
//
// Work split.  One workgroup (four waves) per 32-column strip of C, looping
// over strips (persistent).  The strip's B columns (K-contiguous) and all of
// A are walked in K-slices of 256: each slice is DMA-loaded into LDS with
// coalesced 16 B/lane loads (two 512-byte rows per wave load), and the four
// waves split the slice's 16 MFMA k-steps, each keeping a private fp32
// accumulator of the whole 64 x 32 (or 32 x 32) strip.  At the end the four
// partial strips are summed through LDS and the fused epilogue writes bf16
// C with 16-byte, column-contiguous stores.
//
// Rings.  A (M x 256 per slice) is re-read from L2 by every strip and
// arrives quickly, B (32 x 256 per slice) comes from HBM once, so B is
// prefetched further ahead: A and B rings of SA and SB slices (SA * 32 KiB +
// SB * 16 KiB <= 160 KiB), with SA-1 and SB-1 slices in flight.
//
// LDS rows are 512 bytes (256 bf16, 32 chunks of 16 B); chunk c of row r is
// stored at c ^ (r & 15), which makes the 32-row fragment reads hit distinct
// banks in every 8- and 16-lane group.
#pragma once

#include "device_common.h"
#include "tile_schedule.h"

namespace gb {

template <int FM_, int SA_ = 3, int SB_ = 4, int FN_ = 1, int KS_ = 256>
struct SkinnyConfig {
    static constexpr int FM = FM_;                 // 32-row MFMA blocks: M = 32 * FM
    static constexpr int FN = FN_;                 // 32-column MFMA blocks per strip
    static constexpr int BMr = 32 * FM;            // rows of C
    static constexpr int BN = 32 * FN;             // columns per strip
    static constexpr int KS = KS_;                 // K per slice
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 256;
    static constexpr int kRowBytes = KS * 2;       // 512 for KS = 256
    static constexpr int kChunks = kRowBytes / 16; // 16-byte chunks per row
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;
    static constexpr int kABytes = BMr * kRowBytes;
    static constexpr int kBBytes = BN * kRowBytes;
    static constexpr int SA = SA_, SB = SB_;       // ring depths
    static constexpr int kLdsBytes = SA * kABytes + SB * kBBytes;
    static constexpr int kALoads = BMr / kRowsPerLoad / kWaves;  // 1 KiB wave loads
    static constexpr int kBLoads = BN / kRowsPerLoad / kWaves;
    static constexpr int kStepsPerWave = KS / 16 / kWaves;
    static_assert(FM == 1 || FM == 2, "32 or 64 rows");
    static_assert(KS == 128 || KS == 256, "rows of 256 or 512 bytes");
    static_assert(BMr % (kRowsPerLoad * kWaves) == 0 && BN % (kRowsPerLoad * kWaves) == 0, "loads split");
    static_assert((KS / 16) % kWaves == 0, "k-steps split over the waves");
    static_assert(kLdsBytes <= 160 * 1024, "gfx950 has 160 KiB of LDS per compute unit");
    static_assert(SA >= 2 && SB > SA, "B is prefetched further ahead than A");
    static_assert((SA - 1) * kALoads + (SB - 1) * kBLoads < 64, "vmcnt is a 6-bit counter");
    static_assert(kWaves * BMr * BN * 4 <= kLdsBytes, "partial sums reuse the rings");
};

// Requirements checked by the host: M == 32 * FM, N % 32 == 0, K % 256 == 0,
// K > 0, A/B/C 16-byte aligned, lda/ldb/ldc multiples of 8, and the byte
// offsets of one strip ((BMr-1)*lda + K, (BN-1)*ldb + K, times 2) below 2^31.
template <class Cfg, uint32_t kFlags>
__global__ void __launch_bounds__(Cfg::kThreads)
gemm_skinny_kernel(const GemmArgs args, int num_strips) {
    __shared__ __attribute__((aligned(1024))) char smem[Cfg::kLdsBytes];
    char *const ringA = smem;
    char *const ringB = smem + Cfg::SA * Cfg::kABytes;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lda_bytes = (uint32_t)args.lda * 2u, ldb_bytes = (uint32_t)args.ldb * 2u;

    // Load side: a wave load covers rows 2q, 2q+1; lane i takes row 2q + i/32
    // and LDS chunk position i%32, holding logical chunk (i%32) ^ (row & 15).
    // row & 15 = (2q & 15) + i/32: fold the q-part into a per-load XOR.
    const int lrow = lane / Cfg::kChunks, lpos = lane % Cfg::kChunks;
    // Fragment side: lane l reads row l%32 (+32i) at logical chunk 2s + l/32.
    const uint32_t fragRow = (uint32_t)(lane & 31) * Cfg::kRowBytes;
    const int fragSw = lane & 15 & (Cfg::kChunks - 1);

    const int nk = (int)(args.K / Cfg::KS);

    for (int strip = blockIdx.x; strip < num_strips; strip += gridDim.x) {
        const int64_t n0 = (int64_t)strip * Cfg::BN;
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(args.A, (uint32_t)(((Cfg::BMr - 1) * args.lda + args.K) * 2));
        const __amdgpu_buffer_rsrc_t rB =
            make_rsrc(args.B + n0 * args.ldb, (uint32_t)(((Cfg::BN - 1) * args.ldb + args.K) * 2));

        // Slice j of this strip's order (K-slice ks) into its ring buffer.
        auto issueA = [&](int j, int ks) {
            char *dst = ringA + (j % Cfg::SA) * Cfg::kABytes;
#pragma unroll
            for (int j = 0; j < Cfg::kALoads; ++j) {
                const int q = wave * Cfg::kALoads + j;
                const int row = Cfg::kRowsPerLoad * q + lrow;
                const uint32_t chunk = (uint32_t)(lpos ^ (row & 15 & (Cfg::kChunks - 1)));
                buffer_load_lds16(rA, (GB_LDS void *)(dst + q * 1024), lrow * lda_bytes + chunk * 16,
                                  (uint32_t)(Cfg::kRowsPerLoad * q) * lda_bytes + (uint32_t)ks * Cfg::kRowBytes);
            }
        };
        auto issueB = [&](int j, int ks) {
            char *dst = ringB + (j % Cfg::SB) * Cfg::kBBytes;
#pragma unroll
            for (int j = 0; j < Cfg::kBLoads; ++j) {
                const int q = wave * Cfg::kBLoads + j;
                const int row = Cfg::kRowsPerLoad * q + lrow;
                const uint32_t chunk = (uint32_t)(lpos ^ (row & 15 & (Cfg::kChunks - 1)));
                buffer_load_lds16(rB, (GB_LDS void *)(dst + q * 1024), lrow * ldb_bytes + chunk * 16,
                                  (uint32_t)(Cfg::kRowsPerLoad * q) * ldb_bytes + (uint32_t)ks * Cfg::kRowBytes);
            }
        };

        f32x16 acc[Cfg::FM][Cfg::FN];
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = f32x16{};

        // Previous strip's partial-sum reduction is done with LDS.
        lds_barrier();
        // Slice order: strips start at different K-slices (rotation by the
        // strip's index within its XCD), so the workgroups sharing an L2 do
        // not all request the same A lines at the same moment.
        const int rot = (strip / kNumXcds) % nk;
        auto slice_of = [&](int j) { return (j + rot) % nk; };
        // Prologue: the steady state issues A(j + SA-1), then B(j + SB-1), at
        // slice j's barrier; the prologue replays that order for the virtual
        // barriers j = -(SB-1) .. -1, leaving A(0 .. SA-2) and B(0 .. SB-2)
        // in flight.
        for (int j = -(Cfg::SB - 1); j < 0; ++j) {
            const int a = j + Cfg::SA - 1, b = j + Cfg::SB - 1;
            if (a >= 0 && a < nk) issueA(a, slice_of(a));
            if (b < nk) issueB(b, slice_of(b));
        }

        for (int kt = 0; kt < nk; ++kt) {
            // Slice kt's A and B have landed once only the loads issued after
            // A(kt) are outstanding (B(kt) went out before A(kt) since SB >
            // SA): when every slice up to kt+SB-2 exists these are A(kt+1 ..
            // kt+SA-2) and B(kt+SB-SA .. kt+SB-2); near the end of K the
            // pipeline simply drains.
            if (kt + Cfg::SB - 1 <= nk)
                wait_vmcnt<(Cfg::SA - 2) * Cfg::kALoads + (Cfg::SA - 1) * Cfg::kBLoads>();
            else
                wait_vmcnt<0>();
            lds_barrier();  // everyone's loads landed; slice kt-1 fully read
            if (kt + Cfg::SA - 1 < nk) issueA(kt + Cfg::SA - 1, slice_of(kt + Cfg::SA - 1));
            if (kt + Cfg::SB - 1 < nk) issueB(kt + Cfg::SB - 1, slice_of(kt + Cfg::SB - 1));

            const char *sA = ringA + (kt % Cfg::SA) * Cfg::kABytes;
            const char *sB = ringB + (kt % Cfg::SB) * Cfg::kBBytes;
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
        constexpr int kColBytes = Cfg::BMr * 4 + 16;
        constexpr int kPartBytes = Cfg::BN * kColBytes;
        static_assert(Cfg::kWaves * kPartBytes <= Cfg::kLdsBytes, "partials fit");
        {
            char *part = smem + wave * kPartBytes;
            const int h = lane >> 5;
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
                for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                         acc[i][j][4 * g + 3]};
                        *(GB_LDS f32x4 *)(part + (j * 32 + (lane & 31)) * kColBytes + (i * 32 + g * 8 + h * 4) * 4) =
                            v;
                    }
        }
        lds_barrier();
        constexpr int kChunksPerCol = Cfg::BMr / 8;
        constexpr int kChunks = Cfg::BN * kChunksPerCol;  // 8-row pieces of the strip
        for (int idx = threadIdx.x; idx < kChunks; idx += Cfg::kThreads) {
            const int col = idx / kChunksPerCol, q = idx % kChunksPerCol;
            float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < Cfg::kWaves; ++w) {
                const char *p = smem + w * kPartBytes + col * kColBytes + q * 32;
                const f32x4 lo = *(const GB_LDS f32x4 *)p;
                const f32x4 hi = *(const GB_LDS f32x4 *)(p + 16);
                x[0] += lo.x; x[1] += lo.y; x[2] += lo.z; x[3] += lo.w;
                x[4] += hi.x; x[5] += hi.y; x[6] += hi.z; x[7] += hi.w;
            }
            const int64_t n = n0 + col;
            const int64_t m = (int64_t)q * 8;
            uint16_t *cp = args.C + n * args.ldc + m;
            float bias_v = 0.f;
            if constexpr ((kFlags & kEpiBias) != 0) bias_v = bf16_bits_to_f32(args.bias[n]);
            float cin[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if constexpr ((kFlags & kEpiBeta) != 0) {
                const u32x4 raw = *(const u32x4 *)cp;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    cin[2 * e] = bf16_bits_to_f32(raw[e] & 0xFFFFu);
                    cin[2 * e + 1] = bf16_bits_to_f32(raw[e] >> 16);
                }
            }
            u32x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[e] = pack_bf16x2(epilogue_value<kFlags>(x[2 * e], cin[2 * e], bias_v, args.alpha, args.beta),
                                     epilogue_value<kFlags>(x[2 * e + 1], cin[2 * e + 1], bias_v, args.alpha,
                                                            args.beta));
            __builtin_nontemporal_store(out, (u32x4 *)cp);
        }
    }
}

// One workgroup per compute unit (at most one per strip).
template <class Cfg>
hipError_t launch_skinny(const GemmArgs &args, int cus, hipStream_t stream) {
    const int strips = (int)(args.N / Cfg::BN);
    const dim3 grid(strips < cus ? strips : cus), block(Cfg::kThreads);
    dispatch_flags(args.flags, [&](auto f) {
        hipLaunchKernelGGL((gemm_skinny_kernel<Cfg, decltype(f)::value>), grid, block, 0, stream, args, strips);
    });
    return hipGetLastError();
}

}  // namespace gb
