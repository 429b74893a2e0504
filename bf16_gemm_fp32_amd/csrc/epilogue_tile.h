// epilogue_tile.h -- the fused epilogue of the 32x32-MFMA tile kernels:
// accumulators -> alpha, beta*C, bias, activation in fp32 -> bf16 -> C.
// Cfg supplies the wave tile (WTM x WTN as FM x FN blocks of 32x32), the
// per-wave LDS staging area (kEpiColBytes, kEpiWaveBytes) and whether the
// inputs were FP8 (kFp8: the sums are scaled by scale_a[m] * scale_b[n]).
#pragma once

#include "device_common.h"

namespace gb {

// A 32x32 MFMA result gives lane l the column l % 32 and, in registers
// 4g..4g+3, the four consecutive rows 8g + 4(l/32) + 0..3.  Each wave stages
// 32 columns at a time through its own LDS area as fp32 (column-major,
// columns padded by 16 bytes against bank conflicts), then every lane takes
// 8 consecutive rows of one column: 16 lanes cover a column's WTM rows, so
// each store is 16 bytes and a column's bytes are written contiguously.
// alpha, beta*C (read the same way), bias[n] and the activation are applied
// in fp32, then one RNE to bf16.  The caller has made the staging memory
// free (a barrier after the last LDS read of the main loop).  kMasked:
// columns past N and 8-row chunks past M are skipped, and a chunk that
// straddles M -- or every chunk, when ldc % 8 != 0 or C is not 16-byte
// aligned -- is read and written element by element.
template <class Cfg, uint32_t kFlags, bool kMasked = false>
__device__ __forceinline__ void tile_epilogue(char *smem, const GemmArgs &args, int64_t m0, int64_t n0, int wm,
                                              int wn, int lane, int wave, const f32x16 (&acc)[Cfg::FM][Cfg::FN]) {
    char *stage = smem + wave * Cfg::kEpiWaveBytes;
    constexpr int kColChunks = Cfg::WTM / 8;      // 8-row chunks per column
    constexpr int kIters = 32 * kColChunks / 64;  // per lane per 32 columns
    static_assert((32 * kColChunks) % 64 == 0, "column chunks split over the wave");
    const int h = lane >> 5;
    const bool cvec = !kMasked || ((args.ldc & 7) == 0 && (reinterpret_cast<uintptr_t>(args.C) & 15) == 0);
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
        // accumulators -> LDS
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                const int row = i * 32 + g * 8 + h * 4;
                *(GB_LDS f32x4 *)(stage + (lane & 31) * Cfg::kEpiColBytes + row * 4) = v;
            }
        // LDS -> 8 consecutive rows of one column per lane -> global
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
            float x[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            if constexpr (Cfg::kFp8) {
                // FP8 inputs: the sum times scale_a[m] and scale_b[n] (a
                // missing scale is 1; rows past M are never stored)
                if (args.scale_a) {
                    // a whole chunk's 8 scales as two 16-byte loads; a chunk
                    // that straddles M element by element
                    float sa[8];
                    if (!kMasked || m + 8 <= args.M) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) sa[e] = args.scale_a[m + e];
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) sa[e] = m + e < args.M ? args.scale_a[m + e] : 0.f;
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = x[e] * sa[e];
                }
                if (args.scale_b) {
                    const float sb = args.scale_b[n];
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = x[e] * sb;
                }
            }
            u32x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[e] = pack_bf16x2(
                    epilogue_value<kFlags>(x[2 * e], cin[2 * e], bias_v, args.alpha, args.beta),
                    epilogue_value<kFlags>(x[2 * e + 1], cin[2 * e + 1], bias_v, args.alpha, args.beta));
            if (full) {
                __builtin_nontemporal_store(out, (u32x4 *)p);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) if (m + e < args.M) p[e] = (uint16_t)(out[e >> 1] >> ((e & 1) * 16));
            }
        }
    }
}

}  // namespace gb
