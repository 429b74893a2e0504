// kernel_generic.h -- bounds-checked MFMA GEMM for any shape, leading
// dimension and (2-byte) alignment.
//
// Tail tiles are handled by zero-filling every operand element outside the
// matrix, so they run the same MFMA sequence as full tiles (zero products
// add nothing); stores are masked per element.  This is the boundary
// treatment of the DeepGEMM article (demingchina.com), sections 4.2-4.3.
// It also serves K == 0 (no K-slices: the epilogue sees zero accumulators).
//
// Tile 64 x 64, four waves in a 2 x 2 grid each owning one 32 x 32 MFMA
// block, K-slices of 32 staged through padded LDS rows (80 bytes: 64 data +
// 16 pad, so consecutive rows start in different bank groups).  Loads go
// through registers: a 16-byte vector load when the chunk is in range and
// aligned, element-wise checked loads otherwise.
#pragma once

#include "device_common.h"

namespace gb {

struct GenericConfig {
    static constexpr int BM = 64, BN = 64, BK = 32;
    static constexpr int kThreads = 256;
    static constexpr int kRowBytes = BK * 2 + 16;  // padded
    static constexpr int kABytes = BM * kRowBytes;
    static constexpr int kBBytes = BN * kRowBytes;
};

// Eight consecutive bf16 of one K-contiguous row, elements with k >= K (or a
// row outside the matrix) read as zero.
__device__ __forceinline__ u32x4 load_row_chunk(const uint16_t *row, bool row_ok, int64_t k, int64_t K) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (!row_ok) return v;
    const uint16_t *p = row + k;
    if (k + 8 <= K && (((uintptr_t)p) & 15u) == 0) return *(const u32x4 *)p;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (k + e < K) w[e >> 1] |= (uint32_t)p[e] << ((e & 1) * 16);
    v.x = w[0];
    v.y = w[1];
    v.z = w[2];
    v.w = w[3];
    return v;
}

// Eight consecutive OCP FP8 E4M3 bytes of one K-contiguous row as eight
// bf16 values (exact), elements with k >= K (or a row outside the matrix)
// read as zero.
__device__ __forceinline__ u32x4 load_row_chunk_fp8(const uint8_t *row, bool row_ok, int64_t k, int64_t K) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (!row_ok) return v;
    const uint8_t *p = row + k;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (k + e < K) w[e >> 1] |= fp8_e4m3_to_bf16_bits(p[e]) << ((e & 1) * 16);
    v.x = w[0];
    v.y = w[1];
    v.z = w[2];
    v.w = w[3];
    return v;
}

// kFp8: A and B hold E4M3 bytes (lda, ldb in bytes), converted to bf16 on
// their way into LDS, and the product is scaled by scale_a[m] * scale_b[n].
template <bool kFp8>
__global__ void __launch_bounds__(GenericConfig::kThreads)
gemm_generic_kernel(const GemmArgs args, int64_t tiles_m, int64_t num_tiles) {
    using G = GenericConfig;
    __shared__ __attribute__((aligned(16))) char sA[G::kABytes];
    __shared__ __attribute__((aligned(16))) char sB[G::kBBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    // loader role: one 16-byte chunk of A and one of B per thread and slice
    const int lr = tid >> 2, lc = tid & 3;

    for (int64_t tile = blockIdx.x; tile < num_tiles; tile += gridDim.x) {
        const int64_t m0 = (tile % tiles_m) * G::BM;
        const int64_t n0 = (tile / tiles_m) * G::BN;
        const bool a_ok = m0 + lr < args.M;
        const bool b_ok = n0 + lr < args.N;
        const uint16_t *a_row = args.A + (a_ok && !kFp8 ? (m0 + lr) * args.lda : 0);
        const uint16_t *b_row = args.B + (b_ok && !kFp8 ? (n0 + lr) * args.ldb : 0);
        const uint8_t *a_row8 = reinterpret_cast<const uint8_t *>(args.A) + (a_ok ? (m0 + lr) * args.lda : 0);
        const uint8_t *b_row8 = reinterpret_cast<const uint8_t *>(args.B) + (b_ok ? (n0 + lr) * args.ldb : 0);

        f32x16 acc = {};
        for (int64_t k0 = 0; k0 < args.K; k0 += G::BK) {
            const u32x4 va = kFp8 ? load_row_chunk_fp8(a_row8, a_ok, k0 + lc * 8, args.K)
                                  : load_row_chunk(a_row, a_ok, k0 + lc * 8, args.K);
            const u32x4 vb = kFp8 ? load_row_chunk_fp8(b_row8, b_ok, k0 + lc * 8, args.K)
                                  : load_row_chunk(b_row, b_ok, k0 + lc * 8, args.K);
            *(GB_LDS u32x4 *)(sA + lr * G::kRowBytes + lc * 16) = va;
            *(GB_LDS u32x4 *)(sB + lr * G::kRowBytes + lc * 16) = vb;
            lds_barrier();
#pragma unroll
            for (int kk = 0; kk < G::BK / 16; ++kk) {
                const int chunk = 2 * kk + (lane >> 5);
                const bf16x8 a = *(const GB_LDS bf16x8 *)(sA + (wm * 32 + (lane & 31)) * G::kRowBytes + chunk * 16);
                const bf16x8 b = *(const GB_LDS bf16x8 *)(sB + (wn * 32 + (lane & 31)) * G::kRowBytes + chunk * 16);
                acc = mfma_32x32x16(a, b, acc);
            }
            lds_barrier();
        }

        // lane: column n, rows 8g + 4h + 0..3 of the wave's 32x32 block.
        // With args.Q set the output is int8 (quantizing entry point) and C,
        // if read at all, is the separate bf16 input C0.
        const int64_t n = n0 + wn * 32 + (lane & 31);
        if (n < args.N) {
            const float bias_v = (args.flags & kEpiBias) ? bf16_bits_to_f32(args.bias[n]) : 0.f;
            const float sb = (kFp8 && args.scale_b) ? args.scale_b[n] : 1.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (m < args.M) {
                    const float cin = (args.flags & kEpiBeta) ? bf16_bits_to_f32(args.C[n * args.ldc + m]) : 0.f;
                    float x = acc[r];
                    if (kFp8) x = x * (args.scale_a ? args.scale_a[m] : 1.f) * sb;
                    const float v = epilogue_value_rt(x, cin, bias_v, args);
                    if (args.Q)
                        args.Q[n * args.ldq + m] = (int8_t)quantize_i8(v, args.scale[m], args.zp);
                    else
                        args.C[n * args.ldc + m] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xFFFFu);
                }
            }
        }
    }
}

}  // namespace gb
