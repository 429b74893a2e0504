// kernel_gemv.h -- matrix-vector kernel for decode-sized products (1 to 4
// rows of C).
//
// At M = 1 the product is a matrix-vector product: every byte of B is used
// once, so the work is streaming B (K x N, column-major, so each column is
// K-contiguous) from HBM at full bandwidth.  The DeepGEMM article
// (demingchina.com, section 5.1) reports its tiled kernel at about 15% of
// peak on 1 x 4096 x 4096 because most of a tile's work is spent on rows
// that do not exist; here there are no tiles, no LDS and no MFMA.
//
// Each wave owns kCols consecutive columns of C.  K is walked in blocks of
// 512 * kChunks: in a block, lane l holds the 16-byte chunks at
// k = k0 + 512 j + 8 l (j < kChunks) of every row of A and of each of its
// columns of B, all loaded into registers before any arithmetic, so a wave
// has kCols * kChunks KiB of B in flight.  Each lane accumulates its share
// of the M x kCols dot products in fp32 (bf16 products are exact in fp32),
// a butterfly over the 64 lanes adds the shares, and one lane per output
// applies alpha, beta*C, bias and the activation and writes the bf16 value.
// Chunks past K, columns past N and rows past M are loaded from an
// out-of-range buffer offset and read as zeros.
//
// kFp8: A and B hold OCP FP8 E4M3 bytes (the FP8 input path of the DeepGEMM
// article, sections 1.2 and 6.3): a 16-byte chunk is 16 values, decoded
// exactly in registers (every E4M3 value is a bf16 value), so lane l's
// chunks sit at k = k0 + 1024 j + 16 l; the sum is scaled by scale_a[m] and
// scale_b[n] before the epilogue.
#pragma once

#include "device_common.h"

namespace gb {

struct GemvConfig {
    static constexpr int kCols = 2;      // columns of C per wave
    static constexpr int kChunks = 4;    // 16-byte chunks per lane per column and K-block
    static constexpr int kBlockBytes = 1024 * kChunks;  // bytes of a row or column per K-block
    static constexpr int kWaves = 4;     // waves per workgroup
    static constexpr int kThreads = 64 * kWaves;
};

typedef uint32_t gemv_u32x4 __attribute__((ext_vector_type(4)));

// 16 bytes per lane from a buffer (zeros past its end).  kStream sets the
// non-temporal cache policy bit: B is read once, so it should not displace
// the cached A; it measured up to 12% faster on products of 64 MiB and more.
template <bool kStream>
__device__ __forceinline__ gemv_u32x4 load16_zero(__amdgpu_buffer_rsrc_t r, uint32_t voffset) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0u, kStream ? 2 : 0);
}

// Sum of the 8 products of two 16-byte bf16 chunks, added to acc in fp32.
__device__ __forceinline__ float dot8_bf16(const gemv_u32x4 &a, const gemv_u32x4 &b, float acc) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        acc = __builtin_fmaf(bf16_bits_to_f32(a[e] & 0xFFFFu), bf16_bits_to_f32(b[e] & 0xFFFFu), acc);
        acc = __builtin_fmaf(bf16_bits_to_f32(a[e] >> 16), bf16_bits_to_f32(b[e] >> 16), acc);
    }
    return acc;
}

// The 16 values of a chunk of E4M3 bytes as fp32, two per v_cvt_pk_f32_fp8
// (on gfx950 it decodes the OCP E4M3 encoding exactly: all 256 codes,
// subnormals and NaN included, agree with the exact decode).
__device__ __forceinline__ void decode16_fp8(const gemv_u32x4 &v, float (&out)[16]) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[w], false);
        const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[w], true);
        out[4 * w + 0] = lo.x;
        out[4 * w + 1] = lo.y;
        out[4 * w + 2] = hi.x;
        out[4 * w + 3] = hi.y;
    }
}

// Requirements checked by the host: 1 <= M <= kRows, N >= 1, K a multiple
// of one 16-byte chunk (8 values, 16 with kFp8), A and B 16-byte aligned,
// lda and ldb multiples of a chunk, and the byte offsets of kRows rows of A
// and kCols columns of B (plus K) below 2^31 (the host checks with 4 for
// both).
// C may have any ldc >= M (2-byte stores).
template <int kRows, uint32_t kFlags, bool kFp8 = false>
__global__ void __launch_bounds__(GemvConfig::kThreads) gemm_gemv_kernel(const GemmArgs args) {
    using Cfg = GemvConfig;
    constexpr int kElem = kFp8 ? 1 : 2;        // bytes per value
    constexpr int kPerChunk = 16 / kElem;      // values per 16-byte chunk
    const int lane = threadIdx.x & 63;
    // The wave index through readfirstlane: the compiler then knows n0, and
    // the B buffer descriptor built from it, to be wave-uniform and keeps
    // them in scalar registers (a descriptor it must assume divergent costs
    // a readfirstlane loop around every load).
    const int64_t wave = (int64_t)blockIdx.x * Cfg::kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t n0 = wave * Cfg::kCols;
    if (n0 >= args.N) return;  // whole wave past the last column (wave-uniform)
    const int cols = (int)(args.N - n0 < Cfg::kCols ? args.N - n0 : Cfg::kCols);

    const char *A8 = reinterpret_cast<const char *>(args.A);
    const char *B8 = reinterpret_cast<const char *>(args.B);
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(A8, (uint32_t)(((args.M - 1) * args.lda + args.K) * kElem));
    const __amdgpu_buffer_rsrc_t rB =
        make_rsrc(B8 + n0 * args.ldb * kElem, (uint32_t)(((cols - 1) * args.ldb + args.K) * kElem));
    const uint32_t lda_bytes = (uint32_t)(args.lda * kElem), ldb_bytes = (uint32_t)(args.ldb * kElem);

    float acc[kRows][Cfg::kCols];
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int c = 0; c < Cfg::kCols; ++c) acc[r][c] = 0.f;

    constexpr int kBlockK = Cfg::kBlockBytes / kElem;  // values per K-block
    for (int64_t k0 = 0; k0 < args.K; k0 += kBlockK) {
        gemv_u32x4 b[Cfg::kCols][Cfg::kChunks], a[kRows][Cfg::kChunks];
        // B first: it comes from HBM, A (a few KiB shared by every wave)
        // from L2.
#pragma unroll
        for (int j = 0; j < Cfg::kChunks; ++j) {
            const int64_t k = k0 + 64 * kPerChunk * j + kPerChunk * lane;
            const bool kin = k < args.K;
#pragma unroll
            for (int c = 0; c < Cfg::kCols; ++c) {
                const uint32_t off =
                    (kin && c < cols) ? (uint32_t)c * ldb_bytes + (uint32_t)(k * kElem) : kOobOffset;
                b[c][j] = load16_zero<true>(rB, off);
            }
        }
#pragma unroll
        for (int j = 0; j < Cfg::kChunks; ++j) {
            const int64_t k = k0 + 64 * kPerChunk * j + kPerChunk * lane;
            const bool kin = k < args.K;
#pragma unroll
            for (int r = 0; r < kRows; ++r) {
                const uint32_t off =
                    (kin && r < args.M) ? (uint32_t)r * lda_bytes + (uint32_t)(k * kElem) : kOobOffset;
                a[r][j] = load16_zero<false>(rA, off);
            }
        }
#pragma unroll
        for (int j = 0; j < Cfg::kChunks; ++j) {
            if constexpr (kFp8) {
                float fa[kRows][16];
#pragma unroll
                for (int r = 0; r < kRows; ++r) decode16_fp8(a[r][j], fa[r]);
#pragma unroll
                for (int c = 0; c < Cfg::kCols; ++c) {
                    float fb[16];
                    decode16_fp8(b[c][j], fb);
#pragma unroll
                    for (int r = 0; r < kRows; ++r)
#pragma unroll
                        for (int e = 0; e < 16; ++e) acc[r][c] = __builtin_fmaf(fa[r][e], fb[e], acc[r][c]);
                }
            } else {
#pragma unroll
                for (int r = 0; r < kRows; ++r)
#pragma unroll
                    for (int c = 0; c < Cfg::kCols; ++c) acc[r][c] = dot8_bf16(a[r][j], b[c][j], acc[r][c]);
            }
        }
    }

    // Butterfly: afterwards every lane holds the full sums.
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int c = 0; c < Cfg::kCols; ++c)
#pragma unroll
            for (int s = 32; s >= 1; s >>= 1) acc[r][c] += __shfl_xor(acc[r][c], s, 64);

    // Lane r * kCols + c writes element (r, n0 + c).
    float v = 0.f;
    int r_out = 0, c_out = 0;
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int c = 0; c < Cfg::kCols; ++c)
            if (lane == r * Cfg::kCols + c) {
                v = acc[r][c];
                r_out = r;
                c_out = c;
            }
    if (lane < kRows * Cfg::kCols && r_out < args.M && c_out < cols) {
        const int64_t n = n0 + c_out;
        uint16_t *p = args.C + n * args.ldc + r_out;
        float cin = 0.f, bias_v = 0.f;
        if constexpr ((kFlags & kEpiBeta) != 0) cin = bf16_bits_to_f32(*p);
        if constexpr ((kFlags & kEpiBias) != 0) bias_v = bf16_bits_to_f32(args.bias[n]);
        if constexpr (kFp8) {
            const float sa = args.scale_a ? args.scale_a[r_out] : 1.f;
            const float sb = args.scale_b ? args.scale_b[n] : 1.f;
            v = v * sa * sb;
        }
        const float y = epilogue_value<kFlags>(v, cin, bias_v, args.alpha, args.beta);
        *p = (uint16_t)(pack_bf16x2(y, 0.f) & 0xFFFFu);
    }
}

// One launch per call: waves of kCols columns, four waves per workgroup.
// Two columns and K-blocks of 2048 per wave measured fastest (small waves:
// many resident per SIMD hide each other's memory latency).
template <int kRows, bool kFp8>
hipError_t launch_gemv_rows(const GemmArgs &args, hipStream_t stream) {
    const int64_t waves = (args.N + GemvConfig::kCols - 1) / GemvConfig::kCols;
    const int64_t blocks = (waves + GemvConfig::kWaves - 1) / GemvConfig::kWaves;
    dispatch_flags(args.flags, [&](auto f) {
        hipLaunchKernelGGL((gemm_gemv_kernel<kRows, decltype(f)::value, kFp8>), dim3((unsigned)blocks),
                           dim3(GemvConfig::kThreads), 0, stream, args);
    });
    return hipGetLastError();
}

}  // namespace gb
