// device_common.h -- gfx950 building blocks shared by the GEMM kernels:
// vector types, LDS/wait primitives, buffer resources, bf16 conversion and
// the fp32 epilogue arithmetic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gb {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define GB_LDS __attribute__((address_space(3)))

// Epilogue flags (uniform across the grid).  GELU and ReLU exclude each
// other, so twelve combinations exist.
enum : uint32_t { kEpiBeta = 1u, kEpiBias = 2u, kEpiGelu = 4u, kEpiRelu = 8u };

struct GemmArgs {
    int64_t M, N, K;
    const uint16_t *A;
    int64_t lda;
    const uint16_t *B;
    int64_t ldb;
    uint16_t *C;
    int64_t ldc;
    float alpha, beta;
    const uint16_t *bias;
    uint32_t flags;  // kEpi* bits
    // int8 output (the quantizing entry point only): Q[m + n*ldq] =
    // sat8(rne(fma(v, scale[m], zp))); unused by the bf16 kernels.
    int8_t *Q;
    int64_t ldq;
    const float *scale;
    float zp;
    // fp8 inputs (the fp8 entry point only): A and B hold OCP FP8 E4M3 bytes
    // (lda, ldb in bytes) and the product is scaled by scale_a[m] and
    // scale_b[n] when given.
    const float *scale_a;
    const float *scale_b;
};

// The K split of the tile kernel: `splits` ranges of `kper` K-slices (the
// last may be shorter, none is empty); partial s of the element (m, n) is
// P[s * pstride + n * ldp + m].  tile_major: work unit u is tile u / splits,
// range u % splits (a tile's ranges in consecutive units, so on one XCD);
// otherwise range u / tiles, tile u % tiles.
struct TileSplit {
    float *P;
    int64_t ldp, pstride;
    int splits, kper;
    int tile_major;
};

// Call f(std::integral_constant<uint32_t, flags>) for the run-time flag word,
// so each launcher instantiates its kernel once per valid combination.
template <class F>
__host__ inline void dispatch_flags(uint32_t flags, F &&f) {
    switch (flags) {
    case 0: f(std::integral_constant<uint32_t, 0>{}); break;
    case 1: f(std::integral_constant<uint32_t, 1>{}); break;
    case 2: f(std::integral_constant<uint32_t, 2>{}); break;
    case 3: f(std::integral_constant<uint32_t, 3>{}); break;
    case 4: f(std::integral_constant<uint32_t, 4>{}); break;
    case 5: f(std::integral_constant<uint32_t, 5>{}); break;
    case 6: f(std::integral_constant<uint32_t, 6>{}); break;
    case 7: f(std::integral_constant<uint32_t, 7>{}); break;
    case 8: f(std::integral_constant<uint32_t, 8>{}); break;
    case 9: f(std::integral_constant<uint32_t, 9>{}); break;
    case 10: f(std::integral_constant<uint32_t, 10>{}); break;
    default: f(std::integral_constant<uint32_t, 11>{}); break;
    }
}

// ---------------------------------------------------------------- waits ---
// Explicit waits and barriers as inline asm with a memory clobber: the
// compiler may not move memory operations across them, and __syncthreads()
// would force vmcnt(0), draining the load pipeline we keep in flight.

// All LDS reads of this wave have landed, then a workgroup barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt immediate (gfx9 encoding) that waits for lgkmcnt == 0 only.
constexpr int kWaitLgkm0 = 0xC07F;

// At most N vector-memory operations of this wave still outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ---------------------------------------------------- buffer resources ---
// Raw (stride 0) buffer: num_records bytes from base; loads past the end
// return zero.  Word 3 = 0x00020000 selects the 32-bit data format that
// untyped buffer loads need on gfx9-family parts.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// A buffer offset past every resource this library builds (their sizes and
// offsets stay below 2^31, checked on the host): a load from it is out of
// range and returns zeros -- also into LDS for the direct-to-LDS form.
constexpr uint32_t kOobOffset = 0x80000000u;

// 16-byte per lane direct load from a buffer into LDS.  Lane i of the wave
// writes lds_base + 16*i; lds_base must be wave-uniform.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rsrc, GB_LDS void *lds_base,
                                                  uint32_t voffset, uint32_t soffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds_base, 16, voffset, soffset, 0, 0);
}

// ------------------------------------------------------------ bf16 math ---
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __builtin_bit_cast(float, bits16 << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (round to nearest even) packed low|high: a single
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// GELU, tanh form: 0.5 y (1 + tanh(u)), u = sqrt(2/pi) (y + 0.044715 y^3).
// Uses the identity 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)), evaluated with
// the hardware base-2 exponential and reciprocal, and folds the constants
// so that -2u log2(e) = y (c1 + c3 y^2): one multiply, one fused multiply-add
// and one multiply before the exponential.  Both limits are exact: exp ->
// inf gives y * 0 (large negative y), exp -> 0 gives y.
__device__ __forceinline__ float gelu_tanh_f32(float y) {
    // c1 = -2 log2(e) sqrt(2/pi), c3 = 0.044715 c1
    const float kC1 = -2.30220819814432500f;
    const float kC3 = -0.10294323958002350f;
    const float y2 = y * y;
    const float e = __builtin_amdgcn_exp2f(y * __builtin_fmaf(kC3, y2, kC1));
    return y * __builtin_amdgcn_rcpf(1.0f + e);
}

// OCP FP8 E4M3 byte -> bf16 bits, exactly (every E4M3 value is a bf16
// value): normal values re-bias the exponent (7 -> 127), subnormals m * 2^-9
// go through an exact fp32 product, S.1111.111 is NaN.
__device__ __forceinline__ uint32_t fp8_e4m3_to_bf16_bits(uint32_t b) {
    const uint32_t s = (b & 0x80u) << 8;
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    if (e == 15u && m == 7u) return s | 0x7FC0u;
    if (e != 0u) return s | ((e + 120u) << 7) | (m << 4);
    return s | (__builtin_bit_cast(uint32_t, (float)m * 0x1p-9f) >> 16);
}

// ReLU: negative values become 0; NaN passes through (a compare-select, not
// v_max_f32, which would return 0 for NaN).
__device__ __forceinline__ float relu_f32(float y) { return y < 0.f ? 0.f : y; }

// alpha*acc (+ beta*c_in) (+ bias) then the activation, all in fp32, with the
// epilogue flags known at compile time (the tile kernels are instantiated per
// flag combination, so the plain product carries no epilogue code at all).
template <uint32_t kFlags>
__device__ __forceinline__ float epilogue_value(float acc, float c_in, float bias_v, float alpha, float beta) {
    float v = alpha * acc;
    if constexpr ((kFlags & kEpiBeta) != 0) v += beta * c_in;
    if constexpr ((kFlags & kEpiBias) != 0) v += bias_v;
    if constexpr ((kFlags & kEpiGelu) != 0) v = gelu_tanh_f32(v);
    if constexpr ((kFlags & kEpiRelu) != 0) v = relu_f32(v);
    return v;
}

// The same with run-time flags (the bounds-checked kernel).
__device__ __forceinline__ float epilogue_value_rt(float acc, float c_in, float bias_v, const GemmArgs &a) {
    float v = a.alpha * acc;
    if (a.flags & kEpiBeta) v += a.beta * c_in;
    if (a.flags & kEpiBias) v += bias_v;
    if (a.flags & kEpiGelu) v = gelu_tanh_f32(v);
    if (a.flags & kEpiRelu) v = relu_f32(v);
    return v;
}

// Per-row int8 quantization of an epilogue value: one fused multiply-add in
// fp32, round to nearest even, saturate to [-128, 127]; NaN gives 0 (the
// DeepGEMM article, section 6.2: y = round(x * scale + zero_point), one
// scale per row).
__device__ __forceinline__ int32_t quantize_i8(float v, float scale, float zp) {
    const float t = __builtin_fmaf(v, scale, zp);
    if (!(t == t)) return 0;
    const float r = __builtin_rintf(t);
    return (int32_t)(r < -128.f ? -128.f : (r > 127.f ? 127.f : r));
}

__device__ __forceinline__ f32x16 mfma_32x32x16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// E4M3 x E4M3 block, fp32 accumulate: format selectors 0 / 0 (FP8 E4M3 for
// both operands) and unit block scales (E8M0 exponent 127 = 2^0).  Each lane
// supplies 32 bytes (32 values) of its row of A and of its column of B;
// which 32 of the block's 64 k a lane holds is free as long as A and B agree.
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(const i32x8 &a, const i32x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

}  // namespace gb
