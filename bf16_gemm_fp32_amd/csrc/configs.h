// configs.h -- the tile-kernel configurations and their launch entry points
// (each configuration's kernels live in a translation unit of their own so
// the library builds in parallel).
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"

namespace gb {

// 256x256 output tiles with four waves of 128x128 (256 fp32 accumulators per
// lane, the AGPR half of the register file at one wave per SIMD) for large
// grids, K-slices of 32 in a 5-deep LDS ring (all 160 KiB) so every slice's
// loads have more than two slices to land.  128x128 tiles with four waves of
// 64x64 when the 256-tiles would leave most compute units idle.
struct ShapeL { static constexpr int BM = 256, BN = 256, BK = 32; };
struct ShapeM { static constexpr int BM = 128, BN = 128, BK = 64; };
// 256x256 output tiles with K-slices of 64 (full 128-byte operand rows) in
// a ring of five 32 KiB single-operand units.
struct ShapeRing { static constexpr int BM = 256, BN = 256, BK = 64; };

// Short-and-wide products (at most 64 rows): one workgroup per strip of 32,
// 64 or 128 columns and range of K (split-K) streams B once; K-slices of 256
// for 32- and 64-column strips, 128 for 128-column ones, 512 FP8 values (the
// same 512 bytes) for FP8 operands.
struct ShapeSkinny { static constexpr int KS_N32 = 256, KS_N64 = 256, KS_N128 = 128, KS_FP8 = 512; };

struct SkinnyWork;

// FP8 (E4M3) operands: 256x256 output tiles, K-slices of 128 fp8 (one
// 128-byte line per operand row).
struct ShapeFp8 { static constexpr int BM = 256, BN = 256, BK = 128; };
// FP8 on the 128x128 tiles for small and mid-sized grids: K-slices of 128
// values (128-byte rows, the bytes of a bf16 slice of 64).
struct ShapeFp8M { static constexpr int BM = 128, BN = 128, BK = 128; };

hipError_t launch_tile_large(const GemmArgs &args, int cus, hipStream_t stream);
hipError_t launch_tile_medium(const GemmArgs &args, int cus, hipStream_t stream);
// split-K on the 128x128 tiles (split.P: splits * M * N floats of workspace)
hipError_t launch_tile_medium_splitk(const GemmArgs &args, const TileSplit &split, int cus, hipStream_t stream);
// the same with int8 output (the reduction quantizes per row)
hipError_t launch_tile_medium_splitk_q8(const GemmArgs &args, const TileSplit &split, int cus,
                                        hipStream_t stream);
// the same with tails (zero-filled loads, masked epilogue; split.P padded
// to tile multiples)
hipError_t launch_tile_medium_masked(const GemmArgs &args, int cus, hipStream_t stream);
hipError_t launch_tile_medium_splitk_masked(const GemmArgs &args, const TileSplit &split, int cus,
                                            hipStream_t stream);
hipError_t launch_tile_medium_splitk_q8_masked(const GemmArgs &args, const TileSplit &split, int cus,
                                               hipStream_t stream);
hipError_t launch_tile_ring_mfma32(const GemmArgs &args, int cus, hipStream_t stream);
hipError_t launch_tile_ring(const GemmArgs &args, int cus, hipStream_t stream);
// the same tiles on eight waves of 128x64, two per SIMD (chosen only when forced)
hipError_t launch_tile_ring_w8(const GemmArgs &args, int cus, hipStream_t stream);
hipError_t launch_tile_ring_masked(const GemmArgs &args, int cus, hipStream_t stream);
// int8 output: exact tile multiples, and shapes with tails (masked)
hipError_t launch_tile_ring_q8(const GemmArgs &args, int cus, hipStream_t stream);
hipError_t launch_tile_ring_q8_masked(const GemmArgs &args, int cus, hipStream_t stream);
// FP8 tiles on 16x16x128 MFMAs: exact multiples (the default), and shapes
// with tails (chosen only when forced)
hipError_t launch_tile_fp8(const GemmArgs &args, int cus, hipStream_t stream);
hipError_t launch_tile_fp8_mfma16_masked(const GemmArgs &args, int cus, hipStream_t stream);
// the same tiles on 32x32x64 MFMAs: shapes with tails (the default), and
// exact multiples (chosen only when forced)
hipError_t launch_tile_fp8_mfma32_masked(const GemmArgs &args, int cus, hipStream_t stream);
hipError_t launch_tile_fp8_mfma32(const GemmArgs &args, int cus, hipStream_t stream);
// FP8 on the 128x128 tiles (32x32x64 MFMAs): whole K and split-K, exact
// multiples and shapes with tails (split.P as for the bf16 128x128 split)
hipError_t launch_tile_fp8_medium(const GemmArgs &args, int cus, hipStream_t stream);
hipError_t launch_tile_fp8_medium_masked(const GemmArgs &args, int cus, hipStream_t stream);
hipError_t launch_tile_fp8_medium_splitk(const GemmArgs &args, const TileSplit &split, int cus, hipStream_t stream);
hipError_t launch_tile_fp8_medium_splitk_masked(const GemmArgs &args, const TileSplit &split, int cus,
                                                hipStream_t stream);
// split-K on the 32x32x64 FP8 tiles (split.P: splits * M * N floats of workspace)
hipError_t launch_tile_fp8_splitk(const GemmArgs &args, const TileSplit &split, int cus, hipStream_t stream);
hipError_t launch_tile_fp8_splitk_masked(const GemmArgs &args, const TileSplit &split, int cus,
                                         hipStream_t stream);
// matrix-vector products: 1 <= M <= 4 (fp8: E4M3 operands)
hipError_t launch_gemv(const GemmArgs &args, hipStream_t stream, bool fp8 = false);
// rows: 32 or 64 (the kernel's row block, M <= rows); cols: strip width
hipError_t launch_skinny(int rows, int cols, const GemmArgs &args, const SkinnyWork &work, int cus,
                         hipStream_t stream);
// the same on a transposed product (args already transposed: M' = N <= 64),
// writing C' transposed into C
hipError_t launch_skinny_t(int rows, int cols, const GemmArgs &args, const SkinnyWork &work, int cus,
                           hipStream_t stream);
// int8 output (per-row scale, zero point), 32-column strips
hipError_t launch_skinny_q8(int rows, const GemmArgs &args, const SkinnyWork &work, int cus, hipStream_t stream);
// FP8 (E4M3) operands, 32-column strips with slices of KS_FP8 values
hipError_t launch_skinny_fp8(int rows, const GemmArgs &args, const SkinnyWork &work, int cus, hipStream_t stream);
// the int8-output and FP8 instances on a transposed product (args already
// transposed, FP8 scales swapped), writing C' (and Q') transposed
hipError_t launch_skinny_q8_t(int rows, const GemmArgs &args, const SkinnyWork &work, int cus, hipStream_t stream);
hipError_t launch_skinny_fp8_t(int rows, const GemmArgs &args, const SkinnyWork &work, int cus,
                               hipStream_t stream);

}  // namespace gb
