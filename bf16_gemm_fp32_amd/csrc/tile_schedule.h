// tile_schedule.h -- which output tile each persistent workgroup computes.
//
// The grid holds one workgroup per compute unit (at most); workgroup slot s
// takes tiles order[s], order[s + G], order[s + 2G], ... (G = grid size),
// the persistent loop of "Outperforming cuBLAS on H100: a worklog", section
// "Kernel 6" (with the stride equal to the grid size).
//
// Two MI355X-specific pieces:
//  * XCD remap.  Workgroup ids are dispatched round-robin over the 8
//    accelerator dies (XCDs), each with its own L2.  Workgroup w runs on XCD
//    w % 8, so it is given slot (w % 8) * (G / 8) + w / 8: the 32 compute
//    units of one XCD take a contiguous run of the tile order.  Workgroups
//    past the last multiple of 8 keep their own id (the map stays a
//    bijection for any G).
//  * Tile order.  "grouped": tiles walk down GROUP_M tile-rows before moving
//    one tile-column right, so a contiguous run of the order covers a compact
//    block of C and its A rows and B columns stay in L2 -- the grouped
//    schedule of the worklog's "Kernel 6".  "hilbert": a Hilbert curve over
//    the tile grid, the worklog's "Kernel 11", kept as a measured alternative.
//
// Everything here is plain integer code usable on host and device, so the
// host tests check it is a bijection.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define GB_HD __host__ __device__ __forceinline__
#else
#define GB_HD inline
#endif

namespace gb {

constexpr int kNumXcds = 8;

enum TileOrder : int { kOrderGrouped = 0, kOrderHilbert = 1 };

struct TileSchedule {
    int tiles_m;   // ceil(M / BM)
    int tiles_n;   // ceil(N / BN)
    int group_m;   // tile-rows per group (grouped order)
    int grid;      // number of persistent workgroups
    int order;     // TileOrder
    int hilbert_log2;  // side of the enclosing power-of-two square (hilbert)

    GB_HD int num_tiles() const { return tiles_m * tiles_n; }

    // Slot of workgroup w under round-robin XCD dispatch.
    GB_HD int slot(int w) const {
        int per = grid / kNumXcds;
        if (w >= per * kNumXcds) return w;
        return (w % kNumXcds) * per + w / kNumXcds;
    }

    // Tile coordinates of position t in the grouped order.
    GB_HD void grouped(int t, int &tm, int &tn) const {
        int group_size = group_m * tiles_n;
        int g = t / group_size;
        int first_m = g * group_m;
        int gm = tiles_m - first_m;
        if (gm > group_m) gm = group_m;
        int r = t - g * group_size;
        tm = first_m + r % gm;
        tn = r / gm;
    }

    // Hilbert curve index d -> (x, y) on a 2^k x 2^k square.
    GB_HD static void hilbert_d2xy(int log2n, int d, int &x, int &y) {
        x = 0;
        y = 0;
        for (int s = 1; s < (1 << log2n); s <<= 1) {
            int rx = 1 & (d >> 1);
            int ry = 1 & (d ^ rx);
            if (ry == 0) {
                if (rx == 1) {
                    x = s - 1 - x;
                    y = s - 1 - y;
                }
                int tmp = x;
                x = y;
                y = tmp;
            }
            x += s * rx;
            y += s * ry;
            d >>= 2;
        }
    }

    // Tile coordinates of position t in the schedule's order.  For the
    // Hilbert order, positions of the power-of-two square that fall outside
    // the tile grid are skipped by ranking: position t is the t-th in-grid
    // cell along the curve.  The host precomputes nothing; the device walks
    // the curve from the previous position (see next_hilbert).
    GB_HD void tile(int t, int &tm, int &tn) const { grouped(t, tm, tn); }
};

// Hilbert order over a tiles_m x tiles_n grid, iterated incrementally: the
// caller keeps the curve position d and asks for the next in-grid cell at
// least `skip` cells further along.  Cells outside the grid are passed over.
struct HilbertWalker {
    int d;        // current position on the curve (-1 before the first call)
    int log2n;
    int tiles_m, tiles_n;

    // Advance by `count` in-grid cells; returns false when the curve ends.
    GB_HD bool advance(int count, int &tm, int &tn) {
        const int total = 1 << (2 * log2n);
        while (count > 0) {
            ++d;
            if (d >= total) return false;
            int x, y;
            TileSchedule::hilbert_d2xy(log2n, d, x, y);
            if (x < tiles_m && y < tiles_n) {
                --count;
                tm = x;
                tn = y;
            }
        }
        return true;
    }
};

GB_HD int ceil_log2(int v) {
    int k = 0;
    while ((1 << k) < v) ++k;
    return k;
}

}  // namespace gb
