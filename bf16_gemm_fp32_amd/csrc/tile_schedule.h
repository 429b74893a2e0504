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
//  * Tile order: grouped.  Tiles walk down GROUP_M tile-rows before moving
//    one tile-column right, so a contiguous run of the order covers a compact
//    block of C and its A rows and B columns stay in L2 -- the grouped
//    schedule of the worklog's "Kernel 6".  The 32 compute units of one XCD
//    run their tiles side by side in K, so an XCD's L2 traffic per round is
//    set by how many distinct tile-rows and tile-columns its 32 tiles touch:
//    GROUP_M = 4 gives a 4 x 8 block (12 operand panels), within 7% of the
//    best any 32-tile block can do (about 11.3 panels for a square), which
//    is also all a Hilbert curve (the worklog's "Kernel 11") could give here.
//    Panels are not reused between rounds through L2: at K = 4096 one panel
//    is 2 MiB, so a round's 12 panels stream through the 4 MiB L2.
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

struct TileSchedule {
    int tiles_m;   // ceil(M / BM)
    int tiles_n;   // ceil(N / BN)
    int group_m;   // tile-rows per group (grouped order)
    int grid;      // number of persistent workgroups
    int no_xcd_remap;  // nonzero: slot = workgroup id (for measuring the remap)

    GB_HD int num_tiles() const { return tiles_m * tiles_n; }

    // Slot of workgroup w under round-robin XCD dispatch.
    GB_HD int slot(int w) const {
        int per = grid / kNumXcds;
        if (no_xcd_remap || w >= per * kNumXcds) return w;
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

    // Tile coordinates of position t in the schedule's (grouped) order.
    GB_HD void tile(int t, int &tm, int &tn) const { grouped(t, tm, tn); }
};

}  // namespace gb
