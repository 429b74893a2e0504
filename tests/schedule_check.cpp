// Host check of tile_schedule.h: for many (tiles_m, tiles_n, group_m, grid)
// the persistent schedule must visit every tile exactly once and the XCD
// slot map must be a bijection.  Prints one line per failure and "OK" at the end.
// Also prints, for the 4096^3 launch (16x16 tiles of 256, grid 256), how
// many distinct tile-rows and tile-columns each XCD touches in round 0.
#include <cstdio>
#include <set>
#include <vector>

#include "tile_schedule.h"

using gb::TileSchedule;

static int failures = 0;

static void check(int tm_, int tn_, int gm, int grid) {
    TileSchedule s{};
    s.tiles_m = tm_;
    s.tiles_n = tn_;
    s.group_m = gm;
    s.grid = grid;
    std::vector<int> slot_seen(grid, 0);
    for (int w = 0; w < grid; ++w) {
        int sl = s.slot(w);
        if (sl < 0 || sl >= grid || slot_seen[sl]++) {
            std::printf("slot map not a bijection: tiles %dx%d grid %d w %d\n", tm_, tn_, grid, w);
            ++failures;
            return;
        }
    }
    std::vector<int> seen(tm_ * tn_, 0);
    for (int w = 0; w < grid; ++w)
        for (int t = s.slot(w); t < s.num_tiles(); t += grid) {
            int a, b;
            s.tile(t, a, b);
            if (a < 0 || a >= tm_ || b < 0 || b >= tn_ || seen[a * tn_ + b]++) {
                std::printf("tile visited twice or out of range: %dx%d g%d grid %d t %d -> (%d,%d)\n", tm_, tn_,
                            gm, grid, t, a, b);
                ++failures;
                return;
            }
        }
    for (int i = 0; i < tm_ * tn_; ++i)
        if (!seen[i]) {
            std::printf("tile never visited: %dx%d g%d grid %d tile %d\n", tm_, tn_, gm, grid, i);
            ++failures;
            return;
        }
}

int main() {
    const int dims[] = {1, 2, 3, 5, 8, 16, 17, 32, 56, 64};
    const int groups[] = {1, 2, 4, 8};
    const int grids[] = {1, 7, 8, 64, 100, 256, 257};
    for (int a : dims)
        for (int b : dims)
            for (int g : groups)
                for (int grid : grids) {
                    int tiles = a * b;
                    check(a, b, g, grid < tiles ? grid : tiles);
                }
    // locality of the 4096^3 launch
    TileSchedule s{16, 16, 4, 256};
    for (int x = 0; x < gb::kNumXcds; ++x) {
        std::set<int> rows, cols;
        for (int w = x; w < 256; w += gb::kNumXcds) {
            int a, b;
            s.tile(s.slot(w), a, b);
            rows.insert(a);
            cols.insert(b);
        }
        std::printf("xcd %d rows %zu cols %zu\n", x, rows.size(), cols.size());
    }
    if (failures == 0) std::printf("OK\n");
    return failures ? 1 : 0;
}
