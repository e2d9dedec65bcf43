// Host check of the XCD-aware tile mapping (dg_tiles.h): for each (tiles, workgroups, lead)
// case on the command line, every tile id in [0, tiles) must fall to exactly one workgroup,
// and with one workgroup per tile xcd_tile_owner must name that workgroup.  Prints
// "ok <tiles> <workgroups> <lead>" per case, or the first fault and exits non-zero.
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "dg_tiles.h"

static int check(long long total, int workgroups, int lead)
{
    std::vector<unsigned char> hits((size_t)total, 0);
    std::vector<int> owner((size_t)total, -1);
    const int grid = workgroups + lead;
    for (int id = lead; id < grid; ++id) {
        const dg::TileRange r = dg::xcd_tile_range(total, grid, lead, id);
        if (r.step <= 0) {
            printf("bad step %d at id %d\n", r.step, id);
            return 1;
        }
        for (long long t = r.first; t < r.end; t += r.step) {
            if (t < 0 || t >= total) {
                printf("tile %lld out of range at id %d (%d..%d step %d)\n", t, id, r.first,
                       r.end, r.step);
                return 1;
            }
            if (++hits[(size_t)t] > 1) {
                printf("tile %lld covered twice (id %d)\n", t, id);
                return 1;
            }
            owner[(size_t)t] = id;
        }
    }
    for (long long t = 0; t < total; ++t)
        if (hits[(size_t)t] != 1) {
            printf("tile %lld never covered\n", t);
            return 1;
        }
    if (total == workgroups)
        for (long long t = 0; t < total; ++t)
            if (dg::xcd_tile_owner((int)total, lead, (int)t) != owner[(size_t)t]) {
                printf("owner of tile %lld: %d, not %d\n", t,
                       dg::xcd_tile_owner((int)total, lead, (int)t), owner[(size_t)t]);
                return 1;
            }
    printf("ok %lld %d %d\n", total, workgroups, lead);
    return 0;
}

int main(int argc, char **argv)
{
    for (int i = 1; i + 2 < argc; i += 3)
        if (check(atoll(argv[i]), atoi(argv[i + 1]), atoi(argv[i + 2])))
            return 1;
    return 0;
}
