// Host check of the XCD-aware tile mapping (dg_tiles.h): for each (tiles, workgroups, lead)
// case on the command line, every tile id in [0, tiles) must fall to exactly one workgroup,
// and with one workgroup per tile xcd_tile_owner must name that workgroup.  Prints
// "ok <tiles> <workgroups> <lead>" per case, or the first fault and exits non-zero.  With the
// single argument "tail" it checks the contiguous tail rule instead (tail_count).
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

// The tail rule (tail_count): worked cases, then the rule's properties over a range of sizes.
static int check_tail()
{
    struct Case {
        long long busy, tiles;
        int cus, want;
    };
    const Case cases[] = {
        {2112, 2080, 256, 64},  // 2080 tiles + two served straddles x 16: a wave of 64
        {2128, 2080, 256, 0},   // three straddles: 80 busy workgroups, over a quarter
        {2080, 2080, 256, 32},  // no straddle: exactly an eighth
        {2079, 2079, 256, 0},   // 31: under an eighth
        {304, 304, 256, 48},    //
        {48, 48, 256, 0},       // a lone partial wave: all of it, nothing to leave
        {5, 5, 4, 1},           //
        {100, 100, 0, 0},       // no CUs known
    };
    for (const Case &c : cases)
        if (dg::tail_count(c.busy, c.tiles, c.cus) != c.want) {
            printf("tail_count(%lld, %lld, %d) = %d, not %d\n", c.busy, c.tiles, c.cus,
                   dg::tail_count(c.busy, c.tiles, c.cus), c.want);
            return 1;
        }
    for (int cus = 1; cus <= 320; ++cus)
        for (long long busy = 0; busy <= 1200; ++busy)
            for (long long tiles : {busy, busy - 40}) {
                if (tiles <= 0)
                    continue;
                const int t = dg::tail_count(busy, tiles, cus);
                const long long r = busy % cus;
                const bool in = 8 * r >= cus && 4 * r <= cus && r < tiles;
                if (t != (in ? r : 0)) {
                    printf("tail_count(%lld, %lld, %d) = %d\n", busy, tiles, cus, t);
                    return 1;
                }
            }
    printf("ok tail\n");
    return 0;
}

int main(int argc, char **argv)
{
    if (argc == 2 && argv[1][0] == 't')
        return check_tail();
    for (int i = 1; i + 2 < argc; i += 3)
        if (check(atoll(argv[i]), atoi(argv[i + 1]), atoi(argv[i + 2])))
            return 1;
    return 0;
}
