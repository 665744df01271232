// Answers queries about lin_bwd's host-side sizing decisions (dispatch.h) on
// stdin, one per line, so that they can be checked without a GPU:
//   span n0 l0 n1 l1              -> launch length in slabs
//   tile M K ntx rx ntw rw cap    -> dX reduction ranges on the tile kernel
//   tlen N sx                     -> ranges and range length for sx
//   red N chunk units M K cap     -> small-M kernel splits and split length
//   pair M K N                    -> 1 if both small-M products share a launch
//   r16 M K N                     -> 1 if dX sums whole reductions at small M
#include "dispatch.h"

#include <cstdio>
#include <cstring>

int main() {
    char op[16];
    while (std::scanf("%15s", op) == 1) {
        long long v[8] = {0};
        if (!std::strcmp(op, "span")) {
            if (std::scanf("%lld %lld %lld %lld", v, v + 1, v + 2, v + 3) != 4)
                return 2;
            std::printf("%lld\n", (long long)lb::plan::launch_span(v[0], v[1], v[2], v[3]));
        } else if (!std::strcmp(op, "tile")) {
            if (std::scanf("%lld %lld %lld %lld %lld %lld %lld", v, v + 1, v + 2, v + 3, v + 4, v + 5, v + 6) != 7)
                return 2;
            std::printf("%d\n", lb::plan::tile_dx_splits(v[0], v[1], v[2], v[3], v[4], v[5], v[6]));
        } else if (!std::strcmp(op, "tlen")) {
            if (std::scanf("%lld %lld", v, v + 1) != 2)
                return 2;
            const lb::plan::Split s = lb::plan::tile_split_len(v[0], (int)v[1]);
            std::printf("%lld %lld\n", (long long)s.splits, (long long)s.len);
        } else if (!std::strcmp(op, "red")) {
            if (std::scanf("%lld %lld %lld %lld %lld %lld", v, v + 1, v + 2, v + 3, v + 4, v + 5) != 6)
                return 2;
            const lb::plan::Split s = lb::plan::reduction_split(v[0], v[1], v[2], v[3], v[4], v[5]);
            std::printf("%lld %lld\n", (long long)s.splits, (long long)s.len);
        } else if (!std::strcmp(op, "pair")) {
            if (std::scanf("%lld %lld %lld", v, v + 1, v + 2) != 3)
                return 2;
            std::printf("%d\n", lb::plan::pair_fits(v[0], v[1], v[2]) ? 1 : 0);
        } else if (!std::strcmp(op, "r16")) {
            if (std::scanf("%lld %lld %lld", v, v + 1, v + 2) != 3)
                return 2;
            std::printf("%d\n", lb::plan::rows16_fits(v[0], v[1], v[2]) ? 1 : 0);
        } else {
            return 2;
        }
    }
    return 0;
}
