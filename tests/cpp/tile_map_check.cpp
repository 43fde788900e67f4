// Host check of the workgroup -> tile remap used by the matrix-core kernels:
// for many grid shapes and group sizes, every tile must be produced exactly
// once and lie inside the grid, and the workgroups one XCD runs (ids equal
// mod 8) must form one contiguous range of the remapped order.
#include <cstdio>
#include <vector>

#include "common.h"

int main()
{
    const int sizes[] = {1, 2, 3, 7, 8, 9, 16, 17, 31, 32, 33, 63, 64, 65, 129, 257};
    const int groups[] = {1, 2, 4, 8, 16};
    long checked = 0;
    for (int tm_ : sizes)
        for (int tn_ : sizes)
            for (int gm : groups) {
                const int nb = tm_ * tn_;
                std::vector<int> seen(nb, 0);
                for (int b = 0; b < nb; ++b) {
                    int tm = -1, tn = -1;
                    dgor_tile_of_block(b, tm_, tn_, gm, tm, tn);
                    if (tm < 0 || tm >= tm_ || tn < 0 || tn >= tn_) {
                        std::printf("out of range: tiles %dx%d group %d block %d -> (%d,%d)\n",
                                    tm_, tn_, gm, b, tm, tn);
                        return 1;
                    }
                    seen[tm * tn_ + tn] += 1;
                    ++checked;
                }
                for (int t = 0; t < nb; ++t)
                    if (seen[t] != 1) {
                        std::printf("tile %d produced %d times (tiles %dx%d group %d)\n", t,
                                    seen[t], tm_, tn_, gm);
                        return 1;
                    }
            }
    std::printf("ok %ld\n", checked);
    return 0;
}
