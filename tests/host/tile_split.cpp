// Host checks of the GEMM tile scheduling: the tail split of the 256-row launches (for every
// tile count and every CU count per XCD, the blocks of the launch cover each tile exactly
// once, either whole or as its two 128-row halves, and a split only ever happens in an
// XCD's last round), and the grouped tile order (a bijection on a group's tiles).
#include "common.hpp"

#include <cstdio>
#include <vector>

int main() {
    for (int C : {1, 2, 3, 4, 8, 16, 31, 32, 40}) {
        for (int total = 0; total < 3000; ++total) {
            std::vector<int> seen(2 * (size_t)total + 2, 0);
            const int blocks = 8 * ((total + 7) / 8 + C / 2);
            for (int b = 0; b < blocks; ++b) {
                int half;
                const int t = moe::pick_tile_split(b, total, C, half);
                if (t < 0) continue;
                if (t >= total) {
                    std::printf("C %d total %d: block %d names tile %d\n", C, total, b, t);
                    return 1;
                }
                const int per = (total + 7) / 8, left = total - (b & 7) * per, n = per < left ? per : left;
                if (half >= 0 && (b >> 3) < n - n % C) {
                    std::printf("C %d total %d: block %d splits a tile before the last round\n", C, total, b);
                    return 1;
                }
                if (half < 0) {
                    seen[2 * t] += 1;
                    seen[2 * t + 1] += 1;
                } else {
                    seen[2 * t + half] += 1;
                }
            }
            for (int i = 0; i < 2 * total; ++i)
                if (seen[i] != 1) {
                    std::printf("C %d total %d: half %d of tile %d covered %d times\n", C, total, i % 2, i / 2,
                                seen[i]);
                    return 1;
                }
        }
    }
    // the grouped tile order is a bijection on [0, mtiles * ntn)
    for (int mtiles = 1; mtiles <= 40; ++mtiles)
        for (int ntn = 1; ntn <= 20; ++ntn) {
            std::vector<int> seen((size_t)mtiles * ntn, 0);
            for (int l = 0; l < mtiles * ntn; ++l) {
                int mt, nt;
                moe::grouped_tile<moe::kTileGroup>(l, mtiles, ntn, mt, nt);
                if (mt < 0 || mt >= mtiles || nt < 0 || nt >= ntn) {
                    std::printf("grouped order: mtiles %d ntn %d index %d -> (%d, %d)\n", mtiles, ntn, l, mt, nt);
                    return 1;
                }
                seen[(size_t)mt * ntn + nt] += 1;
            }
            for (int v : seen)
                if (v != 1) {
                    std::printf("grouped order: mtiles %d ntn %d not a bijection\n", mtiles, ntn);
                    return 1;
                }
        }
    std::printf("ok\n");
    return 0;
}
