// Host-side check of the expert-aligned blocked order of the expert GEMMs:
// for random m-tile tables (experts with 0..20 m-tiles, some empty) and
// several n-tile counts, L -> (m-tile, n-tile) is a bijection of
// [0, MT*NT) onto the tiles, and the m-tiles of one group -- one expert's,
// at most GM_MAX of them -- that read the same weight tile (same n-tile)
// are claimed at consecutive L.
// Built by tests/test_schedule_host.py from the library's own header.
#include <cstdio>
#include <random>
#include <vector>

#include "../../routed_grouped_gemm_moe_amd/csrc/gemm_tile.h"

using namespace moe;

int main() {
    long bad = 0, checked = 0;
    std::mt19937 rng(7);
    for (int trial = 0; trial < 300; ++trial) {
        const int EL = 1 + (int)(rng() % 40);
        std::vector<int32_t> base(EL);
        std::vector<MTile> mtiles;
        for (int e = 0; e < EL; ++e) {
            base[e] = (int32_t)mtiles.size();
            const int n = (rng() % 4 == 0) ? 0 : (int)(rng() % 21);
            for (int m = 0; m < n; ++m) mtiles.push_back(MTile{e, 0, 0, 0});
        }
        const int MT = (int)mtiles.size();
        if (MT == 0) continue;
        for (int NT : {1, 3, 16, 112}) {
            std::vector<int> seen((size_t)MT * NT, 0);
            std::vector<int> prevL((size_t)MT * NT, -1);
            for (int L = 0; L < MT * NT; ++L) {
                int mt, nt;
                expert_tile(L, MT, NT, EL, mtiles.data(), base.data(), &mt, &nt);
                ++checked;
                if (mt < 0 || mt >= MT || nt < 0 || nt >= NT) { ++bad; continue; }
                seen[(size_t)mt * NT + nt]++;
                // the previous m-tile of the same group and n-tile sits at L - 1
                const int e = mtiles[mt].e;
                const int g0 = base[e] + (mt - base[e]) / GM_MAX * GM_MAX;
                if (mt > g0) {
                    int pm, pn;
                    expert_tile(L - 1, MT, NT, EL, mtiles.data(), base.data(), &pm, &pn);
                    if (pm != mt - 1 || pn != nt) ++bad;
                }
            }
            for (int v : seen)
                if (v != 1) ++bad;
        }
    }
    std::printf("%ld claims checked, %ld violations\n", checked, bad);
    return bad == 0 ? 0 : 1;
}
