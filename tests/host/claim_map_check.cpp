// Host-side check of the persistent scheduler's down-tile claim map: for
// 2 and 4 K parts, every tile count n2 and grid size G, each tile of the
// blocked order is claimed exactly once whole, or exactly once per K part
// with a unique cut-tile index; the number of cut tiles is what
// dn_split_tiles says, and within every XCD's claim range the whole tiles
// come before the parts.
// Built by tests/test_schedule_host.py from the library's own header.
#include <cstdio>
#include <vector>

#include "../../routed_grouped_gemm_moe_amd/csrc/moe_internal.h"

using namespace moe;

int main() {
    long bad = 0, checked = 0;
    for (int S : {2, 4})
    for (int n2 = 1; n2 <= 4000; ++n2)
        for (int G : {64, 128, 256, 304, 1024}) {
            const int nsp = dn_split_tiles(S, n2, G);
            if (dn_split_tiles(1, n2, G) != 0) ++bad;
            std::vector<int> whole(n2, 0);
            std::vector<std::vector<int>> parts(S, std::vector<int>(n2, 0));
            std::vector<int> st_of(nsp > 0 ? nsp : 1, -1);
            const int n = n2 + (S - 1) * nsp, per = (n + NUM_XCD - 1) / NUM_XCD;
            int prev_part = -1;
            for (int LS = 0; LS < n; ++LS) {
                if (LS % per == 0) prev_part = -1;  // a new XCD range starts
                int L, part, st;
                dn_claim(LS, n2, nsp, S, &L, &part, &st);
                if (L < 0 || L >= n2 || part >= S) { ++bad; continue; }
                if (part < 0) {
                    if (prev_part >= 0) ++bad;  // a whole tile after a part in one range
                    ++whole[L];
                } else {
                    parts[part][L]++;
                    if (st < 0 || st >= nsp) { ++bad; continue; }
                    if (st_of[st] < 0) st_of[st] = L;
                    else if (st_of[st] != L) ++bad;
                }
                prev_part = part;
            }
            int cut = 0;
            for (int L = 0; L < n2; ++L) {
                bool none = true, all = true;
                for (int q = 0; q < S; ++q) {
                    none = none && parts[q][L] == 0;
                    all = all && parts[q][L] == 1;
                }
                const bool w = whole[L] == 1 && none;
                const bool c = whole[L] == 0 && all;
                if (!(w || c)) ++bad;
                cut += c;
            }
            if (cut != nsp) ++bad;
            if (nsp > 0 && (nsp >= G || nsp > SPLIT_MAX)) ++bad;
            ++checked;
        }
    std::printf("claim map: %ld configurations, %ld violations\n", checked, bad);
    return bad != 0;
}
