// Host-only check of the workgroup placement map of the streaming kernels
// (ar_internal.h): for every grid size and exponent tried, xcd_virtual_block
// is a permutation of [0, G) (each tile is processed exactly once), lc = 0 is
// the identity, and inside the renumbered part the workgroups that one XCD
// receives (b mod 8 fixed) walk runs of 2^lc consecutive virtual workgroups.
// xcd_map_lc never makes a run longer than the requested elements or a round
// longer than a range.  Built with hipcc as host code; runs without a GPU.
#include <cstdio>
#include <vector>

#include "ar_internal.h"

int main() {
    long checked = 0;
    for (unsigned G = 1; G <= 2100; G += (G < 300 ? 1 : 37)) {
        for (unsigned lc = 0; lc <= 11; ++lc) {
            std::vector<unsigned char> seen(G, 0);
            for (unsigned b = 0; b < G; ++b) {
                const unsigned v = mpp::xcd_virtual_block(b, G, lc);
                if (v >= G || seen[v]) {
                    std::printf("FAIL not a permutation: G=%u lc=%u b=%u v=%u\n", G, lc, b, v);
                    return 1;
                }
                seen[v] = 1;
                if (lc == 0 && v != b) {
                    std::printf("FAIL identity: G=%u b=%u v=%u\n", G, b, v);
                    return 1;
                }
            }
            // runs: consecutive dispatch slots of one XCD inside the renumbered part
            const unsigned C = 1u << lc, full = G & ~(8u * C - 1u);
            for (unsigned b = 8; b < full; ++b) {
                const unsigned j = b >> 3;
                if (j % C != 0 && mpp::xcd_virtual_block(b, G, lc) != mpp::xcd_virtual_block(b - 8, G, lc) + 1) {
                    std::printf("FAIL run: G=%u lc=%u b=%u\n", G, lc, b);
                    return 1;
                }
            }
            ++checked;
        }
    }
    for (unsigned grid = 1; grid <= 70000; grid = grid * 3 + 1) {
        for (size_t wg = 256; wg <= 4096; wg *= 2) {
            for (size_t run = 1; run <= (size_t(1) << 24); run *= 4) {
                const unsigned lc = mpp::xcd_map_lc(grid, wg, run);
                if (lc > 0 && ((wg << lc) > run || (8u << lc) > grid)) {
                    std::printf("FAIL lc: grid=%u wg=%zu run=%zu lc=%u\n", grid, wg, run, lc);
                    return 1;
                }
                if (lc < 15 && (wg << (lc + 1)) <= run && (size_t(8) << (lc + 1)) <= grid) {
                    std::printf("FAIL lc not maximal: grid=%u wg=%zu run=%zu lc=%u\n", grid, wg, run, lc);
                    return 1;
                }
            }
        }
    }
    // the prefill reduce's launch: 4 ranges of 1024 workgroups of 2048 elements, runs of 2^17
    if (mpp::xcd_map_lc(1024, 2048, size_t(1) << 17) != 6) {
        std::printf("FAIL prefill exponent\n");
        return 1;
    }
    std::printf("OK %ld grid/exponent pairs\n", checked);
    return 0;
}
