// Host-only check of the kernels for a few active partials (ar_internal.h,
// few_compact, and the fold those kernels run): for every set of 2 to 4
// active ranks among R = 2 .. 16, the fold over the compacted active values
// with +0.0 added at the gaps few_compact marks (and -0.0, the identity,
// elsewhere) gives the same bits as the fold over all R ranks in order with
// +0.0 for each inactive rank, for every choice of the active values from a
// set of signed zeros and ordinary values.  Built with hipcc as host code;
// runs without a GPU.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "ar_internal.h"

static uint32_t bits(float x) {
    uint32_t u;
    std::memcpy(&u, &x, 4);
    return u;
}

int main() {
    const float vals[] = {-0.0f, 0.0f, 1.5f, -1.5f, 1e-30f, -3.0f};
    constexpr int NV = sizeof(vals) / sizeof(vals[0]);
    long checked = 0;
    static int dummy[16];
    for (int R = 2; R <= 16; ++R) {
        for (unsigned mask = 1; mask < (1u << R); ++mask) {
            const int A = __builtin_popcount(mask);
            if (A < 2 || A > 4) continue;
            const void *srcs[16];
            for (int r = 0; r < R; ++r) srcs[r] = (mask >> r) & 1u ? &dummy[r] : nullptr;
            const void *act[4] = {};
            unsigned z = 0;
            if (mpp::few_compact(srcs, R, act, &z) != A || z >= (1u << (A + 1))) {
                std::printf("FAIL count R=%d mask=%x\n", R, mask);
                return 1;
            }
            for (int a = 0, r = 0; r < R; ++r) {
                if (srcs[r] != nullptr && act[a++] != srcs[r]) {
                    std::printf("FAIL order R=%d mask=%x\n", R, mask);
                    return 1;
                }
            }
            // every assignment of values to the active ranks (NV^A)
            int total = 1;
            for (int a = 0; a < A; ++a) total *= NV;
            for (int code = 0; code < total; ++code) {
                float v[4];
                for (int a = 0, c = code; a < A; ++a, c /= NV) v[a] = vals[c % NV];
                // the fold over all ranks: w_0 first (+0.0 when inactive), then each in turn
                float full = 0.0f;
                for (int r = 0, a = 0; r < R; ++r) {
                    const float w = srcs[r] != nullptr ? v[a++] : 0.0f;
                    full = r == 0 ? w : full + w;
                }
                // the compacted fold with the gap adds
                float zg[5];
                for (int g = 0; g <= A; ++g) zg[g] = (z >> g) & 1u ? 0.0f : -0.0f;
                float acc = v[0] + zg[0];
                for (int a = 1; a < A; ++a) acc = (acc + zg[a]) + v[a];
                acc = acc + zg[A];
                if (bits(acc) != bits(full)) {
                    std::printf("FAIL fold R=%d mask=%x code=%d: %08x vs %08x\n", R, mask, code, bits(acc),
                                bits(full));
                    return 1;
                }
                ++checked;
            }
        }
    }
    std::printf("OK %ld folds\n", checked);
    return 0;
}
