// Host-only check of the occupancy hold of the two-rank kernels
// (ar_internal.h, hold_lds_bytes): the dynamic LDS it asks for is a multiple
// of 512 bytes that lets exactly the requested number of workgroups share a
// CU (floor(LDS per CU / bytes) == waves), never more than 64 KiB, and 0 --
// no hold -- when the grid would not fill every CU to that many, when the CU's
// LDS is unknown or when no hold is asked for.  Built with hipcc as host code;
// runs without a GPU.
#include <cstdio>

#include "ar_internal.h"

int main() {
    long checked = 0;
    const unsigned lds_sizes[] = {65536u, 98304u, 163840u};
    for (unsigned lds : lds_sizes) {
        for (unsigned cus : {1u, 80u, 256u, 304u}) {
            const mpp::CuLimits cu{cus, lds};
            for (unsigned waves = 1; waves <= 40; ++waves) {
                const unsigned full = cus * waves;
                if (mpp::hold_lds_bytes(cu, full - 1, waves) != 0) {
                    std::printf("FAIL hold below a full grid: lds=%u cus=%u waves=%u\n", lds, cus, waves);
                    return 1;
                }
                const unsigned b = mpp::hold_lds_bytes(cu, full, waves);
                if (b == 0) {
                    // refused only when no multiple of 512 bytes up to 64 KiB gives exactly `waves`
                    for (unsigned t = 512; t <= 65536; t += 512) {
                        if (lds / t == waves) {
                            std::printf("FAIL no hold where %u bytes would do: lds=%u waves=%u\n", t, lds, waves);
                            return 1;
                        }
                    }
                } else if (b % 512 != 0 || b > 65536 || lds / b != waves ||
                           (b > 512 && lds / (b - 512) == waves)) {
                    std::printf("FAIL hold bytes: lds=%u waves=%u bytes=%u\n", lds, waves, b);
                    return 1;
                }
                if (mpp::hold_lds_bytes(cu, uint64_t(full) * 1000, waves) != b) {
                    std::printf("FAIL hold depends on the grid beyond a full one: lds=%u waves=%u\n", lds, waves);
                    return 1;
                }
                ++checked;
            }
            if (mpp::hold_lds_bytes(cu, 1u << 30, 0) != 0 ||
                mpp::hold_lds_bytes(mpp::CuLimits{cus, 0u}, 1u << 30, 14) != 0) {
                std::printf("FAIL hold without a request or without the CU's LDS\n");
                return 1;
            }
        }
    }
    // the prefill call on MI355X (256 CUs, 160 KiB LDS each, 16384 one-wave workgroups)
    const mpp::CuLimits mi355x{256u, 163840u};
    if (mpp::hold_lds_bytes(mi355x, 16384, mpp::kPairWaves) != 8704u ||
        mpp::hold_lds_bytes(mi355x, 16384, mpp::kPairResWaves) != 11264u ||
        mpp::hold_lds_bytes(mi355x, 8, mpp::kPairWaves) != 0u) {
        std::printf("FAIL prefill holds\n");
        return 1;
    }
    std::printf("OK %ld (LDS, CUs, waves) triples\n", checked);
    return 0;
}
