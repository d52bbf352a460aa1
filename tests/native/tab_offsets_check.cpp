// Host check of the packed table addressing of the bf16-grid exp table:
// tab_offsets (two bf16 keys per 32-bit word, 16-bit packed arithmetic) must
// give 8 * tab_index for every key inside the table, a zero entry of the
// key's sign for every key outside it, and flag exactly the keys outside.
// Every first key is paired with a second key from a fixed permutation, for
// the table ranges of T = 1, T = 0.5, the smallest and the largest range.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>

#include "sv_device.h"

using namespace sv;

int main()
{
    long bad = 0, n = 0;
    const uint32_t los[] = {115u << 7, 114u << 7, 1u << 7, (255u - kTabBinades) << 7};
    for (uint32_t lo : los) {
        const u16x2 lo2 = {(unsigned short)lo, (unsigned short)lo};
        for (uint32_t k0 = 0; k0 < 65536; ++k0) {
            const uint32_t k1 = (k0 * 40503u + 12345u) & 0xFFFFu;
            const uint32_t w = k0 | (k1 << 16);
            uint32_t a0, a1;
            u16x2 worst = {0, 0};
            tab_offsets(w, lo2, a0, a1, worst);
            float z0, z1;
            const uint32_t b0 = k0 << 16, b1 = k1 << 16;
            std::memcpy(&z0, &b0, 4);
            std::memcpy(&z1, &b1, 4);
            const int i0 = tab_index(z0, lo), i1 = tab_index(z1, lo);
            auto expect = [](int i, uint32_t key) {
                return i >= 0 ? 8u * (uint32_t)i : 8u * (kTabKeys + (key >> 15) * kTabHalf);
            };
            bool ok = a0 == expect(i0, k0) && a1 == expect(i1, k1);
            ok = ok && (((uint32_t)worst.x >= (uint32_t)kTabKeys) == (i0 < 0));
            ok = ok && (((uint32_t)worst.y >= (uint32_t)kTabKeys) == (i1 < 0));
            if (!ok && bad < 5) std::printf("lo=%u w=%08x offsets=(%u,%u) index=(%d,%d)\n", lo, w, a0, a1, i0, i1);
            bad += !ok;
            ++n;
        }
    }
    std::printf("checked %ld, mismatches %ld\n", n, bad);
    return bad != 0;
}
