// Host driver for the M = 8 copy choice (approximate_multiplier_dnn_amd/csrc/replica.h),
// built by tests/test_replica_host.py with the host compiler. Reads groups from stdin,
// one per line: count pad_w w[0] .. w[31]; writes, per group: top w'[0] .. w'[31].
#include <cstdio>

#include "../approximate_multiplier_dnn_amd/csrc/replica.h"

int main()
{
    int count;
    unsigned pad_w;
    while (std::scanf("%d %u", &count, &pad_w) == 2) {
        uint32_t w[32];
        for (int l = 0; l < 32; ++l) {
            unsigned v;
            if (std::scanf("%u", &v) != 1) return 1;
            w[l] = v;
        }
        const int top = amx::rep8_assign_group(w, count, pad_w);
        std::printf("%d", top);
        for (int l = 0; l < 32; ++l) std::printf(" %u", w[l]);
        std::printf("\n");
    }
    return 0;
}
