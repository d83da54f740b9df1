// Test driver for a sanitizer build of the C ABI's host-side argument checks
// and workspace layout (bit_activation_compression_amd/csrc/fc_validate.h,
// the same code fc_api.hip compiles). Prints, for every argument set of a
// grid, the status, the stage-2 group and the six slice offsets and sizes;
// the Python test compares the lines with what libfc.so returns for the same
// arguments. Test infrastructure only.
#include <stdio.h>

#include "fc_validate.h"

int main() {
    using namespace fc::validate;
    const int Rs[] = {0, 1, 2, 3, 4, 8, 16};
    const int Ts[] = {-1, 0, 1, 7, 8192, 1 << 20};
    const int Hs[] = {0, 8, 96, 256, 4096, 8192, 12288, 1 << 20};
    const int bits[] = {2, 4, 8};
    const int groups[] = {0, 2, 3, 8, 16, 24, 96, 128, 4096, 8192, 16384};
    for (int R : Rs)
        for (int T : Ts)
            for (int H : Hs)
                for (int b1 : bits)
                    for (int b2 : bits)
                        for (int g : groups) {
                            int g2 = 0;
                            const fc_status st = check_shape2(R, T, H, b1, b2, g, &g2);
                            printf("%d %d %d %d %d %d : %d", R, T, H, b1, b2, g, (int)st);
                            if (st == FC_OK) {
                                const Layout L = layout(R, T, H, b1, b2, g, g2);
                                printf(" %d %zu", g2, L.total);
                                for (int i = 0; i < 6; ++i) printf(" %zu %zu", L.off[i], L.size[i]);
                            }
                            printf("\n");
                        }
    // pointer checks
    int a = 0;
    alignas(16) char buf[32];
    printf("ptrs %d %d %d %d\n", (int)check_ptrs(0, {nullptr}), (int)check_ptrs(1, {buf, nullptr}),
           (int)check_ptrs(1, {buf, buf + 8}), (int)check_ptrs(1, {buf, buf + 16}));
    (void)a;
    return 0;
}
