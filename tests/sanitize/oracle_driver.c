/*
 * Test driver for a sanitizer build of the CPU oracle (oracle/fc_oracle.c
 * linked in directly, built with -fsanitize=address,undefined). Reads cases
 * from argv[1], runs every entry point of the oracle on each, and writes all
 * outputs to argv[2]; the Python test compares them byte for byte with the
 * normal build's. Test infrastructure only.
 *
 * Case file: int32 count, then per case int32 R, T, H, dtype, bits1, bits2,
 * group, followed by R*T*H uint16 operands and T*H uint16 residual values.
 * Output per case, in this order: the status of each call (int32), codes1,
 * s1, z1, codes2, s2, z2, y (binary32), out, o32 (binary32), residual sum,
 * uncompressed sum, and the stage-2 quantizer run alone on y.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int ref_stage2_group(int R, int H, int group);
int ref_quantize_groups(const uint16_t *x, int dtype, int R, int T, int H, int bits, int group,
                        uint8_t *codes1, uint16_t *s1, uint16_t *z1);
int ref_dequant_sum_requant_mixed(const uint8_t *codes1, const uint16_t *s1, const uint16_t *z1,
                                  int R, int T, int H, int bits1, int bits2, int group,
                                  uint8_t *codes2, uint16_t *s2, uint16_t *z2, float *y_out);
int ref_dequantize(const uint8_t *codes2, const uint16_t *s2, const uint16_t *z2, int T, int H,
                   int bits, int group2, int dtype, uint16_t *out, float *o32);
int ref_quantize_f32(const float *v, size_t n, int bits, int group, uint8_t *codes, uint16_t *s,
                     uint16_t *z);
int ref_sum_uncompressed(const uint16_t *x, int dtype, int R, int T, int H, uint16_t *out);
int ref_dequantize_residual(const uint8_t *codes2, const uint16_t *s2, const uint16_t *z2, int T,
                            int H, int bits, int group2, int dtype, const uint16_t *residual,
                            uint16_t *out);

static void rd(void *p, size_t sz, size_t n, FILE *f)
{
    if (n && fread(p, sz, n, f) != n) {
        fprintf(stderr, "short read\n");
        exit(2);
    }
}

static void wr(const void *p, size_t sz, size_t n, FILE *f)
{
    if (n && fwrite(p, sz, n, f) != n) {
        fprintf(stderr, "short write\n");
        exit(2);
    }
}

/* exactly-sized buffers, so that any overrun is a sanitizer report */
static void *alloc(size_t n) { return malloc(n ? n : 1); }

int main(int argc, char **argv)
{
    if (argc != 3)
        return 2;
    FILE *in = fopen(argv[1], "rb"), *out = fopen(argv[2], "wb");
    if (!in || !out)
        return 2;
    int32_t count;
    rd(&count, 4, 1, in);
    for (int c = 0; c < count; ++c) {
        int32_t a[7];
        rd(a, 4, 7, in);
        int R = a[0], T = a[1], H = a[2], dt = a[3], b1 = a[4], b2 = a[5], g = a[6];
        size_t n1 = (size_t)R * T * H, n2 = (size_t)T * H;
        int g2 = ref_stage2_group(R, H, g);
        uint16_t *x = alloc(2 * n1), *res = alloc(2 * n2);
        rd(x, 2, n1, in);
        rd(res, 2, n2, in);
        size_t c1n = n1 * b1 / 8, m1 = n1 / g, c2n = n2 * b2 / 8, m2 = n2 / g2;
        uint8_t *codes1 = alloc(c1n), *codes2 = alloc(c2n), *codes3 = alloc(c2n);
        uint16_t *s1 = alloc(2 * m1), *z1 = alloc(2 * m1), *s2 = alloc(2 * m2), *z2 = alloc(2 * m2);
        uint16_t *s3 = alloc(2 * m2), *z3 = alloc(2 * m2);
        uint16_t *o = alloc(2 * n2), *ro = alloc(2 * n2), *su = alloc(2 * n2);
        float *y = alloc(4 * n2), *o32 = alloc(4 * n2);
        int32_t st[6];
        st[0] = ref_quantize_groups(x, dt, R, T, H, b1, g, codes1, s1, z1);
        st[1] = ref_dequant_sum_requant_mixed(codes1, s1, z1, R, T, H, b1, b2, g, codes2, s2, z2, y);
        st[2] = ref_dequantize(codes2, s2, z2, T, H, b2, g2, dt, o, o32);
        st[3] = ref_dequantize_residual(codes2, s2, z2, T, H, b2, g2, dt, res, ro);
        st[4] = ref_sum_uncompressed(x, dt, R, T, H, su);
        st[5] = ref_quantize_f32(y, n2, b2, g2, codes3, s3, z3);
        wr(st, 4, 6, out);
        wr(codes1, 1, c1n, out);
        wr(s1, 2, m1, out);
        wr(z1, 2, m1, out);
        wr(codes2, 1, c2n, out);
        wr(s2, 2, m2, out);
        wr(z2, 2, m2, out);
        wr(y, 4, n2, out);
        wr(o, 2, n2, out);
        wr(o32, 4, n2, out);
        wr(ro, 2, n2, out);
        wr(su, 2, n2, out);
        wr(codes3, 1, c2n, out);
        wr(s3, 2, m2, out);
        wr(z3, 2, m2, out);
        free(x); free(res); free(codes1); free(codes2); free(codes3);
        free(s1); free(z1); free(s2); free(z2); free(s3); free(z3);
        free(o); free(ro); free(su); free(y); free(o32);
    }
    /* argument errors: each returns its status before touching a buffer */
    int32_t e[5];
    e[0] = ref_quantize_groups(NULL, 0, 2, 8, 256, 6, 128, NULL, NULL, NULL);
    e[1] = ref_quantize_groups(NULL, 0, 2, 8, 256, 4, 3, NULL, NULL, NULL);
    e[2] = ref_quantize_groups(NULL, 0, 3, 8, 256, 4, 128, NULL, NULL, NULL);
    e[3] = ref_dequantize(NULL, NULL, NULL, 8, 256, 4, 96, 0, NULL, NULL);
    e[4] = ref_quantize_f32(NULL, 10, 4, 4, NULL, NULL, NULL);
    wr(e, 4, 5, out);
    fclose(in);
    return fclose(out) == 0 ? 0 : 2;
}
