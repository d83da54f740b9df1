/*
 * CPU oracle of the low-bit all-reduce codec. TEST INFRASTRUCTURE ONLY: the
 * tests, the smoke check and the benchmark's CPU-baseline leg are its only
 * users; no product code links or calls it.
 *
 * What it computes follows "Flash Communication: Reducing Tensor
 * Parallelization Bottleneck for Fast Large Language Model Inference":
 *   - TL;DR and Abstract: activations of a tensor-parallel all-reduce are sent
 *     as low-bit codes, and the all-reduce is done in two steps;
 *   - Figure 5 (right): the two steps are a Reduce-Scatter (RS) and an
 *     All-Gather (AG), and activations are quantized before each of them;
 *   - Figure 4: quantization is block-wise along the hidden dimension, with
 *     blocks from the full hidden length (4096) down to 128.
 * The page gives no formula. The quantizer below is the plain asymmetric
 * min/max one with an fp16 scale and an fp16 zero point per group, integer
 * codes in [0, 2^bits - 1] rounded half to even, every binary32 operation
 * rounded on its own (built with -ffp-contract=off: no fused multiply-add),
 * and the reduction summed in binary32 in ascending operand order.
 *
 * Plain, single-threaded and slow on purpose: it follows the steps in the
 * order the method takes them (quantize every operand, reduce each hidden
 * chunk, requantize, dequantize the gathered result).
 *
 * It shares nothing with the GPU library: its own status codes, its own
 * half/bfloat16 conversions (written from the IEEE 754 binary16 and the
 * bfloat16 format definitions), its own loops.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum {
    REF_OK = 0,
    REF_ERR_SHAPE = 2,
    REF_ERR_BITS = 3,
    REF_ERR_RANGE = 8,   /* non-finite input or a scale/zero that overflows fp16 */
    REF_ERR_NOMEM = 9,
};
enum { REF_F16 = 0, REF_BF16 = 1 };

/* ------------------------------------------------------------------------ */
/* binary16 and bfloat16 <-> binary32                                        */
/* ------------------------------------------------------------------------ */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
float ref_half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    float mag;
    if (e == 0)
        mag = ldexpf((float)m, -24);                 /* zero or subnormal: m * 2^-24 */
    else if (e == 31)
        mag = m ? NAN : INFINITY;
    else
        mag = ldexpf((float)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    return sign ? -mag : mag;
}

/* bfloat16: the top 16 bits of a binary32. */
float ref_bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * Round a finite binary32 value to a binary format with `p` significand bits
 * (including the hidden bit), minimum normal exponent `emin` and exponent
 * bias `bias`, to nearest with ties to even, with gradual underflow.
 * The spacing of representable values around |x| is 2^(e - p + 1) with
 * e = max(floor(log2|x|), emin); |x| / spacing is rounded to an integer n
 * (exact in double), and n is written as exponent/fraction fields. A carry
 * of n into the next binade and overflow to infinity fall out of the field
 * arithmetic. NaN input gives the canonical quiet NaN.
 */
static uint16_t round_to_small_float(float x, int p, int emin, int bias, int ebits)
{
    uint16_t sign = (uint16_t)(signbit(x) ? 1u << (ebits + p - 1) : 0u);
    uint32_t emax_field = (1u << ebits) - 1u;
    if (isnan(x))
        return (uint16_t)((emax_field << (p - 1)) | (1u << (p - 2)));
    double a = fabs((double)x);
    if (isinf(x))
        return (uint16_t)(sign | (emax_field << (p - 1)));
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);              /* a = f * 2^e2 with f in [0.5, 1) */
    int e = e2 - 1;             /* floor(log2 a) */
    if (e < emin)
        e = emin;
    double spacing = ldexp(1.0, e - (p - 1));
    double n = nearbyint(a / spacing);          /* ties to even */
    uint32_t field;
    if (e == emin && n < ldexp(1.0, p - 1))
        field = (uint32_t)n;                    /* subnormal (or the carry into the first normal) */
    else
        field = ((uint32_t)(e + bias) << (p - 1)) + ((uint32_t)n - (1u << (p - 1)));
    if (field >= (emax_field << (p - 1)))
        field = emax_field << (p - 1);          /* overflow to infinity */
    return (uint16_t)(sign | field);
}

uint16_t ref_float_to_half(float x) { return round_to_small_float(x, 11, -14, 15, 5); }
uint16_t ref_float_to_bf16(float x) { return round_to_small_float(x, 8, -126, 127, 8); }

static int half_is_finite(uint16_t h) { return ((h >> 10) & 0x1f) != 0x1f; }

static float widen(uint16_t v, int dtype)
{
    return dtype == REF_F16 ? ref_half_to_float(v) : ref_bf16_to_float(v);
}

static uint16_t narrow(float v, int dtype)
{
    return dtype == REF_F16 ? ref_float_to_half(v) : ref_float_to_bf16(v);
}

/* ------------------------------------------------------------------------ */
/* code storage: 8-bit codes one per byte; 4-bit codes two per byte, the     */
/* even element in the low nibble                                           */
/* ------------------------------------------------------------------------ */

static unsigned get_code(const uint8_t *codes, size_t i, int bits)
{
    if (bits == 8)
        return codes[i];
    return (codes[i / 2] >> (4 * (i % 2))) & 0xfu;
}

static void put_code(uint8_t *codes, size_t i, int bits, unsigned q)
{
    if (bits == 8) {
        codes[i] = (uint8_t)q;
    } else {
        unsigned shift = 4 * (unsigned)(i % 2);
        codes[i / 2] = (uint8_t)((codes[i / 2] & ~(0xfu << shift)) | (q << shift));
    }
}

/* ------------------------------------------------------------------------ */
/* one group                                                                 */
/* ------------------------------------------------------------------------ */

/*
 * Quantize n binary32 values (one group) to codes in [0, Q], Q = 2^bits - 1:
 *   mn, mx  = smallest and largest value (a zero result is taken as +0)
 *   s       = fp16(fp32(fp32(mx - mn) / Q))      the scale, stored as fp16
 *   z       = fp16(mn)                           the zero point, stored as fp16
 *   inv     = fp32(1 / s), or 0 when s is 0
 *   q_i     = clamp(round_half_even(fp32(fp32(v_i - z) * inv)), 0, Q)
 * Codes are chosen for the stored fp16 s and z, which is what a receiver has.
 * Returns REF_ERR_RANGE for non-finite input or an s or z that is not a
 * finite fp16.
 */
static int quantize_group(const float *v, size_t n, int bits, uint8_t *q,
                          uint16_t *s_out, uint16_t *z_out)
{
    const float Q = (float)((1 << bits) - 1);
    float mn = v[0], mx = v[0];
    for (size_t i = 0; i < n; ++i) {
        if (!isfinite(v[i]))
            return REF_ERR_RANGE;
        if (v[i] < mn)
            mn = v[i];
        if (v[i] > mx)
            mx = v[i];
    }
    if (mn == 0.0f)
        mn = 0.0f;
    if (mx == 0.0f)
        mx = 0.0f;
    float range = mx - mn;
    float s32 = range / Q;
    uint16_t s16 = ref_float_to_half(s32);
    uint16_t z16 = ref_float_to_half(mn);
    if (!half_is_finite(s16) || !half_is_finite(z16))
        return REF_ERR_RANGE;
    float s = ref_half_to_float(s16);
    float z = ref_half_to_float(z16);
    float inv = (s == 0.0f) ? 0.0f : 1.0f / s;
    for (size_t i = 0; i < n; ++i) {
        float d = v[i] - z;
        float t = d * inv;
        float r = nearbyintf(t);
        if (r < 0.0f)
            r = 0.0f;
        if (r > Q)
            r = Q;
        q[i] = (uint8_t)r;
    }
    *s_out = s16;
    *z_out = z16;
    return REF_OK;
}

/* x_hat = fp32(q * s + z); q * s is exact (<= 8 x 11 significant bits). */
static float dequant(unsigned q, uint16_t s16, uint16_t z16)
{
    float prod = (float)q * ref_half_to_float(s16);
    return prod + ref_half_to_float(z16);
}

/* ------------------------------------------------------------------------ */
/* argument checks                                                           */
/* ------------------------------------------------------------------------ */

int ref_stage2_group(int R, int H, int group)
{
    if (R < 1 || H < 1 || group < 1 || H % R != 0)
        return 0;
    int C = H / R;
    return group < C ? group : C;
}

static int check_args(int R, int T, int H, int bits, int group)
{
    if (bits != 4 && bits != 8)
        return REF_ERR_BITS;
    if (R < 1 || T < 0 || H < 1)
        return REF_ERR_SHAPE;
    if (group < 2 || group % 2 != 0 || H % group != 0)
        return REF_ERR_SHAPE;
    if (H % R != 0)
        return REF_ERR_SHAPE;
    int C = H / R;
    int g2 = ref_stage2_group(R, H, group);
    if (g2 % 2 != 0 || C % g2 != 0)
        return REF_ERR_SHAPE;
    return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* the three steps                                                           */
/* ------------------------------------------------------------------------ */

/*
 * Quantize before the Reduce-Scatter (Figure 5, right). Every operand r,
 * token t and group k (columns [k*group, (k+1)*group) of the hidden
 * dimension, Figure 4) is quantized on its own.
 *   x      [R][T][H]            16-bit values (dtype: 0 = fp16, 1 = bf16)
 *   codes1 [R][T][H*bits/8]     packed codes
 *   s1, z1 [R][T][H/group]      fp16 bit patterns
 */
int ref_quantize_groups(const uint16_t *x, int dtype, int R, int T, int H, int bits,
                        int group, uint8_t *codes1, uint16_t *s1, uint16_t *z1)
{
    int st = check_args(R, T, H, bits, group);
    if (st != REF_OK)
        return st;
    float *v = malloc(sizeof(float) * (size_t)group);
    uint8_t *q = malloc((size_t)group);
    if (!v || !q) {
        free(v);
        free(q);
        return REF_ERR_NOMEM;
    }
    const int G = H / group;
    for (int r = 0; r < R; ++r) {
        for (int t = 0; t < T; ++t) {
            size_t row = (size_t)r * T + t;
            for (int k = 0; k < G; ++k) {
                for (int i = 0; i < group; ++i)
                    v[i] = widen(x[row * H + (size_t)k * group + i], dtype);
                size_t m = row * G + k;
                st = quantize_group(v, (size_t)group, bits, q, &s1[m], &z1[m]);
                if (st != REF_OK)
                    goto done;
                for (int i = 0; i < group; ++i)
                    put_code(codes1, row * H + (size_t)k * group + i, bits, q[i]);
            }
        }
    }
done:
    free(v);
    free(q);
    return st;
}

/*
 * The Reduce-Scatter and the quantization before the All-Gather (Figure 5,
 * right). Rank j owns hidden chunk j, columns [j*C, (j+1)*C) with C = H/R.
 * For each of its columns it dequantizes the R operands' codes with their own
 * stage-1 scale and zero (a stage-1 group wider than C spans several chunks,
 * and each chunk reads the same group metadata) and sums them in binary32 in
 * ascending r, starting from operand 0. The sum is requantized in groups of
 * g2 = min(group, C) columns, which never cross a chunk.
 * bits1 is the width of the incoming (stage-1) codes, bits2 the width of the
 * requantized (stage-2) codes; the page quantizes before both steps and does
 * not say they must be equal.
 *   codes2 [T][H*bits2/8], s2, z2 [T][H/g2]
 *   y      [T][H] binary32 sums (optional, may be NULL)
 */
int ref_dequant_sum_requant_mixed(const uint8_t *codes1, const uint16_t *s1, const uint16_t *z1,
                                  int R, int T, int H, int bits1, int bits2, int group,
                                  uint8_t *codes2, uint16_t *s2, uint16_t *z2, float *y_out)
{
    int st = check_args(R, T, H, bits1, group);
    if (st == REF_OK)
        st = check_args(R, T, H, bits2, group);
    if (st != REF_OK)
        return st;
    const int C = H / R;
    const int g2 = ref_stage2_group(R, H, group);
    const int G1 = H / group, G2 = H / g2;
    float *y = malloc(sizeof(float) * (size_t)C);
    uint8_t *q = malloc((size_t)g2);
    if (!y || !q) {
        free(y);
        free(q);
        return REF_ERR_NOMEM;
    }
    for (int j = 0; j < R; ++j) {
        for (int t = 0; t < T; ++t) {
            for (int c = 0; c < C; ++c) {
                int h = j * C + c;
                float acc = 0.0f;
                for (int r = 0; r < R; ++r) {
                    size_t row = (size_t)r * T + t;
                    size_t m = row * G1 + (size_t)(h / group);
                    float xh = dequant(get_code(codes1, row * H + (size_t)h, bits1), s1[m], z1[m]);
                    acc = (r == 0) ? xh : acc + xh;
                }
                y[c] = acc;
                if (y_out)
                    y_out[(size_t)t * H + h] = acc;
            }
            for (int k = 0; k < C / g2; ++k) {
                int h0 = j * C + k * g2;
                size_t m = (size_t)t * G2 + (size_t)(h0 / g2);
                st = quantize_group(y + (size_t)k * g2, (size_t)g2, bits2, q, &s2[m], &z2[m]);
                if (st != REF_OK)
                    goto done;
                for (int i = 0; i < g2; ++i)
                    put_code(codes2, (size_t)t * H + (size_t)h0 + i, bits2, q[i]);
            }
        }
    }
done:
    free(y);
    free(q);
    return st;
}

/* Same code width before both steps. */
int ref_dequant_sum_requant(const uint8_t *codes1, const uint16_t *s1, const uint16_t *z1,
                            int R, int T, int H, int bits, int group,
                            uint8_t *codes2, uint16_t *s2, uint16_t *z2, float *y_out)
{
    return ref_dequant_sum_requant_mixed(codes1, s1, z1, R, T, H, bits, bits, group, codes2, s2, z2,
                                         y_out);
}

/*
 * Dequantize after the All-Gather: every rank holds all R requantized chunks,
 * and each element becomes o = fp32(q2 * s2 + z2), rounded to the output
 * dtype (nearest, ties to even).
 *   out [T][H] 16-bit; o32 [T][H] binary32 (optional, may be NULL)
 */
int ref_dequantize(const uint8_t *codes2, const uint16_t *s2, const uint16_t *z2,
                   int T, int H, int bits, int group2, int dtype, uint16_t *out, float *o32)
{
    if (bits != 4 && bits != 8)
        return REF_ERR_BITS;
    if (T < 0 || H < 1 || group2 < 2 || group2 % 2 != 0 || H % group2 != 0)
        return REF_ERR_SHAPE;
    const int G2 = H / group2;
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            size_t e = (size_t)t * H + h;
            size_t m = (size_t)t * G2 + (size_t)(h / group2);
            float o = dequant(get_code(codes2, e, bits), s2[m], z2[m]);
            if (o32)
                o32[e] = o;
            out[e] = narrow(o, dtype);
        }
    }
    return REF_OK;
}

/*
 * Quantize a flat run of binary32 values in groups of `group` (the stage-2
 * quantizer on its own; used by the tests to probe it with hand-built sums).
 */
int ref_quantize_f32(const float *v, size_t n, int bits, int group,
                     uint8_t *codes, uint16_t *s, uint16_t *z)
{
    if (bits != 4 && bits != 8)
        return REF_ERR_BITS;
    if (group < 2 || group % 2 != 0 || n % (size_t)group != 0)
        return REF_ERR_SHAPE;
    uint8_t *q = malloc((size_t)group);
    if (!q)
        return REF_ERR_NOMEM;
    int st = REF_OK;
    for (size_t k = 0; k < n / (size_t)group; ++k) {
        st = quantize_group(v + k * group, (size_t)group, bits, q, &s[k], &z[k]);
        if (st != REF_OK)
            break;
        for (int i = 0; i < group; ++i)
            put_code(codes, k * group + i, bits, q[i]);
    }
    free(q);
    return st;
}

/* Array forms of the conversions, for exhaustive checks. */
void ref_half_to_float_n(const uint16_t *h, float *f, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        f[i] = ref_half_to_float(h[i]);
}

void ref_bf16_to_float_n(const uint16_t *b, float *f, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        f[i] = ref_bf16_to_float(b[i]);
}

void ref_float_to_half_n(const float *f, uint16_t *h, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        h[i] = ref_float_to_half(f[i]);
}

void ref_float_to_bf16_n(const float *f, uint16_t *b, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        b[i] = ref_float_to_bf16(f[i]);
}

/*
 * The uncompressed all-reduce the page compares against (Figure 1: an NCCL
 * Ring All-Reduce of FP16 activations): every rank ends with the sum of the
 * R operands. Reading taken here: binary32 accumulation in ascending operand
 * order, starting from operand 0, rounded once to the 16-bit dtype (a ring
 * in the 16-bit type would round after every hop instead).
 *   x [R][T][H] 16-bit -> out [T][H] 16-bit
 */
int ref_sum_uncompressed(const uint16_t *x, int dtype, int R, int T, int H, uint16_t *out)
{
    if (R < 1 || T < 0 || H < 1)
        return REF_ERR_SHAPE;
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int r = 0; r < R; ++r) {
                float v = widen(x[((size_t)r * T + t) * H + h], dtype);
                acc = (r == 0) ? v : acc + v;
            }
            out[(size_t)t * H + h] = narrow(acc, dtype);
        }
    }
    return REF_OK;
}

/*
 * The final dequantize followed by the residual add of the transformer block
 * (Figure 3: each attention and MLP output leaves the block through the
 * all-reduce and is added to the residual stream). Reading taken here: the
 * all-reduce result is first rounded to the model dtype, exactly as the
 * separate dequantize returns it, and then added to the residual in binary32
 * and rounded once more to the dtype -- the result the two separate steps
 * give, so that fusing them changes only where the work is done.
 *   codes2, s2, z2 [T][H] payload, residual [T][H] 16-bit -> out [T][H] 16-bit
 */
int ref_dequantize_residual(const uint8_t *codes2, const uint16_t *s2, const uint16_t *z2,
                            int T, int H, int bits, int group2, int dtype,
                            const uint16_t *residual, uint16_t *out)
{
    if (bits != 4 && bits != 8)
        return REF_ERR_BITS;
    if (T < 0 || H < 1 || group2 < 2 || group2 % 2 != 0 || H % group2 != 0)
        return REF_ERR_SHAPE;
    const int G2 = H / group2;
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            size_t e = (size_t)t * H + h;
            size_t m = (size_t)t * G2 + (size_t)(h / group2);
            uint16_t a = narrow(dequant(get_code(codes2, e, bits), s2[m], z2[m]), dtype);
            float sum = widen(residual[e], dtype) + widen(a, dtype);
            out[e] = narrow(sum, dtype);
        }
    }
    return REF_OK;
}
