/*
 * fc.h -- C ABI of a low-bit all-reduce codec for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one of "Flash Communication: Reducing Tensor
 * Parallelization Bottleneck for Fast Large Language Model Inference":
 *   - TL;DR and Abstract: the activations exchanged by a tensor-parallel
 *     all-reduce travel as low-bit codes, and the all-reduce runs in two
 *     steps instead of a ring;
 *   - Figure 5 (right): the two steps are a Reduce-Scatter (RS) and an
 *     All-Gather (AG), and the activations are quantized before each;
 *   - Figure 4: quantization is block-wise along the hidden dimension, with
 *     block sizes from the full hidden length down to 128.
 * The page gives no formula; this library implements the asymmetric min/max
 * reading (integer codes with an fp16 scale and an fp16 zero point per group,
 * rounded half to even), identical bit for bit to the project's CPU oracle:
 *
 *   per group:  mn, mx = min, max (a zero result taken as +0)
 *               s = fp16(fp32(fp32(mx - mn) / Q)),  z = fp16(mn),  Q = 2^bits - 1
 *               inv = fp32(1 / s), or 0 when s == 0
 *               q = clamp(round_half_even(fp32(fp32(v - z) * inv)), 0, Q)
 *   dequantize: v' = fp32(q * s + z)            (q * s is exact)
 *
 * All R operands live on one GPU: operand r is the partial sum that rank r of
 * a TP group of size R would hold. Hidden chunk j (columns [j*C, (j+1)*C),
 * C = H/R) is the part that rank j reduces in the RS step.
 *
 * Conventions for every entry point:
 *   - Buffer pointers are DEVICE pointers, owned by the caller; the library
 *     never keeps, frees or allocates them, and allocates nothing itself.
 *   - `stream` is a hipStream_t (NULL means the default stream). Calls are
 *     asynchronous: they return once the kernels are enqueued. On any
 *     validation error nothing is enqueued and no buffer is written.
 *   - All device pointers must be 16-byte aligned (FC_ERR_ALIGN otherwise).
 *   - Layouts are dense row-major. 8-bit codes take one byte each; 4-bit
 *     codes take two per byte, the even element in the low nibble.
 *     Scales and zeros are raw IEEE binary16 bit patterns, separate arrays.
 *   - T == 0 is valid and enqueues nothing (pointers may then be NULL).
 *   - Non-finite inputs, or inputs whose scale or zero overflow fp16
 *     (|min| > 65504 or (max - min)/Q > 65504), are outside the contract:
 *     the results are unspecified but every access stays in bounds.
 *   - No global state beyond a per-device cache of the compute-unit count
 *     (atomic) and the payload scratch of fc_allreduce_emulated_noalloc
 *     (one array per device, with its cached address): concurrent calls on
 *     different streams are safe, except overlapping calls of
 *     fc_allreduce_emulated_noalloc on one device.
 *
 * Supported shapes (FC_ERR_SHAPE otherwise): R >= 1, T >= 0, H >= 1,
 * bits in {4, 8} (FC_ERR_BITS), group even, at least 2 and dividing H,
 * H % R == 0, and the stage-2 group g2 = min(group, H/R) even and dividing
 * H/R. Power-of-two groups in [8, 8192] run on the fast kernels; any other
 * even length (24, 96, 6144, ...) runs on generic kernels with the same
 * bits, more slowly.
 */
#ifndef FC_H_
#define FC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FC_OK = 0,
    FC_ERR_NULL = 1,       /* a required pointer is NULL */
    FC_ERR_SHAPE = 2,      /* R, T, H, group or chunking outside the supported set */
    FC_ERR_BITS = 3,       /* bits is not 4 or 8 */
    FC_ERR_ALIGN = 4,      /* a device pointer is not 16-byte aligned */
    FC_ERR_WORKSPACE = 5,  /* workspace smaller than fc_workspace_bytes() */
    FC_ERR_LAUNCH = 6,     /* the HIP runtime reported an error at launch */
    FC_ERR_DTYPE = 7,      /* dtype is not FC_F16 or FC_BF16 */
    FC_ERR_SCRATCH = 8     /* the payloads exceed FC_NOALLOC_SCRATCH_BYTES */
} fc_status;

typedef enum { FC_F16 = 0, FC_BF16 = 1 } fc_dtype;

/*
 * Quantize before the Reduce-Scatter (Figure 5, right; groups as in Figure 4).
 *   x      [R][T][H]            fp16 or bf16 (dt)
 *   codes1 [R][T][H*bits/8]     uint8
 *   s1, z1 [R][T][H/group]      fp16 bit patterns
 * Every (r, t, k) group of `group` consecutive hidden columns is quantized on
 * its own.
 */
fc_status fc_quantize_groups(const void *x, fc_dtype dt, int R, int T, int H, int bits, int group,
                             uint8_t *codes1, uint16_t *s1, uint16_t *z1, void *stream);

/*
 * The Reduce-Scatter reduction and the quantization before the All-Gather
 * (Figure 5, right; TL;DR: the all-reduce in two steps).
 *   codes1, s1, z1  as produced by fc_quantize_groups
 *   codes2 [T][H*bits/8], s2, z2 [T][H/g2] with g2 = fc_stage2_group(R, H, group)
 * For each chunk j, token t and column h of the chunk, the R operands are
 * dequantized with their own stage-1 scale and zero and summed in binary32 in
 * ascending r starting from operand 0; the sums are requantized in groups of
 * g2 consecutive columns (never crossing a chunk).
 */
fc_status fc_dequant_sum_requant(const uint8_t *codes1, const uint16_t *s1, const uint16_t *z1,
                                 int R, int T, int H, int bits, int group,
                                 uint8_t *codes2, uint16_t *s2, uint16_t *z2, void *stream);

/*
 * Dequantize after the All-Gather (Figure 5, right).
 *   codes2 [T][H*bits/8], s2, z2 [T][H/group2]  ->  out [T][H] in dt
 * out = round_half_even_to_dt(fp32(q * s + z)).
 * group2 must be even and divide H.
 */
fc_status fc_dequantize(const uint8_t *codes2, const uint16_t *s2, const uint16_t *z2,
                        int T, int H, int bits, int group2, fc_dtype dt, void *out, void *stream);

/*
 * The whole emulated all-reduce on one GPU (TL;DR: the all-reduce in two
 * steps that replaces a ring; Figure 5, right: quantize, Reduce-Scatter, quantize,
 * All-Gather, dequantize): fc_quantize_groups, then fc_dequant_sum_requant,
 * then fc_dequantize, with both payloads placed in the caller's workspace
 * (layout: fc_workspace_layout). out [T][H] in dt.
 * Launch-bound calls (R*T*H <= 2^24, R <= 8, group == stage-2 group <= 512)
 * run as one kernel launch that writes the same payloads and output, bit for
 * bit; larger ones as the three launches.
 */
fc_status fc_allreduce_emulated(const void *x, fc_dtype dt, int R, int T, int H, int bits, int group,
                                void *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Different code widths before the two steps. The page quantizes before the
 * Reduce-Scatter and before the All-Gather and contrasts the two steps'
 * errors (Figure 5, right) without fixing the widths; these variants take
 * bits1 for the stage-1 payload (codes1) and bits2 for the stage-2 payload
 * (codes2), each 4 or 8 (FC_ERR_BITS otherwise). With bits1 == bits2 they are
 * fc_dequant_sum_requant and fc_allreduce_emulated.
 *   codes1 [R][T][H*bits1/8], codes2 [T][H*bits2/8]; the final dequantize of
 *   codes2 uses bits2.
 */
fc_status fc_dequant_sum_requant_mixed(const uint8_t *codes1, const uint16_t *s1,
                                       const uint16_t *z1, int R, int T, int H, int bits1,
                                       int bits2, int group, uint8_t *codes2, uint16_t *s2,
                                       uint16_t *z2, void *stream);

fc_status fc_allreduce_emulated_mixed(const void *x, fc_dtype dt, int R, int T, int H, int bits1,
                                      int bits2, int group, void *out, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * The final dequantize fused with the residual add that follows the
 * all-reduce in the transformer block (Figure 3: the attention and the MLP
 * outputs are all-reduced and added to the residual stream).
 *   codes2 [T][H*bits/8], s2, z2 [T][H/group2], residual [T][H] in dt
 *   ->  out [T][H] in dt,
 *   out = round_half_even_to_dt(fp32(residual + a)),
 *   a   = round_half_even_to_dt(fp32(q * s + z))   (what fc_dequantize writes)
 * so the result is the one of fc_dequantize followed by a 16-bit add computed
 * in binary32; the all-reduce result itself is not written. `out` may be the
 * same pointer as `residual` (in-place update of the residual stream); any
 * other overlap of the two is not supported. Same checks as fc_dequantize,
 * plus residual (FC_ERR_NULL / FC_ERR_ALIGN).
 */
fc_status fc_dequantize_residual(const uint8_t *codes2, const uint16_t *s2, const uint16_t *z2,
                                 int T, int H, int bits, int group2, fc_dtype dt,
                                 const void *residual, void *out, void *stream);

/*
 * fc_allreduce_emulated_mixed whose last step is fc_dequantize_residual:
 * out [T][H] = residual + the all-reduce of x, rounded as stated there. `out`
 * may be the same pointer as `residual`.
 */
fc_status fc_allreduce_emulated_residual(const void *x, fc_dtype dt, int R, int T, int H,
                                         int bits1, int bits2, int group, const void *residual,
                                         void *out, void *workspace, size_t workspace_bytes,
                                         void *stream);

/*
 * The row-parallel linear layer that produces the all-reduce operands, with
 * the quantization before the Reduce-Scatter done in its epilogue (Figure 3:
 * the attention output projection and the MLP down projection of every rank
 * end in the all-reduce; Figure 5, left, names them o_proj and d_proj).
 *   a  [R][T][K] in dt   rank r's slice of the layer input
 *   w  [R][H][K] in dt   rank r's input columns of the weight ([out][in])
 *   -> codes1, s1, z1 exactly as fc_quantize_groups gives them for
 *      y [R][T][H], y[r] = round_half_even_to_dt(a[r] w[r]^T)
 *   y  optional (NULL: not written): the layer output itself, in dt.
 * The products are accumulated in binary32 on the matrix cores (the order of
 * the accumulation is the hardware's), so y may differ from the exactly
 * rounded product by the accumulation error; the codes are always those of
 * the y this call computes (and writes, when y != NULL).
 * Extra requirements (FC_ERR_SHAPE otherwise): K a positive multiple of 32
 * and at most 2^22, H a multiple of 256 and at most 2^24, group a power of
 * two in [8, 256]. Same checks as fc_quantize_groups otherwise; y, when
 * given, 16-byte aligned.
 */
fc_status fc_linear_quantize(const void *a, const void *w, fc_dtype dt, int R, int T, int K, int H,
                             int bits, int group, uint8_t *codes1, uint16_t *s1, uint16_t *z1,
                             void *y, void *stream);

/*
 * fc_allreduce_emulated for callers that cannot allocate device memory at all
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same result, bit for bit, with both payloads kept in a
 * scratch array that the library itself holds on each device it runs on, of
 * FC_NOALLOC_SCRATCH_BYTES, for as long as the process lives. Nothing is
 * allocated per call (no hipMalloc, hipFree or allocating library routine).
 *   x [R][T][H] in dt  ->  out [T][H] in dt; the caller passes both.
 * Returns FC_ERR_SCRATCH, before enqueueing anything, when
 * fc_workspace_bytes(R, T, H, bits, group) exceeds FC_NOALLOC_SCRATCH_BYTES.
 * Every call on one device uses that device's one array; no part of it has to
 * start at zero (each payload byte a call reads, the same call wrote first),
 * but calls that overlap in time on one device -- on different streams, or
 * from different host threads without ordering -- race on it and their
 * results are then undefined. Calls on one stream are ordered and safe.
 * The array's device address is looked up once per device (first call there).
 */
#define FC_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

fc_status fc_allreduce_emulated_noalloc(const void *x, fc_dtype dt, int R, int T, int H, int bits,
                                        int group, void *out, void *stream);

/* Workspace size and layout for the mixed-width pipeline (same slice order). */
size_t fc_workspace_bytes_mixed(int R, int T, int H, int bits1, int bits2, int group);

fc_status fc_workspace_layout_mixed(int R, int T, int H, int bits1, int bits2, int group,
                                    size_t offsets[6], size_t sizes[6]);

/*
 * The uncompressed all-reduce result the page compares against (Figure 1: an
 * NCCL Ring All-Reduce of FP16 activations), computed on one GPU as the
 * reference point for the codec's speed and error:
 *   out[t][h] = round_half_even_to_dt(x[0][t][h] + x[1][t][h] + ... )
 * summed in binary32 in ascending r from operand 0 and rounded once (a ring
 * in the 16-bit type would round after every hop instead).
 *   x [R][T][H] in dt -> out [T][H] in dt. Requires R >= 1, T >= 0 and
 *   H % 8 == 0 (FC_ERR_SHAPE otherwise).
 */
fc_status fc_sum_uncompressed(const void *x, fc_dtype dt, int R, int T, int H, void *out,
                              void *stream);

/* Bytes of workspace fc_allreduce_emulated needs; 0 if the arguments are unsupported. */
size_t fc_workspace_bytes(int R, int T, int H, int bits, int group);

/*
 * Byte offsets and sizes of the six workspace slices, in this order:
 * codes1, s1, z1, codes2, s2, z2. Each offset is a multiple of 256.
 * Host-only; touches no device memory.
 */
fc_status fc_workspace_layout(int R, int T, int H, int bits, int group,
                              size_t offsets[6], size_t sizes[6]);

/* Stage-2 group length min(group, H/R); 0 if the arguments are unsupported. */
int fc_stage2_group(int R, int H, int group);

/* A static string naming the status. */
const char *fc_status_string(fc_status s);

#ifdef __cplusplus
}
#endif

#endif /* FC_H_ */
