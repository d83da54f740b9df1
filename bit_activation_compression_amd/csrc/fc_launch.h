// Internal launchers of the codec kernels (one per kernel family). Arguments
// are validated by the C ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fc {

// Stage-1 quantizer over n consecutive 16-bit values in groups of `group`
// (n % group == 0): codes [n*bits/8], s, z [n/group].
hipError_t launch_quantize(const uint16_t *x, int dtype, uint64_t n, int bits, int group,
                           uint8_t *codes, uint16_t *s, uint16_t *z, hipStream_t stream);

// Reduce-scatter reduction + requantization over n = T*H positions of R
// operands laid out [R][n]: stage-1 codes of bits1 in groups of `group1`,
// stage-2 codes of bits2 in groups of `group2`.
hipError_t launch_dequant_sum_requant(const uint8_t *codes1, const uint16_t *s1, const uint16_t *z1,
                                      int R, uint64_t n, int bits1, int bits2, int group1,
                                      int group2, uint8_t *codes2, uint16_t *s2, uint16_t *z2,
                                      hipStream_t stream);

// Final dequantization of n codes in groups of `group2` into 16-bit outputs.
hipError_t launch_dequantize(const uint8_t *codes2, const uint16_t *s2, const uint16_t *z2,
                             uint64_t n, int bits, int group2, int dtype, uint16_t *out,
                             hipStream_t stream);

// The same, added to a 16-bit residual [n] (may be the same array as out):
// out = round(residual + round(q*s + z)).
hipError_t launch_dequantize_residual(const uint8_t *codes2, const uint16_t *s2,
                                      const uint16_t *z2, uint64_t n, int bits, int group2,
                                      int dtype, const uint16_t *residual, uint16_t *out,
                                      hipStream_t stream);

// Row-parallel linear layer y[r] = a[r] w[r]^T (a [R][T][K], w [R][H][K]) with
// the stage-1 quantization of y in its epilogue (H % 256 == 0, K % 32 == 0,
// group in {8, ..., 256}); y itself is written only when y != NULL.
hipError_t launch_linear_quantize(const uint16_t *a, const uint16_t *w, int dtype, int R, int T,
                                  int K, int H, int bits, int group, uint8_t *codes, uint16_t *s,
                                  uint16_t *z, uint16_t *y, hipStream_t stream);

// The whole emulated all-reduce in one launch, for launch-bound shapes:
// stage-1 payload (codes1, s1, z1 as launch_quantize writes them), stage-2
// payload (as launch_dequant_sum_requant writes them) and the output (as
// launch_dequantize or, with residual != NULL, launch_dequantize_residual
// writes it), identical bit for bit. Applies when allreduce_small_applies.
constexpr uint64_t kAllreduceSmallMaxElems = uint64_t(1) << 24;   // R * T * H
bool allreduce_small_applies(int R, uint64_t n, int group, int group2);
hipError_t launch_allreduce_small(const uint16_t *x, int dtype, int R, uint64_t n, int bits1,
                                  int bits2, int group, uint8_t *codes1, uint16_t *s1,
                                  uint16_t *z1, uint8_t *codes2, uint16_t *s2, uint16_t *z2,
                                  const uint16_t *residual, uint16_t *out, hipStream_t stream);

// The same three steps for any even group length (the lengths the launchers
// above do not take: not a power of two in [8, 8192]); same bits.
hipError_t launch_quantize_generic(const uint16_t *x, int dtype, uint64_t n, int bits, int group,
                                   uint8_t *codes, uint16_t *s, uint16_t *z, hipStream_t stream);
hipError_t launch_dsr_generic(const uint8_t *codes1, const uint16_t *s1, const uint16_t *z1, int R,
                              uint64_t n, int bits1, int bits2, int group1, int group2,
                              uint8_t *codes2, uint16_t *s2, uint16_t *z2, hipStream_t stream);
// residual: NULL for the plain dequantize, else the residual add
hipError_t launch_dequantize_generic(const uint8_t *codes2, const uint16_t *s2, const uint16_t *z2,
                                     uint64_t n, int bits, int group2, int dtype,
                                     const uint16_t *residual, uint16_t *out, hipStream_t stream);

// Uncompressed R-way sum over n = T*H positions of R operands laid out [R][n].
hipError_t launch_sum(const uint16_t *x, int dtype, int R, uint64_t n, uint16_t *out,
                      hipStream_t stream);

}  // namespace fc
