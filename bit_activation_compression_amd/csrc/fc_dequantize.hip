// Final dequantization after the All-Gather of "Flash Communication:
// Reducing Tensor Parallelization Bottleneck for Fast Large Language Model
// Inference" (Figure 5, right): every rank holds all R requantized chunks and
// expands them to 16-bit activations, out = round_half_even(fp32(q*s + z)).
//
// HBM-bound: per element it reads bits/8 code bytes (plus 4 bytes per group)
// and writes 2 bytes.
//
// The residual variant folds in the add that follows the all-reduce in the
// transformer block (Figure 3): out = round(residual + round(q*s + z)), the
// rounded all-reduce result added in binary32 and rounded once more -- what
// the dequantize and a separate 16-bit add give, without the round trip of
// the all-reduce result through HBM (2 more bytes read per element).
#include "fc_device.h"
#include "fc_launch.h"

namespace fc {
namespace {

constexpr int kSlots = 4;

// `res` and `out` may be the same array (an in-place update of the residual
// stream): every element is read before the lane that owns it writes it.
template <int DT, int BITS, bool RES>
__global__ __launch_bounds__(kBlockThreads) void dequant_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ s,
    const uint16_t *__restrict__ z, uint64_t n, int g_shift, const uint16_t *res,
    uint16_t *out) {
    constexpr int W = BITS == 4 ? 1 : 2;
    const int lane = lane_id();
    const uint64_t wave = wave_index();
    const uint64_t tile = wave * (uint64_t)(kSlots * kSlotElems);
    if (tile >= n) return;
    const uint64_t left = n - tile;
    const uint32_t avail = left < (uint64_t)(kSlots * kSlotElems) ? (uint32_t)left : kSlots * kSlotElems;
    // group index of element tile + rel: (tile >> s) + (((tile mod 2^s) + rel) >> s)
    const uint32_t mis = (uint32_t)tile & ((1u << g_shift) - 1u);
    const uint8_t *cb = codes + tile * BITS / 8;
    const uint16_t *sb = s + (tile >> g_shift);
    const uint16_t *zb = z + (tile >> g_shift);
    uint16_t *ob = out + tile;
    const uint16_t *rb = RES ? res + tile : nullptr;

    uint32_t w[kSlots][W];
    uint16_t sv[kSlots], zv[kSlots];
    u32x4 rv[kSlots];
    // lanes past the end of the data load the tile's first element instead
    // (unconditional loads, all in flight together); their stores are skipped
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
        const uint32_t rel = u * kSlotElems + lane * kLaneElems;
        const uint32_t lrel = rel < avail ? rel : 0u;
        load_codes<BITS, false>(cb, lrel, w[u]);
        const uint32_t m = (mis + lrel) >> g_shift;
        sv[u] = sb[m];
        zv[u] = zb[m];
        if constexpr (RES) rv[u] = ldv<u32x4, true>(rb, lrel * 2);
    }
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
        const uint32_t rel = u * kSlotElems + lane * kLaneElems;
        if (rel >= avail) continue;
        float q[kLaneElems], o[kLaneElems];
        decode8<BITS>(w[u], q);
        const float sf = half_bits_to_float(sv[u]);
        const float zf = half_bits_to_float(zv[u]);
#pragma unroll
        for (int k = 0; k < kLaneElems; ++k) o[k] = __builtin_fmaf(q[k], sf, zf);   // exact product
        u32x4 packed = narrow8<DT>(o);
        if constexpr (RES) {
            float a[kLaneElems], r[kLaneElems];
            widen8<DT>(packed, a);   // the all-reduce result as the dtype holds it
            widen8<DT>(rv[u], r);
#pragma unroll
            for (int k = 0; k < kLaneElems; ++k) a[k] = r[k] + a[k];
            packed = narrow8<DT>(a);
        }
        stv<u32x4, true>(ob, rel * 2, packed);   // streamed out, not re-read
    }
}

template <int DT, int BITS, bool RES>
hipError_t launch_one(const uint8_t *codes, const uint16_t *s, const uint16_t *z, uint64_t n,
                      int g_shift, const uint16_t *res, uint16_t *out, hipStream_t stream) {
    constexpr uint64_t per_block = (uint64_t)kWavesPerBlock * kSlots * kSlotElems;
    const uint64_t blocks = (n + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((dequant_kernel<DT, BITS, RES>), dim3((unsigned)blocks), dim3(kBlockThreads),
                       0, stream, codes, s, z, n, g_shift, res, out);
    return hipGetLastError();
}

template <bool RES>
hipError_t launch_any(const uint8_t *codes2, const uint16_t *s2, const uint16_t *z2, uint64_t n,
                      int bits, int group2, int dtype, const uint16_t *res, uint16_t *out,
                      hipStream_t stream) {
    const int sh = ilog2(group2);
    if (dtype == 0)
        return bits == 4 ? launch_one<0, 4, RES>(codes2, s2, z2, n, sh, res, out, stream)
                         : launch_one<0, 8, RES>(codes2, s2, z2, n, sh, res, out, stream);
    return bits == 4 ? launch_one<1, 4, RES>(codes2, s2, z2, n, sh, res, out, stream)
                     : launch_one<1, 8, RES>(codes2, s2, z2, n, sh, res, out, stream);
}

}  // namespace

hipError_t launch_dequantize(const uint8_t *codes2, const uint16_t *s2, const uint16_t *z2,
                             uint64_t n, int bits, int group2, int dtype, uint16_t *out,
                             hipStream_t stream) {
    return launch_any<false>(codes2, s2, z2, n, bits, group2, dtype, nullptr, out, stream);
}

hipError_t launch_dequantize_residual(const uint8_t *codes2, const uint16_t *s2,
                                      const uint16_t *z2, uint64_t n, int bits, int group2,
                                      int dtype, const uint16_t *residual, uint16_t *out,
                                      hipStream_t stream) {
    return launch_any<true>(codes2, s2, z2, n, bits, group2, dtype, residual, out, stream);
}

}  // namespace fc
