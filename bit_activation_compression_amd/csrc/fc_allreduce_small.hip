// The whole emulated all-reduce of "Flash Communication: Reducing Tensor
// Parallelization Bottleneck for Fast Large Language Model Inference"
// (Figure 5, right: quantize, Reduce-Scatter reduction and requantize,
// All-Gather dequantize) in ONE launch, for shapes where launching the three
// stage kernels one after the other costs more than their memory traffic
// (decode-sized calls: 14.5 MB moved, under 2 us at HBM speed).
//
// Every output position depends only on the same position of the R operands,
// within whole quantization groups. So a wave can take a run of positions
// through all three stages alone: quantize each operand's values, dequantize
// those codes and sum them, requantize the sums, dequantize those. The
// arithmetic is that of the three stage kernels, step for step (the same
// device helpers), and the stage boundaries go through memory as in the
// three-launch path: each stage writes its payload to the caller's workspace
// (the hand-off the real exchange would carry) and the next stage reads it
// back from there.
//
// Work layout: a wave owns one slot of 512 consecutive positions, a lane 8 of
// them (one 16-byte load per operand); a group of G <= 512 positions covers
// G/8 lanes. Used when the stage-1 and stage-2 groups are equal (group <= H/R)
// and R <= 8.
#include <type_traits>

#include "fc_device.h"
#include "fc_launch.h"

namespace fc {
namespace {

constexpr int kMaxR = 8;

// lanes_minmax over aligned groups of L lanes (L given at run time, uniform)
// for the first `count` of N value pairs; one branch for all of them, so the
// pairs' cross-lane steps interleave
template <int N>
__device__ __forceinline__ void lanes_minmax_any(float (&mn)[N], float (&mx)[N], int count, int L) {
    auto all = [&](auto l_tag) {
        constexpr int LL = decltype(l_tag)::value;
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < count) lanes_minmax<LL>(mn[i], mx[i]);
    };
    switch (L) {
    case 2: all(std::integral_constant<int, 2>{}); break;
    case 4: all(std::integral_constant<int, 4>{}); break;
    case 8: all(std::integral_constant<int, 8>{}); break;
    case 16: all(std::integral_constant<int, 16>{}); break;
    case 32: all(std::integral_constant<int, 32>{}); break;
    case 64: all(std::integral_constant<int, 64>{}); break;
    default: break;   // 1 lane: nothing to combine
    }
}

// A stage boundary inside the kernel: the payload this wave has just stored
// is read back from memory (release, then acquire, at workgroup scope). Each
// wave reads back only what it wrote itself -- every position depends only
// on the same position of the operands -- so no other wave's progress is
// involved, and the wave's stores and later loads go in order through its
// CU's vector memory path: the fences only keep the compiler from moving
// loads above the stores, and no cache write-back or invalidation is needed
// (a device-scope fence would write L2 back for nothing).
__device__ __forceinline__ void handoff() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// `res` and `out` may be the same array: every lane reads its residual
// values before it writes its outputs. RT > 0: the operand count is a
// compile-time constant, so the operands' independent chains (group min/max,
// scale, reciprocal, codes) interleave -- a decode call has one wave per
// SIMD, and nothing else hides their latency; RT == 0: any R <= 8.
template <int DT, int BITS1, int BITS2, bool RES, int RT>
__global__ __launch_bounds__(kBlockThreads) void allreduce_small_kernel(
    const uint16_t *__restrict__ x, int R_arg, uint64_t n, int g_shift, uint8_t *__restrict__ codes1,
    uint16_t *__restrict__ s1, uint16_t *__restrict__ z1, uint8_t *__restrict__ codes2,
    uint16_t *__restrict__ s2, uint16_t *__restrict__ z2, const uint16_t *res, uint16_t *out) {
    constexpr int W1 = BITS1 == 4 ? 1 : 2, W2 = BITS2 == 4 ? 1 : 2;
    constexpr int NR = RT > 0 ? RT : kMaxR;              // operand slots
    const int R = RT > 0 ? RT : R_arg;
    const int lane = lane_id();
    const uint64_t tile = wave_index() * (uint64_t)kSlotElems;
    if (tile >= n) return;
    const uint64_t left = n - tile;
    const uint32_t avail = left < (uint64_t)kSlotElems ? (uint32_t)left : (uint32_t)kSlotElems;
    const int L = (1 << g_shift) / kLaneElems;            // lanes per group
    // n is a multiple of the group and the slot holds whole groups, so a
    // group's lanes are all inside the data or all past its end. Lanes past
    // the end (last slot only) load the slot's first positions instead: every
    // load is unconditional; their groups are their own and nothing of them
    // is stored.
    const uint32_t rel = (uint32_t)lane * kLaneElems;
    const bool valid = rel < avail;
    const uint32_t lrel = valid ? rel : 0u;
    const bool leader = valid && (lane & (L - 1)) == 0;    // stores the group's scale and zero
    const uint64_t gpos = (tile + rel) >> g_shift;         // group of the lane's positions

    // all operands' values (and the residual) in flight together
    u32x4 raw[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r)
        if (RT > 0 || r < R) raw[r] = ldv<u32x4, true>(x + (uint64_t)r * n + tile, lrel * 2);
    u32x4 rv = {};
    if constexpr (RES) rv = ldv<u32x4, true>(res + tile, lrel * 2);

    // ---- stage 1: every operand quantized, payload 1 written ----
    // The operands go through each phase together (group minima and maxima,
    // their cross-lane steps, then codes), so their independent chains
    // interleave.
    float v1[NR][kLaneElems], mn1[NR], mx1[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        if (RT == 0 && r >= R) break;
        widen8<DT>(raw[r], v1[r]);
        minmax8(v1[r], mn1[r], mx1[r]);
    }
    lanes_minmax_any<NR>(mn1, mx1, R, L);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        if (RT == 0 && r >= R) break;
        const GroupParams p = group_params<BITS1>(mn1[r], mx1[r]);
        uint32_t w[W1];
        encode8<BITS1>(v1[r], p, w);
        const uint64_t e0 = (uint64_t)r * n + tile;
        if (valid) store_codes<BITS1, false>(codes1 + e0 * BITS1 / 8, rel, w);
        if (leader) {
            const uint64_t g = (uint64_t)r * (n >> g_shift) + gpos;
            s1[g] = p.s16;
            z1[g] = p.z16;
        }
    }

    // ---- stage 2: payload 1 read back, dequantized and summed in ascending
    // r from operand 0, requantized; payload 2 written ----
    handoff();
    const uint64_t gl = (tile + lrel) >> g_shift;          // group of the positions this lane reads
    uint32_t w1[NR][W1];
    uint16_t sv[NR], zv[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        if (RT == 0 && r >= R) break;
        const uint64_t e0 = (uint64_t)r * n + tile;
        const FC_GLOBAL uint8_t *cb = sgpr_ptr(codes1 + e0 * BITS1 / 8);
        const FC_GLOBAL uint16_t *sb = sgpr_ptr(s1 + (uint64_t)r * (n >> g_shift));
        const FC_GLOBAL uint16_t *zb = sgpr_ptr(z1 + (uint64_t)r * (n >> g_shift));
        if constexpr (BITS1 == 4) {
            w1[r][0] = ldg<uint32_t>(cb, lrel / 2);
        } else {
            const u32x2 c = ldg<u32x2>(cb, lrel);
            w1[r][0] = c.x;
            w1[r][W1 - 1] = c.y;
        }
        sv[r] = ldg<uint16_t>(sb, (uint32_t)gl * 2u);
        zv[r] = ldg<uint16_t>(zb, (uint32_t)gl * 2u);
    }
    float y[kLaneElems];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        if (RT == 0 && r >= R) break;
        float xh[kLaneElems];
        dequant8<BITS1>(w1[r], sv[r], zv[r], xh);
#pragma unroll
        for (int k = 0; k < kLaneElems; ++k) y[k] = r == 0 ? xh[k] : y[k] + xh[k];
    }
    float mn[1], mx[1];
    minmax8(y, mn[0], mx[0]);
    lanes_minmax_any<1>(mn, mx, 1, L);
    const GroupParams p2 = group_params<BITS2>(mn[0], mx[0]);
    uint32_t w2[W2];
    encode8<BITS2>(y, p2, w2);
    if (valid) store_codes<BITS2, false>(codes2 + tile * BITS2 / 8, rel, w2);
    if (leader) {
        s2[gpos] = p2.s16;
        z2[gpos] = p2.z16;
    }

    // ---- stage 3: payload 2 read back and dequantized (and the residual
    // added); the output written ----
    handoff();
    uint32_t w3[W2];
    {
        const FC_GLOBAL uint8_t *cb = sgpr_ptr(codes2 + tile * BITS2 / 8);
        if constexpr (BITS2 == 4) {
            w3[0] = ldg<uint32_t>(cb, lrel / 2);
        } else {
            const u32x2 c = ldg<u32x2>(cb, lrel);
            w3[0] = c.x;
            w3[W2 - 1] = c.y;
        }
    }
    const uint16_t s3 = ldg<uint16_t>(sgpr_ptr(s2), (uint32_t)gl * 2u);
    const uint16_t z3 = ldg<uint16_t>(sgpr_ptr(z2), (uint32_t)gl * 2u);
    float o[kLaneElems];
    dequant8<BITS2>(w3, s3, z3, o);
    u32x4 packed = narrow8<DT>(o);
    if constexpr (RES) {
        float a[kLaneElems], rr[kLaneElems];
        widen8<DT>(packed, a);   // the all-reduce result as the dtype holds it
        widen8<DT>(rv, rr);
#pragma unroll
        for (int k = 0; k < kLaneElems; ++k) a[k] = rr[k] + a[k];
        packed = narrow8<DT>(a);
    }
    if (valid) stv<u32x4, true>(out + tile, rel * 2, packed);
}

template <int DT, int BITS1, int BITS2, bool RES, int RT>
hipError_t launch_rt(const uint16_t *x, int R, uint64_t n, int g_shift, uint8_t *codes1,
                     uint16_t *s1, uint16_t *z1, uint8_t *codes2, uint16_t *s2, uint16_t *z2,
                     const uint16_t *res, uint16_t *out, hipStream_t stream) {
    constexpr uint64_t per_block = (uint64_t)kWavesPerBlock * kSlotElems;
    const uint64_t blocks = (n + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((allreduce_small_kernel<DT, BITS1, BITS2, RES, RT>), dim3((unsigned)blocks),
                       dim3(kBlockThreads), 0, stream, x, R, n, g_shift, codes1, s1, z1, codes2, s2,
                       z2, res, out);
    return hipGetLastError();
}

template <int DT, int BITS1, int BITS2, bool RES>
hipError_t launch_one(const uint16_t *x, int R, uint64_t n, int g_shift, uint8_t *codes1,
                      uint16_t *s1, uint16_t *z1, uint8_t *codes2, uint16_t *s2, uint16_t *z2,
                      const uint16_t *res, uint16_t *out, hipStream_t stream) {
#define FC_ARGS x, R, n, g_shift, codes1, s1, z1, codes2, s2, z2, res, out, stream
    switch (R) {
    case 8: return launch_rt<DT, BITS1, BITS2, RES, 8>(FC_ARGS);
    case 4: return launch_rt<DT, BITS1, BITS2, RES, 4>(FC_ARGS);
    case 2: return launch_rt<DT, BITS1, BITS2, RES, 2>(FC_ARGS);
    default: return launch_rt<DT, BITS1, BITS2, RES, 0>(FC_ARGS);
    }
#undef FC_ARGS
}

template <int DT, bool RES>
hipError_t by_bits(const uint16_t *x, int R, uint64_t n, int bits1, int bits2, int g_shift,
                   uint8_t *codes1, uint16_t *s1, uint16_t *z1, uint8_t *codes2, uint16_t *s2,
                   uint16_t *z2, const uint16_t *res, uint16_t *out, hipStream_t stream) {
#define FC_ARGS x, R, n, g_shift, codes1, s1, z1, codes2, s2, z2, res, out, stream
    if (bits1 == 4)
        return bits2 == 4 ? launch_one<DT, 4, 4, RES>(FC_ARGS) : launch_one<DT, 4, 8, RES>(FC_ARGS);
    return bits2 == 4 ? launch_one<DT, 8, 4, RES>(FC_ARGS) : launch_one<DT, 8, 8, RES>(FC_ARGS);
#undef FC_ARGS
}

}  // namespace

bool allreduce_small_applies(int R, uint64_t n, int group, int group2) {
    return R >= 1 && R <= kMaxR && group == group2 && group >= kLaneElems && group <= kSlotElems &&
           (group & (group - 1)) == 0 && (uint64_t)R * n <= kAllreduceSmallMaxElems;
}

hipError_t launch_allreduce_small(const uint16_t *x, int dtype, int R, uint64_t n, int bits1,
                                  int bits2, int group, uint8_t *codes1, uint16_t *s1,
                                  uint16_t *z1, uint8_t *codes2, uint16_t *s2, uint16_t *z2,
                                  const uint16_t *residual, uint16_t *out, hipStream_t stream) {
    const int sh = ilog2(group);
    if (residual) {
        return dtype == 0 ? by_bits<0, true>(x, R, n, bits1, bits2, sh, codes1, s1, z1, codes2, s2,
                                             z2, residual, out, stream)
                          : by_bits<1, true>(x, R, n, bits1, bits2, sh, codes1, s1, z1, codes2, s2,
                                             z2, residual, out, stream);
    }
    return dtype == 0 ? by_bits<0, false>(x, R, n, bits1, bits2, sh, codes1, s1, z1, codes2, s2, z2,
                                          nullptr, out, stream)
                      : by_bits<1, false>(x, R, n, bits1, bits2, sh, codes1, s1, z1, codes2, s2, z2,
                                          nullptr, out, stream);
}

}  // namespace fc
