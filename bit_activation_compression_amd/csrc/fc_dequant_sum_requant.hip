// Reduce-Scatter reduction and requantization before the All-Gather of
// "Flash Communication: Reducing Tensor Parallelization Bottleneck for Fast
// Large Language Model Inference" (Figure 5, right; TL;DR "two-step
// All-Reduce").
//
// Chunk j of the hidden dimension (columns [j*C, (j+1)*C), C = H/R) is what
// rank j reduces. Stage-2 groups of g2 = min(group, C) columns never cross a
// chunk or a row, so over the n = T*H output positions the chunking reduces
// to flat groups of g2: position p reads code p of every operand r (operand
// stride n), dequantizes each with its own stage-1 scale and zero, sums them
// in binary32 in ascending r starting from operand 0, and the sums are
// requantized like stage 1.
//
// Per output element it reads R*bits/8 code bytes (plus 4 bytes per stage-1
// group and operand) and writes bits/8 code bytes (plus 4 per stage-2 group).
// The fp32 work per element grows with R (decode, fma, add per operand).
#include "fc_device.h"
#include "fc_launch.h"

namespace fc {
namespace {

constexpr int kOperandBatch = 4;   // operands whose loads are in flight together

template <int BITS, int G2>
__global__ __launch_bounds__(kBlockThreads) void dsr_kernel(
    const uint8_t *__restrict__ codes1, const uint16_t *__restrict__ s1,
    const uint16_t *__restrict__ z1, int R, uint64_t n, int g1_shift,
    uint8_t *__restrict__ codes2, uint16_t *__restrict__ s2, uint16_t *__restrict__ z2) {
    constexpr int U = tile_slots(G2);
    constexpr int S = G2 > kSlotElems ? G2 / kSlotElems : 1;
    constexpr int L = G2 >= kSlotElems ? kWave : G2 / kLaneElems;
    constexpr int W = BITS == 4 ? 1 : 2;
    static_assert(U % S == 0, "a tile holds whole groups");

    const int lane = threadIdx.x & (kWave - 1);
    const uint64_t wave = (uint64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
    const uint64_t tile = wave * (uint64_t)(U * kSlotElems);
    if (tile >= n) return;

    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        ok[u] = tile + (uint64_t)(u * kSlotElems + lane * kLaneElems) < n;

    float y[U][kLaneElems] = {};
    for (int r0 = 0; r0 < R; r0 += kOperandBatch) {
        uint32_t w[kOperandBatch][U][W];
        uint16_t sb[kOperandBatch][U], zb[kOperandBatch][U];
#pragma unroll
        for (int i = 0; i < kOperandBatch; ++i) {
            if (r0 + i >= R) break;
            const uint64_t base = (uint64_t)(r0 + i) * n;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint64_t e = base + tile + (uint64_t)(u * kSlotElems + lane * kLaneElems);
                if (ok[u]) {
                    load_codes<BITS>(codes1, e, w[i][u]);
                    sb[i][u] = s1[e >> g1_shift];
                    zb[i][u] = z1[e >> g1_shift];
                } else {
#pragma unroll
                    for (int k = 0; k < W; ++k) w[i][u][k] = 0;
                    sb[i][u] = 0;
                    zb[i][u] = 0;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kOperandBatch; ++i) {
            if (r0 + i >= R) break;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float q[kLaneElems];
                decode8<BITS>(w[i][u], q);
                const float s = half_bits_to_float(sb[i][u]);
                const float z = half_bits_to_float(zb[i][u]);
#pragma unroll
                for (int k = 0; k < kLaneElems; ++k) {
                    const float xh = __builtin_fmaf(q[k], s, z);   // q*s exact: equals fp32(q*s + z)
                    y[u][k] = (r0 + i == 0) ? xh : y[u][k] + xh;
                }
            }
        }
    }

    float mn[U], mx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) minmax8(y[u], mn[u], mx[u]);

#pragma unroll
    for (int g = 0; g < U / S; ++g) {
        float a = mn[g * S], b = mx[g * S];
#pragma unroll
        for (int k = 1; k < S; ++k) {
            a = __builtin_fminf(a, mn[g * S + k]);
            b = __builtin_fmaxf(b, mx[g * S + k]);
        }
        lanes_minmax<L>(a, b);
        const GroupParams p = group_params<BITS>(a, b);
#pragma unroll
        for (int k = 0; k < S; ++k) {
            const int u = g * S + k;
            const uint64_t e = tile + (uint64_t)(u * kSlotElems + lane * kLaneElems);
            if (!ok[u]) continue;
            uint32_t w[W];
            encode8<BITS>(y[u], p, w);
            store_codes<BITS>(codes2, e, w);
            const bool leader = (S > 1) ? (k == 0 && lane == 0) : (lane % L == 0);
            if (leader) {
                const uint64_t m = e / G2;
                s2[m] = p.s16;
                z2[m] = p.z16;
            }
        }
    }
}

template <int BITS, int G2>
hipError_t launch_one(const uint8_t *codes1, const uint16_t *s1, const uint16_t *z1, int R,
                      uint64_t n, int g1_shift, uint8_t *codes2, uint16_t *s2, uint16_t *z2,
                      hipStream_t stream) {
    constexpr uint64_t per_block = (uint64_t)kWavesPerBlock * tile_slots(G2) * kSlotElems;
    const uint64_t blocks = (n + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((dsr_kernel<BITS, G2>), dim3((unsigned)blocks), dim3(kBlockThreads), 0, stream,
                       codes1, s1, z1, R, n, g1_shift, codes2, s2, z2);
    return hipGetLastError();
}

template <int BITS>
hipError_t dispatch_group(const uint8_t *codes1, const uint16_t *s1, const uint16_t *z1, int R,
                          uint64_t n, int g1_shift, int group2, uint8_t *codes2, uint16_t *s2,
                          uint16_t *z2, hipStream_t stream) {
#define FC_CASE(G)                                                                               \
    case G: return launch_one<BITS, G>(codes1, s1, z1, R, n, g1_shift, codes2, s2, z2, stream);
    switch (group2) {
        FC_CASE(8) FC_CASE(16) FC_CASE(32) FC_CASE(64) FC_CASE(128) FC_CASE(256) FC_CASE(512)
        FC_CASE(1024) FC_CASE(2048) FC_CASE(4096) FC_CASE(8192)
    default: return hipErrorInvalidValue;
    }
#undef FC_CASE
}

}  // namespace

hipError_t launch_dequant_sum_requant(const uint8_t *codes1, const uint16_t *s1, const uint16_t *z1,
                                      int R, uint64_t n, int bits, int group1, int group2,
                                      uint8_t *codes2, uint16_t *s2, uint16_t *z2,
                                      hipStream_t stream) {
    const int g1_shift = ilog2(group1);
    return bits == 4 ? dispatch_group<4>(codes1, s1, z1, R, n, g1_shift, group2, codes2, s2, z2, stream)
                     : dispatch_group<8>(codes1, s1, z1, R, n, g1_shift, group2, codes2, s2, z2, stream);
}

}  // namespace fc
