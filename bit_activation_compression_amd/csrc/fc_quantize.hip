// Stage-1 quantizer: the quantization before the Reduce-Scatter of
// "Flash Communication: Reducing Tensor Parallelization Bottleneck for Fast
// Large Language Model Inference" (Figure 5, right), with block-wise groups
// along the hidden dimension (Figure 4).
//
// The R operands [R][T][H] are one flat run of n = R*T*H values; groups of G
// consecutive values never cross a token row because G divides H, so the
// flat view gives the same groups as the (r, t, k) indexing.
//
// HBM-bound: per element it reads 2 bytes and writes bits/8 bytes, plus
// 4 bytes of scale and zero per group.
#include "fc_device.h"
#include "fc_launch.h"

namespace fc {
namespace {

template <int DT, int BITS, int G>
__global__ __launch_bounds__(kBlockThreads) void quantize_kernel(
    const uint16_t *__restrict__ x, uint64_t n, uint8_t *__restrict__ codes,
    uint16_t *__restrict__ s_out, uint16_t *__restrict__ z_out) {
    constexpr int U = tile_slots(G);                               // slots per wave tile
    constexpr int S = G > kSlotElems ? G / kSlotElems : 1;        // slots per group
    constexpr int L = G >= kSlotElems ? kWave : G / kLaneElems;   // lanes per group in a slot
    static_assert(U % S == 0, "a tile holds whole groups");

    const int lane = threadIdx.x & (kWave - 1);
    const uint64_t wave = (uint64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
    const uint64_t tile = wave * (uint64_t)(U * kSlotElems);
    if (tile >= n) return;

    float v[U][kLaneElems];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t e = tile + (uint64_t)(u * kSlotElems + lane * kLaneElems);
        ok[u] = e < n;   // n % 8 == 0: a lane's 8 values are all present or all absent
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (ok[u]) raw = *reinterpret_cast<const uint4 *>(x + e);
        widen8<DT>(raw, v[u]);
    }

    float mn[U], mx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) minmax8(v[u], mn[u], mx[u]);

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
            uint32_t w[BITS == 4 ? 1 : 2];
            encode8<BITS>(v[u], p, w);
            store_codes<BITS>(codes, e, w);
            const bool leader = (S > 1) ? (k == 0 && lane == 0) : (lane % L == 0);
            if (leader) {
                const uint64_t m = e / G;
                s_out[m] = p.s16;
                z_out[m] = p.z16;
            }
        }
    }
}

template <int DT, int BITS, int G>
hipError_t launch_one(const uint16_t *x, uint64_t n, uint8_t *codes, uint16_t *s, uint16_t *z,
                      hipStream_t stream) {
    constexpr uint64_t per_block = (uint64_t)kWavesPerBlock * tile_slots(G) * kSlotElems;
    const uint64_t blocks = (n + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((quantize_kernel<DT, BITS, G>), dim3((unsigned)blocks), dim3(kBlockThreads), 0,
                       stream, x, n, codes, s, z);
    return hipGetLastError();
}

template <int DT, int BITS>
hipError_t dispatch_group(const uint16_t *x, uint64_t n, int group, uint8_t *codes, uint16_t *s,
                          uint16_t *z, hipStream_t stream) {
    switch (group) {
    case 8: return launch_one<DT, BITS, 8>(x, n, codes, s, z, stream);
    case 16: return launch_one<DT, BITS, 16>(x, n, codes, s, z, stream);
    case 32: return launch_one<DT, BITS, 32>(x, n, codes, s, z, stream);
    case 64: return launch_one<DT, BITS, 64>(x, n, codes, s, z, stream);
    case 128: return launch_one<DT, BITS, 128>(x, n, codes, s, z, stream);
    case 256: return launch_one<DT, BITS, 256>(x, n, codes, s, z, stream);
    case 512: return launch_one<DT, BITS, 512>(x, n, codes, s, z, stream);
    case 1024: return launch_one<DT, BITS, 1024>(x, n, codes, s, z, stream);
    case 2048: return launch_one<DT, BITS, 2048>(x, n, codes, s, z, stream);
    case 4096: return launch_one<DT, BITS, 4096>(x, n, codes, s, z, stream);
    case 8192: return launch_one<DT, BITS, 8192>(x, n, codes, s, z, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_quantize(const uint16_t *x, int dtype, uint64_t n, int bits, int group,
                           uint8_t *codes, uint16_t *s, uint16_t *z, hipStream_t stream) {
    if (dtype == 0) {
        return bits == 4 ? dispatch_group<0, 4>(x, n, group, codes, s, z, stream)
                         : dispatch_group<0, 8>(x, n, group, codes, s, z, stream);
    }
    return bits == 4 ? dispatch_group<1, 4>(x, n, group, codes, s, z, stream)
                     : dispatch_group<1, 8>(x, n, group, codes, s, z, stream);
}

}  // namespace fc
