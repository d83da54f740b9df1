// Uncompressed all-reduce result, the comparator of "Flash Communication:
// Reducing Tensor Parallelization Bottleneck for Fast Large Language Model
// Inference" (Figure 1: an NCCL Ring All-Reduce of FP16 activations):
// out = round_half_even(sum_r x_r), summed in binary32 in ascending r.
//
// HBM-bound: per output element it reads R 16-bit values and writes one.
#include "fc_device.h"
#include "fc_launch.h"

namespace fc {
namespace {

constexpr int kSumSlots = 2;

template <int DT, int RT>
__global__ __launch_bounds__(kBlockThreads) void sum_kernel(const uint16_t *__restrict__ x, int R_arg,
                                                            uint64_t n, uint16_t *__restrict__ out) {
    constexpr int U = kSumSlots;
    const int R = RT > 0 ? RT : R_arg;
    const int lane = lane_id();
    const uint64_t tile = wave_index() * (uint64_t)(U * kSlotElems);
    if (tile >= n) return;
    const uint64_t left = n - tile;
    const uint32_t avail = left < (uint64_t)(U * kSlotElems) ? (uint32_t)left : U * kSlotElems;
    uint32_t lrel[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t rel = u * kSlotElems + lane * kLaneElems;
        lrel[u] = rel < avail ? rel : 0u;   // past the end: reload the first element, store nothing
    }
    float acc[U][kLaneElems];
    auto add_operand = [&](int r, bool first) {
        const uint16_t *xb = x + (uint64_t)r * n + tile;
        u32x4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = ldv<u32x4, true>(xb, lrel[u] * 2);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float v[kLaneElems];
            widen8<DT>(raw[u], v);
#pragma unroll
            for (int k = 0; k < kLaneElems; ++k) acc[u][k] = first ? v[k] : acc[u][k] + v[k];
        }
    };
    if constexpr (RT > 0) {
        // all R loads of the tile in flight before the first add
        u32x4 raw[RT][U];
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const uint16_t *xb = x + (uint64_t)r * n + tile;
#pragma unroll
            for (int u = 0; u < U; ++u) raw[r][u] = ldv<u32x4, true>(xb, lrel[u] * 2);
        }
#pragma unroll
        for (int r = 0; r < RT; ++r) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float v[kLaneElems];
                widen8<DT>(raw[r][u], v);
#pragma unroll
                for (int k = 0; k < kLaneElems; ++k) acc[u][k] = r == 0 ? v[k] : acc[u][k] + v[k];
            }
        }
    } else {
        add_operand(0, true);
        for (int r = 1; r < R; ++r) add_operand(r, false);
    }
    uint16_t *ob = out + tile;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t rel = u * kSlotElems + lane * kLaneElems;
        if (rel >= avail) continue;
        stv<u32x4, true>(ob, rel * 2, narrow8<DT>(acc[u]));
    }
}

template <int DT, int RT>
hipError_t launch_one(const uint16_t *x, int R, uint64_t n, uint16_t *out, hipStream_t stream) {
    constexpr uint64_t per_block = (uint64_t)kWavesPerBlock * kSumSlots * kSlotElems;
    const uint64_t blocks = (n + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((sum_kernel<DT, RT>), dim3((unsigned)blocks), dim3(kBlockThreads), 0, stream, x, R,
                       n, out);
    return hipGetLastError();
}

template <int DT>
hipError_t dispatch_r(const uint16_t *x, int R, uint64_t n, uint16_t *out, hipStream_t stream) {
    switch (R) {
    case 2: return launch_one<DT, 2>(x, R, n, out, stream);
    case 4: return launch_one<DT, 4>(x, R, n, out, stream);
    case 8: return launch_one<DT, 8>(x, R, n, out, stream);
    default: return launch_one<DT, 0>(x, R, n, out, stream);
    }
}

}  // namespace

hipError_t launch_sum(const uint16_t *x, int dtype, int R, uint64_t n, uint16_t *out, hipStream_t stream) {
    return dtype == 0 ? dispatch_r<0>(x, R, n, out, stream) : dispatch_r<1>(x, R, n, out, stream);
}

}  // namespace fc
