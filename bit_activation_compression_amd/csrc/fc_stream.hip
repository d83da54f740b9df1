// Measurement helpers, not part of the codec. Streaming probes: the HBM
// bandwidth a plain kernel reaches for the traffic shapes of the codec's
// kernels, as the practical ceiling their measured bandwidth is compared
// with. A clock probe: the engine clock the GPU runs at, read between
// kernels of a running pipeline.
//
//   kind 0  copy            read n bytes, write n bytes
//   kind 1  read 4, write 1 read n bytes, write n/4 bytes (the stage-1
//                           quantizer's shape: 16-bit values in, 4-bit codes out)
//   kind 2  read            read n bytes (one 4-byte word written per wave)
//   kind 3  read 1, write 4 read n bytes, write 4n bytes (the final
//                           dequantizer's shape: 4-bit codes in, 16-bit values
//                           out)
//
// Kinds 0 to 2 follow the quantizer's access pattern: a wave owns a tile of U
// slots, a slot is 64 lanes x 16 bytes read (non-temporal), and the written
// part of a slot is one contiguous run per wave (non-temporal). Kind 3
// follows the dequantizer's: a slot is 64 lanes x 4 bytes read (cached) and
// 64 lanes x 16 bytes written (non-temporal). The loaded data feeds what is
// written, so no load can be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fc_device.h"
#include "fc_internal.h"

namespace fc {
namespace {

template <int KIND, int U>
__global__ __launch_bounds__(kBlockThreads) void stream_kernel(const uint8_t *__restrict__ src,
                                                               uint8_t *__restrict__ dst,
                                                               uint64_t n) {
    constexpr uint32_t kSlot = kWave * 16;   // bytes read per slot
    const int lane = lane_id();
    const uint64_t tile = wave_index() * (uint64_t)(U * kSlot);
    if (tile >= n) return;
    const uint64_t left = n - tile;
    const uint32_t avail = left < (uint64_t)(U * kSlot) ? (uint32_t)left : U * kSlot;
    const uint8_t *sb = src + tile;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t rel = u * kSlot + lane * 16u;
        v[u] = ldv<u32x4, true>(sb, rel < avail ? rel : 0u);
    }
    if constexpr (KIND == 0) {
        uint8_t *db = dst + tile;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t rel = u * kSlot + lane * 16u;
            if (rel < avail) stv<u32x4, true>(db, rel, v[u]);
        }
    } else if constexpr (KIND == 1) {
        uint8_t *db = dst + tile / 4;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t rel = u * kSlot + lane * 16u;
            if (rel < avail) stv<uint32_t, true>(db, rel / 4, v[u].x ^ v[u].y ^ v[u].z ^ v[u].w);
        }
    } else {
        uint32_t x = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) x ^= (uint32_t)__shfl_xor((int)x, d);
        if (lane == 0) stv<uint32_t, true>(dst, (uint32_t)(wave_index() * 4u), x);
    }
}

// read 1, write 4: lane words of 4 bytes in, 16 bytes out
template <int U>
__global__ __launch_bounds__(kBlockThreads) void expand_kernel(const uint8_t *__restrict__ src,
                                                               uint8_t *__restrict__ dst,
                                                               uint64_t n) {
    constexpr uint32_t kSlot = kWave * 4;   // bytes read per slot
    const int lane = lane_id();
    const uint64_t tile = wave_index() * (uint64_t)(U * kSlot);
    if (tile >= n) return;
    const uint64_t left = n - tile;
    const uint32_t avail = left < (uint64_t)(U * kSlot) ? (uint32_t)left : U * kSlot;
    const uint8_t *sb = src + tile;
    uint8_t *db = dst + 4 * tile;
    uint32_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t rel = u * kSlot + lane * 4u;
        v[u] = ldv<uint32_t, false>(sb, rel < avail ? rel : 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t rel = u * kSlot + lane * 4u;
        const u32x4 w = {v[u], v[u] ^ 1u, v[u] ^ 2u, v[u] ^ 3u};
        if (rel < avail) stv<u32x4, true>(db, rel * 4u, w);
    }
}

template <int KIND, int U>
hipError_t launch(const void *src, void *dst, uint64_t n, hipStream_t stream) {
    if constexpr (KIND == 3) {
        constexpr uint64_t per_block = (uint64_t)kWavesPerBlock * U * kWave * 4;
        const uint64_t blocks = (n + per_block - 1) / per_block;
        if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((expand_kernel<U>), dim3((unsigned)blocks), dim3(kBlockThreads), 0,
                           stream, static_cast<const uint8_t *>(src), static_cast<uint8_t *>(dst), n);
        return hipGetLastError();
    }
    constexpr uint64_t per_block = (uint64_t)kWavesPerBlock * U * kWave * 16;
    const uint64_t blocks = (n + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((stream_kernel<KIND, U>), dim3((unsigned)blocks), dim3(kBlockThreads), 0,
                       stream, static_cast<const uint8_t *>(src), static_cast<uint8_t *>(dst), n);
    return hipGetLastError();
}

template <int KIND>
hipError_t launch_u(int slots, const void *src, void *dst, uint64_t n, hipStream_t stream) {
    switch (slots) {
    case 1: return launch<KIND, 1>(src, dst, n, stream);
    case 2: return launch<KIND, 2>(src, dst, n, stream);
    case 4: return launch<KIND, 4>(src, dst, n, stream);
    case 8: return launch<KIND, 8>(src, dst, n, stream);
    default: return hipErrorInvalidValue;
    }
}

// One wave: the shader-clock counter (s_memtime) and the constant 100 MHz
// counter (s_memrealtime) around a chain of `iters` dependent fma, written to
// out[0] and out[1]; out[2] keeps the chain's result live.
__global__ void clock_probe_kernel(uint64_t *out, int iters) {
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    float a = (float)lane_id();
    for (int i = 0; i < iters; ++i) a = __builtin_fmaf(a, 0.999f, 1.0f);
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (lane_id() == 0) {
        out[0] = t1 - t0;
        out[1] = r1 - r0;
        out[2] = (uint64_t)__builtin_bit_cast(uint32_t, a);
    }
}

}  // namespace
}  // namespace fc

extern "C" int fc_internal_clock_probe(void *out, int iters, void *stream) {
    if (out == nullptr) return 1;
    if (iters < 1 || iters > (1 << 20)) return 2;
    if ((uintptr_t)out & 7u) return 4;
    hipLaunchKernelGGL(fc::clock_probe_kernel, dim3(1), dim3(fc::kWave), 0,
                       static_cast<hipStream_t>(stream), static_cast<uint64_t *>(out), iters);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}

extern "C" int fc_internal_stream_probe(int kind, int slots, const void *src, void *dst,
                                        size_t bytes, void *stream) {
    if (kind < 0 || kind > 3 || (slots != 1 && slots != 2 && slots != 4 && slots != 8)) return 2;
    if (bytes == 0) return 0;
    if (src == nullptr || dst == nullptr) return 1;
    if (bytes % 16 != 0 || ((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) return 4;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = kind == 0   ? fc::launch_u<0>(slots, src, dst, bytes, s)
                   : kind == 1 ? fc::launch_u<1>(slots, src, dst, bytes, s)
                   : kind == 2 ? fc::launch_u<2>(slots, src, dst, bytes, s)
                               : fc::launch_u<3>(slots, src, dst, bytes, s);
    return e == hipSuccess ? 0 : 6;
}
