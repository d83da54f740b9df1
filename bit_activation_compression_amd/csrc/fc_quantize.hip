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

// Tiles of 2 slots (2 KiB of input per wave, two 16-byte loads per lane in
// flight) with non-temporal loads and code stores. Measured on MI355X inside
// the whole pipeline: a plain read-4 / write-1 stream of this shape runs at
// 103 us over the 70B operands against 108 us with 4 slots and 114 us with
// one, and the quantizer follows it (2 slots 105.6 us, 4 slots 108 us); the
// pipeline step, which also depends on how K2 then reads the codes, goes
// from 171.6 to 166.6 us.
constexpr int kTileSlots = 2;

template <int DT, int BITS, int G>
__global__ __launch_bounds__(kBlockThreads) void quantize_kernel(
    const uint16_t *__restrict__ x, uint64_t n, uint8_t *__restrict__ codes,
    uint16_t *__restrict__ s_out, uint16_t *__restrict__ z_out) {
    constexpr int U = tile_slots(G, kTileSlots);                   // slots per wave tile
    static_assert((U * kSlotElems) % G == 0, "tiles start on a group boundary");

    const int lane = lane_id();
    const uint64_t wave = wave_index();
    const uint64_t tile = wave * (uint64_t)(U * kSlotElems);
    if (tile >= n) return;
    // Wave-uniform bases; tiles start on a group boundary.
    const uint16_t *xb = x + tile;
    uint8_t *cb = codes + tile * BITS / 8;
    uint16_t *sb = s_out + tile / G;
    uint16_t *zb = z_out + tile / G;
    const uint64_t left = n - tile;
    const uint32_t avail = left < (uint64_t)(U * kSlotElems) ? (uint32_t)left : U * kSlotElems;

    // Lanes past the end of the data (last tile only; n % 8 == 0, so a lane
    // has all 8 values or none) load the tile's first vector instead: every
    // load is unconditional and a tile's loads are in flight together. Such
    // lanes form whole groups of their own, and their stores are skipped.
    float v[U][kLaneElems];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t rel = u * kSlotElems + lane * kLaneElems;
        const u32x4 raw = ldv<u32x4, true>(xb, (rel < avail ? rel : 0u) * 2);
        widen8<DT>(raw, v[u]);
    }

    float mn[U], mx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) minmax8(v[u], mn[u], mx[u]);
    quantize_tile<BITS, G, U, true>(v, mn, mx, lane, avail, cb, sb, zb);
}

template <int DT, int BITS, int G>
hipError_t launch_one(const uint16_t *x, uint64_t n, uint8_t *codes, uint16_t *s, uint16_t *z,
                      hipStream_t stream) {
    constexpr uint64_t per_block = (uint64_t)kWavesPerBlock * tile_slots(G, kTileSlots) * kSlotElems;
    const uint64_t blocks = (n + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((quantize_kernel<DT, BITS, G>), dim3((unsigned)blocks), dim3(kBlockThreads), 0,
                       stream, x, n, codes, s, z);
    return hipGetLastError();
}

template <int DT, int BITS>
hipError_t dispatch_group(const uint16_t *x, uint64_t n, int group, uint8_t *codes, uint16_t *s,
                          uint16_t *z, hipStream_t stream) {
#define FC_CASE(G) \
    case G: return launch_one<DT, BITS, G>(x, n, codes, s, z, stream);
    switch (group) {
        FC_CASE(8) FC_CASE(16) FC_CASE(32) FC_CASE(64) FC_CASE(128) FC_CASE(256) FC_CASE(512)
        FC_CASE(1024) FC_CASE(2048) FC_CASE(4096) FC_CASE(8192)
    default: return hipErrorInvalidValue;
    }
#undef FC_CASE
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
