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
// requantized like stage 1. The incoming codes are BITS1 wide, the outgoing
// ones BITS2 (the same unless the caller asks for different widths).
//
// Per output element it reads R*bits1/8 code bytes (plus 4 bytes per stage-1
// group and operand) and writes bits2/8 code bytes (plus 4 per stage-2
// group). The fp32 work per element grows with R (decode, fma, add per
// operand), so for R = 4 the kernel is bound by vector ALU issue rather than
// by HBM.
#include "fc_device.h"
#include "fc_launch.h"

namespace fc {
namespace {

// RT > 0: the operand count is a compile-time constant (all loads of a tile
// are issued before the first use); RT == 0: any R, one operand at a time.
constexpr int base_slots(int RT) { return RT >= 8 ? 2 : 4; }

template <int BITS1, int BITS2, int G2, int RT>
__global__ __launch_bounds__(kBlockThreads) void dsr_kernel(
    const uint8_t *__restrict__ codes1, const uint16_t *__restrict__ s1,
    const uint16_t *__restrict__ z1, int R_arg, uint64_t n, int g1_shift,
    uint8_t *__restrict__ codes2, uint16_t *__restrict__ s2, uint16_t *__restrict__ z2) {
    constexpr int U = tile_slots(G2, base_slots(RT));
    constexpr int W = BITS1 == 4 ? 1 : 2;
    static_assert((U * kSlotElems) % G2 == 0, "tiles start on a group boundary");
    const int R = RT > 0 ? RT : R_arg;

    const int lane = lane_id();
    const uint64_t wave = wave_index();
    const uint64_t tile = wave * (uint64_t)(U * kSlotElems);
    if (tile >= n) return;
    const uint64_t left = n - tile;
    const uint32_t avail = left < (uint64_t)(U * kSlotElems) ? (uint32_t)left : U * kSlotElems;

    // Stage-1 metadata index of element (r, tile + rel):
    //   ((r*n + tile) >> s) + (((tile mod 2^s) + rel) >> s),
    // since r*n is a multiple of the stage-1 group; the second term is the
    // same for every operand.
    // Lanes past the end of the data (last tile only) load the tile's first
    // element instead, so every load is unconditional and all of a tile's
    // loads are in flight together; only their stores are skipped.
    const uint32_t mis = (uint32_t)tile & ((1u << g1_shift) - 1u);
    uint32_t lrel[U], mrel[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t rel = u * kSlotElems + lane * kLaneElems;
        lrel[u] = rel < avail ? rel : 0u;
        mrel[u] = (mis + lrel[u]) >> g1_shift;
    }

    float y[U][kLaneElems];
    auto load_operand = [&](int r, uint32_t (&w)[U][W], uint16_t (&sv)[U], uint16_t (&zv)[U]) {
        const uint64_t e0 = (uint64_t)r * n + tile;
        const uint8_t *cb = codes1 + e0 * BITS1 / 8;
        const uint16_t *sb = s1 + (e0 >> g1_shift);
        const uint16_t *zb = z1 + (e0 >> g1_shift);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            load_codes<BITS1, false>(cb, lrel[u], w[u]);
            sv[u] = sb[mrel[u]];
            zv[u] = zb[mrel[u]];
        }
    };
    // x_hat = fp32(q*s + z), rounded once (dequant8)
    auto add_operand = [&](bool first, const uint32_t (&w)[U][W], const uint16_t (&sv)[U],
                           const uint16_t (&zv)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float xh[kLaneElems];
            dequant8<BITS1>(w[u], sv[u], zv[u], xh);
#pragma unroll
            for (int k = 0; k < kLaneElems; ++k) y[u][k] = first ? xh[k] : y[u][k] + xh[k];
        }
    };

    if constexpr (RT > 0) {
        uint32_t w[RT][U][W];
        uint16_t sv[RT][U], zv[RT][U];
#pragma unroll
        for (int r = 0; r < RT; ++r) load_operand(r, w[r], sv[r], zv[r]);
#pragma unroll
        for (int r = 0; r < RT; ++r) add_operand(r == 0, w[r], sv[r], zv[r]);
    } else {
        uint32_t w[U][W];
        uint16_t sv[U], zv[U];
        load_operand(0, w, sv, zv);
        add_operand(true, w, sv, zv);
        for (int r = 1; r < R; ++r) {
            load_operand(r, w, sv, zv);
            add_operand(false, w, sv, zv);
        }
    }

    // requantize the sums in groups of G2 (tiles start on a group boundary)
    float mn[U], mx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) minmax8(y[u], mn[u], mx[u]);
    quantize_tile<BITS2, G2, U, false>(y, mn, mx, lane, avail, codes2 + tile * BITS2 / 8,
                                       s2 + tile / G2, z2 + tile / G2);
}

template <int BITS1, int BITS2, int G2, int RT>
hipError_t launch_one(const uint8_t *codes1, const uint16_t *s1, const uint16_t *z1, int R,
                      uint64_t n, int g1_shift, uint8_t *codes2, uint16_t *s2, uint16_t *z2,
                      hipStream_t stream) {
    constexpr uint64_t per_block =
        (uint64_t)kWavesPerBlock * tile_slots(G2, base_slots(RT)) * kSlotElems;
    const uint64_t blocks = (n + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((dsr_kernel<BITS1, BITS2, G2, RT>), dim3((unsigned)blocks), dim3(kBlockThreads),
                       0, stream, codes1, s1, z1, R, n, g1_shift, codes2, s2, z2);
    return hipGetLastError();
}

template <int BITS1, int BITS2, int G2>
hipError_t dispatch_r(const uint8_t *codes1, const uint16_t *s1, const uint16_t *z1, int R,
                      uint64_t n, int g1_shift, uint8_t *codes2, uint16_t *s2, uint16_t *z2,
                      hipStream_t stream) {
    // The compile-time operand count keeps R x U code words in flight; it is
    // used only where a tile is the base size, so registers stay bounded.
#define FC_LAUNCH(RT) \
    launch_one<BITS1, BITS2, G2, RT>(codes1, s1, z1, R, n, g1_shift, codes2, s2, z2, stream)
    if constexpr (G2 <= kSlotElems * base_slots(8)) {
        if (R == 8) return FC_LAUNCH(8);
    }
    if constexpr (G2 <= kSlotElems * base_slots(4)) {
        if (R == 4) return FC_LAUNCH(4);
        if (R == 2) return FC_LAUNCH(2);
    }
    return FC_LAUNCH(0);
#undef FC_LAUNCH
}

template <int BITS1, int BITS2>
hipError_t dispatch_group(const uint8_t *codes1, const uint16_t *s1, const uint16_t *z1, int R,
                          uint64_t n, int g1_shift, int group2, uint8_t *codes2, uint16_t *s2,
                          uint16_t *z2, hipStream_t stream) {
#define FC_CASE(G) \
    case G: return dispatch_r<BITS1, BITS2, G>(codes1, s1, z1, R, n, g1_shift, codes2, s2, z2, stream);
    switch (group2) {
        FC_CASE(8) FC_CASE(16) FC_CASE(32) FC_CASE(64) FC_CASE(128) FC_CASE(256) FC_CASE(512)
        FC_CASE(1024) FC_CASE(2048) FC_CASE(4096) FC_CASE(8192)
    default: return hipErrorInvalidValue;
    }
#undef FC_CASE
}

}  // namespace

hipError_t launch_dequant_sum_requant(const uint8_t *codes1, const uint16_t *s1, const uint16_t *z1,
                                      int R, uint64_t n, int bits1, int bits2, int group1,
                                      int group2, uint8_t *codes2, uint16_t *s2, uint16_t *z2,
                                      hipStream_t stream) {
    const int sh = ilog2(group1);
    if (bits1 == 4)
        return bits2 == 4 ? dispatch_group<4, 4>(codes1, s1, z1, R, n, sh, group2, codes2, s2, z2, stream)
                          : dispatch_group<4, 8>(codes1, s1, z1, R, n, sh, group2, codes2, s2, z2, stream);
    return bits2 == 4 ? dispatch_group<8, 4>(codes1, s1, z1, R, n, sh, group2, codes2, s2, z2, stream)
                      : dispatch_group<8, 8>(codes1, s1, z1, R, n, sh, group2, codes2, s2, z2, stream);
}

}  // namespace fc
