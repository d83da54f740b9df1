// Row-parallel linear layer with the stage-1 quantization in its epilogue.
//
// In the tensor-parallel transformer block of "Flash Communication: Reducing
// Tensor Parallelization Bottleneck for Fast Large Language Model Inference"
// (Figure 3) the all-reduced activations are the partial outputs of the
// attention output projection and of the MLP down projection (Figure 5, left:
// o_proj and d_proj). Rank r multiplies its slice of the layer input,
// A_r [T][K], by its input columns of the weight, W_r [H][K], and quantizes
// the partial sum y_r = A_r W_r^T [T][H] before the Reduce-Scatter. This
// kernel does both in one pass: y_r never goes to HBM (unless asked for), the
// quantizer reads it from the matrix-core accumulators.
//
// Result: y_r is rounded from the binary32 accumulator to the activation dtype
// (what the layer would store), and its codes, scales and zeros are exactly
// those the separate stage-1 quantizer gives for that stored y_r.
//
// Work layout (gfx950, wave64, v_mfma_f32_32x32x16_{bf16,f16}):
//   - a workgroup of 4 waves owns a 256 (channels n) x 256 (tokens t) output
//     tile of one rank; wave (wn, wt) owns 128 x 128 of it as 4 x 4 MFMA
//     blocks of 32 x 32;
//   - the MFMA's row operand is W (rows n) and its column operand is A (rows
//     t), so the accumulator of a lane holds, for ONE token t (lane % 32), 16
//     channels n = 8*(v/4) + 4*(lane/32) + v%4 of each block: a quantization
//     group (<= 128 consecutive channels of one token) lies in one lane pair
//     (lane, lane ^ 32), half in each, and its minimum and maximum need one
//     v_permlane32_swap after the in-lane reduction;
//   - K is walked in stages of 64: both 256 x 64 operand tiles are staged in
//     LDS (double-buffered, 128 KiB) straight from global memory
//     (global_load_lds), each row's eight 16-byte chunks placed at
//     chunk ^ (row % 8) so that the fragment reads (32 rows x one chunk) are
//     free of bank conflicts; the next stage's loads are in flight while the
//     matrix cores work on the current one;
//   - workgroups are numbered so that each XCD (its own L2) runs a contiguous
//     run of tiles, ordered 4 token tiles x all channel tiles, so that
//     concurrently running workgroups share their A and W stage tiles in L2.
#include <type_traits>

#include "fc_device.h"
#include "fc_launch.h"

namespace fc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTileN = 256;                 // output channels per workgroup
constexpr int kTileT = 256;                 // tokens per workgroup
constexpr int kTileK = 64;                  // k per LDS stage
constexpr int kWaveSpan = 128;              // channels (and tokens) per wave
constexpr int kBlk = kWaveSpan / 32;        // 32 x 32 MFMA blocks per wave side
constexpr int kStage = (kTileN + kTileT) * kTileK;   // 16-bit elements per stage
constexpr int kGroupT = 4;                  // token tiles per scheduling group
constexpr int kXcds = 8;

static_assert(kBlockThreads == 256, "four waves per workgroup");

template <int DT>
__device__ __forceinline__ f32x16 mfma(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
    if constexpr (DT == 1)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Element offset of chunk c of staged row `row`.
__device__ __forceinline__ uint32_t lds_at(uint32_t row, uint32_t c) {
    return row * kTileK + ((c ^ (row & 7u)) << 3);
}

// Codes of 4 consecutive channels, same arithmetic as the stage-1 quantizer:
// 8-bit codes in the 4 bytes of the result, 4-bit codes in its low 16 bits
// (element 2i in the low nibble of byte i).
template <int BITS>
__device__ __forceinline__ uint32_t encode4(const float *v, const GroupParams &p) {
    float t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = (v[i] - p.z) * p.inv;
    if constexpr (BITS == 8) {
        uint32_t a = __builtin_amdgcn_cvt_pk_u8_f32(t[0], 0, 0u);
        a = __builtin_amdgcn_cvt_pk_u8_f32(t[1], 1, a);
        a = __builtin_amdgcn_cvt_pk_u8_f32(t[2], 2, a);
        return __builtin_amdgcn_cvt_pk_u8_f32(t[3], 3, a);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = __builtin_amdgcn_fmed3f(t[i], 0.0f, 15.0f);
        uint32_t ev = __builtin_amdgcn_cvt_pk_u8_f32(t[0], 0, 0u);
        ev = __builtin_amdgcn_cvt_pk_u8_f32(t[2], 1, ev);
        uint32_t od = __builtin_amdgcn_cvt_pk_u8_f32(t[1], 0, 0u);
        od = __builtin_amdgcn_cvt_pk_u8_f32(t[3], 1, od);
        return ev | (od << 4);
    }
}

// Two binary32 values rounded to the dtype (nearest even) and packed, the
// first in the low half; the as_f32 barrier keeps the conversion a plain
// v_cvt_pk_{bf16,f16}_f32 of the finished binary32 value.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    const f32x2 pair = {as_f32(a), as_f32(b)};
    if constexpr (DT == 1) return __builtin_bit_cast(uint32_t, __builtin_convertvector(pair, bf16x2));
    else return __builtin_bit_cast(uint32_t, __builtin_convertvector(pair, f16x2));
}

template <int DT>
__device__ __forceinline__ void unpack2(uint32_t w, float &a, float &b) {
    if constexpr (DT == 1) {
        a = __builtin_bit_cast(float, w << 16);
        b = __builtin_bit_cast(float, w & 0xFFFF0000u);
    } else {
        const f16x2 h = __builtin_bit_cast(f16x2, w);
        a = (float)h.x;
        b = (float)h.y;
    }
}

// min/max over the lane pair (lane, lane ^ 32): v_permlane32_swap of a value
// with itself leaves the two halves' values in the two results.
__device__ __forceinline__ void pair_minmax(float &mn, float &mx) {
    const auto a = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mn),
                                                    __builtin_bit_cast(uint32_t, mn), false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mx),
                                                    __builtin_bit_cast(uint32_t, mx), false, false);
    mn = __builtin_fminf(__builtin_bit_cast(float, (uint32_t)a[0]),
                         __builtin_bit_cast(float, (uint32_t)a[1]));
    mx = __builtin_fmaxf(__builtin_bit_cast(float, (uint32_t)b[0]),
                         __builtin_bit_cast(float, (uint32_t)b[1]));
}

template <int DT, int BITS, int G>
__global__ __launch_bounds__(kBlockThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void linear_quantize_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ W, int T, int K, int H,
    int tiles_t, int tiles_n, int total, uint8_t *__restrict__ codes, uint16_t *__restrict__ s,
    uint16_t *__restrict__ z, uint16_t *__restrict__ y) {
    static_assert(G >= 8 && G <= kWaveSpan && (G & (G - 1)) == 0, "group of 8..128 channels");
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kStage];

    const uint32_t tid = __builtin_amdgcn_workitem_id_x();
    const int lane = (int)(tid & 63u);
    const int wave = __builtin_amdgcn_readfirstlane((int)(tid >> 6));
    const int wn = wave & 1, wt = wave >> 1;

    // workgroup -> tile: XCD-contiguous runs, then kGroupT token tiles x all
    // channel tiles of one rank
    const int bid = (int)__builtin_amdgcn_workgroup_id_x();
    const int logical = (total % kXcds == 0) ? (bid % kXcds) * (total / kXcds) + bid / kXcds : bid;
    const int per_rank = tiles_t * tiles_n;
    const int r = logical / per_rank;
    const int i = logical - r * per_rank;
    const int grp = i / (kGroupT * tiles_n);
    const int first_t = grp * kGroupT;
    const int gsize = min(tiles_t - first_t, kGroupT);
    const int in_grp = i - grp * kGroupT * tiles_n;
    const int tile_t = first_t + in_grp % gsize;
    const int tile_n = in_grp / gsize;
    const int n0 = tile_n * kTileN, t0 = tile_t * kTileT;

    const uint16_t *Wb = W + ((size_t)r * H + n0) * (size_t)K;
    const uint16_t *Ab = A + ((size_t)r * T + t0) * (size_t)K;
    const uint32_t rowb = (uint32_t)K * 2u;          // bytes per operand row
    const uint32_t last_t = (uint32_t)(T - 1 - t0);  // rows past it re-read it (ragged T)

    // Staging, global -> LDS directly (global_load_lds_dwordx4: lane i's 16
    // bytes land at the instruction's LDS base + 16 i). One instruction fills
    // 8 staged rows; lane i serves row i / 8 at chunk position i % 8, so it
    // fetches the operand's chunk (i % 8) ^ (row % 8) -- the swizzle lds_at
    // reads back. Wave w fills rows w*64 .. w*64+63 of both tiles (8
    // instructions each). Token rows past the end re-read the last one.
    const uint32_t lrow = (uint32_t)lane >> 3;                 // == row % 8
    const uint32_t lchunk = ((uint32_t)lane & 7u) ^ lrow;
    const uint32_t wrow0 = (uint32_t)wave * 64u;
    const char *Wc = reinterpret_cast<const char *>(Wb);
    const char *Ac = reinterpret_cast<const char *>(Ab);
    uint32_t w_off[8], a_off[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t row = wrow0 + 8u * j + lrow;
        w_off[j] = row * rowb + lchunk * 16u;
        a_off[j] = (row < last_t ? row : last_t) * rowb + lchunk * 16u;
    }
    auto stage_in = [&](int kt, int buf) {
        const uint32_t kb = (uint32_t)kt * (kTileK * 2);
        uint16_t *sw = lds + buf * kStage;
        uint16_t *sa = sw + kTileN * kTileK;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t lrow0 = (wrow0 + 8u * j) * kTileK;   // wave-uniform
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(Wc + w_off[j] + kb),
                (__attribute__((address_space(3))) void *)(sw + lrow0), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(Ac + a_off[j] + kb),
                (__attribute__((address_space(3))) void *)(sa + lrow0), 16, 0, 0);
        }
    };

    // fragment reads: row (block base + lane % 32), chunk 2 ks + lane / 32
    const uint32_t frow = (uint32_t)lane & 31u, fhalf = (uint32_t)lane >> 5;
    auto frags = [&](const uint16_t *sw, const uint16_t *sa, int ks, u32x4 (&fw)[kBlk],
                     u32x4 (&fa)[kBlk]) {
        const uint32_t c = 2u * ks + fhalf;
#pragma unroll
        for (int b = 0; b < kBlk; ++b) {
            fw[b] = *reinterpret_cast<const u32x4 *>(sw + lds_at(wn * kWaveSpan + b * 32 + frow, c));
            fa[b] = *reinterpret_cast<const u32x4 *>(sa + lds_at(wt * kWaveSpan + b * 32 + frow, c));
        }
    };

    f32x16 acc[kBlk][kBlk];
#pragma unroll
    for (int a = 0; a < kBlk; ++a)
#pragma unroll
        for (int b = 0; b < kBlk; ++b) acc[a][b] = f32x16{};

    // One stage = 4 steps of k = 16, 16 MFMAs each. Software pipeline: the
    // next stage's staging loads go out at the start; each step's MFMAs are
    // interleaved with the LDS reads of the next step's fragments; the
    // workgroup barrier that publishes the next stage sits before the last
    // step, whose MFMAs then overlap the reads of the next stage's first
    // fragments (every read of the current buffer has been issued and waited
    // for by then, so the following stage may refill it).
    u32x4 fw[2][kBlk], fa[2][kBlk];
    auto step = [&](int ks) {
#pragma unroll
        for (int nb = 0; nb < kBlk; ++nb)
#pragma unroll
            for (int tb = 0; tb < kBlk; ++tb)
                acc[nb][tb] = mfma<DT>(fw[ks & 1][nb], fa[ks & 1][tb], acc[nb][tb]);
    };
    // 16 MFMAs interleaved with 8 LDS reads and optionally 8 staging loads
    auto interleave = [&](bool lds_reads, bool vmem) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (vmem) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            if (lds_reads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto stage = [&](int kt, auto next_tag) {
        constexpr bool NEXT = decltype(next_tag)::value;
        const int buf = kt & 1;
        const uint16_t *sw = lds + buf * kStage;
        const uint16_t *sa = sw + kTileN * kTileK;
        if constexpr (NEXT) stage_in(kt + 1, buf ^ 1);
        frags(sw, sa, 1, fw[1], fa[1]);
        step(0);
        interleave(true, NEXT);
        frags(sw, sa, 2, fw[0], fa[0]);
        step(1);
        interleave(true, NEXT);
        frags(sw, sa, 3, fw[1], fa[1]);
        step(2);
        interleave(true, false);
        if constexpr (NEXT) {
            __builtin_amdgcn_s_waitcnt(0);   // this wave's staging loads have landed
            __syncthreads();
            const uint16_t *nw = lds + (buf ^ 1) * kStage;
            frags(nw, nw + kTileN * kTileK, 0, fw[0], fa[0]);
        }
        step(3);
        interleave(NEXT, false);
    };

    const int KT = K / kTileK;
    stage_in(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    frags(lds, lds + kTileN * kTileK, 0, fw[0], fa[0]);
    for (int kt = 0; kt + 1 < KT; ++kt) stage(kt, std::true_type{});
    stage(KT - 1, std::false_type{});

    // ---- epilogue: round to the dtype, quantize per (token, group) ----
    // Run j = 4 nb + m of a lane holds channels nb*32 + 8m + 4*(lane/32) + 0..3
    // of the wave's span (accumulator entries 4m..4m+3 of block nb); a group
    // of G channels is RG = G/8 consecutive runs of each lane of the pair.
    constexpr int RG = G / 8;
    const int Hg = H / G;
    const uint32_t h4 = 4u * fhalf;
    // wave-uniform bases of this wave's first token row; per-lane 32-bit offsets
    const uint32_t crow_b = (uint32_t)H * BITS / 8;           // code bytes per token row
    const uint32_t lane_c = frow * crow_b;
    const uint32_t lane_y = frow * (uint32_t)H * 2u;
    const uint32_t lane_m = frow * (uint32_t)Hg * 2u;
#pragma unroll
    for (int tb = 0; tb < kBlk; ++tb) {
        const int trow0 = t0 + wt * kWaveSpan + tb * 32;   // wave-uniform
        const bool live = trow0 + (int)frow < T;
        const size_t row0 = (size_t)r * T + (size_t)trow0;
        const size_t col0 = (size_t)(n0 + wn * kWaveSpan);
        uint8_t *cb = codes + (row0 * (size_t)H + col0) * BITS / 8;
        uint16_t *yb = y ? y + row0 * (size_t)H + col0 : nullptr;
        uint16_t *sb = s + row0 * (size_t)Hg + col0 / G;
        uint16_t *zb = z + row0 * (size_t)Hg + col0 / G;
#pragma unroll
        for (int gi = 0; gi < kWaveSpan / G; ++gi) {
            // the group's values rounded to the dtype: packed pairs (yw) and
            // widened back to binary32 (yv) -- what the layer would store
            float yv[RG][4];
            uint32_t yw[RG][2];
#pragma unroll
            for (int jj = 0; jj < RG; ++jj) {
                const int j = gi * RG + jj;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    yw[jj][h] = pack2<DT>(acc[j / 4][tb][(j % 4) * 4 + 2 * h],
                                          acc[j / 4][tb][(j % 4) * 4 + 2 * h + 1]);
                    unpack2<DT>(yw[jj][h], yv[jj][2 * h], yv[jj][2 * h + 1]);
                }
            }
            float mn = yv[0][0], mx = yv[0][0];
#pragma unroll
            for (int jj = 0; jj < RG; ++jj) {
                mn = __builtin_fminf(mn, __builtin_fminf(__builtin_fminf(yv[jj][0], yv[jj][1]),
                                                         __builtin_fminf(yv[jj][2], yv[jj][3])));
                mx = __builtin_fmaxf(mx, __builtin_fmaxf(__builtin_fmaxf(yv[jj][0], yv[jj][1]),
                                                         __builtin_fmaxf(yv[jj][2], yv[jj][3])));
            }
            pair_minmax(mn, mx);
            const GroupParams p = group_params<BITS>(mn, mx);
            if (!live) continue;
#pragma unroll
            for (int jj = 0; jj < RG; ++jj) {
                const int j = gi * RG + jj;
                const uint32_t ch = (uint32_t)((j / 4) * 32 + (j % 4) * 8) + h4;
                const uint32_t q = encode4<BITS>(yv[jj], p);
                if constexpr (BITS == 8)
                    stv<uint32_t, false>(cb, lane_c + ch, q);
                else
                    stv<uint16_t, false>(cb, lane_c + ch / 2, (uint16_t)q);
                if (yb) stv<u32x2, false>(yb, lane_y + ch * 2u, u32x2{yw[jj][0], yw[jj][1]});
            }
            if (fhalf == 0) {
                stv<uint16_t, false>(sb, lane_m + 2u * gi, p.s16);
                stv<uint16_t, false>(zb, lane_m + 2u * gi, p.z16);
            }
        }
    }
}

template <int DT, int BITS, int G>
hipError_t launch_one(const uint16_t *a, const uint16_t *w, int R, int T, int K, int H,
                      uint8_t *codes, uint16_t *s, uint16_t *z, uint16_t *y, hipStream_t stream) {
    const int tiles_t = (T + kTileT - 1) / kTileT;
    const int tiles_n = H / kTileN;
    const long long total = (long long)R * tiles_t * tiles_n;
    if (total > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((linear_quantize_kernel<DT, BITS, G>), dim3((unsigned)total),
                       dim3(kBlockThreads), 0, stream, a, w, T, K, H, tiles_t, tiles_n, (int)total,
                       codes, s, z, y);
    return hipGetLastError();
}

template <int DT, int BITS>
hipError_t by_group(const uint16_t *a, const uint16_t *w, int R, int T, int K, int H, int group,
                    uint8_t *codes, uint16_t *s, uint16_t *z, uint16_t *y, hipStream_t stream) {
    switch (group) {
    case 8: return launch_one<DT, BITS, 8>(a, w, R, T, K, H, codes, s, z, y, stream);
    case 16: return launch_one<DT, BITS, 16>(a, w, R, T, K, H, codes, s, z, y, stream);
    case 32: return launch_one<DT, BITS, 32>(a, w, R, T, K, H, codes, s, z, y, stream);
    case 64: return launch_one<DT, BITS, 64>(a, w, R, T, K, H, codes, s, z, y, stream);
    case 128: return launch_one<DT, BITS, 128>(a, w, R, T, K, H, codes, s, z, y, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_linear_quantize(const uint16_t *a, const uint16_t *w, int dtype, int R, int T,
                                  int K, int H, int bits, int group, uint8_t *codes, uint16_t *s,
                                  uint16_t *z, uint16_t *y, hipStream_t stream) {
    if (dtype == 0)
        return bits == 4 ? by_group<0, 4>(a, w, R, T, K, H, group, codes, s, z, y, stream)
                         : by_group<0, 8>(a, w, R, T, K, H, group, codes, s, z, y, stream);
    return bits == 4 ? by_group<1, 4>(a, w, R, T, K, H, group, codes, s, z, y, stream)
                     : by_group<1, 8>(a, w, R, T, K, H, group, codes, s, z, y, stream);
}

}  // namespace fc
