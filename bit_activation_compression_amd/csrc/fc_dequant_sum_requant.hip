// Reduce-Scatter reduction and requantization before the All-Gather of
// "Flash Communication: Reducing Tensor Parallelization Bottleneck for Fast
// Large Language Model Inference" (Figure 5, right; the TL;DR's all-reduce
// in two steps).
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
// by HBM; its layout is chosen to keep the instructions per element low.
#include "fc_device.h"
#include "fc_launch.h"

namespace fc {
namespace {

// Work layout of this kernel: a lane owns a run of kRun = 32 consecutive
// positions (one 16-byte vector of 4-bit codes, or two of 8-bit codes, per
// operand), a wave slot is 64 runs = 2048 consecutive positions, and a wave
// tile is S slots (S > 1 only for stage-2 groups longer than a slot). With
// groups of 32 or more a lane holds one stage-1 group per operand and one
// stage-2 group, so the per-group work (metadata loads, scale and zero,
// reciprocal) is shared by 32 positions and at most log2(G2/32) cross-lane
// steps remain. A run is decoded and encoded as 4 sub-runs of 8 positions
// (dequant8, encode8).
constexpr int kRun = 32;
constexpr int kSubs = kRun / kLaneElems;      // 4 sub-runs of 8
constexpr int kWaveRun = kWave * kRun;        // 2048 positions per slot
// Workgroups of 8 waves: a wave's resources are then released with seven
// others' rather than three (measured on the 70B step: 165.4 µs against
// 166.4 with 4 waves, 165.8 with 2 and 166.4 with 1; same kernel and
// registers).
constexpr int kK2Threads = 512;
constexpr int kK2Waves = kK2Threads / kWave;

// Min and max of the sub-runs [k0, k0 + nk) of a run.
__device__ __forceinline__ void run_minmax(const float (&v)[kRun], int k0, int nk, float &mn,
                                           float &mx) {
    float a[kLaneElems];
#pragma unroll
    for (int i = 0; i < kLaneElems; ++i) a[i] = v[k0 * kLaneElems + i];
    minmax8(a, mn, mx);
#pragma unroll
    for (int k = 1; k < nk; ++k) {
        float b[kLaneElems], bn, bx;
#pragma unroll
        for (int i = 0; i < kLaneElems; ++i) b[i] = v[(k0 + k) * kLaneElems + i];
        minmax8(b, bn, bx);
        mn = __builtin_fminf(mn, bn);
        mx = __builtin_fmaxf(mx, bx);
    }
}

// RT > 0: the operand count is a compile-time constant (all loads of a tile
// are issued before the first use); RT == 0: any R, one operand at a time.
template <int BITS1, int BITS2, int G2, int RT>
__global__ __launch_bounds__(kK2Threads) void dsr_kernel(
    const uint8_t *__restrict__ codes1, const uint16_t *__restrict__ s1,
    const uint16_t *__restrict__ z1, int R_arg, uint64_t n, int g1_shift,
    uint8_t *__restrict__ codes2, uint16_t *__restrict__ s2, uint16_t *__restrict__ z2) {
    constexpr int S = G2 > kWaveRun ? G2 / kWaveRun : 1;     // slots per tile
    constexpr int GL = G2 < kRun ? kRun / G2 : 1;            // stage-2 groups per run
    constexpr int L = G2 <= kRun ? 1 : (G2 >= kWaveRun ? kWave : G2 / kRun);   // lanes per group
    constexpr int CW1 = BITS1, CW2 = BITS2;                  // 32-bit code words per run
    constexpr int SW1 = BITS1 / 4, SW2 = BITS2 / 4;          // code words per sub-run
    const int R = RT > 0 ? RT : R_arg;

    const int lane = lane_id();
    const uint64_t wave = (uint64_t)__builtin_amdgcn_workgroup_id_x() * kK2Waves +
                          __builtin_amdgcn_readfirstlane(__builtin_amdgcn_workitem_id_x() / kWave);
    const uint64_t tile = wave * (uint64_t)(S * kWaveRun);
    if (tile >= n) return;
    const uint64_t left = n - tile;
    const uint32_t avail = left < (uint64_t)(S * kWaveRun) ? (uint32_t)left : S * kWaveRun;

    // Run u of the lane covers positions [rel[u], rel[u] + 32) of the tile,
    // nv[u] of them valid. n is a multiple of 8 and of G2, so a run is whole
    // unless G2 < 32, and then it ends on a sub-run boundary. Runs wholly past
    // the end (last tile only) load the tile's first run instead and store
    // nothing; inside a partial run, sub-runs past the end load the run's
    // first sub-run. Every load is thus in bounds and unconditional, and a
    // tile's loads are in flight together.
    uint32_t rel[S], nv[S], lrel[S], lnv[S];
    const uint32_t first = avail < (uint32_t)kRun ? avail : (uint32_t)kRun;
#pragma unroll
    for (int u = 0; u < S; ++u) {
        rel[u] = u * kWaveRun + lane * kRun;
        const uint32_t rest = rel[u] < avail ? avail - rel[u] : 0u;
        nv[u] = rest < (uint32_t)kRun ? rest : (uint32_t)kRun;
        lrel[u] = nv[u] ? rel[u] : 0u;
        lnv[u] = nv[u] ? nv[u] : first;
    }

    // Stage-1 metadata index of position (r, tile + p):
    //   ((r*n + tile) >> s) + (((tile mod 2^s) + p) >> s),
    // since r*n is a multiple of the stage-1 group; the second term is the
    // same for every operand. The stage-1 group is at least G2 long, so a run
    // spans at most GL of them: entry j serves positions [j*32/GL, ..).
    const uint32_t mis = (uint32_t)tile & ((1u << g1_shift) - 1u);
    uint32_t mrel[S][GL];
#pragma unroll
    for (int u = 0; u < S; ++u)
#pragma unroll
        for (int j = 0; j < GL; ++j) {
            const uint32_t off = j * (kRun / GL) < lnv[u] ? j * (kRun / GL) : 0u;
            mrel[u][j] = (mis + lrel[u] + off) >> g1_shift;
        }

    auto load_operand = [&](int r, uint32_t (&w)[S][CW1], uint16_t (&sv)[S][GL],
                            uint16_t (&zv)[S][GL]) {
        const uint64_t e0 = (uint64_t)r * n + tile;
        const FC_GLOBAL uint8_t *cb = sgpr_ptr(codes1 + e0 * BITS1 / 8);
        const FC_GLOBAL uint16_t *sb = sgpr_ptr(s1 + (e0 >> g1_shift));
        const FC_GLOBAL uint16_t *zb = sgpr_ptr(z1 + (e0 >> g1_shift));
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const uint32_t byte0 = lrel[u] * BITS1 / 8;
            if (GL == 1 || lnv[u] == (uint32_t)kRun) {
#pragma unroll
                for (int q = 0; q < CW1 / 4; ++q) {
                    const u32x4 v = ldg<u32x4>(cb, byte0 + 16u * q);
                    w[u][4 * q + 0] = v.x;
                    w[u][4 * q + 1] = v.y;
                    w[u][4 * q + 2] = v.z;
                    w[u][4 * q + 3] = v.w;
                }
            } else {
#pragma unroll
                for (int k = 0; k < kSubs; ++k) {
                    const uint32_t sub = k * kLaneElems < lnv[u] ? k * kLaneElems : 0u;
                    const uint32_t off = (lrel[u] + sub) * BITS1 / 8;
                    if constexpr (BITS1 == 4) {
                        w[u][k] = ldg<uint32_t>(cb, off);
                    } else {
                        const u32x2 v = ldg<u32x2>(cb, off);
                        w[u][2 * k] = v.x;
                        w[u][2 * k + 1] = v.y;
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < GL; ++j) {
                sv[u][j] = ldg<uint16_t>(sb, 2u * mrel[u][j]);
                zv[u][j] = ldg<uint16_t>(zb, 2u * mrel[u][j]);
            }
        }
    };

    // x_hat = fp32(q*s + z), rounded once (dequant8), summed in ascending r
    float y[S][kRun];
    auto add_operand = [&](bool first_r, const uint32_t (&w)[S][CW1], const uint16_t (&sv)[S][GL],
                           const uint16_t (&zv)[S][GL]) {
#pragma unroll
        for (int u = 0; u < S; ++u)
#pragma unroll
            for (int k = 0; k < kSubs; ++k) {
                uint32_t t[SW1];
#pragma unroll
                for (int i = 0; i < SW1; ++i) t[i] = w[u][k * SW1 + i];
                float xh[kLaneElems];
                const int j = k * GL / kSubs;
                dequant8<BITS1>(t, sv[u][j], zv[u][j], xh);
#pragma unroll
                for (int i = 0; i < kLaneElems; ++i) {
                    float &acc = y[u][k * kLaneElems + i];
                    acc = first_r ? xh[i] : acc + xh[i];
                }
            }
    };

    if constexpr (RT > 0) {
        uint32_t w[RT][S][CW1];
        uint16_t sv[RT][S][GL], zv[RT][S][GL];
#pragma unroll
        for (int r = 0; r < RT; ++r) load_operand(r, w[r], sv[r], zv[r]);
#pragma unroll
        for (int r = 0; r < RT; ++r) add_operand(r == 0, w[r], sv[r], zv[r]);
    } else {
        uint32_t w[S][CW1];
        uint16_t sv[S][GL], zv[S][GL];
        load_operand(0, w, sv, zv);
        add_operand(true, w, sv, zv);
        for (int r = 1; r < R; ++r) {
            load_operand(r, w, sv, zv);
            add_operand(false, w, sv, zv);
        }
    }

    // ---- requantize the sums in groups of G2 ----
    FC_GLOBAL uint8_t *cb2 = sgpr_ptr(codes2 + tile * BITS2 / 8);
    FC_GLOBAL uint16_t *sb2 = sgpr_ptr(s2 + tile / G2);
    FC_GLOBAL uint16_t *zb2 = sgpr_ptr(z2 + tile / G2);
    if constexpr (GL > 1) {
        // several groups inside each run; a lane's groups are its own
#pragma unroll
        for (int u = 0; u < S; ++u) {
            uint32_t cw[CW2];
            uint16_t ps[GL], pz[GL];
#pragma unroll
            for (int j = 0; j < GL; ++j) {
                constexpr int KG = kSubs / GL;   // sub-runs per group
                float mn, mx;
                run_minmax(y[u], j * KG, KG, mn, mx);
                const GroupParams p = group_params<BITS2>(mn, mx);
                ps[j] = p.s16;
                pz[j] = p.z16;
#pragma unroll
                for (int k = j * KG; k < (j + 1) * KG; ++k) {
                    float v[kLaneElems];
#pragma unroll
                    for (int i = 0; i < kLaneElems; ++i) v[i] = y[u][k * kLaneElems + i];
                    uint32_t t[SW2];
                    encode8<BITS2>(v, p, t);
#pragma unroll
                    for (int i = 0; i < SW2; ++i) cw[k * SW2 + i] = t[i];
                }
            }
            if (nv[u] == (uint32_t)kRun) {
#pragma unroll
                for (int q = 0; q < CW2 / 4; ++q) {
                    const u32x4 v = {cw[4 * q], cw[4 * q + 1], cw[4 * q + 2], cw[4 * q + 3]};
                    stg<u32x4>(cb2, rel[u] * BITS2 / 8 + 16u * q, v);
                }
                if constexpr (GL == 4) {
                    const u32x2 sp = {ps[0] | ((uint32_t)ps[1] << 16), ps[2] | ((uint32_t)ps[3] << 16)};
                    const u32x2 zp = {pz[0] | ((uint32_t)pz[1] << 16), pz[2] | ((uint32_t)pz[3] << 16)};
                    stg<u32x2>(sb2, rel[u] / G2 * 2u, sp);
                    stg<u32x2>(zb2, rel[u] / G2 * 2u, zp);
                } else {
                    stg<uint32_t>(sb2, rel[u] / G2 * 2u, ps[0] | ((uint32_t)ps[1] << 16));
                    stg<uint32_t>(zb2, rel[u] / G2 * 2u, pz[0] | ((uint32_t)pz[1] << 16));
                }
            } else if (nv[u] > 0u) {
                // the run holding the end of the data: its valid groups only
#pragma unroll
                for (int j = 0; j < GL; ++j) {
                    if ((uint32_t)(j * G2) >= nv[u]) continue;
                    constexpr int KG = kSubs / GL;
#pragma unroll
                    for (int k = j * KG; k < (j + 1) * KG; ++k) {
                        const uint32_t off = (rel[u] + k * kLaneElems) * BITS2 / 8;
                        if constexpr (BITS2 == 4) {
                            stg<uint32_t>(cb2, off, cw[k]);
                        } else {
                            const u32x2 v = {cw[2 * k], cw[2 * k + 1]};
                            stg<u32x2>(cb2, off, v);
                        }
                    }
                    stg<uint16_t>(sb2, (rel[u] / G2 + j) * 2u, ps[j]);
                    stg<uint16_t>(zb2, (rel[u] / G2 + j) * 2u, pz[j]);
                }
            }
        }
    } else {
        // one group per run (G2 == 32), per L lanes, or per S slots
        float mn, mx;
        run_minmax(y[0], 0, kSubs, mn, mx);
#pragma unroll
        for (int u = 1; u < S; ++u) {
            float a, b;
            run_minmax(y[u], 0, kSubs, a, b);
            mn = __builtin_fminf(mn, a);
            mx = __builtin_fmaxf(mx, b);
        }
        lanes_minmax<L>(mn, mx);
        const GroupParams p = group_params<BITS2>(mn, mx);
#pragma unroll
        for (int u = 0; u < S; ++u) {
            if (nv[u] == 0u) continue;   // runs are whole here
            uint32_t cw[CW2];
#pragma unroll
            for (int k = 0; k < kSubs; ++k) {
                float v[kLaneElems];
#pragma unroll
                for (int i = 0; i < kLaneElems; ++i) v[i] = y[u][k * kLaneElems + i];
                uint32_t t[SW2];
                encode8<BITS2>(v, p, t);
#pragma unroll
                for (int i = 0; i < SW2; ++i) cw[k * SW2 + i] = t[i];
            }
#pragma unroll
            for (int q = 0; q < CW2 / 4; ++q) {
                const u32x4 v = {cw[4 * q], cw[4 * q + 1], cw[4 * q + 2], cw[4 * q + 3]};
                stg<u32x4>(cb2, rel[u] * BITS2 / 8 + 16u * q, v);
            }
        }
        const bool leader = S > 1 ? lane == 0 : (lane % L == 0 && nv[0] > 0u);
        if (leader) {
            stg<uint16_t>(sb2, rel[0] / G2 * 2u, p.s16);
            stg<uint16_t>(zb2, rel[0] / G2 * 2u, p.z16);
        }
    }
}

template <int BITS1, int BITS2, int G2, int RT>
hipError_t launch_one(const uint8_t *codes1, const uint16_t *s1, const uint16_t *z1, int R,
                      uint64_t n, int g1_shift, uint8_t *codes2, uint16_t *s2, uint16_t *z2,
                      hipStream_t stream) {
    constexpr uint64_t per_block =
        (uint64_t)kK2Waves * (G2 > kWaveRun ? G2 : kWaveRun);
    const uint64_t blocks = (n + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((dsr_kernel<BITS1, BITS2, G2, RT>), dim3((unsigned)blocks), dim3(kK2Threads),
                       0, stream, codes1, s1, z1, R, n, g1_shift, codes2, s2, z2);
    return hipGetLastError();
}

template <int BITS1, int BITS2, int G2>
hipError_t dispatch_r(const uint8_t *codes1, const uint16_t *s1, const uint16_t *z1, int R,
                      uint64_t n, int g1_shift, uint8_t *codes2, uint16_t *s2, uint16_t *z2,
                      hipStream_t stream) {
    // The compile-time operand count keeps all R runs of codes in flight; it
    // is used where a tile is one slot, so registers stay bounded.
#define FC_LAUNCH(RT) \
    launch_one<BITS1, BITS2, G2, RT>(codes1, s1, z1, R, n, g1_shift, codes2, s2, z2, stream)
    if constexpr (G2 <= kWaveRun) {
        if (R == 8) return FC_LAUNCH(8);
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
