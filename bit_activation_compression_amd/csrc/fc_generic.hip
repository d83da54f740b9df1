// The three codec kernels for any even group length: the groups the fast
// kernels do not take (lengths that are not a power of two in [8, 8192], such
// as 24, 96 or 6144). Same arithmetic as the fast kernels and the method of
// "Flash Communication: Reducing Tensor Parallelization Bottleneck for Fast
// Large Language Model Inference" (Figure 5, right; groups along the hidden
// dimension as in Figure 4), hence the same bits; the layout is simpler.
//
// Work layout: a group of G values is P lane units. When G is a multiple of
// 8 (for the reduction step: both group lengths), a unit is M 8-value
// vectors (16 bytes of 16-bit values each, the fast kernels' per-lane code
// paths), interleaved over the group's lanes: lane k of the P takes vectors
// k, k + P, ..., k + (M-1) P, so that each load instruction reads runs of
// 16 P contiguous bytes. With p the largest power of two dividing G/8 (at
// most 64), M = G/8p and P = p when that M is 3, 5, 6, 7, 10 or 12 and
// p >= 4 (groups of 96, 160, 192, 224, 1536, 5120, 6144 ...); otherwise
// M = 1 and P = G/8. Other groups take units of 2 consecutive values
// (P = G/2). G is even and groups start at multiples of G, so a unit never
// straddles two groups, and a 4-bit code pair is one byte. A lane handles
// units:
//   - P <= 64: each group takes an aligned segment of P2 lanes (P2 the next
//     power of two >= P), 64/P2 groups per wave; lanes k >= P of a segment
//     are idle. The group's min/max is reduced over its segment with xor
//     shuffles of distance 1 .. P2/2, which stay inside the segment.
//   - P > 64: one group per wave; lane k takes units k, k + 64, ...; the
//     min/max is reduced over the wave, and the values are read a second
//     time (from the caches) to encode them.
// Idle lanes contribute +inf / -inf to the reductions. Units of M > 1
// vectors always take the first form (P = p <= 64), so their kernels are
// compiled without the second, whose registers would otherwise set theirs
// (measured: K1 41 -> 35 us at g = 160; K2 59 -> 34 us at g = 6144).
#include "fc_device.h"
#include "fc_launch.h"

namespace fc {
namespace {

constexpr float kInf = __builtin_inff();

struct UnitMap {
    uint32_t P;          // lane units per group
    uint32_t p2_shift;   // log2 of the lanes per group segment (P <= 64)
    bool wide;           // P > 64: one group per wave
};

// min/max over the lanes of an aligned segment of 2^shift lanes
__device__ __forceinline__ void segment_minmax(float &mn, float &mx, uint32_t shift) {
    for (uint32_t d = 1; d < (1u << shift); d <<= 1) {
        mn = __builtin_fminf(mn, __shfl_xor(mn, (int)d));
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, (int)d));
    }
}

template <int DT>
__device__ __forceinline__ void widen2(uint32_t w, float &a, float &b) {
    if constexpr (DT == 1) {
        a = __builtin_bit_cast(float, w << 16);
        b = __builtin_bit_cast(float, w & 0xFFFF0000u);
    } else {
        const f16x2 h = __builtin_bit_cast(f16x2, w);
        a = (float)h.x;
        b = (float)h.y;
    }
}

template <int DT>
__device__ __forceinline__ uint32_t narrow2(float a, float b) {
    const f32x2 pair = {as_f32(a), as_f32(b)};
    if constexpr (DT == 1) return __builtin_bit_cast(uint32_t, __builtin_convertvector(pair, bf16x2));
    else return __builtin_bit_cast(uint32_t, __builtin_convertvector(pair, f16x2));
}

// Codes of a pair: q = clamp(round_half_even(fp32(fp32(v - z) * inv)), 0, Q)
// (v_cvt_pk_u8_f32 rounds to nearest even and saturates to [0, 255]), as
// one byte of two 4-bit codes (even value in the low nibble) or two bytes.
template <int BITS>
__device__ __forceinline__ uint32_t encode2(float a, float b, const GroupParams &p) {
    const float ta = (a - p.z) * p.inv;
    const float tb = (b - p.z) * p.inv;
    const uint32_t w = __builtin_amdgcn_cvt_pk_u8_f32(tb, 1, __builtin_amdgcn_cvt_pk_u8_f32(ta, 0, 0u));
    if constexpr (BITS == 4) {
        const uint32_t qa = __builtin_elementwise_min(w & 0xFFu, 15u);
        const uint32_t qb = __builtin_elementwise_min(w >> 8, 15u);
        return qa | (qb << 4);
    } else {
        return w;
    }
}

template <int BITS>
__device__ __forceinline__ void store_pair_codes(uint8_t *codes, uint64_t e, uint32_t c) {
    if constexpr (BITS == 4) codes[e / 2] = (uint8_t)c;
    else *reinterpret_cast<uint16_t *>(codes + e) = (uint16_t)c;
}

template <int BITS>
__device__ __forceinline__ void load_pair_codes(const uint8_t *codes, uint64_t e, float &qa, float &qb) {
    if constexpr (BITS == 4) {
        const uint32_t c = codes[e / 2];
        qa = (float)(c & 15u);
        qb = (float)(c >> 4);
    } else {
        const uint32_t c = *reinterpret_cast<const uint16_t *>(codes + e);
        qa = (float)(c & 0xFFu);
        qb = (float)(c >> 8);
    }
}

// Which group and unit this lane handles (P <= 64), or the group of the
// wave (P > 64). Returns false for a wave wholly past the last group.
struct Slot {
    uint64_t group;
    uint32_t k;        // unit index inside the group (the first one when wide)
    bool active;       // this lane's unit exists (narrow layout)
};

__device__ __forceinline__ bool lane_slot(const UnitMap &m, uint64_t groups, Slot &s) {
    const uint64_t wave = wave_index();
    const uint32_t lane = (uint32_t)lane_id();
    if (m.wide) {
        if (wave >= groups) return false;
        s.group = wave;
        s.k = lane;
        s.active = true;
        return true;
    }
    const uint32_t per_wave = kWave >> m.p2_shift;
    if (wave * per_wave >= groups) return false;
    s.group = wave * per_wave + (lane >> m.p2_shift);
    s.k = lane & ((1u << m.p2_shift) - 1u);
    s.active = s.group < groups && s.k < m.P;
    return true;
}

// Quotient n / d of 32-bit values by a multiply-high (the round-up method of
// T. Granlund and P. Montgomery, "Division by invariant integers using
// multiplication", 1994): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, t = mulhi(m, n) and
// q = (t + ((n - t) >> 1)) >> (l - 1), for every n < 2^32 and d >= 2.
// Positions past 2^32 - 1 (`wide`) divide in 64 bits instead.
struct GroupDiv {
    uint32_t d, m, l1;
    bool wide;
};

__device__ __forceinline__ uint64_t group_of(uint64_t e, const GroupDiv &D) {
    if (D.wide) return e / D.d;
    const uint32_t n = (uint32_t)e;
    const uint32_t t = __umulhi(D.m, n);
    return (t + ((n - t) >> 1)) >> D.l1;
}

// ---------------------------------------------------------------------------
// stage-1 quantizer: x [n] 16-bit -> codes, s, z in `groups` groups of G
// (units of 2 values)
// ---------------------------------------------------------------------------
// In the segment layout a wave of pair units covers only 64 / P2 groups (8
// groups of 10 values: 160 bytes), so the quantizer gives each wave
// kPairSets consecutive such sets, their loads in flight together (measured
// on 84 M values: 152 -> 120 us at g = 10, 189 -> 134 us at g = 6).
constexpr uint32_t kPairSets = 8;

template <int DT, int BITS>
__global__ __launch_bounds__(kBlockThreads) void quantize_generic_kernel(
    const uint16_t *__restrict__ x, uint64_t groups, uint32_t G, UnitMap m,
    uint8_t *__restrict__ codes, uint16_t *__restrict__ s_out, uint16_t *__restrict__ z_out) {
    const uint32_t *xw = reinterpret_cast<const uint32_t *>(x);
    if (!m.wide) {
        const uint64_t wave = wave_index();
        const uint32_t lane = (uint32_t)lane_id();
        const uint32_t per_set = kWave >> m.p2_shift;             // groups per set
        const uint64_t first = wave * (uint64_t)(per_set * kPairSets);
        if (first >= groups) return;
        const uint32_t k = lane & ((1u << m.p2_shift) - 1u);      // pair index in the group
        const uint64_t g0 = first + (lane >> m.p2_shift);
        uint32_t w[kPairSets];
#pragma unroll
        for (uint32_t it = 0; it < kPairSets; ++it) {
            const uint64_t g = g0 + (uint64_t)it * per_set;
            w[it] = g < groups && k < m.P ? xw[((g * G) >> 1) + k] : 0u;
        }
#pragma unroll
        for (uint32_t it = 0; it < kPairSets; ++it) {
            const uint64_t g = g0 + (uint64_t)it * per_set;
            const bool active = g < groups && k < m.P;
            float a = kInf, b = kInf, mn = kInf, mx = -kInf;
            if (active) {
                widen2<DT>(w[it], a, b);
                mn = __builtin_fminf(a, b);
                mx = __builtin_fmaxf(a, b);
            }
            segment_minmax(mn, mx, m.p2_shift);
            const GroupParams p = group_params<BITS>(mn, mx);
            if (active) {
                store_pair_codes<BITS>(codes, g * G + 2 * k, encode2<BITS>(a, b, p));
                if (k == 0) {
                    s_out[g] = p.s16;
                    z_out[g] = p.z16;
                }
            }
        }
        return;
    }
    Slot sl;
    if (!lane_slot(m, groups, sl)) return;
    const uint64_t base = sl.group * G;
    float mn = kInf, mx = -kInf;
    for (uint32_t k = sl.k; k < m.P; k += kWave) {
        float a, b;
        widen2<DT>(xw[(base >> 1) + k], a, b);
        mn = __builtin_fminf(mn, __builtin_fminf(a, b));
        mx = __builtin_fmaxf(mx, __builtin_fmaxf(a, b));
    }
    lanes_minmax<kWave>(mn, mx);
    const GroupParams p = group_params<BITS>(mn, mx);
    for (uint32_t k = sl.k; k < m.P; k += kWave) {
        float a, b;
        widen2<DT>(xw[(base >> 1) + k], a, b);
        store_pair_codes<BITS>(codes, base + 2 * k, encode2<BITS>(a, b, p));
    }
    if (sl.k == 0) {
        s_out[sl.group] = p.s16;
        z_out[sl.group] = p.z16;
    }
}

// Groups of at most kLaneGroupMax values that are not a multiple of 8: a
// lane owns a whole group. It reads the group's value pairs twice (min/max,
// then codes, the second time from the caches) and stores its scale and
// zero: no cross-lane steps, no idle lanes, one scale computation per group
// (measured on 84 M values: 120 -> 47 us at g = 10, 133 -> 110 us at g = 6;
// R = 8 x 11 M values at g = 12: 106 -> 58 us).
constexpr uint32_t kLaneGroupMax = 32;

template <int DT, int BITS>
__global__ __launch_bounds__(kBlockThreads) void quantize_lane_kernel(
    const uint16_t *__restrict__ x, uint64_t groups, uint32_t G, uint8_t *__restrict__ codes,
    uint16_t *__restrict__ s_out, uint16_t *__restrict__ z_out) {
    const uint64_t g = wave_index() * kWave + (uint32_t)lane_id();
    if (g >= groups) return;
    const uint32_t *xw = reinterpret_cast<const uint32_t *>(x) + ((g * G) >> 1);
    const uint32_t pairs = G / 2;
    float mn = kInf, mx = -kInf;
#pragma unroll 4
    for (uint32_t j = 0; j < pairs; ++j) {
        float a, b;
        widen2<DT>(xw[j], a, b);
        mn = __builtin_fminf(mn, __builtin_fminf(a, b));
        mx = __builtin_fmaxf(mx, __builtin_fmaxf(a, b));
    }
    const GroupParams p = group_params<BITS>(mn, mx);
#pragma unroll 4
    for (uint32_t j = 0; j < pairs; ++j) {
        float a, b;
        widen2<DT>(xw[j], a, b);
        store_pair_codes<BITS>(codes, g * G + 2 * j, encode2<BITS>(a, b, p));
    }
    s_out[g] = p.s16;
    z_out[g] = p.z16;
}

// ---------------------------------------------------------------------------
// Reduce-Scatter reduction + requantization: positions p of n = T*H, stage-1
// groups of G1 (per operand, operand stride n; `per_op` = n / G1 of them),
// stage-2 groups of G2 (`groups` = n / G2); D1 divides by G1
// ---------------------------------------------------------------------------

// binary32 sums of the pair of positions (e, e + 1) over the R operands, in
// ascending r starting from operand 0; each term fp32(q*s + z) (q*s exact)
template <int BITS1>
__device__ __forceinline__ void sum_pair(const uint8_t *codes1, const uint16_t *s1,
                                         const uint16_t *z1, int R, uint64_t n, uint64_t per_op,
                                         const GroupDiv &D1, uint64_t e, float &ya, float &yb) {
    const uint64_t g = group_of(e, D1);
    // operands in pairs: both operands' codes, scales and zeros are loaded
    // before the first of their terms is added; an odd last one goes alone
    int r = 0;
    for (; r + 2 <= R; r += 2) {
        float qa[2], qb[2];
        uint16_t sv[2], zv[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            load_pair_codes<BITS1>(codes1, (uint64_t)(r + i) * n + e, qa[i], qb[i]);
            const uint64_t mi = (uint64_t)(r + i) * per_op + g;
            sv[i] = s1[mi];
            zv[i] = z1[mi];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float s = half_bits_to_float(sv[i]);
            const float z = half_bits_to_float(zv[i]);
            const float xa = __builtin_fmaf(qa[i], s, z);
            const float xb = __builtin_fmaf(qb[i], s, z);
            ya = r + i == 0 ? xa : ya + xa;
            yb = r + i == 0 ? xb : yb + xb;
        }
    }
    for (; r < R; ++r) {
        float qa, qb;
        load_pair_codes<BITS1>(codes1, (uint64_t)r * n + e, qa, qb);
        const uint64_t mi = (uint64_t)r * per_op + g;
        const float s = half_bits_to_float(s1[mi]);
        const float z = half_bits_to_float(z1[mi]);
        const float xa = __builtin_fmaf(qa, s, z);
        const float xb = __builtin_fmaf(qb, s, z);
        ya = r == 0 ? xa : ya + xa;
        yb = r == 0 ? xb : yb + xb;
    }
}

template <int BITS1, int BITS2>
__global__ __launch_bounds__(kBlockThreads) void dsr_generic_kernel(
    const uint8_t *__restrict__ codes1, const uint16_t *__restrict__ s1,
    const uint16_t *__restrict__ z1, int R, uint64_t n, uint64_t per_op, GroupDiv D1,
    uint64_t groups, uint32_t G2, UnitMap m, uint8_t *__restrict__ codes2,
    uint16_t *__restrict__ s2, uint16_t *__restrict__ z2) {
    Slot sl;
    if (!lane_slot(m, groups, sl)) return;
    const uint64_t base = sl.group * G2;
    if (!m.wide) {
        float a = kInf, b = kInf, mn = kInf, mx = -kInf;
        if (sl.active) {
            sum_pair<BITS1>(codes1, s1, z1, R, n, per_op, D1, base + 2 * sl.k, a, b);
            mn = __builtin_fminf(a, b);
            mx = __builtin_fmaxf(a, b);
        }
        segment_minmax(mn, mx, m.p2_shift);
        const GroupParams p = group_params<BITS2>(mn, mx);
        if (!sl.active) return;
        store_pair_codes<BITS2>(codes2, base + 2 * sl.k, encode2<BITS2>(a, b, p));
        if (sl.k == 0) {
            s2[sl.group] = p.s16;
            z2[sl.group] = p.z16;
        }
        return;
    }
    float mn = kInf, mx = -kInf;
    for (uint32_t k = sl.k; k < m.P; k += kWave) {
        float a, b;
        sum_pair<BITS1>(codes1, s1, z1, R, n, per_op, D1, base + 2 * k, a, b);
        mn = __builtin_fminf(mn, __builtin_fminf(a, b));
        mx = __builtin_fmaxf(mx, __builtin_fmaxf(a, b));
    }
    lanes_minmax<kWave>(mn, mx);
    const GroupParams p = group_params<BITS2>(mn, mx);
    for (uint32_t k = sl.k; k < m.P; k += kWave) {
        float a, b;
        sum_pair<BITS1>(codes1, s1, z1, R, n, per_op, D1, base + 2 * k, a, b);
        store_pair_codes<BITS2>(codes2, base + 2 * k, encode2<BITS2>(a, b, p));
    }
    if (sl.k == 0) {
        s2[sl.group] = p.s16;
        z2[sl.group] = p.z16;
    }
}

// Equal group lengths of at most kLaneGroupMax that are not a multiple of 8:
// a lane owns a stage-2 group (which is also one stage-1 group of every
// operand). Its sums stay in registers (pair slots up to kLaneGroupMax / 2,
// guarded by the group's pair count), summed in ascending r as in sum_pair.
template <int BITS1, int BITS2>
__global__ __launch_bounds__(kBlockThreads) void dsr_lane_kernel(
    const uint8_t *__restrict__ codes1, const uint16_t *__restrict__ s1,
    const uint16_t *__restrict__ z1, int R, uint64_t n, uint64_t per_op, uint64_t groups,
    uint32_t G, uint8_t *__restrict__ codes2, uint16_t *__restrict__ s2,
    uint16_t *__restrict__ z2) {
    constexpr uint32_t kMaxPairs = kLaneGroupMax / 2;
    const uint64_t g = wave_index() * kWave + (uint32_t)lane_id();
    if (g >= groups) return;
    const uint32_t pairs = G / 2;
    const uint64_t e0 = g * G;
    float ya[kMaxPairs], yb[kMaxPairs];
    for (int r = 0; r < R; ++r) {
        const uint64_t mi = (uint64_t)r * per_op + g;
        const float s = half_bits_to_float(s1[mi]);
        const float z = half_bits_to_float(z1[mi]);
#pragma unroll
        for (uint32_t j = 0; j < kMaxPairs; ++j) {
            if (j < pairs) {
                float qa, qb;
                load_pair_codes<BITS1>(codes1, (uint64_t)r * n + e0 + 2 * j, qa, qb);
                const float xa = __builtin_fmaf(qa, s, z);
                const float xb = __builtin_fmaf(qb, s, z);
                ya[j] = r == 0 ? xa : ya[j] + xa;
                yb[j] = r == 0 ? xb : yb[j] + xb;
            }
        }
    }
    float mn = kInf, mx = -kInf;
#pragma unroll
    for (uint32_t j = 0; j < kMaxPairs; ++j) {
        if (j < pairs) {
            mn = __builtin_fminf(mn, __builtin_fminf(ya[j], yb[j]));
            mx = __builtin_fmaxf(mx, __builtin_fmaxf(ya[j], yb[j]));
        }
    }
    const GroupParams p = group_params<BITS2>(mn, mx);
#pragma unroll
    for (uint32_t j = 0; j < kMaxPairs; ++j)
        if (j < pairs) store_pair_codes<BITS2>(codes2, e0 + 2 * j, encode2<BITS2>(ya[j], yb[j], p));
    s2[g] = p.s16;
    z2[g] = p.z16;
}

// ---------------------------------------------------------------------------
// final dequantize (+ residual add) for stage-2 groups that are not a
// multiple of 8; D2 divides by G2
// ---------------------------------------------------------------------------
// Four pairs (8 positions) per lane: one code load and one 16-byte output
// store per lane (a lane past the last whole 8 goes pair by pair), each
// pair's scale and zero looked up on its own (measured at g = 10, 21 M
// positions: 14.2 us against 22.0 with one pair per lane).
constexpr uint32_t kDqPairs = 4;

template <int DT, int BITS, bool RES>
__global__ __launch_bounds__(kBlockThreads) void dequant_pairs_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ s,
    const uint16_t *__restrict__ z, uint64_t n, GroupDiv D2, const uint16_t *res, uint16_t *out) {
    const uint64_t e0 = (wave_index() * kWave + (uint64_t)lane_id()) * (2 * kDqPairs);
    if (e0 >= n) return;
    const bool whole = e0 + 2 * kDqPairs <= n;
    float qa[kDqPairs], qb[kDqPairs];
    if (whole) {
        if constexpr (BITS == 4) {
            const uint32_t c = *reinterpret_cast<const uint32_t *>(codes + e0 / 2);
#pragma unroll
            for (uint32_t i = 0; i < kDqPairs; ++i) {
                qa[i] = (float)((c >> (8 * i)) & 15u);
                qb[i] = (float)((c >> (8 * i + 4)) & 15u);
            }
        } else {
            const u32x2 c = *reinterpret_cast<const u32x2 *>(codes + e0);
#pragma unroll
            for (uint32_t i = 0; i < kDqPairs; ++i) {
                const uint32_t w = i < 2 ? c.x : c.y;
                qa[i] = (float)((w >> (16 * (i & 1))) & 0xFFu);
                qb[i] = (float)((w >> (16 * (i & 1) + 8)) & 0xFFu);
            }
        }
    } else {
#pragma unroll
        for (uint32_t i = 0; i < kDqPairs; ++i) {
            qa[i] = qb[i] = 0.0f;
            if (e0 + 2 * i < n) load_pair_codes<BITS>(codes, e0 + 2 * i, qa[i], qb[i]);
        }
    }
    uint32_t o[kDqPairs];
#pragma unroll
    for (uint32_t i = 0; i < kDqPairs; ++i) {
        const uint64_t e = e0 + 2 * i;
        const uint64_t g = group_of(e < n ? e : e0, D2);
        const float sf = half_bits_to_float(s[g]);
        const float zf = half_bits_to_float(z[g]);
        o[i] = narrow2<DT>(__builtin_fmaf(qa[i], sf, zf), __builtin_fmaf(qb[i], sf, zf));
    }
    if constexpr (RES) {
        uint32_t rw[kDqPairs];
        if (whole) {
            const u32x4 r4 = *reinterpret_cast<const u32x4 *>(res + e0);
            rw[0] = r4.x; rw[1] = r4.y; rw[2] = r4.z; rw[3] = r4.w;
        } else {
#pragma unroll
            for (uint32_t i = 0; i < kDqPairs; ++i)
                rw[i] = e0 + 2 * i < n ? reinterpret_cast<const uint32_t *>(res + e0)[i] : 0u;
        }
#pragma unroll
        for (uint32_t i = 0; i < kDqPairs; ++i) {
            float a, b, ra, rb;
            widen2<DT>(o[i], a, b);   // the all-reduce result as the dtype holds it
            widen2<DT>(rw[i], ra, rb);
            o[i] = narrow2<DT>(ra + a, rb + b);
        }
    }
    if (whole) {
        *reinterpret_cast<u32x4 *>(out + e0) = u32x4{o[0], o[1], o[2], o[3]};
    } else {
#pragma unroll
        for (uint32_t i = 0; i < kDqPairs; ++i)
            if (e0 + 2 * i < n) reinterpret_cast<uint32_t *>(out + e0)[i] = o[i];
    }
}


// ---------------------------------------------------------------------------
// groups whose length is a multiple of 8: a lane unit is M consecutive
// 8-value vectors (see the top of the file); a UnitMap whose P counts units
// ---------------------------------------------------------------------------

// NT: non-temporal loads, for groups of 64 or more lanes (each load
// instruction then reads whole lines); shorter segments read 64-byte pieces
// of lines whose other halves the next instruction reads, which the cached
// loads serve from L1
template <int DT, int BITS, int M, bool NT>
__global__ __launch_bounds__(kBlockThreads) void quantize_oct_kernel(
    const uint16_t *__restrict__ x, uint64_t groups, uint32_t G, UnitMap m,
    uint8_t *__restrict__ codes, uint16_t *__restrict__ s_out, uint16_t *__restrict__ z_out) {
    constexpr int W = BITS == 4 ? 1 : 2;
    Slot sl;
    if (!lane_slot(m, groups, sl)) return;
    const uint64_t base = sl.group * G;
    const uint16_t *xg = x + base;
    uint8_t *cg = codes + base * BITS / 8;
    // the values of unit k (vectors k, k + P, ... of the group), widened
    auto load_unit = [&](uint32_t k, float (&v)[M][kLaneElems]) {
#pragma unroll
        for (int j = 0; j < M; ++j) widen8<DT>(ldv<u32x4, NT>(xg, (k + j * m.P) * 16u), v[j]);
    };
    auto minmax_unit = [&](const float (&v)[M][kLaneElems], float &mn, float &mx) {
#pragma unroll
        for (int j = 0; j < M; ++j) {
            float a, b;
            minmax8(v[j], a, b);
            mn = __builtin_fminf(mn, a);
            mx = __builtin_fmaxf(mx, b);
        }
    };
    auto store_unit = [&](uint32_t k, const float (&v)[M][kLaneElems], const GroupParams &p) {
#pragma unroll
        for (int j = 0; j < M; ++j) {
            uint32_t w[W];
            encode8<BITS>(v[j], p, w);
            store_codes<BITS, true>(cg, (k + j * m.P) * kLaneElems, w);
        }
    };
    if (M > 1 || !m.wide) {   // units of several vectors: P <= 64, never wide
        float v[M][kLaneElems];
        float mn = kInf, mx = -kInf;
        if (sl.active) {
            load_unit(sl.k, v);
            minmax_unit(v, mn, mx);
        }
        segment_minmax(mn, mx, m.p2_shift);
        const GroupParams p = group_params<BITS>(mn, mx);
        if (!sl.active) return;
        store_unit(sl.k, v, p);
        if (sl.k == 0) {
            s_out[sl.group] = p.s16;
            z_out[sl.group] = p.z16;
        }
        return;
    }
    float mn = kInf, mx = -kInf;
    for (uint32_t k = sl.k; k < m.P; k += kWave) {
        float v[M][kLaneElems];
        load_unit(k, v);
        minmax_unit(v, mn, mx);
    }
    lanes_minmax<kWave>(mn, mx);
    const GroupParams p = group_params<BITS>(mn, mx);
    for (uint32_t k = sl.k; k < m.P; k += kWave) {
        float v[M][kLaneElems];
        load_unit(k, v);
        store_unit(k, v, p);
    }
    if (sl.k == 0) {
        s_out[sl.group] = p.s16;
        z_out[sl.group] = p.z16;
    }
}

// Operand r's term of the binary32 sums of the 8 positions [e, e + 8):
// y = x_0 for r = 0, else y + x_r, with x_r = fp32(q*s + z) (the product
// exact) for the stage-1 scale and zero (s16, z16) of the vector. Called in
// ascending r, this is the sum in the method's order.
template <int BITS1>
__device__ __forceinline__ void add_operand(const uint8_t *codes1, int r, uint64_t n, uint64_t e,
                                            uint16_t s16, uint16_t z16, float (&y)[kLaneElems]) {
    uint32_t w[BITS1 == 4 ? 1 : 2];
    load_codes<BITS1, false>(codes1 + ((uint64_t)r * n + e) * BITS1 / 8, 0, w);
    float xh[kLaneElems];
    dequant8<BITS1>(w, s16, z16, xh);
#pragma unroll
    for (int i = 0; i < kLaneElems; ++i) y[i] = r == 0 ? xh[i] : y[i] + xh[i];
}

// same_groups: G1 == G2 (the stage-1 group of every position of a stage-2
// group is then that group)
template <int BITS1, int BITS2, int M>
__global__ __launch_bounds__(kBlockThreads) void dsr_oct_kernel(
    const uint8_t *__restrict__ codes1, const uint16_t *__restrict__ s1,
    const uint16_t *__restrict__ z1, int R, uint64_t n, uint64_t per_op, GroupDiv D1,
    bool same_groups, uint64_t groups, uint32_t G2, UnitMap m, uint8_t *__restrict__ codes2,
    uint16_t *__restrict__ s2, uint16_t *__restrict__ z2) {
    constexpr int W = BITS2 == 4 ? 1 : 2;
    Slot sl;
    if (!lane_slot(m, groups, sl)) return;
    const uint64_t base = sl.group * G2;
    uint8_t *cg = codes2 + base * BITS2 / 8;
    // the sums of unit k, operand by operand (each stage-1 scale and zero
    // loaded once per operand when the groups coincide). With coinciding
    // groups the operands go in pairs (RB = 2 up to 12 code words per operand
    // and unit, else 1): a pair's codes, scales and zeros are all loaded
    // before its first term is added; an odd last operand goes alone.
    // Measured at R = 4 and 8: 10-20% faster than one operand at a time on
    // groups of 40 to 224, and as fast as batches of 4. Batching the other
    // case too would raise every instance's registers (its scales and zeros
    // are per vector)
    constexpr int W1 = BITS1 == 4 ? 1 : 2;
    constexpr int RB = M * W1 <= 12 ? 2 : 1;
    auto sum_unit = [&](uint32_t k, float (&y)[M][kLaneElems]) {
        auto pos = [&](int j) { return base + (uint64_t)(k + j * m.P) * kLaneElems; };
        if (same_groups) {
            int r = 0;
            for (; r + RB <= R; r += RB) {
                uint32_t w[RB][M][W1];
                uint16_t sv[RB], zv[RB];
#pragma unroll
                for (int b = 0; b < RB; ++b) {
                    const uint64_t mi = (uint64_t)(r + b) * per_op + sl.group;
                    sv[b] = s1[mi];
                    zv[b] = z1[mi];
#pragma unroll
                    for (int j = 0; j < M; ++j)
                        load_codes<BITS1, false>(codes1 + ((uint64_t)(r + b) * n + pos(j)) * BITS1 / 8,
                                                 0, w[b][j]);
                }
#pragma unroll
                for (int b = 0; b < RB; ++b)
#pragma unroll
                    for (int j = 0; j < M; ++j) {
                        float xh[kLaneElems];
                        dequant8<BITS1>(w[b][j], sv[b], zv[b], xh);
#pragma unroll
                        for (int i = 0; i < kLaneElems; ++i)
                            y[j][i] = r + b == 0 ? xh[i] : y[j][i] + xh[i];
                    }
            }
            for (; r < R; ++r) {
                const uint64_t mi = (uint64_t)r * per_op + sl.group;
                const uint16_t s16 = s1[mi], z16 = z1[mi];
#pragma unroll
                for (int j = 0; j < M; ++j) add_operand<BITS1>(codes1, r, n, pos(j), s16, z16, y[j]);
            }
        } else {
            uint64_t g1[M];
#pragma unroll
            for (int j = 0; j < M; ++j) g1[j] = group_of(pos(j), D1);
            for (int r = 0; r < R; ++r) {
#pragma unroll
                for (int j = 0; j < M; ++j) {
                    const uint64_t mi = (uint64_t)r * per_op + g1[j];
                    add_operand<BITS1>(codes1, r, n, pos(j), s1[mi], z1[mi], y[j]);
                }
            }
        }
    };
    auto minmax_unit = [&](const float (&y)[M][kLaneElems], float &mn, float &mx) {
#pragma unroll
        for (int j = 0; j < M; ++j) {
            float a, b;
            minmax8(y[j], a, b);
            mn = __builtin_fminf(mn, a);
            mx = __builtin_fmaxf(mx, b);
        }
    };
    auto store_unit = [&](uint32_t k, const float (&y)[M][kLaneElems], const GroupParams &p) {
#pragma unroll
        for (int j = 0; j < M; ++j) {
            uint32_t w[W];
            encode8<BITS2>(y[j], p, w);
            store_codes<BITS2, false>(cg, (k + j * m.P) * kLaneElems, w);
        }
    };
    if (M > 1 || !m.wide) {   // units of several vectors: P <= 64, never wide
        float y[M][kLaneElems];
        float mn = kInf, mx = -kInf;
        if (sl.active) {
            sum_unit(sl.k, y);
            minmax_unit(y, mn, mx);
        }
        segment_minmax(mn, mx, m.p2_shift);
        const GroupParams p = group_params<BITS2>(mn, mx);
        if (!sl.active) return;
        store_unit(sl.k, y, p);
        if (sl.k == 0) {
            s2[sl.group] = p.s16;
            z2[sl.group] = p.z16;
        }
        return;
    }
    float mn = kInf, mx = -kInf;
    for (uint32_t k = sl.k; k < m.P; k += kWave) {
        float y[M][kLaneElems];
        sum_unit(k, y);
        minmax_unit(y, mn, mx);
    }
    lanes_minmax<kWave>(mn, mx);
    const GroupParams p = group_params<BITS2>(mn, mx);
    for (uint32_t k = sl.k; k < m.P; k += kWave) {
        float y[M][kLaneElems];
        sum_unit(k, y);
        store_unit(k, y, p);
    }
    if (sl.k == 0) {
        s2[sl.group] = p.s16;
        z2[sl.group] = p.z16;
    }
}

// one 8-value vector of positions per lane
template <int DT, int BITS, bool RES>
__global__ __launch_bounds__(kBlockThreads) void dequant_oct_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ s,
    const uint16_t *__restrict__ z, uint64_t n, GroupDiv D2, const uint16_t *res, uint16_t *out) {
    const uint64_t e = (wave_index() * kWave + (uint64_t)lane_id()) * kLaneElems;
    if (e >= n) return;
    uint32_t w[BITS == 4 ? 1 : 2];
    load_codes<BITS, false>(codes + e * BITS / 8, 0, w);
    const uint64_t g = group_of(e, D2);
    float q[kLaneElems], o[kLaneElems];
    decode8<BITS>(w, q);
    const float sf = half_bits_to_float(s[g]);
    const float zf = half_bits_to_float(z[g]);
#pragma unroll
    for (int k = 0; k < kLaneElems; ++k) o[k] = __builtin_fmaf(q[k], sf, zf);   // exact product
    u32x4 packed = narrow8<DT>(o);
    if constexpr (RES) {
        float a[kLaneElems], r[kLaneElems];
        widen8<DT>(packed, a);   // the all-reduce result as the dtype holds it
        widen8<DT>(ldv<u32x4, true>(res + e, 0), r);
#pragma unroll
        for (int k = 0; k < kLaneElems; ++k) a[k] = r[k] + a[k];
        packed = narrow8<DT>(a);
    }
    stv<u32x4, true>(out + e, 0, packed);
}

// unit: the values a lane takes at a time
UnitMap unit_map(uint32_t G, uint32_t unit) {
    UnitMap m;
    m.P = G / unit;
    m.wide = m.P > (uint32_t)kWave;
    m.p2_shift = 0;
    while (!m.wide && (1u << m.p2_shift) < m.P) ++m.p2_shift;
    return m;
}

// vectors of 8 values per lane unit for a group of G (a multiple of 8)
// values (measured on groups of 96, 160 and 6144: the single pass with 12
// vectors per lane beats the two-pass loop over units of 1 or 3 vectors in
// both kernels)
int unit_vectors(uint32_t G) {
    const uint32_t o = G / kLaneElems;
    uint32_t p = 1;
    while (p < (uint32_t)kWave && o % (2 * p) == 0) p *= 2;
    const uint32_t M = o / p;
    const bool ok = p >= 4 && (M == 3 || M == 5 || M == 6 || M == 7 || M == 10 || M == 12);
    return ok ? (int)M : 1;
}

// divisor by d (>= 2) for positions below `n`
GroupDiv group_div(uint32_t d, uint64_t n) {
    GroupDiv D;
    D.d = d;
    D.wide = n > 0xFFFFFFFFull;
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    D.m = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
    D.l1 = l - 1;
    return D;
}

// workgroups for `groups` groups laid out by m
hipError_t grid_for(const UnitMap &m, uint64_t groups, unsigned *blocks, uint32_t sets = 1) {
    const uint64_t per_wave = m.wide ? 1 : (uint64_t)(kWave >> m.p2_shift) * sets;
    const uint64_t waves = (groups + per_wave - 1) / per_wave;
    const uint64_t b = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    if (b > 0x7FFFFFFFull || b == 0) return hipErrorInvalidConfiguration;
    *blocks = (unsigned)b;
    return hipSuccess;
}

template <int DT, int BITS, int M>
void go_quantize_oct(unsigned blocks, hipStream_t stream, const uint16_t *x, uint64_t groups,
                     uint32_t G, const UnitMap &m, uint8_t *codes, uint16_t *s, uint16_t *z) {
    if (m.wide || m.P == (uint32_t)kWave)
        hipLaunchKernelGGL((quantize_oct_kernel<DT, BITS, M, true>), dim3(blocks),
                           dim3(kBlockThreads), 0, stream, x, groups, G, m, codes, s, z);
    else
        hipLaunchKernelGGL((quantize_oct_kernel<DT, BITS, M, false>), dim3(blocks),
                           dim3(kBlockThreads), 0, stream, x, groups, G, m, codes, s, z);
}

// false for an M without kernels
template <int DT, int BITS>
bool go_quantize(int M, unsigned blocks, hipStream_t stream, const uint16_t *x, uint64_t groups,
                 uint32_t G, const UnitMap &m, uint8_t *codes, uint16_t *s, uint16_t *z) {
    switch (M) {
    case 0:
        hipLaunchKernelGGL((quantize_generic_kernel<DT, BITS>), dim3(blocks), dim3(kBlockThreads),
                           0, stream, x, groups, G, m, codes, s, z);
        return true;
#define FC_M(MV)                                                                   \
    case MV:                                                                       \
        go_quantize_oct<DT, BITS, MV>(blocks, stream, x, groups, G, m, codes, s, z); \
        return true
        FC_M(1);
        FC_M(3);
        FC_M(5);
        FC_M(6);
        FC_M(7);
        FC_M(10);
        FC_M(12);
#undef FC_M
    default: return false;
    }
}

template <int B1, int B2, int M>
void go_dsr_oct(unsigned blocks, hipStream_t stream, const uint8_t *codes1, const uint16_t *s1,
                const uint16_t *z1, int R, uint64_t n, uint64_t per_op, const GroupDiv &D1,
                bool same, uint64_t groups, uint32_t G2, const UnitMap &m, uint8_t *codes2,
                uint16_t *s2, uint16_t *z2) {
    hipLaunchKernelGGL((dsr_oct_kernel<B1, B2, M>), dim3(blocks), dim3(kBlockThreads), 0, stream,
                       codes1, s1, z1, R, n, per_op, D1, same, groups, G2, m, codes2, s2, z2);
}

// false for an M without kernels
template <int B1, int B2>
bool go_dsr(int M, unsigned blocks, hipStream_t stream, const uint8_t *codes1, const uint16_t *s1,
            const uint16_t *z1, int R, uint64_t n, uint64_t per_op, const GroupDiv &D1, bool same,
            uint64_t groups, uint32_t G2, const UnitMap &m, uint8_t *codes2, uint16_t *s2,
            uint16_t *z2) {
    switch (M) {
    case 0:
        hipLaunchKernelGGL((dsr_generic_kernel<B1, B2>), dim3(blocks), dim3(kBlockThreads), 0,
                           stream, codes1, s1, z1, R, n, per_op, D1, groups, G2, m, codes2, s2, z2);
        return true;
#define FC_M(MV)                                                                                \
    case MV:                                                                                    \
        go_dsr_oct<B1, B2, MV>(blocks, stream, codes1, s1, z1, R, n, per_op, D1, same, groups, G2, \
                               m, codes2, s2, z2);                                              \
        return true
        FC_M(1);
        FC_M(3);
        FC_M(5);
        FC_M(6);
        FC_M(7);
        FC_M(10);
        FC_M(12);
#undef FC_M
    default: return false;
    }
}

template <int DT, int B, bool RS>
void go_dequant(bool oct, dim3 grid, hipStream_t stream, const uint8_t *codes2,
                const uint16_t *s2, const uint16_t *z2, uint64_t n, const GroupDiv &D2,
                const uint16_t *residual, uint16_t *out) {
    if (oct)
        hipLaunchKernelGGL((dequant_oct_kernel<DT, B, RS>), grid, dim3(kBlockThreads), 0, stream,
                           codes2, s2, z2, n, D2, residual, out);
    else
        hipLaunchKernelGGL((dequant_pairs_kernel<DT, B, RS>), grid, dim3(kBlockThreads), 0,
                           stream, codes2, s2, z2, n, D2, residual, out);
}

}  // namespace

// M = 0 selects the 2-value units
hipError_t launch_quantize_generic(const uint16_t *x, int dtype, uint64_t n, int bits, int group,
                                   uint8_t *codes, uint16_t *s, uint16_t *z, hipStream_t stream) {
    const uint32_t G = (uint32_t)group;
    const int M = G % kLaneElems == 0 ? unit_vectors(G) : 0;
    const UnitMap m = unit_map(G, M ? M * kLaneElems : 2);
    const uint64_t groups = n / G;
    if (M == 0 && G <= kLaneGroupMax) {
        const uint64_t b = (groups + (uint64_t)kWave * kWavesPerBlock - 1) / ((uint64_t)kWave * kWavesPerBlock);
        if (b > 0x7FFFFFFFull || b == 0) return hipErrorInvalidConfiguration;
        const dim3 grid((unsigned)b);
        if (dtype == 0) {
            if (bits == 4)
                hipLaunchKernelGGL((quantize_lane_kernel<0, 4>), grid, dim3(kBlockThreads), 0, stream, x, groups, G, codes, s, z);
            else
                hipLaunchKernelGGL((quantize_lane_kernel<0, 8>), grid, dim3(kBlockThreads), 0, stream, x, groups, G, codes, s, z);
        } else {
            if (bits == 4)
                hipLaunchKernelGGL((quantize_lane_kernel<1, 4>), grid, dim3(kBlockThreads), 0, stream, x, groups, G, codes, s, z);
            else
                hipLaunchKernelGGL((quantize_lane_kernel<1, 8>), grid, dim3(kBlockThreads), 0, stream, x, groups, G, codes, s, z);
        }
        return hipGetLastError();
    }
    unsigned blocks = 0;
    hipError_t e = grid_for(m, groups, &blocks, M == 0 ? kPairSets : 1);
    if (e != hipSuccess) return e;
    const bool ok = dtype == 0
                        ? (bits == 4 ? go_quantize<0, 4>(M, blocks, stream, x, groups, G, m, codes, s, z)
                                     : go_quantize<0, 8>(M, blocks, stream, x, groups, G, m, codes, s, z))
                        : (bits == 4 ? go_quantize<1, 4>(M, blocks, stream, x, groups, G, m, codes, s, z)
                                     : go_quantize<1, 8>(M, blocks, stream, x, groups, G, m, codes, s, z));
    return ok ? hipGetLastError() : hipErrorInvalidValue;
}

hipError_t launch_dsr_generic(const uint8_t *codes1, const uint16_t *s1, const uint16_t *z1, int R,
                              uint64_t n, int bits1, int bits2, int group1, int group2,
                              uint8_t *codes2, uint16_t *s2, uint16_t *z2, hipStream_t stream) {
    const uint32_t G1 = (uint32_t)group1, G2 = (uint32_t)group2;
    const bool same = G1 == G2;
    const int M = G1 % kLaneElems || G2 % kLaneElems ? 0 : unit_vectors(G2);
    const UnitMap m = unit_map(G2, M ? M * kLaneElems : 2);
    const uint64_t groups = n / G2;
    const uint64_t per_op = n / G1;
    const GroupDiv D1 = group_div(G1, n);
    if (M == 0 && same && G2 <= kLaneGroupMax) {
        const uint64_t b = (groups + (uint64_t)kWave * kWavesPerBlock - 1) / ((uint64_t)kWave * kWavesPerBlock);
        if (b > 0x7FFFFFFFull || b == 0) return hipErrorInvalidConfiguration;
#define FC_LANE(B1, B2)                                                                                \
    hipLaunchKernelGGL((dsr_lane_kernel<B1, B2>), dim3((unsigned)b), dim3(kBlockThreads), 0, stream, \
                       codes1, s1, z1, R, n, per_op, groups, G2, codes2, s2, z2)
        if (bits1 == 4) {
            if (bits2 == 4) FC_LANE(4, 4);
            else FC_LANE(4, 8);
        } else {
            if (bits2 == 4) FC_LANE(8, 4);
            else FC_LANE(8, 8);
        }
#undef FC_LANE
        return hipGetLastError();
    }
    unsigned blocks = 0;
    hipError_t e = grid_for(m, groups, &blocks);
    if (e != hipSuccess) return e;
#define FC_GO(B1, B2)                                                                             \
    go_dsr<B1, B2>(M, blocks, stream, codes1, s1, z1, R, n, per_op, D1, same, groups, G2, m, codes2, \
                   s2, z2)
    const bool ok = bits1 == 4 ? (bits2 == 4 ? FC_GO(4, 4) : FC_GO(4, 8))
                               : (bits2 == 4 ? FC_GO(8, 4) : FC_GO(8, 8));
#undef FC_GO
    return ok ? hipGetLastError() : hipErrorInvalidValue;
}

hipError_t launch_dequantize_generic(const uint8_t *codes2, const uint16_t *s2, const uint16_t *z2,
                                     uint64_t n, int bits, int group2, int dtype,
                                     const uint16_t *residual, uint16_t *out, hipStream_t stream) {
    const bool oct = group2 % kLaneElems == 0;
    const uint64_t lanes = oct ? n / kLaneElems : (n + 2 * kDqPairs - 1) / (2 * kDqPairs);
    const uint64_t b = (lanes + kBlockThreads - 1) / kBlockThreads;
    if (b > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)b);
    const GroupDiv D2 = group_div((uint32_t)group2, n);
#define FC_GO(DT, B, RS) go_dequant<DT, B, RS>(oct, grid, stream, codes2, s2, z2, n, D2, residual, out)
    const bool res = residual != nullptr;
    if (dtype == 0) {
        if (bits == 4) { if (res) FC_GO(0, 4, true); else FC_GO(0, 4, false); }
        else { if (res) FC_GO(0, 8, true); else FC_GO(0, 8, false); }
    } else {
        if (bits == 4) { if (res) FC_GO(1, 4, true); else FC_GO(1, 4, false); }
        else { if (res) FC_GO(1, 8, true); else FC_GO(1, 8, false); }
    }
#undef FC_GO
    return hipGetLastError();
}

}  // namespace fc
