// Device helpers shared by the codec kernels (gfx950, wave64).
//
// Work layout of the quantize, dequantize and single-launch kernels (the
// dequant-sum-requant kernel uses runs of 32 elements per lane instead): a
// wave owns a tile of U "slots"; a slot is 64 lanes x 8 consecutive elements
// = 512 consecutive elements, so every lane reads one 16-byte vector of
// 16-bit values (or the matching 4- or 8-byte run of codes) per slot and a
// wave touches 1 KiB of contiguous activations per slot. A quantization group
// of G elements (a power of two, 8 <= G <= 8192) covers G/8 consecutive lanes
// of one slot when G <= 512, or G/512 consecutive slots of one wave when
// G > 512; group minima and maxima are reduced first inside the lane, then
// across lanes with DPP row operations (<= 16 lanes), ds_swizzle (32 lanes)
// and readlane (64 lanes).
//
// Addresses are a wave-uniform base (SGPRs) plus a 32-bit per-lane offset,
// so no lane does 64-bit address arithmetic.
//
// Arithmetic follows the quantizer of "Flash Communication: Reducing Tensor
// Parallelization Bottleneck for Fast Large Language Model Inference"
// (Figures 4 and 5) in the asymmetric min/max reading: every binary32
// operation rounded on its own (built with -ffp-contract=off), fp16 scale and
// zero, codes rounded half to even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fc {

constexpr int kWave = 64;
constexpr int kLaneElems = 8;
constexpr int kSlotElems = kWave * kLaneElems;   // 512
constexpr int kBlockThreads = 256;
constexpr int kWavesPerBlock = kBlockThreads / kWave;

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v >> 1); }

// Slots a wave processes per tile for group length G: at least `base` and a
// whole number of groups.
constexpr int tile_slots(int G, int base) { return G > base * kSlotElems ? G / kSlotElems : base; }

// Lane and wave indices from the hardware registers. The wave index is made
// wave-uniform (SGPR) with readfirstlane: workitem_id / 64 is the same for
// every lane of a wave, but the compiler cannot know it, and every base
// address derived from a per-lane value would be computed in 64-bit VGPR
// arithmetic. (The builtins also avoid the device-library calls behind
// threadIdx/blockIdx, which are not inlined into code built with the IEEE
// mode bit off.)
__device__ __forceinline__ int lane_id() { return (int)(__builtin_amdgcn_workitem_id_x() & (kWave - 1)); }

__device__ __forceinline__ uint64_t wave_index() {
    const uint32_t w = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_workitem_id_x() / kWave);
    return (uint64_t)__builtin_amdgcn_workgroup_id_x() * kWavesPerBlock + w;
}

// Hides a value from the optimizer (no instruction is emitted).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}

// A fresh copy of v that the compiler cannot hoist out of a loop (volatile
// asm, no instruction emitted): values derived from it are recomputed where
// they are used instead of being kept live across the whole loop.
__device__ __forceinline__ uint32_t fresh(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// A wave-uniform global-memory base pinned in scalar registers, and loads
// and stores at that base plus a 32-bit per-lane byte offset. Without the
// pin the compiler may reassociate (uniform base + per-lane offset) +
// uniform offset into 64-bit per-lane address arithmetic; pinned, every
// access takes the scalar-base + 32-bit lane offset form.
#define FC_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ FC_GLOBAL T *sgpr_ptr(T *p) {
    asm("" : "+s"(p));
    return (FC_GLOBAL T *)p;
}

template <typename V>
__device__ __forceinline__ V ldg(const FC_GLOBAL void *base, uint32_t byte_off) {
    return *(const FC_GLOBAL V *)((const FC_GLOBAL uint8_t *)base + byte_off);
}

template <typename V>
__device__ __forceinline__ void stg(FC_GLOBAL void *base, uint32_t byte_off, V v) {
    *(FC_GLOBAL V *)((FC_GLOBAL uint8_t *)base + byte_off) = v;
}

// Pins v as a rounded binary32 register value. Without it the compiler may
// fuse the fma that produced v with a following fp32 -> fp16 conversion into
// one mixed-precision instruction (v_fma_mixlo_f16) that rounds once, straight
// to fp16, where the method rounds to binary32 first and then to fp16.
__device__ __forceinline__ float as_f32(float v) {
    asm("" : "+v"(v));
    return v;
}

// ---------------------------------------------------------------------------
// memory access at a wave-uniform base plus a 32-bit per-lane byte offset;
// NT marks streamed data non-temporal
// ---------------------------------------------------------------------------

template <typename V, bool NT>
__device__ __forceinline__ V ldv(const void *base, uint32_t byte_off) {
    const V *p = reinterpret_cast<const V *>(static_cast<const uint8_t *>(base) + byte_off);
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <typename V, bool NT>
__device__ __forceinline__ void stv(void *base, uint32_t byte_off, V v) {
    V *p = reinterpret_cast<V *>(static_cast<uint8_t *>(base) + byte_off);
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// The lane's 8 codes at element offset `rel` from a wave-uniform base.
template <int BITS, bool NT>
__device__ __forceinline__ void load_codes(const uint8_t *base, uint32_t rel,
                                           uint32_t (&w)[BITS == 4 ? 1 : 2]) {
    if constexpr (BITS == 8) {
        const u32x2 v = ldv<u32x2, NT>(base, rel);
        w[0] = v.x;
        w[1] = v.y;
    } else {
        w[0] = ldv<uint32_t, NT>(base, rel / 2);
    }
}

template <int BITS, bool NT>
__device__ __forceinline__ void store_codes(uint8_t *base, uint32_t rel,
                                            const uint32_t (&w)[BITS == 4 ? 1 : 2]) {
    if constexpr (BITS == 8) {
        const u32x2 v = {w[0], w[1]};
        stv<u32x2, NT>(base, rel, v);
    } else {
        stv<uint32_t, NT>(base, rel / 2, w[0]);
    }
}

// ---------------------------------------------------------------------------
// cross-lane min/max
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Reduce (min, max) over aligned groups of L consecutive lanes; every lane of
// a group ends up holding the group's result.
template <int L>
__device__ __forceinline__ void lanes_minmax(float &mn, float &mx) {
    static_assert(L >= 1 && L <= kWave && (L & (L - 1)) == 0, "L must be a power of two <= 64");
    if constexpr (L >= 2) {   // quad_perm [1,0,3,2]: partner lane ^ 1
        mn = __builtin_fminf(mn, dpp<0xB1>(mn));
        mx = __builtin_fmaxf(mx, dpp<0xB1>(mx));
    }
    if constexpr (L >= 4) {   // quad_perm [2,3,0,1]: partner lane ^ 2
        mn = __builtin_fminf(mn, dpp<0x4E>(mn));
        mx = __builtin_fmaxf(mx, dpp<0x4E>(mx));
    }
    if constexpr (L >= 8) {   // row_half_mirror: lane i <-> 7 - i inside each 8 lanes
        mn = __builtin_fminf(mn, dpp<0x141>(mn));
        mx = __builtin_fmaxf(mx, dpp<0x141>(mx));
    }
    if constexpr (L >= 16) {  // row_mirror: lane i <-> 15 - i inside each row of 16
        mn = __builtin_fminf(mn, dpp<0x140>(mn));
        mx = __builtin_fmaxf(mx, dpp<0x140>(mx));
    }
    if constexpr (L >= 32) {  // ds_swizzle bitmask mode, xor 16 within 32 lanes
        mn = __builtin_fminf(mn, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(
                                              __builtin_bit_cast(int, mn), 0x401F)));
        mx = __builtin_fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(
                                              __builtin_bit_cast(int, mx), 0x401F)));
    }
    if constexpr (L >= 64) {  // the two halves meet through lanes 0 and 32
        const int a = __builtin_amdgcn_readlane(__builtin_bit_cast(int, mn), 0);
        const int b = __builtin_amdgcn_readlane(__builtin_bit_cast(int, mn), 32);
        mn = __builtin_fminf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
        const int c = __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), 0);
        const int d = __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), 32);
        mx = __builtin_fmaxf(__builtin_bit_cast(float, c), __builtin_bit_cast(float, d));
    }
}

// In-lane min and max of 8 values (chains of three-input v_min3/v_max3).
__device__ __forceinline__ void minmax8(const float (&v)[kLaneElems], float &mn, float &mx) {
    mn = __builtin_fminf(__builtin_fminf(__builtin_fminf(__builtin_fminf(v[0], v[1]), v[2]),
                                         __builtin_fminf(v[3], v[4])),
                         __builtin_fminf(__builtin_fminf(v[5], v[6]), v[7]));
    mx = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), v[2]),
                                         __builtin_fmaxf(v[3], v[4])),
                         __builtin_fmaxf(__builtin_fmaxf(v[5], v[6]), v[7]));
}

// ---------------------------------------------------------------------------
// group scale / zero and per-element codes
// ---------------------------------------------------------------------------

struct GroupParams {
    float z;      // fp16 zero point, widened
    float inv;    // fp32(1 / s), 0 when s == 0
    uint16_t s16; // fp16 bit patterns as stored
    uint16_t z16;
};

template <int BITS>
__device__ __forceinline__ GroupParams group_params(float mn, float mx) {
    constexpr float Q = float((1 << BITS) - 1);
    constexpr float RQ = 1.0f / Q;   // binary32 nearest to 1/Q
    mn = mn + 0.0f;                  // a zero minimum or maximum is taken as +0
    mx = mx + 0.0f;
    const float range = mx - mn;
    // fp32(range / Q) without a division: q0 = range * RQ is within an ulp of
    // the quotient, so the remainder range - q0*Q is exact in one fma, and one
    // correction step q0 + rem*RQ rounds to the correctly rounded quotient.
    // Checked exhaustively against IEEE division over every non-negative
    // finite binary32 range, for Q = 15 and Q = 255 (denormals preserved).
    const float q0 = range * RQ;
    const float rem = __builtin_fmaf(-q0, Q, range);
    const float s32 = __builtin_fmaf(rem, RQ, q0);
    const _Float16 sh = (_Float16)as_f32(s32);   // round to nearest even, gradual underflow
    const _Float16 zh = (_Float16)as_f32(mn);
    const float s = (float)sh;
    // fp32(1 / s) for an fp16 scale: v_rcp_f32 is within 1 ulp, one Newton
    // step in fma form leaves a relative error below 2^-44, and 1/s for an
    // 11-bit significand is never closer than 2^-12 ulp to a rounding
    // midpoint, so the final fma rounds exactly as IEEE division would
    // (also checked on the GPU for every positive fp16 scale).
    const float r0 = __builtin_amdgcn_rcpf(s);
    const float e = __builtin_fmaf(-s, r0, 1.0f);
    GroupParams p;
    p.z = (float)zh;
    p.inv = (s == 0.0f) ? 0.0f : __builtin_fmaf(e, r0, r0);
    p.s16 = __builtin_bit_cast(uint16_t, sh);
    p.z16 = __builtin_bit_cast(uint16_t, zh);
    return p;
}

// Codes of the lane's 8 values: q = clamp(round_half_even(fp32(fp32(v - z) *
// inv)), 0, Q). v_cvt_pk_u8_f32 rounds to nearest even and saturates to
// [0, 255] while inserting the byte (checked on the GPU), so 8-bit codes need
// no separate clamp. 4-bit codes are converted the same way into bytes 0 and
// 2 of four words (elements k and 4 + k in word k), clamped to 15 two at a
// time (v_pk_min_u16; clamping the rounded value equals rounding the clamped
// one, the bounds being integers) and then interleaved as nibbles.
// Layout: 4-bit codes in one word, element 2i in the low nibble of byte i;
// 8-bit codes in two words, element i in byte i.
template <int BITS>
__device__ __forceinline__ void encode8(const float (&v)[kLaneElems], const GroupParams &p,
                                        uint32_t (&w)[BITS == 4 ? 1 : 2]) {
    float t[kLaneElems];
#pragma unroll
    for (int i = 0; i < kLaneElems; ++i) t[i] = (v[i] - p.z) * p.inv;
    if constexpr (BITS == 8) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            uint32_t a = __builtin_amdgcn_cvt_pk_u8_f32(t[4 * k + 0], 0, 0u);
            a = __builtin_amdgcn_cvt_pk_u8_f32(t[4 * k + 1], 1, a);
            a = __builtin_amdgcn_cvt_pk_u8_f32(t[4 * k + 2], 2, a);
            w[k] = __builtin_amdgcn_cvt_pk_u8_f32(t[4 * k + 3], 3, a);
        }
    } else {
        uint32_t c[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t b = __builtin_amdgcn_cvt_pk_u8_f32(t[4 + k], 2,
                                                              __builtin_amdgcn_cvt_pk_u8_f32(t[k], 0, 0u));
            const u16x2 m = __builtin_elementwise_min(__builtin_bit_cast(u16x2, b), u16x2{15, 15});
            c[k] = __builtin_bit_cast(uint32_t, m);
        }
        // three v_lshl_or_b32 (opaque keeps the compiler from reassociating)
        const uint32_t h = opaque((opaque((c[3] << 4) | c[2]) << 4) | c[1]);
        w[0] = (h << 4) | c[0];
    }
}

// Unpack 8 codes to binary32 integers (v_cvt_f32_ubyte0..3).
template <int BITS>
__device__ __forceinline__ void decode8(const uint32_t (&w)[BITS == 4 ? 1 : 2], float (&q)[kLaneElems]) {
    if constexpr (BITS == 8) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const uint32_t b = w[k];
            q[4 * k + 0] = (float)(b & 0xFFu);
            q[4 * k + 1] = (float)((b >> 8) & 0xFFu);
            q[4 * k + 2] = (float)((b >> 16) & 0xFFu);
            q[4 * k + 3] = (float)(b >> 24);
        }
    } else {
        const uint32_t lo = opaque(w[0] & 0x0F0F0F0Fu);          // elements 0, 2, 4, 6
        const uint32_t hi = opaque((w[0] >> 4) & 0x0F0F0F0Fu);   // elements 1, 3, 5, 7
        q[0] = (float)(lo & 0xFFu);
        q[2] = (float)((lo >> 8) & 0xFFu);
        q[4] = (float)((lo >> 16) & 0xFFu);
        q[6] = (float)(lo >> 24);
        q[1] = (float)(hi & 0xFFu);
        q[3] = (float)((hi >> 8) & 0xFFu);
        q[5] = (float)((hi >> 16) & 0xFFu);
        q[7] = (float)(hi >> 24);
    }
}

// Dequantized values x_k = fp32(q_k * s + z) of 8 codes, for a scale s and
// zero z given as fp16 bit patterns. Each code is isolated inside a 16-bit
// half of a register, at bits 0..7 or, for the high nibble of a 4-bit pair,
// at bits 4..7; read as fp16, such a half is the subnormal q * 2^-24 or
// q * 2^-20, exactly. One mixed-precision fma per value (v_fma_mix_f32: the
// fp16 half selected in place, the binary32 scale s * 2^24 or s * 2^20, the
// fp16 zero) then forms q * s + z with the exact product (at most 8 x 11
// significant bits) and one rounding, exactly as fp32(q*s + z). Unpacking
// takes 5 bit operations per 8 four-bit codes and 4 per 8 eight-bit codes.
// This needs fp16 subnormals preserved on input (they are: the build keeps
// the default denormal mode, checked by the instruction guard test).
template <int BITS>
__device__ __forceinline__ void dequant8(const uint32_t (&w)[BITS == 4 ? 1 : 2], uint16_t s16,
                                         uint16_t z16, float (&x)[kLaneElems]) {
    const float s = (float)__builtin_bit_cast(_Float16, s16);
    const float sc24 = s * 16777216.0f;   // s * 2^24, exact
    const float z = (float)__builtin_bit_cast(_Float16, z16);
    // the two values whose codes sit in the halves of p
    auto pair = [&](uint32_t p, float sc, int e_lo, int e_hi) {
        const f16x2 h = __builtin_bit_cast(f16x2, p);
        x[e_lo] = __builtin_fmaf((float)h.x, sc, z);
        x[e_hi] = __builtin_fmaf((float)h.y, sc, z);
    };
    if constexpr (BITS == 4) {
        // byte i = q(2i) | q(2i+1) << 4: the low half holds elements 0..3,
        // the high half 4..7, as nibbles at bits 0, 4, 8, 12
        const float sc20 = s * 1048576.0f;   // s * 2^20, exact
        const uint32_t w8 = w[0] >> 8;
        pair(w[0] & 0x000F000Fu, sc24, 0, 4);
        pair(w[0] & 0x00F000F0u, sc20, 1, 5);
        pair(w8 & 0x000F000Fu, sc24, 2, 6);
        pair(w8 & 0x00F000F0u, sc20, 3, 7);
    } else {
        // word j holds elements 4j..4j+3, one per byte; v_perm_b32 moves
        // bytes 1 and 3 to bytes 0 and 2 and zeroes the others
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            pair(w[j] & 0x00FF00FFu, sc24, 4 * j, 4 * j + 2);
            pair(__builtin_amdgcn_perm(w[j], w[j], 0x0C030C01u), sc24, 4 * j + 1, 4 * j + 3);
        }
    }
}

// Quantize a tile of U slots: v holds the lane's 8 values per slot, mn/mx
// their in-lane minima and maxima. Each group's min/max is reduced over its
// S slots and L lanes, its scale/zero/reciprocal computed, and the codes
// written to cb (NT: non-temporal) and the fp16 scale and zero of every group
// to sb and zb (bases of the tile's first group). Slots at or past `avail`
// elements are not stored.
//
// With two slots per tile and groups of one slot spanning at least two
// lanes, every lane holds values of two groups, and the lanes of a group come
// in (even, odd) pairs: the even lane computes the scale, zero and reciprocal
// of its slot-0 group, the odd lane those of its slot-1 group, and each lane
// takes the other one from its partner (DPP quad_perm [0,0,2,2] and
// [1,1,3,3]), instead of computing both. The results are the same values.
template <int BITS, int G, int U, bool NT>
__device__ __forceinline__ void quantize_tile(const float (&v)[U][kLaneElems], const float (&mn)[U],
                                              const float (&mx)[U], int lane, uint32_t avail,
                                              uint8_t *cb, uint16_t *sb, uint16_t *zb) {
    constexpr int S = G > kSlotElems ? G / kSlotElems : 1;        // slots per group
    constexpr int L = G >= kSlotElems ? kWave : G / kLaneElems;   // lanes per group in a slot
    constexpr int W = BITS == 4 ? 1 : 2;
    static_assert(U % S == 0 && (U * kSlotElems) % G == 0, "a tile holds whole groups");
    if constexpr (U == 2 && S == 1 && L >= 2) {
        float a0 = mn[0], b0 = mx[0], a1 = mn[1], b1 = mx[1];
        lanes_minmax<L>(a0, b0);
        lanes_minmax<L>(a1, b1);
        const bool odd = (lane & 1) != 0;
        const GroupParams own = group_params<BITS>(odd ? a1 : a0, odd ? b1 : b0);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            GroupParams p = own;
            p.z = u == 0 ? dpp<0xA0>(own.z) : dpp<0xF5>(own.z);
            p.inv = u == 0 ? dpp<0xA0>(own.inv) : dpp<0xF5>(own.inv);
            const uint32_t rel = u * kSlotElems + lane * kLaneElems;
            if (rel >= avail) continue;
            uint32_t w[W];
            encode8<BITS>(v[u], p, w);
            store_codes<BITS, NT>(cb, rel, w);
            if (lane % L == u) {   // lane & 1 == u: `own` is this slot's group
                sb[rel / G] = own.s16;
                zb[rel / G] = own.z16;
            }
        }
        return;
    }
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
            const uint32_t rel = u * kSlotElems + lane * kLaneElems;
            if (rel >= avail) continue;
            uint32_t w[W];
            encode8<BITS>(v[u], p, w);
            store_codes<BITS, NT>(cb, rel, w);
            const bool leader = (S > 1) ? (k == 0 && lane == 0) : (lane % L == 0);
            if (leader) {
                sb[rel / G] = p.s16;
                zb[rel / G] = p.z16;
            }
        }
    }
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

// 8 packed 16-bit activations -> binary32 (exact).
template <int DT>
__device__ __forceinline__ void widen8(const u32x4 &raw, float (&v)[kLaneElems]) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if constexpr (DT == 1) {   // bfloat16: the high half of a binary32
            v[2 * k + 0] = __builtin_bit_cast(float, w[k] << 16);
            v[2 * k + 1] = __builtin_bit_cast(float, w[k] & 0xFFFF0000u);
        } else {                   // binary16
            const f16x2 h = __builtin_bit_cast(f16x2, w[k]);
            v[2 * k + 0] = (float)h.x;
            v[2 * k + 1] = (float)h.y;
        }
    }
}

// binary32 -> 8 packed 16-bit outputs, round to nearest even
// (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32).
template <int DT>
__device__ __forceinline__ u32x4 narrow8(const float (&o)[kLaneElems]) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f32x2 pair = {as_f32(o[2 * k]), as_f32(o[2 * k + 1])};
        if constexpr (DT == 1) {
            w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pair, bf16x2));
        } else {
            w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pair, f16x2));
        }
    }
    const u32x4 r = {w[0], w[1], w[2], w[3]};
    return r;
}

}  // namespace fc
