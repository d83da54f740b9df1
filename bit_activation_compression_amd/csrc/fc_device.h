// Device helpers shared by the codec kernels (gfx950, wave64).
//
// Work layout common to all kernels: a wave owns a tile of U "slots"; a slot
// is 64 lanes x 8 consecutive elements = 512 consecutive elements, so every
// lane reads one 16-byte vector of 16-bit values (or the matching 4- or
// 8-byte run of codes) per slot and a wave touches 1 KiB of contiguous
// activations per slot. A quantization group of G elements (a power of two,
// 8 <= G <= 8192) covers G/8 consecutive lanes of one slot when G <= 512, or
// G/512 consecutive slots of one wave when G > 512; group minima and maxima
// are reduced first inside the lane, then across lanes with DPP row
// operations (<= 16 lanes), ds_swizzle (32 lanes) and readlane (64 lanes).
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

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v >> 1); }

// Slots a wave processes per tile for group length G: at least 4 (16 KiB of
// bf16 in flight per wave) and a whole number of groups.
constexpr int tile_slots(int G) { return G > 4 * kSlotElems ? G / kSlotElems : 4; }

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

__device__ __forceinline__ void minmax8(const float (&v)[kLaneElems], float &mn, float &mx) {
    mn = __builtin_fminf(__builtin_fminf(__builtin_fminf(v[0], v[1]), __builtin_fminf(v[2], v[3])),
                         __builtin_fminf(__builtin_fminf(v[4], v[5]), __builtin_fminf(v[6], v[7])));
    mx = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), __builtin_fmaxf(v[2], v[3])),
                         __builtin_fmaxf(__builtin_fmaxf(v[4], v[5]), __builtin_fmaxf(v[6], v[7])));
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
    mn = mn + 0.0f;                  // a zero minimum or maximum is taken as +0
    mx = mx + 0.0f;
    const float range = mx - mn;
    const float s32 = range / Q;     // IEEE division (correctly rounded)
    const _Float16 sh = (_Float16)s32;   // round to nearest even, gradual underflow
    const _Float16 zh = (_Float16)mn;
    const float s = (float)sh;
    GroupParams p;
    p.z = (float)zh;
    p.inv = (s == 0.0f) ? 0.0f : 1.0f / s;
    p.s16 = __builtin_bit_cast(uint16_t, sh);
    p.z16 = __builtin_bit_cast(uint16_t, zh);
    return p;
}

// clamp(round_half_even(fp32(fp32(v - z) * inv)), 0, Q): after the clamp,
// adding 1.5 * 2^23 rounds to an integer half to even and leaves that integer
// in the low mantissa bits, so the code is the low byte of the result.
template <int BITS>
__device__ __forceinline__ uint32_t encode(float v, const GroupParams &p) {
    constexpr float Q = float((1 << BITS) - 1);
    const float t = (v - p.z) * p.inv;
    const float c = __builtin_amdgcn_fmed3f(t, 0.0f, Q);
    return __builtin_bit_cast(uint32_t, c + 12582912.0f);
}

// Pack the low bytes of four words.
__device__ __forceinline__ uint32_t pack_lo_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0C0C0400u);   // [a.b0, b.b0, 0, 0]
    const uint32_t hi = __builtin_amdgcn_perm(d, c, 0x04000C0Cu);   // [0, 0, c.b0, d.b0]
    return lo | hi;
}

// Encode the lane's 8 values; 4-bit codes: one word, element 2i in the low
// nibble of byte i; 8-bit codes: two words, element i in byte i.
template <int BITS>
__device__ __forceinline__ void encode8(const float (&v)[kLaneElems], const GroupParams &p,
                                        uint32_t (&w)[BITS == 4 ? 1 : 2]) {
    uint32_t e[kLaneElems];
#pragma unroll
    for (int i = 0; i < kLaneElems; ++i) e[i] = encode<BITS>(v[i], p);
    if constexpr (BITS == 8) {
        w[0] = pack_lo_bytes(e[0], e[1], e[2], e[3]);
        w[1] = pack_lo_bytes(e[4], e[5], e[6], e[7]);
    } else {
        // low byte of (e_odd << 4) | e_even is the two nibbles (codes < 16)
        w[0] = pack_lo_bytes((e[1] << 4) | e[0], (e[3] << 4) | e[2], (e[5] << 4) | e[4],
                             (e[7] << 4) | e[6]);
    }
}

// Unpack 8 codes to binary32 integers.
template <int BITS>
__device__ __forceinline__ void decode8(const uint32_t (&w)[BITS == 4 ? 1 : 2], float (&q)[kLaneElems]) {
    if constexpr (BITS == 8) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            q[4 * k + 0] = (float)(w[k] & 0xFFu);
            q[4 * k + 1] = (float)((w[k] >> 8) & 0xFFu);
            q[4 * k + 2] = (float)((w[k] >> 16) & 0xFFu);
            q[4 * k + 3] = (float)(w[k] >> 24);
        }
    } else {
        const uint32_t lo = w[0] & 0x0F0F0F0Fu;          // elements 0, 2, 4, 6
        const uint32_t hi = (w[0] >> 4) & 0x0F0F0F0Fu;   // elements 1, 3, 5, 7
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

template <int BITS>
__device__ __forceinline__ void load_codes(const uint8_t *__restrict__ codes, uint64_t elem,
                                           uint32_t (&w)[BITS == 4 ? 1 : 2]) {
    if constexpr (BITS == 8) {
        const uint2 v = *reinterpret_cast<const uint2 *>(codes + elem);
        w[0] = v.x;
        w[1] = v.y;
    } else {
        w[0] = *reinterpret_cast<const uint32_t *>(codes + elem / 2);
    }
}

template <int BITS>
__device__ __forceinline__ void store_codes(uint8_t *__restrict__ codes, uint64_t elem,
                                            const uint32_t (&w)[BITS == 4 ? 1 : 2]) {
    if constexpr (BITS == 8) {
        *reinterpret_cast<uint2 *>(codes + elem) = make_uint2(w[0], w[1]);
    } else {
        *reinterpret_cast<uint32_t *>(codes + elem / 2) = w[0];
    }
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

// 8 packed 16-bit activations -> binary32 (exact).
template <int DT>
__device__ __forceinline__ void widen8(const uint4 &raw, float (&v)[kLaneElems]) {
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

// binary32 -> 8 packed 16-bit outputs, round to nearest even.
template <int DT>
__device__ __forceinline__ uint4 narrow8(const float (&o)[kLaneElems]) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f32x2 pair = {o[2 * k], o[2 * k + 1]};
        if constexpr (DT == 1) {
            w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pair, bf16x2));
        } else {
            w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pair, f16x2));
        }
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace fc
