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
//   - a workgroup of 8 waves (2 per SIMD, so that one wave's matrix-core work
//     covers the other's waits) owns a 256 (channels n) x 256 (tokens t)
//     output tile of one rank; wave (wn, wt) owns 128 x 64 of it as 4 x 2
//     MFMA blocks of 32 x 32;
//   - the MFMA's row operand is W (rows n) and its column operand is A (rows
//     t), so the accumulator of a lane holds, for ONE token t (lane % 32), 16
//     channels n = 8*(v/4) + 4*(lane/32) + v%4 of each block: a quantization
//     group (<= 128 consecutive channels of one token) lies in one lane pair
//     (lane, lane ^ 32), half in each, and its minimum and maximum need one
//     v_permlane32_swap after the in-lane reduction;
//   - K is walked in stages of 32, staged in pairs: both 256 x 64 operand
//     tiles of a pair of stages go to one of two LDS buffers (2 x 64 KiB)
//     straight from global memory (buffer_load ... lds), a pair ahead of the
//     matrix cores. A staged row is 64 k values = 128 bytes, one whole L2
//     line per row and load, so the operand traffic reaches L2 as full-line
//     requests; each row's eight 16-byte chunks are rotated by (row / 2) % 8
//     so that the fragment reads (32 rows x one chunk) are free of bank
//     conflicts;
//   - one persistent workgroup per CU walks its tiles; the workgroups of an
//     XCD (its own L2) run 4 token tiles x 8 channel tiles at a time, so
//     that they share their A and W stage tiles in L2. For long rows (large
//     K) the 8 XCDs form a 4 x 2 grid over each rank's tiles (token quarters
//     x channel halves), all on the same rank at once: an A tile is read by
//     2 XCDs and a W tile by 4 at about the same time, one of them from HBM
//     and the others from the Infinity Cache. For short rows each XCD takes
//     its own contiguous run of tiles. A tile's stores drain during the next
//     tile;
//   - for long rows, each workgroup also fetches into L2, kPfDist pairs ahead
//     of its staging, its share of the lines that the tiles running beside
//     it on the same XCD will stage (a dword load per 128-byte line, landing
//     in a 256-byte LDS sink): the staging loads then hit L2 instead of
//     waiting on the Infinity Cache or HBM, which the workgroup barrier of
//     every pair would otherwise wait for.
#include <atomic>
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
constexpr int kTileK = 32;                  // k per stage (2 MFMA steps of 16)
constexpr int kPairK = 2 * kTileK;          // k per staged pair of stages (128-byte rows)
constexpr int kPairs = 2;                   // LDS buffers, one pair each
constexpr int kThreads = 512;               // 8 waves, 2 per SIMD
constexpr int kSpanN = 128;                 // channels per wave
constexpr int kSpanT = 64;                  // tokens per wave
constexpr int kBlkN = kSpanN / 32;          // 32 x 32 MFMA blocks per wave, channel side
constexpr int kBlkT = kSpanT / 32;          // and token side
constexpr int kWPair = kTileN * kPairK;               // elements of one pair's W tile
constexpr int kPair = (kTileN + kTileT) * kPairK;    // 16-bit elements per pair buffer (W, then A)
constexpr int kGroupT = 4;                  // token tiles per scheduling group
constexpr int kXcds = 8;
constexpr int kGridT = 4;                   // XCD grid: token groups (x channel groups kXcds / kGridT)
constexpr int kGridMinK = 3072;             // XCD-grid tile order and L2 prefetch from this K on
constexpr int kPfDist = 2;                  // L2 prefetch distance, in pairs beyond the newest staged
constexpr int kLdsBytes = 160 * 1024;       // LDS per workgroup on gfx950
// buffer resource word 3 for raw (untyped, unswizzled) 32-bit-addressed
// buffers on gfx9-family GPUs
constexpr int kRawBufferFlags = 0x00020000;


template <int DT>
__device__ __forceinline__ f32x16 mfma(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
    if constexpr (DT == 1)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// s_waitcnt until at most N vector-memory operations of this wave are
// outstanding and all of its LDS operations are done (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt left at its maximum, lgkmcnt 0). The LDS part
// makes sure this wave's reads of a buffer have completed before the barrier
// after which another wave may refill it.
template <int N>
__device__ __forceinline__ void wait_loads() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier that orders memory accesses for the compiler but, unlike
// __syncthreads, does not wait for this wave's outstanding loads: the staging
// loads of later stages stay in flight (their completion is waited for with
// wait_loads before the barrier that publishes them).
__device__ __forceinline__ void barrier_keep_loads() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
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

template <int DT, int BITS, int G, int PFD>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void linear_quantize_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ W, int T, int K, int H,
    int tiles_t, int tiles_n, int total, int grid, int xcd_grid, uint8_t *__restrict__ codes,
    uint16_t *__restrict__ s, uint16_t *__restrict__ z, uint16_t *__restrict__ y) {
    static_assert(G >= 8 && G <= kTileN && (G & (G - 1)) == 0, "group of 8..256 channels");
    constexpr bool kPf = PFD > 0;               // L2 prefetch PFD pairs ahead
    // a group of 256 channels is a whole tile row: the two waves that share
    // its tokens (wn = 0, 1) each hold half of it and swap their halves'
    // minimum and maximum through LDS
    constexpr bool kSplitGroup = G > kSpanN;
    constexpr int kGW = kSplitGroup ? kSpanN : G;    // channels of a group in one wave
    // Epilogue staging: a tile's codes (rows padded by 16 bytes to spread the
    // LDS banks), then its scales and zeros. When it fits between the first
    // pair buffer and the end of LDS (all but 8-bit codes in groups of 8), the
    // next tile's first pair is fetched into buffer 0 before this tile's
    // epilogue runs (EARLY); otherwise the staging reuses the buffers.
    constexpr int kCodeRow = kTileN * BITS / 8;      // code bytes of a tile row
    constexpr int kCodePitch = kCodeRow + 16;
    constexpr int kMetaRow = kTileN / G * 2;         // bytes of s (or z) of a tile row
    constexpr int kStagingBytes = kTileT * (kCodePitch + 2 * kMetaRow);
    constexpr int kRingBytes = kPairs * kPair * 2;
    constexpr bool kEarly = kPair * 2 + kStagingBytes <= kLdsBytes;
    constexpr int kStagingOff = kEarly ? kPair * 2 : 0;
    // min/max swap area of split groups: per wave and token block, 32 (min, max) pairs
    constexpr int kXchgOff = (kStagingOff + kStagingBytes + 15) / 16 * 16;
    constexpr int kXchgBytes = kSplitGroup ? kThreads / kWave * kBlkT * 32 * 8 : 0;
    constexpr int kLdsData = kXchgOff + kXchgBytes > kRingBytes ? kXchgOff + kXchgBytes : kRingBytes;
    constexpr int kSinkOff = kLdsData;          // where the prefetch loads land (never read)
    constexpr int kLdsUsed = kLdsData + (kPf ? 256 : 0);
    static_assert(kLdsUsed <= kLdsBytes && kStagingBytes + kXchgBytes <= kRingBytes,
                  "staging fits in LDS");
    __shared__ __attribute__((aligned(16))) uint16_t lds[kLdsUsed / 2];

    const uint32_t tid = __builtin_amdgcn_workitem_id_x();
    const int lane = (int)(tid & 63u);
    const int wave = __builtin_amdgcn_readfirstlane((int)(tid >> 6));
    const int wn = wave & 1, wt = wave >> 1;   // wt in 0..3
    const uint32_t rowb = (uint32_t)K * 2u;          // bytes per operand row
    const int KT = K / kTileK;                       // stages
    const int KP = (KT + 1) / 2;                     // staged pairs (the last may be half used)

    // Persistent workgroups (`grid` of them, one per CU; workgroup b runs on
    // XCD b % 8). What an XCD runs: its own contiguous run of all tiles, or,
    // on the XCD grid (`xcd_grid`, needs tiles_t % 4 == 0 and tiles_n % 2 ==
    // 0), token quarter x % 4 x channel half x / 4 of each rank (XCD x), rank
    // after rank. Within its share, the XCD's workgroups take consecutive
    // tiles in groups of kGroupT token tiles x all channel tiles of the
    // share. A workgroup's stores of one tile drain while it computes the
    // next.
    const int bid = (int)__builtin_amdgcn_workgroup_id_x();
    const bool by_xcd = total % kXcds == 0 && grid % kXcds == 0;
    struct Tile {
        int r, n0, t0;
        uint32_t abytes;                 // bytes of the tile's real token rows of A
        const uint16_t *wb, *ab;         // the tile's first W and A rows
        // L2 prefetch share: this tile's W tile is staged by the w_share
        // tiles of its scheduling group with the same channels (token index
        // pf_t among them), its A tile by the a_share with the same tokens
        // (channel index pf_n); each fetches 1/w_share of the W rows and
        // 1/a_share of the A rows (log2 of the shares; -1: fetch nothing)
        int pf_t, pf_n, w_log, a_log;
    };
    // Tile of iteration `it` of this workgroup; false when there is none.
    // The A resource covers only the tile's real token rows: rows past T read
    // as zeros (their outputs are never stored).
    auto tile_at = [&](int it, Tile &tl) -> bool {
        // r: the rank; i: the index within a share of `span` token tiles from
        // `tbase` x `span_n` channel tiles from `nbase`
        int r, i, span, tbase, span_n = tiles_n, nbase = 0;
        if (by_xcd) {
            const int slot = it * (grid / kXcds) + bid / kXcds;
            if (slot >= total / kXcds) return false;
            if (xcd_grid) {
                const int x = bid % kXcds;
                span = tiles_t / kGridT;
                span_n = tiles_n / (kXcds / kGridT);
                r = slot / (span * span_n);
                i = slot - r * span * span_n;
                tbase = (x % kGridT) * span;
                nbase = (x / kGridT) * span_n;
            } else {
                const int logical = (bid % kXcds) * (total / kXcds) + slot;
                span = tiles_t;
                r = logical / (tiles_t * tiles_n);
                i = logical - r * tiles_t * tiles_n;
                tbase = 0;
            }
        } else {
            const int logical = it * grid + bid;
            if (logical >= total) return false;
            span = tiles_t;
            r = logical / (tiles_t * tiles_n);
            i = logical - r * tiles_t * tiles_n;
            tbase = 0;
        }
        const int grp = i / (kGroupT * span_n);
        const int first_t = grp * kGroupT;
        const int gsize = min(span - first_t, kGroupT);
        const int in_grp = i - grp * kGroupT * span_n;
        tl.r = r;
        tl.t0 = (tbase + first_t + in_grp % gsize) * kTileT;
        tl.n0 = (nbase + in_grp / gsize) * kTileN;
        const uint16_t *Wb = W + ((size_t)r * H + tl.n0) * (size_t)K;
        const uint16_t *Ab = A + ((size_t)r * T + tl.t0) * (size_t)K;
        tl.abytes = (uint32_t)min(kTileT, T - tl.t0) * rowb;
        tl.wb = Wb;
        tl.ab = Ab;
        // the XCD's 32 workgroups run 4 token x 8 channel tiles of a group
        // at a time (fewer channel tiles when the group is narrower)
        const int a_share = span_n >= 8 ? 8 : span_n >= 4 ? 4 : span_n >= 2 ? 2 : 1;
        tl.pf_t = in_grp % gsize;
        tl.pf_n = (in_grp / gsize) % a_share;
        tl.w_log = gsize == 4 ? 2 : gsize == 2 ? 1 : gsize == 1 ? 0 : -1;
        tl.a_log = a_share == 8 ? 3 : a_share == 4 ? 2 : a_share == 2 ? 1 : 0;
        return true;
    };

    // Staging, global -> LDS directly (buffer_load_dwordx4 ... lds: lane i's
    // 16 bytes land at the instruction's LDS base + 16 i). One instruction
    // fills 8 staged rows of 128 bytes; lane i serves row i / 8 at chunk
    // position i % 8, so it fetches the operand's chunk (i % 8) ^ ((row / 2) %
    // 8) -- the rotation the fragment reads undo. Wave w fills rows
    // w*32 .. w*32+31 of both tiles (4 instructions each, 8 per pair).
    // Addresses are the tile's buffer resources (SGPRs), a 32-bit lane offset
    // (one for even and one for odd instructions: the rotation of row
    // w*32 + 8j + i/8 is (4 (j % 2) + i/16) % 8) and, as the scalar offset,
    // the pair's k offset plus the instruction's 8 j rows. The last pair of an odd stage count
    // also fetches k values past the row's end: those bytes belong to the
    // next row, or lie past the resource and read as zeros, and are never
    // used.
    constexpr int kLoadsPerPair = 8;             // per wave
    constexpr bool kSplitIssue = !(BITS == 4 && G == 8);   // a pair's loads in two halves
    const uint32_t wrow0 = (uint32_t)wave * 32u;
    // Per-lane offsets of the staging loads and of the fragment reads (below).
    // They are recomputed from the lane id for every tile and before every
    // batch of staging loads (`fresh` keeps the compiler from hoisting them),
    // so that none of them is live across the epilogue, which needs nearly all
    // of the registers.
    struct LaneOffs {
        uint32_t voff_even, voff_odd;   // staging loads: lane offset of even / odd instructions
        uint32_t cx0, cx1;              // fragment reads: rotated chunk offset of steps 0 / 1
        uint32_t fbw, fba;              // fragment reads: the wave's W and A row bases (bytes)
    };
    auto lane_offs = [&]() {
        const uint32_t l = fresh((uint32_t)lane);
        LaneOffs o;
        const uint32_t lrow = l >> 3;            // row within a staging instruction's 8
        const uint32_t lpos = l & 7u;            // 16-byte position within the staged row
        const uint32_t vrow = (wrow0 + lrow) * rowb;
        o.voff_even = vrow + ((lpos ^ ((lrow >> 1) & 7u)) << 4);
        o.voff_odd = vrow + ((lpos ^ ((4u + (lrow >> 1)) & 7u)) << 4);
        const uint32_t frow = l & 31u, fhalf = l >> 5;
        const uint32_t rotx = fhalf ^ ((frow >> 1) & 7u);
        o.cx0 = rotx << 4;
        o.cx1 = (rotx ^ 2u) << 4;
        o.fbw = (uint32_t)(wn * kSpanN + frow) * (kPairK * 2);
        o.fba = kWPair * 2 + (uint32_t)(wt * kSpanT + frow) * (kPairK * 2);
        return o;
    };
    // part nb (0..3) of pair p: instruction j = nb of both operands
    auto pair_in_part = [&](const LaneOffs &lo, const Tile &tl, int p, int nb) {
        uint16_t *sw = lds + (p & 1) * kPair;
        uint16_t *sa = sw + kWPair;
        const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(tl.wb), (short)0, (int)(kTileN * rowb), kRawBufferFlags);
        const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(tl.ab), (short)0, (int)tl.abytes, kRawBufferFlags);
        {
            const int j = nb;
            const uint32_t l0 = (wrow0 + 8u * j) * kPairK;                // wave-uniform
            const int so = p * (kPairK * 2) + 8 * j * (int)rowb;
            // (a named value: a conditional expression written as the
            // builtin's argument makes the host pass drop the launch stub)
            const uint32_t vo = (nb & 1) ? lo.voff_odd : lo.voff_even;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wres, (__attribute__((address_space(3))) void *)(sw + l0), 16, vo, so, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ares, (__attribute__((address_space(3))) void *)(sa + l0), 16, vo, so, 0, 0);
        }
    };
    auto pair_in = [&](const Tile &tl, int p) {
        const LaneOffs lo = lane_offs();
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) pair_in_part(lo, tl, p, nb);
    };
    // L2 prefetch of this workgroup's share of pair p: one dword per 128-byte
    // staged line (row r of a tile: bytes r * rowb + 128 p). Waves 0..3 take
    // the W rows of the share (64 >> w_log each), waves 4..7 the A rows (64
    // >> a_log each). One instruction per wave whatever the share, so that
    // the wait counts stay fixed: lanes with no line, and pairs past the last,
    // read past the end of the resource (no memory access; zeros land in the
    // sink). Rows past T lie past the A resource too.
    auto prefetch = [&](const Tile &tl, int p) {
        const uint32_t l = fresh((uint32_t)lane);
        const bool on_w = wave < 4;
        const __amdgpu_buffer_rsrc_t res = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(on_w ? tl.wb : tl.ab), (short)0,
            (int)(on_w ? kTileN * rowb : tl.abytes), kRawBufferFlags);
        const int lg = on_w ? tl.w_log : tl.a_log;
        const uint32_t per_wave = lg >= 0 ? 64u >> lg : 0u;          // rows per wave
        const uint32_t first = (uint32_t)(on_w ? tl.pf_t : tl.pf_n) * per_wave * 4u +
                               (uint32_t)(wave & 3) * per_wave;
        const bool live = l < per_wave && p < KP;
        const uint32_t off = live ? (first + l) * rowb + (uint32_t)p * (kPairK * 2) : 0xFFFFFFF0u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            res, (__attribute__((address_space(3))) void *)(lds + kSinkOff / 2), 4, off, 0, 0, 0);
    };

    // fragment reads: row (block base + lane % 32), chunk 4 h + 2 ks + lane / 32
    // for step ks of stage kt = 2 p + h (half h of pair p). The rotation of a
    // fragment row, (row / 2) % 8, is (lane % 32 / 2) % 8 for every block, and
    // the chunk's three bits are h, ks and lane / 32, so the rotated chunk is
    // (4 h) ^ (2 ks) ^ rotx: a read is the wave's W or A row base, plus the
    // per-lane chunk offset of ks XOR the stage's half bit (64 bytes), plus
    // the pair buffer's and the block's offsets.
    const uint8_t *lbytes = reinterpret_cast<const uint8_t *>(lds);
    // fragments b (W rows and A rows of block b) of step ks of stage kt
    auto frag_w = [&](const LaneOffs &lo, int kt, int ks, int b, u32x4 (&fw)[kBlkN]) {
        const uint32_t off = ((ks ? lo.cx1 : lo.cx0) ^ ((uint32_t)(kt & 1) << 6)) +
                             (uint32_t)b * (32 * kPairK * 2);
        const uint32_t pb = (uint32_t)((kt >> 1) & 1);
        fw[b] = *reinterpret_cast<const u32x4 *>(lbytes + lo.fbw + off + pb * (kPair * 2));
    };
    auto frag_a = [&](const LaneOffs &lo, int kt, int ks, int b, u32x4 (&fa)[kBlkT]) {
        const uint32_t off = ((ks ? lo.cx1 : lo.cx0) ^ ((uint32_t)(kt & 1) << 6)) +
                             (uint32_t)b * (32 * kPairK * 2);
        const uint32_t pb = (uint32_t)((kt >> 1) & 1);
        fa[b] = *reinterpret_cast<const u32x4 *>(lbytes + lo.fba + off + pb * (kPair * 2));
    };
    // the fragments of chunk nb of a step: W block nb, and A block nb while there is one
    auto frag_part = [&](const LaneOffs &lo, int kt, int ks, int nb, u32x4 (&fw)[kBlkN],
                         u32x4 (&fa)[kBlkT]) {
        frag_w(lo, kt, ks, nb, fw);
        if (nb < kBlkT) frag_a(lo, kt, ks, nb, fa);
    };

    Tile cur;
    if (!tile_at(0, cur)) return;
    pair_in(cur, 0);
    if (KP > 1) pair_in(cur, 1);
    for (int it = 0;; ++it) {
        f32x16 acc[kBlkN][kBlkT];
#pragma unroll
        for (int a = 0; a < kBlkN; ++a)
#pragma unroll
            for (int b = 0; b < kBlkT; ++b) acc[a][b] = f32x16{};

        // One stage = 2 steps of k = 16, 8 MFMAs each; a pair = 2 stages in
        // one LDS buffer. Pair p + 1 is in flight while pair p is computed:
        // in the middle of stage 2p + 1 this wave waits for its loads of pair
        // p + 1 and the workgroup barrier publishes them (every wave has then
        // also read its last fragments of pair p: fragments are read one step
        // ahead); the next step's MFMAs overlap the first fragment reads of
        // pair p + 1 and the issue of half of pair p + 2 into pair p's buffer,
        // the step after it the other half (two bursts of staging requests
        // instead of one: measured 1-3% faster; not for 4-bit codes in groups
        // of 8, which would then run out of registers). With the L2 prefetch,
        // the step after that issues the prefetch of pair p + 2 + PFD, the one
        // load that stays in flight across the wait (vmcnt(1)); otherwise
        // nothing else is outstanding there, and the wait is vmcnt(0). (Loads
        // complete in order, so these counts hold with the previous tile's
        // stores still in flight too.)
        // The wait, the barrier and the issue sit behind uniform branches; the
        // matrix-core work is never under a condition, which would make the
        // compiler spill the accumulators.
        u32x4 fw[2][kBlkN], fa[2][kBlkT];
        // A step in four chunks: chunk nb = the 2 MFMAs of W block nb, then
        // `side(nb)` (the LDS reads and staging loads that overlap them);
        // nothing moves across chunks, so the loads are spread between the
        // MFMAs.
        auto step = [&](int ks, auto &&side) {
#pragma unroll
            for (int nb = 0; nb < kBlkN; ++nb) {
#pragma unroll
                for (int tb = 0; tb < kBlkT; ++tb)
                    acc[nb][tb] = mfma<DT>(fw[ks & 1][nb], fa[ks & 1][tb], acc[nb][tb]);
                side(nb);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        const LaneOffs lo = lane_offs();
        // pairs 0 and (when there is one) 1 are in flight: wait for pair 0
        if (KP > 1) wait_loads<kLoadsPerPair>();
        else wait_loads<0>();
        barrier_keep_loads();
#pragma unroll
        for (int b = 0; b < kBlkN; ++b) frag_part(lo, 0, 0, b, fw[0], fa[0]);
        for (int kt = 0; kt + 1 < KT; ++kt) {
            // second half of the pair issued after the previous (odd) stage's barrier
            const bool issue_b = kSplitIssue && (kt & 1) == 0 && kt >= 2 && ((kt - 1) >> 1) + 2 < KP;
            step(0, [&](int nb) {
                frag_part(lo, kt, 1, nb, fw[1], fa[1]);
                if (issue_b && (nb & 1)) pair_in_part(lo, cur, ((kt - 1) >> 1) + 2, 2 + (nb >> 1));
            });
            const bool odd = (kt & 1) != 0;
            if (odd) {
                if constexpr (kPf) wait_loads<1>();   // all but the prefetch of stage kt - 1
                else wait_loads<0>();
                barrier_keep_loads();
            }
            const bool issue = odd && (kt >> 1) + 2 < KP;
            step(1, [&](int nb) {
                frag_part(lo, kt + 1, 0, nb, fw[0], fa[0]);
                if constexpr (kPf) {
                    // every even stage but the last, after its staging loads
                    if (!odd && nb == 0) prefetch(cur, (kt >> 1) + 1 + PFD);
                }
                if constexpr (kSplitIssue) {
                    if (issue && (nb & 1)) pair_in_part(lo, cur, (kt >> 1) + 2, nb >> 1);
                } else {
                    if (issue) pair_in_part(lo, cur, (kt >> 1) + 2, nb);
                }
            });
        }
        step(0, [&](int nb) { frag_part(lo, KT - 1, 1, nb, fw[1], fa[1]); });
        step(1, [&](int) {});

        __syncthreads();   // every wave has read its last operand fragments
        Tile nxt;
        const bool more = tile_at(it + 1, nxt);
        if constexpr (kEarly) {
            if (more) pair_in(nxt, 0);
        }

        // ---- epilogue: round to the dtype, quantize per (token, group) ----
        // Run j = 4 nb + m of a lane holds channels nb*32 + 8m + 4*(lane/32) + 0..3
        // of the wave's span (accumulator entries 4m..4m+3 of block nb); a group
        // of G channels is RG = G/8 consecutive runs of each lane of the pair
        // (of 256 channels: the wave's 16 runs, and the partner wave's 16).
        // Codes, scales and zeros of the whole tile are first gathered in LDS
        // (kStagingOff) and then written out row by row in 16-byte pieces: a
        // token row of the tile is one contiguous run of codes.
        constexpr int RG = kGW / 8;
        uint8_t *lc = reinterpret_cast<uint8_t *>(lds) + kStagingOff;
        uint8_t *lsz = lc + kTileT * kCodePitch;         // s rows, then z rows
        const int Hg = H / G;
        const uint32_t frow = (uint32_t)lane & 31u, fhalf = (uint32_t)lane >> 5;
        const uint32_t h4 = 4u * fhalf;
        const uint32_t lane_y = frow * (uint32_t)H * 2u;
        const int r = cur.r, n0 = cur.n0, t0 = cur.t0;
    #pragma unroll
        for (int tb = 0; tb < kBlkT; ++tb) {
            const uint32_t tl = (uint32_t)(wt * kSpanT + tb * 32) + frow;   // token in the tile
            const int trow0 = t0 + wt * kSpanT + tb * 32;
            const bool live = trow0 + (int)frow < T;
            uint16_t *yb = y ? y + ((size_t)r * T + (size_t)trow0) * (size_t)H +
                                   (size_t)(n0 + wn * kSpanN)
                             : nullptr;
    #pragma unroll
            for (int gi = 0; gi < kSpanN / kGW; ++gi) {
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
                if constexpr (kSplitGroup) {
                    // swap with the wave holding the other 128 channels of these tokens
                    float *xc = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(lds) + kXchgOff) +
                                (size_t)tb * (kThreads / kWave) * 64;
                    if (fhalf == 0) {
                        xc[(uint32_t)wave * 64u + frow * 2u] = mn;
                        xc[(uint32_t)wave * 64u + frow * 2u + 1u] = mx;
                    }
                    wait_loads<63>();
                    barrier_keep_loads();
                    mn = __builtin_fminf(mn, xc[(uint32_t)(wave ^ 1) * 64u + frow * 2u]);
                    mx = __builtin_fmaxf(mx, xc[(uint32_t)(wave ^ 1) * 64u + frow * 2u + 1u]);
                }
                const GroupParams p = group_params<BITS>(mn, mx);
    #pragma unroll
                for (int jj = 0; jj < RG; ++jj) {
                    const int j = gi * RG + jj;
                    const uint32_t ch = (uint32_t)((j / 4) * 32 + (j % 4) * 8) + h4;   // in the wave span
                    const uint32_t q = encode4<BITS>(yv[jj], p);
                    const uint32_t at = tl * kCodePitch + (wn * kSpanN + ch) * BITS / 8;
                    if constexpr (BITS == 8)
                        *reinterpret_cast<uint32_t *>(lc + at) = q;
                    else
                        *reinterpret_cast<uint16_t *>(lc + at) = (uint16_t)q;
                    if (yb && live) stv<u32x2, false>(yb, lane_y + ch * 2u, u32x2{yw[jj][0], yw[jj][1]});
                }
                if (fhalf == 0 && (!kSplitGroup || wn == 0)) {
                    const uint32_t m = tl * kMetaRow + (uint32_t)(wn * (kSpanN / kGW) + gi) * 2u;
                    *reinterpret_cast<uint16_t *>(lsz + m) = p.s16;
                    *reinterpret_cast<uint16_t *>(lsz + kTileT * kMetaRow + m) = p.z16;
                }
            }
            // one token block at a time: interleaving all of them would need
            // more registers than there are
            __builtin_amdgcn_sched_barrier(0);
        }
        // this wave's LDS writes are done (the next tile's staging loads may
        // stay in flight), then every wave's
        wait_loads<63>();
        barrier_keep_loads();

        // write-out of the tile's live token rows. The thread's offsets are
        // recomputed for every tile from a fresh copy of its id: hoisted out
        // of the tile loop they would all stay live across the main loop.
        const uint32_t wtid = fresh(tid);
        const int rows = min(kTileT, T - t0);
        const size_t grow0 = (size_t)r * T + (size_t)t0;
        FC_GLOBAL uint8_t *cg = sgpr_ptr(codes + (grow0 * (size_t)H + (size_t)n0) * BITS / 8);
        const uint32_t cpitch = (uint32_t)H * BITS / 8;
        constexpr int kCodeChunks = kCodeRow / 16;
    #pragma unroll
        for (int i = 0; i < kTileT * kCodeChunks / kThreads; ++i) {
            const uint32_t id = (uint32_t)i * kThreads + wtid;
            const uint32_t row = id / kCodeChunks, c = id % kCodeChunks;
            if ((int)row < rows)
                stg<u32x4>(cg, row * cpitch + c * 16u,
                           *reinterpret_cast<const u32x4 *>(lc + row * kCodePitch + c * 16u));
        }
        FC_GLOBAL uint16_t *sg = sgpr_ptr(s + grow0 * (size_t)Hg + (size_t)(n0 / G));
        FC_GLOBAL uint16_t *zg = sgpr_ptr(z + grow0 * (size_t)Hg + (size_t)(n0 / G));
        const uint32_t mpitch = (uint32_t)Hg * 2u;
        if constexpr (kMetaRow >= 4) {
            constexpr int kMetaWords = kMetaRow / 4;     // 4-byte pieces of a row
    #pragma unroll
            for (int i = 0; i < (kTileT * kMetaWords + kThreads - 1) / kThreads; ++i) {
                const uint32_t id = (uint32_t)i * kThreads + wtid;
                const uint32_t row = id / kMetaWords, c = id % kMetaWords;
                if ((int)row < rows) {
                    const uint32_t at = row * kMetaRow + c * 4u;
                    stg<uint32_t>(sg, row * mpitch + c * 4u, *reinterpret_cast<const uint32_t *>(lsz + at));
                    stg<uint32_t>(zg, row * mpitch + c * 4u,
                                  *reinterpret_cast<const uint32_t *>(lsz + kTileT * kMetaRow + at));
                }
            }
        } else {
            // one group per tile row: a 2-byte scale and zero per row
            if ((int)wtid < rows) {
                stg<uint16_t>(sg, wtid * mpitch, *reinterpret_cast<const uint16_t *>(lsz + wtid * 2u));
                stg<uint16_t>(zg, wtid * mpitch,
                              *reinterpret_cast<const uint16_t *>(lsz + kTileT * kMetaRow + wtid * 2u));
            }
        }

        wait_loads<63>();   // the staging area has been read out by every wave
        barrier_keep_loads();
        if (!more) break;
        if constexpr (!kEarly) pair_in(nxt, 0);
        if (KP > 1) pair_in(nxt, 1);
        cur = nxt;
    }
}

// Compute units of the current device (one persistent workgroup each),
// looked up once per device. The cache is atomic: calls from several host
// threads may fill it at once (with the same value).
int compute_units() {
    static std::atomic<int> cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            return -1;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// order: 1 the XCD-grid tile order, 0 the XCD runs, -1 the grid exactly when
// K >= kGridMinK (measured on the 70B layer shapes, K = 2048 ... 7168: the
// grid is 2-5% faster from K = 3072 on, where the shared reads come from the
// Infinity Cache; at K = 2048 the XCD runs are 2% faster). The grid needs the
// XCD split of the tiles, tiles_t % 4 == 0 and tiles_n % 2 == 0. The L2
// prefetch runs from K = kGridMinK on, in either order (measured on the 70B
// and 8B layer shapes: 3-6% faster at K = 3584 and 7168; at K = 1024 and
// 2048, where the operands nearly fit the Infinity Cache, 0.5-2% slower).
template <int DT, int BITS, int G>
hipError_t launch_one(const uint16_t *a, const uint16_t *w, int R, int T, int K, int H,
                      uint8_t *codes, uint16_t *s, uint16_t *z, uint16_t *y, hipStream_t stream,
                      int order = -1) {
    const int tiles_t = (T + kTileT - 1) / kTileT;
    const int tiles_n = H / kTileN;
    const long long total = (long long)R * tiles_t * tiles_n;
    if (total > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
    const int cus = compute_units();
    if (cus <= 0) return hipErrorInvalidDevice;
    const int grid = (int)(total < cus ? total : cus);
    const bool can_grid = total % kXcds == 0 && grid % kXcds == 0 && tiles_t % kGridT == 0 &&
                          tiles_n % (kXcds / kGridT) == 0;
    const int xcd_grid = can_grid && (order < 0 ? K >= kGridMinK : order != 0);
    if (K >= kGridMinK)
        hipLaunchKernelGGL((linear_quantize_kernel<DT, BITS, G, kPfDist>), dim3((unsigned)grid),
                           dim3(kThreads), 0, stream, a, w, T, K, H, tiles_t, tiles_n, (int)total,
                           grid, xcd_grid, codes, s, z, y);
    else
        hipLaunchKernelGGL((linear_quantize_kernel<DT, BITS, G, 0>), dim3((unsigned)grid),
                           dim3(kThreads), 0, stream, a, w, T, K, H, tiles_t, tiles_n, (int)total,
                           grid, xcd_grid, codes, s, z, y);
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
    case 256: return launch_one<DT, BITS, 256>(a, w, R, T, K, H, codes, s, z, y, stream);
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
