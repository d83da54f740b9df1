// Argument checks and workspace layout of the C ABI (include/fc.h): plain
// C++, no HIP runtime calls, so that host builds with sanitizers can exercise
// them on their own.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <initializer_list>

#include "fc.h"

namespace fc {
namespace validate {

constexpr size_t kSliceAlign = 256;
constexpr int kMinGroup = 8;
constexpr int kMaxGroup = 8192;
// fc_linear_quantize: channel tile, k stage and the largest group (one
// channel tile row)
constexpr int kLinearTileN = 256;
constexpr int kLinearTileK = 32;
constexpr int kLinearMaxGroup = 256;
// and the largest K and H whose tile offsets fit the kernel's 32-bit buffer
// and lane offsets (256 rows of 2K bytes; 256 token rows of H codes)
constexpr int kLinearMaxK = 1 << 22;
constexpr int kLinearMaxH = 1 << 24;

// Group lengths the fast kernels take; any other even length runs on the
// generic kernels (fc_generic.hip).
inline bool pow2_in_range(int g) { return g >= kMinGroup && g <= kMaxGroup && (g & (g - 1)) == 0; }

// A group length the codec accepts: even (a 4-bit code pair is one byte, and
// groups start at even positions) and at least 2.
inline bool group_ok(int g) { return g >= 2 && g % 2 == 0; }

inline bool aligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t round_up(size_t v) { return (v + kSliceAlign - 1) / kSliceAlign * kSliceAlign; }

// Checks R, T, H, bits and group; on success sets g2 = min(group, H/R).
inline fc_status check_shape(int R, int T, int H, int bits, int group, int *g2) {
    if (bits != 4 && bits != 8) return FC_ERR_BITS;
    if (R < 1 || T < 0 || H < 1) return FC_ERR_SHAPE;
    if (!group_ok(group) || H % group != 0) return FC_ERR_SHAPE;
    if (H % R != 0) return FC_ERR_SHAPE;
    const int C = H / R;
    const int g = group < C ? group : C;
    if (!group_ok(g) || C % g != 0) return FC_ERR_SHAPE;
    *g2 = g;
    return FC_OK;
}

inline fc_status check_ptrs(size_t n, std::initializer_list<const void *> ptrs) {
    if (n == 0) return FC_OK;
    for (const void *p : ptrs)
        if (p == nullptr) return FC_ERR_NULL;
    for (const void *p : ptrs)
        if (!aligned(p)) return FC_ERR_ALIGN;
    return FC_OK;
}

struct Layout {
    size_t off[6];
    size_t size[6];
    size_t total;
};

inline Layout layout(int R, int T, int H, int bits1, int bits2, int group, int g2) {
    const size_t n1 = (size_t)R * (size_t)T * (size_t)H;
    const size_t n2 = (size_t)T * (size_t)H;
    Layout L;
    L.size[0] = n1 * (size_t)bits1 / 8;
    L.size[1] = n1 / (size_t)group * 2;
    L.size[2] = L.size[1];
    L.size[3] = n2 * (size_t)bits2 / 8;
    L.size[4] = n2 / (size_t)g2 * 2;
    L.size[5] = L.size[4];
    size_t o = 0;
    for (int i = 0; i < 6; ++i) {
        L.off[i] = o;
        o += round_up(L.size[i]);
    }
    L.total = o;
    return L;
}

// Shape and both code widths; on success sets g2.
inline fc_status check_shape2(int R, int T, int H, int bits1, int bits2, int group, int *g2) {
    fc_status st = check_shape(R, T, H, bits1, group, g2);
    if (st != FC_OK) return st;
    if (bits2 != 4 && bits2 != 8) return FC_ERR_BITS;
    return FC_OK;
}

}  // namespace validate
}  // namespace fc
