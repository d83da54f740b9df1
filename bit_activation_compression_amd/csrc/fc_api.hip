// C ABI of the codec (declared in include/fc.h): argument checks, workspace
// layout and the three launches. Every check happens before anything is
// enqueued, and nothing here calls the HIP runtime until the launches.
#include <stdint.h>

#include <initializer_list>

#include "fc.h"
#include "fc_launch.h"

namespace {

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

bool pow2_in_range(int g) { return g >= kMinGroup && g <= kMaxGroup && (g & (g - 1)) == 0; }

bool aligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t v) { return (v + kSliceAlign - 1) / kSliceAlign * kSliceAlign; }

// Checks R, T, H, bits and group; on success sets g2 = min(group, H/R).
fc_status check_shape(int R, int T, int H, int bits, int group, int *g2) {
    if (bits != 4 && bits != 8) return FC_ERR_BITS;
    if (R < 1 || T < 0 || H < 1) return FC_ERR_SHAPE;
    if (!pow2_in_range(group) || H % group != 0) return FC_ERR_SHAPE;
    if (H % R != 0) return FC_ERR_SHAPE;
    const int C = H / R;
    const int g = group < C ? group : C;
    if (!pow2_in_range(g) || C % g != 0) return FC_ERR_SHAPE;
    *g2 = g;
    return FC_OK;
}

fc_status check_ptrs(size_t n, std::initializer_list<const void *> ptrs) {
    if (n == 0) return FC_OK;
    for (const void *p : ptrs)
        if (p == nullptr) return FC_ERR_NULL;
    for (const void *p : ptrs)
        if (!aligned(p)) return FC_ERR_ALIGN;
    return FC_OK;
}

fc_status from_hip(hipError_t e) { return e == hipSuccess ? FC_OK : FC_ERR_LAUNCH; }

struct Layout {
    size_t off[6];
    size_t size[6];
    size_t total;
};

Layout layout(int R, int T, int H, int bits1, int bits2, int group, int g2) {
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
fc_status check_shape2(int R, int T, int H, int bits1, int bits2, int group, int *g2) {
    fc_status st = check_shape(R, T, H, bits1, group, g2);
    if (st != FC_OK) return st;
    if (bits2 != 4 && bits2 != 8) return FC_ERR_BITS;
    return FC_OK;
}

// The emulated all-reduce: the three stage launches, or for launch-bound
// shapes (decode-sized) the single launch that computes the same payloads and
// output; with_residual: the result is added to `residual`.
fc_status allreduce_emulated(const void *x, fc_dtype dt, int R, int T, int H, int bits1, int bits2,
                             int group, bool with_residual, const void *residual, void *out,
                             void *workspace, size_t workspace_bytes, void *stream) {
    int g2 = 0;
    fc_status st = check_shape2(R, T, H, bits1, bits2, group, &g2);
    if (st != FC_OK) return st;
    if (dt != FC_F16 && dt != FC_BF16) return FC_ERR_DTYPE;
    const uint64_t n = (uint64_t)T * (uint64_t)H;
    st = with_residual ? check_ptrs(n, {x, residual, out, workspace})
                       : check_ptrs(n, {x, out, workspace});
    if (st != FC_OK) return st;
    const Layout L = layout(R, T, H, bits1, bits2, group, g2);
    if (n != 0 && workspace_bytes < L.total) return FC_ERR_WORKSPACE;
    if (n == 0) return FC_OK;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    uint8_t *codes1 = ws + L.off[0];
    uint16_t *s1 = reinterpret_cast<uint16_t *>(ws + L.off[1]);
    uint16_t *z1 = reinterpret_cast<uint16_t *>(ws + L.off[2]);
    uint8_t *codes2 = ws + L.off[3];
    uint16_t *s2 = reinterpret_cast<uint16_t *>(ws + L.off[4]);
    uint16_t *z2 = reinterpret_cast<uint16_t *>(ws + L.off[5]);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (fc::allreduce_small_applies(R, n, group, g2))
        return from_hip(fc::launch_allreduce_small(
            static_cast<const uint16_t *>(x), (int)dt, R, n, bits1, bits2, group, codes1, s1, z1,
            codes2, s2, z2, with_residual ? static_cast<const uint16_t *>(residual) : nullptr,
            static_cast<uint16_t *>(out), s));
    st = from_hip(fc::launch_quantize(static_cast<const uint16_t *>(x), (int)dt, n * (uint64_t)R, bits1,
                                      group, codes1, s1, z1, s));
    if (st != FC_OK) return st;
    st = from_hip(fc::launch_dequant_sum_requant(codes1, s1, z1, R, n, bits1, bits2, group, g2, codes2,
                                                 s2, z2, s));
    if (st != FC_OK) return st;
    if (with_residual)
        return from_hip(fc::launch_dequantize_residual(codes2, s2, z2, n, bits2, g2, (int)dt,
                                                       static_cast<const uint16_t *>(residual),
                                                       static_cast<uint16_t *>(out), s));
    return from_hip(fc::launch_dequantize(codes2, s2, z2, n, bits2, g2, (int)dt,
                                          static_cast<uint16_t *>(out), s));
}

}  // namespace

extern "C" {

fc_status fc_quantize_groups(const void *x, fc_dtype dt, int R, int T, int H, int bits, int group,
                             uint8_t *codes1, uint16_t *s1, uint16_t *z1, void *stream) {
    int g2 = 0;
    fc_status st = check_shape(R, T, H, bits, group, &g2);
    if (st != FC_OK) return st;
    if (dt != FC_F16 && dt != FC_BF16) return FC_ERR_DTYPE;
    const uint64_t n = (uint64_t)R * (uint64_t)T * (uint64_t)H;
    st = check_ptrs(n, {x, codes1, s1, z1});
    if (st != FC_OK || n == 0) return st;
    return from_hip(fc::launch_quantize(static_cast<const uint16_t *>(x), (int)dt, n, bits, group,
                                        codes1, s1, z1, static_cast<hipStream_t>(stream)));
}

fc_status fc_dequant_sum_requant_mixed(const uint8_t *codes1, const uint16_t *s1,
                                       const uint16_t *z1, int R, int T, int H, int bits1,
                                       int bits2, int group, uint8_t *codes2, uint16_t *s2,
                                       uint16_t *z2, void *stream) {
    int g2 = 0;
    fc_status st = check_shape2(R, T, H, bits1, bits2, group, &g2);
    if (st != FC_OK) return st;
    const uint64_t n = (uint64_t)T * (uint64_t)H;
    st = check_ptrs(n, {codes1, s1, z1, codes2, s2, z2});
    if (st != FC_OK || n == 0) return st;
    return from_hip(fc::launch_dequant_sum_requant(codes1, s1, z1, R, n, bits1, bits2, group, g2,
                                                   codes2, s2, z2, static_cast<hipStream_t>(stream)));
}

fc_status fc_dequant_sum_requant(const uint8_t *codes1, const uint16_t *s1, const uint16_t *z1,
                                 int R, int T, int H, int bits, int group,
                                 uint8_t *codes2, uint16_t *s2, uint16_t *z2, void *stream) {
    return fc_dequant_sum_requant_mixed(codes1, s1, z1, R, T, H, bits, bits, group, codes2, s2, z2,
                                        stream);
}

fc_status fc_dequantize(const uint8_t *codes2, const uint16_t *s2, const uint16_t *z2,
                        int T, int H, int bits, int group2, fc_dtype dt, void *out, void *stream) {
    if (bits != 4 && bits != 8) return FC_ERR_BITS;
    if (T < 0 || H < 1 || !pow2_in_range(group2) || H % group2 != 0) return FC_ERR_SHAPE;
    if (dt != FC_F16 && dt != FC_BF16) return FC_ERR_DTYPE;
    const uint64_t n = (uint64_t)T * (uint64_t)H;
    fc_status st = check_ptrs(n, {codes2, s2, z2, out});
    if (st != FC_OK || n == 0) return st;
    return from_hip(fc::launch_dequantize(codes2, s2, z2, n, bits, group2, (int)dt,
                                          static_cast<uint16_t *>(out),
                                          static_cast<hipStream_t>(stream)));
}

fc_status fc_allreduce_emulated_mixed(const void *x, fc_dtype dt, int R, int T, int H, int bits1,
                                      int bits2, int group, void *out, void *workspace,
                                      size_t workspace_bytes, void *stream) {
    return allreduce_emulated(x, dt, R, T, H, bits1, bits2, group, false, nullptr, out, workspace,
                              workspace_bytes, stream);
}

fc_status fc_allreduce_emulated_residual(const void *x, fc_dtype dt, int R, int T, int H,
                                         int bits1, int bits2, int group, const void *residual,
                                         void *out, void *workspace, size_t workspace_bytes,
                                         void *stream) {
    return allreduce_emulated(x, dt, R, T, H, bits1, bits2, group, true, residual, out, workspace,
                              workspace_bytes, stream);
}

fc_status fc_dequantize_residual(const uint8_t *codes2, const uint16_t *s2, const uint16_t *z2,
                                 int T, int H, int bits, int group2, fc_dtype dt,
                                 const void *residual, void *out, void *stream) {
    if (bits != 4 && bits != 8) return FC_ERR_BITS;
    if (T < 0 || H < 1 || !pow2_in_range(group2) || H % group2 != 0) return FC_ERR_SHAPE;
    if (dt != FC_F16 && dt != FC_BF16) return FC_ERR_DTYPE;
    const uint64_t n = (uint64_t)T * (uint64_t)H;
    fc_status st = check_ptrs(n, {codes2, s2, z2, residual, out});
    if (st != FC_OK || n == 0) return st;
    return from_hip(fc::launch_dequantize_residual(codes2, s2, z2, n, bits, group2, (int)dt,
                                                   static_cast<const uint16_t *>(residual),
                                                   static_cast<uint16_t *>(out),
                                                   static_cast<hipStream_t>(stream)));
}

fc_status fc_allreduce_emulated(const void *x, fc_dtype dt, int R, int T, int H, int bits, int group,
                                void *out, void *workspace, size_t workspace_bytes, void *stream) {
    return fc_allreduce_emulated_mixed(x, dt, R, T, H, bits, bits, group, out, workspace,
                                       workspace_bytes, stream);
}

fc_status fc_sum_uncompressed(const void *x, fc_dtype dt, int R, int T, int H, void *out,
                              void *stream) {
    if (R < 1 || T < 0 || H < 1 || H % 8 != 0) return FC_ERR_SHAPE;
    if (dt != FC_F16 && dt != FC_BF16) return FC_ERR_DTYPE;
    const uint64_t n = (uint64_t)T * (uint64_t)H;
    fc_status st = check_ptrs(n, {x, out});
    if (st != FC_OK || n == 0) return st;
    return from_hip(fc::launch_sum(static_cast<const uint16_t *>(x), (int)dt, R, n,
                                   static_cast<uint16_t *>(out), static_cast<hipStream_t>(stream)));
}

fc_status fc_linear_quantize(const void *a, const void *w, fc_dtype dt, int R, int T, int K, int H,
                             int bits, int group, uint8_t *codes1, uint16_t *s1, uint16_t *z1,
                             void *y, void *stream) {
    int g2 = 0;
    fc_status st = check_shape(R, T, H, bits, group, &g2);
    if (st != FC_OK) return st;
    if (K < kLinearTileK || K % kLinearTileK != 0 || K > kLinearMaxK || H % kLinearTileN != 0 ||
        H > kLinearMaxH || group > kLinearMaxGroup)
        return FC_ERR_SHAPE;
    if (dt != FC_F16 && dt != FC_BF16) return FC_ERR_DTYPE;
    const uint64_t n = (uint64_t)R * (uint64_t)T * (uint64_t)H;
    st = check_ptrs(n, {a, w, codes1, s1, z1});
    if (st != FC_OK || n == 0) return st;
    if (y != nullptr && !aligned(y)) return FC_ERR_ALIGN;
    return from_hip(fc::launch_linear_quantize(static_cast<const uint16_t *>(a),
                                               static_cast<const uint16_t *>(w), (int)dt, R, T, K,
                                               H, bits, group, codes1, s1, z1,
                                               static_cast<uint16_t *>(y),
                                               static_cast<hipStream_t>(stream)));
}

size_t fc_workspace_bytes_mixed(int R, int T, int H, int bits1, int bits2, int group) {
    int g2 = 0;
    if (check_shape2(R, T, H, bits1, bits2, group, &g2) != FC_OK) return 0;
    return layout(R, T, H, bits1, bits2, group, g2).total;
}

size_t fc_workspace_bytes(int R, int T, int H, int bits, int group) {
    return fc_workspace_bytes_mixed(R, T, H, bits, bits, group);
}

fc_status fc_workspace_layout_mixed(int R, int T, int H, int bits1, int bits2, int group,
                                    size_t offsets[6], size_t sizes[6]) {
    int g2 = 0;
    fc_status st = check_shape2(R, T, H, bits1, bits2, group, &g2);
    if (st != FC_OK) return st;
    if (offsets == nullptr || sizes == nullptr) return FC_ERR_NULL;
    const Layout L = layout(R, T, H, bits1, bits2, group, g2);
    for (int i = 0; i < 6; ++i) {
        offsets[i] = L.off[i];
        sizes[i] = L.size[i];
    }
    return FC_OK;
}

fc_status fc_workspace_layout(int R, int T, int H, int bits, int group, size_t offsets[6],
                              size_t sizes[6]) {
    return fc_workspace_layout_mixed(R, T, H, bits, bits, group, offsets, sizes);
}

int fc_stage2_group(int R, int H, int group) {
    int g2 = 0;
    // T and bits do not affect g2; pass valid placeholders.
    if (check_shape(R, 1, H, 4, group, &g2) != FC_OK) return 0;
    return g2;
}

const char *fc_status_string(fc_status s) {
    switch (s) {
    case FC_OK: return "FC_OK";
    case FC_ERR_NULL: return "FC_ERR_NULL: a required pointer is NULL";
    case FC_ERR_SHAPE: return "FC_ERR_SHAPE: unsupported R, T, H, group or chunking";
    case FC_ERR_BITS: return "FC_ERR_BITS: bits must be 4 or 8";
    case FC_ERR_ALIGN: return "FC_ERR_ALIGN: device pointers must be 16-byte aligned";
    case FC_ERR_WORKSPACE: return "FC_ERR_WORKSPACE: workspace smaller than fc_workspace_bytes()";
    case FC_ERR_LAUNCH: return "FC_ERR_LAUNCH: the HIP runtime reported a launch error";
    case FC_ERR_DTYPE: return "FC_ERR_DTYPE: dtype must be FC_F16 or FC_BF16";
    }
    return "unknown fc_status";
}

}  // extern "C"
