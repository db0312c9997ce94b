// Internal launch description of the deformable-convolution kernels (dcn.hip),
// filled by the host API (dcn_api.cpp).  Not part of the public ABI.
//
// Lane layout: a lane covers VEC consecutive channels (16 bytes of input: 4
// binary32 or 8 16-bit elements, else 1).  The Dv = D / VEC vectors of a group
// take Lg lanes (the next power of two, at most 64; lanes past Dv idle), the G
// groups of one output pixel take Lp = min(64, G * Lg) lanes, so a wave holds
// 64 / Lp pixels, and a lane covers NV = G * Lg / Lp groups of its pixel.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace da {

struct DcnArgs {
    const void* input;       // [N, H, W, C] of in_dtype
    const float* om;         // [N, Ho, Wo, G, 3K]
    void* out;               // [N, Ho, Wo, C] of out_dtype
    const void* grad_out;    // [N, Ho, Wo, C] of out_dtype
    float* grad_input;       // [N, H, W, C]
    float* grad_om;          // [N, Ho, Wo, G, 3K]
    int64_t n_pix;           // N * Ho * Wo
    uint32_t in_bytes;       // buffer range of input; also the "outside" offset
    uint32_t gi_bytes;       // buffer range of grad_input
    uint32_t om_bytes;       // buffer range of offset_mask
    int32_t N, H, W, C, G, D, KH, KW, SH, SW, PH, PW, DH, DW, Ho, Wo, K;
    int32_t Dv, Lg, log2Lg, Lp, log2Lp;
    int32_t out_dtype, go_dtype;
    int32_t out_vec4;        // out 16-byte aligned, VEC % 4 == 0: 8- or 16-byte vector stores
    int32_t go_vec4;         // grad_out 16-byte aligned, VEC % 4 == 0: vector loads (any type)
    // Backward by input tiles: workgroup (n, tile, group) owns TY x TX input pixels
    // of one group and sums their gradient in LDS as 64-bit fixed point (pixel
    // stride Dp = D + 1 words).  Samples whose grid point lies within M + 1 pixels
    // of a tile reach it through its ring loop; corners farther than that are
    // listed in fb (sample * 4 + corner) and added afterwards with atomics.
    int32_t TY, TX, M, tiles_y, tiles_x, Dp;
    int32_t bLg, blog2Lg, bNVL;   // backward lanes: bLg lanes per sample, bNVL vectors per lane
    uint32_t* ctrl;          // workspace control words (zeroed first): kDcnCtrl*
    uint32_t* fb;            // workspace: [4 * N * Ho * Wo * G * K]
    int32_t log2_terms;      // ceil(log2(most terms one tile sum can take))
};

// Workspace control words
constexpr int kDcnCtrlFar = 0;      // entries in fb
constexpr int kDcnCtrlMaxGo = 1;    // max |grad_out| (binary32 bits)
constexpr int kDcnCtrlMaxM = 2;     // max |m|

// vec: channels per lane vector (1, 4 or 8); nv: groups per lane (1, 2, 4 or 8)
hipError_t launch_dcn_forward(const DcnArgs& a, int in_dtype, int vec, int nv, hipStream_t stream);
// Backward: the bound of the fixed-point terms, the tile kernel (grad_offset_mask,
// and grad_input stored tile by tile), then the far corners by atomics.
// lds_bytes: the tile kernel's dynamic LDS.
hipError_t launch_dcn_backward(const DcnArgs& a, int in_dtype, int vec, size_t lds_bytes,
                               hipStream_t stream);
// Dynamic LDS of the backward tile kernel: the [TY*TX][Dp] 64-bit sums, the number of
// terms each tile pixel took (one 32-bit counter per pixel), per wave a list of up to
// 64 records (kDcnListWords words each: the shared home records, then the accepted
// ring candidates), and the fixed shape's tap table.
constexpr int kDcnTileThreads = 512;   // backward tile kernel workgroup
constexpr int kDcnBwdWaves = kDcnTileThreads / 64;
constexpr int kDcnListWords = 5;
// taps whose home ranges the fixed-shape tile kernel keeps in an LDS table (8 words
// each); kernels with more taps take the general form
constexpr int kDcnShareTaps = 16;
inline size_t dcn_tile_lds_bytes(int ty, int tx, int dp) {
    return (size_t)ty * tx * dp * 8 + (size_t)ty * tx * 4 +
           (size_t)kDcnBwdWaves * 64 * kDcnListWords * 4 + (size_t)kDcnShareTaps * 32;
}

}  // namespace da
