// Internal launch description shared by the host API (da_api.cpp) and the
// gfx950 kernels (da_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace da {

constexpr int kMaxLevels = 64;     // DA_MAX_LEVELS
constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kMaxWaves = 8;       // waves per workgroup (512 threads)
constexpr int kLdsBudget = 48 * 1024;

// (H, W, first row) of every (camera, scale) level, camera-major.
struct LevelTable {
    int32_t H[kMaxLevels];
    int32_t W[kMaxLevels];
    int32_t start[kMaxLevels];
};

// Everything a forward or backward launch needs.  One workgroup handles one
// (batch, anchor); its waves split the anchor's samples.  Inside a wave, a
// "row group" of L lanes (L a power of two, 64 / L row groups per wave) reads
// one feature row: lane li covers vectors li, li + L, li + 2L, ... of VEC
// consecutive channels each.
struct KArgs {
    const void* feat;          // [bs, num_feat, C] f32 or bf16
    const float* loc;          // [bs, A, P, K, 2]
    const float* weights;      // [bs, A, P, K, S, G]
    const float* grad_out;     // [bs, A, C]
    float* out;                // [bs, A, C]
    float* grad_feat;          // [bs, num_feat, C]
    float* grad_loc;           // [bs, A, P, K, 2]
    float* grad_weights;       // [bs, A, P, K, S, G]
    int64_t feat_batch_bytes;  // num_feat * C * elem: byte stride between batch images
    int64_t gfeat_batch_bytes; // num_feat * C * 4
    uint32_t feat_image_bytes; // buffer range of one feature image; also the "outside" offset
    uint32_t gfeat_image_bytes;
    int32_t A, C, P, K, S, G, D;   // D = C / G
    int32_t npk;               // P * K (point, camera) pairs per anchor
    int32_t pk_chunk;          // pairs staged in LDS at once
    int32_t L, log2L;          // lanes per row group
    int32_t nv;                // vectors per lane over all channels: C / (L * VEC)
    int32_t nv_chunk;          // vectors per lane handled by one workgroup (grid.y splits C)
    int32_t row_bytes;         // C * elem
    int32_t grow_bytes;        // C * 4
    int32_t seg;               // backward: group-reduction segment (lanes), see kernels
    LevelTable lv;
};

// Launch shapes chosen by the host.
struct LaunchShape {
    int vec;            // channels per lane vector (1, 4 for f32 / 8 for bf16)
    int nvc;            // compile-time vectors per lane (1, 2, 4, 8, 16)
    int waves;          // waves per workgroup
    int chunks;         // grid.y
    size_t lds_bytes;   // dynamic LDS
};

// Sizes of the per-sample descriptors kept in LDS.
constexpr int kFwdDescBytes = 32;   // 4 byte offsets + 4 corner weights
constexpr int kBwdDescBytes = 80;   // 4 feat offsets + 4 grad offsets + 3 x 4 coefficients

hipError_t launch_forward(const KArgs& a, const LaunchShape& s, int64_t n_anchors_total,
                          bool bf16, hipStream_t stream);
hipError_t launch_backward(const KArgs& a, const LaunchShape& s, int64_t n_anchors_total,
                           bool bf16, hipStream_t stream);
hipError_t launch_zero(float* p, int64_t n, hipStream_t stream);

}  // namespace da
