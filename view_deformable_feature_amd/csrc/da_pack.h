// Internal launch description of the level packing kernels (da_pack.hip),
// filled by the host API (da_api.cpp).  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace da {

constexpr int kPackMaxScales = 64;

struct PackArgs {
    void* maps[kPackMaxScales];            // per scale: [B, N, C, H_s * W_s]
    void* packed;                          // [B, num_feat, C]
    int64_t hw[kPackMaxScales];            // H_s * W_s
    int64_t start_in_cam[kPackMaxScales];  // first row of scale s inside a camera's block
    int64_t tile_base[kPackMaxScales + 1]; // prefix of per-scale tile counts (per (b, k))
    int64_t rows_per_cam;                  // sum_s H_s * W_s
    int64_t num_feat;                      // N * rows_per_cam
    int64_t c_tiles;                       // ceil(C / 64)
    int32_t B, N, S, C;
    int32_t pairs;                         // 16-bit elements moved two at a time
};

hipError_t launch_pack(const PackArgs& a, int elem_bytes, bool pack, hipStream_t stream);

}  // namespace da
