// Packing of per-scale camera feature maps into the flattened multi-camera,
// multi-scale layout the aggregation reads, and back.
//
// Definition followed: the Sparse4D deformable_aggregation walkthrough
// (mhpn.cn/news/1081857), section 6 (feature_maps_format turns the per-scale
// [B, N, C, H, W] maps into one flattened feature tensor plus its level table,
// and back) and section 3.1 (each level stored HWC: element (i, j, c) at
// (i W + j) C + c).  Level (camera k, scale s) occupies rows
// k * sum_s' H_s' W_s' + sum_{s' < s} H_s' W_s' onward (camera-major).
//
// Both directions are a transpose of each (b, k, s) map between C x HW and
// HW x C, done through a 64 x 64 LDS tile so that global reads and writes are
// both contiguous along a row of the tile.  Elements are moved as raw 2- or
// 4-byte words (bit-exact for every element type).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "da_pack.h"

namespace da {
namespace {

constexpr int kTile = 64;
constexpr int kPackThreads = 256;
constexpr int kRowsPerPass = kPackThreads / kTile;   // 4

// Which (scale, tile) a block handles: tiles of scale s are
// [tile_base[s], tile_base[s + 1]) within one (b, k) map set.
__device__ __forceinline__ int scale_of(const PackArgs& a, int64_t t) {
    int s = 0;
    while (s + 1 < a.S && a.tile_base[s + 1] <= t) ++s;
    return s;
}

// PACK: map[b, k, c, p] -> packed[b, row0 + p, c]; otherwise the reverse.
template <typename W, bool PACK>
__global__ void __launch_bounds__(kPackThreads) pack_kernel(PackArgs a) {
    __shared__ W tile[kTile][kTile + 1];
    const int64_t t = blockIdx.x;
    const int bk = blockIdx.y;                 // b * N + k
    const int b = bk / a.N, k = bk - (bk / a.N) * a.N;
    const int s = scale_of(a, t);
    const int64_t local = t - a.tile_base[s];
    const int64_t hw = a.hw[s];
    const int64_t p0 = (local / a.c_tiles) * kTile;             // pixel tile
    const int64_t c0 = (local - (local / a.c_tiles) * a.c_tiles) * kTile;
    const int tx = threadIdx.x % kTile, ty = threadIdx.x / kTile;
    const int64_t C = a.C;
    const int64_t row0 = (int64_t)k * a.rows_per_cam + a.start_in_cam[s];
    W* map = static_cast<W*>(a.maps[s]) + (int64_t)bk * C * hw;      // [C, hw]
    W* packed = static_cast<W*>(a.packed) + ((int64_t)b * a.num_feat + row0) * C;   // [hw, C]

    if (PACK) {
        for (int r = ty; r < kTile; r += kRowsPerPass) {      // channel c0 + r, pixels along x
            const int64_t c = c0 + r, p = p0 + tx;
            if (c < C && p < hw) tile[r][tx] = map[c * hw + p];
        }
        __syncthreads();
        for (int r = ty; r < kTile; r += kRowsPerPass) {      // pixel p0 + r, channels along x
            const int64_t p = p0 + r, c = c0 + tx;
            if (c < C && p < hw) packed[p * C + c] = tile[tx][r];
        }
    } else {
        for (int r = ty; r < kTile; r += kRowsPerPass) {      // pixel p0 + r, channels along x
            const int64_t p = p0 + r, c = c0 + tx;
            if (c < C && p < hw) tile[tx][r] = packed[p * C + c];
        }
        __syncthreads();
        for (int r = ty; r < kTile; r += kRowsPerPass) {      // channel c0 + r, pixels along x
            const int64_t c = c0 + r, p = p0 + tx;
            if (c < C && p < hw) map[c * hw + p] = tile[r][tx];
        }
    }
}

// 16-bit elements moved in pairs: each global access is a 32-bit word of two
// consecutive elements along the contiguous direction (pixels of one channel in
// a map, channels of one pixel in the packed tensor), as wide per lane as the
// 32-bit kernel's.  Needs C and every H_s * W_s even (the host checks).
template <bool PACK>
__global__ void __launch_bounds__(kPackThreads) pack_pairs_kernel(PackArgs a) {
    __shared__ uint16_t tile[kTile][kTile + 2];
    const int64_t t = blockIdx.x;
    const int bk = blockIdx.y;
    const int b = bk / a.N, k = bk - (bk / a.N) * a.N;
    const int s = scale_of(a, t);
    const int64_t local = t - a.tile_base[s];
    const int64_t hw = a.hw[s];
    const int64_t p0 = (local / a.c_tiles) * kTile;
    const int64_t c0 = (local - (local / a.c_tiles) * a.c_tiles) * kTile;
    constexpr int kHalf = kTile / 2;                        // 32 pairs per tile row
    constexpr int kRows = kPackThreads / kHalf;             // 8 tile rows per pass
    const int tx = threadIdx.x % kHalf, ty = threadIdx.x / kHalf;
    const int64_t C = a.C;
    const int64_t row0 = (int64_t)k * a.rows_per_cam + a.start_in_cam[s];
    uint16_t* map = static_cast<uint16_t*>(a.maps[s]) + (int64_t)bk * C * hw;
    uint16_t* packed = static_cast<uint16_t*>(a.packed) + ((int64_t)b * a.num_feat + row0) * C;

    if (PACK) {
        for (int r = ty; r < kTile; r += kRows) {           // channel c0 + r: pixel pairs
            const int64_t c = c0 + r, p = p0 + 2 * tx;
            if (c < C && p < hw) {
                const uint32_t w = *reinterpret_cast<const uint32_t*>(map + c * hw + p);
                tile[r][2 * tx] = (uint16_t)(w & 0xffffu);
                tile[r][2 * tx + 1] = (uint16_t)(w >> 16);
            }
        }
        __syncthreads();
        for (int r = ty; r < kTile; r += kRows) {           // pixel p0 + r: channel pairs
            const int64_t p = p0 + r, c = c0 + 2 * tx;
            if (c < C && p < hw)
                *reinterpret_cast<uint32_t*>(packed + p * C + c) =
                    (uint32_t)tile[2 * tx][r] | ((uint32_t)tile[2 * tx + 1][r] << 16);
        }
    } else {
        for (int r = ty; r < kTile; r += kRows) {           // pixel p0 + r: channel pairs
            const int64_t p = p0 + r, c = c0 + 2 * tx;
            if (c < C && p < hw) {
                const uint32_t w = *reinterpret_cast<const uint32_t*>(packed + p * C + c);
                tile[2 * tx][r] = (uint16_t)(w & 0xffffu);
                tile[2 * tx + 1][r] = (uint16_t)(w >> 16);
            }
        }
        __syncthreads();
        for (int r = ty; r < kTile; r += kRows) {           // channel c0 + r: pixel pairs
            const int64_t c = c0 + r, p = p0 + 2 * tx;
            if (c < C && p < hw)
                *reinterpret_cast<uint32_t*>(map + c * hw + p) =
                    (uint32_t)tile[r][2 * tx] | ((uint32_t)tile[r][2 * tx + 1] << 16);
        }
    }
}

}  // namespace

hipError_t launch_pack(const PackArgs& a, int elem_bytes, bool pack, hipStream_t stream) {
    const dim3 grid((unsigned)a.tile_base[a.S], (unsigned)(a.B * a.N));
    const dim3 block(kPackThreads);
    if (elem_bytes == 4) {
        if (pack) hipLaunchKernelGGL((pack_kernel<uint32_t, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((pack_kernel<uint32_t, false>), grid, block, 0, stream, a);
    } else if (a.pairs) {
        if (pack) hipLaunchKernelGGL((pack_pairs_kernel<true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((pack_pairs_kernel<false>), grid, block, 0, stream, a);
    } else {
        if (pack) hipLaunchKernelGGL((pack_kernel<uint16_t, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((pack_kernel<uint16_t, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace da
