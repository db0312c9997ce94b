// Internal launch description shared by the host API (da_api.cpp) and the
// gfx950 kernels (da_forward.hip, da_backward.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace da {

constexpr int kMaxLevels = 64;     // DA_MAX_LEVELS
constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kMaxWaves = 8;       // waves per workgroup (512 threads)
constexpr int kLdsBudget = 48 * 1024;

// Scan of the per-row entry counts: one workgroup per tile of kScanTile rows.
constexpr int kScanThreads = 256;
constexpr int kScanItems = 16;
constexpr int kScanTile = kScanThreads * kScanItems;   // 4096
// The row-ordered backward's bucket kernel forms the prefix of the tile totals
// itself (in LDS, every workgroup) where there are at most this many tiles --
// one pass of its 256 threads.  Measured: 22 tiles (nuScenes shape) save the
// separate launch (step -0.9 us, deterministic -4.3 us); with 498 tiles (4 x
// 510k rows) every one of ~9,750 workgroups repeating a two-pass prefix cost
// more (+4 us) than the launch.
constexpr int kBucketLdsTiles = 256;
// Levels with at most this many rows are counted in an LDS histogram first
// (measured: merging pays even when a workgroup's 1024 corners spread over
// 2816 rows, against same-address traffic from every XCD).
constexpr int kCountThreads = 256;
constexpr int kCountLdsRows = 16 * kCountThreads;
// Samples per thread on levels counted in LDS: kCountLdsPer where a level has at
// least kCountChunkMinPairs (anchor, point) pairs per batch image, else one.
// Measured: 4 images of 1500 anchors x 13 points, bfloat16 features: counting
// 152 -> 116 us; 900 anchors x 13 points: 18.8 -> 21.1 us (too few workgroups
// left to hide the latency), so that size keeps one sample per thread.
constexpr int kCountLdsPer = 8;
constexpr int kCountChunkMinPairs = 16384;
// Levels of more than kCountTileRows rows are counted by row tiles: one workgroup
// owns kCountTileRows rows of the level, scans all of the level's samples and
// counts the corners that fall in its rows in LDS, so no global atomic is needed
// (returning atomics from every XCD are performed beyond L2, where same-row ones
// serialise).  Measured on 4 images of 160x400 levels: 90 us less per backward
// with bfloat16 features, 22 us less with binary32; on 64x176 levels the tile
// workgroups' scans cost more than the atomics they save, so levels up to
// kCountTileRows rows keep the atomics.
constexpr int kCountTileThreads = 1024;
constexpr int kCountTileRows = 16384;
// Entries covered by one wave of the feature-gradient gather, and the longest
// row a single wave sums whole (longer rows are added range by range).
constexpr int kGatherChunk = 64;
constexpr int kGatherLong = 64;
// Threads per workgroup of the gather.  One-wave workgroups keep more waves
// resident (a freed slot on any SIMD takes the next range) but made each wave
// slower by as much: no faster at 900 anchors, 1-2 % slower at 4 x 1500.
constexpr int kGatherThreads = 256;
// Deterministic backward: a long row (> kGatherLong entries) starting at entry
// `first` owns the int64 accumulation row first / kSlotStride -- unique, since
// the next long row starts at least kSlotStride entries later.
constexpr int kSlotStride = kGatherLong + 1;
// Words of the control block at the start of the backward workspace.
constexpr int kCtrlScanDone = 0;   // (reserved: the bucket kernel, or above 256 tiles a second
                                   // launch, adds the scan's tile totals; no completion count)
constexpr int kCtrlMaxGo = 1;      // max |grad_out| (float bits)
constexpr int kCtrlMaxW = 2;       // max |weight| (float bits)
constexpr int kCtrlMaxCnt = 3;     // max entries of one row
constexpr int kCtrlLongRows = 4;   // long rows listed in long_rows (deterministic form)

// One (sample, corner) contribution to the feature gradient, bucketed by row.
// Offsets are stored in bytes so that the gather does no index arithmetic.
struct Entry {
    uint32_t row;      // flat row b * num_feat + r; bit 31 set when the row is long
                       // (more than kGatherLong entries: summed range by range)
    uint32_t w_off;    // byte offset of the sample's weight row: sample * G * 4
    float cw;          // bilinear corner weight
    uint32_t go_off;   // byte offset of the anchor's grad_out row, (b*A + a) * C * 4,
                       // plus the corner index 0..3 in the two low bits
};
static_assert(sizeof(Entry) == 16, "Entry layout");
constexpr uint32_t kEntryLongRow = 0x80000000u;

// Level slices.  MI355X dispatches workgroup i to XCD i mod 8, and each XCD has
// its own L2.  When the features outgrow one L2, the per-anchor kernels run 8
// workgroups per anchor; workgroup (anchor, x) takes only the samples of the
// levels in slice x, so each XCD's L2 serves only its slice's levels.
constexpr int kSlices = 8;
constexpr int kMaxSliceLevels = kMaxLevels / kSlices;   // 8

// (H, W, first row) of every (camera, scale) level, camera-major.
struct LevelTable {
    int32_t H[kMaxLevels];
    int32_t W[kMaxLevels];
    int32_t start[kMaxLevels];
    // slice x holds levels slice_level[x][0 .. slice_nlev[x]) (used when sliced)
    int8_t slice_level[kSlices][kMaxSliceLevels];
    int8_t slice_nlev[kSlices];
};

// Everything a launch needs.  The per-anchor kernels run one workgroup per
// (batch, anchor); its waves split the anchor's samples.  Inside a wave, a
// "row group" of L lanes (L a power of two, 64 / L row groups per wave) reads
// one feature row: lane li covers vectors li, li + L, li + 2L, ... of VEC
// consecutive channels each.
struct KArgs {
    const void* feat;          // [bs, num_feat, C] of feat_dtype
    const float* loc;          // [bs, A, P, K, 2]
    const float* weights;      // [bs, A, P, K, S, G]
    const void* grad_out;      // [bs, A, C] of go_dtype (binary32 in the gather form)
    void* out;                 // [bs, A, C] of out_dtype
    float* grad_feat;          // [bs, num_feat, C]
    float* grad_loc;           // [bs, A, P, K, 2]
    float* grad_weights;       // [bs, A, P, K, S, G]
    // feature-gradient gather workspace
    uint32_t* scan_done;       // control words (kCtrl*), zeroed with cnt, which follows them
    uint32_t* cnt;             // [n_rows] entries per row, then per-row rank source
    uint32_t* local_start;     // [n_rows] exclusive prefix of cnt inside its scan tile, with
                               // kEntryLongRow set for rows of more than kGatherLong entries
    uint32_t* tile_prefix;     // [n_tiles + 1] exclusive prefix of tile totals; [n_tiles] = total
    uint32_t* tile_tot;        // [n_tiles] the scan tiles' totals
    int32_t tot_in_bucket;     // 1: bucket_kernel forms tile_prefix (no scan_totals_kernel)
    uint32_t* rank;            // [bs, K*S, A*P, 4] rank of (sample, corner) inside its row
    Entry* entries;            // [4 * n_samples] row-sorted entries
    // sliced per-anchor kernels
    float* fwd_part;           // [kSlices, bs*A, C] forward partial sums, one per slice
    float* loc_part;           // [n_samples, 2] location-gradient partial of every sample
    int32_t sliced;            // 1: 8 workgroups per anchor, one per level slice
    int32_t max_slice_samples; // P * max over slices of the slice's level count
    int32_t sample_chunk;      // sliced kernels: samples staged in LDS at once
    int32_t fwd_sweep;         // sliced forward: one wave per (anchor, slice), samples in y order
    // Blocks past anchor_blocks of a gather-form per-anchor launch zero the
    // feature-gradient rows that need it; blocks past gather_blocks of the
    // gather launch add up the location partials (sliced form).
    uint32_t anchor_blocks;
    uint32_t gather_blocks;
    // Row-ordered backward: the gather also forms, for every entry, the dot
    // products of its grad_out row with its feature row per weight group;
    // finalize_kernel turns them into grad_weights and grad_loc.
    int32_t fused;
    uint32_t feat_all_bytes;   // bs * num_feat * C * elem (< 2^32 on this path)
    float* dots;               // [n_samples, 4, G]: entry (q, corner) at (4q + corner) * G
    int32_t w_vec4;            // weights / grad_weights rows readable as float4
    int32_t gather_deep;       // row-ordered gather: deeper batches (feature rows sparse)
    // Deterministic backward: feature-gradient sums in 64-bit fixed point
    int32_t det;
    long long* slots;          // [n_slots, C] accumulation rows of the long rows
    uint32_t* long_rows;       // [n_slots] the long rows, in no particular order
    uint32_t n_slots;
    uint32_t* bound_part;      // [count_kernel blocks][2] each block's max |grad_out|, max |w|
    uint32_t count_blocks;
    int32_t count_per;         // count_kernel: samples per thread on levels counted in LDS
    int32_t count_tile_rows;   // levels of more rows are counted by count_tiles_kernel
    int64_t feat_batch_bytes;  // num_feat * C * elem: byte stride between batch images
    int64_t gfeat_batch_bytes; // num_feat * C * 4
    uint32_t feat_image_bytes; // buffer range of one feature image; also the "outside" offset
    uint32_t gfeat_image_bytes;
    uint32_t n_rows;           // bs * num_feat
    uint32_t n_samples;        // bs * A * P * K * S
    uint32_t n_anchors;        // bs * A
    uint32_t n_tiles;          // ceil(n_rows / kScanTile)
    int32_t num_feat;
    int32_t A, C, P, K, S, G, D;   // D = C / G
    int32_t npk;               // P * K (point, camera) pairs per anchor
    int32_t pk_chunk;          // pairs staged in LDS at once
    int32_t L, log2L;          // lanes per row group
    int32_t nv;                // vectors per lane over all channels: C / (L * VEC)
    int32_t nv_chunk;          // vectors per lane handled by one workgroup (a divisor of nv;
                               // grid.y = nv / nv_chunk splits the channels)
    int32_t row_bytes;         // C * elem
    int32_t grow_bytes;        // C * 4
    int32_t seg;               // backward: group-reduction segment (lanes), see kernels
    int32_t gather_vec;        // feature-gradient gather: channels per lane vector (1 or 4)
    int32_t accumulate;        // feature-gradient gather: add to grad_feat instead of overwrite
    int32_t out_dtype;         // kF32 / kBF16 / kF16: element type of out
    int32_t go_dtype;          // element type of grad_out as the kernels read it
    const void* go_src;        // gather form, 16-bit grad_out: the caller's tensor, converted
    int32_t go_src_dtype;      // into grad_out (workspace) by the first launch
    LevelTable lv;
};

// Element types (the values of da_dtype).
constexpr int kF32 = 0, kBF16 = 1, kF16 = 2;

// Launch shapes chosen by the host.
struct LaunchShape {
    int vec;            // channels per lane vector (1, 4 for f32 / 8 for 16-bit types)
    int nvc;            // compile-time vectors per lane (forward 1..8, backward 1..16)
    int waves;          // waves per workgroup
    int chunks;         // grid.y
    size_t lds_bytes;   // dynamic LDS
    int gather_nv;      // feature-gradient gather: vectors per lane (1, 2, 4, 8, 16)
};

// Sizes of the per-sample descriptors kept in LDS.
constexpr int kFwdDescBytes = 32;   // 4 byte offsets + 4 corner weights
constexpr int kBwdDescBytes = 80;   // 4 feat offsets + 4 grad offsets + 3 x 4 coefficients

hipError_t launch_forward(const KArgs& a, const LaunchShape& s, int64_t n_anchors_total,
                          int feat_dtype, hipStream_t stream);
// Forward by level slices: per-slice partials into a.fwd_part, then their sum
// in fixed slice order into a.out.
hipError_t launch_forward_sliced(const KArgs& a, const LaunchShape& s, int64_t n_anchors_total,
                                 int feat_dtype, hipStream_t stream);
// Backward, scatter form: grad_feat must already hold zeros (or the sum to add to).
hipError_t launch_backward_scatter(const KArgs& a, const LaunchShape& s, int64_t n_anchors_total,
                                   int feat_dtype, hipStream_t stream);
// Backward, gather form: count, scan, per-anchor pass (location / weight
// gradients and entry fill), then the row-parallel feature-gradient gather.
hipError_t launch_backward_gather(const KArgs& a, const LaunchShape& s, int64_t n_anchors_total,
                                  int feat_dtype, hipStream_t stream);
hipError_t launch_fill_zero(void* p, int64_t n_words, hipStream_t stream);

}  // namespace da
