/*
 * libdeformagg -- Sparse4D-style deformable aggregation on AMD Instinct MI355X (gfx950).
 *
 * For each (batch b, anchor a, channel c) the forward pass computes
 *
 *   out[b,a,c] = sum over points p, cameras k, scales s of
 *                weights[b,a,p,k,s,g(c)] * bilinear(level (k,s) of mc_ms_feat[b], loc[b,a,p,k], c)
 *
 * and the backward pass returns the gradients of a scalar loss with respect to
 * the features, the sampling locations and the weights, given grad_out.
 *
 * Definition: the Sparse4D deformable_aggregation walkthrough
 * (mhpn.cn/news/1081857) --
 *   section 3.1  HWC layout of each level: element (i, j, c) at i*W*C + j*C + c;
 *   section 3.2  bilinear sampling: low corner floor(h), floor(w); high corner one
 *                further; fractions lh, lw; corner weights hh*hw, hh*lw, lh*hw, lh*lw;
 *                a corner outside the level reads zero;
 *   section 4.1  gradients: grad_feat gets corner weight * grad_out * weight at each
 *                inside corner; grad_loc[0] = W * (lh (v4 - v3) + hh (v2 - v1)) * top
 *                and grad_loc[1] = H * (lw (v4 - v2) + hw (v3 - v1)) * top with
 *                top = grad_out * weight; grad_weights += grad_out * sampled value;
 *   section 5.1  the sum runs over points x cameras x scales for every
 *                (batch, anchor, channel);
 *   section 6    DeformableAggregationFunction(mc_ms_feat, spatial_shape,
 *                scale_start_index, sampling_location, weights).
 * Where the page is silent the library takes these readings:
 *   - normalised location (x, y) in level (H, W) maps to pixel coordinates
 *     w = x*W - 0.5, h = y*H - 0.5, each computed in binary32 as a product rounded
 *     to float and then a subtraction rounded to float (no fused multiply-add);
 *   - a sample contributes only when -1 < h < H and -1 < w < W (NaN locations
 *     therefore contribute nothing);
 *   - channel c belongs to group g(c) = c / (C / G);
 *   - location component 0 is x (width), component 1 is y (height).
 *
 * Conventions for every entry point
 *   - All tensors are dense, row-major (C order).  Device pointers point to memory
 *     allocated on the current HIP device; `stream` is a hipStream_t (NULL = the
 *     legacy default stream).  spatial_shape and scale_start_index are HOST arrays
 *     read during the call; they are not retained.
 *   - The caller owns every buffer, including the backward workspace.  The library
 *     never allocates or frees device memory and keeps no state between calls;
 *     calls are asynchronous on `stream` and may be captured into a HIP graph
 *     (zero fills are kernels, not memset nodes).  Faults inside a kernel surface
 *     at the caller's next synchronisation.
 *   - All argument checks run on the host before anything is enqueued.  On any
 *     error no work is enqueued and no output is touched; da_last_error() returns
 *     a message naming the failed check (per calling thread).
 *   - Floating-point results are computed in binary32.  The forward pass is
 *     deterministic (no atomics); so are the location and weight gradients.  The
 *     feature gradient's summation order may vary from run to run (see da_backward).
 */
#ifndef DEFORMAGG_H
#define DEFORMAGG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of the C ABI; the library exports nothing else. */
#if defined(__GNUC__) || defined(__clang__)
#define DA_API __attribute__((visibility("default")))
#else
#define DA_API
#endif

#define DA_VERSION 120         /* 1.2.0 */
#define DA_MAX_LEVELS 64       /* num_cams * num_scale */
#define DA_MAX_EXTENT 32768    /* H and W of every level */

typedef enum {
    DA_OK = 0,
    DA_ERR_INVALID_ARG = 1,    /* a size, pointer or level entry is malformed */
    DA_ERR_UNSUPPORTED = 2,    /* well formed, but outside what the kernels handle */
    DA_ERR_HIP = 3             /* the HIP runtime refused a launch */
} da_status;

/* Element types of mc_ms_feat (feat_dtype) and of out / grad_out (out_dtype).
 * 16-bit types are raw 16-bit patterns.  Arithmetic is binary32 throughout: a
 * 16-bit feature converts exactly, and out is rounded once (to nearest, ties to
 * even) from the binary32 sum; a 16-bit grad_out converts exactly. */
typedef enum {
    DA_F32 = 0,                /* binary32 */
    DA_BF16 = 1,               /* bfloat16 */
    DA_F16 = 2                 /* IEEE binary16 */
} da_dtype;

/*
 * Level slices.  MI355X places workgroup i on accelerator die (XCD) i mod 8, and each
 * die has its own 4 MiB L2.  When the features of one batch image exceed 8 MiB and the
 * num_cams * num_scale levels split into 8 nearly equal shares (at least 8 levels, at
 * most a quarter of the slots idle), the per-anchor kernels run 8 workgroups per anchor:
 * workgroup (anchor, x) takes only the samples of the levels in slice x (levels dealt
 * largest first, round-robin), so each die's L2 caches one eighth of the features.  The
 * partial sums are then added in a fixed order, so results stay deterministic; they may
 * differ from the unsliced kernels' in rounding.  These flags override the choice:
 */
#define DA_FLAG_SLICES_ALWAYS 1  /* slice whatever the sizes (where the lane layout allows) */
#define DA_FLAG_SLICES_NEVER 2   /* one workgroup per anchor                                */
/* Backward form (see da_backward): where feature rows are shared by several
 * corners (on the largest level, 4 * num_anchors * num_pts / (H * W) >= 2) the
 * location and weight gradients come from dot products formed while the feature
 * gradient is gathered in row order; elsewhere, where the lane layout does not
 * allow that form, or with this flag, per-anchor kernels gather the corner rows
 * again instead. */
#define DA_FLAG_BWD_REGATHER 4
#define DA_FLAG_BWD_ROW_ORDER 8  /* the row-ordered backward wherever the lane layout allows */
/* Deterministic backward (da_backward, da_backward_accumulate): every feature-gradient
 * term is rounded once to a multiple of 2^-E and the terms of a row are summed as 64-bit
 * integers, which makes grad_feat independent of the order the terms arrive in: bit for
 * bit the same across runs, backward forms and level slices.  E is derived on the GPU
 * from max|grad_out| * max|weights| * (most terms of any row), leaving ~2^-50 of that
 * bound as the resolution.  grad_out and weights must be finite.  Costs the workspace
 * a 64-bit row per long row (see da_backward_workspace_size). */
#define DA_FLAG_DETERMINISTIC 16

/* Problem sizes.  bs, num_anchors and num_pts may be 0 (then there is nothing to
 * sample: out and grad_feat are filled with zeros).  All other sizes are >= 1,
 * num_embeds % num_groups == 0 and num_cams * num_scale <= DA_MAX_LEVELS. */
typedef struct {
    int64_t bs;           /* batch size                                    */
    int64_t num_feat;     /* rows of one batch image of mc_ms_feat         */
    int64_t num_embeds;   /* C, channels per row                           */
    int64_t num_anchors;  /* A                                             */
    int64_t num_pts;      /* P, keypoints per anchor                       */
    int64_t num_cams;     /* K                                             */
    int64_t num_scale;    /* S                                             */
    int64_t num_groups;   /* G, weight groups over the channels            */
    int32_t feat_dtype;   /* da_dtype of mc_ms_feat                        */
    int32_t flags;        /* DA_FLAG_* bits (SLICES_ALWAYS / _NEVER exclusive, and so are
                             BWD_REGATHER / BWD_ROW_ORDER) */
    int32_t out_dtype;    /* da_dtype of out (forward) and grad_out (backward) */
    int32_t reserved;     /* must be 0                                     */
} da_problem;

/*
 * da_forward_workspace_size -- bytes of device workspace that let da_forward use level
 * slices for `problem`: 8 * bs * A * C * 4 when slices are wanted, else 0.  Only the
 * sizes and flags in `problem` are read.
 */
DA_API da_status da_forward_workspace_size(const da_problem* problem, size_t* bytes);

/*
 * da_forward -- the forward pass (sections 3.2 and 5.1).
 *
 *   mc_ms_feat         device [bs, num_feat, C], feat_dtype.  Level (k, s) occupies rows
 *                      scale_start_index[k,s] .. + H*W - 1 of each batch image, row-major
 *                      (H, W), C contiguous channels per row.  Element aligned; 16-byte
 *                      alignment with C and C/G multiples of 16 bytes' worth of elements
 *                      enables 16-byte vector loads.
 *   spatial_shape      HOST int32 [K, S, 2]: (H, W) of each level, 1 <= H, W <= DA_MAX_EXTENT.
 *   scale_start_index  HOST int32 [K, S]: first row of each level; start + H*W <= num_feat.
 *   sampling_location  device float [bs, A, P, K, 2], normalised (x, y); 8-byte aligned.
 *   weights            device float [bs, A, P, K, S, G]; 4-byte aligned.
 *   out                device [bs, A, C] of out_dtype, fully overwritten; element aligned.
 *   workspace          NULL, or device scratch of at least da_forward_workspace_size()
 *                      bytes, 256-byte aligned, owned by the caller (contents on entry do
 *                      not matter; garbage on return).  With NULL the forward always runs
 *                      one workgroup per anchor; with a workspace it uses level slices
 *                      when they are wanted.  Overlapping calls must not share it.
 *
 * Returns DA_OK, DA_ERR_INVALID_ARG (null pointer where data is needed, misaligned
 * pointer, malformed sizes, flags or level table, a misaligned or too small
 * workspace), DA_ERR_UNSUPPORTED (one batch image of the
 * features -- or, in the backward, of the feature gradient -- plus two rows above
 * 2^32 - 1 bytes; num_embeds > 2^20; bs * A * 512 >= 2^32; one (point, camera) pair's
 * stencils and weights above 48 KiB of LDS; in the backward, num_embeds above 1024 or
 * more than 16 times the largest power of two dividing C / G, capped at 64) or
 * DA_ERR_HIP.
 */
DA_API da_status da_forward(const da_problem* problem,
                     const void* mc_ms_feat,
                     const int32_t* spatial_shape,
                     const int32_t* scale_start_index,
                     const float* sampling_location,
                     const float* weights,
                     void* out,
                     void* workspace,
                     size_t workspace_bytes,
                     void* stream);

/*
 * da_backward_workspace_size -- bytes of device workspace da_backward and
 * da_backward_accumulate need for `problem` (0 when there is no sample): about
 * 8 * bs * num_feat + (88 + 16 * G) * bs*A*P*K*S where the row-ordered backward
 * may apply, else 8 * bs * num_feat + 88 * bs*A*P*K*S; with DA_FLAG_DETERMINISTIC
 * another (8 * C + 4) * (4 * bs*A*P*K*S / 65 + 1) + 8 * bs*K*S * ceil(A*P / 256);
 * with a 16-bit out_dtype another 4 * bs*A*C (grad_out converted to binary32).
 * Only the sizes and flags in `problem` are read.  Returns DA_ERR_UNSUPPORTED when bs * num_feat
 * >= 2^31, the sample count bs*A*P*K*S >= 2^29, or grad_out or weights exceed
 * 2^32 - 1 bytes (da_backward_atomic still works).
 */
DA_API da_status da_backward_workspace_size(const da_problem* problem, size_t* bytes);

/*
 * da_backward -- the backward pass (section 4.1).  Same inputs as da_forward, plus
 *
 *   grad_out           device [bs, A, C] of out_dtype; element aligned.
 *   grad_feat          device float [bs, num_feat, C] (binary32 also for 16-bit features):
 *                      fully overwritten (rows no sample touches are zero); 4-byte aligned.
 *   grad_loc           device float [bs, A, P, K, 2], fully overwritten; 8-byte aligned.
 *   grad_weights       device float [bs, A, P, K, S, G], fully overwritten.
 *   workspace          device scratch of at least da_backward_workspace_size() bytes,
 *                      256-byte aligned, owned by the caller; its contents on entry do
 *                      not matter and are garbage on return.  May be NULL when the size
 *                      is 0.  Calls that overlap in time must not share a workspace.
 *
 * The feature gradient is formed as a gather: every (sample, corner) term is first
 * bucketed by feature row, then each row is summed by one wave and stored, so almost
 * no floating-point atomics are issued.  The per-anchor pass uses level slices when
 * they are wanted (see DA_FLAG_SLICES_ALWAYS); the workspace then also holds every
 * sample's location-gradient partial.  The order in which a row's terms are added
 * depends on the order integer atomics retire in, so grad_feat may differ in rounding
 * from run to run; grad_loc and grad_weights are deterministic.
 * Same errors as da_forward, plus DA_ERR_INVALID_ARG for a missing, misaligned or too
 * small workspace and the DA_ERR_UNSUPPORTED cases of da_backward_workspace_size.
 */
DA_API da_status da_backward(const da_problem* problem,
                      const void* mc_ms_feat,
                      const int32_t* spatial_shape,
                      const int32_t* scale_start_index,
                      const float* sampling_location,
                      const float* weights,
                      const void* grad_out,
                      float* grad_feat,
                      float* grad_loc,
                      float* grad_weights,
                      void* workspace,
                      size_t workspace_bytes,
                      void* stream);

/*
 * da_backward_accumulate -- as da_backward, except that grad_feat is NOT overwritten:
 * the feature gradient is added to what grad_feat already holds (for several
 * aggregations that read one feature map, or a caller that keeps a running gradient).
 * grad_loc and grad_weights are still overwritten.  Same arguments and errors.
 */
DA_API da_status da_backward_accumulate(const da_problem* problem,
                                 const void* mc_ms_feat,
                                 const int32_t* spatial_shape,
                                 const int32_t* scale_start_index,
                                 const float* sampling_location,
                                 const float* weights,
                                 const void* grad_out,
                                 float* grad_feat,
                                 float* grad_loc,
                                 float* grad_weights,
                                 void* workspace,
                                 size_t workspace_bytes,
                                 void* stream);

/*
 * da_backward_atomic -- the backward pass in the page's scatter form, with no
 * workspace: grad_feat is zero-filled, then every (sample, corner, channel) term is
 * added with a binary32 atomic (section 4.1 adds them the same way).  Results equal
 * da_backward's up to rounding; it is slower wherever atomics are the bottleneck.
 * Arguments as da_backward without the workspace; same errors as da_forward, and
 * DA_ERR_UNSUPPORTED with DA_FLAG_DETERMINISTIC.
 */
DA_API da_status da_backward_atomic(const da_problem* problem,
                             const void* mc_ms_feat,
                             const int32_t* spatial_shape,
                             const int32_t* scale_start_index,
                             const float* sampling_location,
                             const float* weights,
                             const void* grad_out,
                             float* grad_feat,
                             float* grad_loc,
                             float* grad_weights,
                             void* stream);

/*
 * da_backward_noalloc -- for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): da_backward
 * with its workspace taken from a fixed array of DA_NOALLOC_SCRATCH_BYTES inside the
 * library's code object instead of from the caller.  The call allocates and frees
 * nothing.  Every GPU the library runs on holds its own copy of the array until the
 * process ends; its device address is looked up on the first call on each device.
 *
 * Arguments as da_backward without workspace / workspace_bytes; grad_feat, grad_loc and
 * grad_weights are fully overwritten.  Every call on one GPU shares that GPU's array,
 * whose contents a call leaves behind (nothing in it needs to start at zero): calls
 * that overlap in time on one GPU -- on different streams or threads -- race, and the
 * caller must serialise them.  Returns da_backward's errors, plus DA_ERR_UNSUPPORTED
 * (checked after the arguments, before anything is enqueued) when
 * da_backward_workspace_size reports more than DA_NOALLOC_SCRATCH_BYTES for the problem
 * -- enough for the nuScenes-shaped
 * problem (6 cameras, 4 scales from 64x176, C = 256, 900 anchors, 13 points) in every
 * backward form, deterministic included -- and DA_ERR_HIP if the array's device
 * address cannot be found.
 */
#define DA_NOALLOC_SCRATCH_BYTES (96ull << 20)   /* 96 MiB per device */

DA_API da_status da_backward_noalloc(const da_problem* problem,
                              const void* mc_ms_feat,
                              const int32_t* spatial_shape,
                              const int32_t* scale_start_index,
                              const float* sampling_location,
                              const float* weights,
                              const void* grad_out,
                              float* grad_feat,
                              float* grad_loc,
                              float* grad_weights,
                              void* stream);

/*
 * Level packing -- section 6 of the walkthrough: feature_maps_format turns the list of
 * per-scale camera feature maps into the flattened tensor the aggregation reads (plus
 * its level table), and back.  The page prints this step only in garbled form; the
 * library takes the layout of section 3.1: each level HWC, levels camera-major, scales
 * in order inside a camera.  Level (k, s) starts at row
 *     k * sum_s' H_s' W_s'  +  sum_{s' < s} H_s' W_s'.
 * Packing is a pure rearrangement: values are copied bit for bit.
 */
typedef struct {
    int64_t bs;           /* B                                               */
    int64_t num_cams;     /* N, cameras; num_cams * num_scale <= DA_MAX_LEVELS */
    int64_t num_scale;    /* S                                               */
    int64_t num_embeds;   /* C                                               */
    int32_t dtype;        /* da_dtype of the maps and of the packed tensor   */
    int32_t reserved;     /* must be 0                                       */
} da_pack_problem;

/*
 * da_pack_layout -- host only.  scale_hw: HOST int32 [S, 2], (H_s, W_s) of scale s
 * (the same for every camera).  Writes spatial_shape HOST int32 [N, S, 2],
 * scale_start_index HOST int32 [N, S] and *num_feat (rows of one packed batch image)
 * -- the level table da_forward / da_backward take.  Errors: DA_ERR_INVALID_ARG for
 * NULL pointers or malformed sizes, DA_ERR_UNSUPPORTED when num_feat >= 2^31 or
 * bs * num_cams > 65535.
 */
DA_API da_status da_pack_layout(const da_pack_problem* problem, const int32_t* scale_hw,
                         int32_t* spatial_shape, int32_t* scale_start_index, int64_t* num_feat);

/*
 * da_pack_levels -- packed[b, row(k, s) + i*W_s + j, c] = maps[s][b, k, c, i, j].
 *   maps     HOST array of S device pointers; maps[s] is [B, N, C, H_s, W_s], contiguous,
 *            element aligned.
 *   packed   device [B, num_feat, C], fully overwritten; element aligned.
 * Asynchronous on `stream`.  Same errors as da_pack_layout, plus DA_ERR_INVALID_ARG for
 * NULL or misaligned tensors and DA_ERR_HIP.
 */
DA_API da_status da_pack_levels(const da_pack_problem* problem, const int32_t* scale_hw,
                         const void* const* maps, void* packed, void* stream);

/*
 * da_unpack_levels -- the inverse: maps[s][b, k, c, i, j] = packed[b, row(k, s) + i*W_s + j, c]
 * (every element of every map overwritten).  Used for the gradient of the packing:
 * it carries d loss / d packed back to the per-scale maps.  Arguments and errors as
 * da_pack_levels.
 */
DA_API da_status da_unpack_levels(const da_pack_problem* problem, const int32_t* scale_hw,
                           const void* packed, void* const* maps, void* stream);

/* Static description of a status code. */
DA_API const char* da_status_string(da_status status);

/* Message of the last failed call on the calling thread ("" if none). */
DA_API const char* da_last_error(void);

/* DA_VERSION of the built library. */
DA_API int32_t da_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DEFORMAGG_H */
