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
 *   - The caller owns every buffer.  The library never allocates or frees device
 *     memory and keeps no state between calls; calls are asynchronous on `stream`
 *     and may be captured into a HIP graph.  Faults inside a kernel surface at the
 *     caller's next synchronisation.
 *   - All argument checks run on the host before anything is enqueued.  On any
 *     error no work is enqueued and no output is touched; da_last_error() returns
 *     a message naming the failed check (per calling thread).
 *   - Floating-point results are computed in binary32.  The forward pass is
 *     deterministic (no atomics).  The backward feature gradient is accumulated
 *     with binary32 atomic adds, so its rounding may differ from run to run.
 */
#ifndef DEFORMAGG_H
#define DEFORMAGG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DA_VERSION 100         /* 1.0.0 */
#define DA_MAX_LEVELS 64       /* num_cams * num_scale */
#define DA_MAX_EXTENT 32768    /* H and W of every level */

typedef enum {
    DA_OK = 0,
    DA_ERR_INVALID_ARG = 1,    /* a size, pointer or level entry is malformed */
    DA_ERR_UNSUPPORTED = 2,    /* well formed, but outside what the kernels handle */
    DA_ERR_HIP = 3             /* the HIP runtime refused a launch */
} da_status;

typedef enum {
    DA_F32 = 0,                /* mc_ms_feat holds float */
    DA_BF16 = 1                /* mc_ms_feat holds bfloat16 (raw 16-bit patterns) */
} da_dtype;

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
    int32_t feat_dtype;   /* da_dtype                                      */
    int32_t reserved;     /* must be 0                                     */
} da_problem;

/*
 * da_forward -- the forward pass (sections 3.2 and 5.1).
 *
 *   mc_ms_feat         device [bs, num_feat, C], feat_dtype.  Level (k, s) occupies rows
 *                      scale_start_index[k,s] .. + H*W - 1 of each batch image, row-major
 *                      (H, W), C contiguous channels per row.  16-byte aligned, and
 *                      C * element size must be a multiple of 4 bytes.
 *   spatial_shape      HOST int32 [K, S, 2]: (H, W) of each level, 1 <= H, W <= DA_MAX_EXTENT.
 *   scale_start_index  HOST int32 [K, S]: first row of each level; start + H*W <= num_feat.
 *   sampling_location  device float [bs, A, P, K, 2], normalised (x, y); 8-byte aligned.
 *   weights            device float [bs, A, P, K, S, G]; 4-byte aligned.
 *   out                device float [bs, A, C], fully overwritten; 16-byte aligned.
 *
 * Returns DA_OK, DA_ERR_INVALID_ARG (null pointer where data is needed, malformed
 * sizes or level table), DA_ERR_UNSUPPORTED (alignment, one batch image of the
 * features or of the feature gradient larger than 4 GiB - 64 KiB, grid limits) or
 * DA_ERR_HIP.
 */
da_status da_forward(const da_problem* problem,
                     const void* mc_ms_feat,
                     const int32_t* spatial_shape,
                     const int32_t* scale_start_index,
                     const float* sampling_location,
                     const float* weights,
                     float* out,
                     void* stream);

/*
 * da_backward -- the backward pass (section 4.1).  Same inputs as da_forward, plus
 *
 *   grad_out           device float [bs, A, C]; 4-byte aligned.
 *   grad_feat          device float [bs, num_feat, C] (binary32 also for bf16 features):
 *                      zeroed by the call, then accumulated; 16-byte aligned.
 *   grad_loc           device float [bs, A, P, K, 2], fully overwritten.
 *   grad_weights       device float [bs, A, P, K, S, G], fully overwritten.
 *
 * Rows of grad_feat that no sample touches come back as zero.  Same errors as
 * da_forward.
 */
da_status da_backward(const da_problem* problem,
                      const void* mc_ms_feat,
                      const int32_t* spatial_shape,
                      const int32_t* scale_start_index,
                      const float* sampling_location,
                      const float* weights,
                      const float* grad_out,
                      float* grad_feat,
                      float* grad_loc,
                      float* grad_weights,
                      void* stream);

/*
 * da_backward_accumulate -- as da_backward, except that grad_feat is NOT zeroed: the
 * feature gradient is added to what grad_feat already holds (for several
 * aggregations that read one feature map, or for a caller that keeps a
 * zero-initialised gradient buffer).  grad_loc and grad_weights are still
 * overwritten.  Same arguments and errors as da_backward.
 */
da_status da_backward_accumulate(const da_problem* problem,
                                 const void* mc_ms_feat,
                                 const int32_t* spatial_shape,
                                 const int32_t* scale_start_index,
                                 const float* sampling_location,
                                 const float* weights,
                                 const float* grad_out,
                                 float* grad_feat,
                                 float* grad_loc,
                                 float* grad_weights,
                                 void* stream);

/* Static description of a status code. */
const char* da_status_string(da_status status);

/* Message of the last failed call on the calling thread ("" if none). */
const char* da_last_error(void);

/* DA_VERSION of the built library. */
int32_t da_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DEFORMAGG_H */
