/*
 * dcn.h -- deformable convolution (the DCNv3 / DCNv4 operator) in libdeformagg.
 *
 * Definition: the DCNv4 paper notes (docsaid.org, "DCNv4"), section "Defining the
 * problem": the output of channel group g at output position p0 is the sum over the
 * K taps p_k of a kernel grid (3 x 3 there) of a modulation scalar m_gk times the
 * input of group g sampled bilinearly at p0 + p_k + dp_gk.  The offsets dp_gk and the
 * scalars m_gk belong to one output position and one group; the D = C / G channels
 * of a group share them.  Section "Removing softmax": the scalars are unbounded
 * (any normalisation is the model's business).  Section "Moving less data":
 * channels are the contiguous (last) dimension.
 *
 * Conventions taken where the page leaves a step open:
 *   - output pixel (ho, wo) has grid origin (ho*stride_h - pad_h, wo*stride_w - pad_w)
 *     and tap k = i*kernel_w + j adds (i*dilation_h, j*dilation_w); Ho =
 *     (H + 2 pad_h - dilation_h (kernel_h - 1) - 1) / stride_h + 1, Wo alike;
 *   - positions are in pixels (pixel (y, x) at integer coordinates); the sampling
 *     position y = (grid row) + dy and x = (grid column) + dx is formed in binary32;
 *     a corner outside the image reads zero and a position with y <= -1, y >= H,
 *     x <= -1 or x >= W (or NaN) contributes nothing;
 *   - offset_mask [N, Ho, Wo, G, 3K] float: for each group (dx_k, dy_k) for k = 0..K-1,
 *     x along the width, then m_0 .. m_{K-1} (one tensor, as DCNv4 produces offsets and
 *     scalars with one linear layer).
 *
 * Conventions of the library (see deformagg.h): the caller owns every buffer, calls
 * are asynchronous on `stream`, every check runs on the host before anything is
 * enqueued, da_last_error() names a failed check, arithmetic is binary32.
 */
#ifndef DCN_H
#define DCN_H

#include "deformagg.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Problem description.  batch may be 0 (nothing to do).  All other sizes >= 1 except
 * pad_* >= 0; channels % groups == 0; the output size must be >= 1. */
typedef struct {
    int64_t batch;        /* N                                                   */
    int64_t height;       /* H                                                   */
    int64_t width;        /* W                                                   */
    int64_t channels;     /* C                                                   */
    int64_t groups;       /* G: offsets and scalars per group of C / G channels  */
    int32_t kernel_h, kernel_w;
    int32_t stride_h, stride_w;
    int32_t pad_h, pad_w;
    int32_t dilation_h, dilation_w;
    int32_t in_dtype;     /* da_dtype of input                                   */
    int32_t out_dtype;    /* da_dtype of out (forward) and grad_out (backward)    */
    int32_t flags;        /* must be 0                                           */
    int32_t reserved;     /* must be 0                                           */
} dcn_problem;

/* dcn_out_size -- host only: the output height and width of `problem`.  Errors:
 * DA_ERR_INVALID_ARG for NULL pointers or malformed sizes. */
DA_API da_status dcn_out_size(const dcn_problem* problem, int64_t* out_h, int64_t* out_w);

/*
 * dcn_forward -- out[n, ho, wo, g*D + d] = sum_k m_gk * bilinear(input[n, :, :, g*D + d],
 * position of tap k).
 *   input        device [N, H, W, C] of in_dtype, channel-last, element aligned.
 *   offset_mask  device float [N, Ho, Wo, G, 3K], 4-byte aligned.
 *   out          device [N, Ho, Wo, C] of out_dtype, fully overwritten, element aligned.
 * Deterministic (no atomics).  Errors: DA_ERR_INVALID_ARG (NULL or misaligned pointer,
 * malformed problem), DA_ERR_UNSUPPORTED (input or its binary32 gradient, out as
 * binary32, or offset_mask of 2^32 bytes or more, C > 2^16, more than 2^31 output
 * pixels), DA_ERR_HIP.
 */
DA_API da_status dcn_forward(const dcn_problem* problem, const void* input, const float* offset_mask,
                      void* out, void* stream);

/*
 * dcn_backward_workspace_size -- bytes of device workspace dcn_backward needs:
 * 8448 + 16 * N*Ho*Wo*G*K (0 when there is no output pixel) -- control words, a
 * reduction buffer, and room to list every (sample, corner) whose offset carries it
 * more than 4 pixels past its tile.
 */
DA_API da_status dcn_backward_workspace_size(const dcn_problem* problem, size_t* bytes);

/*
 * dcn_backward -- the gradients of dcn_forward's definition.
 *   grad_out          device [N, Ho, Wo, C] of out_dtype, element aligned.
 *   grad_input        device float [N, H, W, C] (binary32 for every in_dtype), fully
 *                     overwritten; 4-byte aligned.
 *   grad_offset_mask  device float [N, Ho, Wo, G, 3K], fully overwritten: per group and
 *                     tap, m * sum_d grad_out * d(value)/dx, the same for y, and
 *                     sum_d grad_out * value; zero for taps that contribute nothing.
 *   workspace         device scratch of dcn_backward_workspace_size() bytes, 256-byte
 *                     aligned (may be NULL when that is 0); contents on entry do not
 *                     matter.
 * The input gradient is summed tile by tile in LDS by the workgroup that owns the
 * tile, in 64-bit fixed point (each term rounded once to a multiple of 2^-E, E from
 * max|grad_out| * max|m| and from the most terms one sum can take, so that no sum can
 * overflow: a resolution of 2^-46 to 2^-45 of that bound for a 56x56 output and a 3x3
 * kernel, finer for fewer output pixels), and stored once; only corners carried more
 * than 4 pixels past their tile are added afterwards with binary32 atomics.
 * grad_offset_mask is deterministic, and so is grad_input when no corner is that far.
 * Same errors as dcn_forward,
 * plus DA_ERR_UNSUPPORTED for 2^30 samples (N*Ho*Wo*G*K) or more and
 * DA_ERR_INVALID_ARG for a missing, misaligned or small workspace.
 */
DA_API da_status dcn_backward(const dcn_problem* problem, const void* input, const float* offset_mask,
                       const void* grad_out, float* grad_input, float* grad_offset_mask,
                       void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif /* DCN_H */
