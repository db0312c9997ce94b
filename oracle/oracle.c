/*
 * Plain fp64 CPU oracle for Sparse4D-style deformable aggregation.
 *
 * TEST INFRASTRUCTURE ONLY.  Tests, the smoke check and the benchmark's CPU
 * baseline call this code to check and to time the GPU library; nothing in
 * the product path links, loads or calls it.  It shares no code, header or
 * constant with the HIP library.
 *
 * Source of the definition: the Sparse4D deformable_aggregation walkthrough
 * (mhpn.cn/news/1081857):
 *   section 3.1  HWC layout: element (i, j, k) sits at i*W*C + j*C + k;
 *   section 3.2  bilinear sampling: floor to the low corner, the high corner
 *                is one further, fractions lh, lw and their complements
 *                hh = 1 - lh, hw = 1 - lw, four corner products, a corner
 *                outside the map reads zero;
 *   section 4.1  backward: the feature gradient adds corner weight x
 *                grad_out x weight into each corner; the location gradient
 *                is width * (lh (v4 - v3) + hh (v2 - v1)) * top for x and
 *                height * (lw (v4 - v2) + hw (v3 - v1)) * top for y; the
 *                weight gradient adds grad_out x sampled value;
 *   section 5.1  the six work dimensions batch x points x channels x
 *                anchors x cameras x scales, summed into out[b, a, c].
 *
 * Readings taken where the page leaves a step open (each one is a named
 * point in the design notes of the repository):
 *   - normalised (x, y) maps to pixel coordinates w = x*W - 0.5,
 *     h = y*H - 0.5 (pixel centres at (j + 0.5)/W); the page fixes the
 *     factor W by the location gradient, the -0.5 is the offset under which
 *     the op equals grid_sample(align_corners=False, padding zeros);
 *   - that pixel coordinate is computed in binary32, two roundings, exactly
 *     as the kernel does: floor() of it picks the cell, and both sides must
 *     take that integer decision in the same precision.  Everything after
 *     it is fp64;
 *   - a sample contributes only when -1 < h < H and -1 < w < W;
 *   - channel c belongs to group c / (C / G);
 *   - location component 0 is x (width), component 1 is y (height).
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared oracle.c -o liboracle.so -lm
 * (no fast-math: the binary32 pixel coordinate must be rounded twice).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* One bilinear stencil: the four corners (low/low, low/high, high/low,
 * high/high in (h, w) order, as in section 3.2), each either a row of the
 * flattened feature tensor or -1 when outside the level. */
typedef struct {
    int inside;          /* 0: the sample is skipped entirely */
    int64_t row[4];      /* absolute row within one batch image, or -1 */
    double lh, lw, hh, hw;
    double cw[4];        /* hh*hw, hh*lw, lh*hw, lh*lw */
} stencil;

/* binary32 pixel coordinate; see the header for why it is not fp64 */
static float pixel_coord(float u, int32_t extent) {
    volatile float prod = u * (float)extent;
    volatile float shifted = prod - 0.5f;
    return shifted;
}

static stencil make_stencil(float x, float y, int32_t H, int32_t W, int64_t start) {
    stencil st;
    memset(&st, 0, sizeof st);
    st.row[0] = st.row[1] = st.row[2] = st.row[3] = -1;
    const float w_im = pixel_coord(x, W);
    const float h_im = pixel_coord(y, H);
    if (!(h_im > -1.0f && w_im > -1.0f && h_im < (float)H && w_im < (float)W))
        return st;
    st.inside = 1;
    const double hd = (double)h_im, wd = (double)w_im;
    const double hlf = floor(hd), wlf = floor(wd);
    const int64_t h_low = (int64_t)hlf, w_low = (int64_t)wlf;
    const int64_t h_high = h_low + 1, w_high = w_low + 1;
    st.lh = hd - hlf;
    st.lw = wd - wlf;
    st.hh = 1.0 - st.lh;
    st.hw = 1.0 - st.lw;
    const int64_t hs[4] = {h_low, h_low, h_high, h_high};
    const int64_t ws[4] = {w_low, w_high, w_low, w_high};
    for (int i = 0; i < 4; ++i) {
        if (hs[i] >= 0 && hs[i] <= H - 1 && ws[i] >= 0 && ws[i] <= W - 1)
            st.row[i] = start + hs[i] * (int64_t)W + ws[i];
    }
    st.cw[0] = st.hh * st.hw;
    st.cw[1] = st.hh * st.lw;
    st.cw[2] = st.lh * st.hw;
    st.cw[3] = st.lh * st.lw;
    return st;
}

/* Exact widening of a stored feature element to fp64. */
static double feat_at(const void* feat, int feat_is_bf16, int64_t idx) {
    if (feat_is_bf16) {
        const uint16_t bits = ((const uint16_t*)feat)[idx];
        const uint32_t w = (uint32_t)bits << 16;
        float f;
        memcpy(&f, &w, sizeof f);
        return (double)f;
    }
    return (double)((const float*)feat)[idx];
}

typedef struct {
    int64_t bs, num_feat, C, A, P, K, S, G;
    const void* feat;
    int feat_is_bf16;
    const int32_t* spatial_shape;      /* [K, S, 2] (H, W) */
    const int32_t* scale_start_index;  /* [K, S] */
    const float* loc;                  /* [bs, A, P, K, 2] */
    const float* weights;              /* [bs, A, P, K, S, G] */
} problem;

static int check_problem(const problem* pb) {
    if (pb->bs < 0 || pb->A < 0 || pb->P < 0 || pb->K < 1 || pb->S < 1 || pb->C < 1 ||
        pb->G < 1 || pb->num_feat < 1)
        return 1;
    if (pb->C % pb->G != 0) return 1;
    for (int64_t l = 0; l < pb->K * pb->S; ++l) {
        const int64_t H = pb->spatial_shape[2 * l], W = pb->spatial_shape[2 * l + 1];
        const int64_t st = pb->scale_start_index[l];
        if (H < 1 || W < 1 || st < 0 || st + H * W > pb->num_feat) return 1;
    }
    return 0;
}

static stencil stencil_for(const problem* pb, int64_t b, int64_t a, int64_t p, int64_t k,
                           int64_t s) {
    const int64_t l = k * pb->S + s;
    const int32_t H = pb->spatial_shape[2 * l], W = pb->spatial_shape[2 * l + 1];
    const float* xy = pb->loc + ((((b * pb->A + a) * pb->P + p) * pb->K + k) * 2);
    return make_stencil(xy[0], xy[1], H, W, pb->scale_start_index[l]);
}

static double corner_value(const problem* pb, const stencil* st, int i, int64_t b, int64_t c) {
    if (st->row[i] < 0) return 0.0;
    return feat_at(pb->feat, pb->feat_is_bf16, (b * pb->num_feat + st->row[i]) * pb->C + c);
}

/* out[b, a, c] = sum over p, k, s of weights[b,a,p,k,s,g(c)] * bilinear(c) */
static void forward_anchor(const problem* pb, int64_t b, int64_t a, double* out_row) {
    const int64_t D = pb->C / pb->G;
    for (int64_t c = 0; c < pb->C; ++c) out_row[c] = 0.0;
    for (int64_t p = 0; p < pb->P; ++p)
        for (int64_t k = 0; k < pb->K; ++k)
            for (int64_t s = 0; s < pb->S; ++s) {
                const stencil st = stencil_for(pb, b, a, p, k, s);
                if (!st.inside) continue;
                const float* w = pb->weights +
                    ((((b * pb->A + a) * pb->P + p) * pb->K + k) * pb->S + s) * pb->G;
                for (int64_t c = 0; c < pb->C; ++c) {
                    double val = 0.0;
                    for (int i = 0; i < 4; ++i) val += st.cw[i] * corner_value(pb, &st, i, b, c);
                    out_row[c] += (double)w[c / D] * val;
                }
            }
}

/* All three gradients contributed by anchor (b, a).  grad_feat_add(b, row,
 * c, value) receives every feature-gradient term; the per-anchor location
 * and weight gradients are written to gl [P,K,2] and gw [P,K,S,G]. */
typedef void (*feat_sink)(void* ctx, int64_t b, int64_t row, int64_t c, double v);

static void backward_anchor(const problem* pb, int64_t b, int64_t a, const float* grad_out,
                            double* gl, double* gw, feat_sink sink, void* ctx) {
    const int64_t D = pb->C / pb->G;
    const float* go = grad_out + (b * pb->A + a) * pb->C;
    if (gl) memset(gl, 0, sizeof(double) * (size_t)(pb->P * pb->K * 2));
    if (gw) memset(gw, 0, sizeof(double) * (size_t)(pb->P * pb->K * pb->S * pb->G));
    for (int64_t p = 0; p < pb->P; ++p)
        for (int64_t k = 0; k < pb->K; ++k)
            for (int64_t s = 0; s < pb->S; ++s) {
                const stencil st = stencil_for(pb, b, a, p, k, s);
                if (!st.inside) continue;
                const int64_t l = k * pb->S + s;
                const double H = pb->spatial_shape[2 * l], W = pb->spatial_shape[2 * l + 1];
                const int64_t widx = (((b * pb->A + a) * pb->P + p) * pb->K + k) * pb->S + s;
                const float* w = pb->weights + widx * pb->G;
                for (int64_t c = 0; c < pb->C; ++c) {
                    const int64_t g = c / D;
                    const double v1 = corner_value(pb, &st, 0, b, c);
                    const double v2 = corner_value(pb, &st, 1, b, c);
                    const double v3 = corner_value(pb, &st, 2, b, c);
                    const double v4 = corner_value(pb, &st, 3, b, c);
                    const double top = (double)go[c] * (double)w[g];
                    if (sink)
                        for (int i = 0; i < 4; ++i)
                            if (st.row[i] >= 0) sink(ctx, b, st.row[i], c, st.cw[i] * top);
                    if (gl) {
                        const double gx = st.lh * (v4 - v3) + st.hh * (v2 - v1);
                        const double gy = st.lw * (v4 - v2) + st.hw * (v3 - v1);
                        gl[(p * pb->K + k) * 2 + 0] += W * gx * top;
                        gl[(p * pb->K + k) * 2 + 1] += H * gy * top;
                    }
                    if (gw) {
                        const double val = st.cw[0] * v1 + st.cw[1] * v2 + st.cw[2] * v3 +
                                           st.cw[3] * v4;
                        gw[((p * pb->K + k) * pb->S + s) * pb->G + g] += (double)go[c] * val;
                    }
                }
            }
}

/* ---- feature-gradient sinks ---------------------------------------------------- */

typedef struct { double* gf; int64_t num_feat, C; } dense_sink_ctx;

static void dense_sink(void* vctx, int64_t b, int64_t row, int64_t c, double v) {
    dense_sink_ctx* ctx = (dense_sink_ctx*)vctx;
    ctx->gf[(b * ctx->num_feat + row) * ctx->C + c] += v;
}

/* rows selected by the caller: slot[b*num_feat + row] = output row or -1 */
typedef struct { double* gf; const int64_t* slot; int64_t num_feat, C; } rows_sink_ctx;

static void rows_sink(void* vctx, int64_t b, int64_t row, int64_t c, double v) {
    rows_sink_ctx* ctx = (rows_sink_ctx*)vctx;
    const int64_t o = ctx->slot[b * ctx->num_feat + row];
    if (o >= 0) ctx->gf[o * ctx->C + c] += v;
}

/* ---- exported entry points -------------------------------------------------------- */

#define ORACLE_PROBLEM_ARGS                                                                 \
    int64_t bs, int64_t num_feat, int64_t C, int64_t A, int64_t P, int64_t K, int64_t S,   \
        int64_t G, const void *feat, int feat_is_bf16, const int32_t *spatial_shape,       \
        const int32_t *scale_start_index, const float *loc, const float *weights

#define ORACLE_FILL_PROBLEM(pb)                                                             \
    problem pb = {bs, num_feat, C, A, P, K, S, G, feat, feat_is_bf16, spatial_shape,       \
                  scale_start_index, loc, weights}

/* Forward.  anchor_ids (flat b*A + a) selects n_ids anchors, or NULL for all
 * bs*A in order.  out: [n, C] fp64.  Returns 0, or 1 on a malformed problem. */
int oracle_forward(ORACLE_PROBLEM_ARGS, const int64_t* anchor_ids, int64_t n_ids, double* out) {
    ORACLE_FILL_PROBLEM(pb);
    if (check_problem(&pb)) return 1;
    const int64_t n = anchor_ids ? n_ids : bs * A;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t id = anchor_ids ? anchor_ids[i] : i;
        if (id < 0 || id >= bs * A) return 1;
        forward_anchor(&pb, id / A, id % A, out + i * C);
    }
    return 0;
}

/* Forward of every anchor, spread over `threads` OpenMP threads by (b, a): each
 * anchor writes only its own out row, so the result equals oracle_forward's bit
 * for bit.  *threads_used receives the thread count of the parallel region.
 * Used only to time the definition on all host cores beside the one-thread loop. */
int oracle_forward_parallel(ORACLE_PROBLEM_ARGS, int threads, double* out, int* threads_used) {
    ORACLE_FILL_PROBLEM(pb);
    if (check_problem(&pb) || threads < 1) return 1;
    const int64_t n = bs * A;
    int used = 1;
#pragma omp parallel num_threads(threads)
    {
#pragma omp single
        used = omp_get_num_threads();
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < n; ++i) forward_anchor(&pb, i / A, i % A, out + i * C);
    }
    if (threads_used) *threads_used = used;
    return 0;
}

/* Full backward.  Any of grad_feat [bs,num_feat,C], grad_loc [bs,A,P,K,2],
 * grad_weights [bs,A,P,K,S,G] (all fp64) may be NULL to skip it. */
int oracle_backward(ORACLE_PROBLEM_ARGS, const float* grad_out, double* grad_feat,
                    double* grad_loc, double* grad_weights) {
    ORACLE_FILL_PROBLEM(pb);
    if (check_problem(&pb)) return 1;
    dense_sink_ctx dctx = {grad_feat, num_feat, C};
    if (grad_feat) memset(grad_feat, 0, sizeof(double) * (size_t)(bs * num_feat * C));
    for (int64_t b = 0; b < bs; ++b)
        for (int64_t a = 0; a < A; ++a)
            backward_anchor(&pb, b, a, grad_out,
                            grad_loc ? grad_loc + (b * A + a) * P * K * 2 : NULL,
                            grad_weights ? grad_weights + (b * A + a) * P * K * S * G : NULL,
                            grad_feat ? dense_sink : NULL, &dctx);
    return 0;
}

/* Location and weight gradients of selected anchors only:
 * grad_loc [n,P,K,2], grad_weights [n,P,K,S,G] (fp64). */
int oracle_backward_anchors(ORACLE_PROBLEM_ARGS, const float* grad_out, const int64_t* anchor_ids,
                            int64_t n_ids, double* grad_loc, double* grad_weights) {
    ORACLE_FILL_PROBLEM(pb);
    if (check_problem(&pb)) return 1;
    for (int64_t i = 0; i < n_ids; ++i) {
        const int64_t id = anchor_ids[i];
        if (id < 0 || id >= bs * A) return 1;
        backward_anchor(&pb, id / A, id % A, grad_out, grad_loc + i * P * K * 2,
                        grad_weights + i * P * K * S * G, NULL, NULL);
    }
    return 0;
}

/* Feature gradient of selected rows only (flat b*num_feat + row, distinct):
 * out [n_rows, C] fp64.  Visits every sample of every anchor. */
int oracle_grad_feat_rows(ORACLE_PROBLEM_ARGS, const float* grad_out, const int64_t* rows,
                          int64_t n_rows, double* out) {
    ORACLE_FILL_PROBLEM(pb);
    if (check_problem(&pb)) return 1;
    int64_t* slot = (int64_t*)malloc(sizeof(int64_t) * (size_t)(bs * num_feat));
    if (!slot) return 2;
    for (int64_t i = 0; i < bs * num_feat; ++i) slot[i] = -1;
    for (int64_t i = 0; i < n_rows; ++i) {
        if (rows[i] < 0 || rows[i] >= bs * num_feat || slot[rows[i]] >= 0) {
            free(slot);
            return 1;
        }
        slot[rows[i]] = i;
    }
    memset(out, 0, sizeof(double) * (size_t)(n_rows * C));
    rows_sink_ctx rctx = {out, slot, num_feat, C};
    /* the sink is only reached for valid corners, so walking the stencils of
     * every sample and skipping the per-channel work of samples that touch no
     * selected row gives the same sums as the dense backward */
    for (int64_t b = 0; b < bs; ++b)
        for (int64_t a = 0; a < A; ++a) {
            int touches = 0;
            for (int64_t p = 0; p < P && !touches; ++p)
                for (int64_t k = 0; k < K && !touches; ++k)
                    for (int64_t s = 0; s < S && !touches; ++s) {
                        const stencil st = stencil_for(&pb, b, a, p, k, s);
                        for (int i = 0; i < 4; ++i)
                            if (st.inside && st.row[i] >= 0 && slot[b * num_feat + st.row[i]] >= 0)
                                touches = 1;
                    }
            if (touches) backward_anchor(&pb, b, a, grad_out, NULL, NULL, rows_sink, &rctx);
        }
    free(slot);
    return 0;
}
