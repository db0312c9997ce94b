/*
 * Plain fp64 CPU oracle for deformable convolution (DCNv3 / DCNv4 operator).
 *
 * TEST INFRASTRUCTURE ONLY.  Tests, the smoke check and the benchmark's CPU
 * baseline call this code to check and to time the GPU library; nothing in
 * the product path links, loads or calls it.  It shares no code, header or
 * constant with the HIP library.
 *
 * Source of the definition: the DCNv4 paper notes (docsaid.org, "DCNv4"):
 *   section "Defining the problem" -- output of group g at position p0 is the
 *     sum over the K points p_k of a 3 x 3 grid (K = 9) of the modulation
 *     scalar m_gk times the input of group g sampled at p0 + p_k + dp_gk; the
 *     offsets dp_gk and the scalars m_gk are per position and per group, and
 *     every one of the D = C / G channels of a group shares them; sampling at
 *     a fractional position is bilinear over the 4 surrounding pixels; input
 *     and output are H x W x C;
 *   section "Removing softmax" -- DCNv4 takes m_gk as any real number (no
 *     softmax over the K points: that is a model choice, outside the op);
 *   section "Moving less data" -- channel-last memory, channels of a pixel
 *     contiguous.
 *
 * Readings taken where the page leaves a step open (each one is a named point
 * in the design notes of the repository):
 *   - the grid generalises to kernel_h x kernel_w taps with stride, padding and
 *     dilation: output pixel (ho, wo) has p0 = (ho*stride_h - pad_h,
 *     wo*stride_w - pad_w) and tap k = i*kernel_w + j adds (i*dil_h, j*dil_w);
 *     the output is Ho x Wo with Ho = (H + 2 pad_h - dil_h (kernel_h - 1) - 1)
 *     / stride_h + 1 (same for W).  Kernel 3, stride 1, pad 1, dilation 1 gives
 *     the page's 3 x 3 neighbourhood and an output the size of the input;
 *   - positions are in pixels, pixel (y, x) at integer coordinates; the
 *     sampling position is (p0_y + i dil_h) + dy and (p0_x + j dil_w) + dx in
 *     binary32 (one rounding each), as the kernel computes it: floor() of it
 *     picks the cell, so both sides must take that integer decision in the same
 *     precision.  Everything after it is fp64;
 *   - bilinear weights as for any bilinear sampling: with fractions ly, lx of
 *     the position over its low corner, corners (low,low), (low,high),
 *     (high,low), (high,high) in (y, x) order weigh (1-ly)(1-lx), (1-ly)lx,
 *     ly(1-lx), ly lx; a corner outside the image reads zero, and a position
 *     with y <= -1, y >= H, x <= -1 or x >= W (all corners outside, or NaN)
 *     contributes nothing;
 *   - offset_mask is one tensor [N, Ho, Wo, G, 3K] (DCNv4 computes offsets and
 *     scalars with one linear layer): for group g, (dx_k, dy_k) for k = 0..K-1
 *     (x along the width), then m_0 .. m_{K-1};
 *   - channel c belongs to group c / D.
 *
 * Gradients (the derivatives of that definition): with v1..v4 the corner
 * values of one channel and go its output gradient,
 *   grad_input[corner] += cw[corner] * m * go,
 *   grad_m            += go * sum_corners cw * v,
 *   grad_dx           += m * go * (-(1-ly) v1 + (1-ly) v2 - ly v3 + ly v4),
 *   grad_dy           += m * go * (-(1-lx) v1 - lx v2 + (1-lx) v3 + lx v4),
 * the last three summed over the D channels of the group.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (with oracle.c) -lm.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t N, H, W, C, G, KH, KW, SH, SW, PH, PW, DH, DW;
    int64_t Ho, Wo, K, D;
} dcn_problem;

typedef struct {
    int inside;
    int64_t y[4], x[4];    /* corner pixel, or -1 when outside the image */
    double ly, lx;
    double cw[4];
} dcn_stencil;

static int dcn_setup(dcn_problem* p) {
    if (p->N < 0 || p->H < 1 || p->W < 1 || p->C < 1 || p->G < 1 || p->C % p->G != 0 ||
        p->KH < 1 || p->KW < 1 || p->SH < 1 || p->SW < 1 || p->PH < 0 || p->PW < 0 ||
        p->DH < 1 || p->DW < 1)
        return 1;
    p->Ho = (p->H + 2 * p->PH - p->DH * (p->KH - 1) - 1) / p->SH + 1;
    p->Wo = (p->W + 2 * p->PW - p->DW * (p->KW - 1) - 1) / p->SW + 1;
    if (p->Ho < 1 || p->Wo < 1) return 2;
    p->K = p->KH * p->KW;
    p->D = p->C / p->G;
    return 0;
}

/* binary32 sampling position: an integer grid position (exact in binary32 for
 * the sizes allowed) plus the offset, rounded once */
static float sample_pos(int64_t grid, float off) {
    volatile float s = (float)grid + off;
    return s;
}

static dcn_stencil dcn_make_stencil(const dcn_problem* p, int64_t ho, int64_t wo, int64_t k,
                                    float dx, float dy) {
    dcn_stencil st;
    memset(&st, 0, sizeof st);
    const int64_t i = k / p->KW, j = k % p->KW;
    const float yf = sample_pos(ho * p->SH - p->PH + i * p->DH, dy);
    const float xf = sample_pos(wo * p->SW - p->PW + j * p->DW, dx);
    if (!(yf > -1.0f && xf > -1.0f && yf < (float)p->H && xf < (float)p->W)) return st;
    st.inside = 1;
    const double y = (double)yf, x = (double)xf;
    const double y0 = floor(y), x0 = floor(x);
    st.ly = y - y0;
    st.lx = x - x0;
    const int64_t ylo = (int64_t)y0, xlo = (int64_t)x0;
    const int64_t ys[4] = {ylo, ylo, ylo + 1, ylo + 1};
    const int64_t xs[4] = {xlo, xlo + 1, xlo, xlo + 1};
    const double hy = 1.0 - st.ly, hx = 1.0 - st.lx;
    const double cw[4] = {hy * hx, hy * st.lx, st.ly * hx, st.ly * st.lx};
    for (int c = 0; c < 4; ++c) {
        const int in = ys[c] >= 0 && ys[c] < p->H && xs[c] >= 0 && xs[c] < p->W;
        st.y[c] = in ? ys[c] : -1;
        st.x[c] = in ? xs[c] : -1;
        st.cw[c] = cw[c];
    }
    return st;
}

static double in_at(const dcn_problem* p, const float* input, int64_t n, const dcn_stencil* st,
                    int corner, int64_t c) {
    if (st->y[corner] < 0) return 0.0;
    return (double)input[((n * p->H + st->y[corner]) * p->W + st->x[corner]) * p->C + c];
}

#define DCN_ARGS                                                                              \
    int64_t N, int64_t H, int64_t W, int64_t C, int64_t G, int64_t KH, int64_t KW, int64_t SH, \
        int64_t SW, int64_t PH, int64_t PW, int64_t DH, int64_t DW
#define DCN_INIT                                                                 \
    dcn_problem p = {N, H, W, C, G, KH, KW, SH, SW, PH, PW, DH, DW, 0, 0, 0, 0}; \
    const int rc = dcn_setup(&p);                                                \
    if (rc) return rc;

/* out [N, Ho, Wo, C] */
int oracle_dcn_forward(DCN_ARGS, const float* input, const float* offset_mask, double* out) {
    DCN_INIT
    for (int64_t n = 0; n < p.N; ++n)
        for (int64_t ho = 0; ho < p.Ho; ++ho)
            for (int64_t wo = 0; wo < p.Wo; ++wo) {
                const int64_t pix = (n * p.Ho + ho) * p.Wo + wo;
                double* o = out + pix * p.C;
                for (int64_t c = 0; c < p.C; ++c) o[c] = 0.0;
                for (int64_t g = 0; g < p.G; ++g) {
                    const float* om = offset_mask + (pix * p.G + g) * 3 * p.K;
                    for (int64_t k = 0; k < p.K; ++k) {
                        const dcn_stencil st =
                            dcn_make_stencil(&p, ho, wo, k, om[2 * k], om[2 * k + 1]);
                        if (!st.inside) continue;
                        const double m = (double)om[2 * p.K + k];
                        for (int64_t d = 0; d < p.D; ++d) {
                            const int64_t c = g * p.D + d;
                            double v = 0.0;
                            for (int q = 0; q < 4; ++q) v += st.cw[q] * in_at(&p, input, n, &st, q, c);
                            o[c] += m * v;
                        }
                    }
                }
            }
    return 0;
}

/* grad_input [N, H, W, C] (overwritten), grad_offset_mask [N, Ho, Wo, G, 3K] */
int oracle_dcn_backward(DCN_ARGS, const float* input, const float* offset_mask,
                        const float* grad_out, double* grad_input, double* grad_offset_mask) {
    DCN_INIT
    memset(grad_input, 0, sizeof(double) * (size_t)(p.N * p.H * p.W * p.C));
    for (int64_t n = 0; n < p.N; ++n)
        for (int64_t ho = 0; ho < p.Ho; ++ho)
            for (int64_t wo = 0; wo < p.Wo; ++wo) {
                const int64_t pix = (n * p.Ho + ho) * p.Wo + wo;
                const float* go = grad_out + pix * p.C;
                for (int64_t g = 0; g < p.G; ++g) {
                    const float* om = offset_mask + (pix * p.G + g) * 3 * p.K;
                    double* gom = grad_offset_mask + (pix * p.G + g) * 3 * p.K;
                    for (int64_t k = 0; k < p.K; ++k) {
                        gom[2 * k] = gom[2 * k + 1] = gom[2 * p.K + k] = 0.0;
                        const dcn_stencil st =
                            dcn_make_stencil(&p, ho, wo, k, om[2 * k], om[2 * k + 1]);
                        if (!st.inside) continue;
                        const double m = (double)om[2 * p.K + k];
                        const double hy = 1.0 - st.ly, hx = 1.0 - st.lx;
                        double gm = 0.0, gx = 0.0, gy = 0.0;
                        for (int64_t d = 0; d < p.D; ++d) {
                            const int64_t c = g * p.D + d;
                            const double gv = (double)go[c];
                            double v[4];
                            for (int q = 0; q < 4; ++q) v[q] = in_at(&p, input, n, &st, q, c);
                            gm += gv * (st.cw[0] * v[0] + st.cw[1] * v[1] + st.cw[2] * v[2] +
                                        st.cw[3] * v[3]);
                            gx += gv * (-hy * v[0] + hy * v[1] - st.ly * v[2] + st.ly * v[3]);
                            gy += gv * (-hx * v[0] - st.lx * v[1] + hx * v[2] + st.lx * v[3]);
                            for (int q = 0; q < 4; ++q) {
                                if (st.y[q] < 0) continue;
                                grad_input[((n * p.H + st.y[q]) * p.W + st.x[q]) * p.C + c] +=
                                    st.cw[q] * m * gv;
                            }
                        }
                        gom[2 * k] = m * gx;
                        gom[2 * k + 1] = m * gy;
                        gom[2 * p.K + k] = gm;
                    }
                }
            }
    return 0;
}

/* output size, for the caller's allocations */
int oracle_dcn_out_size(DCN_ARGS, int64_t* ho, int64_t* wo) {
    DCN_INIT
    *ho = p.Ho;
    *wo = p.Wo;
    return 0;
}
