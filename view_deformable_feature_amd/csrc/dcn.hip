// Deformable convolution (the DCNv3 / DCNv4 operator) on MI355X.
//
// Definition followed: the DCNv4 paper notes (docsaid.org, "DCNv4"), section
// "Defining the problem": out(p0) of group g sums, over the K taps of the kernel
// grid, the modulation scalar m_gk times the group's input sampled bilinearly at
// p0 + p_k + dp_gk; the D = C / G channels of a group share dp_gk and m_gk.
// Section "Moving less data": channel-last memory.  The conventions for the grid,
// the position arithmetic and the offset_mask layout are stated in include/dcn.h.
//
// Design: the same gather building blocks as the aggregation (bounds-checked
// buffer loads whose out-of-range offset reads zero, 16-byte vectors over
// contiguous channels, DPP group sums).  A lane covers 16 bytes of one group's
// channels of one output pixel; the group's lanes share the stencil.  The
// backward recomputes the corner values for the offset and scalar gradients
// and scatters the input gradient with binary32 buffer atomics.  Blocks are
// laid out so that each XCD (workgroup i runs on XCD i mod 8) walks one
// contiguous band of output pixels, keeping the 3 x 3 neighbourhoods it reads
// in its own L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "da_device.h"
#include "dcn_internal.h"

namespace da {
namespace {

constexpr int kDcnThreads = 256;
constexpr int kDcnWaves = kDcnThreads / kWave;

// Logical block of hardware block b: XCD x (= b mod 8) takes the x-th
// contiguous share of the nb logical blocks.
__device__ __forceinline__ uint32_t xcd_order(uint32_t b, uint32_t nb) {
    const uint32_t per = nb / 8, rem = nb % 8, x = b % 8, i = b / 8;
    return x * per + min(x, rem) + i;
}

// One lane's view: the output pixel and, for each of its NV groups, the group
// and the first channel.
template <int VEC, int NV>
struct DcnLane {
    int64_t pix;
    int n, ho, wo;
    int g[NV];           // group (G and above: a lane slot past the last group)
    int gq[NV];          // the group whose offsets and scalars the lane reads (0 past G)
    int c0[NV];
    bool valid[NV];      // the vector exists (lanes past D / VEC idle)
    bool last[NV];       // last lane of its group (holds the DPP group sum)
};

template <int VEC, int NV>
__device__ __forceinline__ bool dcn_lane(const DcnArgs& a, DcnLane<VEC, NV>& L) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const uint32_t lb = xcd_order(blockIdx.x, gridDim.x);
    const int ppw = kWave >> a.log2Lp;
    L.pix = ((int64_t)lb * kDcnWaves + wave) * ppw + (lane >> a.log2Lp);
    if (L.pix >= a.n_pix) return false;
    const int64_t hw = (int64_t)a.Ho * a.Wo;
    L.n = (int)(L.pix / hw);
    const int r = (int)(L.pix - (int64_t)L.n * hw);
    L.ho = r / a.Wo;
    L.wo = r - L.ho * a.Wo;
    const int li = lane & (a.Lp - 1);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int s = li + a.Lp * i;
        const int j = s & (a.Lg - 1);
        L.g[i] = s >> a.log2Lg;
        L.gq[i] = L.g[i] < a.G ? L.g[i] : 0;
        L.valid[i] = L.g[i] < a.G && j < a.Dv;
        L.c0[i] = L.valid[i] ? L.g[i] * a.D + j * VEC : 0;
        L.last[i] = j == a.Lg - 1;
    }
    return true;
}

// Bilinear stencil of one (pixel, group, tap) sample: byte offsets of the four
// corners' VEC-channel vectors (the out-of-range offset for a corner outside the
// image) and their weights (all zero when the sample contributes nothing).
struct DcnStencil {
    uint32_t off[4];
    float cw[4];
    float ly, lx;
    bool inside;
};

__device__ __forceinline__ DcnStencil dcn_stencil(const DcnArgs& a, int n, int gy, int gx, float dy,
                                                  float dx, int c0, int elem) {
#pragma clang fp contract(off)
    DcnStencil st;
    const float y = (float)gy + dy;      // binary32 position, one rounding
    const float x = (float)gx + dx;
    st.inside = y > -1.0f && x > -1.0f && y < (float)a.H && x < (float)a.W;
    const float yf = st.inside ? floorf(y) : 0.0f;
    const float xf = st.inside ? floorf(x) : 0.0f;
    st.ly = st.inside ? y - yf : 0.0f;
    st.lx = st.inside ? x - xf : 0.0f;
    const float hy = 1.0f - st.ly, hx = 1.0f - st.lx;
    const int y0 = (int)yf, x0 = (int)xf;
    const bool in_y0 = y0 >= 0, in_y1 = y0 + 1 < a.H, in_x0 = x0 >= 0, in_x1 = x0 + 1 < a.W;
    const uint32_t base =
        (uint32_t)((((int64_t)n * a.H + y0) * a.W + x0) * a.C + c0) * (uint32_t)elem;
    const uint32_t row = (uint32_t)a.W * (uint32_t)a.C * (uint32_t)elem;
    const uint32_t col = (uint32_t)a.C * (uint32_t)elem;
    const uint32_t oor = a.in_bytes;
    st.off[0] = st.inside && in_y0 && in_x0 ? base : oor;
    st.off[1] = st.inside && in_y0 && in_x1 ? base + col : oor;
    st.off[2] = st.inside && in_y1 && in_x0 ? base + row : oor;
    st.off[3] = st.inside && in_y1 && in_x1 ? base + row + col : oor;
    st.cw[0] = st.inside ? hy * hx : 0.0f;
    st.cw[1] = st.inside ? hy * st.lx : 0.0f;
    st.cw[2] = st.inside ? st.ly * hx : 0.0f;
    st.cw[3] = st.inside ? st.ly * st.lx : 0.0f;
    return st;
}

template <int VEC>
__device__ __forceinline__ void store_out_vec(const DcnArgs& a, int64_t i, const float (&v)[VEC]) {
    void* out = a.out;
    const int dtype = a.out_dtype;
    if (dtype == kF32 && VEC == 4 && a.out_vec4) {
        *reinterpret_cast<float4*>(static_cast<float*>(out) + i) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) store_elem(out, i + e, v[e], dtype);
    }
}

template <typename T, int VEC, int NV>
__global__ void __launch_bounds__(kDcnThreads) dcn_forward_kernel(DcnArgs a) {
    DcnLane<VEC, NV> L;
    if (!dcn_lane(a, L)) return;
    constexpr int kElem = (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t r_in = make_rsrc(a.input, a.in_bytes);
    const int K3 = 3 * a.K;
    float acc[NV][VEC];
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[i][e] = 0.0f;
    for (int k = 0; k < a.K; ++k) {
        const int ki = k / a.KW, kj = k - (k / a.KW) * a.KW;
        const int gy = L.ho * a.SH - a.PH + ki * a.DH;
        const int gx = L.wo * a.SW - a.PW + kj * a.DW;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const float* om = a.om + (L.pix * a.G + L.gq[i]) * K3;
            const float dx = om[2 * k], dy = om[2 * k + 1], m = om[2 * a.K + k];
            const DcnStencil st = dcn_stencil(a, L.n, gy, gx, dy, dx, L.c0[i], kElem);
            float v[4][VEC];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                VecLoad<T, VEC>::run(r_in, L.valid[i] ? st.off[q] : a.in_bytes, 0u, v[q]);
            const float w0 = m * st.cw[0], w1 = m * st.cw[1], w2 = m * st.cw[2], w3 = m * st.cw[3];
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                acc[i][e] += w0 * v[0][e] + w1 * v[1][e] + w2 * v[2][e] + w3 * v[3][e];
        }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i)
        if (L.valid[i]) store_out_vec<VEC>(a, L.pix * a.C + L.c0[i], acc[i]);
}

template <typename T, int VEC, int NV>
__global__ void __launch_bounds__(kDcnThreads) dcn_backward_kernel(DcnArgs a) {
    DcnLane<VEC, NV> L;
    if (!dcn_lane(a, L)) return;     // whole pixels only: a group's lanes stay together
    constexpr int kElem = (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t r_in = make_rsrc(a.input, a.in_bytes);
    const __amdgpu_buffer_rsrc_t r_gi = make_rsrc(a.grad_input, a.gi_bytes);
    const int K3 = 3 * a.K;
    float go[NV][VEC];
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            go[i][e] = L.valid[i] ? load_elem(a.grad_out, L.pix * a.C + L.c0[i] + e, a.go_dtype) : 0.0f;
    for (int k = 0; k < a.K; ++k) {
        const int ki = k / a.KW, kj = k - (k / a.KW) * a.KW;
        const int gy = L.ho * a.SH - a.PH + ki * a.DH;
        const int gx = L.wo * a.SW - a.PW + kj * a.DW;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            // every lane of the group, idle ones too, takes the group's own stencil:
            // the group's sums end in its last lane, which may hold no channels
            const int64_t rec = (L.pix * a.G + L.gq[i]) * K3;
            const float* om = a.om + rec;
            const float dx = om[2 * k], dy = om[2 * k + 1], m = om[2 * a.K + k];
            // gradient offsets: the same corners as the input, in binary32 elements
            const DcnStencil st = dcn_stencil(a, L.n, gy, gx, dy, dx, L.c0[i], kElem);
            float v[4][VEC];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                VecLoad<T, VEC>::run(r_in, L.valid[i] ? st.off[q] : a.in_bytes, 0u, v[q]);
            const float hy = 1.0f - st.ly, hx = 1.0f - st.lx;
            float pm = 0.0f, px = 0.0f, py = 0.0f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float val = st.cw[0] * v[0][e] + st.cw[1] * v[1][e] + st.cw[2] * v[2][e] +
                                  st.cw[3] * v[3][e];
                const float ddx = hy * (v[1][e] - v[0][e]) + st.ly * (v[3][e] - v[2][e]);
                const float ddy = hx * (v[2][e] - v[0][e]) + st.lx * (v[3][e] - v[1][e]);
                pm += go[i][e] * val;
                px += go[i][e] * ddx;
                py += go[i][e] * ddy;
            }
            pm = group_sum(pm, a.Lg);
            px = group_sum(px, a.Lg);
            py = group_sum(py, a.Lg);
            if (L.last[i] && L.g[i] < a.G) {     // the group's sums sit in its last lane
                const bool live = st.inside;
                a.grad_om[rec + 2 * k] = live ? m * px : 0.0f;
                a.grad_om[rec + 2 * k + 1] = live ? m * py : 0.0f;
                a.grad_om[rec + 2 * a.K + k] = live ? pm : 0.0f;
            }
            // input gradient: corner q gets cw_q * m * grad_out (dropped outside)
            if (L.valid[i]) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t goff = st.off[q] == a.in_bytes
                                              ? a.gi_bytes
                                              : st.off[q] / (uint32_t)kElem * 4u;
                    const float w = st.cw[q] * m;
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(w * go[i][e], r_gi,
                                                                        goff + 4u * e, 0, 0);
                }
            }
        }
    }
}

template <typename T, int VEC, int NV>
hipError_t dcn_launch(const DcnArgs& a, bool backward, hipStream_t st) {
    const int64_t ppw = kWave / a.Lp;
    const int64_t blocks = (a.n_pix + ppw * kDcnWaves - 1) / (ppw * kDcnWaves);
    if (backward)
        hipLaunchKernelGGL((dcn_backward_kernel<T, VEC, NV>), dim3((unsigned)blocks),
                           dim3(kDcnThreads), 0, st, a);
    else
        hipLaunchKernelGGL((dcn_forward_kernel<T, VEC, NV>), dim3((unsigned)blocks),
                           dim3(kDcnThreads), 0, st, a);
    return hipGetLastError();
}

template <typename T, int VEC>
hipError_t dcn_dispatch_nv(const DcnArgs& a, int nv, bool backward, hipStream_t st) {
    switch (nv) {
        case 1: return dcn_launch<T, VEC, 1>(a, backward, st);
        case 2: return dcn_launch<T, VEC, 2>(a, backward, st);
        case 4: return dcn_launch<T, VEC, 4>(a, backward, st);
        case 8: return dcn_launch<T, VEC, 8>(a, backward, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t dcn_dispatch(const DcnArgs& a, int in_dtype, int vec, int nv, bool backward,
                        hipStream_t st) {
    return with_elem(in_dtype, [&](auto t) {
        using T = decltype(t);
        constexpr int V = sizeof(T) == 2 ? 8 : 4;
        return vec == V ? dcn_dispatch_nv<T, V>(a, nv, backward, st)
                        : dcn_dispatch_nv<T, 1>(a, nv, backward, st);
    });
}

}  // namespace

hipError_t launch_dcn_forward(const DcnArgs& a, int in_dtype, int vec, int nv, hipStream_t stream) {
    if (a.n_pix == 0) return hipSuccess;
    return dcn_dispatch(a, in_dtype, vec, nv, false, stream);
}

hipError_t launch_dcn_backward(const DcnArgs& a, int in_dtype, int vec, int nv,
                               hipStream_t stream) {
    const hipError_t e =
        launch_fill_zero(a.grad_input, (int64_t)a.N * a.H * a.W * a.C, stream);
    if (e != hipSuccess || a.n_pix == 0) return e;
    return dcn_dispatch(a, in_dtype, vec, nv, true, stream);
}

}  // namespace da
