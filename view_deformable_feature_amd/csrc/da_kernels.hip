// gfx950 (CDNA4) kernels for Sparse4D-style deformable aggregation.
//
// Definition: the Sparse4D deformable_aggregation walkthrough
// (mhpn.cn/news/1081857), sections 3.1-3.2 (HWC bilinear sampling with
// per-corner zero padding), 4.1 (feature / location / weight gradients) and
// 5.1 (sum over points x cameras x scales per batch, anchor and channel).
//
// Design (not the page's thread-per-element layout):
//  * one workgroup per (batch, anchor); its waves split the anchor's
//    samples.  The anchor's per-sample stencils (four corner byte offsets and
//    coefficients) and its weights are computed / copied once into LDS, by one
//    thread per sample, instead of once per channel;
//  * lanes run over contiguous channels, so each corner of a sample is one
//    coalesced read of a whole HWC feature row (16-byte vectors per lane when
//    the group width allows);
//  * feature reads and feature-gradient atomics go through bounds-checked raw
//    buffer instructions: a corner outside its level gets an offset past the
//    end of the buffer, so the hardware returns 0 for the load and drops the
//    atomic -- the page's "outside corners read zero" without branches;
//  * the forward keeps binary32 partial sums in registers and adds the waves'
//    partials in LDS: no atomics, deterministic;
//  * the backward adds binary32 atomics into the feature gradient and reduces
//    the location / weight gradients across lanes with cross-lane shuffles,
//    each output element then stored by exactly one lane (no atomics there).
// The arithmetic is gather-bound (about 0.5 flop per byte), so there is no
// matrix-core (MFMA) work here.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "da_internal.h"

namespace da {
namespace {

// Word 3 of a raw (untyped, stride 0) buffer resource on gfx9-family parts:
// 32-bit data format, range checking on the byte offset.
constexpr int kRawBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kRawBufferWord3);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Load VEC consecutive channels as floats.  voff: per-lane byte offset (an
// out-of-range value yields zeros); soff: wave-uniform byte offset.
template <typename T, int VEC>
struct VecLoad;

template <>
struct VecLoad<float, 1> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff, float (&v)[1]) {
        v[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
    }
};

template <>
struct VecLoad<float, 4> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff, float (&v)[4]) {
        auto q = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
        v[0] = __uint_as_float(q[0]);
        v[1] = __uint_as_float(q[1]);
        v[2] = __uint_as_float(q[2]);
        v[3] = __uint_as_float(q[3]);
    }
};

template <>
struct VecLoad<uint16_t, 1> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff, float (&v)[1]) {
        v[0] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0)
                               << 16);
    }
};

template <>
struct VecLoad<uint16_t, 8> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff, float (&v)[8]) {
        auto q = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = bf16_lo(q[e]);
            v[2 * e + 1] = bf16_hi(q[e]);
        }
    }
};

struct FwdDesc {
    uint32_t off[4];   // byte offsets of the four corner rows in the feature image
    float cw[4];       // hh*hw, hh*lw, lh*hw, lh*lw
};
static_assert(sizeof(FwdDesc) == kFwdDescBytes, "FwdDesc layout");

struct BwdDesc {
    uint32_t off[4];   // feature image byte offsets
    uint32_t goff[4];  // feature-gradient image byte offsets
    float cw[4];       // corner weights
    float gx[4];       // d val / d x per corner value: W * (-hh, hh, -lh, lh)
    float gy[4];       // d val / d y per corner value: H * (-hw, -lw, hw, lw)
};
static_assert(sizeof(BwdDesc) == kBwdDescBytes, "BwdDesc layout");

// Bilinear stencil of sample t = pk * S + s of anchor `ba` (section 3.2).  The
// pixel coordinate is a binary32 product rounded, then a rounded subtraction:
// floor() of it selects the corner cell, so it must not be fused.
struct Stencil {
    bool inside;
    int32_t row[4];        // absolute row in the batch image or -1
    float cw[4];
    float lh, lw, hh, hw;
    float H, W;
};

__device__ __forceinline__ Stencil make_stencil(const KArgs& a, int64_t ba, int t) {
    // t < P*K*S < 2^31 and ba < 2^23 are guaranteed by the host checks
    Stencil st;
    const int pk = t / a.S;
    const int s = t - pk * a.S;
    const int k = pk % a.K;
    const int lvl = k * a.S + s;
    const int32_t H = a.lv.H[lvl], W = a.lv.W[lvl], start = a.lv.start[lvl];
    const float2 xy = *reinterpret_cast<const float2*>(a.loc + (ba * a.npk + pk) * 2);
    float w_im, h_im;
    {
#pragma clang fp contract(off)
        const float wx = xy.x * (float)W;
        const float hy = xy.y * (float)H;
        w_im = wx - 0.5f;
        h_im = hy - 0.5f;
    }
    st.H = (float)H;
    st.W = (float)W;
    st.inside = h_im > -1.0f && w_im > -1.0f && h_im < (float)H && w_im < (float)W;
    const float hlf = st.inside ? floorf(h_im) : 0.0f;
    const float wlf = st.inside ? floorf(w_im) : 0.0f;
    const int h_low = (int)hlf, w_low = (int)wlf;
    st.lh = st.inside ? h_im - hlf : 0.0f;
    st.lw = st.inside ? w_im - wlf : 0.0f;
    st.hh = 1.0f - st.lh;
    st.hw = 1.0f - st.lw;
    const int hs[4] = {h_low, h_low, h_low + 1, h_low + 1};
    const int ws[4] = {w_low, w_low + 1, w_low, w_low + 1};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool ok = st.inside && hs[i] >= 0 && hs[i] <= H - 1 && ws[i] >= 0 && ws[i] <= W - 1;
        st.row[i] = ok ? start + hs[i] * W + ws[i] : -1;
    }
    const float m = st.inside ? 1.0f : 0.0f;
    st.cw[0] = m * st.hh * st.hw;
    st.cw[1] = m * st.hh * st.lw;
    st.cw[2] = m * st.lh * st.hw;
    st.cw[3] = m * st.lh * st.lw;
    return st;
}

__device__ __forceinline__ float xor_shfl(float v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

// ------------------------------------------------------------------------------------
// forward
// ------------------------------------------------------------------------------------
template <typename T, int VEC, int NVC>
__global__ void __launch_bounds__(kWave * kMaxWaves)
da_forward_kernel(KArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int64_t ba = blockIdx.x;
    const int64_t b = (int64_t)(blockIdx.x / (uint32_t)a.A);
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int L = a.L;
    const int spw = kWave >> a.log2L;            // row groups per wave
    const int rg = wave * spw + (lane >> a.log2L);
    const int n_rg = (nthreads / kWave) * spw;
    const int li = lane & (L - 1);
    constexpr int kElem = (int)sizeof(T);

    const int ns_max = a.pk_chunk * a.S;
    FwdDesc* desc = reinterpret_cast<FwdDesc*>(smem);
    float* wts = reinterpret_cast<float*>(smem + (size_t)ns_max * sizeof(FwdDesc));
    float* red = wts + (size_t)ns_max * a.G;     // [waves][chunk channels]

    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(
        static_cast<const unsigned char*>(a.feat) + b * a.feat_batch_bytes, a.feat_image_bytes);

    const int v0 = blockIdx.y * a.nv_chunk;      // first vector (per lane) of this chunk
    const int nvh = min(a.nv_chunk, a.nv - v0);
    const uint32_t lane_off = (uint32_t)(li * VEC * kElem);
    uint32_t soff[NVC];
    int gi[NVC];
#pragma unroll
    for (int i = 0; i < NVC; ++i) {
        const int vidx = li + L * (v0 + i);      // vector index within the row
        soff[i] = (uint32_t)(L * (v0 + i) * VEC * kElem);
        gi[i] = min(vidx * VEC / a.D, a.G - 1);
    }

    float acc[NVC][VEC];
#pragma unroll
    for (int i = 0; i < NVC; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[i][e] = 0.0f;

    const int64_t wbase = ba * (int64_t)a.npk * a.S * a.G;
    for (int pk0 = 0; pk0 < a.npk; pk0 += a.pk_chunk) {
        const int ns = min(a.pk_chunk, a.npk - pk0) * a.S;
        for (int t = tid; t < ns; t += nthreads) {
            const Stencil st = make_stencil(a, ba, pk0 * a.S + t);
            FwdDesc d;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                d.off[i] = st.row[i] >= 0 ? (uint32_t)st.row[i] * (uint32_t)a.row_bytes
                                          : a.feat_image_bytes;
                d.cw[i] = st.cw[i];
            }
            desc[t] = d;
        }
        const float* wsrc = a.weights + wbase + (int64_t)pk0 * a.S * a.G;
        for (int i = tid; i < ns * a.G; i += nthreads) wts[i] = wsrc[i];
        __syncthreads();

        for (int t = rg; t < ns; t += n_rg) {
            const FwdDesc d = desc[t];
#pragma unroll
            for (int i = 0; i < NVC; ++i) {
                if (i < nvh) {
                    float v[4][VEC];
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        VecLoad<T, VEC>::run(rsrc, d.off[c] + lane_off, soff[i], v[c]);
                    const float w = wts[t * a.G + gi[i]];
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const float val = d.cw[0] * v[0][e] + d.cw[1] * v[1][e] +
                                          d.cw[2] * v[2][e] + d.cw[3] * v[3][e];
                        acc[i][e] += w * val;
                    }
                }
            }
        }
        __syncthreads();
    }

    // row groups of one wave: add across lanes li, li + L, ... with shuffles
#pragma unroll
    for (int i = 0; i < NVC; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            for (int m = L; m < kWave; m <<= 1) acc[i][e] += xor_shfl(acc[i][e], m);

    // waves: add through LDS (channels of this chunk: nvh * L * VEC)
    const int nch = nvh * L * VEC;
    if (lane < L) {
#pragma unroll
        for (int i = 0; i < NVC; ++i)
            if (i < nvh)
#pragma unroll
                for (int e = 0; e < VEC; ++e) red[wave * nch + (li + L * i) * VEC + e] = acc[i][e];
    }
    __syncthreads();
    const int nwaves = nthreads / kWave;
    float* orow = a.out + ba * a.C + (int64_t)v0 * L * VEC;
    for (int c = tid; c < nch; c += nthreads) {
        float sum = 0.0f;
        for (int w = 0; w < nwaves; ++w) sum += red[w * nch + c];
        orow[c] = sum;
    }
    (void)n_rg;
}

// ------------------------------------------------------------------------------------
// backward
// ------------------------------------------------------------------------------------
// Lanes hold single channels: lane li of a row group covers channels li + L*i.
// Group reduction: each element is summed over `seg` lanes (seg = D when one
// row of L lanes spans several groups, seg = L otherwise).
template <typename T, int NVC>
__global__ void __launch_bounds__(kWave * kMaxWaves)
da_backward_kernel(KArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int64_t ba = blockIdx.x;
    const int64_t b = (int64_t)(blockIdx.x / (uint32_t)a.A);
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int L = a.L;
    const int spw = kWave >> a.log2L;
    const int rg = wave * spw + (lane >> a.log2L);
    const int n_rg = (nthreads / kWave) * spw;
    const int li = lane & (L - 1);
    const int seg = a.seg;
    constexpr int kElem = (int)sizeof(T);

    const int ns_max = a.pk_chunk * a.S;
    BwdDesc* desc = reinterpret_cast<BwdDesc*>(smem);
    float* wts = reinterpret_cast<float*>(smem + (size_t)ns_max * sizeof(BwdDesc));

    const __amdgpu_buffer_rsrc_t rf = make_rsrc(
        static_cast<const unsigned char*>(a.feat) + b * a.feat_batch_bytes, a.feat_image_bytes);
    const __amdgpu_buffer_rsrc_t rg_rsrc = make_rsrc(
        reinterpret_cast<unsigned char*>(a.grad_feat) + b * a.gfeat_batch_bytes,
        a.gfeat_image_bytes);

    const int nv = a.nv;
    const uint32_t lane_off = (uint32_t)(li * kElem);
    const uint32_t lane_goff = (uint32_t)(li * 4);
    float go[NVC];
    int gi[NVC];
#pragma unroll
    for (int i = 0; i < NVC; ++i) {
        const int c = li + L * i;
        go[i] = (i < nv) ? a.grad_out[ba * a.C + c] : 0.0f;
        gi[i] = (i < nv) ? c / a.D : 0;
    }

    const int64_t wbase = ba * (int64_t)a.npk * a.S * a.G;
    for (int pk0 = 0; pk0 < a.npk; pk0 += a.pk_chunk) {
        const int npk_here = min(a.pk_chunk, a.npk - pk0);
        const int ns = npk_here * a.S;
        for (int t = tid; t < ns; t += nthreads) {
            const Stencil st = make_stencil(a, ba, pk0 * a.S + t);
            BwdDesc d;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = st.row[i] >= 0;
                d.off[i] = ok ? (uint32_t)st.row[i] * (uint32_t)a.row_bytes : a.feat_image_bytes;
                d.goff[i] = ok ? (uint32_t)st.row[i] * (uint32_t)a.grow_bytes : a.gfeat_image_bytes;
                d.cw[i] = st.cw[i];
            }
            const float m = st.inside ? 1.0f : 0.0f;
            d.gx[0] = -m * st.W * st.hh;
            d.gx[1] = m * st.W * st.hh;
            d.gx[2] = -m * st.W * st.lh;
            d.gx[3] = m * st.W * st.lh;
            d.gy[0] = -m * st.H * st.hw;
            d.gy[1] = -m * st.H * st.lw;
            d.gy[2] = m * st.H * st.hw;
            d.gy[3] = m * st.H * st.lw;
            desc[t] = d;
        }
        const float* wsrc = a.weights + wbase + (int64_t)pk0 * a.S * a.G;
        for (int i = tid; i < ns * a.G; i += nthreads) wts[i] = wsrc[i];
        __syncthreads();

        for (int pk = rg; pk < npk_here; pk += n_rg) {
            float gxs = 0.0f, gys = 0.0f;
            for (int s = 0; s < a.S; ++s) {
                const int t = pk * a.S + s;
                const BwdDesc d = desc[t];
                float tc[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // sum_i top_i * v_corner
                float gwp[NVC];
#pragma unroll
                for (int i = 0; i < NVC; ++i) {
                    gwp[i] = 0.0f;
                    if (i < nv) {
                        const uint32_t soff = (uint32_t)(L * i * kElem);
                        const uint32_t sgoff = (uint32_t)(L * i * 4);
                        float v[4];
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            float one[1];
                            VecLoad<T, 1>::run(rf, d.off[c] + lane_off, soff, one);
                            v[c] = one[0];
                        }
                        const float top = go[i] * wts[t * a.G + gi[i]];
                        const float val = d.cw[0] * v[0] + d.cw[1] * v[1] + d.cw[2] * v[2] +
                                          d.cw[3] * v[3];
                        gwp[i] = go[i] * val;
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            tc[c] += top * v[c];
                            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
                                d.cw[c] * top, rg_rsrc, d.goff[c] + lane_goff, sgoff, 0);
                        }
                    }
                }
                gxs += d.gx[0] * tc[0] + d.gx[1] * tc[1] + d.gx[2] * tc[2] + d.gx[3] * tc[3];
                gys += d.gy[0] * tc[0] + d.gy[1] * tc[1] + d.gy[2] * tc[2] + d.gy[3] * tc[3];

                // weight gradient: sum grad_out * val over the channels of each group
#pragma unroll
                for (int i = 0; i < NVC; ++i)
                    for (int m = 1; m < seg; m <<= 1) gwp[i] += xor_shfl(gwp[i], m);
                float* gwrow = a.grad_weights + wbase + ((int64_t)(pk0 + pk) * a.S + s) * a.G;
                if (seg < L) {
                    if ((li & (seg - 1)) == 0) {
#pragma unroll
                        for (int i = 0; i < NVC; ++i)
                            if (i < nv) gwrow[gi[i]] = gwp[i];
                    }
                } else if (li == 0) {
                    float run = 0.0f;
#pragma unroll
                    for (int i = 0; i < NVC; ++i) {
                        if (i < nv) {
                            run += gwp[i];
                            if (i + 1 >= nv || gi[(i + 1) < NVC ? i + 1 : i] != gi[i]) {
                                gwrow[gi[i]] = run;
                                run = 0.0f;
                            }
                        }
                    }
                }
            }
            for (int m = 1; m < L; m <<= 1) {
                gxs += xor_shfl(gxs, m);
                gys += xor_shfl(gys, m);
            }
            if (li == 0) {
                float2* gl = reinterpret_cast<float2*>(a.grad_loc + (ba * a.npk + pk0 + pk) * 2);
                *gl = make_float2(gxs, gys);
            }
        }
        __syncthreads();
    }
}

__global__ void zero_kernel(float* __restrict__ p, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool vec_ok = (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
    if (vec_ok) {
        float4* p4 = reinterpret_cast<float4*>(p);
        const int64_t n4 = n / 4;
        for (int64_t j = i; j < n4; j += stride) p4[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int64_t j = n4 * 4 + i; j < n; j += stride) p[j] = 0.0f;
    } else {
        for (int64_t j = i; j < n; j += stride) p[j] = 0.0f;
    }
}

template <typename T, int VEC>
hipError_t fwd_dispatch_nvc(const KArgs& a, const LaunchShape& s, dim3 grid, hipStream_t st) {
    const dim3 block(kWave * s.waves);
    switch (s.nvc) {
        case 1: hipLaunchKernelGGL((da_forward_kernel<T, VEC, 1>), grid, block, s.lds_bytes, st, a); break;
        case 2: hipLaunchKernelGGL((da_forward_kernel<T, VEC, 2>), grid, block, s.lds_bytes, st, a); break;
        case 4: hipLaunchKernelGGL((da_forward_kernel<T, VEC, 4>), grid, block, s.lds_bytes, st, a); break;
        case 8: hipLaunchKernelGGL((da_forward_kernel<T, VEC, 8>), grid, block, s.lds_bytes, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t bwd_dispatch_nvc(const KArgs& a, const LaunchShape& s, dim3 grid, hipStream_t st) {
    const dim3 block(kWave * s.waves);
    switch (s.nvc) {
        case 1: hipLaunchKernelGGL((da_backward_kernel<T, 1>), grid, block, s.lds_bytes, st, a); break;
        case 2: hipLaunchKernelGGL((da_backward_kernel<T, 2>), grid, block, s.lds_bytes, st, a); break;
        case 4: hipLaunchKernelGGL((da_backward_kernel<T, 4>), grid, block, s.lds_bytes, st, a); break;
        case 8: hipLaunchKernelGGL((da_backward_kernel<T, 8>), grid, block, s.lds_bytes, st, a); break;
        case 16: hipLaunchKernelGGL((da_backward_kernel<T, 16>), grid, block, s.lds_bytes, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(const KArgs& a, const LaunchShape& s, int64_t n_anchors_total, bool bf16,
                          hipStream_t stream) {
    const dim3 grid((unsigned)n_anchors_total, (unsigned)s.chunks);
    if (bf16) {
        return s.vec == 8 ? fwd_dispatch_nvc<uint16_t, 8>(a, s, grid, stream)
                          : fwd_dispatch_nvc<uint16_t, 1>(a, s, grid, stream);
    }
    return s.vec == 4 ? fwd_dispatch_nvc<float, 4>(a, s, grid, stream)
                      : fwd_dispatch_nvc<float, 1>(a, s, grid, stream);
}

hipError_t launch_backward(const KArgs& a, const LaunchShape& s, int64_t n_anchors_total, bool bf16,
                           hipStream_t stream) {
    const dim3 grid((unsigned)n_anchors_total, 1);
    return bf16 ? bwd_dispatch_nvc<uint16_t>(a, s, grid, stream)
                : bwd_dispatch_nvc<float>(a, s, grid, stream);
}

hipError_t launch_zero(float* p, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int block = 256;
    int64_t blocks = (n / 4 + block - 1) / block;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(block), 0, stream, p, n);
    return hipGetLastError();
}

}  // namespace da
