// gfx950 (CDNA4) forward kernel of Sparse4D-style deformable aggregation.
//
// Definition: the Sparse4D deformable_aggregation walkthrough
// (mhpn.cn/news/1081857), sections 3.2 (bilinear sampling) and 5.1 (for every
// batch, anchor and channel, the weighted sum over points x cameras x scales).
//
// Design (not the page's thread-per-element layout): one workgroup per
// (batch, anchor).  The anchor's per-sample stencils (four corner byte offsets
// and corner weights) and its weights are built once into LDS by one thread
// per sample.  Lanes then run over contiguous channels, so each corner of a
// sample is one coalesced read of a whole HWC row (16-byte vectors per lane
// when the group width allows), through bounds-checked buffer loads that
// answer outside corners with zeros.  Partial sums stay in registers and the
// waves' partials are added in LDS: no atomics, deterministic.  The arithmetic
// is gather-bound (about 0.5 flop per byte), so there is no matrix-core work.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "da_device.h"

namespace da {
namespace {

// ------------------------------------------------------------------------------------
// forward
// ------------------------------------------------------------------------------------
// Row group rg walks samples t = rg, rg + n_rg, ... of the staged chunk.  The
// loop is software-pipelined two deep: the four corner rows of the next
// sample are requested before the current one is accumulated, so a wave
// always has two samples' worth of loads in flight.  Past the last sample the
// prefetch reads the null descriptor (all offsets outside the buffer), which
// the hardware answers with zeros and no memory traffic.
template <typename T, int VEC, int NV>
__device__ __forceinline__ void fwd_load(const __amdgpu_buffer_rsrc_t& r, const FwdDesc& d,
                                         uint32_t lane_off, const uint32_t (&soff)[NV],
                                         float (&v)[NV][4][VEC]) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) VecLoad<T, VEC>::run(r, d.off[c] + lane_off, soff[i], v[i][c]);
}

template <int VEC, int NV>
__device__ __forceinline__ void fwd_accumulate(const FwdDesc& d, const float* wrow,
                                               const int (&gi)[NV], const float (&v)[NV][4][VEC],
                                               float (&acc)[NV][VEC]) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const float w = wrow[gi[i]];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float val = d.cw[0] * v[i][0][e] + d.cw[1] * v[i][1][e] + d.cw[2] * v[i][2][e] +
                              d.cw[3] * v[i][3][e];
            acc[i][e] += w * val;
        }
    }
}

__device__ __forceinline__ FwdDesc null_fwd_desc(uint32_t outside) {
    FwdDesc d;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        d.off[i] = outside;
        d.cw[i] = 0.0f;
    }
    return d;
}

template <typename T, int VEC, int NV>
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

    const int ns_max = a.pk_chunk * a.S;         // desc[ns_max] is the null descriptor
    FwdDesc* desc = reinterpret_cast<FwdDesc*>(smem);
    float* wts = reinterpret_cast<float*>(smem + (size_t)(ns_max + 1) * sizeof(FwdDesc));
    float* red = wts + (size_t)ns_max * a.G;     // [waves][chunk channels]

    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(
        static_cast<const unsigned char*>(a.feat) + b * a.feat_batch_bytes, a.feat_image_bytes);

    const int v0 = blockIdx.y * NV;              // first vector (per lane) of this chunk
    const uint32_t lane_off = (uint32_t)(li * VEC * kElem);
    uint32_t soff[NV];
    int gi[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        soff[i] = (uint32_t)(L * (v0 + i) * VEC * kElem);
        gi[i] = (li + L * (v0 + i)) * VEC / a.D;
    }

    float acc[NV][VEC];
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[i][e] = 0.0f;

    if (tid == 0) desc[ns_max] = null_fwd_desc(a.feat_image_bytes);
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

        int t = rg;
        if (t < ns) {
            FwdDesc dA = desc[t], dB;
            float vA[NV][4][VEC], vB[NV][4][VEC];
            fwd_load<T, VEC, NV>(rsrc, dA, lane_off, soff, vA);
            while (true) {
                int tn = t + n_rg;
                dB = desc[tn < ns ? tn : ns_max];
                fwd_load<T, VEC, NV>(rsrc, dB, lane_off, soff, vB);
                fwd_accumulate<VEC, NV>(dA, wts + t * a.G, gi, vA, acc);
                if (tn >= ns) break;
                t = tn;
                tn = t + n_rg;
                dA = desc[tn < ns ? tn : ns_max];
                fwd_load<T, VEC, NV>(rsrc, dA, lane_off, soff, vA);
                fwd_accumulate<VEC, NV>(dB, wts + t * a.G, gi, vB, acc);
                if (tn >= ns) break;
                t = tn;
            }
        }
        __syncthreads();
    }

    // row groups of one wave: add across lanes li, li + L, ... with shuffles
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            for (int m = L; m < kWave; m <<= 1) acc[i][e] += xor_shfl(acc[i][e], m);

    // waves: add through LDS (channels of this chunk: NV * L * VEC)
    const int nch = NV * L * VEC;
    if (lane < L) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int e = 0; e < VEC; ++e) red[wave * nch + (li + L * i) * VEC + e] = acc[i][e];
    }
    __syncthreads();
    const int nwaves = nthreads / kWave;
    const int64_t o0 = ba * a.C + (int64_t)v0 * L * VEC;
    for (int c = tid; c < nch; c += nthreads) {
        float sum = 0.0f;
        for (int w = 0; w < nwaves; ++w) sum += red[w * nch + c];
        store_elem(a.out, o0 + c, sum, a.out_dtype);
    }
}

// ------------------------------------------------------------------------------------
// forward by level slices
// ------------------------------------------------------------------------------------
// Workgroup (anchor, x) -- on XCD x -- sums the samples of the levels in slice
// x only, in the fixed order of slice_sample(), and writes its partial output
// row to fwd_part[x]; fwd_reduce_kernel then adds the 8 partials in slice
// order.  Same staging, lane layout and two-deep pipeline as the per-anchor
// kernel above.
template <typename T, int VEC, int NV>
__global__ void __launch_bounds__(kWave * kMaxWaves)
da_forward_sliced_kernel(KArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int x = (int)(blockIdx.x % (uint32_t)kSlices);
    const int64_t ba = blockIdx.x / (uint32_t)kSlices;
    const int64_t b = ba / a.A;
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int L = a.L;
    const int spw = kWave >> a.log2L;
    const int rg = wave * spw + (lane >> a.log2L);
    const int n_rg = (nthreads / kWave) * spw;
    const int li = lane & (L - 1);
    constexpr int kElem = (int)sizeof(T);

    const int ns_max = a.sample_chunk;           // desc[ns_max] is the null descriptor
    FwdDesc* desc = reinterpret_cast<FwdDesc*>(smem);
    float* wts = reinterpret_cast<float*>(smem + (size_t)(ns_max + 1) * sizeof(FwdDesc));
    float* red = wts + (size_t)ns_max * a.G;

    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(
        static_cast<const unsigned char*>(a.feat) + b * a.feat_batch_bytes, a.feat_image_bytes);

    const int v0 = blockIdx.y * NV;
    const uint32_t lane_off = (uint32_t)(li * VEC * kElem);
    uint32_t soff[NV];
    int gi[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        soff[i] = (uint32_t)(L * (v0 + i) * VEC * kElem);
        gi[i] = (li + L * (v0 + i)) * VEC / a.D;
    }
    float acc[NV][VEC];
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[i][e] = 0.0f;

    if (tid == 0) desc[ns_max] = null_fwd_desc(a.feat_image_bytes);
    const int m = a.lv.slice_nlev[x];
    const int n = a.P * m;
    // level table and this slice's level list in LDS: every lane of the
    // staging loops looks up its own level
    __shared__ int32_t lvl_lds[3 * kMaxLevels + kMaxSliceLevels];
    int32_t* slice_lv = lvl_lds + 3 * kMaxLevels;
    if (tid < m) slice_lv[tid] = a.lv.slice_level[x][tid];
    const LevelsLds lv = stage_levels(a, lvl_lds);
    const int64_t wbase = ba * (int64_t)a.npk * a.S * a.G;
    for (int j0 = 0; j0 < n; j0 += ns_max) {
        const int nsc = min(ns_max, n - j0);
        for (int jj = tid; jj < nsc; jj += nthreads) {
            const Stencil st = make_stencil(a, ba, slice_sample(a, slice_lv, m, j0 + jj), lv);
            FwdDesc d;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                d.off[i] = st.row[i] >= 0 ? (uint32_t)st.row[i] * (uint32_t)a.row_bytes
                                          : a.feat_image_bytes;
                d.cw[i] = st.cw[i];
            }
            desc[jj] = d;
        }
        for (int i = tid; i < nsc * a.G; i += nthreads) {
            const int jj = i / a.G;
            wts[i] = a.weights[wbase + (int64_t)slice_sample(a, slice_lv, m, j0 + jj) * a.G + (i - jj * a.G)];
        }
        __syncthreads();

        int t = rg;
        if (t < nsc) {
            FwdDesc dA = desc[t], dB;
            float vA[NV][4][VEC], vB[NV][4][VEC];
            fwd_load<T, VEC, NV>(rsrc, dA, lane_off, soff, vA);
            while (true) {
                int tn = t + n_rg;
                dB = desc[tn < nsc ? tn : ns_max];
                fwd_load<T, VEC, NV>(rsrc, dB, lane_off, soff, vB);
                fwd_accumulate<VEC, NV>(dA, wts + t * a.G, gi, vA, acc);
                if (tn >= nsc) break;
                t = tn;
                tn = t + n_rg;
                dA = desc[tn < nsc ? tn : ns_max];
                fwd_load<T, VEC, NV>(rsrc, dA, lane_off, soff, vA);
                fwd_accumulate<VEC, NV>(dB, wts + t * a.G, gi, vB, acc);
                if (tn >= nsc) break;
                t = tn;
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            for (int mk = L; mk < kWave; mk <<= 1) acc[i][e] += xor_shfl(acc[i][e], mk);
    const int nch = NV * L * VEC;
    if (lane < L) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int e = 0; e < VEC; ++e) red[wave * nch + (li + L * i) * VEC + e] = acc[i][e];
    }
    __syncthreads();
    const int nwaves = nthreads / kWave;
    float* prow = a.fwd_part + ((int64_t)x * a.n_anchors + ba) * a.C + (int64_t)v0 * L * VEC;
    for (int c = tid; c < nch; c += nthreads) {
        float sum = 0.0f;
        for (int w = 0; w < nwaves; ++w) sum += red[w * nch + c];
        prow[c] = sum;
    }
}

// Sweep form of the sliced forward: one wave per (anchor, slice).  Each wave
// sorts its slice's samples (at most 64) by normalised y and walks them in that
// order, so the waves resident together read the rows of about one band of
// every level at a time instead of the whole slice: fewer L2 misses where a
// slice's levels exceed an XCD's L2.  Taken where a wave holds at least two
// samples per step (two or more row groups); with one, the wave's chain of
// samples is twice as long and the form measured slower.  The partial is a sum
// in y order (ties and NaN by sample order): fixed for given inputs.
template <typename T, int VEC, int NV>
__global__ void __launch_bounds__(kWave) da_forward_sweep_kernel(KArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int x = (int)(blockIdx.x % (uint32_t)kSlices);
    const int64_t ba = blockIdx.x / (uint32_t)kSlices;
    const int64_t b = ba / a.A;
    const int lane = threadIdx.x;
    const int L = a.L;
    const int rg = lane >> a.log2L;
    const int n_rg = kWave >> a.log2L;
    const int li = lane & (L - 1);
    constexpr int kElem = (int)sizeof(T);

    FwdDesc* desc = reinterpret_cast<FwdDesc*>(smem);          // [kWave + 1]
    float* wts = reinterpret_cast<float*>(smem + (size_t)(kWave + 1) * sizeof(FwdDesc));

    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(
        static_cast<const unsigned char*>(a.feat) + b * a.feat_batch_bytes, a.feat_image_bytes);
    const int v0 = blockIdx.y * NV;
    const uint32_t lane_off = (uint32_t)(li * VEC * kElem);
    uint32_t soff[NV];
    int gi[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        soff[i] = (uint32_t)(L * (v0 + i) * VEC * kElem);
        gi[i] = (li + L * (v0 + i)) * VEC / a.D;
    }
    float acc[NV][VEC];
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[i][e] = 0.0f;

    const int m = a.lv.slice_nlev[x];
    const int n = a.P * m;                        // <= kWave (the host checks)
    __shared__ int32_t lvl_lds[3 * kMaxLevels + kMaxSliceLevels];
    int32_t* slice_lv = lvl_lds + 3 * kMaxLevels;
    if (lane < m) slice_lv[lane] = a.lv.slice_level[x][lane];
    const LevelsLds lv = stage_levels(a, lvl_lds);

    // lane j stages sample j at its rank in y order
    int t = 0;
    float key = __builtin_huge_valf();
    if (lane < n) {
        t = slice_sample(a, slice_lv, m, lane);
        const float y = a.loc[(ba * a.npk + t / a.S) * 2 + 1];
        key = y == y ? y : 2.0f;
    }
    int rank = 0;
    for (int i = 0; i < kWave; ++i) {
        const float ki = __shfl(key, i, kWave);
        rank += (ki < key || (ki == key && i < lane)) ? 1 : 0;
    }
    if (lane < n) {
        const Stencil st = make_stencil(a, ba, t, lv);
        FwdDesc d;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            d.off[i] = st.row[i] >= 0 ? (uint32_t)st.row[i] * (uint32_t)a.row_bytes
                                      : a.feat_image_bytes;
            d.cw[i] = st.cw[i];
        }
        desc[rank] = d;
        const float* wsrc = a.weights + (ba * (int64_t)a.npk * a.S + t) * a.G;
        for (int g = 0; g < a.G; ++g) wts[rank * a.G + g] = wsrc[g];
    }
    if (lane == 0) desc[kWave] = null_fwd_desc(a.feat_image_bytes);
    __syncthreads();

    int s = rg;
    if (s < n) {
        FwdDesc dA = desc[s], dB;
        float vA[NV][4][VEC], vB[NV][4][VEC];
        fwd_load<T, VEC, NV>(rsrc, dA, lane_off, soff, vA);
        while (true) {
            int sn = s + n_rg;
            dB = desc[sn < n ? sn : kWave];
            fwd_load<T, VEC, NV>(rsrc, dB, lane_off, soff, vB);
            fwd_accumulate<VEC, NV>(dA, wts + s * a.G, gi, vA, acc);
            if (sn >= n) break;
            s = sn;
            sn = s + n_rg;
            dA = desc[sn < n ? sn : kWave];
            fwd_load<T, VEC, NV>(rsrc, dA, lane_off, soff, vA);
            fwd_accumulate<VEC, NV>(dB, wts + s * a.G, gi, vB, acc);
            if (sn >= n) break;
            s = sn;
        }
    }

#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            for (int mk = L; mk < kWave; mk <<= 1) acc[i][e] += xor_shfl(acc[i][e], mk);
    if (lane < L) {
        float* prow = a.fwd_part + ((int64_t)x * a.n_anchors + ba) * a.C + (int64_t)v0 * L * VEC;
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int e = 0; e < VEC; ++e) prow[(li + L * i) * VEC + e] = acc[i][e];
    }
}

// out = sum of the 8 slice partials, added in slice order.
__global__ void __launch_bounds__(256) fwd_reduce_kernel(KArgs a) {
    const int64_t n = (int64_t)a.n_anchors * a.C;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        float s = 0.0f;
#pragma unroll
        for (int x = 0; x < kSlices; ++x) s += a.fwd_part[x * n + i];
        store_elem(a.out, i, s, a.out_dtype);
    }
}

template <typename T, int VEC, int NV>
hipError_t fwd_sliced_launch(const KArgs& a, const LaunchShape& s, dim3 grid, hipStream_t st) {
    if (a.fwd_sweep)
        hipLaunchKernelGGL((da_forward_sweep_kernel<T, VEC, NV>), grid, dim3(kWave), s.lds_bytes,
                           st, a);
    else
        hipLaunchKernelGGL((da_forward_sliced_kernel<T, VEC, NV>), grid, dim3(kWave * s.waves),
                           s.lds_bytes, st, a);
    return hipGetLastError();
}

template <typename T, int VEC>
hipError_t fwd_sliced_dispatch(const KArgs& a, const LaunchShape& s, dim3 grid, hipStream_t st) {
    switch (s.nvc) {
        case 1: return fwd_sliced_launch<T, VEC, 1>(a, s, grid, st);
        case 2: return fwd_sliced_launch<T, VEC, 2>(a, s, grid, st);
        case 4: return fwd_sliced_launch<T, VEC, 4>(a, s, grid, st);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, int VEC, int NV>
hipError_t fwd_launch(const KArgs& a, const LaunchShape& s, dim3 grid, hipStream_t st) {
    hipLaunchKernelGGL((da_forward_kernel<T, VEC, NV>), grid, dim3(kWave * s.waves), s.lds_bytes,
                       st, a);
    return hipGetLastError();
}

template <typename T, int VEC>
hipError_t fwd_dispatch_nv(const KArgs& a, const LaunchShape& s, dim3 grid, hipStream_t st) {
    switch (s.nvc) {
        case 1: return fwd_launch<T, VEC, 1>(a, s, grid, st);
        case 2: return fwd_launch<T, VEC, 2>(a, s, grid, st);
        case 3: return fwd_launch<T, VEC, 3>(a, s, grid, st);
        case 4: return fwd_launch<T, VEC, 4>(a, s, grid, st);
        case 5: return fwd_launch<T, VEC, 5>(a, s, grid, st);
        case 6: return fwd_launch<T, VEC, 6>(a, s, grid, st);
        case 7: return fwd_launch<T, VEC, 7>(a, s, grid, st);
        case 8: return fwd_launch<T, VEC, 8>(a, s, grid, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_forward_sliced(const KArgs& a, const LaunchShape& s, int64_t n_anchors_total,
                                 int feat_dtype, hipStream_t stream) {
    const dim3 grid((unsigned)(n_anchors_total * kSlices), (unsigned)s.chunks);
    const hipError_t e = with_elem(feat_dtype, [&](auto t) {
        using T = decltype(t);
        constexpr int V = sizeof(T) == 2 ? 8 : 4;   // 16-byte vectors
        return s.vec == V ? fwd_sliced_dispatch<T, V>(a, s, grid, stream)
                          : fwd_sliced_dispatch<T, 1>(a, s, grid, stream);
    });
    if (e != hipSuccess) return e;
    int64_t blocks = ((int64_t)a.n_anchors * a.C + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fwd_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_forward(const KArgs& a, const LaunchShape& s, int64_t n_anchors_total,
                          int feat_dtype, hipStream_t stream) {
    const dim3 grid((unsigned)n_anchors_total, (unsigned)s.chunks);
    return with_elem(feat_dtype, [&](auto t) {
        using T = decltype(t);
        constexpr int V = sizeof(T) == 2 ? 8 : 4;
        return s.vec == V ? fwd_dispatch_nv<T, V>(a, s, grid, stream)
                          : fwd_dispatch_nv<T, 1>(a, s, grid, stream);
    });
}

}  // namespace da
