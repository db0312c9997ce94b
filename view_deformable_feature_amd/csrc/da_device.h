// Device-side building blocks shared by the forward and backward kernels:
// buffer resources, vector loads, the bilinear stencil, LDS descriptors.
//
// Definition followed: the Sparse4D deformable_aggregation walkthrough
// (mhpn.cn/news/1081857), section 3.1 (HWC offsets) and section 3.2
// (bilinear sampling with per-corner zero padding).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "da_internal.h"

namespace da {

// Word 3 of a raw (untyped, stride 0) buffer resource on gfx9-family parts:
// 32-bit data format, range checking on the byte offset.  Loads whose offset
// lies past num_records return 0 and atomics there are dropped, without any
// memory request.
constexpr int kRawBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kRawBufferWord3);
}

// 16-bit element types: bfloat16 is held as uint16_t, IEEE binary16 as _Float16.
// Both convert to binary32 exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_bits(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ float f16_lo(uint32_t w) { return f16_bits(w & 0xffffu); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return f16_bits(w >> 16); }

// binary32 -> bfloat16, round to nearest, ties to even (NaN stays a quiet NaN)
__device__ __forceinline__ uint16_t bf16_rne(float v) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// One element of a tensor whose type is a run-time (wave-uniform) value.
__device__ __forceinline__ void store_elem(void* base, int64_t i, float v, int dtype) {
    if (dtype == kBF16)
        static_cast<uint16_t*>(base)[i] = bf16_rne(v);
    else if (dtype == kF16)
        static_cast<_Float16*>(base)[i] = (_Float16)v;   // round to nearest even
    else
        static_cast<float*>(base)[i] = v;
}
__device__ __forceinline__ float load_elem(const void* base, int64_t i, int dtype) {
    if (dtype == kBF16) return __uint_as_float((uint32_t)static_cast<const uint16_t*>(base)[i] << 16);
    if (dtype == kF16) return (float)static_cast<const _Float16*>(base)[i];
    return static_cast<const float*>(base)[i];
}

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
struct VecLoad<uint16_t, 4> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff, float (&v)[4]) {
        auto q = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
        v[0] = bf16_lo(q[0]);
        v[1] = bf16_hi(q[0]);
        v[2] = bf16_lo(q[1]);
        v[3] = bf16_hi(q[1]);
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

template <>
struct VecLoad<_Float16, 1> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff, float (&v)[1]) {
        v[0] = f16_bits((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
    }
};

template <>
struct VecLoad<_Float16, 4> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff, float (&v)[4]) {
        auto q = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
        v[0] = f16_lo(q[0]);
        v[1] = f16_hi(q[0]);
        v[2] = f16_lo(q[1]);
        v[3] = f16_hi(q[1]);
    }
};

template <>
struct VecLoad<_Float16, 8> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff, float (&v)[8]) {
        auto q = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = f16_lo(q[e]);
            v[2 * e + 1] = f16_hi(q[e]);
        }
    }
};

// VEC consecutive 16-bit elements kept as the raw 32-bit words they arrive in
// (half the registers of floats), converted when used.
template <typename T, int VEC>
struct RawVec {
    static_assert(sizeof(T) == 2, "16-bit element types; binary32 is specialised below");
    static constexpr int kWords = VEC * (int)sizeof(T) / 4;
    static_assert(kWords >= 1, "at least one 32-bit word");
    uint32_t w[kWords];
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
        if constexpr (kWords == 4) {
            auto q = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = q[e];
        } else if constexpr (kWords == 2) {
            auto q = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
            w[0] = q[0];
            w[1] = q[1];
        } else {
            w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
        }
    }
    __device__ __forceinline__ void to_float(float (&v)[VEC]) const {
#pragma unroll
        for (int e = 0; e < kWords; ++e) {
            if constexpr (std::is_same<T, _Float16>::value) {
                v[2 * e] = f16_lo(w[e]);
                v[2 * e + 1] = f16_hi(w[e]);
            } else {
                v[2 * e] = bf16_lo(w[e]);
                v[2 * e + 1] = bf16_hi(w[e]);
            }
        }
    }
};

// binary32 rows stay floats, loaded as before (the same registers; storing them as
// words measured slower in the row-ordered gather)
template <int VEC>
struct RawVec<float, VEC> {
    float v[VEC];
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
        VecLoad<float, VEC>::run(r, voff, soff, v);
    }
    __device__ __forceinline__ void to_float(float (&o)[VEC]) const {
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = v[e];
    }
};

// Calls f(T{}) with T the element type of dtype: float, uint16_t (bfloat16) or
// _Float16.  Host side, to pick kernel instantiations.
template <typename F>
hipError_t with_elem(int dtype, F&& f) {
    switch (dtype) {
        case kBF16: return f(uint16_t{});
        case kF16: return f(_Float16{});
        default: return f(float{});
    }
}

struct FwdDesc {
    uint32_t off[4];   // byte offsets of the four corner rows in the feature image
    float cw[4];       // hh*hw, hh*lw, lh*hw, lh*lw
};
static_assert(sizeof(FwdDesc) == kFwdDescBytes, "FwdDesc layout");

struct BwdDesc {
    uint32_t off[4];   // feature image byte offsets
    uint32_t goff[4];  // feature-gradient image byte offsets (scatter path)
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

// The level table as read by one sample: straight from the kernel arguments
// (fine where the level is the same across a wave), or from a copy in LDS
// (where every lane may sit on a different level).
struct LevelsArg {
    const KArgs& a;
    __device__ __forceinline__ void get(int l, int32_t& H, int32_t& W, int32_t& st) const {
        H = a.lv.H[l];
        W = a.lv.W[l];
        st = a.lv.start[l];
    }
};
struct LevelsLds {
    const int32_t* hws;   // [3][kMaxLevels]: H, W, start
    __device__ __forceinline__ void get(int l, int32_t& H, int32_t& W, int32_t& st) const {
        H = hws[l];
        W = hws[kMaxLevels + l];
        st = hws[2 * kMaxLevels + l];
    }
};

// Copy the level table to LDS (every thread of the block must call this).
__device__ __forceinline__ LevelsLds stage_levels(const KArgs& a, int32_t* lds) {
    const int nlev = a.K * a.S;
    for (int i = threadIdx.x; i < nlev; i += blockDim.x) {
        lds[i] = a.lv.H[i];
        lds[kMaxLevels + i] = a.lv.W[i];
        lds[2 * kMaxLevels + i] = a.lv.start[i];
    }
    __syncthreads();
    return LevelsLds{lds};
}

template <typename Levels>
__device__ __forceinline__ Stencil make_stencil(const KArgs& a, int64_t ba, int t, const Levels& lv) {
    // t < P*K*S and ba < 2^23 are guaranteed by the host checks
    Stencil st;
    const int pk = t / a.S;
    const int s = t - pk * a.S;
    const int k = pk % a.K;
    const int lvl = k * a.S + s;
    int32_t H, W, start;
    lv.get(lvl, H, W, start);
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

__device__ __forceinline__ Stencil make_stencil(const KArgs& a, int64_t ba, int t) {
    return make_stencil(a, ba, t, LevelsArg{a});
}

__device__ __forceinline__ float xor_shfl(float v, int mask) { return __shfl_xor(v, mask, kWave); }

// v from lane (DPP control `ctrl`) in the rows of `row_mask`, 0 in the others.
template <int ctrl, int row_mask>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, row_mask, 0xF, false));
}

// Sum of v over each aligned group of n lanes (n a power of two, 1..64, the same
// in every lane).  The group's total ends up in its LAST lane; the other lanes
// hold partial sums.  Only gfx9 data-parallel-primitive forms whose source
// lane lies in the same group are used, so a group whose lanes are all active
// is summed correctly whatever the other groups of the wave do:
//   quad_perm [1,0,3,2] and [2,3,0,1] (lane xor 1, xor 2), row_half_mirror
//   (lane i <-> 7-i inside 8), row_mirror (i <-> 15-i inside 16): after these
//   every lane of a 16-lane row holds the row's total; row_bcast:15 then adds
//   row r-1's total into odd rows, and row_bcast:31 the total of rows 0-1 into
//   rows 2-3.
__device__ __forceinline__ float group_sum(float v, int n) {
    if (n > 1) v += dpp<0xB1, 0xF>(v);     // quad_perm [1,0,3,2]
    if (n > 2) v += dpp<0x4E, 0xF>(v);     // quad_perm [2,3,0,1]
    if (n > 4) v += dpp<0x141, 0xF>(v);    // row_half_mirror
    if (n > 8) v += dpp<0x140, 0xF>(v);    // row_mirror
    if (n > 16) v += dpp<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    if (n > 32) v += dpp<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return v;
}

// Sample j of level slice x (m levels): j = p * m + i takes point p at the
// slice's i-th level (k, s); returns t = (p * K + k) * S + s.  The order is
// fixed, so every sum over a slice's samples is deterministic.
__device__ __forceinline__ int slice_sample(const KArgs& a, int x, int m, int j) {
    const int p = j / m;
    const int l = a.lv.slice_level[x][j - p * m];
    const int k = l / a.S;
    const int s = l - k * a.S;
    return (p * a.K + k) * a.S + s;
}

// The same, with slice x's level list copied to LDS (`levels`, m entries).
__device__ __forceinline__ int slice_sample(const KArgs& a, const int32_t* levels, int m, int j) {
    const int p = j / m;
    const int l = levels[j - p * m];
    const int k = l / a.S;
    const int s = l - k * a.S;
    return (p * a.K + k) * a.S + s;
}

// Launch-shape bookkeeping common to the per-anchor kernels: one workgroup per
// (batch, anchor); row group rg = L consecutive lanes.
struct AnchorCtx {
    int64_t ba, b;
    int tid, nthreads, wave, lane, L, spw, rg, n_rg, li;
};

__device__ __forceinline__ AnchorCtx anchor_ctx(const KArgs& a) {
    AnchorCtx c;
    c.ba = blockIdx.x;
    c.b = (int64_t)(blockIdx.x / (uint32_t)a.A);
    c.tid = threadIdx.x;
    c.nthreads = blockDim.x;
    c.wave = c.tid / kWave;
    c.lane = c.tid % kWave;
    c.L = a.L;
    c.spw = kWave >> a.log2L;
    c.rg = c.wave * c.spw + (c.lane >> a.log2L);
    c.n_rg = (c.nthreads / kWave) * c.spw;
    c.li = c.lane & (c.L - 1);
    return c;
}

}  // namespace da
