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
// contiguous channels, DPP group sums).  Forward: a lane covers 16 bytes of one
// group's channels of one output pixel; blocks are laid out so that each XCD
// (workgroup i runs on XCD i mod 8) walks one contiguous band of output pixels,
// keeping the neighbourhoods it reads in its own L2.  Backward: workgroups own
// input tiles and sum their gradient in LDS (see below), so the scatter that the
// page's design does with one global atomic per term becomes LDS additions and
// one store per element.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
    if constexpr (VEC % 4 == 0) {
        if (a.out_vec4 && dtype == kF32) {                  // 16-byte stores
#pragma unroll
            for (int h = 0; h < VEC / 4; ++h)
                reinterpret_cast<float4*>(static_cast<float*>(out) + i)[h] =
                    make_float4(v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]);
            return;
        }
        if (a.out_vec4) {                                   // 16-bit: 8- or 16-byte stores
            uint32_t w[VEC / 2];
#pragma unroll
            for (int h = 0; h < VEC / 2; ++h) {
                const float x0 = v[2 * h], x1 = v[2 * h + 1];
                const uint32_t lo = dtype == kBF16 ? (uint32_t)bf16_rne(x0)
                                                   : (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x0);
                const uint32_t hi = dtype == kBF16 ? (uint32_t)bf16_rne(x1)
                                                   : (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x1);
                w[h] = lo | hi << 16;
            }
            uint16_t* o16 = static_cast<uint16_t*>(out) + i;
            if constexpr (VEC == 4) {
                *reinterpret_cast<uint2*>(o16) = make_uint2(w[0], w[1]);
            } else {
#pragma unroll
                for (int h = 0; h < VEC / 8; ++h)
                    reinterpret_cast<uint4*>(o16)[h] =
                        make_uint4(w[4 * h], w[4 * h + 1], w[4 * h + 2], w[4 * h + 3]);
            }
            return;
        }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) store_elem(out, i + e, v[e], dtype);
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
    if (a.K == 9 && NV == 1 && a.Lg >= 7) {
        // 3x3 kernel, a group spanning 7 lanes or more: lane j of the group loads
        // 16-byte chunk j of the group's 27 offsets and scalars (lanes 7 and up
        // none), and each tap takes its three values from the lanes holding them
        // (cross-lane permutes) -- the record is read once per group, not once per
        // lane.  Lanes of one group belong to one pixel, so all are active together.
        const __amdgpu_buffer_rsrc_t r_om = make_rsrc(a.om, a.om_bytes);
        const int lane = threadIdx.x % kWave;
        const int jg = lane & (a.Lg - 1), gbase = lane - jg;
        const uint32_t ro = ((uint32_t)L.pix * (uint32_t)a.G + (uint32_t)L.gq[0]) * 108u;
        float q4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (jg < 7) {
            const auto q = __builtin_amdgcn_raw_buffer_load_b128(r_om, ro + 16u * (uint32_t)jg, 0u, 0);
#pragma unroll
            for (int c = 0; c < 4; ++c) q4[c] = __uint_as_float(q[c]);
        }
#pragma unroll
        for (int k = 0; k < 9; ++k) {
            const int ki = k / 3, kj = k % 3;
            const int gy = L.ho * a.SH - a.PH + ki * a.DH;
            const int gx = L.wo * a.SW - a.PW + kj * a.DW;
            const float dx = __shfl(q4[(2 * k) % 4], gbase + (2 * k) / 4, kWave);
            const float dy = __shfl(q4[(2 * k + 1) % 4], gbase + (2 * k + 1) / 4, kWave);
            const float m = __shfl(q4[(18 + k) % 4], gbase + (18 + k) / 4, kWave);
            const DcnStencil st = dcn_stencil(a, L.n, gy, gx, dy, dx, L.c0[0], kElem);
            float v[4][VEC];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
                VecLoad<T, VEC>::run(r_in, L.valid[0] ? st.off[qq] : a.in_bytes, 0u, v[qq]);
            const float w0 = m * st.cw[0], w1 = m * st.cw[1], w2 = m * st.cw[2], w3 = m * st.cw[3];
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                acc[0][e] += w0 * v[0][e] + w1 * v[1][e] + w2 * v[2][e] + w3 * v[3][e];
        }
    } else if (a.K == 9) {
        // 3x3 kernel: a group's 27 offsets and scalars in seven 16-byte loads (the
        // 28th float is the next record's, or outside the buffer: zero), one group
        // at a time; each group's sum still runs over the taps in order
        const __amdgpu_buffer_rsrc_t r_om = make_rsrc(a.om, a.om_bytes);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float rec[28];
            const uint32_t ro = ((uint32_t)L.pix * (uint32_t)a.G + (uint32_t)L.gq[i]) * 108u;
#pragma unroll
            for (int j = 0; j < 7; ++j) {
                const auto q = __builtin_amdgcn_raw_buffer_load_b128(r_om, ro + 16u * j, 0u, 0);
                rec[4 * j] = __uint_as_float(q[0]);
                rec[4 * j + 1] = __uint_as_float(q[1]);
                rec[4 * j + 2] = __uint_as_float(q[2]);
                rec[4 * j + 3] = __uint_as_float(q[3]);
            }
#pragma unroll
            for (int k = 0; k < 9; ++k) {
                const int ki = k / 3, kj = k % 3;
                const int gy = L.ho * a.SH - a.PH + ki * a.DH;
                const int gx = L.wo * a.SW - a.PW + kj * a.DW;
                const DcnStencil st = dcn_stencil(a, L.n, gy, gx, rec[2 * k + 1], rec[2 * k], L.c0[i], kElem);
                float v[4][VEC];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    VecLoad<T, VEC>::run(r_in, L.valid[i] ? st.off[q] : a.in_bytes, 0u, v[q]);
                const float m = rec[18 + k];
                const float w0 = m * st.cw[0], w1 = m * st.cw[1], w2 = m * st.cw[2], w3 = m * st.cw[3];
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    acc[i][e] += w0 * v[0][e] + w1 * v[1][e] + w2 * v[2][e] + w3 * v[3][e];
            }
        }
    } else
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

// ------------------------------------------------------------------------------------
// backward by input tiles
// ------------------------------------------------------------------------------------
// Workgroup (n, ty, tx, g) owns the gradient of input pixels [Iy0, Iy0 + TY) x
// [Ix0, Ix0 + TX) (clipped to the image) in channel group g, summed in LDS and
// stored once.  The LDS sums are 64-bit fixed point: binary32 atomic addition in
// LDS runs several times slower than integer addition on this part, and exact
// integer sums also make each tile's result independent of the order of its
// terms.  A sample (output pixel, group, tap) has grid point (gy, gx) =
// (ho*SH - PH + i*DH, wo*SW - PW + j*DW); its home is the tile holding that point
// clamped into the image.  The home workgroup forms the sample's offset and scalar
// gradients and adds the corners that fall in its own tile.  A corner in another
// tile is added by that tile's workgroup when the grid point lies in the tile's
// window -- rows [Iy0 - M - 1, Iy0 + TY - 1 + M], columns alike, which
// holds every corner of a sample whose offsets are at most M -- through its ring
// loop; otherwise the home appends (sample, corner) to the far list, added by
// atomics after every tile is stored.

struct DcnRec {
    int32_t pix;        // output pixel
    float m;            // modulation scalar
    float ly, lx;       // fractions over the low corner
    int32_t y0, x0;     // low corner (meaningful when inside)
    uint32_t flags;     // bit 0 inside; bit 1 + q: corner q in the image; bit 5 + q: in this
                        // tile; bit 9 + q: far (no tile's ring reaches it; home samples only);
                        // kRecHome: a home sample to take (records shared within a quad)
};
constexpr uint32_t kRecHome = 1u << 31;

// Output indices o in [0, O) whose grid coordinate o*S - P + off lies in [lo, hi].
__device__ __forceinline__ void out_range(int lo, int hi, int S, int P, int off, int O, int& o_lo,
                                          int& o_hi) {
    const int a = lo + P - off, b = hi + P - off;
    o_lo = a <= 0 ? 0 : (a + S - 1) / S;
    o_hi = b < 0 ? -1 : min(b / S, O - 1);
}

struct TileCtx {
    int n, g, Iy0, Ix0, Iy1, Ix1;   // owned tile [Iy0, Iy1) x [Ix0, Ix1)
};

// The offsets (dx, dy) and the scalar of sample (pixel, group g, tap k).
struct DcnOm {
    float dx, dy, m;
};

// (every tensor of the operator is under 4 GiB: 32-bit element indices)
__device__ __forceinline__ DcnOm load_om(const DcnArgs& a, int pix, int g, int k) {
    const float* om = a.om + ((uint32_t)pix * (uint32_t)a.G + (uint32_t)g) * (uint32_t)(3 * a.K);
    return DcnOm{om[2 * k], om[2 * k + 1], om[2 * a.K + k]};
}

// Phase A of one sample with grid point (gy, gx): its stencil record.  For a home
// sample the corners that no other tile's ring reaches are flagged far: a corner's
// tile reaches the sample through its ring only when the grid point lies in that
// tile's window.  Tile sides are powers of two, and the flags are formed without
// branches, so the records of several samples are formed side by side.
__device__ __forceinline__ DcnRec dcn_record(const DcnArgs& a, const TileCtx& t, int pix, int gy,
                                             int gx, const DcnOm& o, bool home, int TY, int TX,
                                             int M) {
#pragma clang fp contract(off)
    DcnRec r;
    r.pix = pix;
    r.m = o.m;
    const float y = (float)gy + o.dy, x = (float)gx + o.dx;
    const bool inside = y > -1.0f && x > -1.0f && y < (float)a.H && x < (float)a.W;
    const float yf = inside ? floorf(y) : 0.0f, xf = inside ? floorf(x) : 0.0f;
    r.ly = inside ? y - yf : 0.0f;
    r.lx = inside ? x - xf : 0.0f;
    r.y0 = (int)yf;
    r.x0 = (int)xf;
    uint32_t f = inside ? 1u : 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int cy = r.y0 + (q >> 1), cx = r.x0 + (q & 1);
        const bool img = inside && cy >= 0 && cy < a.H && cx >= 0 && cx < a.W;
        const bool own = img && cy >= t.Iy0 && cy < t.Iy1 && cx >= t.Ix0 && cx < t.Ix1;
        f |= (img ? 1u : 0u) << (1 + q);
        f |= (own ? 1u : 0u) << (5 + q);
    }
    // With -M <= dy <= M every corner row cy satisfies gy - M <= cy <= gy + M + 1
    // (binary32 rounding of gy + dy is monotonic and gy +- M is exact), so gy lies
    // in the row window of the corner's tile; the same for x.  Only a sample with a
    // larger offset (or none at all) can have a far corner.
    const float fm = (float)M;
    if (home && !(o.dy >= -fm && o.dy <= fm && o.dx >= -fm && o.dx <= fm)) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int cy = r.y0 + (q >> 1), cx = r.x0 + (q & 1);
            const int oy = cy & -TY, ox = cx & -TX;         // origin of the corner's tile
            const bool reach = gy >= oy - M - 1 && gy <= oy + TY - 1 + M &&
                               gx >= ox - M - 1 && gx <= ox + TX - 1 + M;
            const bool img = f >> (1 + q) & 1u, own = f >> (5 + q) & 1u;
            f |= (img && !own && !reach ? 1u : 0u) << (9 + q);
        }
    }
    r.flags = f;
    return r;
}

// How the backward kernels read grad_out: element loads of the run-time type
// go_dtype, or (16-byte aligned rows, VEC a multiple of 4) vector loads of a width
// fixed at compile time -- binary32, or 16-bit (bfloat16 or binary16 by a
// wave-uniform test after the load) -- so that the binary32 loads of a sample issue
// with its corner loads, no branch on the type between them.
constexpr int kGoElem = 0, kGoVecF32 = 1, kGoVec16 = 2;

// grad_out[i .. i + VEC) in binary32
template <int VEC, int GOV>
__device__ __forceinline__ void load_go(const DcnArgs& a, uint32_t i, float (&go)[VEC]) {
    if constexpr (GOV != kGoElem) {
        static_assert(VEC % 4 == 0, "vector grad_out loads cover 4 channels or more");
        if constexpr (GOV == kGoVecF32) {
            const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.grad_out) + i);
#pragma unroll
            for (int h = 0; h < VEC / 4; ++h) {
                const float4 v = p[h];
                go[4 * h] = v.x;
                go[4 * h + 1] = v.y;
                go[4 * h + 2] = v.z;
                go[4 * h + 3] = v.w;
            }
        } else {
            const uint16_t* p16 = static_cast<const uint16_t*>(a.grad_out) + i;
            uint32_t w[VEC / 2];
            if constexpr (VEC == 4) {
                const uint2 q = *reinterpret_cast<const uint2*>(p16);
                w[0] = q.x;
                w[1] = q.y;
            } else {
#pragma unroll
                for (int h = 0; h < VEC / 8; ++h) {
                    const uint4 q = reinterpret_cast<const uint4*>(p16)[h];
                    w[4 * h] = q.x;
                    w[4 * h + 1] = q.y;
                    w[4 * h + 2] = q.z;
                    w[4 * h + 3] = q.w;
                }
            }
            const bool bf = a.go_dtype == kBF16;
#pragma unroll
            for (int h = 0; h < VEC / 2; ++h) {
                go[2 * h] = bf ? bf16_lo(w[h]) : f16_lo(w[h]);
                go[2 * h + 1] = bf ? bf16_hi(w[h]) : f16_hi(w[h]);
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) go[e] = load_elem(a.grad_out, i + e, a.go_dtype);
    }
}

__device__ __forceinline__ void corner_weights(const DcnRec& r, float (&cw)[4]) {
#pragma clang fp contract(off)
    const float hy = 1.0f - r.ly, hx = 1.0f - r.lx;
    const bool in = r.flags & 1u;
    cw[0] = in ? hy * hx : 0.0f;
    cw[1] = in ? hy * r.lx : 0.0f;
    cw[2] = in ? r.ly * hx : 0.0f;
    cw[3] = in ? r.ly * r.lx : 0.0f;
}

// Scale of the fixed-point tile sums.  Every term is cw * m * grad_out with
// cw <= 1, so |term| <= B = max|m| * max|grad_out|, and one tile sum takes at
// most 2^log2_terms terms: with E = 61 - (exponent of B) - log2_terms every sum
// stays below 2^61 and every term below 2^51 (log2_terms >= 10).  Rounding a term
// to RNE(t 2^E): adding 1.5 * 2^52 in binary64 puts t 2^E on the integer grid of
// the binade [2^52, 2^53), whose encoding is the integer plus a constant.
// One wave of 1024-thread blocks (one per CU): the blocks finish together, and each
// takes one ticket from a single counter, so fewer blocks shorten that tail.
constexpr int kBoundThreads = 1024;
constexpr int kBoundWaves = kBoundThreads / kWave;
constexpr int kBoundGrid = 256;

__global__ void __launch_bounds__(kBoundThreads) dcn_bound_kernel(DcnArgs a) {
    __shared__ uint32_t red[2][kBoundWaves];
    constexpr int U = 4;                    // loads in flight per thread
    // element counts are below 2^30 (every tensor is under 4 GiB)
    const uint32_t stride = gridDim.x * kBoundThreads;
    const uint32_t i0 = blockIdx.x * kBoundThreads + threadIdx.x;
    uint32_t mg = 0, mm = 0;
    const uint32_t n_go = (uint32_t)(a.n_pix * a.C);
    if (a.go_dtype == kF32 && a.go_vec4) {        // 16-byte loads (C % 4 == 0, aligned)
        const float4* g4 = static_cast<const float4*>(a.grad_out);
        const uint32_t n4 = n_go / 4;
        uint32_t i = i0;
        for (; i + (U - 1) * stride < n4; i += U * stride) {
            float4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = g4[i + u * stride];
#pragma unroll
            for (int u = 0; u < U; ++u)
                mg = max(mg, max(max(__float_as_uint(fabsf(v[u].x)), __float_as_uint(fabsf(v[u].y))),
                                 max(__float_as_uint(fabsf(v[u].z)), __float_as_uint(fabsf(v[u].w)))));
        }
        for (; i < n4; i += stride) {
            const float4 v = g4[i];
            mg = max(mg, max(max(__float_as_uint(fabsf(v.x)), __float_as_uint(fabsf(v.y))),
                             max(__float_as_uint(fabsf(v.z)), __float_as_uint(fabsf(v.w)))));
        }
    } else if (a.go_vec4 && (n_go & 7u) == 0) {      // 16-bit: 16-byte loads of 8 values
        const uint4* g8 = static_cast<const uint4*>(a.grad_out);
        const uint32_t n8 = n_go / 8;
        const bool bf = a.go_dtype == kBF16;
        auto take8 = [&](const uint4& q) {
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float x0 = bf ? bf16_lo(w[h]) : f16_lo(w[h]);
                const float x1 = bf ? bf16_hi(w[h]) : f16_hi(w[h]);
                mg = max(mg, max(__float_as_uint(fabsf(x0)), __float_as_uint(fabsf(x1))));
            }
        };
        uint32_t i = i0;
        for (; i + (U - 1) * stride < n8; i += U * stride) {
            uint4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = g8[i + u * stride];
#pragma unroll
            for (int u = 0; u < U; ++u) take8(v[u]);
        }
        for (; i < n8; i += stride) take8(g8[i]);
    } else {
        for (uint32_t i = i0; i < n_go; i += stride)
            mg = max(mg, __float_as_uint(fabsf(load_elem(a.grad_out, i, a.go_dtype))));
    }
    // the scalars: the last K of every 3K-float record, read as one coalesced stream
    // of 16-byte vectors; r tracks the record position of a vector's first float
    const uint32_t K3 = (uint32_t)(3 * a.K), K2 = (uint32_t)(2 * a.K);
    const uint32_t n_om = (uint32_t)(a.n_pix * a.G) * K3;
    if ((reinterpret_cast<uintptr_t>(a.om) & 15) == 0) {
        const float4* o4 = reinterpret_cast<const float4*>(a.om);
        const uint32_t n4 = n_om / 4;
        const uint32_t step = (stride * 4u) % K3;
        uint32_t r = (i0 * 4u) % K3;
        auto take = [&](const float4& v, uint32_t r0) {
            const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t pos = r0 + (uint32_t)e;
                pos = pos >= K3 ? pos - K3 : pos;
                // a select, not a branch, so that the loads stay unconditional
                mm = max(mm, pos >= K2 ? __float_as_uint(fabsf(f[e])) : 0u);
            }
        };
        auto advance = [&](uint32_t x) {
            x += step;
            return x >= K3 ? x - K3 : x;
        };
        uint32_t i = i0;
        for (; i + (U - 1) * stride < n4; i += U * stride) {
            float4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = o4[i + u * stride];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                take(v[u], r);
                r = advance(r);
            }
        }
        for (; i < n4; i += stride) {
            take(o4[i], r);
            r = advance(r);
        }
        for (uint32_t j = n4 * 4 + i0; j < n_om; j += stride)
            if (j % K3 >= K2) mm = max(mm, __float_as_uint(fabsf(a.om[j])));
    } else {
        for (uint32_t j = i0; j < n_om; j += stride)
            if (j % K3 >= K2) mm = max(mm, __float_as_uint(fabsf(a.om[j])));
    }
    for (int d = 1; d < kWave; d <<= 1) {
        mg = max(mg, (uint32_t)__shfl_xor((int)mg, d, kWave));
        mm = max(mm, (uint32_t)__shfl_xor((int)mm, d, kWave));
    }
    if (threadIdx.x % kWave == 0) {
        red[0][threadIdx.x / kWave] = mg;
        red[1][threadIdx.x / kWave] = mm;
    }
    __syncthreads();
    // the block's maxima into the (zeroed) control words: device-scope atomics, no
    // fence (the tile kernel reads them after this kernel ends); a maximum over
    // binary32 magnitudes is the maximum over their bit patterns
    if (threadIdx.x == 0) {
        for (int w = 1; w < kBoundWaves; ++w) {
            mg = max(mg, red[0][w]);
            mm = max(mm, red[1][w]);
        }
        atomicMax(a.ctrl + kDcnCtrlMaxGo, mg);
        atomicMax(a.ctrl + kDcnCtrlMaxM, mm);
    }
}

__device__ __forceinline__ int dcn_fixed_exponent(const DcnArgs& a) {
    const double b = (double)__uint_as_float(a.ctrl[kDcnCtrlMaxGo]) *
                     (double)__uint_as_float(a.ctrl[kDcnCtrlMaxM]);
    if (!(b > 0.0) || !(b < 1e300)) return 0;
    int e;
    frexp(b, &e);                       // b < 2^e
    return 61 - e - a.log2_terms;
}
constexpr double kFixMagicD = 6755399441055744.0;             // 1.5 * 2^52

// idx / n and idx % n for 0 <= idx < 2^24 and a wave-uniform n, by a float
// reciprocal corrected by one step (integer division costs tens of instructions)
__device__ __forceinline__ void divmod_small(int idx, int n, float inv, int& q, int& r) {
    q = (int)((float)idx * inv);
    r = idx - q * n;
    if (r < 0) {
        --q;
        r += n;
    } else if (r >= n) {
        ++q;
        r -= n;
    }
}

// group_sum of four values at once over groups of n lanes (a power of two): the
// set bits of n - 1 are the steps to take, tested on one scalar per step
__device__ __forceinline__ void group_sum4(float (&v)[4], int n) {
    const uint32_t steps = (uint32_t)n - 1u;
    if (steps & 1u)
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += dpp<0xB1, 0xF>(v[q]);     // quad_perm [1,0,3,2]
    if (steps & 2u)
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += dpp<0x4E, 0xF>(v[q]);     // quad_perm [2,3,0,1]
    if (steps & 4u)
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += dpp<0x141, 0xF>(v[q]);    // row_half_mirror
    if (steps & 8u)
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += dpp<0x140, 0xF>(v[q]);    // row_mirror
    if (steps & 16u)
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += dpp<0x142, 0xA>(v[q]);    // row_bcast:15
    if (steps & 32u)
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += dpp<0x143, 0xC>(v[q]);    // row_bcast:31
}

// Lanes: in the home loop a group of bLg lanes takes one sample at a time; lane jj
// covers the NVL vectors jj, jj + bLg, ... of VEC channels of the group, and every
// lane of the group forms the (cheap) stencil itself, so the waves never wait for
// one another.  The ring loop tests one candidate per lane and appends the accepted
// ones (a corner in this tile: about one candidate in eight for offsets of a pixel
// or so) to the wave's LDS list at their rank among the wave's accepted lanes; the
// list collects several taps' candidates before the lane groups take listed samples
// one at a time, so that their loads and additions run on full waves.
//
// Tile sums: a term t is added as the binary64 encoding of RNE(t 2^E) + 1.5 * 2^52,
// an integer in [2^52, 2^53) whose encoding is kFixMagicBits + RNE(t 2^E), and each
// tile pixel counts the terms it takes (the same count for every channel of the
// group: the group's first lane adds 1 per term).  The store subtracts
// count * kFixMagicBits modulo 2^64, which leaves the exact sum of the rounded terms.
constexpr unsigned long long kFixMagicBits = 0x4338000000000000ull;   // encoding of 1.5 * 2^52

// Tile shape and lane layout of the tile kernel: from the arguments, or (FIXED = 1)
// the compile-time shape that every group of 32 channels gets -- 8 x 16 pixels,
// pixel stride 33 words, 4 lanes per sample, margin 4 -- which frees the scalar
// registers those values and their products would hold.
template <int FIXED>
struct TileShape {
    int TY, TX, Dp, Lg, log2Lg, M;
    __device__ explicit TileShape(const DcnArgs& a)
        : TY(a.TY), TX(a.TX), Dp(a.Dp), Lg(a.bLg), log2Lg(a.blog2Lg), M(a.M) {}
};
template <>
struct TileShape<1> {
    static constexpr int TY = 8, TX = 16, Dp = 33, Lg = 4, log2Lg = 2, M = 4;
    __device__ explicit TileShape(const DcnArgs&) {}
};

template <typename T, int VEC, int NVL, int GOV, int FIXED>
__global__ void __launch_bounds__(kDcnTileThreads) __attribute__((amdgpu_waves_per_eu(6)))
dcn_bwd_tile_kernel(DcnArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const TileShape<FIXED> sh(a);
    const int TY = sh.TY, TX = sh.TX;
    unsigned long long* acc = reinterpret_cast<unsigned long long*>(smem);    // [TY*TX][Dp]
    uint32_t* cnt = reinterpret_cast<uint32_t*>(acc + TY * TX * sh.Dp);        // [TY*TX]
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    uint32_t* wl = cnt + TY * TX + wave * (kDcnListWords * kWave);
    const int E = dcn_fixed_exponent(a);
    const double scale = ldexp(1.0, E);

    // block -> (n, ty, tx, g), group fastest, neighbouring tiles on one XCD
    uint32_t lb = xcd_order(blockIdx.x, gridDim.x);
    TileCtx t;
    t.g = (int)(lb % (uint32_t)a.G);
    lb /= (uint32_t)a.G;
    const int tx = (int)(lb % (uint32_t)a.tiles_x);
    lb /= (uint32_t)a.tiles_x;
    const int ty = (int)(lb % (uint32_t)a.tiles_y);
    t.n = (int)(lb / (uint32_t)a.tiles_y);
    t.Iy0 = ty * TY;
    t.Ix0 = tx * TX;
    t.Iy1 = min(t.Iy0 + TY, a.H);
    t.Ix1 = min(t.Ix0 + TX, a.W);

    // (fixed shape) each tap's home range: h0, w0, nw, nh, oy, ox, 1 / nw
    int* taps = reinterpret_cast<int*>(cnt + TY * TX + kDcnBwdWaves * kDcnListWords * kWave);
    for (int i = tid; i < TY * TX * sh.Dp; i += kDcnTileThreads) acc[i] = 0ull;
    for (int i = tid; i < TY * TX; i += kDcnTileThreads) cnt[i] = 0u;
    if (FIXED == 1 && tid < a.K) {
        const int k = tid, ki = k / a.KW, kj = k - (k / a.KW) * a.KW;
        int h0, h1, w0, w1;
        out_range(t.Iy0 == 0 ? -(1 << 28) : t.Iy0, t.Iy1 == a.H ? (1 << 28) : t.Iy1 - 1, a.SH, a.PH,
                  ki * a.DH, a.Ho, h0, h1);
        out_range(t.Ix0 == 0 ? -(1 << 28) : t.Ix0, t.Ix1 == a.W ? (1 << 28) : t.Ix1 - 1, a.SW, a.PW,
                  kj * a.DW, a.Wo, w0, w1);
        const int nw = w1 - w0 + 1;
        const int nh = (h1 >= h0 && nw > 0) ? (h1 - h0 + 1) * nw : 0;
        *reinterpret_cast<int4*>(taps + 8 * k) = int4{h0, w0, nw, nh};
        *reinterpret_cast<int4*>(taps + 8 * k + 4) =
            int4{ki * a.DH - a.PH, kj * a.DW - a.PW, __float_as_int(nw > 0 ? 1.0f / (float)nw : 0.0f), 0};
    }
    __syncthreads();

    const int jj = tid & (sh.Lg - 1), slot = tid >> sh.log2Lg, spp = kDcnTileThreads >> sh.log2Lg;
    int cl[NVL];             // channel offsets inside the group
    bool vv[NVL];
#pragma unroll
    for (int u = 0; u < NVL; ++u) {
        const int vi = jj + sh.Lg * u;
        vv[u] = FIXED == 1 || vi < a.Dv;   // (the fixed shape's vectors fill the group)
        cl[u] = vv[u] ? vi * VEC : 0;
    }
    const uint32_t gD = (uint32_t)(t.g * a.D);
    const __amdgpu_buffer_rsrc_t r_in = make_rsrc(a.input, a.in_bytes);
    constexpr int kElem = (int)sizeof(T);
    const bool last = jj == sh.Lg - 1;
    // byte steps from corner 0 to corner q, and of the lane's vectors
    const uint32_t cq[4] = {0u, (uint32_t)(a.C * kElem), (uint32_t)(a.W * a.C * kElem),
                            (uint32_t)((a.W + 1) * a.C * kElem)};
    uint32_t clb[NVL], vvm[NVL];
#pragma unroll
    for (int u = 0; u < NVL; ++u) {
        clb[u] = (uint32_t)(cl[u] * kElem);
        vvm[u] = vv[u] ? ~0u : 0u;
    }

    // the terms of R's corners that lie in this tile; gd: the lane's grad_out values
    // in binary64 (idle vectors add nothing)
    // tile-pixel and sum-row steps from corner 0 to corner q
    const int dpq[4] = {0, 1, TX, TX + 1};
    const int dpr[4] = {0, sh.Dp, TX * sh.Dp, (TX + 1) * sh.Dp};
    auto add_tile = [&](const DcnRec& R, const float (&cw)[4], const double (&gd)[NVL][VEC]) {
        const int pb = (R.y0 - t.Iy0) * TX + (R.x0 - t.Ix0);   // corner 0 (may lie outside)
        const int rb = pb * sh.Dp;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (!(R.flags >> (5 + q) & 1u)) continue;
            if (jj == 0) atomicAdd(&cnt[pb + dpq[q]], 1u);   // once per term
            const double ws = (double)(cw[q] * R.m) * scale;
            unsigned long long* row = acc + (rb + dpr[q]);
#pragma unroll
            for (int u = 0; u < NVL; ++u) {
                if (!vv[u]) continue;
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    atomicAdd(&row[cl[u] + e], (unsigned long long)__double_as_longlong(
                                                   fma(gd[u][e], ws, kFixMagicD)));
            }
        }
    };

    // ---- home samples: offset / scalar gradients, corners in this tile ----
    // One home sample R of tap k: the group's loads, its offset and scalar
    // gradients, and its corners in this tile.
    auto home_sample = [&](const DcnRec& R, int k) {
        if (jj == 0 && (R.flags >> 9 & 0xfu)) {       // far corners (rare): listed
            const uint32_t sid = ((uint32_t)R.pix * (uint32_t)a.G + (uint32_t)t.g) *
                                     (uint32_t)a.K + (uint32_t)k;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (R.flags >> (9 + q) & 1u) a.fb[atomicAdd(a.ctrl + kDcnCtrlFar, 1u)] = sid * 4u + q;
        }
        // byte offset of corner 0's group channels (modulo 2^32: a corner outside
        // the image is never addressed, and the others come out in range)
        const uint32_t ib0 =
            (((uint32_t)(t.n * a.H + R.y0) * (uint32_t)a.W + (uint32_t)R.x0) * (uint32_t)a.C + gD) *
            (uint32_t)kElem;
        float go[NVL][VEC];
        float v[NVL][4][VEC];
#pragma unroll
        for (int u = 0; u < NVL; ++u) {
            load_go<VEC, GOV>(a, (uint32_t)R.pix * (uint32_t)a.C + gD + cl[u], go[u]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // all ones when the corner is in the image and the vector exists
                const uint32_t m = (0u - (R.flags >> (1 + q) & 1u)) & vvm[u];
                const uint32_t off = ((ib0 + cq[q] + clb[u]) & m) | (a.in_bytes & ~m);
                VecLoad<T, VEC>::run(r_in, off, 0u, v[u][q]);
            }
        }
        // S_q = sum over the group's channels of grad_out * corner q: the value,
        // x- and y-derivative sums are fixed combinations of the four
        float cw[4];
        corner_weights(R, cw);
        float S[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        double gd[NVL][VEC];
#pragma unroll
        for (int u = 0; u < NVL; ++u) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float g = vv[u] ? go[u][e] : 0.0f;
                gd[u][e] = (double)g;
#pragma unroll
                for (int q = 0; q < 4; ++q) S[q] += g * v[u][q][e];
            }
        }
        group_sum4(S, sh.Lg);
        if (last) {
            const bool live = R.flags & 1u;
            const float hy = 1.0f - R.ly, hx = 1.0f - R.lx;
            const float px = hy * (S[1] - S[0]) + R.ly * (S[3] - S[2]);
            const float py = hx * (S[2] - S[0]) + R.lx * (S[3] - S[1]);
            const float pm = cw[0] * S[0] + cw[1] * S[1] + cw[2] * S[2] + cw[3] * S[3];
            float* gom = a.grad_om + ((uint32_t)R.pix * (uint32_t)a.G + (uint32_t)t.g) *
                                         (uint32_t)(3 * a.K);
            gom[2 * k] = live ? R.m * px : 0.0f;
            gom[2 * k + 1] = live ? R.m * py : 0.0f;
            gom[2 * a.K + k] = live ? pm : 0.0f;
        }
        add_tile(R, cw, gd);
    };
    if constexpr (FIXED == 1) {
        // A lane group is one quad.  Lane jj of a quad forms the record of tap
        // k0 + jj at the quad's slot and puts it in the wave's list area (pixel,
        // scalar, position, flags); the quad then takes the (up to) four samples one
        // at a time, every lane reading the record back: each stencil is formed
        // once instead of once per lane of its group.  The list area is written and
        // read by this wave only (as in the ring pass below).
        static_assert(TileShape<1>::Lg == 4, "lane groups of four lanes");
        for (int k0 = 0; k0 < a.K; k0 += 4) {
            const int kk = k0 + jj;
            // the largest of the four taps' counts (every quad holds the same taps)
            int nmax = kk < a.K ? taps[8 * kk + 3] : 0;
            nmax = max(nmax, __builtin_amdgcn_update_dpp(0, nmax, 0xB1, 0xF, 0xF, false));
            nmax = max(nmax, __builtin_amdgcn_update_dpp(0, nmax, 0x4E, 0xF, 0xF, false));
            nmax = __builtin_amdgcn_readfirstlane(nmax);
            for (int idx = slot; idx < nmax; idx += spp) {
                uint32_t pix = 0u, flags = 0u;
                float m = 0.0f, y = 0.0f, x = 0.0f;
                if (kk < a.K) {
                    const int4 tr = *reinterpret_cast<const int4*>(taps + 8 * kk);   // h0 w0 nw nh
                    if (idx < tr.w) {
                        const int4 to = *reinterpret_cast<const int4*>(taps + 8 * kk + 4);
                        int oh, ow;
                        divmod_small(idx, tr.z, __int_as_float(to.z), oh, ow);
                        const int gy = (tr.x + oh) * a.SH + to.x, gx = (tr.y + ow) * a.SW + to.y;
                        pix = (uint32_t)((t.n * a.Ho + tr.x + oh) * a.Wo + tr.y + ow);
                        const DcnOm o = load_om(a, (int)pix, t.g, kk);
                        const DcnRec R = dcn_record(a, t, (int)pix, gy, gx, o, true, TY, TX, sh.M);
                        m = o.m;
                        y = (float)gy + o.dy;
                        x = (float)gx + o.dx;
                        flags = R.flags | kRecHome;
                    }
                }
                __builtin_amdgcn_wave_barrier();
                wl[lane] = pix;
                wl[kWave + lane] = __float_as_uint(m);
                wl[2 * kWave + lane] = __float_as_uint(y);
                wl[3 * kWave + lane] = __float_as_uint(x);
                wl[4 * kWave + lane] = flags;
                __builtin_amdgcn_wave_barrier();
#pragma unroll 1
                for (int j = 0; j < 4; ++j) {
                    if (k0 + j >= a.K) break;
                    const int src = (lane & ~3) | j;
                    DcnRec Q;
                    Q.flags = wl[4 * kWave + src];
                    if (Q.flags & kRecHome) {
                        // corner 0 and fractions from the position, as the record has them
                        const float qy = __uint_as_float(wl[2 * kWave + src]);
                        const float qx = __uint_as_float(wl[3 * kWave + src]);
                        const bool inside = Q.flags & 1u;
                        const float yf = inside ? floorf(qy) : 0.0f, xf = inside ? floorf(qx) : 0.0f;
                        Q.pix = (int)wl[src];
                        Q.m = __uint_as_float(wl[kWave + src]);
                        Q.ly = inside ? qy - yf : 0.0f;
                        Q.lx = inside ? qx - xf : 0.0f;
                        Q.y0 = (int)yf;
                        Q.x0 = (int)xf;
                        home_sample(Q, k0 + j);
                    }
                }
                __builtin_amdgcn_wave_barrier();     // the list is rewritten next
            }
        }
    } else {
        for (int k = 0; k < a.K; ++k) {
            const int ki = k / a.KW, kj = k - (k / a.KW) * a.KW;
            const int oy = ki * a.DH - a.PH, ox = kj * a.DW - a.PW;
            int h0, h1, w0, w1;
            out_range(t.Iy0 == 0 ? -(1 << 28) : t.Iy0, t.Iy1 == a.H ? (1 << 28) : t.Iy1 - 1, a.SH,
                      a.PH, ki * a.DH, a.Ho, h0, h1);
            out_range(t.Ix0 == 0 ? -(1 << 28) : t.Ix0, t.Ix1 == a.W ? (1 << 28) : t.Ix1 - 1, a.SW,
                      a.PW, kj * a.DW, a.Wo, w0, w1);
            const int nw = w1 - w0 + 1;
            const int nh = (h1 >= h0 && nw > 0) ? (h1 - h0 + 1) * nw : 0;
            const float inv_nw = nw > 0 ? 1.0f / (float)nw : 0.0f;
            for (int idx = slot; idx < nh; idx += spp) {
                int oh, ow;
                divmod_small(idx, nw, inv_nw, oh, ow);
                const int pix = (t.n * a.Ho + h0 + oh) * a.Wo + w0 + ow;
                home_sample(dcn_record(a, t, pix, (h0 + oh) * a.SH + oy, (w0 + ow) * a.SW + ox,
                                       load_om(a, pix, t.g, k), true, TY, TX, sh.M),
                            k);
            }
        }
    }

    // ---- ring: other tiles' samples whose grid point lies in this tile's window ----
    const int gpw = kWave >> sh.log2Lg;              // lane groups per wave
    const int grp = lane >> sh.log2Lg;
    // The wave's list collects the accepted candidates of every tap and is drained
    // (each lane group taking listed samples one at a time) only when the next batch
    // would not fit, and once at the end: one tap accepts only a few candidates per
    // wave, and draining after each would leave most lane groups idle.  The list is
    // written and read by this wave only, and LDS executes one wave's instructions
    // in order: no barrier, only no reordering across the writes and reads.
    int n_list = 0;                                  // wave-uniform
    auto drain = [&]() {
        __builtin_amdgcn_wave_barrier();
        // lane r forms the record of entry r in place (the test pass keeps only the
        // pixel, the tap and the position): scalar, fractions, low corner relative
        // to the tile and the in-tile corner bits -- an accepted sample lies inside
        // the image, and every corner in the tile is in the image
        if (lane < n_list) {
            const uint32_t pix = wl[lane];
            const int k = (int)wl[kWave + lane];
            const float y = __uint_as_float(wl[2 * kWave + lane]);
            const float x = __uint_as_float(wl[3 * kWave + lane]);
            const float m = a.om[(pix * (uint32_t)a.G + (uint32_t)t.g) * (uint32_t)(3 * a.K) +
                                 (uint32_t)(2 * a.K + k)];
            const float yf = floorf(y), xf = floorf(x);
            const int y0 = (int)yf, x0 = (int)xf;
            uint32_t f = 1u;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int cy = y0 + (q >> 1), cx = x0 + (q & 1);
                const bool own = cy >= t.Iy0 && cy < t.Iy1 && cx >= t.Ix0 && cx < t.Ix1;
                f |= (own ? 1u : 0u) << (5 + q);
            }
            wl[kWave + lane] = __float_as_uint(m);
            wl[2 * kWave + lane] = __float_as_uint(y - yf);
            wl[3 * kWave + lane] = __float_as_uint(x - xf);
            wl[4 * kWave + lane] = (uint32_t)(y0 - t.Iy0 + 1) | (uint32_t)(x0 - t.Ix0 + 1) << 8 | f << 16;
        }
        __builtin_amdgcn_wave_barrier();
        for (int r = grp; r < n_list; r += gpw) {
            DcnRec L;
            L.pix = (int)wl[r];
            L.m = __uint_as_float(wl[kWave + r]);
            L.ly = __uint_as_float(wl[2 * kWave + r]);
            L.lx = __uint_as_float(wl[3 * kWave + r]);
            const uint32_t pk = wl[4 * kWave + r];
            L.y0 = (int)(pk & 0xffu) - 1 + t.Iy0;
            L.x0 = (int)(pk >> 8 & 0xffu) - 1 + t.Ix0;
            L.flags = pk >> 16;
            float cw[4];
            corner_weights(L, cw);
            double gd[NVL][VEC];
#pragma unroll
            for (int u = 0; u < NVL; ++u) {
                float go[VEC];
                if (vv[u]) {
                    load_go<VEC, GOV>(a, (uint32_t)L.pix * (uint32_t)a.C + gD + cl[u], go);
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) go[e] = 0.0f;
                }
#pragma unroll
                for (int e = 0; e < VEC; ++e) gd[u][e] = (double)go[e];
            }
            add_tile(L, cw, gd);
        }
        __builtin_amdgcn_wave_barrier();            // the list is rewritten next
        n_list = 0;
    };
    for (int k = 0; k < a.K; ++k) {
        const int ki = k / a.KW, kj = k - (k / a.KW) * a.KW;
        const int oy = ki * a.DH - a.PH, ox = kj * a.DW - a.PW;
        int h0, h1, w0, w1;
        out_range(t.Iy0 - sh.M - 1, t.Iy0 + TY - 1 + sh.M, a.SH, a.PH, ki * a.DH, a.Ho, h0, h1);
        out_range(t.Ix0 - sh.M - 1, t.Ix0 + TX - 1 + sh.M, a.SW, a.PW, kj * a.DW, a.Wo, w0, w1);
        const int nw = w1 - w0 + 1;
        const int nh = (h1 >= h0 && nw > 0) ? (h1 - h0 + 1) * nw : 0;
        const float inv_nw = nw > 0 ? 1.0f / (float)nw : 0.0f;
        for (int base = wave * kWave; base < nh; base += kDcnTileThreads) {    // wave-uniform
            const int idx = base + lane;
            int oh, ow;
            divmod_small(idx < nh ? idx : base, nw, inv_nw, oh, ow);
            const int gy = (h0 + oh) * a.SH + oy, gx = (w0 + ow) * a.SW + ox;
            const int pix = (t.n * a.Ho + h0 + oh) * a.Wo + w0 + ow;
            const int cy = min(max(gy, 0), a.H - 1), cx = min(max(gx, 0), a.W - 1);
            const bool cand = idx < nh && !(cy >= t.Iy0 && cy < t.Iy1 && cx >= t.Ix0 && cx < t.Ix1);
            // A candidate has a corner in this tile exactly when it lies inside the
            // image (as the record defines it) with its low corner in rows
            // [Iy0 - 1, Iy1 - 1] and columns [Ix0 - 1, Ix1 - 1]: only the offsets
            // are read here, the record is formed when the list is drained.
            float y = 0.0f, x = 0.0f;
            bool take = false;
            if (cand) {
                const float* om = a.om + ((uint32_t)pix * (uint32_t)a.G + (uint32_t)t.g) *
                                             (uint32_t)(3 * a.K);
                y = (float)gy + om[2 * k + 1];
                x = (float)gx + om[2 * k];
                take = y > -1.0f && x > -1.0f && y < (float)a.H && x < (float)a.W &&
                       y >= (float)(t.Iy0 - 1) && y < (float)t.Iy1 && x >= (float)(t.Ix0 - 1) &&
                       x < (float)t.Ix1;
            }
            const unsigned long long mask = __ballot(take);
            const int n_take = __popcll(mask);
            if (n_list + n_take > kWave) drain();
            if (take) {
                const int r = n_list + (int)__builtin_amdgcn_mbcnt_hi(
                    (uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
                wl[r] = (uint32_t)pix;
                wl[kWave + r] = (uint32_t)k;
                wl[2 * kWave + r] = __float_as_uint(y);
                wl[3 * kWave + r] = __float_as_uint(x);
            }
            n_list += n_take;
        }
    }
    drain();

    // ---- store the tile ----
    __syncthreads();
    const double inv = ldexp(1.0, -E);
    const int cols = t.Ix1 - t.Ix0, npx = (t.Iy1 - t.Iy0) * cols;
    for (int i = tid; i < npx * a.D; i += kDcnTileThreads) {
        const int p = i / a.D, c = i - (i / a.D) * a.D;
        const int py = p / cols, px = p - (p / cols) * cols;
        const int tp = py * TX + px;
        const long long code =
            (long long)(acc[tp * sh.Dp + c] -
                        (unsigned long long)cnt[tp] * kFixMagicBits);
        a.grad_input[(((int64_t)t.n * a.H + t.Iy0 + py) * a.W + t.Ix0 + px) * a.C + gD + c] =
            (float)((double)code * inv);
    }
}

// The far list: corner q of sample s gets cw_q * m * grad_out by atomics (after every
// tile has been stored).  Lg lanes per entry, a grid-stride loop over the entries.
template <typename T, int VEC, int NVL, int GOV>
__global__ void __launch_bounds__(kDcnThreads) dcn_far_kernel(DcnArgs a) {
#pragma clang fp contract(off)
    const uint32_t count = a.ctrl[kDcnCtrlFar];
    const int jj = threadIdx.x & (a.bLg - 1);
    const __amdgpu_buffer_rsrc_t r_gi = make_rsrc(a.grad_input, a.gi_bytes);
    const uint32_t per_block = kDcnThreads >> a.blog2Lg;
    for (uint32_t e = blockIdx.x * per_block + (threadIdx.x >> a.blog2Lg); e < count;
         e += gridDim.x * per_block) {
        const uint32_t ent = a.fb[e];
        const int q = (int)(ent & 3u);
        uint32_t s = ent >> 2;
        const int k = (int)(s % (uint32_t)a.K);
        s /= (uint32_t)a.K;
        const int g = (int)(s % (uint32_t)a.G);
        const int pix = (int)(s / (uint32_t)a.G);
        const int wo = pix % a.Wo, ho = (pix / a.Wo) % a.Ho, n = pix / (a.Wo * a.Ho);
        const int ki = k / a.KW, kj = k - (k / a.KW) * a.KW;
        TileCtx t{n, g, 0, 0, 0, 0};            // empty tile: no corner counts as owned
        const DcnRec R = dcn_record(a, t, pix, ho * a.SH - a.PH + ki * a.DH,
                                    wo * a.SW - a.PW + kj * a.DW, load_om(a, pix, g, k), false,
                                    a.TY, a.TX, a.M);
        float cw[4];
        corner_weights(R, cw);
        const float w = cw[q] * R.m;
#pragma unroll
        for (int u = 0; u < NVL; ++u) {
            const int vi = jj + a.bLg * u;
            if (vi >= a.Dv) continue;
            const int c0 = g * a.D + vi * VEC;
            const uint32_t goff =
                (uint32_t)(((int64_t)(n * a.H + R.y0 + (q >> 1)) * a.W + R.x0 + (q & 1)) * a.C + c0) * 4u;
            float go[VEC];
            load_go<VEC, GOV>(a, (uint32_t)pix * (uint32_t)a.C + (uint32_t)c0, go);
#pragma unroll
            for (int e2 = 0; e2 < VEC; ++e2)
                __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(w * go[e2], r_gi, goff + 4u * e2, 0, 0);
        }
    }
}

template <typename T, int VEC, int NV>
hipError_t dcn_fwd_launch(const DcnArgs& a, hipStream_t st) {
    const int64_t ppw = kWave / a.Lp;
    const int64_t blocks = (a.n_pix + ppw * kDcnWaves - 1) / (ppw * kDcnWaves);
    hipLaunchKernelGGL((dcn_forward_kernel<T, VEC, NV>), dim3((unsigned)blocks), dim3(kDcnThreads),
                       0, st, a);
    return hipGetLastError();
}

template <typename T, int VEC>
hipError_t dcn_fwd_dispatch_nv(const DcnArgs& a, int nv, hipStream_t st) {
    switch (nv) {
        case 1: return dcn_fwd_launch<T, VEC, 1>(a, st);
        case 2: return dcn_fwd_launch<T, VEC, 2>(a, st);
        case 4: return dcn_fwd_launch<T, VEC, 4>(a, st);
        case 8: return dcn_fwd_launch<T, VEC, 8>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, int VEC, int NVL, int GOV>
hipError_t dcn_bwd_launch(const DcnArgs& a, size_t lds, hipStream_t st) {
    const unsigned blocks = (unsigned)((int64_t)a.N * a.tiles_y * a.tiles_x * a.G);
    hipLaunchKernelGGL(dcn_bound_kernel, dim3(kBoundGrid), dim3(kBoundThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.TY == TileShape<1>::TY && a.TX == TileShape<1>::TX && a.Dp == TileShape<1>::Dp &&
        a.bLg == TileShape<1>::Lg && a.blog2Lg == TileShape<1>::log2Lg && a.M == TileShape<1>::M &&
        a.K <= kDcnShareTaps && a.Dv == TileShape<1>::Lg * NVL)
        hipLaunchKernelGGL((dcn_bwd_tile_kernel<T, VEC, NVL, GOV, 1>), dim3(blocks),
                           dim3(kDcnTileThreads), lds, st, a);
    else
        hipLaunchKernelGGL((dcn_bwd_tile_kernel<T, VEC, NVL, GOV, 0>), dim3(blocks),
                           dim3(kDcnTileThreads), lds, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dcn_far_kernel<T, VEC, NVL, GOV>), dim3(1024), dim3(kDcnThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dcn_forward(const DcnArgs& a, int in_dtype, int vec, int nv, hipStream_t stream) {
    if (a.n_pix == 0) return hipSuccess;
    return with_elem(in_dtype, [&](auto t) {
        using T = decltype(t);
        constexpr int V = sizeof(T) == 2 ? 8 : 4;
        return vec == V ? dcn_fwd_dispatch_nv<T, V>(a, nv, stream)
                        : dcn_fwd_dispatch_nv<T, 1>(a, nv, stream);
    });
}

hipError_t launch_dcn_backward(const DcnArgs& a, int in_dtype, int vec, size_t lds_bytes,
                               hipStream_t stream) {
    if (a.n_pix == 0)       // no output pixel: the input gradient is zero
        return launch_fill_zero(a.grad_input, (int64_t)a.N * a.H * a.W * a.C, stream);
    const hipError_t e = launch_fill_zero(a.ctrl, 4, stream);
    if (e != hipSuccess) return e;
    // vectors per lane (the host's choice)
    auto by_nvl = [&](auto tv, auto vv, auto gv) -> hipError_t {
        using T = decltype(tv);
        constexpr int V = decltype(vv)::value;
        constexpr int G = decltype(gv)::value;
        switch (a.bNVL) {
            case 1: return dcn_bwd_launch<T, V, 1, G>(a, lds_bytes, stream);
            case 2:       // two vectors per lane only where a vector holds 4 channels or fewer
                if constexpr (V <= 4) return dcn_bwd_launch<T, V, 2, G>(a, lds_bytes, stream);
                return hipErrorInvalidValue;
            default: return hipErrorInvalidValue;
        }
    };
    using I1 = std::integral_constant<int, 1>;
    using GoE = std::integral_constant<int, kGoElem>;
    using GoF = std::integral_constant<int, kGoVecF32>;
    using GoH = std::integral_constant<int, kGoVec16>;
    return with_elem(in_dtype, [&](auto t) {
        using T = decltype(t);
        using V = std::integral_constant<int, sizeof(T) == 2 ? 8 : 4>;
        if (vec == V::value && a.go_vec4)
            return a.go_dtype == kF32 ? by_nvl(t, V{}, GoF{}) : by_nvl(t, V{}, GoH{});
        if (vec == V::value) return by_nvl(t, V{}, GoE{});
        return by_nvl(t, I1{}, GoE{});
    });
}

}  // namespace da
