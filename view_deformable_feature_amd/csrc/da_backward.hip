// gfx950 (CDNA4) backward kernels of Sparse4D-style deformable aggregation.
//
// Definition: the Sparse4D deformable_aggregation walkthrough
// (mhpn.cn/news/1081857), section 4.1: with top = grad_out * weight, every
// inside corner receives corner weight * top in the feature gradient; the
// location gradient is W * (lh (v4 - v3) + hh (v2 - v1)) * top for x and
// H * (lw (v4 - v2) + hw (v3 - v1)) * top for y; the weight gradient adds
// grad_out * sampled value over the group's channels.
//
// The page adds every feature-gradient term with an atomic.  On MI355X a
// binary32 atomic add retires at about a fifth of the rate of a plain store
// to the same rows, which would make those atomics the whole cost of the
// pass.  So the default path turns the scatter into a gather:
//   1. count:   one thread per sample; each inside corner takes a rank in its
//               feature row with a 32-bit integer atomic on a per-row counter;
//   2. scan:    exclusive prefix of the counts (tiles of 4096 rows, then the
//               tile totals) gives each row's first entry;
//   3. anchor:  one workgroup per (batch, anchor) gathers the corner values as
//               the forward does, reduces the location and weight gradients
//               across lanes (stored once, no atomics) and writes each
//               (sample, corner) entry into its row's bucket;
//   4. gather:  each wave sums a fixed-size chunk of the row-sorted entries,
//               lanes over channels, and writes every row it owns with a plain
//               store; only a row split between two chunks is added with
//               atomics (at most two per chunk).
// The scatter form (binary32 atomics straight into the feature gradient) is
// kept for callers that cannot provide the workspace.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "da_device.h"

namespace da {
namespace {

// ------------------------------------------------------------------------------------
// per-anchor kernel
// ------------------------------------------------------------------------------------
// Lane li of a row group covers vectors li, li + L, ... of VEC consecutive
// channels (VEC = 1 in the scatter form, so that each atomic instruction
// covers 64 consecutive floats).  Each row group walks its (point, camera)
// pairs and, inside each, the S scales; the location gradient of a pair is
// reduced and stored after its last scale.  The loop is software-pipelined two
// deep: the next sample's corner values are requested before the current
// sample is processed (so a wait on loads never waits for atomics issued
// earlier -- the memory counter retires in order), and past the last sample
// the prefetch reads the null descriptor (offsets outside the buffer: zeros,
// no memory traffic).
//
// Per vector i and corner c, dot_c = sum_e grad_out[e] * v_c[e] gives both
// terms that need the corner values: the location partial w * dot_c and the
// weight-gradient partial sum_c cw_c * dot_c.  The weight gradient of a group
// is then summed over `seg` lanes (seg = D / VEC when one row of L lanes spans
// several groups, seg = L otherwise).
template <typename T, int VEC, int NV>
__device__ __forceinline__ void bwd_load(const __amdgpu_buffer_rsrc_t& r, const BwdDesc& d,
                                         uint32_t lane_off, const uint32_t (&soff)[NV],
                                         float (&v)[NV][4][VEC]) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) VecLoad<T, VEC>::run(r, d.off[c] + lane_off, soff[i], v[i][c]);
}

__device__ __forceinline__ BwdDesc null_bwd_desc(uint32_t outside, uint32_t goutside) {
    BwdDesc d;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        d.off[i] = outside;
        d.goff[i] = goutside;
        d.cw[i] = 0.0f;
        d.gx[i] = 0.0f;
        d.gy[i] = 0.0f;
    }
    return d;
}

__device__ __forceinline__ uint32_t row_first_entry(const KArgs& a, uint32_t flat_row) {
    return a.tile_prefix[flat_row / (uint32_t)kScanTile] + a.local_start[flat_row];
}

template <typename T, int VEC, int NV, bool SCATTER>
__global__ void __launch_bounds__(kWave * kMaxWaves)
da_backward_anchor_kernel(KArgs a) {
    static_assert(!SCATTER || VEC == 1, "the scatter form uses one channel per lane");
    extern __shared__ __align__(16) unsigned char smem[];
    const AnchorCtx x = anchor_ctx(a);
    const int64_t ba = x.ba, b = x.b;
    const int L = x.L, li = x.li, rg = x.rg, n_rg = x.n_rg;
    const int seg = a.seg;
    const int S = a.S;
    constexpr int kElem = (int)sizeof(T);

    const int ns_max = a.pk_chunk * S;           // desc[ns_max] is the null descriptor
    BwdDesc* desc = reinterpret_cast<BwdDesc*>(smem);
    float* wts = reinterpret_cast<float*>(smem + (size_t)(ns_max + 1) * sizeof(BwdDesc));

    const __amdgpu_buffer_rsrc_t rf = make_rsrc(
        static_cast<const unsigned char*>(a.feat) + b * a.feat_batch_bytes, a.feat_image_bytes);
    const __amdgpu_buffer_rsrc_t rgr = make_rsrc(
        reinterpret_cast<unsigned char*>(a.grad_feat) + b * a.gfeat_batch_bytes,
        a.gfeat_image_bytes);

    const uint32_t lane_off = (uint32_t)(li * VEC * kElem);
    const uint32_t lane_goff = (uint32_t)(li * 4);
    uint32_t soff[NV];
    float go[NV][VEC];
    int gi[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c0 = (li + L * i) * VEC;
        soff[i] = (uint32_t)(L * i * VEC * kElem);
        gi[i] = c0 / a.D;
#pragma unroll
        for (int e = 0; e < VEC; ++e) go[i][e] = a.grad_out[ba * a.C + c0 + e];
    }

    if (x.tid == 0) desc[ns_max] = null_bwd_desc(a.feat_image_bytes, a.gfeat_image_bytes);
    const int64_t wbase = ba * (int64_t)a.npk * S * a.G;
    const uint32_t q_anchor = (uint32_t)ba * (uint32_t)(a.npk * S);   // first flat sample
    for (int pk0 = 0; pk0 < a.npk; pk0 += a.pk_chunk) {
        const int npk_here = min(a.pk_chunk, a.npk - pk0);
        const int ns = npk_here * S;
        for (int t = x.tid; t < ns; t += x.nthreads) {
            const Stencil st = make_stencil(a, ba, pk0 * S + t);
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
            if (!SCATTER) {
                // bucket this sample's inside corners for the feature-gradient gather
                const uint32_t q = q_anchor + (uint32_t)(pk0 * S + t);
                const uint4 rk = *reinterpret_cast<const uint4*>(a.rank + (size_t)q * 4);
                const uint32_t rks[4] = {rk.x, rk.y, rk.z, rk.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (st.row[i] >= 0) {
                        const uint32_t flat_row =
                            (uint32_t)b * (uint32_t)a.num_feat + (uint32_t)st.row[i];
                        Entry e;
                        e.row = flat_row;
                        e.sample = q;
                        e.cw = st.cw[i];
                        e.ba = (uint32_t)ba;
                        const uint32_t pos = row_first_entry(a, flat_row) + rks[i];
                        if (pos < 4u * a.n_samples) a.entries[pos] = e;
                    }
                }
            }
        }
        const float* wsrc = a.weights + wbase + (int64_t)pk0 * S * a.G;
        for (int i = x.tid; i < ns * a.G; i += x.nthreads) wts[i] = wsrc[i];
        __syncthreads();

        float gxs = 0.0f, gys = 0.0f;
        // one sample: (scatter form) feature-gradient atomics, weight gradient,
        // location partials
        auto process = [&](const BwdDesc& d, const float (&v)[NV][4][VEC], int pk, int s) {
            const int t = pk * S + s;
            float tc[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // sum over lanes' channels of top * v_c
            float gwp[NV];
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const float w = wts[t * a.G + gi[i]];
                float dot[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    dot[c] = 0.0f;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) dot[c] += go[i][e] * v[i][c][e];
                    tc[c] += w * dot[c];
                }
                gwp[i] = d.cw[0] * dot[0] + d.cw[1] * dot[1] + d.cw[2] * dot[2] + d.cw[3] * dot[3];
                if constexpr (SCATTER) {
                    const float top = go[i][0] * w;
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
                            d.cw[c] * top, rgr, d.goff[c] + lane_goff, L * i * 4, 0);
                }
            }
            gxs += d.gx[0] * tc[0] + d.gx[1] * tc[1] + d.gx[2] * tc[2] + d.gx[3] * tc[3];
            gys += d.gy[0] * tc[0] + d.gy[1] * tc[1] + d.gy[2] * tc[2] + d.gy[3] * tc[3];

            // weight gradient: grad_out * val summed over the channels of each group
#pragma unroll
            for (int i = 0; i < NV; ++i)
                for (int m = 1; m < seg; m <<= 1) gwp[i] += xor_shfl(gwp[i], m);
            float* gwrow = a.grad_weights + wbase + ((int64_t)(pk0 + pk) * S + s) * a.G;
            if (seg < L) {
                if ((li & (seg - 1)) == 0) {
#pragma unroll
                    for (int i = 0; i < NV; ++i) gwrow[gi[i]] = gwp[i];
                }
            } else if (li == 0) {
                float run = 0.0f;
#pragma unroll
                for (int i = 0; i < NV; ++i) {
                    run += gwp[i];
                    if (i + 1 == NV || gi[i + 1 < NV ? i + 1 : i] != gi[i]) {
                        gwrow[gi[i]] = run;
                        run = 0.0f;
                    }
                }
            }
            if (s == S - 1) {   // last scale of this pair: location gradient
                for (int m = 1; m < L; m <<= 1) {
                    gxs += xor_shfl(gxs, m);
                    gys += xor_shfl(gys, m);
                }
                if (li == 0) {
                    float2* gl = reinterpret_cast<float2*>(a.grad_loc + (ba * a.npk + pk0 + pk) * 2);
                    *gl = make_float2(gxs, gys);
                }
                gxs = 0.0f;
                gys = 0.0f;
            }
        };

        if (rg < npk_here) {
            int pk = rg, s = 0;
            BwdDesc dA = desc[pk * S], dB;
            float vA[NV][4][VEC], vB[NV][4][VEC];
            bwd_load<T, VEC, NV>(rf, dA, lane_off, soff, vA);
            while (true) {
                int s_n = s + 1, pk_n = pk;
                if (s_n == S) { s_n = 0; pk_n += n_rg; }
                bool more = pk_n < npk_here;
                dB = desc[more ? pk_n * S + s_n : ns_max];
                bwd_load<T, VEC, NV>(rf, dB, lane_off, soff, vB);
                process(dA, vA, pk, s);
                if (!more) break;
                pk = pk_n;
                s = s_n;
                s_n = s + 1;
                pk_n = pk;
                if (s_n == S) { s_n = 0; pk_n += n_rg; }
                more = pk_n < npk_here;
                dA = desc[more ? pk_n * S + s_n : ns_max];
                bwd_load<T, VEC, NV>(rf, dA, lane_off, soff, vA);
                process(dB, vB, pk, s);
                if (!more) break;
                pk = pk_n;
                s = s_n;
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------------------------
// gather form: count, scan, gather
// ------------------------------------------------------------------------------------
// Level-major counting.  Workgroup (x, level, b) takes 256 consecutive
// (anchor, point) pairs of batch b at one (camera, scale) level, one thread per
// sample, and gives every inside corner the next slot of its feature row.
// Small levels -- where many samples land on the same row, and same-address
// global atomics would serialise -- are first counted in an LDS histogram of
// the level; one global atomic per touched row then reserves the workgroup's
// block of slots.  Large levels count straight into global memory.  The slot
// order inside a row is whatever order the atomics retire in.
__global__ void __launch_bounds__(256) count_kernel(KArgs a) {
    __shared__ uint32_t hist[kCountLdsRows];
    const int lvl = blockIdx.y;
    const int k = lvl / a.S, s = lvl - (lvl / a.S) * a.S;
    const int32_t nrow = a.lv.H[lvl] * a.lv.W[lvl];
    const int32_t start = a.lv.start[lvl];
    const bool in_lds = nrow <= kCountLdsRows;
    const uint32_t b = blockIdx.z;
    const uint32_t n_ap = (uint32_t)a.A * (uint32_t)a.P;
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;   // (anchor, point) in batch b
    const bool valid = i < n_ap;
    const uint32_t ap = valid ? i : 0u;
    const uint32_t ba = b * (uint32_t)a.A + ap / (uint32_t)a.P;
    const int p = (int)(ap % (uint32_t)a.P);
    const int t = (p * a.K + k) * a.S + s;                      // sample within the anchor
    const uint32_t q = ba * (uint32_t)(a.npk * a.S) + (uint32_t)t;
    const uint32_t row0 = b * (uint32_t)a.num_feat;

    if (in_lds) {
        for (int j = threadIdx.x; j < nrow; j += blockDim.x) hist[j] = 0u;
        __syncthreads();
    }
    const Stencil st = make_stencil(a, (int64_t)ba, t);
    uint32_t rk[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const bool hit = valid && st.row[c] >= 0;
        if (in_lds)
            rk[c] = hit ? atomicAdd(&hist[st.row[c] - start], 1u) : 0u;
        else
            rk[c] = hit ? atomicAdd(a.cnt + row0 + (uint32_t)st.row[c], 1u) : 0u;
    }
    if (in_lds) {
        __syncthreads();
        for (int j = threadIdx.x; j < nrow; j += blockDim.x) {
            const uint32_t c = hist[j];
            if (c) hist[j] = atomicAdd(a.cnt + row0 + (uint32_t)(start + j), c);
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (valid && st.row[c] >= 0) rk[c] += hist[st.row[c] - start];
    }
    if (valid)
        *reinterpret_cast<uint4*>(a.rank + (size_t)q * 4) = make_uint4(rk[0], rk[1], rk[2], rk[3]);
}

// Inclusive prefix sum of v over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v, int lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

// Exclusive prefix sum of cnt inside tiles of kScanTile rows; tile totals to
// tile_prefix[tile].
__global__ void __launch_bounds__(kScanThreads) scan_tiles_kernel(KArgs a) {
    __shared__ uint32_t wave_tot[kScanThreads / kWave];
    const uint32_t n = a.n_rows;
    const uint32_t base = blockIdx.x * (uint32_t)kScanTile + threadIdx.x * (uint32_t)kScanItems;
    uint32_t v[kScanItems];
    if (base + kScanItems <= n) {
        const uint4* src = reinterpret_cast<const uint4*>(a.cnt + base);
#pragma unroll
        for (int j = 0; j < kScanItems / 4; ++j) {
            const uint4 q = src[j];
            v[4 * j] = q.x;
            v[4 * j + 1] = q.y;
            v[4 * j + 2] = q.z;
            v[4 * j + 3] = q.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kScanItems; ++j) v[j] = (base + j < n) ? a.cnt[base + j] : 0u;
    }
    uint32_t tot = 0;
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) {
        const uint32_t c = v[j];
        v[j] = tot;
        tot += c;
    }
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const uint32_t incl = wave_inclusive_scan(tot, lane);
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w) before += wave_tot[w];
    const uint32_t excl = before + incl - tot;
    if (base + kScanItems <= n) {
        uint4* dst = reinterpret_cast<uint4*>(a.local_start + base);
#pragma unroll
        for (int j = 0; j < kScanItems / 4; ++j)
            dst[j] = make_uint4(excl + v[4 * j], excl + v[4 * j + 1], excl + v[4 * j + 2],
                                excl + v[4 * j + 3]);
    } else {
#pragma unroll
        for (int j = 0; j < kScanItems; ++j)
            if (base + j < n) a.local_start[base + j] = excl + v[j];
    }
    if (threadIdx.x == kScanThreads - 1) a.tile_prefix[blockIdx.x] = excl + tot;
}

// In-place exclusive prefix sum of the tile totals (one workgroup); the grand
// total lands in tile_prefix[n_tiles].
__global__ void __launch_bounds__(1024) scan_tile_totals_kernel(KArgs a) {
    __shared__ uint32_t wave_tot[1024 / kWave];
    __shared__ uint32_t carry_s;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    if (threadIdx.x == 0) carry_s = 0;
    __syncthreads();
    for (uint32_t base = 0; base < a.n_tiles; base += blockDim.x) {
        const uint32_t i = base + threadIdx.x;
        const uint32_t v = i < a.n_tiles ? a.tile_prefix[i] : 0u;
        const uint32_t incl = wave_inclusive_scan(v, lane);
        if (lane == kWave - 1) wave_tot[wave] = incl;
        __syncthreads();
        uint32_t before = 0;
        for (int w = 0; w < wave; ++w) before += wave_tot[w];
        const uint32_t carry = carry_s;
        if (i < a.n_tiles) a.tile_prefix[i] = carry + before + incl - v;
        __syncthreads();
        if (threadIdx.x == blockDim.x - 1) carry_s = carry + before + incl;
        __syncthreads();
    }
    if (threadIdx.x == 0) a.tile_prefix[a.n_tiles] = carry_s;
}

// Each wave sums entries [e0, e0 + kGatherChunk) of the row-sorted list.  A row
// whose entries all lie in the chunk is written with plain stores (or added
// to, when accumulating); a row cut by the chunk boundary is added with
// atomics onto the zero-filled (or existing) gradient.
template <int VEC, int NV>
__global__ void __launch_bounds__(256) gather_kernel(KArgs a) {
    constexpr int U = 4;   // entries in flight per wave
    const uint32_t total = min(a.tile_prefix[a.n_tiles], 4u * a.n_samples);
    const uint32_t w = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    const int lane = threadIdx.x % kWave;
    const uint32_t e0 = w * (uint32_t)kGatherChunk;
    if (e0 >= total) return;
    const uint32_t e1 = min(e0 + (uint32_t)kGatherChunk, total);
    const int C = a.C, G = a.G;
    const int nvec = C / VEC;
    bool on[NV];
    int gi[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int v = lane + kWave * i;
        on[i] = v < nvec;
        gi[i] = on[i] ? v * VEC / a.D : 0;
    }
    const Entry* ent = a.entries;
    uint32_t cur = ent[e0].row;
    bool cur_whole_start = (e0 == 0) || ent[e0 - 1].row != cur;
    if (cur >= a.n_rows) cur = 0u;   // out-of-range entries are read as row 0 (see below)
    float acc[NV][VEC];
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int j = 0; j < VEC; ++j) acc[i][j] = 0.0f;

    auto flush = [&](uint32_t row, bool whole) {
        float* dst = a.grad_feat + (size_t)row * C;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            if (!on[i]) continue;
            float* p = dst + (lane + kWave * i) * VEC;
            if (whole) {
                if constexpr (VEC == 4) {
                    float4 o = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
                    if (a.accumulate) {
                        const float4 old = *reinterpret_cast<const float4*>(p);
                        o.x += old.x; o.y += old.y; o.z += old.z; o.w += old.w;
                    }
                    *reinterpret_cast<float4*>(p) = o;
                } else {
#pragma unroll
                    for (int j = 0; j < VEC; ++j) p[j] = a.accumulate ? p[j] + acc[i][j] : acc[i][j];
                }
            } else {
#pragma unroll
                for (int j = 0; j < VEC; ++j) unsafeAtomicAdd(p + j, acc[i][j]);
            }
#pragma unroll
            for (int j = 0; j < VEC; ++j) acc[i][j] = 0.0f;
        }
    };

    for (uint32_t e = e0; e < e1; e += U) {
        Entry en[U];
        float gov[U][NV][VEC];
        float wv[U][NV];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            en[u] = ent[min(e + u, e1 - 1)];
            // every slot below the total was filled by the anchor pass; an entry
            // that is out of range anyway (a workspace shared by overlapping
            // calls) is read as a zero-weight term of row 0
            if (en[u].row >= a.n_rows || en[u].ba >= a.n_anchors || en[u].sample >= a.n_samples) {
                en[u].row = 0u;
                en[u].ba = 0u;
                en[u].sample = 0u;
                en[u].cw = 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float* gorow = a.grad_out + (size_t)en[u].ba * C;
            const float* wrow = a.weights + (size_t)en[u].sample * G;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int v = on[i] ? lane + kWave * i : 0;
                if constexpr (VEC == 4) {
                    const float4 g4 = *reinterpret_cast<const float4*>(gorow + v * 4);
                    gov[u][i][0] = g4.x;
                    gov[u][i][1] = g4.y;
                    gov[u][i][2] = g4.z;
                    gov[u][i][3] = g4.w;
                } else {
                    gov[u][i][0] = gorow[v];
                }
                wv[u][i] = wrow[gi[i]];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (e + u >= e1) break;
            if (en[u].row != cur) {
                flush(cur, cur_whole_start);
                cur = en[u].row;
                cur_whole_start = true;
            }
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const float s = en[u].cw * wv[u][i];
#pragma unroll
                for (int j = 0; j < VEC; ++j) acc[i][j] += s * gov[u][i][j];
            }
        }
    }
    const bool ends_here = (e1 == total) || ent[e1].row != cur;
    flush(cur, cur_whole_start && ends_here);
}

// ------------------------------------------------------------------------------------
// launch helpers
// ------------------------------------------------------------------------------------
__global__ void fill_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool vec_ok = (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
    if (vec_ok) {
        uint4* p4 = reinterpret_cast<uint4*>(p);
        const int64_t n4 = n / 4;
        for (int64_t j = i; j < n4; j += stride) p4[j] = make_uint4(0u, 0u, 0u, 0u);
        for (int64_t j = n4 * 4 + i; j < n; j += stride) p[j] = 0u;
    } else {
        for (int64_t j = i; j < n; j += stride) p[j] = 0u;
    }
}

template <typename T, int VEC, int NV, bool SCATTER>
hipError_t anchor_launch(const KArgs& a, const LaunchShape& s, dim3 grid, hipStream_t st) {
    hipLaunchKernelGGL((da_backward_anchor_kernel<T, VEC, NV, SCATTER>), grid, dim3(kWave * s.waves),
                       s.lds_bytes, st, a);
    return hipGetLastError();
}

// one channel per lane: 1..16 vectors per lane
template <typename T, bool SCATTER>
hipError_t anchor_dispatch_scalar(const KArgs& a, const LaunchShape& s, dim3 grid, hipStream_t st) {
    switch (s.nvc) {
        case 1: return anchor_launch<T, 1, 1, SCATTER>(a, s, grid, st);
        case 2: return anchor_launch<T, 1, 2, SCATTER>(a, s, grid, st);
        case 3: return anchor_launch<T, 1, 3, SCATTER>(a, s, grid, st);
        case 4: return anchor_launch<T, 1, 4, SCATTER>(a, s, grid, st);
        case 5: return anchor_launch<T, 1, 5, SCATTER>(a, s, grid, st);
        case 6: return anchor_launch<T, 1, 6, SCATTER>(a, s, grid, st);
        case 7: return anchor_launch<T, 1, 7, SCATTER>(a, s, grid, st);
        case 8: return anchor_launch<T, 1, 8, SCATTER>(a, s, grid, st);
        case 9: return anchor_launch<T, 1, 9, SCATTER>(a, s, grid, st);
        case 10: return anchor_launch<T, 1, 10, SCATTER>(a, s, grid, st);
        case 11: return anchor_launch<T, 1, 11, SCATTER>(a, s, grid, st);
        case 12: return anchor_launch<T, 1, 12, SCATTER>(a, s, grid, st);
        case 13: return anchor_launch<T, 1, 13, SCATTER>(a, s, grid, st);
        case 14: return anchor_launch<T, 1, 14, SCATTER>(a, s, grid, st);
        case 15: return anchor_launch<T, 1, 15, SCATTER>(a, s, grid, st);
        case 16: return anchor_launch<T, 1, 16, SCATTER>(a, s, grid, st);
        default: return hipErrorInvalidValue;
    }
}

// 16-byte vectors per lane (gather form only): 1..8 vectors per lane
template <typename T, int VEC>
hipError_t anchor_dispatch_vec(const KArgs& a, const LaunchShape& s, dim3 grid, hipStream_t st) {
    switch (s.nvc) {
        case 1: return anchor_launch<T, VEC, 1, false>(a, s, grid, st);
        case 2: return anchor_launch<T, VEC, 2, false>(a, s, grid, st);
        case 3: return anchor_launch<T, VEC, 3, false>(a, s, grid, st);
        case 4: return anchor_launch<T, VEC, 4, false>(a, s, grid, st);
        case 5: return anchor_launch<T, VEC, 5, false>(a, s, grid, st);
        case 6: return anchor_launch<T, VEC, 6, false>(a, s, grid, st);
        case 7: return anchor_launch<T, VEC, 7, false>(a, s, grid, st);
        case 8: return anchor_launch<T, VEC, 8, false>(a, s, grid, st);
        default: return hipErrorInvalidValue;
    }
}

template <int VEC>
hipError_t gather_dispatch(const KArgs& a, const LaunchShape& s, dim3 grid, hipStream_t st) {
    switch (s.gather_nv) {
        case 1: hipLaunchKernelGGL((gather_kernel<VEC, 1>), grid, dim3(256), 0, st, a); break;
        case 2: hipLaunchKernelGGL((gather_kernel<VEC, 2>), grid, dim3(256), 0, st, a); break;
        case 4: hipLaunchKernelGGL((gather_kernel<VEC, 4>), grid, dim3(256), 0, st, a); break;
        case 8: hipLaunchKernelGGL((gather_kernel<VEC, 8>), grid, dim3(256), 0, st, a); break;
        case 16: hipLaunchKernelGGL((gather_kernel<VEC, 16>), grid, dim3(256), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

unsigned blocks_for(int64_t n, int per_block) {
    return (unsigned)((n + per_block - 1) / per_block);
}

}  // namespace

hipError_t launch_fill_zero(void* p, int64_t n_words, hipStream_t stream) {
    if (n_words <= 0) return hipSuccess;
    const int block = 256;
    int64_t blocks = (n_words / 4 + block - 1) / block;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(block), 0, stream,
                       static_cast<uint32_t*>(p), n_words);
    return hipGetLastError();
}

hipError_t launch_backward_scatter(const KArgs& a, const LaunchShape& s, int64_t n_anchors_total,
                                   bool bf16, hipStream_t stream) {
    const dim3 grid((unsigned)n_anchors_total, 1);
    return bf16 ? anchor_dispatch_scalar<uint16_t, true>(a, s, grid, stream)
                : anchor_dispatch_scalar<float, true>(a, s, grid, stream);
}

hipError_t launch_backward_gather(const KArgs& a, const LaunchShape& s, int64_t n_anchors_total,
                                  bool bf16, hipStream_t stream) {
    hipError_t e = launch_fill_zero(a.cnt, a.n_rows, stream);
    if (e != hipSuccess) return e;
    const dim3 cgrid(blocks_for((int64_t)a.A * a.P, 256), (unsigned)(a.K * a.S),
                     (unsigned)(a.n_anchors / (uint32_t)a.A));
    hipLaunchKernelGGL(count_kernel, cgrid, dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(scan_tiles_kernel, dim3(a.n_tiles), dim3(kScanThreads), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(scan_tile_totals_kernel, dim3(1), dim3(1024), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 grid((unsigned)n_anchors_total, 1);
    if (bf16)
        e = s.vec == 8 ? anchor_dispatch_vec<uint16_t, 8>(a, s, grid, stream)
                       : anchor_dispatch_scalar<uint16_t, false>(a, s, grid, stream);
    else
        e = s.vec == 4 ? anchor_dispatch_vec<float, 4>(a, s, grid, stream)
                       : anchor_dispatch_scalar<float, false>(a, s, grid, stream);
    if (e != hipSuccess) return e;
    // one wave per chunk of the largest possible entry count (4 per sample);
    // waves past the real total return at once
    const int64_t waves = ((int64_t)a.n_samples * 4 + kGatherChunk - 1) / kGatherChunk;
    const dim3 ggrid(blocks_for(waves, 256 / kWave));
    return a.gather_vec == 4 ? gather_dispatch<4>(a, s, ggrid, stream)
                             : gather_dispatch<1>(a, s, ggrid, stream);
}

}  // namespace da
