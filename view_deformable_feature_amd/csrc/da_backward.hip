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
//   4. gather:  each wave owns the short rows whose first entry falls in its
//               64-entry range of the row-sorted list and writes each once with
//               plain stores (lanes over channels); the few long rows are added
//               range by range with atomics; rows with no entry are zeroed by a
//               separate pass.
// The scatter form (binary32 atomics straight into the feature gradient) is
// kept for callers that cannot provide the workspace.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "da_device.h"

#include <algorithm>
#include <type_traits>

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


// LDS descriptor of one sample: corner offsets and the per-corner factors of
// the location gradient (section 4.1).
__device__ __forceinline__ BwdDesc bwd_desc(const KArgs& a, const Stencil& st) {
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
    return d;
}

// Bucket the inside corners of flat sample q for the feature-gradient gather:
// each goes to its row's slot rank[q][corner] (taken by count_kernel).  All
// lookups are issued before any store (outside corners read row 0 and store
// nothing), so a thread waits for one round of loads, not one per corner.
// Inclusive prefix sum of v over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v, int lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

// Exclusive prefix of the tile totals into tp[0 .. n_tiles), the grand total in
// tp[n_tiles] (every thread of the block calls this; tp in LDS or global memory).
__device__ __forceinline__ void tile_totals_prefix(const KArgs& a, uint32_t* tp) {
    __shared__ uint32_t wsum[kScanThreads / kWave];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int nw = (int)blockDim.x / kWave;
    uint32_t carry = 0;
    for (uint32_t b0 = 0; b0 < a.n_tiles; b0 += blockDim.x) {
        const uint32_t i = b0 + threadIdx.x;
        const uint32_t t = i < a.n_tiles ? a.tile_tot[i] : 0u;
        const uint32_t inc = wave_inclusive_scan(t, lane);
        __syncthreads();                       // wsum of the previous round is read
        if (lane == kWave - 1) wsum[wave] = inc;
        __syncthreads();
        uint32_t pre = 0, all = 0;
        for (int w2 = 0; w2 < nw; ++w2) {
            if (w2 < wave) pre += wsum[w2];
            all += wsum[w2];
        }
        if (i < a.n_tiles) tp[i] = carry + pre + inc - t;
        carry += all;
    }
    if (threadIdx.x == 0) tp[a.n_tiles] = carry;
    __syncthreads();
}

// Deterministic form: the count blocks' maxima of |grad_out| and |w| into the
// control words (one block).
__device__ __forceinline__ void reduce_det_bounds(const KArgs& a) {
    __shared__ uint32_t red[2][kScanThreads / kWave];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int nw = (int)blockDim.x / kWave;
    uint32_t mg = 0, mw = 0;
    for (uint32_t i = threadIdx.x; i < a.count_blocks; i += blockDim.x) {
        mg = max(mg, a.bound_part[2 * i]);
        mw = max(mw, a.bound_part[2 * i + 1]);
    }
    for (int m = 1; m < kWave; m <<= 1) {
        mg = max(mg, (uint32_t)__shfl_xor((int)mg, m, kWave));
        mw = max(mw, (uint32_t)__shfl_xor((int)mw, m, kWave));
    }
    if (lane == 0) {
        red[0][wave] = mg;
        red[1][wave] = mw;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w2 = 1; w2 < nw; ++w2) {
            mg = max(mg, red[0][w2]);
            mw = max(mw, red[1][w2]);
        }
        a.scan_done[kCtrlMaxGo] = mg;
        a.scan_done[kCtrlMaxW] = mw;
    }
}

// Rank slot of sample t of anchor ba (in batch image b).  The ranks are stored
// level-major -- [image][level][anchor-point] -- the order in which the counting
// kernels write them and the bucket kernel reads them.
__device__ __forceinline__ uint32_t rank_slot(const KArgs& a, uint32_t b, uint32_t ba, int t) {
    const int pk = t / a.S, s = t - pk * a.S;
    const int p = pk / a.K, k = pk - p * a.K;
    const uint32_t n_ap = (uint32_t)a.A * (uint32_t)a.P;
    const uint32_t ap = (ba - b * (uint32_t)a.A) * (uint32_t)a.P + (uint32_t)p;
    return (b * (uint32_t)(a.K * a.S) + (uint32_t)(k * a.S + s)) * n_ap + ap;
}

// q: the flat sample index (its weight row); rs: its rank slot.
__device__ __forceinline__ void bucket_sample(const KArgs& a, const Stencil& st, int64_t b,
                                              int64_t ba, uint32_t q, uint32_t rs,
                                              const uint32_t* tprefix) {
    const uint4 rk = *reinterpret_cast<const uint4*>(a.rank + (size_t)rs * 4);
    const uint32_t rks[4] = {rk.x, rk.y, rk.z, rk.w};
    const uint32_t base = (uint32_t)b * (uint32_t)a.num_feat;
    uint32_t fr[4], ls[4], first[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fr[i] = base + (uint32_t)(st.row[i] >= 0 ? st.row[i] : 0);
    // local_start carries the row's long flag in its top bit (set by the scan)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ls[i] = a.local_start[fr[i]];
        first[i] = tprefix[fr[i] / (uint32_t)kScanTile] + (ls[i] & ~kEntryLongRow);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        Entry e;
        e.row = fr[i] | (ls[i] & kEntryLongRow);
        e.w_off = q * (uint32_t)a.G * 4u;
        e.cw = st.cw[i];
        e.go_off = (uint32_t)ba * (uint32_t)a.C * 4u + (uint32_t)i;
        const uint32_t pos = first[i] + rks[i];
        if (st.row[i] >= 0 && pos < 4u * a.n_samples) a.entries[pos] = e;
    }
}

// Per-lane dot products of one sample: tc[c] = sum over the lane's channels of
// weight * grad_out * v_c, and gwp[i] = sum_c cw_c * (grad_out . v_c) over
// vector i (the lane's share of the weight gradient of group gi[i]).
template <int VEC, int NV>
__device__ __forceinline__ void sample_dots(const BwdDesc& d, const float (&v)[NV][4][VEC],
                                            const float (&go)[NV][VEC], const float* wrow,
                                            const int (&gi)[NV], float (&tc)[4],
                                            float (&gwp)[NV], float (&w)[NV]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) tc[c] = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        w[i] = wrow[gi[i]];
        float dot[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            dot[c] = 0.0f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) dot[c] += go[i][e] * v[i][c][e];
            tc[c] += w[i] * dot[c];
        }
        gwp[i] = d.cw[0] * dot[0] + d.cw[1] * dot[1] + d.cw[2] * dot[2] + d.cw[3] * dot[3];
    }
}

// Sum gwp over the `seg` lanes that share a group and store the sample's
// weight-gradient row (gwrow = grad_weights row of the sample).  The sums land
// in the last lane of each seg-lane segment.
template <int NV>
__device__ __forceinline__ void store_grad_weights(float (&gwp)[NV], const int (&gi)[NV],
                                                   float* gwrow, int seg, int L, int li) {
#pragma unroll
    for (int i = 0; i < NV; ++i) gwp[i] = group_sum(gwp[i], seg);
    if (seg < L) {
        if ((li & (seg - 1)) == seg - 1) {
#pragma unroll
            for (int i = 0; i < NV; ++i) gwrow[gi[i]] = gwp[i];
        }
    } else if (li == L - 1) {
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
}

// First entry of a row in the row-sorted list.
// tprefix: the exclusive prefix of the tile totals (a.tile_prefix, or a copy in LDS)
__device__ __forceinline__ uint32_t first_entry(const KArgs& a, const uint32_t* tprefix,
                                                uint32_t row) {
    return tprefix[row / (uint32_t)kScanTile] + (a.local_start[row] & ~kEntryLongRow);
}

// Zero the feature-gradient rows r0 .. r0+63 (r0 = 64 w) that have no entry,
// and the long rows that gather_kernel adds to range by range.
template <int ZVEC>
__device__ __forceinline__ void zero_rows_wave(const KArgs& a, uint32_t w, int lane,
                                               const uint32_t* tprefix) {
    const uint32_t r0 = w * (uint32_t)kWave;
    if (r0 >= a.n_rows) return;
    const uint32_t r = r0 + (uint32_t)lane;
    const uint32_t c = r < a.n_rows ? a.cnt[r] : 1u;
    // rows the gather does not store whole: no entry (unless accumulating), or
    // long (summed range by range: onto the zeroed row, or in the deterministic
    // form onto its zeroed 64-bit accumulation row)
    const bool empty = c == 0u && !a.accumulate;
    const bool long_row = c > (uint32_t)kGatherLong;
    uint64_t m = __ballot(empty || (long_row && !a.det && !a.accumulate));
    const int nvec = a.C / ZVEC;
    while (m) {
        const int l = __ffsll((unsigned long long)m) - 1;
        m &= m - 1;
        float* row = a.grad_feat + (size_t)(r0 + (uint32_t)l) * a.C;
        for (int v = lane; v < nvec; v += kWave) {
            if constexpr (ZVEC == 4)
                reinterpret_cast<float4*>(row)[v] = make_float4(0.f, 0.f, 0.f, 0.f);
            else
                row[v] = 0.0f;
        }
    }
    if (a.det) {
        m = __ballot(long_row);
        if (m != 0) {
            // list this wave's long rows for long_rows_kernel
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(a.scan_done + kCtrlLongRows, (uint32_t)__popcll(m));
            base = (uint32_t)__shfl((int)base, 0, kWave);
            const uint32_t rank = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
            if (long_row && base + rank < a.n_slots) a.long_rows[base + rank] = r;
        }
        // every lane looks up its own long row's slot before the loop
        const uint32_t slot_id = long_row ? first_entry(a, tprefix, r) / kSlotStride : 0u;
        while (m) {
            const int l = __ffsll((unsigned long long)m) - 1;
            m &= m - 1;
            long long* slot =
                a.slots + (size_t)(uint32_t)__builtin_amdgcn_readlane((int)slot_id, l) * a.C;
            if ((a.C & 1) == 0) {      // rows start 16-byte aligned
                for (int v = lane; v < a.C / 2; v += kWave)
                    reinterpret_cast<longlong2*>(slot)[v] = make_longlong2(0, 0);
            } else {
                for (int v = lane; v < a.C; v += kWave) slot[v] = 0;
            }
        }
    }
}

// The zeroing role of the blocks past anchor_blocks: 64 rows per wave.
__device__ __forceinline__ void zero_rows_role(const KArgs& a, const uint32_t* tprefix) {
    const uint32_t w = (blockIdx.x - a.anchor_blocks) * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (a.gather_vec == 4)
        zero_rows_wave<4>(a, w, lane, tprefix);
    else
        zero_rows_wave<1>(a, w, lane, tprefix);
}

template <typename T, int VEC, int NV, bool SCATTER>
__global__ void __launch_bounds__(kWave * kMaxWaves)
da_backward_anchor_kernel(KArgs a) {
    if constexpr (!SCATTER) {
        if (blockIdx.x >= a.anchor_blocks) {
            zero_rows_role(a, a.tile_prefix);
            return;
        }
    }
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
        for (int e = 0; e < VEC; ++e) go[i][e] = load_elem(a.grad_out, ba * a.C + c0 + e, a.go_dtype);
    }

    if (x.tid == 0) desc[ns_max] = null_bwd_desc(a.feat_image_bytes, a.gfeat_image_bytes);
    const int64_t wbase = ba * (int64_t)a.npk * S * a.G;
    const uint32_t q_anchor = (uint32_t)ba * (uint32_t)(a.npk * S);   // first flat sample
    for (int pk0 = 0; pk0 < a.npk; pk0 += a.pk_chunk) {
        const int npk_here = min(a.pk_chunk, a.npk - pk0);
        const int ns = npk_here * S;
        for (int t = x.tid; t < ns; t += x.nthreads) {
            const Stencil st = make_stencil(a, ba, pk0 * S + t);
            desc[t] = bwd_desc(a, st);
            if (!SCATTER)
                bucket_sample(a, st, b, ba, q_anchor + (uint32_t)(pk0 * S + t),
                              rank_slot(a, (uint32_t)b, (uint32_t)ba, pk0 * S + t), a.tile_prefix);
        }
        const float* wsrc = a.weights + wbase + (int64_t)pk0 * S * a.G;
        for (int i = x.tid; i < ns * a.G; i += x.nthreads) wts[i] = wsrc[i];
        __syncthreads();

        float gxs = 0.0f, gys = 0.0f;
        // one sample: (scatter form) feature-gradient atomics, weight gradient,
        // location partials
        auto process = [&](const BwdDesc& d, const float (&v)[NV][4][VEC], int pk, int s) {
            const int t = pk * S + s;
            float tc[4], gwp[NV], w[NV];
            sample_dots<VEC, NV>(d, v, go, wts + t * a.G, gi, tc, gwp, w);
            if constexpr (SCATTER) {
#pragma unroll
                for (int i = 0; i < NV; ++i) {
                    const float top = go[i][0] * w[i];
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
                            d.cw[c] * top, rgr, d.goff[c] + lane_goff, L * i * 4, 0);
                }
            }
            gxs += d.gx[0] * tc[0] + d.gx[1] * tc[1] + d.gx[2] * tc[2] + d.gx[3] * tc[3];
            gys += d.gy[0] * tc[0] + d.gy[1] * tc[1] + d.gy[2] * tc[2] + d.gy[3] * tc[3];
            // weight gradient: grad_out * val summed over the channels of each group
            store_grad_weights<NV>(gwp, gi, a.grad_weights + wbase + ((int64_t)(pk0 + pk) * S + s) * a.G,
                                   seg, L, li);
            if (s == S - 1) {   // last scale of this pair: location gradient
                gxs = group_sum(gxs, L);
                gys = group_sum(gys, L);
                if (li == L - 1) {
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
// per-anchor kernel by level slices (gather form)
// ------------------------------------------------------------------------------------
// Workgroup (anchor, x) -- on XCD x -- takes the samples of the levels in
// slice x only, in the order of slice_sample().  Everything but the location
// gradient is per sample, as in the kernel above.  A point-camera pair's
// scales are spread over slices, so each sample's location partial (summed
// over the lanes of its row group) goes to loc_part[q], and loc_reduce_role
// adds a pair's S partials in scale order.
template <typename T, int VEC, int NV>
__global__ void __launch_bounds__(kWave * kMaxWaves)
da_backward_sliced_kernel(KArgs a) {
    if (blockIdx.x >= a.anchor_blocks) {
        zero_rows_role(a, a.tile_prefix);
        return;
    }
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
    const int seg = a.seg;
    constexpr int kElem = (int)sizeof(T);

    const int ns_max = a.sample_chunk;           // desc[ns_max] is the null descriptor
    BwdDesc* desc = reinterpret_cast<BwdDesc*>(smem);
    float* wts = reinterpret_cast<float*>(smem + (size_t)(ns_max + 1) * sizeof(BwdDesc));
    int32_t* tix = reinterpret_cast<int32_t*>(wts + (size_t)ns_max * a.G);

    const __amdgpu_buffer_rsrc_t rf = make_rsrc(
        static_cast<const unsigned char*>(a.feat) + b * a.feat_batch_bytes, a.feat_image_bytes);

    const uint32_t lane_off = (uint32_t)(li * VEC * kElem);
    uint32_t soff[NV];
    float go[NV][VEC];
    int gi[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c0 = (li + L * i) * VEC;
        soff[i] = (uint32_t)(L * i * VEC * kElem);
        gi[i] = c0 / a.D;
#pragma unroll
        for (int e = 0; e < VEC; ++e) go[i][e] = load_elem(a.grad_out, ba * a.C + c0 + e, a.go_dtype);
    }

    if (tid == 0) desc[ns_max] = null_bwd_desc(a.feat_image_bytes, a.gfeat_image_bytes);
    const int m = a.lv.slice_nlev[x];
    const int n = a.P * m;
    const int64_t wbase = ba * (int64_t)a.npk * a.S * a.G;
    const uint32_t q_anchor = (uint32_t)ba * (uint32_t)(a.npk * a.S);   // first flat sample
    for (int j0 = 0; j0 < n; j0 += ns_max) {
        const int nsc = min(ns_max, n - j0);
        for (int jj = tid; jj < nsc; jj += nthreads) {
            const int t = slice_sample(a, x, m, j0 + jj);
            const Stencil st = make_stencil(a, ba, t);
            desc[jj] = bwd_desc(a, st);
            tix[jj] = t;
            bucket_sample(a, st, b, ba, q_anchor + (uint32_t)t,
                          rank_slot(a, (uint32_t)b, (uint32_t)ba, t), a.tile_prefix);
        }
        for (int i = tid; i < nsc * a.G; i += nthreads) {
            const int jj = i / a.G;
            wts[i] = a.weights[wbase + (int64_t)slice_sample(a, x, m, j0 + jj) * a.G + (i - jj * a.G)];
        }
        __syncthreads();

        auto process = [&](const BwdDesc& d, const float (&v)[NV][4][VEC], int jj) {
            const int t = tix[jj];
            float tc[4], gwp[NV], w[NV];
            sample_dots<VEC, NV>(d, v, go, wts + jj * a.G, gi, tc, gwp, w);
            float gx = d.gx[0] * tc[0] + d.gx[1] * tc[1] + d.gx[2] * tc[2] + d.gx[3] * tc[3];
            float gy = d.gy[0] * tc[0] + d.gy[1] * tc[1] + d.gy[2] * tc[2] + d.gy[3] * tc[3];
            store_grad_weights<NV>(gwp, gi, a.grad_weights + wbase + (int64_t)t * a.G, seg, L, li);
            gx = group_sum(gx, L);
            gy = group_sum(gy, L);
            if (li == L - 1)
                reinterpret_cast<float2*>(a.loc_part)[q_anchor + (uint32_t)t] = make_float2(gx, gy);
        };

        int j = rg;
        if (j < nsc) {
            BwdDesc dA = desc[j], dB;
            float vA[NV][4][VEC], vB[NV][4][VEC];
            bwd_load<T, VEC, NV>(rf, dA, lane_off, soff, vA);
            while (true) {
                int jn = j + n_rg;
                dB = desc[jn < nsc ? jn : ns_max];
                bwd_load<T, VEC, NV>(rf, dB, lane_off, soff, vB);
                process(dA, vA, j);
                if (jn >= nsc) break;
                j = jn;
                jn = j + n_rg;
                dA = desc[jn < nsc ? jn : ns_max];
                bwd_load<T, VEC, NV>(rf, dA, lane_off, soff, vA);
                process(dB, vB, j);
                if (jn >= nsc) break;
                j = jn;
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------------------------
// row-ordered backward: bucketing, then (after the gather) the per-sample gradients
// ------------------------------------------------------------------------------------
// One thread per sample: its stencil, and its inside corners into the row-sorted
// entry list.  Blocks past anchor_blocks zero the rows the gather does not
// store whole.
// Workgroups in (batch image, level, chunk of 256 anchor-point pairs) order,
// that list cut into kSlices contiguous parts and part x given to the
// workgroups on XCD x (ids congruent to x): each XCD then writes one contiguous
// stretch of the row-sorted entries and reads one stretch of local_start, in its
// own L2, instead of every XCD touching every level's lines.
//
// tot_in_bucket: every workgroup first forms the prefix of the scan's tile
// totals in LDS (at most kBucketLdsTiles of them), and workgroup 0 also stores
// it as tile_prefix and reduces the deterministic form's bounds, for the
// kernels that follow: one launch fewer than a separate scan of the totals.
__global__ void __launch_bounds__(256) bucket_kernel(KArgs a) {
    __shared__ uint32_t tp_lds[kBucketLdsTiles + 1];
    const uint32_t* tprefix = a.tile_prefix;
    if (a.tot_in_bucket) {
        tile_totals_prefix(a, tp_lds);
        if (blockIdx.x == 0) {
            for (uint32_t i = threadIdx.x; i <= a.n_tiles; i += blockDim.x) a.tile_prefix[i] = tp_lds[i];
            if (a.det) reduce_det_bounds(a);
        }
        tprefix = tp_lds;
    }
    if (blockIdx.x >= a.anchor_blocks) {
        zero_rows_role(a, tprefix);
        return;
    }
    __shared__ int32_t lvl_lds[3 * kMaxLevels];
    const LevelsLds lv = stage_levels(a, lvl_lds);
    const uint32_t n_ap = (uint32_t)a.A * (uint32_t)a.P;
    const uint32_t nlev = (uint32_t)(a.K * a.S);
    const uint32_t cpl = (n_ap + 255u) / 256u;                      // chunks per level
    const uint32_t total = (a.n_anchors / (uint32_t)a.A) * nlev * cpl;
    const uint32_t per_x = a.anchor_blocks / (uint32_t)kSlices;
    const uint32_t tri = (blockIdx.x % (uint32_t)kSlices) * per_x + blockIdx.x / (uint32_t)kSlices;
    if (tri >= total) return;
    const uint32_t b = tri / (nlev * cpl);
    const uint32_t rem = tri - b * nlev * cpl;
    const uint32_t lvl = rem / cpl;
    const uint32_t ap = (rem - lvl * cpl) * 256u + threadIdx.x;
    if (ap >= n_ap) return;
    const int k = (int)lvl / a.S, s = (int)lvl - ((int)lvl / a.S) * a.S;
    const uint32_t ba = b * (uint32_t)a.A + ap / (uint32_t)a.P;
    const int t = ((int)(ap % (uint32_t)a.P) * a.K + k) * a.S + s;
    const uint32_t q = ba * (uint32_t)(a.npk * a.S) + (uint32_t)t;
    const Stencil st = make_stencil(a, (int64_t)ba, t, lv);
    bucket_sample(a, st, (int64_t)b, (int64_t)ba, q, (b * nlev + lvl) * n_ap + ap, tprefix);
}

constexpr int kFinalizeLdsGroups = 8;   // finalize_kernel stages the dot products for G <= 8
// Three waves per workgroup: with G = 8 a workgroup stages 26 KB of dot products,
// so six fit a CU and 280,800 samples run in one round (at 256 threads, 35 KB,
// four fit and the last 7 % of the workgroups ran as a second round).
constexpr int kFinalizeThreads = 192;

// One thread per sample q: from the per-corner group dot products
// d[c][g] = sum over the channels of group g of grad_out * corner value c (formed
// by the gather), section 4.1's gradients --
//   grad_weights[q][g] = sum_c cw_c d[c][g]
//   grad_loc of q's (point, camera) = sum over its S scales of
//                                     sum_c (dx_c, dy_c) * sum_g w[q][g] d[c][g]
// with (dx_c, dy_c) the derivatives of the corner weights: W (-hh, hh, -lh, lh)
// and H (-hw, -lw, hw, lw).  Corners outside the level have no entry and count
// 0.  The S samples of a (point, camera) are consecutive threads: with S a power
// of two their location terms are summed across lanes (total in the last lane),
// otherwise each sample's term goes to loc_part and loc_reduce_kernel adds them.
__global__ void __launch_bounds__(kFinalizeThreads) finalize_kernel(KArgs a) {
    __shared__ int32_t lvl_lds[3 * kMaxLevels];
    // the block's dot products (kFinalizeThreads samples x 4 corners x G <= 8 floats, one
    // contiguous range), copied with coalesced 16-byte loads; an odd row stride
    // keeps each thread's reads of its own row free of bank conflicts
    constexpr int kDotRow = 4 * kFinalizeLdsGroups + 1;
    __shared__ float sdots[kFinalizeThreads * kDotRow];
    const bool staged = a.w_vec4 && a.G <= kFinalizeLdsGroups;
    if (staged) {
        const uint32_t q0 = blockIdx.x * blockDim.x;
        const uint32_t nq = min((uint32_t)blockDim.x, a.n_samples - q0);
        const int row = 4 * a.G;                           // floats per sample, a multiple of 16
        const float4* src = reinterpret_cast<const float4*>(a.dots + (size_t)q0 * row);
        // at most G <= 8 vectors per thread: all loads issued before the first store
        const uint32_t n4 = nq * (uint32_t)row / 4;
        float4 v[kFinalizeLdsGroups];
#pragma unroll
        for (int k = 0; k < kFinalizeLdsGroups; ++k) {
            const uint32_t i = threadIdx.x + (uint32_t)(k * kFinalizeThreads);
            if (i < n4) v[k] = src[i];
        }
#pragma unroll
        for (int k = 0; k < kFinalizeLdsGroups; ++k) {
            const uint32_t i = threadIdx.x + (uint32_t)(k * kFinalizeThreads);
            if (i < n4) {
                const uint32_t e = 4 * i, sq = e / (uint32_t)row, j = e - sq * (uint32_t)row;
                float* d = sdots + sq * kDotRow + j;
                d[0] = v[k].x;
                d[1] = v[k].y;
                d[2] = v[k].z;
                d[3] = v[k].w;
            }
        }
    }
    const LevelsLds lv = stage_levels(a, lvl_lds);      // (its barrier also covers sdots)
    const uint32_t q = blockIdx.x * blockDim.x + threadIdx.x;
    const bool valid = q < a.n_samples;
    const uint32_t qq = valid ? q : 0u;
    const uint32_t per_anchor = (uint32_t)(a.npk * a.S);
    const uint32_t ba = qq / per_anchor;
    const int t = (int)(qq - ba * per_anchor);
    const Stencil st = make_stencil(a, (int64_t)ba, t, lv);
    const int G = a.G;
    const float* wrow = a.weights + (size_t)qq * G;
    float* gwrow = a.grad_weights + (size_t)qq * G;
    const float* drow = a.dots + (size_t)qq * 4 * G;
    bool in[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) in[c] = st.row[c] >= 0;
    float tc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (a.w_vec4) {
        const float* srow = sdots + threadIdx.x * kDotRow;
        for (int g = 0; g < G; g += 4) {
            const float4 w = *reinterpret_cast<const float4*>(wrow + g);
            float4 d[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float* sp = srow + c * G + g;
                const float4 v = staged ? make_float4(sp[0], sp[1], sp[2], sp[3])
                                        : *reinterpret_cast<const float4*>(drow + c * G + g);
                d[c] = in[c] ? v : make_float4(0.f, 0.f, 0.f, 0.f);
                tc[c] += w.x * d[c].x + w.y * d[c].y + w.z * d[c].z + w.w * d[c].w;
            }
            float4 gw;
            gw.x = st.cw[0] * d[0].x + st.cw[1] * d[1].x + st.cw[2] * d[2].x + st.cw[3] * d[3].x;
            gw.y = st.cw[0] * d[0].y + st.cw[1] * d[1].y + st.cw[2] * d[2].y + st.cw[3] * d[3].y;
            gw.z = st.cw[0] * d[0].z + st.cw[1] * d[1].z + st.cw[2] * d[2].z + st.cw[3] * d[3].z;
            gw.w = st.cw[0] * d[0].w + st.cw[1] * d[1].w + st.cw[2] * d[2].w + st.cw[3] * d[3].w;
            if (valid) *reinterpret_cast<float4*>(gwrow + g) = gw;
        }
    } else {
        for (int g = 0; g < G; ++g) {
            float d[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) d[c] = in[c] ? drow[c * G + g] : 0.0f;
            const float gw = st.cw[0] * d[0] + st.cw[1] * d[1] + st.cw[2] * d[2] + st.cw[3] * d[3];
            if (valid) gwrow[g] = gw;
            const float w = wrow[g];
#pragma unroll
            for (int c = 0; c < 4; ++c) tc[c] += w * d[c];
        }
    }
    const float m = st.inside ? 1.0f : 0.0f;
    float gx = m * st.W * (st.hh * (tc[1] - tc[0]) + st.lh * (tc[3] - tc[2]));
    float gy = m * st.H * (st.hw * (tc[2] - tc[0]) + st.lw * (tc[3] - tc[1]));
    const int S = a.S;
    if ((S & (S - 1)) == 0 && S <= kWave) {
        gx = group_sum(gx, S);
        gy = group_sum(gy, S);
        if (valid && (t % S) == S - 1)
            reinterpret_cast<float2*>(a.grad_loc)[(size_t)ba * a.npk + t / S] = make_float2(gx, gy);
    } else if (valid) {
        reinterpret_cast<float2*>(a.loc_part)[q] = make_float2(gx, gy);
    }
}

// grad_loc of each (anchor, point, camera) = sum of its S partials, in scale order.
__global__ void __launch_bounds__(256) loc_reduce_kernel(KArgs a) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)a.n_anchors * a.npk) return;
    const float2* part = reinterpret_cast<const float2*>(a.loc_part);
    float gx = 0.0f, gy = 0.0f;
    for (int s = 0; s < a.S; ++s) {
        const float2 v = part[i * a.S + s];
        gx += v.x;
        gy += v.y;
    }
    reinterpret_cast<float2*>(a.grad_loc)[i] = make_float2(gx, gy);
}

// grad_loc of each (anchor, point, camera) = sum of its S scale partials, in
// scale order: the role of the gather launch's blocks past gather_blocks, one
// thread per pair.
__device__ __forceinline__ void loc_reduce_role(const KArgs& a) {
    const int64_t i = (int64_t)(blockIdx.x - a.gather_blocks) * blockDim.x + threadIdx.x;
    if (i >= (int64_t)a.n_anchors * a.npk) return;
    const float2* part = reinterpret_cast<const float2*>(a.loc_part);
    float gx = 0.0f, gy = 0.0f;
    for (int s = 0; s < a.S; ++s) {
        const float2 v = part[i * a.S + s];
        gx += v.x;
        gy += v.y;
    }
    reinterpret_cast<float2*>(a.grad_loc)[i] = make_float2(gx, gy);
}

// ------------------------------------------------------------------------------------
// gather form: count, scan, gather
// ------------------------------------------------------------------------------------
// max |p[i]| over i = i0, i0 + stride, ... below n, as float bits (which order
// like the values for values >= 0)
__device__ __forceinline__ uint32_t abs_max_bits(const float* p, int64_t n, int64_t i0,
                                                 int64_t stride) {
    uint32_t m = 0;
    if ((reinterpret_cast<uintptr_t>(p) & 15) == 0) {      // 16-byte loads, then the tail
        const int64_t n4 = n / 4;
        const float4* p4 = reinterpret_cast<const float4*>(p);
        int64_t i = i0;
        for (; i + 3 * stride < n4; i += 4 * stride) {      // four loads in flight
            float4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = p4[i + u * stride];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                m = max(m, max(max(__float_as_uint(fabsf(v[u].x)), __float_as_uint(fabsf(v[u].y))),
                               max(__float_as_uint(fabsf(v[u].z)), __float_as_uint(fabsf(v[u].w)))));
        }
        for (; i < n4; i += stride) {
            const float4 v = p4[i];
            m = max(m, max(max(__float_as_uint(fabsf(v.x)), __float_as_uint(fabsf(v.y))),
                           max(__float_as_uint(fabsf(v.z)), __float_as_uint(fabsf(v.w)))));
        }
        for (int64_t i = n4 * 4 + i0; i < n; i += stride) m = max(m, __float_as_uint(fabsf(p[i])));
    } else {
        for (int64_t i = i0; i < n; i += stride) m = max(m, __float_as_uint(fabsf(p[i])));
    }
    return m;
}


// Level-major counting.  Workgroup (x, level, b) takes 256 consecutive
// (anchor, point) pairs of batch b at one (camera, scale) level (kCountLdsPer
// times as many on levels counted in LDS), and gives every inside corner the
// next slot of its feature row.
// Small levels -- where many samples land on the same row, and same-address
// global atomics would serialise -- are first counted in an LDS histogram of
// the level; one global atomic per touched row then reserves the workgroup's
// block of slots.  Medium levels count straight into global memory, and levels
// above count_tile_rows rows are left to count_tiles_kernel.  The slot
// order inside a row is whatever order the atomics retire in.  The
// deterministic form also takes the maxima of |weights| and |grad_out| here
// (in every workgroup, whatever its level).
template <int PER>
__global__ void __launch_bounds__(kCountThreads) count_kernel(KArgs a) {
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

    if (!in_lds && nrow <= a.count_tile_rows) {
        const Stencil st = make_stencil(a, (int64_t)ba, t);
        uint32_t rk[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bool hit = valid && st.row[c] >= 0;
            rk[c] = hit ? atomicAdd(a.cnt + row0 + (uint32_t)st.row[c], 1u) : 0u;
        }
        if (valid)
            *reinterpret_cast<uint4*>(a.rank + ((size_t)(b * (uint32_t)(a.K * a.S) + (uint32_t)lvl) * n_ap + i) * 4) =
                make_uint4(rk[0], rk[1], rk[2], rk[3]);
    }
    // Levels of at most kCountLdsRows rows: PER samples per thread, so that the LDS
    // histogram gathers many corners per row before the one global atomic per
    // touched row (with one sample per thread a 4000-row level saw about one corner
    // per row per workgroup, and the histogram saved almost no atomics).  Blocks
    // past the level's last chunk have nothing to count.  PER is a template
    // argument: its register arrays would otherwise cost the other paths occupancy.
    const uint32_t i0 = blockIdx.x * (uint32_t)(PER * kCountThreads);
    if (in_lds && i0 < n_ap) {
        for (int j = threadIdx.x; j < nrow; j += blockDim.x) hist[j] = 0u;
        __syncthreads();
        int32_t rows[PER][4];               // level-relative rows of inside corners, else -1
        uint32_t qs[PER];
        // every sample's stencil (and so its location load) before the first atomic
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const uint32_t iu = i0 + (uint32_t)u * kCountThreads + threadIdx.x;
            const bool vu = iu < n_ap;
            const uint32_t apu = vu ? iu : 0u;
            const uint32_t bau = b * (uint32_t)a.A + apu / (uint32_t)a.P;
            const int tu = ((int)(apu % (uint32_t)a.P) * a.K + k) * a.S + s;
            qs[u] = vu ? (b * (uint32_t)(a.K * a.S) + (uint32_t)lvl) * n_ap + iu : 0xffffffffu;   // rank slot
            const Stencil st = make_stencil(a, (int64_t)bau, tu);
#pragma unroll
            for (int c = 0; c < 4; ++c) rows[u][c] = (vu && st.row[c] >= 0) ? st.row[c] - start : -1;
        }
        uint32_t rk[PER][4];
#pragma unroll
        for (int u = 0; u < PER; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) rk[u][c] = rows[u][c] >= 0 ? atomicAdd(&hist[rows[u][c]], 1u) : 0u;
        // reserve each touched row's block of slots; every atomic is issued
        // before any result is needed
        constexpr int kPer = kCountLdsRows / kCountThreads;
        __syncthreads();
        uint32_t c[kPer], base[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int j = (int)threadIdx.x + u * kCountThreads;
            c[u] = j < nrow ? hist[j] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int j = (int)threadIdx.x + u * kCountThreads;
            base[u] = c[u] ? atomicAdd(a.cnt + row0 + (uint32_t)(start + j), c[u]) : 0u;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int j = (int)threadIdx.x + u * kCountThreads;
            if (c[u]) hist[j] = base[u];
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < PER; ++u) {
#pragma unroll
            for (int c2 = 0; c2 < 4; ++c2)
                if (rows[u][c2] >= 0) rk[u][c2] += hist[rows[u][c2]];
            if (qs[u] != 0xffffffffu)
                *reinterpret_cast<uint4*>(a.rank + (size_t)qs[u] * 4) =
                    make_uint4(rk[u][0], rk[u][1], rk[u][2], rk[u][3]);
        }
    }
    if (a.det) {
        // bounds for the fixed point: this sample's weights and a share of
        // grad_out; the block's maxima go to bound_part (reduced by the scan)
        __shared__ uint32_t red[2][kCountThreads / kWave];
        const uint32_t fb = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
        const uint32_t nb = gridDim.x * gridDim.y * gridDim.z;
        uint32_t mw = 0;
        if (in_lds) {
            // the samples this block counted (PER per thread)
            for (int u = 0; u < PER; ++u) {
                const uint32_t iu = i0 + (uint32_t)u * kCountThreads + threadIdx.x;
                if (iu >= n_ap) break;
                const uint32_t bau = b * (uint32_t)a.A + iu / (uint32_t)a.P;
                const int tu = ((int)(iu % (uint32_t)a.P) * a.K + k) * a.S + s;
                const uint32_t qu = bau * (uint32_t)(a.npk * a.S) + (uint32_t)tu;
                mw = max(mw, abs_max_bits(a.weights + (size_t)qu * a.G, a.G, 0, 1));
            }
        } else if (valid) {
            mw = abs_max_bits(a.weights + (size_t)q * a.G, a.G, 0, 1);
        }
        uint32_t mg = abs_max_bits(static_cast<const float*>(a.grad_out), (int64_t)a.n_anchors * a.C,
                                   (int64_t)fb * kCountThreads + threadIdx.x,
                                   (int64_t)nb * kCountThreads);
        for (int m = 1; m < kWave; m <<= 1) {
            mg = max(mg, (uint32_t)__shfl_xor((int)mg, m, kWave));
            mw = max(mw, (uint32_t)__shfl_xor((int)mw, m, kWave));
        }
        const int wave = threadIdx.x / kWave;
        if (threadIdx.x % kWave == 0) {
            red[0][wave] = mg;
            red[1][wave] = mw;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int w = 1; w < kCountThreads / kWave; ++w) {
                mg = max(mg, red[0][w]);
                mw = max(mw, red[1][w]);
            }
            a.bound_part[2 * fb] = mg;
            a.bound_part[2 * fb + 1] = mw;
        }
    }
}

// Counting of the levels above count_tile_rows rows.  Workgroup (x, level, b) owns
// tile x of the level's rows (in batch b) and scans every
// (anchor, point) pair of the level: each inside corner that falls in its rows
// takes the next slot of an LDS histogram, and the histogram is then stored as
// those rows' counts.  Each row has one owner, so there is no global atomic;
// every workgroup reads all of the level's locations (8 bytes per pair).  Blocks
// of small levels, and tiles past a level's last row, return at once.
__global__ void __launch_bounds__(kCountTileThreads) count_tiles_kernel(KArgs a) {
    __shared__ uint32_t hist[kCountTileRows];
    const int lvl = blockIdx.y;
    const int32_t nrow = a.lv.H[lvl] * a.lv.W[lvl];
    // every tiled level is cut into the same gridDim.x tiles (of at most
    // kCountTileRows rows: the grid is sized for the largest level), so that each
    // workgroup counts about the same number of corners -- every level has the
    // same samples
    const int32_t tr = (nrow + (int32_t)gridDim.x - 1) / (int32_t)gridDim.x;
    const int32_t r0 = (int32_t)blockIdx.x * tr;
    if (nrow <= a.count_tile_rows || r0 >= nrow) return;
    const int32_t nr = min(tr, nrow - r0);
    const int k = lvl / a.S, s = lvl - k * a.S;
    const int32_t lo = a.lv.start[lvl] + r0;          // first owned row in the batch image
    const uint32_t b = blockIdx.z;
    const uint32_t n_ap = (uint32_t)a.A * (uint32_t)a.P;
    const uint32_t row0 = b * (uint32_t)a.num_feat;
    for (int j = threadIdx.x; j < nr; j += blockDim.x) hist[j] = 0u;
    __syncthreads();
    // kU pairs per thread and step: their stencils (and so their location loads)
    // are all formed before the first atomic or store, one memory latency per step
    constexpr int kU = 4;
    for (uint32_t ap0 = threadIdx.x; ap0 < n_ap; ap0 += kU * blockDim.x) {
        Stencil st[kU];
        uint32_t qs[kU];
        bool ok[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const uint32_t ap = ap0 + (uint32_t)u * blockDim.x;
            ok[u] = ap < n_ap;
            const uint32_t apc = ok[u] ? ap : 0u;
            const uint32_t ba = b * (uint32_t)a.A + apc / (uint32_t)a.P;
            const int p = (int)(apc % (uint32_t)a.P);
            const int t = (p * a.K + k) * a.S + s;
            qs[u] = (b * (uint32_t)(a.K * a.S) + (uint32_t)lvl) * n_ap + apc;   // rank slot
            st[u] = make_stencil(a, (int64_t)ba, t);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                // rows of the level outside the tile give a negative or too large
                // index (outside corners have row -1: also rejected)
                const int32_t j = st[u].row[c] - lo;
                if (ok[u] && st[u].row[c] >= 0 && j >= 0 && j < nr)
                    a.rank[(size_t)qs[u] * 4 + c] = atomicAdd(&hist[j], 1u);
            }
        }
    }
    __syncthreads();
    for (int j = threadIdx.x; j < nr; j += blockDim.x) a.cnt[row0 + (uint32_t)(lo + j)] = hist[j];
}

// Exclusive prefix sum of cnt inside tiles of kScanTile rows, tile totals to
// tile_prefix[tile]; scan_totals_kernel then turns those into their exclusive
// prefix.  (A last-workgroup-finishes pattern in one launch needs a device-scope
// fence per workgroup, which on this part writes back and invalidates the XCD's
// whole L2: 33 us for 498 tiles, against 7 + 5 us in two launches.)
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
    // v becomes the exclusive prefix; lng marks the long rows (more than
    // kGatherLong entries), whose flag goes into local_start's top bit (the
    // prefix inside a tile stays below 2^31: the host caps the sample count)
    uint32_t tot = 0, vmax = 0, lng = 0;
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) {
        const uint32_t c = v[j];
        v[j] = tot;
        tot += c;
        vmax = max(vmax, c);
        lng |= (c > (uint32_t)kGatherLong ? 1u : 0u) << j;
    }
    if (a.det) {   // the longest row bounds every row sum of the deterministic form
        for (int m = 1; m < kWave; m <<= 1)
            vmax = max(vmax, (uint32_t)__shfl_xor((int)vmax, m, kWave));
        if (threadIdx.x % kWave == 0) atomicMax(a.scan_done + kCtrlMaxCnt, vmax);
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
        auto f = [&](int j) { return (excl + v[j]) | (lng >> j & 1u ? kEntryLongRow : 0u); };
#pragma unroll
        for (int j = 0; j < kScanItems / 4; ++j)
            dst[j] = make_uint4(f(4 * j), f(4 * j + 1), f(4 * j + 2), f(4 * j + 3));
    } else {
#pragma unroll
        for (int j = 0; j < kScanItems; ++j)
            if (base + j < n)
                a.local_start[base + j] = (excl + v[j]) | (lng >> j & 1u ? kEntryLongRow : 0u);
    }
    if (threadIdx.x == kScanThreads - 1) a.tile_tot[blockIdx.x] = excl + tot;
}

// One workgroup: tile_prefix becomes the exclusive prefix of the tile totals
// (with the grand total in tile_prefix[n_tiles]), and the deterministic form's
// bounds are reduced.  The row-ordered backward leaves both to bucket_kernel
// where the tiles are few.
__global__ void __launch_bounds__(kScanThreads) scan_totals_kernel(KArgs a) {
    tile_totals_prefix(a, a.tile_prefix);
    if (a.det) reduce_det_bounds(a);
}

// ------------------------------------------------------------------------------------
// deterministic backward: 64-bit fixed point
// ------------------------------------------------------------------------------------
// Every feature-gradient term cw * w * grad_out is rounded once to a multiple
// of 2^-E and summed as a 64-bit integer, so a row's sum does not depend on the
// order its terms are added in (nor on how a long row is split).  E is chosen
// from bound = max|grad_out| * max|w| * (longest row) -- cw <= 1 -- so that
// |sum| * 2^E < 2^50 (one bit spare for the rounding of a term's product); the
// rounding error of a term is at most 2^-(E+1).
__device__ __forceinline__ int det_exponent(const KArgs& a) {
    const double bound = (double)__uint_as_float(a.scan_done[kCtrlMaxGo]) *
                         (double)__uint_as_float(a.scan_done[kCtrlMaxW]) *
                         (double)a.scan_done[kCtrlMaxCnt];
    if (!(bound > 0.0) || !(bound < 1e300)) return 0;
    int e;
    frexp(bound, &e);                      // bound < 2^e
    return 50 - e;
}
// Rounding a term t to the integer RNE(t 2^E) in three instructions: with
// |t 2^E| < 2^51, t 2^E + 1.5 * 2^52 lies in [2^52, 2^53), where binary64 spacing
// is 1 (so the fma rounds t 2^E to an integer, ties to even: the constant is
// even) and the encoding of an integer is that integer plus a fixed offset.
// Encodings are summed as 64-bit words (wrapping); fixed_value() removes the
// offset once per term summed.
constexpr double kFixMagic = 6755399441055744.0;            // 1.5 * 2^52
__device__ __forceinline__ unsigned long long fixed_code(float t, double scale) {
    return (unsigned long long)__double_as_longlong(fma((double)t, scale, kFixMagic));
}
__device__ __forceinline__ long long fixed_value(unsigned long long code_sum, uint32_t terms) {
    return (long long)(code_sum -
                       (unsigned long long)terms * (unsigned long long)__double_as_longlong(kFixMagic));
}
__device__ __forceinline__ float from_fixed(long long v, int E) {
    return (float)ldexp((double)v, -E);
}

// After the gather: each long row's fixed-point sum to binary32, stored (or added,
// when accumulating) into grad_feat.  One wave per listed long row.
__global__ void __launch_bounds__(256) long_rows_kernel(KArgs a) {
    const uint32_t w = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    const int lane = threadIdx.x % kWave;
    if (w >= min(a.scan_done[kCtrlLongRows], a.n_slots)) return;
    const int E = det_exponent(a);
    const uint32_t row = a.long_rows[w];
    const long long* slot = a.slots + (size_t)(first_entry(a, a.tile_prefix, row) / kSlotStride) * a.C;
    float* out = a.grad_feat + (size_t)row * a.C;
    for (int c = lane; c < a.C; c += kWave) {
        const float v = from_fixed(slot[c], E);
        out[c] = a.accumulate ? out[c] + v : v;
    }
}

// Each wave covers the range [e0, e0 + kGatherChunk) of the row-sorted entry
// list.  A row with at most kGatherLong entries is owned by the wave whose
// range holds its first entry: that wave follows it past the range end and
// writes it once with plain stores (or adds to it, when accumulating), so the
// sum of a short row needs no atomic.  A longer row (the coarse levels'
// rows, hit by hundreds of samples) is summed range by range and each range's
// partial sum is added with atomics onto the pre-zeroed row; this keeps every
// wave's walk under 2 * kGatherChunk entries instead of letting one wave walk
// a whole hot row.
//
// The walk is scalar work per entry (the wave moves through the entries one at
// a time, lanes over channels), and the scalar unit is shared by the whole
// compute unit, so it is kept to a few instructions per entry: the entries
// (two windows of 64) sit in lane registers and are read back with readlane;
// they carry ready byte offsets; grad_out rows and weights are read through
// buffer resources with a scalar offset; the walk is split into the entries
// inside the range (only a row-change test each) and a tail (the rest of a
// short row that crosses the range end).  Batches of U entries are issued one
// batch ahead of the one being added up.
//
// Row-ordered backward (FUSED): every entry also loads its feature row (a
// repeat of the previous entry's row is an L1 hit) and, per weight group, the
// dot product of that row with the entry's grad_out row is summed over the
// group's lanes and stored for finalize_kernel.
// The walk is latency-bound: small batches that leave room for many waves per
// SIMD beat deep batches (row-ordered, nuScenes-shaped: 2 entries per batch at 7
// waves per SIMD 154 us per backward call, 4 entries at 5 waves 179 us).
// SEG: lanes per weight group in the row-ordered form when fixed at compile time
// (0: read from D), so that the group sums unroll to their DPP steps alone.
template <typename T, int VEC, int NV, bool FUSED, bool DET, int SEG = 0, int UB = 0>
__global__ void __launch_bounds__(256, NV == 1 ? (DET && sizeof(T) == 4 ? 4 : 5) : (NV == 2 ? 4 : 1)) gather_kernel(KArgs a) {
    if (blockIdx.x >= a.gather_blocks) {
        loc_reduce_role(a);
        return;
    }
    // entries per batch, within the register budget.  One vector per lane: two
    // entries per batch in the row-ordered form (66 registers, 7 waves per SIMD)
    // and four in the plain form measured faster than larger batches at lower
    // occupancy.  UB overrides the row-ordered form's batch where feature rows are
    // sparse (most entries load a row of their own, and the wave waits on those
    // loads): there more entries in flight per wave pay for the lower occupancy.
    constexpr int U = UB ? UB
                         : FUSED ? (NV == 1 ? 2 : (NV >= 4 ? 1 : 4 / NV))
                                 : (NV == 1 ? 4 : (NV >= 8 ? 1 : 8 / NV));
    // FUSED: the feature row of the entry being added; a batch loads an entry's
    // row only where it differs from the previous entry's (else the load points
    // past the buffer: no memory request, zeros, and the row is kept here)
    float fcur[NV][VEC];
    static_assert(!FUSED || VEC == 4, "the row-ordered backward reads 4 channels per lane");
    constexpr uint32_t kNone = 0xffffffffu;
    static_assert(kGatherChunk == kWave && kGatherLong <= kGatherChunk, "window layout");
    static_assert(kWave % U == 0, "batches tile a window");
    // Every value the walk branches on is wave-uniform; readfirstlane says so,
    // so that the loops below run on scalar branches.
    auto uni = [](uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); };
    const uint32_t total = uni(min(a.tile_prefix[a.n_tiles], 4u * a.n_samples));
    const uint32_t w = uni((blockIdx.x * blockDim.x + threadIdx.x) / kWave);
    const int lane = threadIdx.x % kWave;
    const uint32_t e0 = w * (uint32_t)kGatherChunk;
    if (e0 >= total) return;
    const int n1 = (int)(min(e0 + (uint32_t)kGatherChunk, total) - e0);   // entries in range
    const int C = a.C;
    const uint32_t go_bytes = a.n_anchors * (uint32_t)C * 4u;
    const uint32_t w_bytes = a.n_samples * (uint32_t)a.G * 4u;

    // 64 consecutive entries, one per lane; past the end the row is kNone.  An
    // entry that is out of range anyway (a workspace shared by overlapping
    // calls) is read as a zero-weight term of row 0.
    auto load_window = [&](uint32_t base) -> uint4 {
        const uint32_t e = base + (uint32_t)lane;
        uint4 v = make_uint4(kNone, 0u, 0u, 0u);
        if (e < total) {
            v = *reinterpret_cast<const uint4*>(a.entries + e);
            if ((v.x & ~kEntryLongRow) >= a.n_rows || v.y >= w_bytes || v.w >= go_bytes)
                v = make_uint4(0u, 0u, 0u, 0u);
        }
        return v;
    };
    const uint4 win0 = load_window(e0);
    const uint4 win1 = load_window(e0 + (uint32_t)kWave);
    const uint32_t last0 = (uint32_t)__builtin_amdgcn_readlane((int)win0.x, kWave - 1);
    const uint32_t before = (e0 == 0) ? kNone : uni(a.entries[e0 - 1].row);

    // where this wave starts: at e0, unless the row there began earlier and is
    // short (then its owner covers it) -- then at the first row start in range.
    // The shuffle runs on all lanes before the select: executed only by lanes
    // != 0 it would read lane 0 as inactive, i.e. as 0.
    const uint32_t up0 = (uint32_t)__shfl_up((int)win0.x, 1, kWave);
    const uint32_t prev0 = lane == 0 ? before : up0;
    const uint64_t starts = __ballot(lane < n1 && win0.x != prev0);
    const uint32_t row_at_e0 = (uint32_t)__builtin_amdgcn_readlane((int)win0.x, 0);
    int sp = 0;
    if (before == row_at_e0 && !(row_at_e0 & kEntryLongRow)) {
        if (starts == 0) return;            // the whole range continues a short row owned earlier
        sp = __ffsll((unsigned long long)starts) - 1;
    }
    uint32_t cur = (uint32_t)__builtin_amdgcn_readlane((int)win0.x, sp);

    const int nvec = C / VEC;
    int vv[NV];
    uint32_t lo_go[NV], lo_w[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int v = lane + kWave * i;
        vv[i] = v < nvec ? v : 0;
        lo_go[i] = (uint32_t)(vv[i] * VEC * 4);
        lo_w[i] = (uint32_t)(vv[i] * VEC / a.D * 4);
    }
    const __amdgpu_buffer_rsrc_t r_go = make_rsrc(a.grad_out, go_bytes);
    const __amdgpu_buffer_rsrc_t r_w = make_rsrc(a.weights, w_bytes);
    // FUSED: feature rows of every batch image, by flat row
    const __amdgpu_buffer_rsrc_t r_f = make_rsrc(a.feat, FUSED ? a.feat_all_bytes : 0u);
    const int G = a.G;
    const int seg = SEG ? SEG : (FUSED ? a.D / VEC : 1);   // lanes per weight group (a power of two)
    uint32_t lo_f[NV];
    bool dvalid[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        lo_f[i] = (uint32_t)(vv[i] * VEC * (int)sizeof(T));
        dvalid[i] = lane + kWave * i < nvec && (lane & (seg - 1)) == seg - 1;
    }

    // DET: 64-bit fixed-point sums (multiples of 2^-E) kept as sums of the
    // terms' codes (fixed_code), `terms` of them; else binary32
    using Acc = typename std::conditional<DET, unsigned long long, float>::type;
    const int E = DET ? det_exponent(a) : 0;
    const double scale = DET ? ldexp(1.0, E) : 0.0;
    uint32_t terms = 0;
    Acc acc[NV][VEC];
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int k = 0; k < VEC; ++k) acc[i][k] = 0;

    // Write (or add) the row's sum through a buffer resource that spans exactly
    // that row: lanes past its last vector fall outside the range and their
    // stores / atomics are dropped by the hardware, so no lane-dependent branch
    // enters the walk (it would turn every exit of the loops into exec-masked
    // code).
    auto flush = [&](uint32_t row_bits) {
        const uint32_t row = row_bits & ~kEntryLongRow;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(a.grad_feat + (size_t)row * C, (uint32_t)C * 4u);
        long long* slot = nullptr;
        if constexpr (DET) {
            if (row_bits & kEntryLongRow)
                slot = a.slots + (size_t)(first_entry(a, a.tile_prefix, row) / kSlotStride) * C;
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const uint32_t off = (uint32_t)((lane + kWave * i) * VEC * 4);
            if (row_bits & kEntryLongRow) {
                if constexpr (DET) {
                    // 64-bit integer additions: exact, so their order does not matter
                    const int c0 = (lane + kWave * i) * VEC;
                    if (c0 < C) {
#pragma unroll
                        for (int k = 0; k < VEC; ++k)
                            atomicAdd(reinterpret_cast<unsigned long long*>(slot + c0 + k),
                                      (unsigned long long)fixed_value(acc[i][k], terms));
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < VEC; ++k)
                        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[i][k], r, off + 4u * k,
                                                                        0, 0);
                }
            } else {
                float o[VEC];
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    if constexpr (DET)
                        o[k] = from_fixed(fixed_value(acc[i][k], terms), E);
                    else
                        o[k] = acc[i][k];
                }
                if (a.accumulate) {
                    float old[VEC];
                    VecLoad<float, VEC>::run(r, off, 0u, old);
#pragma unroll
                    for (int k = 0; k < VEC; ++k) o[k] += old[k];
                }
                if constexpr (VEC == 4) {
                    __builtin_amdgcn_raw_buffer_store_b128(
                        __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int,
                                           make_float4(o[0], o[1], o[2], o[3])),
                        r, off, 0, 0);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[0]), r, off, 0, 0);
                }
            }
#pragma unroll
            for (int k = 0; k < VEC; ++k) acc[i][k] = 0;
        }
        terms = 0;
    };

    struct Batch {
        uint32_t row[U];
        float cw[U];
        float go[U][NV][VEC];
        float wt[U][NV];
        RawVec<T, VEC> f[U][NV];   // FUSED: the entry's feature row, where it starts a new row
        bool fnew[U];          // FUSED: the entry's row differs from the previous entry's
        uint32_t dof[U];       // FUSED: float index of the entry's dot products
    };
    // entries at positions p0 .. p0+U-1 of window `win` (p0 a multiple of U);
    // row_before: the row of the entry before the window (kNone for the first
    // window, so that the first entry a wave takes always loads its row)
    // with_rows = false: the entries are only added where they continue the
    // current row, whose feature row is loaded already
    auto issue = [&](const uint4& win, uint32_t row_before, int p0, Batch& B, bool with_rows) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = p0 + u;
            B.row[u] = (uint32_t)__builtin_amdgcn_readlane((int)win.x, idx);
            const uint32_t wo = (uint32_t)__builtin_amdgcn_readlane((int)win.y, idx);
            B.cw[u] = __int_as_float(__builtin_amdgcn_readlane((int)win.z, idx));
            const uint32_t gow = (uint32_t)__builtin_amdgcn_readlane((int)win.w, idx);
            const uint32_t go = gow & ~3u;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                VecLoad<float, VEC>::run(r_go, lo_go[i], go, B.go[u][i]);
                B.wt[u][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_w, lo_w[i], wo, 0));
            }
            if constexpr (FUSED) {
                // previous entry's row: in this batch, the window before p0, or
                // none (the first entry a wave takes always loads its row)
                const uint32_t prev =
                    u > 0 ? B.row[u > 0 ? u - 1 : 0]
                          : (p0 > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)win.x, p0 > 0 ? p0 - 1 : 0)
                                    : row_before);
                B.fnew[u] = with_rows && B.row[u] != prev;
                if (B.fnew[u]) {
                    const uint32_t rb = (B.row[u] & ~kEntryLongRow) * (uint32_t)a.row_bytes;
#pragma unroll
                    for (int i = 0; i < NV; ++i) B.f[u][i].load(r_f, lo_f[i], rb);
                }
                // (4 q + corner) * G with wo = 4 q G
                B.dof[u] = wo + (gow & 3u) * (uint32_t)G;
            }
        }
    };
    auto add = [&](const Batch& B, int u) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const float sc = B.cw[u] * B.wt[u][i];
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                if constexpr (DET)
                    acc[i][k] += fixed_code(sc * B.go[u][i][k], scale);
                else
                    acc[i][k] += sc * B.go[u][i][k];
            }
        }
        if constexpr (DET) ++terms;
        if constexpr (FUSED) {
            if (B.fnew[u]) {
#pragma unroll
                for (int i = 0; i < NV; ++i) B.f[u][i].to_float(fcur[i]);
            }
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                float d = 0.0f;
#pragma unroll
                for (int k = 0; k < VEC; ++k) d += B.go[u][i][k] * fcur[i][k];
                d = group_sum(d, seg);
                if (dvalid[i]) a.dots[B.dof[u] + (uint32_t)(lo_w[i] >> 2)] = d;
            }
        }
    };

    // phase 1: positions sp .. n1-1 of win0; a row change flushes the finished row
    Batch A, B;
    {
        const int first = sp - sp % U;
        int p = first;
        issue(win0, kNone, p, A, true);
        while (true) {
            const int pn = min(p + U, kWave - U);
            issue(win0, kNone, pn, B, true);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int pos = p + u;
                if (pos >= sp && pos < n1) {
                    if (A.row[u] != cur) {
                        flush(cur);
                        cur = A.row[u];
                    }
                    add(A, u);
                }
            }
            p += U;
            if (p >= n1) break;
            const int pn2 = min(p + U, kWave - U);
            issue(win0, kNone, pn2, A, true);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int pos = p + u;
                if (pos < n1) {
                    if (B.row[u] != cur) {
                        flush(cur);
                        cur = B.row[u];
                    }
                    add(B, u);
                }
            }
            p += U;
            if (p >= n1) break;
        }
    }
    // phase 2: a short row that runs past the range end is finished here (it can
    // only continue into win1: a range that ends early ends at the last entry).
    // Its entries continue the current row, whose feature row is loaded already.
    // Batches of up to 2 entries keep the two-batch pipeline; with deeper batches
    // the batch it prefetches past the row's end cost more than the overlap saves.
    if (n1 == kWave && !(cur & kEntryLongRow)) {
        bool done = false;
        if constexpr (U <= 2) {
            int p = 0;
            issue(win1, last0, 0, A, false);
            while (true) {
                issue(win1, last0, min(p + U, kWave - U), B, false);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (!done) {
                        if (A.row[u] != cur)   // row ended (kNone past the last entry)
                            done = true;
                        else
                            add(A, u);
                    }
                }
                p += U;
                if (done || p >= kWave) break;
                issue(win1, last0, min(p + U, kWave - U), A, false);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (!done) {
                        if (B.row[u] != cur)
                            done = true;
                        else
                            add(B, u);
                    }
                }
                p += U;
                if (done || p >= kWave) break;
            }
        } else {
            for (int p = 0; p < kWave && !done; p += U) {
                issue(win1, last0, p, A, false);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (!done) {
                        if (A.row[u] != cur)
                            done = true;
                        else
                            add(A, u);
                    }
                }
            }
        }
    }
    flush(cur);
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

template <typename T, int VEC, int NV>
hipError_t sliced_launch(const KArgs& a, const LaunchShape& s, dim3 grid, hipStream_t st) {
    hipLaunchKernelGGL((da_backward_sliced_kernel<T, VEC, NV>), grid, dim3(kWave * s.waves),
                       s.lds_bytes, st, a);
    return hipGetLastError();
}

template <typename T, int VEC>
hipError_t sliced_dispatch(const KArgs& a, const LaunchShape& s, dim3 grid, hipStream_t st) {
    switch (s.nvc) {
        case 1: return sliced_launch<T, VEC, 1>(a, s, grid, st);
        case 2: return sliced_launch<T, VEC, 2>(a, s, grid, st);
        case 4: return sliced_launch<T, VEC, 4>(a, s, grid, st);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, int VEC, bool FUSED, bool DET>
hipError_t gather_dispatch_det(const KArgs& a, const LaunchShape& s, dim3 grid, hipStream_t st) {
    // C <= 1024 in the backward: 16-byte vectors need at most 4 per lane
    switch (s.gather_nv) {
        case 1:
            if constexpr (FUSED) {
                // 32 channels per weight group (C = 256 with G = 8, and the like)
                if (a.D == 8 * VEC) {
                    if (a.gather_deep)
                        hipLaunchKernelGGL((gather_kernel<T, VEC, 1, FUSED, DET, 8, 4>), grid,
                                           dim3(kGatherThreads), 0, st, a);
                    else
                        hipLaunchKernelGGL((gather_kernel<T, VEC, 1, FUSED, DET, 8>), grid,
                                           dim3(kGatherThreads), 0, st, a);
                    break;
                }
            }
            hipLaunchKernelGGL((gather_kernel<T, VEC, 1, FUSED, DET>), grid, dim3(kGatherThreads), 0, st, a);
            break;
        case 2: hipLaunchKernelGGL((gather_kernel<T, VEC, 2, FUSED, DET>), grid, dim3(kGatherThreads), 0, st, a); break;
        case 4: hipLaunchKernelGGL((gather_kernel<T, VEC, 4, FUSED, DET>), grid, dim3(kGatherThreads), 0, st, a); break;
        case 8:
            if constexpr (VEC == 1) {
                hipLaunchKernelGGL((gather_kernel<T, 1, 8, false, DET>), grid, dim3(kGatherThreads), 0, st, a);
                break;
            }
            return hipErrorInvalidValue;
        case 16:
            if constexpr (VEC == 1) {
                hipLaunchKernelGGL((gather_kernel<T, 1, 16, false, DET>), grid, dim3(kGatherThreads), 0, st, a);
                break;
            }
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, int VEC, bool FUSED>
hipError_t gather_dispatch(const KArgs& a, const LaunchShape& s, dim3 grid, hipStream_t st) {
    return a.det ? gather_dispatch_det<T, VEC, FUSED, true>(a, s, grid, st)
                 : gather_dispatch_det<T, VEC, FUSED, false>(a, s, grid, st);
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
                                   int feat_dtype, hipStream_t stream) {
    KArgs k = a;
    k.anchor_blocks = (uint32_t)n_anchors_total;
    const dim3 grid((unsigned)n_anchors_total, 1);
    return with_elem(feat_dtype, [&](auto t) {
        return anchor_dispatch_scalar<decltype(t), true>(k, s, grid, stream);
    });
}

// The gather form's first launch: zero the control words and row counts and,
// for a 16-bit grad_out, write its binary32 copy.
__global__ void __launch_bounds__(256) prep_kernel(uint32_t* __restrict__ zero, int64_t n_zero,
                                                    const void* __restrict__ src, int dtype,
                                                    float* __restrict__ dst, int64_t n_conv) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint4* z4 = reinterpret_cast<uint4*>(zero);           // 256-byte aligned
    for (int64_t j = i0; j < n_zero / 4; j += stride) z4[j] = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t j = n_zero / 4 * 4 + i0; j < n_zero; j += stride) zero[j] = 0u;
    for (int64_t j = i0; j < n_conv; j += stride) dst[j] = load_elem(src, j, dtype);
}

hipError_t launch_backward_gather(const KArgs& a, const LaunchShape& s, int64_t n_anchors_total,
                                  int feat_dtype, hipStream_t stream) {
    if (a.go_dtype != kF32) return hipErrorInvalidValue;   // the gather reads binary32 rows
    // the control words and the row counts are one zeroed range; a 16-bit
    // grad_out (go_src) is converted into a.grad_out in the same launch
    const int64_t n_zero = (int64_t)(a.cnt - a.scan_done) + a.n_rows;
    const int64_t n_conv = a.go_src ? (int64_t)a.n_anchors * a.C : 0;
    hipLaunchKernelGGL(prep_kernel,
                       dim3((unsigned)std::min<int64_t>(8192, blocks_for(std::max(n_zero / 4, n_conv), 256))),
                       dim3(256), 0, stream, a.scan_done, n_zero, a.go_src, a.go_src_dtype,
                       const_cast<float*>(static_cast<const float*>(a.grad_out)), n_conv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the blocks of the atomic and tile paths take 256 samples each; the LDS path
    // count_per (1 or kCountLdsPer) times as many, its blocks past the level's
    // samples idle
    const dim3 cgrid(blocks_for((int64_t)a.A * a.P, kCountThreads), (unsigned)(a.K * a.S),
                     (unsigned)(a.n_anchors / (uint32_t)a.A));
    if (a.det && (uint64_t)cgrid.x * cgrid.y * cgrid.z != a.count_blocks) return hipErrorInvalidValue;
    // Row tiles take the levels above kCountTileRows rows.  Once they run, they also
    // take every level above the LDS histogram's kCountLdsRows: each tile workgroup
    // scans a whole level's pairs whatever its rows, so the extra levels' workgroups
    // run beside the others at no cost in time, and their returning atomics go.
    int32_t max_rows = 0;
    for (int l = 0; l < a.K * a.S; ++l) max_rows = std::max(max_rows, a.lv.H[l] * a.lv.W[l]);
    KArgs ca = a;
    ca.count_tile_rows = max_rows > kCountTileRows ? kCountLdsRows : kCountTileRows;
    if (a.count_per == kCountLdsPer)
        hipLaunchKernelGGL(count_kernel<kCountLdsPer>, cgrid, dim3(kCountThreads), 0, stream, ca);
    else
        hipLaunchKernelGGL(count_kernel<1>, cgrid, dim3(kCountThreads), 0, stream, ca);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (max_rows > kCountTileRows) {
        const dim3 tgrid((unsigned)((max_rows + kCountTileRows - 1) / kCountTileRows),
                         (unsigned)(a.K * a.S), (unsigned)(a.n_anchors / (uint32_t)a.A));
        hipLaunchKernelGGL(count_tiles_kernel, tgrid, dim3(kCountTileThreads), 0, stream, ca);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(scan_tiles_kernel, dim3(a.n_tiles), dim3(kScanThreads), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    KArgs k = a;
    // the row-ordered form's bucket kernel adds up the tile totals itself
    k.tot_in_bucket = a.fused && a.n_tiles <= (uint32_t)kBucketLdsTiles ? 1 : 0;
    if (!k.tot_in_bucket) {
        hipLaunchKernelGGL(scan_totals_kernel, dim3(1), dim3(kScanThreads), 0, stream, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int64_t row_waves = ((int64_t)a.n_rows + kWave - 1) / kWave;
    // rows to zero before the gather: none when accumulating, unless long rows
    // need their 64-bit accumulation rows zeroed
    const int64_t zwaves = (a.accumulate && !a.det) ? 0 : row_waves;
    const int64_t waves = ((int64_t)a.n_samples * 4 + kGatherChunk - 1) / kGatherChunk;
    if (a.fused) {
        // bucketing (+ zeroing blocks), the gather with the dot products, then
        // the per-sample gradients
        {
            // kSlices equal parts of the (image, level, 256-pair chunk) list
            const int64_t triples = (int64_t)(a.n_anchors / (uint32_t)a.A) * a.K * a.S *
                                    blocks_for((int64_t)a.A * a.P, 256);
            k.anchor_blocks = (uint32_t)(kSlices * ((triples + kSlices - 1) / kSlices));
        }
        hipLaunchKernelGGL(bucket_kernel, dim3((unsigned)(k.anchor_blocks + blocks_for(zwaves, 256 / kWave))),
                           dim3(256), 0, stream, k);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        k.gather_blocks = blocks_for(waves, kGatherThreads / kWave);
        const dim3 ggrid(k.gather_blocks);
        e = with_elem(feat_dtype, [&](auto t) {
            return gather_dispatch<decltype(t), 4, true>(k, s, ggrid, stream);
        });
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(finalize_kernel, dim3(blocks_for((int64_t)a.n_samples, kFinalizeThreads)),
                           dim3(kFinalizeThreads),
                           0, stream, k);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((a.S & (a.S - 1)) != 0 || a.S > kWave) {
            hipLaunchKernelGGL(loc_reduce_kernel, dim3(blocks_for((int64_t)a.n_anchors * a.npk, 256)),
                               dim3(256), 0, stream, k);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    } else {
        // per-anchor kernel, followed by blocks that zero the rows the gather
        // does not store whole
        k.anchor_blocks = (uint32_t)(a.sliced ? n_anchors_total * kSlices : n_anchors_total);
        const dim3 grid((unsigned)(k.anchor_blocks + blocks_for(zwaves, s.waves)), 1);
        e = with_elem(feat_dtype, [&](auto t) {
            using T = decltype(t);
            constexpr int V = sizeof(T) == 2 ? 8 : 4;
            if (a.sliced)
                return s.vec == V ? sliced_dispatch<T, V>(k, s, grid, stream)
                                  : sliced_dispatch<T, 1>(k, s, grid, stream);
            return s.vec == V ? anchor_dispatch_vec<T, V>(k, s, grid, stream)
                              : anchor_dispatch_scalar<T, false>(k, s, grid, stream);
        });
        if (e != hipSuccess) return e;
        // gather: one wave per chunk of the largest possible entry count (4 per
        // sample; waves past the real total return at once), followed in the
        // sliced form by blocks that add up the location partials
        k.gather_blocks = blocks_for(waves, kGatherThreads / kWave);
        const int64_t lr = a.sliced ? blocks_for((int64_t)a.n_anchors * a.npk, kGatherThreads) : 0;
        const dim3 ggrid((unsigned)(k.gather_blocks + lr));
        e = a.gather_vec == 4 ? gather_dispatch<float, 4, false>(k, s, ggrid, stream)
                              : gather_dispatch<float, 1, false>(k, s, ggrid, stream);
        if (e != hipSuccess) return e;
    }
    if (a.det) {
        hipLaunchKernelGGL(long_rows_kernel, dim3(blocks_for(a.n_slots, 256 / kWave)), dim3(256), 0,
                           stream, k);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace da
