// libdeformagg host side: argument checks, launch-shape selection, dispatch.
//
// Every check runs before anything is enqueued, so a failing call leaves all
// outputs untouched and needs no GPU.  See include/deformagg.h for the
// contract of each entry point.

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "da_internal.h"
#include "da_pack.h"
#include "deformagg.h"
#include "host_errors.h"

namespace {

thread_local char g_last_error[512] = "";

da_status fail(da_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int64_t pow2_factor(int64_t x) { return x & -x; }   // largest power of two dividing x (x > 0)

int ilog2(int64_t x) {
    int r = 0;
    while ((int64_t(1) << (r + 1)) <= x) ++r;
    return r;
}

constexpr uint64_t kU32Max = 0xffffffffull;

static_assert(da::kF32 == DA_F32 && da::kBF16 == DA_BF16 && da::kF16 == DA_F16, "da_dtype values");
bool valid_dtype(int32_t t) { return t == DA_F32 || t == DA_BF16 || t == DA_F16; }
int elem_bytes(int32_t t) { return t == DA_F32 ? 4 : 2; }

struct Plan {
    da::KArgs ka;
    da::LaunchShape shape;
    int64_t n_anchors;   // bs * A
    int feat_dtype;
    int elem;            // bytes per feature element
};

// Checks shared by both directions: problem sizes, the level table, the input
// pointers.  Fills ka with everything but the output pointers and the layout.
da_status check_common(const da_problem* p, const void* feat, const int32_t* shape,
                       const int32_t* start, const float* loc, const float* weights,
                       Plan& plan) {
    if (!p) return fail(DA_ERR_INVALID_ARG, "problem is NULL");
    if ((p->flags & ~(DA_FLAG_SLICES_ALWAYS | DA_FLAG_SLICES_NEVER | DA_FLAG_BWD_REGATHER |
                      DA_FLAG_BWD_ROW_ORDER | DA_FLAG_DETERMINISTIC)) != 0 ||
        (p->flags & DA_FLAG_SLICES_ALWAYS && p->flags & DA_FLAG_SLICES_NEVER) ||
        (p->flags & DA_FLAG_BWD_REGATHER && p->flags & DA_FLAG_BWD_ROW_ORDER))
        return fail(DA_ERR_INVALID_ARG, "problem.flags = %d is not a valid combination",
                    (int)p->flags);
    if (p->bs < 0 || p->num_anchors < 0 || p->num_pts < 0)
        return fail(DA_ERR_INVALID_ARG, "bs, num_anchors and num_pts must be >= 0");
    if (p->num_feat < 1 || p->num_embeds < 1 || p->num_cams < 1 || p->num_scale < 1 ||
        p->num_groups < 1)
        return fail(DA_ERR_INVALID_ARG,
                    "num_feat, num_embeds, num_cams, num_scale and num_groups must be >= 1");
    if (p->num_cams > DA_MAX_LEVELS || p->num_scale > DA_MAX_LEVELS ||
        p->num_cams * p->num_scale > DA_MAX_LEVELS)
        return fail(DA_ERR_INVALID_ARG, "num_cams * num_scale = %lld exceeds DA_MAX_LEVELS (%d)",
                    (long long)(p->num_cams * p->num_scale), DA_MAX_LEVELS);
    if (p->num_embeds % p->num_groups != 0)
        return fail(DA_ERR_INVALID_ARG, "num_embeds (%lld) is not a multiple of num_groups (%lld)",
                    (long long)p->num_embeds, (long long)p->num_groups);
    if (!valid_dtype(p->feat_dtype))
        return fail(DA_ERR_INVALID_ARG, "feat_dtype %d is not a da_dtype", (int)p->feat_dtype);
    if (!valid_dtype(p->out_dtype))
        return fail(DA_ERR_INVALID_ARG, "out_dtype %d is not a da_dtype", (int)p->out_dtype);
    if (p->reserved != 0) return fail(DA_ERR_INVALID_ARG, "problem.reserved must be 0");
    if (!shape || !start) return fail(DA_ERR_INVALID_ARG, "spatial_shape / scale_start_index is NULL");
    // sizes that must fit the kernels' 32-bit index arithmetic
    if (p->num_embeds > (1 << 20)) return fail(DA_ERR_UNSUPPORTED, "num_embeds > 2^20");
    if (p->num_anchors > INT32_MAX || p->num_pts > INT32_MAX ||
        p->num_pts * p->num_cams > INT32_MAX / 64)
        return fail(DA_ERR_UNSUPPORTED, "num_anchors or num_pts * num_cams too large");

    const int elem = elem_bytes(p->feat_dtype);
    const int64_t C = p->num_embeds;
    const int64_t nlev = p->num_cams * p->num_scale;
    da::KArgs& ka = plan.ka;
    memset(&ka, 0, sizeof ka);
    for (int64_t l = 0; l < nlev; ++l) {
        const int64_t H = shape[2 * l], W = shape[2 * l + 1], st = start[l];
        if (H < 1 || W < 1 || H > DA_MAX_EXTENT || W > DA_MAX_EXTENT)
            return fail(DA_ERR_INVALID_ARG, "level %lld: (H, W) = (%lld, %lld) outside [1, %d]",
                        (long long)l, (long long)H, (long long)W, DA_MAX_EXTENT);
        if (st < 0 || st + H * W > p->num_feat)
            return fail(DA_ERR_INVALID_ARG,
                        "level %lld: rows [%lld, %lld) do not lie inside num_feat = %lld",
                        (long long)l, (long long)st, (long long)(st + H * W),
                        (long long)p->num_feat);
        ka.lv.H[l] = (int32_t)H;
        ka.lv.W[l] = (int32_t)W;
        ka.lv.start[l] = (int32_t)st;
    }
    // one batch image is addressed by a 32-bit buffer offset, with one row of
    // headroom for the "outside" offset plus a lane offset
    const uint64_t feat_img = (uint64_t)p->num_feat * (uint64_t)C * (uint64_t)elem;
    if (feat_img + 2 * (uint64_t)C * elem > kU32Max)
        return fail(DA_ERR_UNSUPPORTED, "one batch image of mc_ms_feat (%llu bytes) exceeds 4 GiB",
                    (unsigned long long)feat_img);

    const int64_t n_anchor = p->bs * p->num_anchors;
    const bool any_sample = n_anchor > 0 && p->num_pts > 0;
    if (p->bs > 0 && !feat) return fail(DA_ERR_INVALID_ARG, "mc_ms_feat is NULL");
    if (any_sample && (!loc || !weights))
        return fail(DA_ERR_INVALID_ARG, "sampling_location / weights is NULL");
    if (!aligned(feat, elem)) return fail(DA_ERR_INVALID_ARG, "mc_ms_feat is not element aligned");
    if (!aligned(loc, 8)) return fail(DA_ERR_INVALID_ARG, "sampling_location is not 8-byte aligned");
    if (!aligned(weights, 4)) return fail(DA_ERR_INVALID_ARG, "weights is not 4-byte aligned");
    if ((uint64_t)n_anchor * (da::kWave * da::kMaxWaves) > kU32Max)
        return fail(DA_ERR_UNSUPPORTED, "bs * num_anchors = %lld exceeds the grid limit",
                    (long long)n_anchor);

    ka.feat = feat;
    ka.loc = loc;
    ka.weights = weights;
    ka.A = (int32_t)p->num_anchors;
    ka.C = (int32_t)C;
    ka.P = (int32_t)p->num_pts;
    ka.K = (int32_t)p->num_cams;
    ka.S = (int32_t)p->num_scale;
    ka.G = (int32_t)p->num_groups;
    ka.D = (int32_t)(C / p->num_groups);
    ka.npk = (int32_t)(p->num_pts * p->num_cams);
    ka.feat_batch_bytes = (int64_t)feat_img;
    ka.feat_image_bytes = (uint32_t)feat_img;
    ka.row_bytes = (int32_t)(C * elem);
    ka.grow_bytes = (int32_t)(C * 4);
    ka.out_dtype = p->out_dtype;
    ka.go_dtype = p->out_dtype;
    plan.n_anchors = n_anchor;
    plan.feat_dtype = p->feat_dtype;
    plan.elem = elem;
    return DA_OK;
}

// Largest number of (point, camera) pairs whose stencils and weights fit LDS.
da_status choose_pk_chunk(da::KArgs& ka, int desc_bytes, size_t fixed, size_t& lds) {
    const size_t per_pair = (size_t)ka.S * (desc_bytes + 4 * (size_t)ka.G);
    if (fixed + per_pair > (size_t)da::kLdsBudget)
        return fail(DA_ERR_UNSUPPORTED,
                    "one (point, camera) pair needs %zu bytes of LDS (num_scale * num_groups too large)",
                    per_pair + fixed);
    const int64_t fit = (int64_t)((da::kLdsBudget - fixed) / per_pair);
    ka.pk_chunk = (int32_t)std::max<int64_t>(1, std::min<int64_t>(ka.npk, fit));
    lds = fixed + per_pair * ka.pk_chunk;
    return DA_OK;
}

// Level slices pay off once the features outgrow one XCD's L2 (4 MiB): take
// them from twice that, when the levels split into 8 nearly equal shares.
constexpr uint64_t kSliceMinImageBytes = 8ull << 20;

bool want_slices(const da_problem* p) {
    if (p->flags & DA_FLAG_SLICES_NEVER) return false;
    if (p->flags & DA_FLAG_SLICES_ALWAYS) return true;
    const int64_t nlev = p->num_cams * p->num_scale;
    if (nlev < da::kSlices) return false;
    const int64_t m = (nlev + da::kSlices - 1) / da::kSlices;
    if (4 * m * da::kSlices > 5 * nlev) return false;   // more than 1/4 of the slots idle
    const uint64_t elem = (uint64_t)elem_bytes(p->feat_dtype);
    return (uint64_t)p->num_feat * (uint64_t)p->num_embeds * elem >= kSliceMinImageBytes;
}

// Assign the levels to slices: largest first (ties in level order), dealt
// round-robin, so every slice holds the same number of levels give or take
// one.  Returns P * the largest slice's level count.
int32_t fill_slices(da::KArgs& ka) {
    const int nlev = ka.K * ka.S;
    int order[da::kMaxLevels];
    for (int l = 0; l < nlev; ++l) order[l] = l;
    std::stable_sort(order, order + nlev, [&](int u, int v) {
        return (int64_t)ka.lv.H[u] * ka.lv.W[u] > (int64_t)ka.lv.H[v] * ka.lv.W[v];
    });
    for (int x = 0; x < da::kSlices; ++x) ka.lv.slice_nlev[x] = 0;
    for (int i = 0; i < nlev; ++i) {
        const int x = i % da::kSlices;
        ka.lv.slice_level[x][ka.lv.slice_nlev[x]++] = (int8_t)order[i];
    }
    int m = 0;
    for (int x = 0; x < da::kSlices; ++x) m = std::max<int>(m, ka.lv.slice_nlev[x]);
    ka.max_slice_samples = ka.P * m;
    return ka.max_slice_samples;
}

// Waves per workgroup of the sliced kernels.  A slice of one anchor holds few
// samples (P * levels / 8, 39 for 13 points over 24 levels), so small
// workgroups -- many of them resident per CU -- hide the staging latency best;
// measured on MI355X over the nuScenes-shaped and 4 x 510k-row workloads.
constexpr int kSlicedFwdWaves = 4;
constexpr int kSlicedBwdWaves = 2;

// Samples of a slice staged in LDS at once.
bool choose_sample_chunk(da::KArgs& ka, size_t per_sample, size_t fixed, size_t& lds) {
    if (fixed + per_sample > (size_t)da::kLdsBudget) return false;
    const int64_t fit = (int64_t)((da::kLdsBudget - fixed) / per_sample);
    ka.sample_chunk = (int32_t)std::max<int64_t>(1, std::min<int64_t>(ka.max_slice_samples, fit));
    lds = fixed + per_sample * ka.sample_chunk;
    return true;
}

bool sliced_nv_supported(int nv) { return nv == 1 || nv == 2 || nv == 4; }

uint64_t fwd_workspace_bytes(const da_problem* p) {
    if (!want_slices(p)) return 0;
    return (uint64_t)da::kSlices * p->bs * p->num_anchors * p->num_embeds * 4;
}

// Switch a planned forward to level slices when wanted and supported.
void plan_forward_sliced(const da_problem* p, Plan& plan) {
    da::KArgs& ka = plan.ka;
    da::LaunchShape& s = plan.shape;
    if (!want_slices(p) || !sliced_nv_supported(s.nvc) || plan.n_anchors * da::kSlices > INT32_MAX)
        return;
    const int64_t n = fill_slices(ka);
    const int64_t spw = da::kWave / ka.L;
    const int waves =
        (int)std::max<int64_t>(1, std::min<int64_t>(kSlicedFwdWaves, (n + 4 * spw - 1) / (4 * spw)));
    const size_t fixed = (size_t)waves * ka.nv_chunk * ka.L * s.vec * 4 + da::kFwdDescBytes;
    size_t lds = 0;
    if (!choose_sample_chunk(ka, da::kFwdDescBytes + 4 * (size_t)ka.G, fixed, lds)) return;
    ka.sliced = 1;
    s.waves = waves;
    s.lds_bytes = lds;
    // the sweep form (one wave per anchor and slice, samples in y order) where a
    // wave holds two or more samples per step and a slice's samples fit one wave
    const size_t sweep_lds =
        (size_t)(da::kWave + 1) * da::kFwdDescBytes + (size_t)da::kWave * ka.G * 4;
    if (spw >= 2 && n <= da::kWave && sweep_lds <= (size_t)da::kLdsBudget) {
        ka.fwd_sweep = 1;
        s.waves = 1;
        s.lds_bytes = sweep_lds;
    }
}

// Switch a planned gather backward to level slices when wanted and supported.
void plan_backward_sliced(const da_problem* p, Plan& plan) {
    da::KArgs& ka = plan.ka;
    da::LaunchShape& s = plan.shape;
    if (!want_slices(p) || !sliced_nv_supported(s.nvc) || plan.n_anchors * da::kSlices > INT32_MAX)
        return;
    const int64_t n = fill_slices(ka);
    const int64_t spw = da::kWave / ka.L;
    const int waves =
        (int)std::max<int64_t>(1, std::min<int64_t>(kSlicedBwdWaves, (n + 2 * spw - 1) / (2 * spw)));
    size_t lds = 0;
    if (!choose_sample_chunk(ka, da::kBwdDescBytes + 4 * (size_t)ka.G + 4, da::kBwdDescBytes, lds))
        return;
    ka.sliced = 1;
    s.waves = waves;
    s.lds_bytes = lds;
}

da_status plan_forward(const da_problem* p, Plan& plan) {
    da::KArgs& ka = plan.ka;
    const int64_t C = ka.C, D = ka.D;
    const int elem = plan.elem;
    const int vwide = 16 / elem;           // 16-byte vectors
    const int vec = (C % vwide == 0 && D % vwide == 0 && aligned(ka.feat, 16)) ? vwide : 1;
    const int64_t nvec = C / vec;                       // vectors per row
    const int64_t L = std::min<int64_t>(da::kWave, pow2_factor(nvec));
    ka.L = (int32_t)L;
    ka.log2L = ilog2(L);
    ka.nv = (int32_t)(nvec / L);
    // vectors per lane handled by one workgroup: the largest divisor of nv that
    // is <= 8 and keeps a chunk within 1024 channels; grid.y covers the rest
    const int64_t cap = std::min<int64_t>(8, std::max<int64_t>(1, 1024 / (L * vec)));
    int64_t nvc = 1;
    for (int64_t d = std::min<int64_t>(cap, ka.nv); d >= 1; --d)
        if (ka.nv % d == 0) { nvc = d; break; }
    ka.nv_chunk = (int32_t)nvc;
    da::LaunchShape& s = plan.shape;
    s.vec = vec;
    s.nvc = (int)nvc;
    s.chunks = (int)(ka.nv / nvc);
    const int64_t spw = da::kWave / L;
    const int64_t ns = (int64_t)ka.npk * ka.S;
    s.waves = (int)std::max<int64_t>(1, std::min<int64_t>(da::kMaxWaves, (ns + 4 * spw - 1) / (4 * spw)));
    // cross-wave partial sums plus the null descriptor slot
    const size_t fixed = (size_t)s.waves * ka.nv_chunk * L * vec * 4 + da::kFwdDescBytes;
    (void)elem;
    (void)p;
    return choose_pk_chunk(ka, da::kFwdDescBytes, fixed, s.lds_bytes);
}

// Lane layout of the per-anchor backward kernel for vectors of `vec` channels:
// L lanes per row group, `seg` lanes per weight-gradient group reduction, nv
// vectors per lane.  False when more than max_nv vectors per lane are needed.
bool bwd_layout(int64_t C, int64_t D, int64_t vec, int64_t max_nv, int64_t& L, int64_t& seg,
                int64_t& nv) {
    const int64_t Cv = C / vec, Dv = D / vec;
    L = std::min<int64_t>(da::kWave, pow2_factor(Cv));
    if (Dv % L == 0) {
        seg = L;                                  // a lane row lies inside one group
    } else if (pow2_factor(Dv) == Dv) {
        seg = Dv;                                 // a lane row spans L / Dv whole groups
    } else {
        L = std::min<int64_t>(da::kWave, pow2_factor(Dv));
        seg = L;
    }
    nv = Cv / L;
    return nv <= max_nv;
}

// Largest num_embeds the feature-gradient gather handles: 64 lanes of at most 16
// channels (gather_kernel's vectors per lane: 1..4 of 4 channels, 1..16 single
// channels).
constexpr int64_t kGatherMaxC = 1024;

da_status plan_backward(const da_problem* p, Plan& plan, bool gather, const float* grad_feat) {
    da::KArgs& ka = plan.ka;
    const int64_t C = ka.C, D = ka.D;
    if (gather && C > kGatherMaxC)
        return fail(DA_ERR_UNSUPPORTED,
                    "backward: num_embeds = %lld exceeds the feature-gradient gather's %lld",
                    (long long)C, (long long)kGatherMaxC);
    // the gather form only reads features: 16-byte vectors per lane when the
    // rows and groups allow; the scatter form keeps one channel per lane so that
    // each atomic instruction covers consecutive floats
    const int64_t vw = 16 / plan.elem;
    int64_t L = 0, seg = 0, nv = 0, vec = 1;
    if (gather && C % vw == 0 && D % vw == 0 && aligned(ka.feat, 16) &&
        bwd_layout(C, D, vw, 8, L, seg, nv)) {
        vec = vw;
    } else if (!bwd_layout(C, D, 1, 16, L, seg, nv)) {
        return fail(DA_ERR_UNSUPPORTED,
                    "backward: %lld channels per lane (num_embeds / %lld) exceeds 16",
                    (long long)nv, (long long)L);
    }
    ka.L = (int32_t)L;
    ka.log2L = ilog2(L);
    ka.nv = (int32_t)nv;
    ka.nv_chunk = (int32_t)nv;
    ka.seg = (int32_t)seg;
    // feature-gradient gather: 16-byte vectors when rows, groups and the
    // grad_feat pointer allow; then the vectors each lane covers (a power of two)
    ka.gather_vec = (C % 4 == 0 && D % 4 == 0 && aligned(grad_feat, 16)) ? 4 : 1;
    const int64_t gvec = (C / ka.gather_vec + da::kWave - 1) / da::kWave;
    int gnv = 1;
    while (gnv < gvec) gnv <<= 1;
    const uint64_t gimg = (uint64_t)p->num_feat * (uint64_t)C * 4u;
    if (gimg + 8 * (uint64_t)C > kU32Max)
        return fail(DA_ERR_UNSUPPORTED, "one batch image of grad_feat (%llu bytes) exceeds 4 GiB",
                    (unsigned long long)gimg);
    ka.gfeat_batch_bytes = (int64_t)gimg;
    ka.gfeat_image_bytes = (uint32_t)gimg;
    da::LaunchShape& s = plan.shape;
    s.vec = (int)vec;
    s.nvc = (int)nv;
    s.gather_nv = gnv;
    s.chunks = 1;
    const int64_t spw = da::kWave / L;
    s.waves = (int)std::max<int64_t>(
        1, std::min<int64_t>(da::kMaxWaves, (ka.npk + 2 * spw - 1) / (2 * spw)));
    return choose_pk_chunk(ka, da::kBwdDescBytes, da::kBwdDescBytes, s.lds_bytes);
}

da_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return DA_OK;
    return fail(DA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

namespace da {

da_status report_error(da_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

da_status report_hip(hipError_t e, const char* what) { return hip_status(e, what); }

}  // namespace da

namespace {

// The row-ordered backward applies when 4 channels per lane fit the groups
// (C/G a multiple of 4 with C/G/4 a power of two, at most 1024 channels), there
// are at most 16 weight groups, and all batch images together are addressable
// by one 32-bit buffer range.  Only sizes and flags are read.
bool fused_capable(const da_problem* p) {
    if (p->flags & DA_FLAG_BWD_REGATHER) return false;
    const int64_t C = p->num_embeds, G = p->num_groups;
    if (G < 1 || C % G != 0) return false;
    const int64_t D = C / G;
    if (C % 4 != 0 || D % 4 != 0 || C > 1024 || G > 16) return false;
    const int64_t seg = D / 4;
    if (seg > 64 || (seg & (seg - 1)) != 0) return false;
    const uint64_t elem = (uint64_t)elem_bytes(p->feat_dtype);
    const uint64_t all = (uint64_t)p->bs * (uint64_t)p->num_feat * (uint64_t)C * elem;
    return all + 2 * (uint64_t)C * elem <= kU32Max;
}

// The row-ordered form loads a feature row once per run of entries on that row;
// it pays when rows are shared.  Expected corners per row on the largest level
// for spread-out sampling: 4 A P / (H W).  Measured: at 4.2 (nuScenes-shaped)
// row-ordered 154-162 us against per-anchor 189 us; at 1.2 (4 images of
// 160x400 levels, 1500 anchors) the two forms tie within 1.5 % for uniform
// locations (2.00 against 1.98 ms) and row-ordered wins by 12 % for clustered
// ones (1.80 against 2.04 ms), which share rows more than the estimate says.
// Below one corner per row each entry loads a row of its own.
double min_corners_per_row(const da_problem* p, const da::KArgs& ka) {
    double worst = 1e30;
    for (int l = 0; l < ka.K * ka.S; ++l)
        worst = std::min(worst, 4.0 * (double)p->num_anchors * (double)p->num_pts /
                                    ((double)ka.lv.H[l] * (double)ka.lv.W[l]));
    return worst;
}

bool rows_reused(const da_problem* p, const da::KArgs& ka) {
    if (p->flags & DA_FLAG_BWD_ROW_ORDER) return true;
    return min_corners_per_row(p, ka) >= 1.0;
}

// Workspace of the gather form of the backward, each part 256-byte aligned.
struct WsLayout {
    size_t scan_done, cnt, local_start, tile_prefix, rank, entries, loc_part, dots, slots, go32,
        total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Accumulation rows of the deterministic form: one per possible long row.
uint64_t det_slots(uint64_t n_samples) { return 4 * n_samples / (uint64_t)da::kSlotStride + 1; }
// Blocks of count_kernel: 256 (anchor, point) pairs at one level of one batch image.
uint64_t count_blocks(const da_problem* p) {
    return (uint64_t)((p->num_anchors * p->num_pts + 255) / 256) * p->num_cams * p->num_scale *
           p->bs;
}
// grad_out as binary32, when it arrives in a 16-bit type
uint64_t go32_bytes(const da_problem* p) {
    return p->out_dtype == DA_F32 ? 0 : (uint64_t)p->bs * p->num_anchors * p->num_embeds * 4;
}
// the accumulation rows, the list of long rows, then the count blocks' maxima
uint64_t det_bytes(const da_problem* p, uint64_t n_samples) {
    return det_slots(n_samples) * ((uint64_t)p->num_embeds * 8 + 4) + 8 * count_blocks(p);
}

WsLayout ws_layout(uint64_t n_rows, uint64_t n_samples, uint64_t dot_groups, uint64_t slot_bytes,
                   uint64_t go32_bytes) {
    WsLayout w;
    const uint64_t n_tiles = (n_rows + da::kScanTile - 1) / da::kScanTile;
    size_t off = 0;
    w.scan_done = off;          // one counter; cnt follows it directly
    off += 256;
    w.cnt = off;
    off += align256(n_rows * 4);
    w.local_start = off;
    off += align256(n_rows * 4);
    w.tile_prefix = off;                  // then the n_tiles tile totals
    off += align256((2 * n_tiles + 1) * 4);
    w.rank = off;
    off += align256(n_samples * 16);
    w.entries = off;
    off += align256(n_samples * 4 * sizeof(da::Entry));
    w.loc_part = off;
    off += align256(n_samples * 8);
    w.dots = off;
    off += align256(n_samples * 4 * dot_groups * 4);
    w.slots = off;
    off += align256(slot_bytes);
    w.go32 = off;
    off += align256(go32_bytes);
    w.total = off;
    return w;
}

// Sizes of the gather form; fails when its 32-bit row / entry indices overflow.
da_status gather_sizes(const da_problem* p, uint64_t& n_rows, uint64_t& n_samples) {
    n_rows = (uint64_t)p->bs * (uint64_t)p->num_feat;
    n_samples = (uint64_t)p->bs * p->num_anchors * p->num_pts * p->num_cams * p->num_scale;
    // the gather reads grad_out and weights through 32-bit buffer offsets
    const uint64_t go_bytes = (uint64_t)p->bs * p->num_anchors * p->num_embeds * 4;
    const uint64_t w_bytes = n_samples * (uint64_t)p->num_groups * 4;
    if (go_bytes > kU32Max || w_bytes > kU32Max)
        return fail(DA_ERR_UNSUPPORTED,
                    "backward: grad_out (%llu bytes) or weights (%llu bytes) exceed 4 GiB for the "
                    "gather workspace (use da_backward_atomic)",
                    (unsigned long long)go_bytes, (unsigned long long)w_bytes);
    // (entry positions, 4 per sample, stay below 2^31: their top bit is a flag)
    if (n_rows >= (1ull << 31) || n_samples >= (1ull << 29))
        return fail(DA_ERR_UNSUPPORTED,
                    "backward: bs * num_feat (%llu) or the sample count (%llu) is too large for the "
                    "gather workspace (use da_backward_atomic)",
                    (unsigned long long)n_rows, (unsigned long long)n_samples);
    return DA_OK;
}

enum class BwdMode { kGather, kGatherAccumulate, kScatter };

// resolve_ws (may be NULL): supplies the workspace once every argument check has
// passed, given the bytes the call needs (see da::WorkspaceResolver).
da_status backward_impl(BwdMode mode, const da_problem* p, const void* feat,
                        const int32_t* shape, const int32_t* start, const float* loc,
                        const float* weights, const void* grad_out, float* grad_feat,
                        float* grad_loc, float* grad_weights, void* workspace,
                        size_t workspace_bytes, void* stream,
                        da::WorkspaceResolver resolve_ws = nullptr) {
    Plan plan;
    da_status st = check_common(p, feat, shape, start, loc, weights, plan);
    if (st != DA_OK) return st;
    const bool any_sample = plan.n_anchors > 0 && p->num_pts > 0;
    if (p->bs > 0 && !grad_feat) return fail(DA_ERR_INVALID_ARG, "grad_feat is NULL");
    if (plan.n_anchors > 0 && !grad_out) return fail(DA_ERR_INVALID_ARG, "grad_out is NULL");
    if (any_sample && (!grad_loc || !grad_weights))
        return fail(DA_ERR_INVALID_ARG, "grad_loc / grad_weights is NULL");
    if (!aligned(grad_out, elem_bytes(p->out_dtype)))
        return fail(DA_ERR_INVALID_ARG, "grad_out is not element aligned");
    if (!aligned(grad_feat, 4) || !aligned(grad_weights, 4))
        return fail(DA_ERR_INVALID_ARG, "grad_feat / grad_weights not 4-byte aligned");
    if (!aligned(grad_loc, 8)) return fail(DA_ERR_INVALID_ARG, "grad_loc is not 8-byte aligned");
    if (mode == BwdMode::kScatter && (p->flags & DA_FLAG_DETERMINISTIC))
        return fail(DA_ERR_UNSUPPORTED,
                    "da_backward_atomic has no deterministic form (use da_backward)");
    st = plan_backward(p, plan, mode != BwdMode::kScatter, grad_feat);
    if (st != DA_OK) return st;
    da::KArgs& ka = plan.ka;
    ka.grad_out = grad_out;
    ka.grad_feat = grad_feat;
    ka.grad_loc = grad_loc;
    ka.grad_weights = grad_weights;
    hipStream_t s = static_cast<hipStream_t>(stream);

    if (mode != BwdMode::kScatter) {
        uint64_t n_rows = 0, n_samples = 0;
        st = gather_sizes(p, n_rows, n_samples);
        if (st != DA_OK) return st;
        if (any_sample) {
            const bool fusable = fused_capable(p);
            const bool det = p->flags & DA_FLAG_DETERMINISTIC;
            const WsLayout w = ws_layout(n_rows, n_samples, fusable ? (uint64_t)p->num_groups : 0,
                                         det ? det_bytes(p, n_samples) : 0, go32_bytes(p));
            if (resolve_ws) {
                st = resolve_ws(w.total, &workspace, &workspace_bytes);
                if (st != DA_OK) return st;
            }
            if (!workspace) return fail(DA_ERR_INVALID_ARG, "workspace is NULL");
            if (!aligned(workspace, 256))
                return fail(DA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
            if (workspace_bytes < w.total)
                return fail(DA_ERR_INVALID_ARG, "workspace has %zu bytes, %zu needed",
                            workspace_bytes, w.total);
            unsigned char* base = static_cast<unsigned char*>(workspace);
            ka.scan_done = reinterpret_cast<uint32_t*>(base + w.scan_done);
            ka.cnt = reinterpret_cast<uint32_t*>(base + w.cnt);
            ka.local_start = reinterpret_cast<uint32_t*>(base + w.local_start);
            ka.tile_prefix = reinterpret_cast<uint32_t*>(base + w.tile_prefix);
            ka.tile_tot = ka.tile_prefix + (n_rows + da::kScanTile - 1) / da::kScanTile + 1;
            ka.rank = reinterpret_cast<uint32_t*>(base + w.rank);
            ka.entries = reinterpret_cast<da::Entry*>(base + w.entries);
            ka.loc_part = reinterpret_cast<float*>(base + w.loc_part);
            ka.det = det ? 1 : 0;
            ka.slots = reinterpret_cast<long long*>(base + w.slots);
            ka.n_slots = (uint32_t)det_slots(n_samples);
            ka.long_rows = reinterpret_cast<uint32_t*>(ka.slots + (size_t)ka.n_slots * p->num_embeds);
            ka.bound_part = ka.long_rows + ka.n_slots;
            ka.count_blocks = (uint32_t)count_blocks(p);
            ka.count_per = p->num_anchors * p->num_pts >= da::kCountChunkMinPairs ? da::kCountLdsPer : 1;
            if (p->out_dtype != DA_F32) {   // the gather reads binary32 grad_out rows
                ka.go_src = grad_out;
                ka.go_src_dtype = p->out_dtype;
                ka.grad_out = base + w.go32;
                ka.go_dtype = DA_F32;
            }
            ka.n_rows = (uint32_t)n_rows;
            ka.n_samples = (uint32_t)n_samples;
            ka.n_anchors = (uint32_t)plan.n_anchors;
            ka.n_tiles = (uint32_t)((n_rows + da::kScanTile - 1) / da::kScanTile);
            ka.num_feat = (int32_t)p->num_feat;
            ka.accumulate = mode == BwdMode::kGatherAccumulate ? 1 : 0;
            if (fusable && ka.gather_vec == 4 && aligned(feat, 16) && rows_reused(p, ka)) {
                ka.fused = 1;
                ka.dots = reinterpret_cast<float*>(base + w.dots);
                ka.feat_all_bytes =
                    (uint32_t)((uint64_t)p->bs * p->num_feat * p->num_embeds * plan.elem);
                ka.w_vec4 = p->num_groups % 4 == 0 && aligned(weights, 16) &&
                            aligned(grad_weights, 16);
                // 16-bit rows with under two expected corners per row on the largest
                // level: most entries load a row of their own, and deeper batches
                // keep more of those loads in flight
                ka.gather_deep = plan.elem == 2 && min_corners_per_row(p, ka) < 2.0 ? 1 : 0;
            } else {
                plan_backward_sliced(p, plan);
            }
        }
    }
    // the scatter form adds into zeros; the gather form zeroes only the rows no
    // sample touches (inside launch_backward_gather), unless nothing is sampled
    const bool full_fill = mode == BwdMode::kScatter || (mode == BwdMode::kGather && !any_sample);
    if (full_fill && p->bs > 0) {
        st = hip_status(da::launch_fill_zero(grad_feat, p->bs * p->num_feat * p->num_embeds, s),
                        "grad_feat zero fill");
        if (st != DA_OK) return st;
    }
    if (!any_sample) return DA_OK;
    if (mode == BwdMode::kScatter)
        return hip_status(da::launch_backward_scatter(ka, plan.shape, plan.n_anchors, plan.feat_dtype, s),
                          "backward kernel launch");
    return hip_status(da::launch_backward_gather(ka, plan.shape, plan.n_anchors, plan.feat_dtype, s),
                      "backward kernel launch");
}

// Checks and layout shared by the packing entry points.
da_status pack_plan(const da_pack_problem* p, const int32_t* scale_hw, da::PackArgs& pa,
                    int& elem) {
    if (!p) return fail(DA_ERR_INVALID_ARG, "problem is NULL");
    if (p->reserved != 0) return fail(DA_ERR_INVALID_ARG, "problem.reserved must be 0");
    if (p->bs < 0) return fail(DA_ERR_INVALID_ARG, "bs must be >= 0");
    if (p->num_cams < 1 || p->num_scale < 1 || p->num_embeds < 1)
        return fail(DA_ERR_INVALID_ARG, "num_cams, num_scale and num_embeds must be >= 1");
    if (p->num_cams * p->num_scale > DA_MAX_LEVELS)
        return fail(DA_ERR_INVALID_ARG, "num_cams * num_scale = %lld exceeds DA_MAX_LEVELS (%d)",
                    (long long)(p->num_cams * p->num_scale), DA_MAX_LEVELS);
    if (!valid_dtype(p->dtype)) return fail(DA_ERR_INVALID_ARG, "dtype %d is not a da_dtype", (int)p->dtype);
    if (!scale_hw) return fail(DA_ERR_INVALID_ARG, "scale_hw is NULL");
    if (p->bs * p->num_cams > 65535)
        return fail(DA_ERR_UNSUPPORTED, "bs * num_cams = %lld exceeds 65535",
                    (long long)(p->bs * p->num_cams));
    memset(&pa, 0, sizeof pa);
    elem = elem_bytes(p->dtype);
    const int64_t C = p->num_embeds;
    const int64_t c_tiles = (C + 63) / 64;
    int64_t rows = 0, tiles = 0;
    for (int64_t s = 0; s < p->num_scale; ++s) {
        const int64_t H = scale_hw[2 * s], W = scale_hw[2 * s + 1];
        if (H < 1 || W < 1 || H > DA_MAX_EXTENT || W > DA_MAX_EXTENT)
            return fail(DA_ERR_INVALID_ARG, "scale %lld: (H, W) = (%lld, %lld) outside [1, %d]",
                        (long long)s, (long long)H, (long long)W, DA_MAX_EXTENT);
        pa.hw[s] = H * W;
        pa.start_in_cam[s] = rows;
        pa.tile_base[s] = tiles;
        rows += H * W;
        tiles += (H * W + 63) / 64 * c_tiles;
    }
    pa.tile_base[p->num_scale] = tiles;
    if (tiles > INT32_MAX) return fail(DA_ERR_UNSUPPORTED, "too many tiles per camera map");
    pa.rows_per_cam = rows;
    pa.num_feat = rows * p->num_cams;
    if (pa.num_feat > INT32_MAX)
        return fail(DA_ERR_UNSUPPORTED, "num_feat = %lld exceeds 2^31 - 1", (long long)pa.num_feat);
    pa.c_tiles = c_tiles;
    pa.B = (int32_t)p->bs;
    pa.N = (int32_t)p->num_cams;
    pa.S = (int32_t)p->num_scale;
    if (C > INT32_MAX) return fail(DA_ERR_UNSUPPORTED, "num_embeds too large");
    pa.C = (int32_t)C;
    // 16-bit elements go two at a time when every row of both layouts has an even
    // length (then every pair is 4-byte aligned, given 4-byte aligned tensors)
    bool even = C % 2 == 0;
    for (int64_t s = 0; s < p->num_scale; ++s) even = even && pa.hw[s] % 2 == 0;
    pa.pairs = elem == 2 && even ? 1 : 0;
    return DA_OK;
}

da_status pack_pointers(const da_pack_problem* p, const void* const* maps, const void* packed,
                        int elem, da::PackArgs& pa) {
    if (p->bs == 0) return DA_OK;
    if (!maps) return fail(DA_ERR_INVALID_ARG, "maps is NULL");
    if (!packed) return fail(DA_ERR_INVALID_ARG, "packed is NULL");
    if (!aligned(packed, elem)) return fail(DA_ERR_INVALID_ARG, "packed is not element aligned");
    for (int64_t s = 0; s < p->num_scale; ++s) {
        if (!maps[s]) return fail(DA_ERR_INVALID_ARG, "maps[%lld] is NULL", (long long)s);
        if (!aligned(maps[s], elem))
            return fail(DA_ERR_INVALID_ARG, "maps[%lld] is not element aligned", (long long)s);
        pa.maps[s] = const_cast<void*>(maps[s]);
    }
    pa.packed = const_cast<void*>(packed);
    if (pa.pairs) {
        bool al = aligned(packed, 4);
        for (int64_t s = 0; s < p->num_scale; ++s) al = al && aligned(maps[s], 4);
        if (!al) pa.pairs = 0;
    }
    return DA_OK;
}

}  // namespace

extern "C" {

da_status da_pack_layout(const da_pack_problem* p, const int32_t* scale_hw, int32_t* spatial_shape,
                         int32_t* scale_start_index, int64_t* num_feat) {
    da::PackArgs pa;
    int elem = 0;
    const da_status st = pack_plan(p, scale_hw, pa, elem);
    if (st != DA_OK) return st;
    if (!spatial_shape || !scale_start_index || !num_feat)
        return fail(DA_ERR_INVALID_ARG, "spatial_shape / scale_start_index / num_feat is NULL");
    for (int64_t k = 0; k < p->num_cams; ++k)
        for (int64_t s = 0; s < p->num_scale; ++s) {
            const int64_t l = k * p->num_scale + s;
            spatial_shape[2 * l] = scale_hw[2 * s];
            spatial_shape[2 * l + 1] = scale_hw[2 * s + 1];
            scale_start_index[l] = (int32_t)(k * pa.rows_per_cam + pa.start_in_cam[s]);
        }
    *num_feat = pa.num_feat;
    return DA_OK;
}

da_status da_pack_levels(const da_pack_problem* p, const int32_t* scale_hw, const void* const* maps,
                         void* packed, void* stream) {
    da::PackArgs pa;
    int elem = 0;
    da_status st = pack_plan(p, scale_hw, pa, elem);
    if (st != DA_OK) return st;
    st = pack_pointers(p, maps, packed, elem, pa);
    if (st != DA_OK || p->bs == 0) return st;
    return hip_status(da::launch_pack(pa, elem, true, static_cast<hipStream_t>(stream)),
                      "pack kernel launch");
}

da_status da_unpack_levels(const da_pack_problem* p, const int32_t* scale_hw, const void* packed,
                           void* const* maps, void* stream) {
    da::PackArgs pa;
    int elem = 0;
    da_status st = pack_plan(p, scale_hw, pa, elem);
    if (st != DA_OK) return st;
    st = pack_pointers(p, const_cast<const void* const*>(maps), packed, elem, pa);
    if (st != DA_OK || p->bs == 0) return st;
    return hip_status(da::launch_pack(pa, elem, false, static_cast<hipStream_t>(stream)),
                      "unpack kernel launch");
}

da_status da_forward_workspace_size(const da_problem* p, size_t* bytes) {
    if (!bytes) return fail(DA_ERR_INVALID_ARG, "bytes is NULL");
    if (!p) return fail(DA_ERR_INVALID_ARG, "problem is NULL");
    if (p->bs < 0 || p->num_anchors < 0 || p->num_embeds < 1 || p->num_feat < 1 ||
        p->num_cams < 1 || p->num_scale < 1)
        return fail(DA_ERR_INVALID_ARG, "malformed problem sizes");
    *bytes = (size_t)fwd_workspace_bytes(p);
    return DA_OK;
}

da_status da_forward(const da_problem* p, const void* feat, const int32_t* shape,
                     const int32_t* start, const float* loc, const float* weights, void* out,
                     void* workspace, size_t workspace_bytes, void* stream) {
    Plan plan;
    da_status st = check_common(p, feat, shape, start, loc, weights, plan);
    if (st != DA_OK) return st;
    if (plan.n_anchors > 0 && !out) return fail(DA_ERR_INVALID_ARG, "out is NULL");
    if (!aligned(out, elem_bytes(p->out_dtype)))
        return fail(DA_ERR_INVALID_ARG, "out is not element aligned");
    st = plan_forward(p, plan);
    if (st != DA_OK) return st;
    if (workspace) {
        const uint64_t need = fwd_workspace_bytes(p);
        if (!aligned(workspace, 256))
            return fail(DA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
        if (workspace_bytes < need)
            return fail(DA_ERR_INVALID_ARG, "workspace has %zu bytes, %llu needed",
                        workspace_bytes, (unsigned long long)need);
    }
    if (plan.n_anchors == 0) return DA_OK;
    plan.ka.out = out;
    plan.ka.n_anchors = (uint32_t)plan.n_anchors;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (workspace) {
        plan_forward_sliced(p, plan);
        if (plan.ka.sliced) {
            plan.ka.fwd_part = static_cast<float*>(workspace);
            return hip_status(da::launch_forward_sliced(plan.ka, plan.shape, plan.n_anchors,
                                                        plan.feat_dtype, s),
                              "forward kernel launch");
        }
    }
    return hip_status(da::launch_forward(plan.ka, plan.shape, plan.n_anchors, plan.feat_dtype, s),
                      "forward kernel launch");
}

da_status da_backward_workspace_size(const da_problem* p, size_t* bytes) {
    if (!bytes) return fail(DA_ERR_INVALID_ARG, "bytes is NULL");
    if (!p) return fail(DA_ERR_INVALID_ARG, "problem is NULL");
    if (p->bs < 0 || p->num_anchors < 0 || p->num_pts < 0 || p->num_feat < 1 ||
        p->num_cams < 1 || p->num_scale < 1)
        return fail(DA_ERR_INVALID_ARG, "malformed problem sizes");
    if (!valid_dtype(p->out_dtype))
        return fail(DA_ERR_INVALID_ARG, "out_dtype %d is not a da_dtype", (int)p->out_dtype);
    uint64_t n_rows = 0, n_samples = 0;
    const da_status st = gather_sizes(p, n_rows, n_samples);
    if (st != DA_OK) return st;
    const bool det = p->flags & DA_FLAG_DETERMINISTIC;
    *bytes = n_samples == 0
                 ? 0
                 : ws_layout(n_rows, n_samples, fused_capable(p) ? (uint64_t)p->num_groups : 0,
                             det ? det_bytes(p, n_samples) : 0, go32_bytes(p))
                       .total;
    return DA_OK;
}

da_status da_backward(const da_problem* p, const void* feat, const int32_t* shape,
                      const int32_t* start, const float* loc, const float* weights,
                      const void* grad_out, float* grad_feat, float* grad_loc,
                      float* grad_weights, void* workspace, size_t workspace_bytes, void* stream) {
    return backward_impl(BwdMode::kGather, p, feat, shape, start, loc, weights, grad_out,
                         grad_feat, grad_loc, grad_weights, workspace, workspace_bytes, stream);
}

da_status da_backward_accumulate(const da_problem* p, const void* feat, const int32_t* shape,
                                 const int32_t* start, const float* loc, const float* weights,
                                 const void* grad_out, float* grad_feat, float* grad_loc,
                                 float* grad_weights, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    return backward_impl(BwdMode::kGatherAccumulate, p, feat, shape, start, loc, weights,
                         grad_out, grad_feat, grad_loc, grad_weights, workspace, workspace_bytes,
                         stream);
}

da_status da_backward_atomic(const da_problem* p, const void* feat, const int32_t* shape,
                             const int32_t* start, const float* loc, const float* weights,
                             const void* grad_out, float* grad_feat, float* grad_loc,
                             float* grad_weights, void* stream) {
    return backward_impl(BwdMode::kScatter, p, feat, shape, start, loc, weights, grad_out,
                         grad_feat, grad_loc, grad_weights, nullptr, 0, stream);
}

}  // extern "C"

namespace da {

da_status backward_resolved(const da_problem* p, const void* feat, const int32_t* shape,
                            const int32_t* start, const float* loc, const float* weights,
                            const void* grad_out, float* grad_feat, float* grad_loc,
                            float* grad_weights, void* stream, WorkspaceResolver resolve_ws) {
    return backward_impl(BwdMode::kGather, p, feat, shape, start, loc, weights, grad_out,
                         grad_feat, grad_loc, grad_weights, nullptr, 0, stream, resolve_ws);
}

}  // namespace da

extern "C" {

const char* da_status_string(da_status s) {
    switch (s) {
        case DA_OK: return "DA_OK";
        case DA_ERR_INVALID_ARG: return "DA_ERR_INVALID_ARG: malformed argument";
        case DA_ERR_UNSUPPORTED: return "DA_ERR_UNSUPPORTED: outside what the kernels handle";
        case DA_ERR_HIP: return "DA_ERR_HIP: the HIP runtime refused the launch";
    }
    return "unknown da_status";
}

const char* da_last_error(void) { return g_last_error; }

int32_t da_version(void) { return DA_VERSION; }

}  // extern "C"
