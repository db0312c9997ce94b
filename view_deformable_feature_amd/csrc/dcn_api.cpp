// Host side of the deformable convolution: argument checks, lane layout,
// dispatch.  Every check runs before anything is enqueued.  Contract:
// include/dcn.h.
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "da_internal.h"
#include "dcn.h"
#include "dcn_internal.h"
#include "host_errors.h"

namespace {

using da::report_error;

constexpr uint64_t kU32Max = 0xffffffffull;

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }
bool valid_dtype(int32_t t) { return t == DA_F32 || t == DA_BF16 || t == DA_F16; }
int elem_bytes(int32_t t) { return t == DA_F32 ? 4 : 2; }

int next_pow2(int64_t x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}
int log2i(int x) {
    int r = 0;
    while ((1 << (r + 1)) <= x) ++r;
    return r;
}

struct DcnPlan {
    da::DcnArgs a;
    int vec, nv;
    size_t lds_bytes;    // backward tile kernel
};

constexpr int kDcnMargin = 4;                 // offsets up to 4 px reach a tile through its ring
constexpr size_t kDcnTileLds = 48 * 1024;     // LDS for one tile's gradient sums

// Workspace: control words, then the far list (one 32-bit entry per (sample, corner)).
constexpr uint64_t kDcnFarOffset = 256;
uint64_t dcn_workspace_bytes(int64_t n_samples) {
    return n_samples == 0 ? 0 : kDcnFarOffset + (uint64_t)n_samples * 16;
}

// Sizes, types and the output extent; fills the size fields of a.
da_status check_problem(const dcn_problem* p, int64_t& ho, int64_t& wo) {
    if (!p) return report_error(DA_ERR_INVALID_ARG, "problem is NULL");
    if (p->flags != 0 || p->reserved != 0)
        return report_error(DA_ERR_INVALID_ARG, "problem.flags and problem.reserved must be 0");
    if (p->batch < 0) return report_error(DA_ERR_INVALID_ARG, "batch must be >= 0");
    if (p->height < 1 || p->width < 1 || p->channels < 1 || p->groups < 1)
        return report_error(DA_ERR_INVALID_ARG, "height, width, channels and groups must be >= 1");
    if (p->channels % p->groups != 0)
        return report_error(DA_ERR_INVALID_ARG, "channels (%lld) is not a multiple of groups (%lld)",
                            (long long)p->channels, (long long)p->groups);
    if (p->kernel_h < 1 || p->kernel_w < 1 || p->stride_h < 1 || p->stride_w < 1 ||
        p->dilation_h < 1 || p->dilation_w < 1 || p->pad_h < 0 || p->pad_w < 0)
        return report_error(DA_ERR_INVALID_ARG,
                            "kernel, stride and dilation must be >= 1 and padding >= 0");
    if (!valid_dtype(p->in_dtype) || !valid_dtype(p->out_dtype))
        return report_error(DA_ERR_INVALID_ARG, "in_dtype %d / out_dtype %d is not a da_dtype",
                            (int)p->in_dtype, (int)p->out_dtype);
    if (p->height > (1 << 20) || p->width > (1 << 20) || p->kernel_h * p->kernel_w > 1024 ||
        p->pad_h > (1 << 20) || p->pad_w > (1 << 20) || p->dilation_h > (1 << 20) ||
        p->dilation_w > (1 << 20) || p->stride_h > (1 << 20) || p->stride_w > (1 << 20))
        return report_error(DA_ERR_UNSUPPORTED,
                            "extent, padding, stride or dilation above 2^20, or more than 1024 taps");
    ho = (p->height + 2 * (int64_t)p->pad_h - (int64_t)p->dilation_h * (p->kernel_h - 1) - 1) /
             p->stride_h + 1;
    wo = (p->width + 2 * (int64_t)p->pad_w - (int64_t)p->dilation_w * (p->kernel_w - 1) - 1) /
             p->stride_w + 1;
    if (ho < 1 || wo < 1 ||
        p->height + 2 * (int64_t)p->pad_h < (int64_t)p->dilation_h * (p->kernel_h - 1) + 1 ||
        p->width + 2 * (int64_t)p->pad_w < (int64_t)p->dilation_w * (p->kernel_w - 1) + 1)
        return report_error(DA_ERR_INVALID_ARG, "the kernel does not fit the padded input");
    if (p->channels > (1 << 16))
        return report_error(DA_ERR_UNSUPPORTED, "channels > 2^16");
    return DA_OK;
}

// Everything but the tensor pointers; the lane layout.
da_status plan_dcn(const dcn_problem* p, const void* input, DcnPlan& plan) {
    int64_t ho = 0, wo = 0;
    da_status st = check_problem(p, ho, wo);
    if (st != DA_OK) return st;
    const int elem = elem_bytes(p->in_dtype);
    const uint64_t in_bytes = (uint64_t)p->batch * p->height * p->width * p->channels * elem;
    const uint64_t gi_bytes = (uint64_t)p->batch * p->height * p->width * p->channels * 4;
    if (gi_bytes + 64 > kU32Max || in_bytes + 64 > kU32Max)
        return report_error(DA_ERR_UNSUPPORTED,
                            "input (%llu bytes) or its binary32 gradient reaches 4 GiB",
                            (unsigned long long)in_bytes);
    const int64_t n_pix = p->batch * ho * wo;
    if (n_pix >= (int64_t(1) << 31)) return report_error(DA_ERR_UNSUPPORTED, "2^31 output pixels or more");
    // the kernels index out / grad_out (as binary32) and offset_mask with 32-bit offsets
    const uint64_t out_bytes = (uint64_t)n_pix * p->channels * 4;
    const uint64_t om_bytes = (uint64_t)n_pix * p->groups * 3 * p->kernel_h * p->kernel_w * 4;
    if (out_bytes + 64 > kU32Max || om_bytes + 64 > kU32Max)
        return report_error(DA_ERR_UNSUPPORTED,
                            "output (%llu bytes as binary32) or offset_mask (%llu bytes) reaches 4 GiB",
                            (unsigned long long)out_bytes, (unsigned long long)om_bytes);
    if (n_pix * p->groups * p->kernel_h * p->kernel_w >= (int64_t(1) << 30))
        return report_error(DA_ERR_UNSUPPORTED, "2^30 samples (pixel, group, tap) or more");
    const int64_t C = p->channels, G = p->groups, D = C / G;
    // 16 bytes of channels per lane where the groups and the pointer allow it
    const int wide = 16 / elem;
    const int vec = (D % wide == 0 && aligned(input, 16)) ? wide : 1;
    const int64_t dv = D / vec;
    if (dv > da::kWave)
        return report_error(DA_ERR_UNSUPPORTED, "channels per group (%lld) above %lld", (long long)D,
                            (long long)(da::kWave * vec));
    const int lg = next_pow2(dv);
    const int64_t lanes = G * lg;
    const int lp = lanes >= da::kWave ? da::kWave : next_pow2(lanes);
    const int nv = next_pow2((lanes + lp - 1) / lp);
    if (nv > 8)
        return report_error(DA_ERR_UNSUPPORTED, "groups x lanes per group (%lld) above 512",
                            (long long)lanes);
    da::DcnArgs& a = plan.a;
    memset(&a, 0, sizeof a);
    a.n_pix = n_pix;
    a.in_bytes = (uint32_t)in_bytes;
    a.gi_bytes = (uint32_t)gi_bytes;
    a.om_bytes = (uint32_t)om_bytes;
    a.N = (int32_t)p->batch;
    a.H = (int32_t)p->height;
    a.W = (int32_t)p->width;
    a.C = (int32_t)C;
    a.G = (int32_t)G;
    a.D = (int32_t)D;
    a.KH = p->kernel_h;
    a.KW = p->kernel_w;
    a.SH = p->stride_h;
    a.SW = p->stride_w;
    a.PH = p->pad_h;
    a.PW = p->pad_w;
    a.DH = p->dilation_h;
    a.DW = p->dilation_w;
    a.Ho = (int32_t)ho;
    a.Wo = (int32_t)wo;
    a.K = p->kernel_h * p->kernel_w;
    a.Dv = (int32_t)dv;
    a.Lg = lg;
    a.log2Lg = log2i(lg);
    a.Lp = lp;
    a.log2Lp = log2i(lp);
    a.out_dtype = p->out_dtype;
    a.go_dtype = p->out_dtype;
    // backward tiles: halve 32 x 32 (rows first) until the 64-bit sums fit the LDS
    // budget; the pixel stride D + 1 words keeps neighbouring pixels' channels in
    // different banks
    a.Dp = (int32_t)(D + 1);
    int ty = 32, tx = 32;
    while ((ty > 1 || tx > 1) && da::dcn_tile_lds_bytes(ty, tx, a.Dp) > kDcnTileLds) {
        if (ty >= tx && ty > 1) ty >>= 1;
        else tx >>= 1;
    }
    a.TY = ty;
    a.TX = tx;
    a.M = kDcnMargin;
    a.tiles_y = (int32_t)((p->height + ty - 1) / ty);
    a.tiles_x = (int32_t)((p->width + tx - 1) / tx);
    plan.lds_bytes = da::dcn_tile_lds_bytes(ty, tx, a.Dp);
    // at most every sample of one (image, group) plane adds to one tile sum
    a.log2_terms = std::max(10, log2i((int)std::min<int64_t>(ho * wo * a.K, 1 << 30)) + 1);
    // backward: up to 8 channels per lane, two vectors where the group has them
    // (fewer lanes repeat each sample's stencil; more channels per lane cost the
    // registers that keep six waves per SIMD)
    a.bNVL = (dv >= 2 && vec <= 4) ? 2 : 1;
    a.bLg = next_pow2((dv + a.bNVL - 1) / a.bNVL);
    a.blog2Lg = log2i(a.bLg);
    plan.vec = vec;
    plan.nv = nv;
    return DA_OK;
}

}  // namespace

extern "C" {

da_status dcn_out_size(const dcn_problem* p, int64_t* out_h, int64_t* out_w) {
    if (!out_h || !out_w) return report_error(DA_ERR_INVALID_ARG, "out_h / out_w is NULL");
    int64_t ho = 0, wo = 0;
    const da_status st = check_problem(p, ho, wo);
    if (st != DA_OK) return st;
    *out_h = ho;
    *out_w = wo;
    return DA_OK;
}

da_status dcn_forward(const dcn_problem* p, const void* input, const float* offset_mask, void* out,
                      void* stream) {
    DcnPlan plan;
    da_status st = plan_dcn(p, input, plan);
    if (st != DA_OK) return st;
    if (plan.a.n_pix == 0) return DA_OK;
    if (!input || !offset_mask || !out)
        return report_error(DA_ERR_INVALID_ARG, "input / offset_mask / out is NULL");
    if (!aligned(input, elem_bytes(p->in_dtype)) || !aligned(out, elem_bytes(p->out_dtype)) ||
        !aligned(offset_mask, 4))
        return report_error(DA_ERR_INVALID_ARG, "input / offset_mask / out is not element aligned");
    da::DcnArgs& a = plan.a;
    a.input = input;
    a.om = offset_mask;
    a.out = out;
    a.out_vec4 = plan.vec % 4 == 0 && aligned(out, 16);
    return da::report_hip(
        da::launch_dcn_forward(a, p->in_dtype, plan.vec, plan.nv, static_cast<hipStream_t>(stream)),
        "dcn forward launch");
}

da_status dcn_backward_workspace_size(const dcn_problem* p, size_t* bytes) {
    if (!bytes) return report_error(DA_ERR_INVALID_ARG, "bytes is NULL");
    int64_t ho = 0, wo = 0;
    const da_status st = check_problem(p, ho, wo);
    if (st != DA_OK) return st;
    *bytes = (size_t)dcn_workspace_bytes(p->batch * ho * wo * p->groups * p->kernel_h * p->kernel_w);
    return DA_OK;
}

da_status dcn_backward(const dcn_problem* p, const void* input, const float* offset_mask,
                       const void* grad_out, float* grad_input, float* grad_offset_mask,
                       void* workspace, size_t workspace_bytes, void* stream) {
    DcnPlan plan;
    da_status st = plan_dcn(p, input, plan);
    if (st != DA_OK) return st;
    if (p->batch > 0 && !grad_input) return report_error(DA_ERR_INVALID_ARG, "grad_input is NULL");
    if (plan.a.n_pix > 0 && (!input || !offset_mask || !grad_out || !grad_offset_mask))
        return report_error(DA_ERR_INVALID_ARG,
                            "input / offset_mask / grad_out / grad_offset_mask is NULL");
    if (!aligned(input, elem_bytes(p->in_dtype)) || !aligned(grad_out, elem_bytes(p->out_dtype)) ||
        !aligned(offset_mask, 4) || !aligned(grad_input, 4) || !aligned(grad_offset_mask, 4))
        return report_error(DA_ERR_INVALID_ARG, "a tensor is not element aligned");
    da::DcnArgs& a = plan.a;
    a.input = input;
    a.om = offset_mask;
    a.grad_out = grad_out;
    a.grad_input = grad_input;
    a.grad_om = grad_offset_mask;
    a.go_vec4 = plan.vec % 4 == 0 && aligned(grad_out, 16);
    if (p->batch == 0) return DA_OK;
    const uint64_t need = dcn_workspace_bytes(a.n_pix * a.G * a.K);
    if (need) {
        if (!workspace) return report_error(DA_ERR_INVALID_ARG, "workspace is NULL");
        if (!aligned(workspace, 256))
            return report_error(DA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
        if (workspace_bytes < need)
            return report_error(DA_ERR_INVALID_ARG, "workspace has %zu bytes, %llu needed",
                                workspace_bytes, (unsigned long long)need);
        unsigned char* base = static_cast<unsigned char*>(workspace);
        a.ctrl = reinterpret_cast<uint32_t*>(base);
        a.fb = reinterpret_cast<uint32_t*>(base + kDcnFarOffset);
    }
    return da::report_hip(da::launch_dcn_backward(a, p->in_dtype, plan.vec, plan.lds_bytes,
                                                  static_cast<hipStream_t>(stream)),
                          "dcn backward launch");
}

}  // extern "C"
