// da_backward_noalloc: the backward pass for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  It is da_backward with the caller's workspace replaced by
// a file-scope device array of fixed size, so the call allocates nothing.
//
// The array lives in the library's code object: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host code
// the name `scratch` denotes a host-side stand-in, not device memory, so the
// device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is ever passed to kernels.
//
// Every call on one GPU shares that GPU's array and leaves its contents behind;
// the backward clears what must start at zero (its control words and row
// counts) in its own first kernel, so stale contents do not matter.  Calls
// that overlap in time on one GPU (different streams, different threads)
// race on the array and must be serialised by the caller.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "deformagg.h"
#include "host_errors.h"

namespace {

static_assert(DA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[DA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch` (looked up on the
// first call on each device).
da_status scratch_for_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return da::report_hip(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return da::report_error(DA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev,
                                kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return da::report_hip(e, "hipGetSymbolAddress(scratch)");
        if (!p || reinterpret_cast<uintptr_t>(p) % 256 != 0)
            return da::report_error(DA_ERR_HIP, "scratch array has no 256-byte aligned address");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return DA_OK;
}

// Called by the backward once every argument check has passed.
da_status resolve_scratch(size_t need, void** workspace, size_t* workspace_bytes) {
    if (need > (size_t)DA_NOALLOC_SCRATCH_BYTES)
        return da::report_error(DA_ERR_UNSUPPORTED,
                                "da_backward_noalloc: this problem needs %zu bytes of scratch, "
                                "the library's static array holds %llu (use da_backward with a "
                                "workspace)",
                                need, (unsigned long long)DA_NOALLOC_SCRATCH_BYTES);
    const da_status st = scratch_for_current_device(workspace);
    if (st != DA_OK) return st;
    *workspace_bytes = (size_t)DA_NOALLOC_SCRATCH_BYTES;
    return DA_OK;
}

}  // namespace

extern "C" {

da_status da_backward_noalloc(const da_problem* p, const void* feat, const int32_t* shape,
                              const int32_t* start, const float* loc, const float* weights,
                              const void* grad_out, float* grad_feat, float* grad_loc,
                              float* grad_weights, void* stream) {
    return da::backward_resolved(p, feat, shape, start, loc, weights, grad_out, grad_feat,
                                 grad_loc, grad_weights, stream, resolve_scratch);
}

}  // extern "C"
