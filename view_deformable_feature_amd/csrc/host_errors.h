// Host-side error reporting shared by the entry points of every operator in the
// library: the per-thread message behind da_last_error().  Not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>

#include "deformagg.h"

namespace da {

// Records the message (printf format) and returns st.
da_status report_error(da_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// DA_OK for hipSuccess, else DA_ERR_HIP with the runtime's message.
da_status report_hip(hipError_t e, const char* what);

// Supplies a backward workspace of at least `need` bytes (256-byte aligned) once
// every argument check of the call has passed; anything but DA_OK ends the call
// with nothing enqueued.
typedef da_status (*WorkspaceResolver)(size_t need, void** workspace, size_t* workspace_bytes);

// da_backward whose workspace comes from resolve_ws instead of the caller.
da_status backward_resolved(const da_problem* p, const void* feat, const int32_t* shape,
                            const int32_t* start, const float* loc, const float* weights,
                            const void* grad_out, float* grad_feat, float* grad_loc,
                            float* grad_weights, void* stream, WorkspaceResolver resolve_ws);

}  // namespace da
