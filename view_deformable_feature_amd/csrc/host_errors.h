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

}  // namespace da
