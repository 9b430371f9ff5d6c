// HIP error to library status, for the kernel files' launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <string>

#include "pa.h"

namespace pa {

inline pa_status hip_status(hipError_t e, std::string *why, const char *where) {
    if (e == hipSuccess) return PA_OK;
    if (why) *why = std::string(where) + ": " + hipGetErrorString(e);
    return PA_ERR_HIP;
}

}  // namespace pa
