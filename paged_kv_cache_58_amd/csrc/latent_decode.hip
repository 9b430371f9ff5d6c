// Latent-mode (576-wide shared latent, 512-wide value view) paged decode.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace pa {

pa_status launch_latent_decode(const DecodeShape &, const DecodeArgs &, const DecodePlan &,
                               hipStream_t, std::string *why) {
    if (why) *why = "decode (latent): not built yet";
    return PA_ERR_UNSUPPORTED;
}

}  // namespace pa
