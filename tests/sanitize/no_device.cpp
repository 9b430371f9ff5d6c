// Launchers for a host-only build of the C ABI (api.cpp, plan.cpp and
// block_manager.cpp without any kernel): every launch reports that there is
// no device.  Used to run the host-side suites under AddressSanitizer and
// UndefinedBehaviorSanitizer, which instrument host code only.
#include "launch.h"

namespace pa {
namespace {
pa_status none(std::string *why) {
    if (why) *why = "host-only build: no device";
    return PA_ERR_HIP;
}
}  // namespace

pa_status launch_append(const AppendArgs &, const AppendPlan &, void *, std::string *why) {
    return none(why);
}
pa_status launch_grouped_decode(const DecodeShape &, const DecodeArgs &, const DecodePlan &,
                                void *, std::string *why) {
    return none(why);
}
pa_status launch_gqa_mfma_decode(const DecodeShape &, const DecodeArgs &, const DecodePlan &,
                                 void *, std::string *why) {
    return none(why);
}
pa_status launch_append_mxfp8(const MxAppendArgs &, void *, std::string *why) { return none(why); }
pa_status launch_mxfp8_decode(const DecodeShape &, const DecodeArgs &, const DecodePlan &, void *,
                              std::string *why) {
    return none(why);
}
pa_status launch_copy_blocks(void *, int64_t, const int32_t *, const int32_t *, int32_t, void *,
                             std::string *why) {
    return none(why);
}
pa_status launch_attention_scores(float *, const void *, const void *, const int32_t *,
                                  const int32_t *, const float *, float, int32_t, int32_t,
                                  int32_t, int32_t, int32_t, int32_t, int32_t, int32_t, void *,
                                  std::string *why) {
    return none(why);
}
pa_status launch_latent_decode(const DecodeShape &, const DecodeArgs &, const DecodePlan &, void *,
                               std::string *why) {
    return none(why);
}
pa_status noalloc_scratch(void **, std::string *why) { return none(why); }
}  // namespace pa
