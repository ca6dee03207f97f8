// Kernel launchers for a host-only build of the C ABI (api.cpp + plan.cpp) under the address and
// undefined-behaviour sanitizers.  Every launcher reports a device failure: such a build checks
// arguments, plans workspaces and maps errors, and can never compute anything.
#include "../../cross_layer_token_amd/csrc/clsa_internal.h"

namespace clsa {

namespace {
constexpr int kNoDevice = 100;  // hipErrorNoDevice
}

int launch_index_scores_decode(const RowsDev&, int, int, const uint16_t*, int64_t, const uint16_t*, float*, int64_t,
                               uint16_t*, uint32_t*, int, int, uint32_t*, int, void*) {
  return kNoDevice;
}
int launch_index_scores_prefill(const RowsDev&, int, const uint16_t*, const uint16_t*, float*, int64_t, uint32_t*, int,
                                void*) {
  return kNoDevice;
}
int launch_topk(const RowsDev&, int, const TopkPlan&, const float*, int64_t, int32_t*, int32_t*, void*, bool, void*,
                bool) {
  return kNoDevice;
}
int launch_gather(const RowsDev&, int, int, const uint16_t*, const uint16_t*, const int32_t*, const int32_t*,
                  uint16_t*, uint16_t*, void*) {
  return kNoDevice;
}
int launch_attn(const RowsDev&, int, int, int, int, float, const AttnPlan&, const uint16_t*, int64_t, const uint16_t*,
                const uint16_t*, const uint16_t*, const uint16_t*, const int32_t*, const int32_t*, uint16_t*, int64_t,
                void*, uint32_t*, bool, void*, const SelectIn*, int32_t*, int32_t*) {
  return kNoDevice;
}
int launch_index_project(int, int, int, int, int64_t, const uint16_t*, const uint16_t*, const uint16_t*,
                         const int32_t*, uint16_t*, uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, uint16_t*,
                         void*) {
  return kNoDevice;
}
int launch_distill(const RowsDev&, int64_t, int, int, int, float, const uint16_t*, int64_t, const uint16_t*,
                   const float*, int64_t, float*, float*, void*, const DistillPlan&, void*) {
  return kNoDevice;
}
const char* device_error_string(int) { return "no device (host-only sanitizer build)"; }
int no_alloc_scratch(void** ptr, std::string& err) {
  *ptr = nullptr;
  err = "no device (host-only sanitizer build)";
  return kNoDevice;
}

}  // namespace clsa
