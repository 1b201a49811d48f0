// Host-only stand-ins for the kernel launchers, so the planner and the C ABI's
// validation can be built with the host sanitizers (no device code). A launch
// reports hipErrorNotSupported; none is reached by the sanitizer driver.
#include <hip/hip_runtime.h>

#include "../../attention_bsr_paged_amd/csrc/kernels.h"

namespace abp {

hipError_t launch_decode(const Config&, const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }
bool decode_mfma_applies(const Config&) { return false; }
hipError_t launch_decode_mfma(const Config&, const AttnArgs&, hipStream_t) {
  return hipErrorNotSupported;
}
int decode_mfma_blocks_per_cu(const Config&) { return 1; }
int decode_blocks_per_cu(const Config&) { return 1; }
int append_blocks_per_cu(const Config&) { return 1; }
hipError_t launch_append(const Config&, const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }
bool pod_applies(const Config&) { return true; }
hipError_t launch_pod(const Config&, const AttnArgs&, const AttnArgs&, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_upload(void*, const void*, size_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_plan_merge(const Config&, const AttnArgs&, int32_t, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_cascade_merge(const AttnArgs&, const AttnArgs&, int32_t, void*, float*, int,
                                hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_page_append(const void*, const void*, const int32_t*, void*, void*,
                              const int32_t*, const int32_t*, const int32_t*, int32_t, int64_t,
                              int32_t, int32_t, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_merge_two(const void*, const float*, const void*, const float*, void*, float*,
                            int64_t, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_merge_states(const void*, const float*, int32_t, int64_t, int, int, void*,
                               float*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace abp
