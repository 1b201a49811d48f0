// Append / prefill attention (MFMA): not built yet in this revision.
#include "common.h"
#include "kernels.h"

namespace abp {

hipError_t launch_append(const Config&, const AttnArgs&, hipStream_t) {
  return hipErrorNotSupported;
}

int append_blocks_per_cu(const Config&) { return 1; }

}  // namespace abp
