// Large-query-block (prefill) kernel: not built yet.
#include "ua_device.h"

namespace ua {
hipError_t launch_large(const Params&, int, int, int, bool, dim3, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace ua
