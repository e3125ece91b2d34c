#include "kda_common.h"
#include "kda_launch.h"
namespace kda {
size_t prefill_workspace_bytes(int32_t, int64_t, int32_t) { return 0; }
hipError_t launch_prefill(const PrefillParams&, const int32_t*, bool, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace kda
