#include "kda_common.h"
#include "kda_launch.h"
namespace kda {
hipError_t launch_verify(const VerifyParams&, bool, hipStream_t) { return hipErrorNotSupported; }
}  // namespace kda
