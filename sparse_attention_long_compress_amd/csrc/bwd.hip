// bwd.hip -- selection-branch backward (placeholder launchers; kernels follow).
#include "nsa_device.h"
#include "nsa_launch.h"

namespace nsa {
hipError_t launch_bwd_prep(bool, const Shape&, const void*, const void*, const void*, const void*,
                           void*, float*, void*, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_revmap(const Shape&, const int32_t*, uint64_t*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_bwd_dq(bool, const Shape&, const void*, const void*, const void*, const void*,
                         const int32_t*, const float*, const float*, const void*, void*,
                         hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_dkdv(bool, const Shape&, const void*, const void*, const void*, const float*,
                           const float*, const void*, const uint64_t*, void*, void*, float*,
                           hipStream_t) { return hipErrorNotSupported; }
}  // namespace nsa
