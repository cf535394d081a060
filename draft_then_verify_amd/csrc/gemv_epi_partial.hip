// Instances of the weight-streaming / matrix-core linear for EPI_PARTIAL.
#include "gemv_launch.hpp"

namespace sv {
hipError_t launch_gemv_partial(bool bf16, const GemvArgs& a, int M, hipStream_t s) {
  return bf16 ? gemvl::launch_all<uint16_t, EPI_PARTIAL>(a, M, s) : gemvl::launch_all<float, EPI_PARTIAL>(a, M, s);
}
}  // namespace sv
