// Instances of the weight-streaming / matrix-core linear for EPI_STORE.
#include "gemv_launch.hpp"

namespace sv {
hipError_t launch_gemv_store(bool bf16, const GemvArgs& a, int M, hipStream_t s) {
  return bf16 ? gemvl::launch_all<uint16_t, EPI_STORE>(a, M, s) : gemvl::launch_all<float, EPI_STORE>(a, M, s);
}
}  // namespace sv
