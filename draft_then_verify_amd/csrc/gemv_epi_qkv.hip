// Instances of the weight-streaming / matrix-core linear for EPI_QKV.
#include "gemv_launch.hpp"

namespace sv {
hipError_t launch_gemv_qkv(bool bf16, const GemvArgs& a, int M, hipStream_t s) {
  return bf16 ? gemvl::launch_all<uint16_t, EPI_QKV>(a, M, s) : gemvl::launch_all<float, EPI_QKV>(a, M, s);
}
}  // namespace sv
