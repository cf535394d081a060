// The LM head's statistics epilogue (EPI_LMSTAT): matrix cores, bf16 only.
#include "gemv_launch.hpp"

namespace sv {
hipError_t launch_gemv_lmstat(bool bf16, const GemvArgs& a, int M, hipStream_t s) {
  if (!bf16 || a.ksplit != 1 || a.K % mfma::KB || !a.tpart) return hipErrorInvalidValue;
  GemvArgs b = a;
  if (b.ldw == 0) b.ldw = b.K;
  if (b.ldx == 0) b.ldx = b.K;
  return gemvl::launch_gemm<EPI_LMSTAT>(b, M, s);
}
}  // namespace sv
