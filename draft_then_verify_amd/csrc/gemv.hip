// Dispatch of the linear by epilogue, and the K-slice choice of the residual
// linears.  The kernels and their launch shapes are in gemv_kernels.hpp,
// gemm_mfma.hpp and gemv_launch.hpp.
#include <algorithm>

#include "gemm_mfma.hpp"
#include "gemv_kernels.hpp"

namespace sv {

hipError_t launch_gemv_store(bool bf16, const GemvArgs& a, int M, hipStream_t s);
hipError_t launch_gemv_partial(bool bf16, const GemvArgs& a, int M, hipStream_t s);
hipError_t launch_gemv_resid(bool bf16, const GemvArgs& a, int M, hipStream_t s);
hipError_t launch_gemv_swiglu(bool bf16, const GemvArgs& a, int M, hipStream_t s);
hipError_t launch_gemv_qkv(bool bf16, const GemvArgs& a, int M, hipStream_t s);
hipError_t launch_gemv_lmstat(bool bf16, const GemvArgs& a, int M, hipStream_t s);

namespace {
constexpr int kCUs = 256;
using gemv::kMaxLds;
}  // namespace

int gemv_ksplit(bool bf16, int M, int N, int K) {
  if (bf16 && M > 8 && K % mfma::KB == 0) {
    // matrix-core path: enough workgroups (one per CU) from row blocks x
    // weight tiles x K slices; each slice more is a partial of rows x N
    // float32 that the residual-sum kernel reads back (two per CU: B = 256
    // verify step 1.131 -> 1.165 ms)
    const int tiles = ((M + mfma::BM - 1) / mfma::BM) * ((N + mfma::BN - 1) / mfma::BN);
    int best = 1;
    for (int ks = 1; ks <= 8; ++ks) {
      if (K % (ks * mfma::KB)) continue;
      best = ks;
      if (tiles * ks >= kCUs) break;
    }
    return best;
  }
  // weight-streaming path: one workgroup per CU stages its rows' slice of x
  // in LDS; split K only when a block of rows does not fit
  const int elt = bf16 ? 2 : 4;
  const int step = kWave * (16 / elt);
  const int mb = std::min(M, 8);
  for (int ks = 1; ks <= 8; ++ks) {
    if (K % (ks * step)) continue;
    if (static_cast<size_t>(mb) * (K / ks) * elt <= static_cast<size_t>(kMaxLds)) return ks;
  }
  return 1;
}

hipError_t launch_gemv(bool bf16, int epi, const GemvArgs& a, int M, hipStream_t s) {
  if (M <= 0 || a.N <= 0) return hipSuccess;
  switch (epi) {
    case EPI_STORE: return launch_gemv_store(bf16, a, M, s);
    case EPI_PARTIAL: return launch_gemv_partial(bf16, a, M, s);
    case EPI_RESID: return launch_gemv_resid(bf16, a, M, s);
    case EPI_SWIGLU: return launch_gemv_swiglu(bf16, a, M, s);
    case EPI_LMSTAT: return launch_gemv_lmstat(bf16, a, M, s);
    default: return launch_gemv_qkv(bf16, a, M, s);
  }
}

}  // namespace sv
