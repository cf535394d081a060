// Host dispatch of the weight-streaming linear (kernel in gemv_kernels.hpp).
//
// A persistent grid of a few workgroups per CU; each wave walks a strided
// list of R-row tiles.  Launch shapes per epilogue were chosen by timing the
// 8B-shaped matrices on MI355X with M = 5 (rows per tile R, ring depth U,
// minimum waves per SIMD, workgroups per CU):
//   gate/up (SwiGLU)  R=1 U=4, 4 waves/SIMD, 3 workgroups/CU  -> 5.5 TB/s
//   LM head / store   R=4 U=4, 2 waves/SIMD, 1 workgroup/CU   -> 6.6 TB/s
//   residual (O, down) R=2 U=8, 3 waves/SIMD
//   QKV (RoPE pairs)  R=4 U=4, 2 waves/SIMD
// U is lowered to the largest of 8, 4, 2, 1 that divides the steps per row.
// Activation rows go through in blocks of at most 8 that fit the LDS.
#include <algorithm>

#include "gemv_kernels.hpp"

namespace sv {
namespace {

using gemv::kMaxLds;
using gemv::kThreads;
using gemv::kWavesPerBlock;

constexpr int kCUs = 256;

template <int EPI> struct Cfg;
template <> struct Cfg<EPI_SWIGLU> { static constexpr int R = 1, U = 4, WPE = 4, BPC = 3; };
template <> struct Cfg<EPI_STORE> { static constexpr int R = 4, U = 4, WPE = 2, BPC = 1; };
template <> struct Cfg<EPI_RESID> { static constexpr int R = 2, U = 8, WPE = 3, BPC = 2; };
template <> struct Cfg<EPI_QKV> { static constexpr int R = 4, U = 4, WPE = 2, BPC = 2; };

template <typename WT, int M, int U, int EPI>
hipError_t launch_mu(const GemvArgs& a, hipStream_t s) {
  constexpr int R = Cfg<EPI>::R;
  auto kern = gemv::gemv_kernel<WT, M, R, U, EPI, Cfg<EPI>::WPE>;
  static bool lds_opt_in = false;
  if (!lds_opt_in) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    if (e != hipSuccess) return e;
    lds_opt_in = true;
  }
  constexpr int STEP = kWave * (16 / static_cast<int>(sizeof(WT)));
  const size_t kp = static_cast<size_t>((a.K + STEP - 1) / STEP) * STEP;
  const size_t lds = static_cast<size_t>(M) * kp * sizeof(WT);
  const int tiles = gemv::num_tiles<EPI, R>(a.N);
  const int per_cu = std::max(1, std::min(Cfg<EPI>::BPC, static_cast<int>(kMaxLds / std::max<size_t>(lds, 1))));
  const int blocks = std::min((tiles + kWavesPerBlock - 1) / kWavesPerBlock, kCUs * per_cu);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <typename WT, int M, int EPI>
hipError_t launch_m(const GemvArgs& a, hipStream_t s) {
  constexpr int STEP = kWave * (16 / static_cast<int>(sizeof(WT)));
  // (residual with 7-8 rows: ring depth 4 keeps the 168-register budget)
  constexpr int U0 = (EPI == EPI_RESID && M > 6) ? 4 : Cfg<EPI>::U;
  const int S = (a.K + STEP - 1) / STEP;
  if (U0 >= 8 && S % 8 == 0) return launch_mu<WT, M, (U0 >= 8 ? 8 : U0), EPI>(a, s);
  if (S % 4 == 0) return launch_mu<WT, M, 4, EPI>(a, s);
  if (S % 2 == 0) return launch_mu<WT, M, 2, EPI>(a, s);
  return launch_mu<WT, M, 1, EPI>(a, s);
}

template <typename WT, int EPI>
hipError_t launch_rows(const GemvArgs& a, int mb, hipStream_t s) {
  switch (mb) {
    case 1: return launch_m<WT, 1, EPI>(a, s);
    case 2: return launch_m<WT, 2, EPI>(a, s);
    case 3: return launch_m<WT, 3, EPI>(a, s);
    case 4: return launch_m<WT, 4, EPI>(a, s);
    case 5: return launch_m<WT, 5, EPI>(a, s);
    case 6: return launch_m<WT, 6, EPI>(a, s);
    case 7: return launch_m<WT, 7, EPI>(a, s);
    default: return launch_m<WT, 8, EPI>(a, s);
  }
}

template <typename WT, int EPI>
hipError_t launch_all(const GemvArgs& a0, int M, hipStream_t s) {
  constexpr int STEP = kWave * (16 / static_cast<int>(sizeof(WT)));
  const size_t kp = static_cast<size_t>((a0.K + STEP - 1) / STEP) * STEP;
  const int fit = static_cast<int>(kMaxLds / (kp * sizeof(WT)));
  if (fit < 1) return hipErrorInvalidValue;
  const int blk = std::min(8, fit);
  for (int m0 = 0; m0 < M; m0 += blk) {
    GemvArgs a = a0;
    const int mb = std::min(blk, M - m0);
    a.M = mb;
    a.row0 = a0.row0 + m0;
    a.x = static_cast<const WT*>(a0.x) + static_cast<size_t>(m0) * a.K;
    if (a.y) a.y = a0.y + static_cast<size_t>(m0) * a.ldy;
    if (a.z) a.z = static_cast<WT*>(a0.z) + static_cast<size_t>(m0) * a.ldz;
    if (a.norm_out) a.norm_out = static_cast<WT*>(a0.norm_out) + static_cast<size_t>(m0) * a.N;
    hipError_t e = launch_rows<WT, EPI>(a, mb, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename WT>
hipError_t launch_dtype(int epi, const GemvArgs& a, int M, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return launch_all<WT, EPI_STORE>(a, M, s);
    case EPI_RESID: return launch_all<WT, EPI_RESID>(a, M, s);
    case EPI_SWIGLU: return launch_all<WT, EPI_SWIGLU>(a, M, s);
    default: return launch_all<WT, EPI_QKV>(a, M, s);
  }
}

}  // namespace

hipError_t launch_gemv(bool bf16, int epi, const GemvArgs& a, int M, hipStream_t s) {
  if (M <= 0 || a.N <= 0) return hipSuccess;
  return bf16 ? launch_dtype<uint16_t>(epi, a, M, s) : launch_dtype<float>(epi, a, M, s);
}

}  // namespace sv
