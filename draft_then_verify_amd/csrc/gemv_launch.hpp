// Host dispatch templates of the weight-streaming linear (kernel in
// gemv_kernels.hpp); each epilogue is instantiated in its own source file
// (gemv_epi_*.hip) so the instances compile in parallel.
//
// A persistent grid of a few workgroups per CU (times the K slices); each
// wave walks a strided list of R-row tiles.  Launch shapes per epilogue
// (rows per tile R, ring depth U, minimum waves per SIMD, workgroups per CU,
// threads per workgroup) were chosen by timing the 8B-shaped matrices on
// MI355X with M = 5, 36 distinct matrices per replayed graph so the weights
// come from HBM.  Wide workgroups, one per CU, stage the activations once per
// CU: with 3 narrow workgroups per CU the 40 KB of staged rows per workgroup
// came to as many bytes as the QKV and O weights themselves.  A launch whose
// wide workgroups would occupy fewer than half the CUs (the drafter-sized O
// and down) uses 256-thread workgroups instead.  U is lowered to
// the largest of 8, 4, 2, 1 that divides the steps per row.  Activation rows
// go through in blocks of at most 8 that fit the LDS.  bf16 passes with more than 8 rows go to the matrix-core
// kernel (gemm_mfma.hpp), which reads the weights once per 64 rows.
#pragma once

#include <algorithm>
#include <type_traits>

#include "gemm_mfma.hpp"
#include "gemv_kernels.hpp"

namespace sv {
namespace gemvl {

using gemv::kMaxLds;

constexpr int kCUs = 256;

template <int EPI> struct Cfg;
template <> struct Cfg<EPI_SWIGLU> { static constexpr int R = 1, U = 4, WPE = 4, BPC = 1, NT = 1024; };
template <> struct Cfg<EPI_STORE> { static constexpr int R = 4, U = 4, WPE = 2, BPC = 1, NT = 256; };
template <> struct Cfg<EPI_PARTIAL> { static constexpr int R = 1, U = 4, WPE = 4, BPC = 1, NT = 1024; };
template <> struct Cfg<EPI_RESID> { static constexpr int R = 1, U = 4, WPE = 4, BPC = 1, NT = 1024; };
template <> struct Cfg<EPI_QKV> { static constexpr int R = 2, U = 4, WPE = 4, BPC = 1, NT = 768; };

template <typename WT> constexpr int step_elems() { return kWave * (16 / static_cast<int>(sizeof(WT))); }

template <typename WT, int M, int U, int EPI, int NT, int WPE>
hipError_t launch_mu_nt(const GemvArgs& a, hipStream_t s) {
  using C = Cfg<EPI>;
  auto kern = gemv::gemv_kernel<WT, M, C::R, U, EPI, WPE, NT>;
  static bool lds_opt_in = false;
  if (!lds_opt_in) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    if (e != hipSuccess) return e;
    lds_opt_in = true;
  }
  constexpr int STEP = step_elems<WT>();
  const size_t kp = static_cast<size_t>((a.K + STEP - 1) / STEP) * STEP;
  const size_t lds = static_cast<size_t>(M) * kp * sizeof(WT);
  const int tiles = gemv::num_tiles<EPI, C::R>(a.N);
  const int per_cu = std::max(1, std::min(C::BPC, static_cast<int>(kMaxLds / std::max<size_t>(lds, 1))));
  const int wpb = NT / kWave;
  const int bx = std::max(1, std::min((tiles + wpb - 1) / wpb, kCUs * per_cu / a.ksplit));
  hipLaunchKernelGGL(kern, dim3(bx, a.ksplit), dim3(NT), lds, s, a);
  return hipGetLastError();
}

// Wide workgroups unless they would occupy fewer than half the CUs: then
// 256-thread workgroups, so that the stream spreads over the chip.  (The
// 0.6B-shaped drafter, one row: O and down, 64 wide workgroups, 4.46 -> 4.19
// and 5.80 -> 4.97 us narrow; QKV and gate/up, 171 and 192 wide workgroups,
// were faster wide: 6.15 and 6.19 against 6.48 and 6.53 us.)
//
// QKV and gate/up also have a middle shape (512 and 768 threads) for a wide
// grid between half and all the CUs, taken when it gives every CU a
// workgroup (the drafter's QKV: 171 wide workgroups -> 256 of 512 threads;
// its gate/up: 192 -> 256 of 768 threads).
template <typename WT, int M, int U, int EPI>
hipError_t launch_mu(const GemvArgs& a, hipStream_t s) {
  using C = Cfg<EPI>;
  if constexpr (C::NT > 256) {
    const int tiles = gemv::num_tiles<EPI, C::R>(a.N);
    const int wide = (tiles + C::NT / kWave - 1) / (C::NT / kWave);
    // the narrower shapes run one workgroup per CU: their register budget is
    // that of NT / 256 waves per SIMD
    if (wide * a.ksplit < kCUs / 2) return launch_mu_nt<WT, M, U, EPI, 256, 2>(a, s);
    if constexpr (EPI == EPI_QKV || EPI == EPI_SWIGLU) {
      constexpr int MID = EPI == EPI_QKV ? 512 : 768;
      const int mid = (tiles + MID / kWave - 1) / (MID / kWave);
      if (wide * a.ksplit < kCUs && mid * a.ksplit >= kCUs) return launch_mu_nt<WT, M, U, EPI, MID, MID / 256>(a, s);
    }
  }
  return launch_mu_nt<WT, M, U, EPI, C::NT, C::WPE>(a, s);
}

template <typename WT, int M, int EPI>
hipError_t launch_m(const GemvArgs& a, hipStream_t s) {
  constexpr int STEP = step_elems<WT>();
  constexpr int U0 = Cfg<EPI>::U;
  const int S = (a.K + STEP - 1) / STEP;
  // residual linears of 6 steps per row (the 0.6B-shaped drafter's down
  // linear, K = 3072): the whole row in flight, not 2 steps of it
  if constexpr (EPI == EPI_RESID) {
    if (S == 6) return launch_mu<WT, M, 6, EPI>(a, s);
  }
  if (U0 >= 8 && S % 8 == 0) return launch_mu<WT, M, (U0 >= 8 ? 8 : U0), EPI>(a, s);
  if (U0 >= 4 && S % 4 == 0) return launch_mu<WT, M, (U0 >= 4 ? 4 : U0), EPI>(a, s);
  if (U0 >= 2 && S % 2 == 0) return launch_mu<WT, M, (U0 >= 2 ? 2 : U0), EPI>(a, s);
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

template <int EPI, int BMT, int BNT>
hipError_t launch_gemm_t(const GemvArgs& a, hipStream_t s) {
  const int mt = (a.M + BMT - 1) / BMT, nt = mfma::n_tiles<EPI, BNT>(a);
  const int total = mt * nt;
  const int grid = (total + mfma::kXcds - 1) / mfma::kXcds * mfma::kXcds;
  if constexpr (BNT == 256) {
    hipLaunchKernelGGL((mfma::gemm_kernel2<EPI, BMT, BNT, mfma::kDmaStages256, mfma::kDmaKB256>), dim3(grid, a.ksplit),
                       dim3(2 * BNT), 0, s, a, mt, nt);
  } else if constexpr (mfma::kDmaStages > 0) {
    constexpr int NS = BMT == 128 ? mfma::kDmaStages : mfma::kDmaStages64;
    constexpr int KBD = BMT == 128 ? mfma::kDmaKB : mfma::kDmaKB64;
    hipLaunchKernelGGL((mfma::gemm_kernel2<EPI, BMT, BNT, NS, KBD>), dim3(grid, a.ksplit), dim3(2 * BNT), 0, s, a, mt,
                       nt);
  } else {
    hipLaunchKernelGGL((mfma::gemm_kernel<EPI, BMT>), dim3(grid, a.ksplit), dim3(mfma::NTH), 0, s, a, mt, nt);
  }
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_gemm(const GemvArgs& b, int M, hipStream_t s) {
  GemvArgs a = b;
  a.M = M;
  // The largest tile that still gives every CU a workgroup (K slices count):
  // 256 x 256 (one workgroup of 8 waves per CU), else 128 x 128 (two of 4
  // waves), else 64 x 128.  The LM head's statistics epilogue (exp of every
  // logit, cross-wave merges) keeps 128 x 128: with one workgroup per CU
  // nothing overlaps it.
  if constexpr (EPI != EPI_QKV && EPI != EPI_LMSTAT) {
    if constexpr (mfma::kDmaStages256 > 0) {
      const long long tiles256 = static_cast<long long>((M + 255) / 256) * mfma::n_tiles<EPI, 256>(a) * a.ksplit;
      if (tiles256 >= kCUs) return launch_gemm_t<EPI, 256, 256>(a, s);
    }
  }
  const long long tiles128 = static_cast<long long>((M + 127) / 128) * mfma::n_tiles<EPI>(a) * a.ksplit;
  if (tiles128 >= kCUs) return launch_gemm_t<EPI, 128, 128>(a, s);
  return launch_gemm_t<EPI, 64, 128>(a, s);
}

template <typename WT, int EPI>
hipError_t launch_all(const GemvArgs& a0, int M, hipStream_t s) {
  constexpr int STEP = step_elems<WT>();
  constexpr int VE = 16 / static_cast<int>(sizeof(WT));
  GemvArgs b = a0;
  if (b.ksplit < 1 || b.K % b.ksplit) return hipErrorInvalidValue;
  if (b.ldw == 0) b.ldw = b.K;
  if (b.ldx == 0) b.ldx = b.K;
  if (b.ksplit > 1 && (EPI != EPI_PARTIAL || b.ysplit == 0)) return hipErrorInvalidValue;
  b.K /= b.ksplit;  // the kernel sees one slice
  if (b.K % VE || b.ldw % VE || b.ldx % VE) return hipErrorInvalidValue;
  if (EPI == EPI_QKV && (b.N % 2 || b.hd % 2)) return hipErrorInvalidValue;
  // the normalising prologue reads whole residual rows: one K slice, GEMV path
  if (b.hn && (b.ksplit != 1 || M > 8 || b.K % 4)) return hipErrorInvalidValue;
  // x merged from attention partials: one row, one K slice, whole heads of VE-element chunks
  if (b.apo && (M != 1 || b.ksplit != 1 || b.hn || b.mfma || !b.apml || b.asplit < 1 ||
                b.asplit > kMaxAttnSplits || b.ahd <= 0 || b.ahd % VE || b.aH * b.ahd != b.K))
    return hipErrorInvalidValue;
  if (std::is_same<WT, uint16_t>::value && (M > 8 || b.mfma) && b.K % mfma::KB == 0 &&
      (EPI != EPI_QKV || b.hd == 128 || b.hd == 64))
    return launch_gemm<EPI>(b, M, s);
  if (b.mfma) return hipErrorInvalidValue;
  const size_t kp = static_cast<size_t>((b.K + STEP - 1) / STEP) * STEP;
  const int fit = static_cast<int>(kMaxLds / (kp * sizeof(WT)));
  if (fit < 1) return hipErrorInvalidValue;
  const int blk = std::min(8, fit);
  for (int m0 = 0; m0 < M; m0 += blk) {
    GemvArgs a = b;
    const int mb = std::min(blk, M - m0);
    a.M = mb;
    a.row0 = b.row0 + m0;
    if (b.x) a.x = static_cast<const WT*>(b.x) + static_cast<size_t>(m0) * b.ldx;
    if (b.hn) a.hn = b.hn + static_cast<size_t>(m0) * b.K;
    if (a.y) a.y = b.y + static_cast<size_t>(m0) * b.ldy;
    if (a.z) a.z = static_cast<WT*>(b.z) + static_cast<size_t>(m0) * b.ldz;
    hipError_t e = launch_rows<WT, EPI>(a, mb, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gemvl
}  // namespace sv
