// Weight-streaming GEMV for the verify pass: y[M][N] = x[M][K] . W[N][K]^T
// with M <= 8 rows per launch.
//
// The pass is bound by reading the weights: a decode/verify pass "reads the
// entire ... weight set and then does about two floating-point operations per
// weight" (first page, section "The speedup is borrowed"), and checking five
// positions instead of one "reads the same weights" (same section).  So every
// weight byte is loaded exactly once per launch and used for all M rows:
//
//  * A wave owns R output columns (2R weight rows for SwiGLU: gate and up).
//    Its 64 lanes cover 64 x 16 B = 1 KiB of one weight row per step, so each
//    load instruction is a fully used, contiguous 1 KiB; U steps are issued
//    before any is consumed, keeping U*R 16-byte loads in flight per lane.
//  * The M activation rows (bf16 under the precision contract, or float32)
//    are staged in LDS once per workgroup and read back 16 B per lane.
//  * bf16: v_dot2_f32_bf16 multiplies two bf16 pairs and accumulates in
//    float32 without converting the weights; float32 models use fma.
//  * Each lane keeps R*M partial sums over its slice of K; one butterfly
//    reduction per (column, row) at the end.  The epilogue stores, adds into
//    the float32 residual stream, or applies silu(g) * u.
#include "common.hpp"
#include "kernels.hpp"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kLdsBytes = 64 * 1024;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Weights are read once: non-temporal loads keep them from displacing the
// activations and KV rows in the caches.
__device__ __forceinline__ uint4 load_stream(const void* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <typename WT> struct Dot;
template <> struct Dot<uint16_t> {  // 8 bf16 x 8 bf16, float32 accumulate
  __device__ __forceinline__ static float run(const uint4& w, const uint4& x, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), __builtin_bit_cast(bf16x2_t, x.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), __builtin_bit_cast(bf16x2_t, x.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), __builtin_bit_cast(bf16x2_t, x.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), __builtin_bit_cast(bf16x2_t, x.w), acc, false);
    return acc;
  }
};
template <> struct Dot<float> {  // 4 float32 x 4 float32
  __device__ __forceinline__ static float run(const uint4& w, const uint4& x, float acc) {
    acc = fmaf(__uint_as_float(w.x), __uint_as_float(x.x), acc);
    acc = fmaf(__uint_as_float(w.y), __uint_as_float(x.y), acc);
    acc = fmaf(__uint_as_float(w.z), __uint_as_float(x.z), acc);
    acc = fmaf(__uint_as_float(w.w), __uint_as_float(x.w), acc);
    return acc;
  }
};

template <typename WT, int M, int R, int U, int EPI>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const WT* __restrict__ W, const WT* __restrict__ X,
                                                        int N, int K, int KC, float* __restrict__ Y, int ldy,
                                                        WT* __restrict__ Z, int ldz) {
  extern __shared__ uint4 smem_v[];
  WT* xs = reinterpret_cast<WT*>(smem_v);
  constexpr int VE = 16 / sizeof(WT);
  constexpr int STEP = kWave * VE;
  constexpr int NW = (EPI == EPI_SWIGLU) ? 2 * R : R;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col0 = (blockIdx.x * kWavesPerBlock + wave) * R;
  const bool active = col0 < N;

  const WT* wp[NW];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = min(col0 + r, N - 1);
    wp[r] = W + static_cast<size_t>(c) * K;
    if constexpr (EPI == EPI_SWIGLU) wp[R + r] = W + static_cast<size_t>(c + N) * K;
  }
  float acc[NW][M];
#pragma unroll
  for (int r = 0; r < NW; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.f;

  for (int kc = 0; kc < K; kc += KC) {
    const int len = min(KC, K - kc);
    const int vpr = len / VE;
    __syncthreads();
    for (int idx = threadIdx.x; idx < M * vpr; idx += kThreads) {
      const int m = idx / vpr, v = idx - m * vpr;
      reinterpret_cast<uint4*>(xs + m * KC)[v] =
          *reinterpret_cast<const uint4*>(X + static_cast<size_t>(m) * K + kc + v * VE);
    }
    __syncthreads();
    if (active) {
      for (int k0 = lane * VE; k0 < len; k0 += STEP * U) {
        uint4 wv[U][NW];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int k = k0 + u * STEP;
#pragma unroll
          for (int r = 0; r < NW; ++r) wv[u][r] = (k < len) ? load_stream(wp[r] + kc + k) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int k = k0 + u * STEP;
          if (k < len) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
              const uint4 xv = *reinterpret_cast<const uint4*>(xs + m * KC + k);
#pragma unroll
              for (int r = 0; r < NW; ++r) acc[r][m] = Dot<WT>::run(wv[u][r], xv, acc[r][m]);
            }
          }
        }
      }
    }
  }
  if (!active) return;
#pragma unroll
  for (int r = 0; r < NW; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = wave_sum(acc[r][m]);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = col0 + r;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if (lane == r * M + m && c < N) {
        if constexpr (EPI == EPI_STORE) {
          Y[static_cast<size_t>(m) * ldy + c] = acc[r][m];
        } else if constexpr (EPI == EPI_RESID) {
          Y[static_cast<size_t>(m) * ldy + c] += acc[r][m];
        } else {
          const float g = acc[r][m], u = acc[R + r][m];
          Z[static_cast<size_t>(m) * ldz + c] = Elt<WT>::from_f(g / (1.f + expf(-g)) * u);
        }
      }
    }
  }
}

template <typename WT, int M, int EPI>
hipError_t launch_m(const WT* W, const WT* X, int N, int K, float* Y, int ldy, WT* Z, int ldz, hipStream_t s) {
  constexpr int VE = 16 / sizeof(WT);
  constexpr int STEP = kWave * VE;
  constexpr int R = (EPI == EPI_SWIGLU) ? 2 : 4;
  constexpr int U = 4;
  int KC = kLdsBytes / (M * static_cast<int>(sizeof(WT)));
  KC = (KC / STEP) * STEP;
  if (KC >= K) KC = K;
  const size_t lds = static_cast<size_t>(M) * KC * sizeof(WT);
  const int blocks = (N + kWavesPerBlock * R - 1) / (kWavesPerBlock * R);
  hipLaunchKernelGGL((gemv_kernel<WT, M, R, U, EPI>), dim3(blocks), dim3(kThreads), lds, s, W, X, N, K, KC, Y, ldy,
                     Z, ldz);
  return hipGetLastError();
}

template <typename WT, int EPI>
hipError_t launch_typed(const WT* W, const WT* X, int M, int N, int K, float* Y, int ldy, WT* Z, int ldz,
                        hipStream_t s) {
  for (int m0 = 0; m0 < M; m0 += 8) {
    const int mb = min(8, M - m0);
    const WT* x = X + static_cast<size_t>(m0) * K;
    float* y = Y ? Y + static_cast<size_t>(m0) * ldy : nullptr;
    WT* z = Z ? Z + static_cast<size_t>(m0) * ldz : nullptr;
    hipError_t e = hipSuccess;
    switch (mb) {
      case 1: e = launch_m<WT, 1, EPI>(W, x, N, K, y, ldy, z, ldz, s); break;
      case 2: e = launch_m<WT, 2, EPI>(W, x, N, K, y, ldy, z, ldz, s); break;
      case 3: e = launch_m<WT, 3, EPI>(W, x, N, K, y, ldy, z, ldz, s); break;
      case 4: e = launch_m<WT, 4, EPI>(W, x, N, K, y, ldy, z, ldz, s); break;
      case 5: e = launch_m<WT, 5, EPI>(W, x, N, K, y, ldy, z, ldz, s); break;
      case 6: e = launch_m<WT, 6, EPI>(W, x, N, K, y, ldy, z, ldz, s); break;
      case 7: e = launch_m<WT, 7, EPI>(W, x, N, K, y, ldy, z, ldz, s); break;
      default: e = launch_m<WT, 8, EPI>(W, x, N, K, y, ldy, z, ldz, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename WT>
hipError_t launch_dtype(int epi, const void* W, const void* x, int M, int N, int K, float* y, int ldy, void* z,
                        int ldz, hipStream_t s) {
  const WT* w = static_cast<const WT*>(W);
  const WT* xx = static_cast<const WT*>(x);
  WT* zz = static_cast<WT*>(z);
  switch (epi) {
    case EPI_STORE: return launch_typed<WT, EPI_STORE>(w, xx, M, N, K, y, ldy, zz, ldz, s);
    case EPI_RESID: return launch_typed<WT, EPI_RESID>(w, xx, M, N, K, y, ldy, zz, ldz, s);
    default: return launch_typed<WT, EPI_SWIGLU>(w, xx, M, N, K, y, ldy, zz, ldz, s);
  }
}

}  // namespace

hipError_t launch_gemv(bool bf16, int epi, const void* W, const void* x, int M, int N, int K, float* y, int ldy,
                       void* z, int ldz, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  return bf16 ? launch_dtype<uint16_t>(epi, W, x, M, N, K, y, ldy, z, ldz, s)
              : launch_dtype<float>(epi, W, x, M, N, K, y, ldy, z, ldz, s);
}

}  // namespace sv
