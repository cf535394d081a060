// The verify pass of at most 8 rows (bf16 models) as one persistent launch.
//
// The pass streams every weight once and does about two flops per weight
// byte (first page, section "The speedup is borrowed"), so its time is the
// weight bytes over the HBM bandwidth plus whatever keeps the weight stream
// from flowing.  Run as one kernel per linear, each launch pays dispatch,
// ramp-up and drain: about 6 us per linear at the 8B shape, a third of the
// pass.  Here one workgroup per CU runs every layer; the data dependencies
// between the steps of a layer (QKV -> attention -> O -> gate/up -> down)
// become grid barriers, and before waiting at one each wave already has the
// first weights of its next tile in flight, so HBM keeps streaming through
// the barrier.
//
// Workgroup: 512 threads (8 waves, 2 per SIMD, so each wave may hold 256
// registers).  Tiles of 2 weight rows (a RoPE pair for QKV, gate + up rows
// for SwiGLU, 2 consecutive rows otherwise) are dealt wave-major over waves
// 0-6: tile t goes to wave t / G of workgroup t % G, so every CU gets the
// same share.  A ring of U register slots (U = 4 at the 8B shape) keeps U
// steps (2 x 1 KiB per step) in flight per wave, 56 KiB per CU.
// Wave 7 streams nothing: it arrives at and polls the barriers, so its
// polling loads never queue behind weight loads (vector loads complete in
// issue order), and it helps with staging and attention.
//
// Memory between workgroups.  The L2 of an XCD is not coherent with the
// others, so data one workgroup writes and another reads inside the launch
// (q, the new K/V rows, the attention output, h, z) is stored with
// agent-scope (sc1) stores and loaded with agent-scope (sc1) buffer loads;
// a wave drains its stores (vmcnt 0) before its workgroup arrives at a
// barrier.  No L2 write-back or invalidate is needed.  The weights, the
// cached keys and values of earlier passes and the embedding kernel's
// outputs were written before the launch and use ordinary loads.
//
// Residual stream.  O and down have the same tiles (2 output columns of
// d), so the lane that owns h[m][c] owns it for the whole pass: h stays in
// its register (a wave has at most 2 such tiles), each residual add is a
// register add, and the owner stores the new value for the RMSNorm that the
// next step's staging computes.
//
// Grid barrier: arrivals striped over 8 counters (workgroup id mod 8, one
// atomic add each), polled by one wave that reads all 8 with one load per
// lane.  Every wait is bounded: past the spin limit the workgroup sets the
// error word and leaves, so a launch always ends.  The counters are zeroed
// by the embedding kernel that precedes every pass.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "attn_unit.hpp"
#include "common.hpp"
#include "gemv_kernels.hpp"
#include "kernels.hpp"

namespace sv {
namespace fused {

constexpr int NT = 512;
constexpr int NWV = NT / kWave;    // waves per workgroup
constexpr int kPoller = NWV - 1;   // wave that arrives at and polls the barrier
constexpr int kTileWaves = NWV - 1;  // waves that stream weights
constexpr int STEP = kWave * 8;    // bf16 columns per ring step (64 lanes x 16 B)
constexpr int KT = 32;             // attention keys per wave per trip
constexpr unsigned kSpinLimit = 1u << 22;
constexpr int kMaxLds = 150 * 1024;  // dynamic LDS: the staged activation rows

using unit::load_sc1;
using unit::rsrc;
using unit::store_sc1;
using unit::v4u;

__device__ __forceinline__ void drain_stores() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

// A weight matrix as a list of 2-row tiles.  KIND 0: rows {2t, 2t+1} of N
// (clamped); 1: gate/up rows {t, t + N} (N = d_ff); 2: the RoPE pair
// {j, j + HD/2} of head t / (HD/2).
struct Ph {
  const uint16_t* W;
  int K;       // columns (row stride)
  int S;       // ring steps per row: ceil(K / STEP)
  int ntiles;
  int N;
};

__device__ __forceinline__ Ph make_ph(const void* W, int K, int N, int ntiles) {
  Ph p;
  p.W = static_cast<const uint16_t*>(W);
  p.K = K;
  p.S = (K + STEP - 1) / STEP;
  p.N = N;
  p.ntiles = ntiles;
  return p;
}

template <int KIND, int HD>
__device__ __forceinline__ void tile_ptrs(const Ph& p, int t, const uint16_t* (&r)[2]) {
  int r0, r1;
  if constexpr (KIND == 0) {
    r0 = min(2 * t, p.N - 1);
    r1 = min(2 * t + 1, p.N - 1);
  } else if constexpr (KIND == 1) {
    r0 = t;
    r1 = t + p.N;
  } else {
    constexpr int half = HD / 2;
    const int hh = t / half, j = t - hh * half;
    r0 = hh * HD + j;
    r1 = r0 + half;
  }
  r[0] = p.W + static_cast<size_t>(r0) * p.K;
  r[1] = p.W + static_cast<size_t>(r1) * p.K;
}

__device__ __forceinline__ void load_step(const uint16_t* const (&r)[2], int st, int K, int lane, uint4 (&dst)[2]) {
  const int k = min(st * STEP + lane * 8, K - 8);
  dst[0] = gemv::load_stream(r[0] + k);
  dst[1] = gemv::load_stream(r[1] + k);
}

// Put the first U steps of tile t in flight.  A wave without tile t gets
// zeros: every slot is written either way, so no earlier ring contents stay
// live (in registers) across the code in between.
template <int KIND, int HD, int U>
__device__ __forceinline__ void ring_fill(const Ph& p, int t, int lane, uint4 (&wv)[U][2]) {
  if (t >= p.ntiles) {
#pragma unroll
    for (int u = 0; u < U; ++u) wv[u][0] = wv[u][1] = make_uint4(0, 0, 0, 0);
    return;
  }
  const uint16_t* r[2];
  tile_ptrs<KIND, HD>(p, t, r);
#pragma unroll
  for (int u = 0; u < U; ++u) load_step(r, u, p.K, lane, wv[u]);
}

using LayerW = FusedLayer;
using PassArgs = FusedArgs;

// ---- staging of the activation rows into LDS (bf16, row stride KP, zero padded)

template <int M>
__device__ __forceinline__ void stage_rows(const uint16_t* src, int K, int KP, bool coherent, uint16_t* xs) {
  const int kv = K / 8, kpv = KP / 8;
  const __amdgpu_buffer_rsrc_t r = rsrc(src, static_cast<uint32_t>(M) * K * 2);
#pragma unroll
  for (int mm = 0; mm < M; ++mm) {
    for (int v = threadIdx.x; v < kpv; v += NT) {
      uint4 val = make_uint4(0, 0, 0, 0);
      if (v < kv) {
        if (coherent) {
          const v4u t = load_sc1(r, static_cast<uint32_t>(mm * K + v * 8) * 2);
          val = make_uint4(t.x, t.y, t.z, t.w);
        } else {
          val = reinterpret_cast<const uint4*>(src + static_cast<size_t>(mm) * K)[v];
        }
      }
      reinterpret_cast<uint4*>(xs + static_cast<size_t>(mm) * KP)[v] = val;
    }
  }
}

// x = bf16(RMSNorm(h) * gain) for the M rows of h [M][d] (agent-scope loads),
// written to LDS with the padding columns zeroed.
template <int M>
__device__ __forceinline__ void stage_norm(const float* h, int d, int KP, const float* gain, float eps, uint16_t* xs,
                                           float (*red)[8]) {
  using NR = NormRegs<NT, M>;
  NR nr;
  const int d4 = d / 4;
  const __amdgpu_buffer_rsrc_t r = rsrc(h, static_cast<uint32_t>(M) * d * 4);
#pragma unroll
  for (int g = 0; g < M; ++g) {
#pragma unroll
    for (int c = 0; c < NR::CPT; ++c) {
      const int e4 = min(static_cast<int>(threadIdx.x) + c * NT, d4 - 1);
      const v4u t = load_sc1(r, static_cast<uint32_t>(g * d + 4 * e4) * 4);
      nr.v[g][c] = make_float4(__uint_as_float(t.x), __uint_as_float(t.y), __uint_as_float(t.z), __uint_as_float(t.w));
    }
  }
  norm_commit<NT, M>(nr, d, gain, eps, xs, KP, red);
#pragma unroll
  for (int mm = 0; mm < M; ++mm)
    for (int c = d + threadIdx.x; c < KP; c += NT) xs[static_cast<size_t>(mm) * KP + c] = 0;
}

// ---- one streaming step: every tile of this wave, ring carried in and out

template <int KIND, int HD, int M, int U, class Epi>
__device__ __forceinline__ void stream(const Ph& p, uint4 (&wv)[U][2], const uint16_t* xs, int KP, int gw, int TW,
                                       int lane, Epi&& epi) {
  const uint16_t* cur[2];
  const uint16_t* nxt[2];
  if (gw < p.ntiles) tile_ptrs<KIND, HD>(p, gw, cur);
  for (int t = gw; t < p.ntiles; t += TW) {
    const bool more = t + TW < p.ntiles;
    if (more) tile_ptrs<KIND, HD>(p, t + TW, nxt);
    float acc[2][M];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int mm = 0; mm < M; ++mm) acc[r][mm] = 0.f;
    auto compute = [&](int st, const uint4 (&w)[2]) {
      const int k = st * STEP + lane * 8;
#pragma unroll
      for (int mm = 0; mm < M; ++mm) {
        const uint4 xv = *reinterpret_cast<const uint4*>(xs + static_cast<size_t>(mm) * KP + k);
        acc[0][mm] = gemv::Dot<uint16_t>::run(w[0], xv, acc[0][mm]);
        acc[1][mm] = gemv::Dot<uint16_t>::run(w[1], xv, acc[1][mm]);
      }
    };
    for (int s0 = 0; s0 + U < p.S; s0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        compute(s0 + u, wv[u]);
        load_step(cur, s0 + U + u, p.K, lane, wv[u]);
      }
    }
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        compute(p.S - U + u, wv[u]);
        load_step(nxt, u, p.K, lane, wv[u]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) compute(p.S - U + u, wv[u]);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int mm = 0; mm < M; ++mm) acc[r][mm] = wave_sum(acc[r][mm]);
    epi(t, acc);
    if (more) {
      cur[0] = nxt[0];
      cur[1] = nxt[1];
    }
  }
}

// ---- grid barrier ----------------------------------------------------------------

constexpr int kStripes = 8;
constexpr int kStripeWords = 64;

// All threads call it after draining their stores.  Returns false (error
// word set) if the wait timed out.
__device__ __forceinline__ bool grid_barrier(unsigned* bar, unsigned target, int* err, int* flag_sh) {
  __syncthreads();
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  if (wave == kPoller) {
    if (lane == 0)
      __hip_atomic_fetch_add(bar + kStripeWords * (blockIdx.x % kStripes), 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    bool ok = true;
    unsigned n = 0;
    while (true) {
      unsigned v = lane < kStripes
                       ? __hip_atomic_load(bar + kStripeWords * lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                       : 0u;
      v += __shfl_xor(v, 1, kWave);
      v += __shfl_xor(v, 2, kWave);
      v += __shfl_xor(v, 4, kWave);
      if (__shfl(v, 0, kWave) >= target) break;
      __builtin_amdgcn_s_sleep(1);
      if (++n > kSpinLimit) {
        ok = false;
        break;
      }
    }
    if (lane == 0) {
      *flag_sh = ok;
      if (!ok) __hip_atomic_fetch_or(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  return *flag_sh != 0;
}

// ---- the kernel ----------------------------------------------------------------------

template <int M, int U, int HD>
__global__ __launch_bounds__(NT) void pass_kernel(PassArgs a) {
  extern __shared__ uint4 smem_v[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem_v);
  __shared__ float red[NWV][8];
  __shared__ int flag_sh;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int G = gridDim.x, TW = G * kTileWaves;
  // the poller has no tiles: its index lies past every list (and 2 (gw +
  // 2 TW) stays in int range)
  const int gw = wave < kTileWaves ? wave * G + blockIdx.x : (1 << 28);
  const int d = a.d, H = a.H, Hkv = a.Hkv, F = a.F;
  const int hq = H * HD;
  const int units = a.B * H * a.m;
  const bool attn_wg = static_cast<int>(blockIdx.x) < units;
  const int KPd = (d + STEP - 1) / STEP * STEP, KPo = (hq + STEP - 1) / STEP * STEP;
  const int KPf = (F + STEP - 1) / STEP * STEP;
  unsigned target = 0;

  // The residual columns this lane owns in O and down: tiles gw and gw + TW,
  // rows {2t, 2t + 1}; lane r * M + mm holds h[mm][2t + r].
  const int own_r = lane / M, own_m = lane - own_r * M;
  float hreg[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = 2 * (gw + k * TW) + own_r;
    hreg[k] = (wave < kTileWaves && lane < 2 * M && c < d) ? a.h[static_cast<size_t>(own_m) * d + c] : 0.f;
  }

  auto ph_qkv = [&](int l) { return make_ph(a.layers[l].wqkv, d, HD, (H + 2 * Hkv) * (HD / 2)); };
  auto ph_o = [&](int l) { return make_ph(a.layers[l].wo, hq, d, (d + 1) / 2); };
  auto ph_gu = [&](int l) { return make_ph(a.layers[l].wgu, d, F, F); };
  auto ph_dn = [&](int l) { return make_ph(a.layers[l].wd, F, d, (d + 1) / 2); };
  const Ph ph_lm = make_ph(a.lm_head, d, a.V, (a.V + 1) / 2);

  // Epilogues (the wave sums are in every lane; lane r * M + mm writes
  // output row mm of weight row r).
  auto pick = [&](const float (&acc)[2][M], int r_sel, int m_sel) {
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int mm = 0; mm < M; ++mm)
        if (r == r_sel && mm == m_sel) v = acc[r][mm];
    return v;
  };
  auto epi_resid = [&](int t, const float (&acc)[2][M]) {
    const int c = 2 * t + own_r;
    if (lane < 2 * M && c < d) {
      const float v = pick(acc, own_r, own_m);
      float hv;
      if (t == gw) {
        hreg[0] += v;
        hv = hreg[0];
      } else {
        hreg[1] += v;
        hv = hreg[1];
      }
      store_sc1(a.h + static_cast<size_t>(own_m) * d + c, hv);
    }
  };
  auto epi_swiglu = [&](int t, const float (&acc)[2][M]) {
    if (lane < M) {
      const float g = pick(acc, 0, lane), uu = pick(acc, 1, lane);
      store_sc1(static_cast<uint16_t*>(a.z) + static_cast<size_t>(lane) * F + t, f2bf(g / (1.f + expf(-g)) * uu));
    }
  };
  int cur_layer = 0;
  auto epi_qkv = [&](int t, const float (&acc)[2][M]) {
    if (lane < M) {
      const int half = HD / 2, hh = t / half, j = t - hh * half;
      const int rg = lane, b = rg / a.m, i = rg - b * a.m;
      const float x0 = pick(acc, 0, lane), y0 = pick(acc, 1, lane);
      if (hh < H + Hkv) {
        const float2 c = a.cs[static_cast<size_t>(rg) * half + j];
        const float r0 = x0 * c.x - y0 * c.y, s0 = y0 * c.x + x0 * c.y;
        if (hh < H) {
          float* qr = a.q + static_cast<size_t>(rg) * hq + hh * HD;
          store_sc1(qr + j, r0);
          store_sc1(qr + j + half, s0);
        } else {
          const int pos = a.len[b] + i;
          if (pos >= 0 && pos < a.max_ctx) {
            uint16_t* dst = static_cast<uint16_t*>(a.kc) +
                            (((static_cast<size_t>(cur_layer) * a.kvB + b) * Hkv + (hh - H)) * a.max_ctx + pos) * HD;
            store_sc1(dst + j, f2bf(r0));
            store_sc1(dst + j + half, f2bf(s0));
          }
        }
      } else {
        const int pos = a.len[b] + i;
        if (pos >= 0 && pos < a.max_ctx) {
          uint16_t* dst = static_cast<uint16_t*>(a.vc) +
                          (((static_cast<size_t>(cur_layer) * a.kvB + b) * Hkv + (hh - H - Hkv)) * a.max_ctx + pos) *
                              HD;
          store_sc1(dst + j, f2bf(x0));
          store_sc1(dst + j + half, f2bf(y0));
        }
      }
    }
  };
  auto epi_lm = [&](int t, const float (&acc)[2][M]) {
    if (lane < 2 * M) {
      const int c = 2 * t + own_r;
      if (c < a.V) a.logits[static_cast<size_t>(own_m) * a.V + c] = pick(acc, own_r, own_m);
    }
  };

  // Drain this wave's stores, optionally put the next step's first tile in
  // flight, then meet at the barrier.
  uint4 wv[U][2];
  auto handoff = [&](auto kind, const Ph& next, bool prefetch) {
    drain_stores();
    if (prefetch) ring_fill<decltype(kind)::value, HD, U>(next, gw, lane, wv);
    target += G;
    return grid_barrier(a.bar, target, a.err, &flag_sh);
  };
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;
  using K2 = std::integral_constant<int, 2>;

  ring_fill<2, HD, U>(ph_qkv(0), gw, lane, wv);
  for (int l = 0; l < a.L; ++l) {
    cur_layer = l;
    const LayerW lw = a.layers[l];
    // QKV + RoPE + K/V append
    if (l == 0) {
      stage_rows<M>(static_cast<const uint16_t*>(a.xn), d, KPd, false, xs);
    } else {
      stage_norm<M>(a.h, d, KPd, lw.attn_norm, a.eps, xs, red);
    }
    __syncthreads();
    stream<2, HD, M, U>(ph_qkv(l), wv, xs, KPd, gw, TW, lane, epi_qkv);
    // attention: units (sequence, head, row) over the workgroups; the others
    // put their O tiles in flight right after the barrier, these after their
    // units (no ring is live across the attention code)
    if (!handoff(K0{}, ph_o(l), false)) return;
    if (attn_wg) {
      const unit::AttnUnitArgs ua{a.q, a.kc, a.vc, a.len, a.xo, a.B, a.m, H, Hkv, a.kvB, a.max_ctx, l};
      for (int uu = blockIdx.x; uu < units; uu += G)
        unit::attn_unit<HD, NWV, KT>(ua, uu, reinterpret_cast<char*>(smem_v));
    }
    if (!handoff(K0{}, ph_o(l), true)) return;
    // O + residual
    stage_rows<M>(static_cast<const uint16_t*>(a.xo), hq, KPo, true, xs);
    __syncthreads();
    stream<0, HD, M, U>(ph_o(l), wv, xs, KPo, gw, TW, lane, epi_resid);
    if (!handoff(K1{}, ph_gu(l), true)) return;
    // MLP RMSNorm + gate/up + SwiGLU
    stage_norm<M>(a.h, d, KPd, lw.mlp_norm, a.eps, xs, red);
    __syncthreads();
    stream<1, HD, M, U>(ph_gu(l), wv, xs, KPd, gw, TW, lane, epi_swiglu);
    if (!handoff(K0{}, ph_dn(l), true)) return;
    // down + residual
    stage_rows<M>(static_cast<const uint16_t*>(a.z), F, KPf, true, xs);
    __syncthreads();
    stream<0, HD, M, U>(ph_dn(l), wv, xs, KPf, gw, TW, lane, epi_resid);
    if (l + 1 < a.L) {
      if (!handoff(K2{}, ph_qkv(l + 1), true)) return;
    } else {
      if (!handoff(K0{}, ph_lm, a.logits != nullptr)) return;
    }
  }
  if (!a.logits) return;  // a pass without the LM head (prefill)
  // final RMSNorm + LM head
  stage_norm<M>(a.h, d, KPd, a.final_norm, a.eps, xs, red);
  __syncthreads();
  stream<0, HD, M, U>(ph_lm, wv, xs, KPd, gw, TW, lane, epi_lm);
}

}  // namespace fused

namespace {

int device_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
  }
  return n;
}

template <int M, int U, int HD>
hipError_t launch_t(const FusedArgs& a, size_t lds, hipStream_t s) {
  auto kern = fused::pass_kernel<M, U, HD>;
  static bool lds_opt_in = false;
  if (!lds_opt_in) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, fused::kMaxLds);
    if (e != hipSuccess) return e;
    lds_opt_in = true;
  }
  const int grid = device_cus();
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &cap);
  if (e != hipSuccess) return e;
  if (cap == hipStreamCaptureStatusNone) {
    // the launch fails rather than run if the grid cannot be co-resident
    FusedArgs arg = a;
    void* args[] = {&arg};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kern), dim3(grid), dim3(fused::NT), args, lds, s);
  }
  // Under stream capture: an ordinary launch of one workgroup per CU on a
  // device with nothing else running before it in the graph; the bounded
  // barrier waits end the launch if a workgroup could not start.
  hipLaunchKernelGGL(kern, dim3(grid), dim3(fused::NT), lds, s, a);
  return hipGetLastError();
}

template <int U, int HD>
hipError_t launch_m(const FusedArgs& a, int M, size_t lds, hipStream_t s) {
  switch (M) {
    case 1: return launch_t<1, U, HD>(a, lds, s);
    case 2: return launch_t<2, U, HD>(a, lds, s);
    case 3: return launch_t<3, U, HD>(a, lds, s);
    case 4: return launch_t<4, U, HD>(a, lds, s);
    case 5: return launch_t<5, U, HD>(a, lds, s);
    case 6: return launch_t<6, U, HD>(a, lds, s);
    case 7: return launch_t<7, U, HD>(a, lds, s);
    case 8: return launch_t<8, U, HD>(a, lds, s);
    default: return hipErrorInvalidValue;
  }
}

int steps(int K) { return (K + fused::STEP - 1) / fused::STEP; }

}  // namespace

int fused_pass_ring(int d, int hq, int F) {
  for (int U : {4, 2})
    if (steps(d) % U == 0 && steps(hq) % U == 0 && steps(F) % U == 0) return U;
  return 0;
}

size_t fused_pass_lds(int rows, int d, int hq, int F, int hd) {
  const size_t kp = static_cast<size_t>(std::max(steps(d), std::max(steps(hq), steps(F)))) * fused::STEP;
  const size_t stage = static_cast<size_t>(rows) * kp * 2;
  const size_t attn = sizeof(float) * fused::NWV * hd + sizeof(float2) * fused::NWV;
  return std::max(stage, attn);
}

bool fused_pass_supported(bool bf16, int rows, int d, int H, int Hkv, int hd, int F) {
  if (!bf16 || rows < 1 || rows > 8 || (hd != 64 && hd != 128)) return false;
  if (d % 8 || F % 8 || d > 4096 || H % Hkv) return false;
  if ((d + 1) / 2 > 2 * 256 * fused::kTileWaves) return false;  // at most 2 O/down tiles per wave
  if (fused_pass_ring(d, H * hd, F) == 0) return false;
  return fused_pass_lds(rows, d, H * hd, F, hd) <= static_cast<size_t>(fused::kMaxLds);
}

hipError_t launch_fused_pass(const FusedArgs& a, int hd, hipStream_t s) {
  const int M = a.B * a.m;
  const int U = fused_pass_ring(a.d, a.H * hd, a.F);
  const size_t lds = fused_pass_lds(M, a.d, a.H * hd, a.F, hd);
  if (U == 0 || lds > static_cast<size_t>(fused::kMaxLds)) return hipErrorInvalidValue;
  if (hd == 128) return U == 4 ? launch_m<4, 128>(a, M, lds, s) : launch_m<2, 128>(a, M, lds, s);
  if (hd == 64) return U == 4 ? launch_m<4, 64>(a, M, lds, s) : launch_m<2, 64>(a, M, lds, s);
  return hipErrorInvalidValue;
}

}  // namespace sv
