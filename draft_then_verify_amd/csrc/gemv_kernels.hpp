// Weight-streaming GEMV kernel for the verify pass:
//   y[M][N] = x[M][K] . W[N][K]^T, M <= 8 activation rows per launch.
//
// The pass is bound by reading the weights: a decode or verify pass streams
// every weight once and does about two floating-point operations per weight
// read, and scoring the gamma + 1 positions of a round streams the same bytes
// as scoring one (first page, section "The speedup is borrowed").  So every
// weight byte is loaded exactly once per launch and used for all M rows.
//
// Structure (persistent, one launch streams the whole matrix):
//  * The grid is a few workgroups per CU (x) times the K slices (y).  Each
//    workgroup stages its slice of the M activation rows in LDS once (up to
//    159 KiB on gfx950); slicing K keeps that staging small enough for
//    several workgroups per CU, and each slice writes its own partial y.
//  * Each wave walks its own list of row tiles (R rows; 2R for SwiGLU's gate
//    and up rows) as one continuous stream of 1 KiB steps: 64 lanes x 16 B of
//    one weight row per load instruction.  A ring of U register slots keeps
//    U * R loads per lane in flight across tile boundaries, so the stream only
//    drains at the very end of the matrix.  The activation rows are loaded
//    first and the first U weight steps right behind them (vector loads
//    complete in issue order), so staging overlaps the weight stream.
//  * bf16: v_dot2_f32_bf16 multiplies two bf16 pairs and accumulates in
//    float32 without converting the weights; float32 models use fma.
//  * At the end of a tile: one wave reduction per (row, activation row) and
//    the epilogue -- store, add into the float32 residual stream,
//    silu(g) * u, or (QKV) RoPE on q/k and the K/V append.  For QKV a wave's
//    2 rows are {j, j+hd/2} of one head, the two halves of a rotated pair.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace sv {
namespace gemv {

constexpr int kMaxLds = 159 * 1024;  // dynamic LDS; 1 KiB is left for static arrays
// Weight steps a wave issues before the activation staging (see the
// prologue of gemv_kernel); the rest of the ring follows it.  Per epilogue,
// from the 8B-shaped 5-row step and the 0.6B-shaped drafter round (3 runs of
// each, graph-replayed): the same 2 steps everywhere gave 3.292 ms and 2.906
// ms; the whole ring of 4 for the residual linears (O, down: a short bf16
// copy stages their input) 3.243 and 2.850; with 3 for QKV as well (an
// RMSNorm of float32 rows stages its input) 3.249 and 2.851.  One step for
// the residual linears, or 4 for QKV, was slower.  Gate/up keeps 2: with 3
// the step gained ~0.015 ms, but back-to-back gate/up launches (the
// dominant kernel timed on its own) ran 4% slower than inside the step.
// The residual linears issue their whole ring, whatever its depth (8 caps
// it): with a ring of 6 (rows of 6 steps), 6 rather than 4 took the second
// workload's B = 1 verify step from 0.304 to 0.301 ms.
template <int EPI> constexpr int pre_steps() {
  return EPI == EPI_RESID ? 8 : EPI == EPI_QKV ? 3 : 2;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 global_u32x4;

// Weights are read once: non-temporal loads keep them from displacing the
// activations and KV rows in the caches.  The explicit global address space
// keeps these as global (not flat) loads, which count only against vmcnt, so
// waiting for the LDS activation reads never drains the weight stream.
__device__ __forceinline__ uint4 load_stream(const void* p) {
  u32x4 v = __builtin_nontemporal_load((global_u32x4*)(p));
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

template <int EPI, int R> struct Tiles {
  static_assert(EPI != EPI_QKV || R == 2, "QKV tiles are rotated pairs");
  static constexpr int NW = (EPI == EPI_SWIGLU) ? 2 * R : R;  // weight rows per tile
};

// Number of R-row tiles of a launch.
template <int EPI, int R>
__host__ __device__ inline int num_tiles(int N) {
  return EPI == EPI_QKV ? N / 2 : (N + R - 1) / R;
}

// Weight rows of tile t (clamped into range; the epilogue checks validity).
template <int EPI, int R>
__device__ __forceinline__ void tile_rows(const GemvArgs& a, int t, int (&rows)[Tiles<EPI, R>::NW]) {
  if constexpr (EPI == EPI_QKV) {
    const int half = a.hd / 2;
    const int hh = t / half, j = t - hh * half;
    rows[0] = hh * a.hd + j;
    rows[1] = hh * a.hd + j + half;
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      rows[r] = min(t * R + r, a.N - 1);
      if constexpr (EPI == EPI_SWIGLU) rows[R + r] = rows[r] + a.N;
    }
  }
}

// Stage this workgroup's slice of the M activation rows into LDS (model
// dtype, row stride KP >= K, zero-padded to KP).
template <typename WT, int M, int NT>
__device__ __forceinline__ void stage_x(const WT* x, int ldx, int K, WT* xs, int KP) {
  constexpr int VE = 16 / sizeof(WT);
  const int kv = K / VE, kpv = KP / VE;
#pragma unroll 4
  for (int idx = threadIdx.x; idx < M * kpv; idx += NT) {
    const int m = idx / kpv, v = idx - m * kpv;
    reinterpret_cast<uint4*>(xs)[idx] =
        (v < kv) ? reinterpret_cast<const uint4*>(x + static_cast<size_t>(m) * ldx)[v] : make_uint4(0, 0, 0, 0);
  }
}

// Values the epilogue of tile t reads from memory, loaded when the tile
// starts so that the loads are back by its end: the RoPE (cos, sin) and the
// cache position of lane m's row (QKV), or the residual value the lane adds
// to (EPI_RESID).  A lane that writes nothing loads nothing.
struct EpiPre {
  float2 cs = make_float2(0.f, 0.f);
  int pos = -1;
  float y = 0.f;
};

template <typename WT, int M, int R, int EPI>
__device__ __forceinline__ EpiPre epilogue_pre(const GemvArgs& a, const float* y, int t, int lane) {
  EpiPre e;
  if constexpr (EPI == EPI_QKV) {
    if (lane < M) {
      const int half = a.hd / 2;
      const int hh = t / half, j = t - hh * half;
      const int rg = a.row0 + lane;
      const int b = rg / a.m_per_seq, i = rg - b * a.m_per_seq;
      if (hh < a.H + a.Hkv) e.cs = a.cs[static_cast<size_t>(rg) * half + j];
      if (hh >= a.H) e.pos = a.len[b] + i;
    }
  } else if constexpr (EPI == EPI_RESID) {
    const int r = lane / M, m = lane - r * M;
    const int c = t * R + r;
    if (r < R && c < a.N) {
      const float* src = y + static_cast<size_t>(m) * a.ldy + c;
      e.y = *src;
    }
  }
  return e;
}

template <typename WT, int M, int R, int EPI>
__device__ __forceinline__ void epilogue(const GemvArgs& a, float* y, int t, float (&acc)[Tiles<EPI, R>::NW][M],
                                         int lane, const EpiPre& pre) {
  if constexpr (EPI == EPI_QKV) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if (lane != m) continue;
      const int H = a.H, Hkv = a.Hkv, hd = a.hd, half = hd / 2;
      const int hh = t / half, j = t - hh * half;
      const int rg = a.row0 + m;
      const int b = rg / a.m_per_seq;
      const float x0 = acc[0][m], y0 = acc[1][m];
      if (hh < H + Hkv) {
        const float2 c = pre.cs;
        const float r0 = x0 * c.x - y0 * c.y, s0 = y0 * c.x + x0 * c.y;
        if (hh < H) {
          float* qr = a.q + static_cast<size_t>(rg) * (H * hd) + hh * hd;
          qr[j] = r0;
          qr[j + half] = s0;
        } else {
          const int pos = pre.pos;
          if (pos >= 0 && pos < a.max_ctx) {
            WT* dst = static_cast<WT*>(a.kc) +
                      (((static_cast<size_t>(a.layer) * a.kvB + b) * Hkv + (hh - H)) * a.max_ctx + pos) * hd;
            dst[j] = Elt<WT>::from_f(r0);
            dst[j + half] = Elt<WT>::from_f(s0);
          }
        }
      } else {
        const int pos = pre.pos;
        if (pos >= 0 && pos < a.max_ctx) {
          WT* dst = static_cast<WT*>(a.vc) +
                    (((static_cast<size_t>(a.layer) * a.kvB + b) * Hkv + (hh - H - Hkv)) * a.max_ctx + pos) * hd;
          dst[j] = Elt<WT>::from_f(x0);
          dst[j + half] = Elt<WT>::from_f(y0);
        }
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int c = t * R + r;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if (lane == r * M + m && c < a.N) {
          if constexpr (EPI == EPI_STORE || EPI == EPI_PARTIAL) {
            y[static_cast<size_t>(m) * a.ldy + c] = acc[r][m];
          } else if constexpr (EPI == EPI_RESID) {
            y[static_cast<size_t>(m) * a.ldy + c] = pre.y + acc[r][m];
          } else {
            const float g = acc[r][m], u = acc[R + r][m];
            static_cast<WT*>(a.z)[static_cast<size_t>(m) * a.ldz + c] = Elt<WT>::from_f(g / (1.f + expf(-g)) * u);
          }
        }
      }
    }
  }
}

// Steps of a row: S = ceil(K / STEP); U must divide S.
// WPE: minimum waves per SIMD the register allocation must allow; NT threads.
// Workgroup blockIdx.x of gridDim.x over K slice blockIdx.y.
template <typename WT, int M, int R, int U, int EPI, int WPE, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(WPE))) void gemv_kernel(GemvArgs a) {
  const int wg = blockIdx.x, nwg = gridDim.x, slice = blockIdx.y;
  extern __shared__ uint4 smem_v[];
  WT* xs = reinterpret_cast<WT*>(smem_v);
  constexpr int VE = 16 / sizeof(WT);
  constexpr int STEP = kWave * VE;
  constexpr int NW = Tiles<EPI, R>::NW;
  constexpr int WPB = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int K = a.K;  // columns of this workgroup's slice
  const int S = (K + STEP - 1) / STEP;
  const int KP = S * STEP;
  const WT* W = static_cast<const WT*>(a.W) + static_cast<size_t>(slice) * K;
  float* y = a.y ? a.y + static_cast<size_t>(slice) * a.ysplit : nullptr;
  const int n_tiles = num_tiles<EPI, R>(a.N);
  const int gw = wg * WPB + wave;
  const int TW = nwg * WPB;
  const int my_tiles = gw < n_tiles ? (n_tiles - gw + TW - 1) / TW : 0;
  // per-lane column of step s: clamped into the row (the padded x is zero there)
  const int lk = lane * VE;

  const WT* cur[NW];
  const WT* nxt[NW];
  auto set_rows = [&](int t, const WT* (&p)[NW]) {
    int rows[NW];
    tile_rows<EPI, R>(a, t, rows);
#pragma unroll
    for (int r = 0; r < NW; ++r) p[r] = W + static_cast<size_t>(rows[r]) * a.ldw;
  };
  auto load_step = [&](const WT* const (&p)[NW], int st, uint4 (&dst)[NW]) {
    const int k = min(st * STEP + lk, K - VE);
#pragma unroll
    for (int r = 0; r < NW; ++r) dst[r] = load_stream(p[r] + k);
  };

  // Prologue.  Loads complete in issue order (per wave, and through the
  // CU's vector L1 across waves), so:
  //  1. every wave issues its activation loads, and a bare s_barrier (no
  //     fence, no wait) keeps all of them ahead of every wave's weight loads;
  //     an activation load queued behind weight loads (HBM misses, at the
  //     start of a launch the whole chip's burst) would wait for them;
  //  2. every wave issues its first kPre weight steps, in straight-line code
  //     (a wave without tiles streams tile 0's and never uses them): behind a
  //     branch the compiler cannot count the loads in flight and its wait for
  //     the activations becomes a wait for everything;
  //  3. the rows are normalised or copied into LDS; the staging ends at a
  //     workgroup barrier, which a wave only reaches once its loads are
  //     issued, so kPre steps go before it: the whole ring where a short
  //     copy stages the rows, fewer before a normalising staging (there,
  //     with the whole ring, the late waves of a CU wait for the early
  //     waves' weights to come back while the early waves idle at the
  //     barrier; pre_steps has the measurements);
  //  4. the rest of the ring is issued.
  // (bf16: x chunks per thread loaded ahead of the weights, 32 registers; the
  // float32 kernels keep their registers for the 4-fma dot products)
  constexpr bool kBf16 = sizeof(WT) == 2;
  constexpr int kPre = U < pre_steps<EPI>() ? U : pre_steps<EPI>();
  constexpr int XR = kBf16 ? 8 : 1;
  constexpr bool kEarlyNorm = kBf16 && M * NormRegs<NT, M>::CPT <= 10;  // 40 registers at most
  __shared__ float red[kNormBlocks][8];
  NormRegs<NT, kEarlyNorm ? M : 1> nr;
  uint4 xr[XR];
  const int xkv = K / VE, xkpv = KP / VE, xtot = M * xkpv;
  const WT* xg = (a.hn || a.apo) ? nullptr : static_cast<const WT*>(a.x) + static_cast<size_t>(slice) * K;
  // one row merged from attention partials (the O linear of a split
  // one-row pass): chunk j = threadIdx.x is loaded here, ahead of the weights
  constexpr bool kApart = M == 1;
  AttnPart<VE> ap;
  auto apart_load = [&](int v) {
    const int col = v * VE, hh = col / a.ahd;
    const size_t pi = static_cast<size_t>(hh) * a.asplit;
    attn_part_load<VE>(a.apo + pi * a.ahd, a.apml + pi, a.asplit, a.ahd, col - hh * a.ahd, ap);
  };
  if (a.hn) {
    if constexpr (kEarlyNorm) norm_issue<NT, M>(a.hn, K, K, a.gain, nr);
  } else if (kApart && a.apo) {
    if (static_cast<int>(threadIdx.x) < xkv) apart_load(threadIdx.x);
  } else {
    // a wave issues only the chunks that hold rows (the issue slots of the
    // vector memory unit are what the start of a launch waits on)
    const int wbase = wave * kWave;
#pragma unroll
    for (int c = 0; c < XR; ++c) {
      if (wbase + c * NT < xtot) {
        const int idx = min(static_cast<int>(threadIdx.x) + c * NT, xtot - 1);
        const int m = idx / xkpv, v = min(idx - m * xkpv, xkv - 1);
        xr[c] = reinterpret_cast<const uint4*>(xg + static_cast<size_t>(m) * a.ldx)[v];
      }
    }
  }
  __builtin_amdgcn_s_barrier();
  uint4 wv[U][NW];
  set_rows(my_tiles > 0 ? gw : 0, cur);
#pragma unroll
  for (int u = 0; u < kPre; ++u) load_step(cur, u, wv[u]);
  if (a.hn) {
    // x = cvt(RMSNorm(h) * gain), made in LDS (one K slice: K = d); the
    // padding columns K .. KP-1 are zero
    if constexpr (kEarlyNorm) {
      norm_commit<NT, M>(nr, K, a.eps, xs, KP, red);
    } else {
      norm_rows<NT, M, WT>(a.hn, K, K, a.gain, a.eps, xs, KP);
    }
    for (int idx = threadIdx.x; idx < M * (KP - K); idx += NT) {
      const int m = idx / (KP - K);
      xs[static_cast<size_t>(m) * KP + K + (idx - m * (KP - K))] = Elt<WT>::from_f(0.f);
    }
  } else if (kApart && a.apo) {
    for (int v = threadIdx.x; v < xkpv; v += NT) {
      uint4 val = make_uint4(0, 0, 0, 0);
      if (v < xkv) {
        if (v != static_cast<int>(threadIdx.x)) apart_load(v);
        float out[VE];
        attn_part_merge<VE>(ap, a.asplit, out);
        val = pack_chunk<WT>(out);
      }
      reinterpret_cast<uint4*>(xs)[v] = val;
    }
  } else {
#pragma unroll
    for (int c = 0; c < XR; ++c) {
      const int idx = threadIdx.x + c * NT;
      if (idx < xtot) reinterpret_cast<uint4*>(xs)[idx] = (idx % xkpv < xkv) ? xr[c] : make_uint4(0, 0, 0, 0);
    }
    for (int idx = threadIdx.x + XR * NT; idx < xtot; idx += NT) {
      const int m = idx / xkpv, v = idx - m * xkpv;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (v < xkv) val = reinterpret_cast<const uint4*>(xg + static_cast<size_t>(m) * a.ldx)[v];
      reinterpret_cast<uint4*>(xs)[idx] = val;
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = kPre; u < U; ++u) load_step(cur, u, wv[u]);

  float acc[NW][M];
  auto compute = [&](int st, const uint4 (&w)[NW]) {
    const int k = st * STEP + lk;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint4 xv = *reinterpret_cast<const uint4*>(xs + static_cast<size_t>(m) * KP + k);
#pragma unroll
      for (int r = 0; r < NW; ++r) acc[r][m] = Dot<WT>::run(w[r], xv, acc[r][m]);
    }
  };
  auto finish = [&](int t, const EpiPre& pre) {
#pragma unroll
    for (int r = 0; r < NW; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) acc[r][m] = wave_sum(acc[r][m]);
    epilogue<WT, M, R, EPI>(a, y, t, acc, lane, pre);
  };

  for (int ti = 0; ti < my_tiles; ++ti) {
    const int t = gw + ti * TW;
    const bool more = ti + 1 < my_tiles;
    const EpiPre pre = epilogue_pre<WT, M, R, EPI>(a, y, t, lane);
    if (more) set_rows(t + TW, nxt);
#pragma unroll
    for (int r = 0; r < NW; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) acc[r][m] = 0.f;
    // groups whose refills stay inside this tile
    for (int s0 = 0; s0 + U < S; s0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        compute(s0 + u, wv[u]);
        load_step(cur, s0 + U + u, wv[u]);
      }
    }
    // last group: refill with the next tile's first steps
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        compute(S - U + u, wv[u]);
        load_step(nxt, u, wv[u]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) compute(S - U + u, wv[u]);
    }
    finish(t, pre);
    if (more) {
#pragma unroll
      for (int r = 0; r < NW; ++r) cur[r] = nxt[r];
    }
  }
}

}  // namespace gemv
}  // namespace sv
