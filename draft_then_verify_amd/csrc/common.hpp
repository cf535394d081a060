// Device helpers shared by the gfx950 kernels: bf16 conversion, fixed-order
// wave/block reductions, 16-byte vector loads.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace sv {

constexpr int kWave = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// float32 -> bfloat16, round to nearest, ties to even; NaN stays NaN.  One
// v_cvt_pk_bf16_f32 on gfx950 (a bit-level rounding with its NaN test costs
// about 20 instructions and an exec-mask branch per element).
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

// Model element type: float (f32 models) or uint16_t holding bf16 bits.
template <typename T> struct Elt;
template <> struct Elt<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static float to_f(float x) { return x; }
  __device__ __forceinline__ static float from_f(float x) { return x; }
};
template <> struct Elt<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p) { return bf2f(*p); }
  __device__ __forceinline__ static float to_f(uint16_t x) { return bf2f(x); }
  __device__ __forceinline__ static uint16_t from_f(float x) { return f2bf(x); }
};

// VE values (8 as bf16 or 4 as float32) as one 16-byte chunk.
template <typename WT>
__device__ __forceinline__ uint4 pack_chunk(const float (&v)[16 / sizeof(WT)]) {
  if constexpr (sizeof(WT) == 2) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f2bf(v[2 * i])) | (static_cast<uint32_t>(f2bf(v[2 * i + 1])) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
  }
}

// ---- attention context splits ---------------------------------------------------------
// A head's context split over S workgroups leaves S partials: an unnormalised
// output o_s (relative to the split's max m_s) and its weight l_s.  The
// merged output is sum_s w_s o_s / sum_s w_s l_s with w_s = exp(m_s - max_s
// m_s) (0 for an empty split), summed in split order.  attn_part_load issues
// the loads of VE consecutive dimensions dd0 .. of one (row, head) (po and
// pml point at its S partials), attn_part_merge does the arithmetic, so a
// caller can issue other loads in between.
constexpr int kMaxAttnSplits = 4;
template <int VE> struct AttnPart {
  float4 o[kMaxAttnSplits][VE / 4];
  float2 ml[kMaxAttnSplits];
};
template <int VE>
__device__ __forceinline__ void attn_part_load(const float* po, const float2* pml, int S, int hd, int dd0,
                                               AttnPart<VE>& p) {
#pragma unroll
  for (int s = 0; s < kMaxAttnSplits; ++s) {
    if (s < S) {
      p.ml[s] = pml[s];
#pragma unroll
      for (int c = 0; c < VE / 4; ++c) p.o[s][c] = reinterpret_cast<const float4*>(po + s * hd + dd0)[c];
    }
  }
}
template <int VE>
__device__ __forceinline__ void attn_part_merge(const AttnPart<VE>& p, int S, float (&out)[VE]) {
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxAttnSplits; ++s)
    if (s < S) M = fmaxf(M, p.ml[s].x);
  float l = 0.f, acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxAttnSplits; ++s) {
    if (s < S) {
      const float w = p.ml[s].x == -INFINITY ? 0.f : expf(p.ml[s].x - M);
      l = fmaf(p.ml[s].y, w, l);
#pragma unroll
      for (int c = 0; c < VE / 4; ++c) {
        acc[4 * c + 0] = fmaf(p.o[s][c].x, w, acc[4 * c + 0]);
        acc[4 * c + 1] = fmaf(p.o[s][c].y, w, acc[4 * c + 1]);
        acc[4 * c + 2] = fmaf(p.o[s][c].z, w, acc[4 * c + 2]);
        acc[4 * c + 3] = fmaf(p.o[s][c].w, w, acc[4 * c + 3]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < VE; ++e) out[e] = l > 0.f ? acc[e] / l : 0.f;
}

// Reductions over the 64 lanes of a wave with DPP lane moves (no LDS
// round trip): pairs, quads, mirrored halves and rows of 16 lanes, then the
// four row results read as uniform values and combined as (r0 + r1) + (r2 + r3).
// Every lane receives the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
constexpr int kDppQuadSwap1 = 0xb1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4e;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within 16
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<kDppQuadSwap1>(v);
  v += dpp_mov<kDppQuadSwap2>(v);
  v += dpp_mov<kDppHalfMirror>(v);
  v += dpp_mov<kDppMirror>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<kDppQuadSwap1>(v));
  v = fmaxf(v, dpp_mov<kDppQuadSwap2>(v));
  v = fmaxf(v, dpp_mov<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_mov<kDppMirror>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Sum over the N (8 or 16) consecutive lanes of a DPP row group; every lane
// of the group gets the same bits (each step adds a commuted pair).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_mov<kDppQuadSwap1>(v);
  v += dpp_mov<kDppQuadSwap2>(v);
  v += dpp_mov<kDppHalfMirror>(v);
  if constexpr (N == 16) v += dpp_mov<kDppMirror>(v);
  return v;
}

// Max / sum over the lanes l, l ^ FROM, l ^ 2 FROM, ... (FROM = 8 or 16):
// the RPI row groups of a wave; all lanes get the same bits.
template <int FROM>
__device__ __forceinline__ float groups_max(float v) {
#pragma unroll
  for (int off = FROM; off < kWave; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}
template <int FROM>
__device__ __forceinline__ float groups_sum(float v) {
#pragma unroll
  for (int off = FROM; off < kWave; off <<= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Block reductions for blockDim.x == NT (a multiple of 64).  `red` is LDS
// scratch of NT/64 elements.  Fixed order: wave butterflies, then waves in
// index order.  All threads receive the result.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  __syncthreads();
  float s = red[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) s += red[i];
  return s;
}
template <int NT>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  __syncthreads();
  float s = red[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) s = fmaxf(s, red[i]);
  return s;
}
template <int NT>
__device__ __forceinline__ unsigned long long block_sum_u64(unsigned long long v, unsigned long long* red) {
  v = wave_sum_u64(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  __syncthreads();
  unsigned long long s = red[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) s += red[i];
  return s;
}

// RMSNorm of G consecutive residual rows (h [G][ld] -> out [G][ldo] in the
// model dtype; out may be global or LDS) by one workgroup of NT threads:
// x = cvt(h * rsqrt(mean(h^2) + eps) * g).  d % 4 == 0, d <= 4096,
// ld % 4 == 0.  In two halves: norm_issue puts every load of the rows in
// flight (16-byte loads, indexes clamped, surplus chunks weigh zero: one
// memory round trip), norm_commit reduces and writes, so a caller can issue
// other loads in between.  The sum of squares is taken in one fixed order
// whatever the workgroup size, so every RMSNorm of the library gives the
// same bits for the same row: the row is cut into blocks of 64 16-byte
// chunks (256 elements); in a block each lane adds the squares of its 4
// elements (one fma chain) and the wave adds its lanes by butterfly; the
// (at most 16) block sums are added by a 16-lane butterfly, zeros standing
// in for the blocks past the row (norm_scales).
constexpr int kNormBlocks = 16;  // blocks of a row of at most 4096 elements

// scale[g] = rsqrt(total_g / d + eps) in every lane, for rows g < G (<= 8),
// from the block sums red[b][g] (b < nblk <= 16).  Lanes 16k .. 16k + 15
// take the blocks of row g0 + k, four rows per pass: each wave computes a
// row's total and scale once per 16 lanes, not once per thread (the
// per-thread form kept the staging of a 5-row linear VALU-bound for ~3 us).
template <int G>
__device__ __forceinline__ void norm_scales(const float (*red)[8], int nblk, int d, float eps, float (&scale)[G]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int b = lane & 15, k = lane >> 4;
#pragma unroll
  for (int g0 = 0; g0 < G; g0 += 4) {
    const int g = g0 + k;
    float v = (g < G && b < nblk) ? red[b][g < G ? g : 0] : 0.f;
    v = group_sum<16>(v);
    const float sc = rsqrtf(v / static_cast<float>(d) + eps);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      if (g0 + kk < G)
        scale[g0 + kk] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc), 16 * kk));
  }
}
template <int NT, int G> struct NormRegs {
  static constexpr int CPT = (4 * 256 + NT - 1) / NT;  // 16-byte chunks per thread and row (d <= 4096)
  float4 v[G][CPT];
  float4 g[CPT];  // the gain's chunks (loaded with the rows: loads return in issue order)
};

template <int NT, int G>
__device__ __forceinline__ void norm_issue(const float* h, int ld, int d, const float* gain, NormRegs<NT, G>& r) {
  constexpr int CPT = NormRegs<NT, G>::CPT;
  const int d4 = d / 4;
  const int wbase = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) & ~(kWave - 1));
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    r.g[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (wbase + c * NT < d4)
      r.g[c] = reinterpret_cast<const float4*>(gain)[min(static_cast<int>(threadIdx.x) + c * NT, d4 - 1)];
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float4* hr = reinterpret_cast<const float4*>(h + static_cast<size_t>(g) * ld);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      // whole waves past the row issue nothing (their chunks weigh zero)
      if (wbase + c * NT < d4) {
        const int e4 = min(static_cast<int>(threadIdx.x) + c * NT, d4 - 1);
        r.v[g][c] = hr[e4];
      } else {
        r.v[g][c] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  }
}

// o[0..3] = cvt(v * scale * g) as one 8-byte (bf16) or 16-byte store; o is
// aligned to it.
template <typename OT>
__device__ __forceinline__ void store4(OT* o, const float4& v, float scale, const float4& g) {
  if constexpr (sizeof(OT) == 2) {
    uint2 pk;
    pk.x = static_cast<uint32_t>(f2bf(v.x * scale * g.x)) | (static_cast<uint32_t>(f2bf(v.y * scale * g.y)) << 16);
    pk.y = static_cast<uint32_t>(f2bf(v.z * scale * g.z)) | (static_cast<uint32_t>(f2bf(v.w * scale * g.w)) << 16);
    *reinterpret_cast<uint2*>(o) = pk;
  } else {
    *reinterpret_cast<float4*>(o) = make_float4(v.x * scale * g.x, v.y * scale * g.y, v.z * scale * g.z, v.w * scale * g.w);
  }
}

template <int NT, int G, typename OT>
__device__ __forceinline__ void norm_commit(const NormRegs<NT, G>& r, int d, float eps, OT* out, int ldo,
                                            float (*red)[8]) {
  constexpr int CPT = NormRegs<NT, G>::CPT;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int d4 = d / 4, nblk = (d4 + kWave - 1) / kWave;
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      if (wave * kWave + c * NT < d4) {  // the wave holds block c * NT / 64 + wave
        float ss = 0.f;
        if (static_cast<int>(threadIdx.x) + c * NT < d4) {
          ss = fmaf(r.v[g][c].x, r.v[g][c].x, ss);
          ss = fmaf(r.v[g][c].y, r.v[g][c].y, ss);
          ss = fmaf(r.v[g][c].z, r.v[g][c].z, ss);
          ss = fmaf(r.v[g][c].w, r.v[g][c].w, ss);
        }
        ss = wave_sum(ss);
        if (lane == 0) red[c * (NT / kWave) + wave][g] = ss;
      }
    }
  }
  __syncthreads();
  float scale[G];
  norm_scales<G>(red, nblk, d, eps, scale);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    OT* o = out + static_cast<size_t>(g) * ldo;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int e4 = threadIdx.x + c * NT;
      if (e4 < d4) store4<OT>(o + 4 * e4, r.v[g][c], scale[g], r.g[c]);
    }
  }
  __syncthreads();
}

template <int NT, int G, typename OT>
__device__ __forceinline__ void norm_group(const float* h, int ld, int d, const float* gain, float eps, OT* out,
                                           int ldo, float (*red)[8]) {
  NormRegs<NT, G> r;
  norm_issue<NT, G>(h, ld, d, gain, r);
  norm_commit<NT, G>(r, d, eps, out, ldo, red);
}

// RMSNorm of M (1..8, a compile-time count) rows: one round trip for M <= 5,
// two otherwise (rows 0-3, then the rest).  Output row stride ldo.
template <int NT, int M, typename OT>
__device__ __forceinline__ void norm_rows(const float* h, int ld, int d, const float* gain, float eps, OT* out,
                                          int ldo) {
  static_assert(M >= 1 && M <= 8, "1..8 rows");
  __shared__ float red_nr[kNormBlocks][8];
  if constexpr (M <= 5) {
    norm_group<NT, M, OT>(h, ld, d, gain, eps, out, ldo, red_nr);
  } else {
    norm_group<NT, 4, OT>(h, ld, d, gain, eps, out, ldo, red_nr);
    norm_group<NT, M - 4, OT>(h + 4 * static_cast<size_t>(ld), ld, d, gain, eps, out + 4 * static_cast<size_t>(ldo),
                                  ldo, red_nr);
  }
}

// True in exactly one of the n workgroups that arrive at `ticket`: the last
// (which resets it to zero).  Writes made before the call by all n are
// visible to that workgroup afterwards.  Every wave first drains its own
// stores (vmcnt(0): the workgroup barrier alone does not wait for global
// stores); then one thread per workgroup publishes with an agent-scope
// release, and only the last workgroup acquires.
__device__ __forceinline__ bool last_block(int* ticket, int n, int* flag_sh) {
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev == n - 1;
    if (last) {
      __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    *flag_sh = last;
  }
  __syncthreads();
  return *flag_sh;
}

}  // namespace sv
