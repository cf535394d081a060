// Softmax statistics of logit rows in 128-column tiles, shared by the
// matrix-core LM head (which produces them in its epilogue, so the logits of
// a large pass need not be written) and the sampler (which produces the same
// bits from materialised logits).
//
// The target's distribution over the vocabulary is p = softmax(l / T)
// ("How Speculative Decoding Works (and When It Doesn't)", section "Why the
// output doesn't change": p and q are the two models' next-token
// distributions).  A row's statistics are built bottom-up, in a fixed order:
//   * tile (128 columns, c0 .. c0+127): v = l / T (-inf past the vocabulary);
//     M_t = max v; column c0 + 64 h + 16 j + c belongs to lane c of a 16-lane
//     group for half h, slot j.  Each lane sums e = exp(v - M_t) over its
//     four slots in slot order, the 16 lanes are summed by the DPP butterfly
//     (a balanced tree), and Z_t = Z_half0 + Z_half1;
//   * chunk (4096 columns = 32 tiles): M_c = max M_t, Z_c = sum over tiles in
//     order of Z_t exp(M_t - M_c) (fused multiply-add);
//   * row: the chunk pairs merged by wave_stats in the sampler.
// Every producer follows these steps, so the statistics -- and every
// p(v) = exp(l_v / T - M) / Z -- are bitwise the same whichever kernel made them.
#pragma once

#include <math.h>

#include "common.hpp"

namespace sv {
namespace lmstat {

constexpr int kTile = 128;
constexpr int kTilesPerChunk = 32;  // 4096-entry sampler chunks

__device__ __forceinline__ float group16_max(float v) {
  v = fmaxf(v, dpp_mov<kDppQuadSwap1>(v));
  v = fmaxf(v, dpp_mov<kDppQuadSwap2>(v));
  v = fmaxf(v, dpp_mov<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_mov<kDppMirror>(v));
  return v;
}

// exp(v - M) of one column; a column at -inf weighs zero
__device__ __forceinline__ float col_exp(float v, float M) { return v == -INFINITY ? 0.f : expf(__fsub_rn(v, M)); }

// A lane's sum over its four slots, in slot order.
__device__ __forceinline__ float slot_sum(const float (&v)[4], float M) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += col_exp(v[j], M);
  return s;
}

// (M_c, Z_c) of a chunk from its tiles' (M_t, Z_t), tiles in order.
__device__ __forceinline__ float2 merge_tiles(const float2* t, int n) {
  float M = -INFINITY;
  for (int i = 0; i < n; ++i) M = fmaxf(M, t[i].x);
  float Z = 0.f;
  for (int i = 0; i < n; ++i)
    if (t[i].y != 0.f) Z = fmaf(t[i].y, expf(__fsub_rn(t[i].x, M)), Z);
  return make_float2(M, Z);
}

// Greedy statistics: (value, lowest index) of the largest entry; any merge
// order gives the same pair (larger value, then lower index, is a total order
// on non-NaN values; a NaN is never selected).
__device__ __forceinline__ void argmax_merge(float& m, int& i, float m2, int i2) {
  if (m2 > m || (m2 == m && i2 < i)) {
    m = m2;
    i = i2;
  }
}

__device__ __forceinline__ void group16_argmax(float& m, int& i) {
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off, kWave);
    const int i2 = __shfl_xor(i, off, kWave);
    argmax_merge(m, i, m2, i2);
  }
}

}  // namespace lmstat
}  // namespace sv
