// Attention of the verify pass: m query rows per sequence (the last committed
// token and the gamma drafts) against the sequence's KV cache.
//
// The pages: "the cache read serves every query position" (first page,
// section "The speedup is borrowed"), and decode-time attention stays
// memory-bound, its KV traffic growing with context and batch ("How
// Speculative Decoding Works", section "Prefill and Decode").  So one
// workgroup reads each K/V tile once for all G*m query rows of a KV head
// (G = H / Hkv query heads share it), with the tile staged in LDS.  At B = 1
// there are only Hkv (b, kv-head) pairs, so the context is split across
// workgroups and the partial (max, sum, output) rows are merged afterwards
// in a fixed order (log-sum-exp combine) -- deterministic, no atomics.
//
// Causality inside the new block: query row i sits at position len + i and
// sees keys 0 .. len + i.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int QT = 32;  // query rows per workgroup tile
constexpr int KT = 32;  // keys per LDS tile

// Rotate-half RoPE of q (in place) and k; k and v rows go to the cache at
// position len[b] + i.  Row r = b*m + i.
template <typename ET>
__global__ __launch_bounds__(kThreads) void rope_append_kernel(float* __restrict__ qkv, const float2* __restrict__ cs,
                                                               const int32_t* __restrict__ len, int m, int H, int Hkv,
                                                               int hd, ET* __restrict__ kc, ET* __restrict__ vc,
                                                               int layer, int kvB, int max_ctx) {
  const int r = blockIdx.x;
  const int b = r / m, i = r - b * m;
  const int pos = len[b] + i;
  const bool store = pos >= 0 && pos < max_ctx;
  const int half = hd / 2;
  const int ld = (H + 2 * Hkv) * hd;
  float* row = qkv + static_cast<size_t>(r) * ld;
  const float2* csr = cs + static_cast<size_t>(r) * half;
  const size_t cache_row = ((static_cast<size_t>(layer) * kvB + b) * Hkv) * max_ctx + (store ? pos : 0);
  for (int idx = threadIdx.x; idx < (H + Hkv) * half; idx += kThreads) {
    const int hh = idx / half, j = idx - hh * half;
    const float x1 = row[hh * hd + j], x2 = row[hh * hd + j + half];
    const float2 c = csr[j];
    const float y1 = x1 * c.x - x2 * c.y;
    const float y2 = x2 * c.x + x1 * c.y;
    if (hh < H) {
      row[hh * hd + j] = y1;
      row[hh * hd + j + half] = y2;
    } else if (store) {
      ET* dst = kc + (cache_row + static_cast<size_t>(hh - H) * max_ctx) * hd;
      dst[j] = Elt<ET>::from_f(y1);
      dst[j + half] = Elt<ET>::from_f(y2);
    }
  }
  if (store) {
    const float* vrow = row + (H + Hkv) * hd;
    for (int idx = threadIdx.x; idx < Hkv * hd; idx += kThreads) {
      const int kvh = idx / hd, dd = idx - kvh * hd;
      vc[(cache_row + static_cast<size_t>(kvh) * max_ctx) * hd + dd] = Elt<ET>::from_f(vrow[idx]);
    }
  }
}

// grid: x = b * Hkv + kvh, y = context split, z = query tile.
// Thread t: local query row t / 8, sub-lane t % 8 (scores for keys sub*4 ..
// sub*4+3 of a tile; output dims sub + 8*k).
template <typename ET, int HD>
__global__ __launch_bounds__(kThreads) void attn_partial_kernel(const float* __restrict__ qkv, const ET* __restrict__ kc,
                                                                const ET* __restrict__ vc, const int32_t* __restrict__ len,
                                                                int m, int H, int Hkv, int layer, int kvB, int max_ctx,
                                                                int n_split, float* __restrict__ part_o,
                                                                float2* __restrict__ part_ml) {
  constexpr int DPT = HD / 8;
  __shared__ float qs[QT][HD + 1];
  __shared__ float ks[KT][HD + 1];
  __shared__ float vs[KT][HD + 1];
  __shared__ float ps[QT][KT + 1];

  const int G = H / Hkv;
  const int b = blockIdx.x / Hkv, kvh = blockIdx.x - b * Hkv;
  const int s = blockIdx.y, qt = blockIdx.z;
  const int nq = G * m;
  const int t = threadIdx.x;
  const int row = t >> 3, sub = t & 7;
  const int qr = qt * QT + row;
  const bool row_valid = qr < nq;
  const int g = row_valid ? qr / m : 0;
  const int i = row_valid ? qr - g * m : 0;
  const int h = kvh * G + g;
  const int Lb = len[b];
  const int n_keys = max(0, min(Lb + m, max_ctx));
  const int per = (n_keys + n_split - 1) / n_split;
  const int kbeg = s * per;
  const int kend = min(kbeg + per, n_keys);
  const int lim = Lb + i;
  const int qkv_ld = (H + 2 * Hkv) * HD;
  const float scale = 1.0f / sqrtf(static_cast<float>(HD));

  for (int idx = t; idx < QT * HD; idx += kThreads) {
    const int rr = idx / HD, dd = idx - rr * HD;
    const int q2 = qt * QT + rr;
    float v = 0.f;
    if (q2 < nq) {
      const int g2 = q2 / m, i2 = q2 - g2 * m;
      v = qkv[static_cast<size_t>(b * m + i2) * qkv_ld + (kvh * G + g2) * HD + dd] * scale;
    }
    qs[rr][dd] = v;
  }

  float mrow = -INFINITY, lrow = 0.f;
  float acc[DPT];
#pragma unroll
  for (int k = 0; k < DPT; ++k) acc[k] = 0.f;
  const size_t kvbase = ((static_cast<size_t>(layer) * kvB + b) * Hkv + kvh) * max_ctx;

  for (int k0 = kbeg; k0 < kend; k0 += KT) {
    __syncthreads();
    for (int idx = t; idx < KT * HD; idx += kThreads) {
      const int jj = idx / HD, dd = idx - jj * HD;
      const int j = k0 + jj;
      float kv = 0.f, vv = 0.f;
      if (j < kend) {
        kv = Elt<ET>::load(kc + (kvbase + j) * HD + dd);
        vv = Elt<ET>::load(vc + (kvbase + j) * HD + dd);
      }
      ks[jj][dd] = kv;
      vs[jj][dd] = vv;
    }
    __syncthreads();
    float sc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int jj = sub * 4 + c;
      float a = 0.f;
#pragma unroll 8
      for (int dd = 0; dd < HD; ++dd) a = fmaf(qs[row][dd], ks[jj][dd], a);
      const int j = k0 + jj;
      sc[c] = (row_valid && j < kend && j <= lim) ? a : -INFINITY;
    }
    float tmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 1, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 2, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 4, kWave));
    const float mnew = fmaxf(mrow, tmax);
    const float alpha = (mnew == -INFINITY) ? 1.f : expf(mrow - mnew);
    float psum = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float p = (sc[c] == -INFINITY) ? 0.f : expf(sc[c] - mnew);
      ps[row][sub * 4 + c] = p;
      psum += p;
    }
    psum += __shfl_xor(psum, 1, kWave);
    psum += __shfl_xor(psum, 2, kWave);
    psum += __shfl_xor(psum, 4, kWave);
    lrow = lrow * alpha + psum;
    mrow = mnew;
#pragma unroll
    for (int k = 0; k < DPT; ++k) acc[k] *= alpha;
    __syncthreads();
    for (int jj = 0; jj < KT; ++jj) {
      const float p = ps[row][jj];
#pragma unroll
      for (int k = 0; k < DPT; ++k) acc[k] = fmaf(p, vs[jj][sub + 8 * k], acc[k]);
    }
  }
  if (row_valid) {
    const size_t prow = ((static_cast<size_t>(b) * H + h) * m + i) * n_split + s;
    if (sub == 0) part_ml[prow] = make_float2(mrow, lrow);
#pragma unroll
    for (int k = 0; k < DPT; ++k) part_o[prow * HD + sub + 8 * k] = acc[k];
  }
}

// One block per (row r = b*m + i, head h); HD threads.  Fixed split order.
template <typename XT, int HD>
__global__ __launch_bounds__(HD) void attn_combine_kernel(const float* __restrict__ part_o,
                                                          const float2* __restrict__ part_ml, int m, int H, int n_split,
                                                          XT* __restrict__ x) {
  const int idx = blockIdx.x;
  const int h = idx % H, r = idx / H;
  const int b = r / m, i = r - b * m;
  const int d = threadIdx.x;
  const size_t prow0 = ((static_cast<size_t>(b) * H + h) * m + i) * n_split;
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, part_ml[prow0 + s].x);
  float l = 0.f, o = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const float2 ml = part_ml[prow0 + s];
    const float w = (ml.x == -INFINITY) ? 0.f : expf(ml.x - M);
    l = fmaf(ml.y, w, l);
    o = fmaf(part_o[(prow0 + s) * HD + d], w, o);
  }
  x[static_cast<size_t>(r) * (H * HD) + h * HD + d] = Elt<XT>::from_f(l > 0.f ? o / l : 0.f);
}

template <typename ET, int HD>
hipError_t attention_typed(const float* qkv, const ET* kc, const ET* vc, const int32_t* len, int B, int m, int H,
                           int Hkv, int layer, int kvB, int max_ctx, int n_split, float* part_o, float2* part_ml,
                           ET* x, hipStream_t s) {
  const int G = H / Hkv;
  dim3 grid(B * Hkv, n_split, (G * m + QT - 1) / QT);
  hipLaunchKernelGGL((attn_partial_kernel<ET, HD>), grid, dim3(kThreads), 0, s, qkv, kc, vc, len, m, H, Hkv, layer,
                     kvB, max_ctx, n_split, part_o, part_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_combine_kernel<ET, HD>), dim3(B * m * H), dim3(HD), 0, s, part_o, part_ml, m, H, n_split,
                     x);
  return hipGetLastError();
}

}  // namespace

int attn_num_splits(int B, int Hkv, int G, int m, int max_ctx) {
  const int units = B * Hkv * ((G * m + QT - 1) / QT);
  int n = (512 + units - 1) / units;
  n = min(n, max(1, max_ctx / (2 * KT)));
  return max(1, min(n, 32));
}

hipError_t launch_rope_append(bool bf16, float* qkv, const float2* cs, const int32_t* len, int B, int m, int H, int Hkv,
                              int hd, void* kc, void* vc, int layer, int kvB, int max_ctx, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(rope_append_kernel<uint16_t>, dim3(B * m), dim3(kThreads), 0, s, qkv, cs, len, m, H, Hkv, hd,
                       static_cast<uint16_t*>(kc), static_cast<uint16_t*>(vc), layer, kvB, max_ctx);
  else
    hipLaunchKernelGGL(rope_append_kernel<float>, dim3(B * m), dim3(kThreads), 0, s, qkv, cs, len, m, H, Hkv, hd,
                       static_cast<float*>(kc), static_cast<float*>(vc), layer, kvB, max_ctx);
  return hipGetLastError();
}

hipError_t launch_attention(bool bf16, const float* qkv, const void* kc, const void* vc, const int32_t* len, int B,
                            int m, int H, int Hkv, int hd, int layer, int kvB, int max_ctx, int n_split, float* part_o,
                            float2* part_ml, void* x, hipStream_t s) {
  if (bf16) {
    const uint16_t *k = static_cast<const uint16_t*>(kc), *v = static_cast<const uint16_t*>(vc);
    uint16_t* xx = static_cast<uint16_t*>(x);
    return hd == 128 ? attention_typed<uint16_t, 128>(qkv, k, v, len, B, m, H, Hkv, layer, kvB, max_ctx, n_split,
                                                      part_o, part_ml, xx, s)
                     : attention_typed<uint16_t, 64>(qkv, k, v, len, B, m, H, Hkv, layer, kvB, max_ctx, n_split,
                                                     part_o, part_ml, xx, s);
  }
  const float *k = static_cast<const float*>(kc), *v = static_cast<const float*>(vc);
  float* xx = static_cast<float*>(x);
  return hd == 128 ? attention_typed<float, 128>(qkv, k, v, len, B, m, H, Hkv, layer, kvB, max_ctx, n_split, part_o,
                                                 part_ml, xx, s)
                   : attention_typed<float, 64>(qkv, k, v, len, B, m, H, Hkv, layer, kvB, max_ctx, n_split, part_o,
                                                part_ml, xx, s);
}

}  // namespace sv
