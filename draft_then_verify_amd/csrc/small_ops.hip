// Small ops of the verify pass: the embedding gather (+ the RoPE angle table
// of the pass), the residual sum + RMSNorm between linears, round and KV
// length bookkeeping, and the n-gram prompt lookup.  They move kilobytes.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace sv {
namespace {

constexpr int kThreads = 256;

// Verify input assembly and gather: row r = b*m + i of the pass takes
// [last committed token, x_1 .. x_gamma] (first page, Algorithm 1: the target
// runs on prefix, prefix + [x_1], ..., prefix + [x_1 .. x_gamma]).
template <typename ET>
__global__ __launch_bounds__(kThreads) void embed_kernel(const ET* __restrict__ E, int vocab, int d,
                                                         const int32_t* __restrict__ tokens,
                                                         const int32_t* __restrict__ last,
                                                         const int32_t* __restrict__ draft,
                                                         const int32_t* __restrict__ len, int m, int hd,
                                                         float theta, const float* __restrict__ gain, float eps,
                                                         float* __restrict__ h, ET* __restrict__ x,
                                                         float2* __restrict__ cs, int* __restrict__ ctr, int n_ctr) {
  const int r = blockIdx.x;
  const int b = r / m, i = r - b * m;
  for (int c = r * kThreads + threadIdx.x; c < n_ctr; c += gridDim.x * kThreads) ctr[c] = 0;
  int tok = tokens ? tokens[r] : (i == 0 ? last[b] : draft[b * (m - 1) + i - 1]);
  tok = min(max(tok, 0), vocab - 1);
  const ET* src = E + static_cast<size_t>(tok) * d;
  float* dst = h + static_cast<size_t>(r) * d;
#pragma unroll 4
  for (int j = threadIdx.x; j < d; j += kThreads) dst[j] = Elt<ET>::load(src + j);
  __syncthreads();
  if (x) norm_rows<kThreads, 1>(dst, d, d, gain, eps, x + static_cast<size_t>(r) * d, d);
  // RoPE angles in double precision, rounded once to float.
  const int half = hd / 2;
  if (threadIdx.x < half) {
    const int j = threadIdx.x;
    const double pos = static_cast<double>(len[b] + i);
    const double inv_freq = pow(static_cast<double>(theta), -2.0 * j / hd);
    double sn, cn;
    sincos(pos * inv_freq, &sn, &cn);
    cs[static_cast<size_t>(r) * half + j] = make_float2(static_cast<float>(cn), static_cast<float>(sn));
  }
}

// One row per workgroup: h += (part[0] + ... + part[KS-1]) (slices summed in
// order first), then x = cvt(RMSNorm(h) * gain).  Every load of the row is
// issued before any is used: one memory round trip.
template <typename OT, int KS>
__global__ __launch_bounds__(kThreads) void resid_norm_kernel(float* __restrict__ h, const float* __restrict__ part,
                                                              size_t pstride, int d, const float* __restrict__ gain,
                                                              float eps, OT* __restrict__ x) {
  constexpr int CPT = 4;  // 16-byte chunks per thread (d <= 16 * 256)
  static_assert(CPT * kThreads / kWave == kNormBlocks, "one sum per block of the row");
  __shared__ float red[kNormBlocks][8];
  const size_t r = blockIdx.x;
  const int d4 = d / 4;
  float4* hr = reinterpret_cast<float4*>(h + r * d);
  float4 v[CPT], pv[KS][CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int e4 = min(static_cast<int>(threadIdx.x) + c * kThreads, d4 - 1);
    v[c] = hr[e4];
#pragma unroll
    for (int k = 0; k < KS; ++k) pv[k][c] = reinterpret_cast<const float4*>(part + k * pstride + r * d)[e4];
  }
  // sum of squares in the fixed block order of norm_commit (common.hpp)
  const int wave = threadIdx.x / kWave, nblk = (d4 + kWave - 1) / kWave;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    float4 acc = pv[0][c];
#pragma unroll
    for (int k = 1; k < KS; ++k) {
      acc.x += pv[k][c].x;
      acc.y += pv[k][c].y;
      acc.z += pv[k][c].z;
      acc.w += pv[k][c].w;
    }
    v[c].x += acc.x;
    v[c].y += acc.y;
    v[c].z += acc.z;
    v[c].w += acc.w;
    if (wave * kWave + c * kThreads < d4) {
      float ss = 0.f;
      if (static_cast<int>(threadIdx.x) + c * kThreads < d4) {
        hr[threadIdx.x + c * kThreads] = v[c];
        ss = fmaf(v[c].x, v[c].x, ss);
        ss = fmaf(v[c].y, v[c].y, ss);
        ss = fmaf(v[c].z, v[c].z, ss);
        ss = fmaf(v[c].w, v[c].w, ss);
      }
      ss = wave_sum(ss);
      if ((threadIdx.x & (kWave - 1)) == 0) red[c * (kThreads / kWave) + wave][0] = ss;
    }
  }
  __syncthreads();
  float sc[1];
  norm_scales<1>(red, nblk, d, eps, sc);
  const float scale = sc[0];
  OT* o = x + r * d;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int e4 = threadIdx.x + c * kThreads;
    if (e4 < d4) store4<OT>(o + 4 * e4, v[c], scale, reinterpret_cast<const float4*>(gain)[e4]);
  }
}

template <typename OT>
hipError_t launch_resid_norm_t(float* h, const float* part, int ks, size_t pstride, int rows, int d,
                               const float* gain, float eps, OT* x, hipStream_t s) {
  const dim3 g(rows), b(kThreads);
  switch (ks) {
    case 1: hipLaunchKernelGGL((resid_norm_kernel<OT, 1>), g, b, 0, s, h, part, pstride, d, gain, eps, x); break;
    case 2: hipLaunchKernelGGL((resid_norm_kernel<OT, 2>), g, b, 0, s, h, part, pstride, d, gain, eps, x); break;
    case 3: hipLaunchKernelGGL((resid_norm_kernel<OT, 3>), g, b, 0, s, h, part, pstride, d, gain, eps, x); break;
    case 4: hipLaunchKernelGGL((resid_norm_kernel<OT, 4>), g, b, 0, s, h, part, pstride, d, gain, eps, x); break;
    case 5: hipLaunchKernelGGL((resid_norm_kernel<OT, 5>), g, b, 0, s, h, part, pstride, d, gain, eps, x); break;
    case 6: hipLaunchKernelGGL((resid_norm_kernel<OT, 6>), g, b, 0, s, h, part, pstride, d, gain, eps, x); break;
    case 7: hipLaunchKernelGGL((resid_norm_kernel<OT, 7>), g, b, 0, s, h, part, pstride, d, gain, eps, x); break;
    case 8: hipLaunchKernelGGL((resid_norm_kernel<OT, 8>), g, b, 0, s, h, part, pstride, d, gain, eps, x); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Round bookkeeping on the device: append x_1 .. x_n, t to each sequence's
// output and make (x_n or the old last token, t) the next round's inputs.
__global__ void commit_round_kernel(int B, int gamma, const int32_t* __restrict__ n_acc,
                                    const int32_t* __restrict__ emitted, int32_t* __restrict__ tok2,
                                    int32_t* __restrict__ last, int32_t* __restrict__ out, int32_t* __restrict__ out_len,
                                    int cap, int n_stop, int32_t* __restrict__ kv_len, int32_t* __restrict__ n_rounds,
                                    int32_t* __restrict__ n_log, int log_cap) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int n = min(max(n_acc[b], 0), gamma);
  const int len = out_len[b];
  if (n_stop > 0 && len >= n_stop) {
    // finished before this round: discard the round and undo its KV commit
    if (kv_len) kv_len[b] -= n + 1;
    return;
  }
  const int32_t* em = emitted + static_cast<size_t>(b) * (gamma + 1);
  for (int i = 0; i <= n; ++i)
    if (len + i < cap) out[static_cast<size_t>(b) * cap + len + i] = em[i];
  out_len[b] = len + n + 1;
  const int32_t t = em[n];
  const int32_t prev = n > 0 ? em[n - 1] : tok2[2 * b + 1];
  tok2[2 * b] = prev;
  tok2[2 * b + 1] = t;
  if (last) last[b] = t;
  if (n_rounds) {
    const int r = n_rounds[b];
    if (n_log && r < log_cap) n_log[static_cast<size_t>(b) * log_cap + r] = n;
    n_rounds[b] = r + 1;
  }
}

// Prompt lookup, one workgroup per sequence: for a match length n every
// thread tests its share of the candidate starts (the n tokens at s equal the
// context's last n, s <= L - n - 1), the block keeps the largest such s, and
// the tokens after it are the proposal (the n-gram drafter of the second
// page, section "The three proposers").  The lengths are tried from n_max
// down to n_min and the first that occurs is taken (the match window of the
// same page, section "Dial It In").  The context is the prefix row followed
// by the tokens committed since.
constexpr int kNgramThreads = 256;
__global__ __launch_bounds__(kNgramThreads) void ngram_kernel(int n_min, int n_max, int gamma, const int32_t* __restrict__ prefix,
                                                              const int32_t* __restrict__ prefix_len, int P,
                                                              const int32_t* __restrict__ out,
                                                              const int32_t* __restrict__ out_len, int cap,
                                                              const int32_t* __restrict__ fill_off,
                                                              int32_t* __restrict__ drafts,
                                                              int32_t* __restrict__ n_draft,
                                                              int32_t* __restrict__ n_found) {
  __shared__ int best_w[kNgramThreads / kWave];
  __shared__ int key[16];
  const int b = blockIdx.x;
  const int lp = prefix_len ? min(max(prefix_len[b], 0), P) : P;
  const int lo = cap > 0 ? min(max(out_len[b], 0), cap) : 0;
  const int L = lp + lo;
  const int32_t* pre = prefix + static_cast<size_t>(b) * P;
  const int32_t* post = cap > 0 ? out + static_cast<size_t>(b) * cap : nullptr;
  auto tok = [&](int i) { return i < lp ? pre[i] : post[i - lp]; };
  int best = -1, n = n_min;
  // L and the block maximum are the same in every thread, so every thread
  // takes the same trips and the barriers below match.  The barrier after
  // the key is written also keeps the next trip's best_w writes behind the
  // last reads of this trip's.
  for (int nn = n_max; gamma > 0 && nn >= n_min; --nn) {
    if (L < nn + 1) continue;
    if (static_cast<int>(threadIdx.x) < nn) key[threadIdx.x] = tok(L - nn + threadIdx.x);
    __syncthreads();
    int cand = -1;
    for (int s = threadIdx.x; s <= L - nn - 1; s += kNgramThreads) {
      bool eq = true;
      for (int j = 0; j < nn && eq; ++j) eq = tok(s + j) == key[j];
      if (eq) cand = max(cand, s);
    }
    // block max of cand, waves in order
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) cand = max(cand, __shfl_xor(cand, off, kWave));
    if ((threadIdx.x & (kWave - 1)) == 0) best_w[threadIdx.x / kWave] = cand;
    __syncthreads();
    cand = best_w[0];
#pragma unroll
    for (int w = 1; w < kNgramThreads / kWave; ++w) cand = max(cand, best_w[w]);
    if (cand >= 0) {
      best = cand;
      n = nn;
      break;
    }
  }
  const int found = best >= 0 ? min(gamma, L - (best + n)) : 0;
  const int total = fill_off ? gamma : found;
  for (int i = threadIdx.x; i < gamma; i += kNgramThreads) {
    int32_t v = -1;
    if (i < found) {
      v = tok(best + n + i);
    } else if (fill_off) {
      v = pre[min(max(fill_off[b] + (i - found), 0), P - 1)];
    }
    drafts[static_cast<size_t>(b) * gamma + i] = v;
  }
  if (threadIdx.x == 0) {
    n_draft[b] = total;
    if (n_found) n_found[b] = found;
  }
}

__global__ void kv_len_kernel(int32_t* len, const int32_t* src, int add, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) len[b] = (src ? src[b] : len[b]) + add;
}

}  // namespace

hipError_t launch_embed(bool bf16, const void* embed, int vocab, int d, const int32_t* tokens, const int32_t* last,
                        const int32_t* draft, const int32_t* len, int B, int m, int hd, float theta,
                        const float* gain, float eps, float* h, void* x, float2* cs, int* ctr, int n_ctr,
                        hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(embed_kernel<uint16_t>, dim3(B * m), dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(embed), vocab, d, tokens, last, draft, len, m, hd, theta, gain,
                       eps, h, static_cast<uint16_t*>(x), cs, ctr, n_ctr);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(B * m), dim3(kThreads), 0, s, static_cast<const float*>(embed),
                       vocab, d, tokens, last, draft, len, m, hd, theta, gain, eps, h, static_cast<float*>(x), cs,
                       ctr, n_ctr);
  return hipGetLastError();
}

hipError_t launch_resid_norm(bool bf16, float* h, const float* part, int ks, size_t pstride, int rows, int d,
                             const float* gain, float eps, void* x, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (d % 4 != 0 || d > 16 * kThreads || pstride % 4 != 0) return hipErrorInvalidValue;
  if (bf16) return launch_resid_norm_t(h, part, ks, pstride, rows, d, gain, eps, static_cast<uint16_t*>(x), s);
  return launch_resid_norm_t(h, part, ks, pstride, rows, d, gain, eps, static_cast<float*>(x), s);
}

hipError_t launch_commit_round(int B, int gamma, const int32_t* n_acc, const int32_t* emitted, int32_t* tok2,
                               int32_t* last, int32_t* out, int32_t* out_len, int cap, int n_stop, int32_t* kv_len,
                               int32_t* n_rounds, int32_t* n_log, int log_cap, hipStream_t s) {
  hipLaunchKernelGGL(commit_round_kernel, dim3((B + 255) / 256), dim3(256), 0, s, B, gamma, n_acc, emitted, tok2,
                     last, out, out_len, cap, n_stop, kv_len, n_rounds, n_log, log_cap);
  return hipGetLastError();
}

hipError_t launch_ngram(int B, int n_min, int n_max, int gamma, const int32_t* prefix, const int32_t* prefix_len, int P,
                        const int32_t* out, const int32_t* out_len, int cap, const int32_t* fill_off,
                        int32_t* drafts, int32_t* n_draft, int32_t* n_found, hipStream_t s) {
  hipLaunchKernelGGL(ngram_kernel, dim3(B), dim3(kNgramThreads), 0, s, n_min, n_max, gamma, prefix, prefix_len, P, out, out_len,
                     cap, fill_off, drafts, n_draft, n_found);
  return hipGetLastError();
}

// ---- validation (SPEC_CHECK=1) ----------------------------------------------------
// flag |= 1: a token id outside [0, vocab); flag |= 2: a non-finite value.
__global__ void check_clear_kernel(int* flag) { *flag = 0; }

__global__ void check_ids_kernel(const int32_t* __restrict__ ids, int rows, int per_row,
                                 const int32_t* __restrict__ n_valid, int vocab, int* flag) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(rows) * per_row) return;
  const int r = static_cast<int>(i / per_row), c = static_cast<int>(i - static_cast<int64_t>(r) * per_row);
  const int n = n_valid ? min(max(n_valid[r], 0), per_row) : per_row;
  const int32_t t = ids[i];
  if (c < n && (t < 0 || t >= vocab)) __hip_atomic_fetch_or(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void check_finite_kernel(const float* __restrict__ v, int64_t n, int* flag) {
  bool bad = false;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    bad |= !isfinite(v[i]);
  if (__ballot(bad) && (threadIdx.x & (kWave - 1)) == 0)
    __hip_atomic_fetch_or(flag, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_check_clear(int* flag, hipStream_t s) {
  hipLaunchKernelGGL(check_clear_kernel, dim3(1), dim3(1), 0, s, flag);
  return hipGetLastError();
}

hipError_t launch_check_ids(const int32_t* ids, int rows, int per_row, const int32_t* n_valid, int vocab, int* flag,
                            hipStream_t s) {
  const int64_t n = static_cast<int64_t>(rows) * per_row;
  if (n <= 0 || !ids) return hipSuccess;
  hipLaunchKernelGGL(check_ids_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, ids, rows,
                     per_row, n_valid, vocab, flag);
  return hipGetLastError();
}

hipError_t launch_check_finite(const float* v, int64_t n, int* flag, hipStream_t s) {
  if (n <= 0 || !v) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(check_finite_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, v, n, flag);
  return hipGetLastError();
}

hipError_t launch_kv_len(int32_t* len, const int32_t* src, int add, int B, hipStream_t s) {
  hipLaunchKernelGGL(kv_len_kernel, dim3((B + 255) / 256), dim3(256), 0, s, len, src, add, B);
  return hipGetLastError();
}

}  // namespace sv
