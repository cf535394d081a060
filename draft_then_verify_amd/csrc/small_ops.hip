// Small ops of the verify pass: the embedding gather (+ the RoPE angle table
// of the pass) and KV length bookkeeping.  They move kilobytes.
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
  norm_rows<kThreads, 1>(dst, d, d, gain, eps, x + static_cast<size_t>(r) * d);
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

hipError_t launch_kv_len(int32_t* len, const int32_t* src, int add, int B, hipStream_t s) {
  hipLaunchKernelGGL(kv_len_kernel, dim3((B + 255) / 256), dim3(256), 0, s, len, src, add, B);
  return hipGetLastError();
}

}  // namespace sv
