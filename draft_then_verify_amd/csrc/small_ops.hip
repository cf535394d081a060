// Row-wise small ops of the verify pass: embedding gather (+ the RoPE angle
// table of the pass), RMSNorm producing the next linear's input, and KV
// length bookkeeping.  All are one workgroup per row; they move kilobytes.
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
                                                         float theta, float* __restrict__ h, float2* __restrict__ cs) {
  const int r = blockIdx.x;
  const int b = r / m, i = r - b * m;
  int tok = tokens ? tokens[r] : (i == 0 ? last[b] : draft[b * (m - 1) + i - 1]);
  tok = min(max(tok, 0), vocab - 1);
  const ET* src = E + static_cast<size_t>(tok) * d;
  float* dst = h + static_cast<size_t>(r) * d;
  for (int j = threadIdx.x; j < d; j += kThreads) dst[j] = Elt<ET>::load(src + j);
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

template <typename XT>
__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(const float* __restrict__ h, const float* __restrict__ g,
                                                           int d, float eps, XT* __restrict__ x) {
  __shared__ float red[kThreads / kWave];
  const int r = blockIdx.x;
  const float* hr = h + static_cast<size_t>(r) * d;
  float ss = 0.f;
  for (int j = threadIdx.x; j < d; j += kThreads) ss = fmaf(hr[j], hr[j], ss);
  ss = block_sum<kThreads>(ss, red);
  const float scale = rsqrtf(ss / static_cast<float>(d) + eps);
  XT* xr = x + static_cast<size_t>(r) * d;
  for (int j = threadIdx.x; j < d; j += kThreads) xr[j] = Elt<XT>::from_f(hr[j] * scale * g[j]);
}

__global__ void kv_len_kernel(int32_t* len, const int32_t* src, int add, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) len[b] = (src ? src[b] : len[b]) + add;
}

}  // namespace

hipError_t launch_embed(bool bf16, const void* embed, int vocab, int d, const int32_t* tokens, const int32_t* last,
                        const int32_t* draft, const int32_t* len, int B, int m, int hd, float theta, float* h,
                        float2* cs, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(embed_kernel<uint16_t>, dim3(B * m), dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(embed), vocab, d, tokens, last, draft, len, m, hd, theta, h, cs);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(B * m), dim3(kThreads), 0, s, static_cast<const float*>(embed),
                       vocab, d, tokens, last, draft, len, m, hd, theta, h, cs);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(bool bf16, const float* h, const float* g, int rows, int d, float eps, void* x,
                          hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(rmsnorm_kernel<uint16_t>, dim3(rows), dim3(kThreads), 0, s, h, g, d, eps,
                       static_cast<uint16_t*>(x));
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(rows), dim3(kThreads), 0, s, h, g, d, eps, static_cast<float*>(x));
  return hipGetLastError();
}

hipError_t launch_kv_len(int32_t* len, const int32_t* src, int add, int B, hipStream_t s) {
  hipLaunchKernelGGL(kv_len_kernel, dim3((B + 255) / 256), dim3(256), 0, s, len, src, add, B);
  return hipGetLastError();
}

}  // namespace sv
