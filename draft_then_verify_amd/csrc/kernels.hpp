// Host-side launchers of the gfx950 kernels (internal to libspecverify).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

enum GemvEpi { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2 };

// y[M][N] (op) x[M][K] . W[N][K]^T, M any size (streamed in blocks of 8 rows).
//   EPI_STORE : y[m][n]  = acc            (y float32, ld ldy)
//   EPI_RESID : y[m][n] += acc            (y float32 residual stream, ld ldy)
//   EPI_SWIGLU: z[m][n]  = silu(g) * u    with g from W rows n, u from rows n + N;
//               z in the model dtype (ld ldz)
// W, x, z: model dtype (bf16 bits or float32).
hipError_t launch_gemv(bool bf16, int epi, const void* W, const void* x, int M, int N, int K,
                       float* y, int ldy, void* z, int ldz, hipStream_t s);

// h[r][:] = embed[tok(r)][:] (float32) and the RoPE table cs[r][j] = (cos, sin)
// of angle pos(r) * theta^(-2j/hd), pos(r) = len[b] + i for row r = b*m + i.
// tok(r) = tokens[r] if tokens, else (i == 0 ? last[b] : draft[b*(m-1) + i-1]).
hipError_t launch_embed(bool bf16, const void* embed, int vocab, int d, const int32_t* tokens,
                        const int32_t* last, const int32_t* draft, const int32_t* len, int B, int m,
                        int hd, float theta, float* h, float2* cs, hipStream_t s);

// x[r][:] = cvt(h[r][:] * rsqrt(mean(h^2) + eps) * g), cvt = bf16 rounding or none.
hipError_t launch_rmsnorm(bool bf16, const float* h, const float* g, int rows, int d, float eps, void* x,
                          hipStream_t s);

// RoPE on q (in place in qkv) and k; append k, v rows to the cache of `layer`.
hipError_t launch_rope_append(bool bf16, float* qkv, const float2* cs, const int32_t* len, int B, int m,
                              int H, int Hkv, int hd, void* kc, void* vc, int layer, int kvB, int max_ctx,
                              hipStream_t s);

// Split-context GQA attention for m query rows per sequence, causal inside
// the new block, then the log-sum-exp combine into x[r][h*hd + d] (model dtype).
int attn_num_splits(int B, int Hkv, int G, int m, int max_ctx);
hipError_t launch_attention(bool bf16, const float* qkv, const void* kc, const void* vc, const int32_t* len,
                            int B, int m, int H, int Hkv, int hd, int layer, int kvB, int max_ctx,
                            int n_split, float* part_o, float2* part_ml, void* x, hipStream_t s);

// len[b] = (src ? src[b] : len[b]) + add
hipError_t launch_kv_len(int32_t* len, const int32_t* src, int add, int B, hipStream_t s);

// ---- sampler ----------------------------------------------------------------
int sampler_chunks(int vocab);
// part[row][c] = (max, sum exp(l/T - max)) over chunk c of each row.
hipError_t launch_row_partials(const float* logits, int64_t rows, int vocab, float temperature, float2* part,
                               hipStream_t s);
// probs = exp(l/T - m) / Z with the row statistics combined from part.
hipError_t launch_softmax_write(const float* logits, int64_t rows, int vocab, float temperature,
                                const float2* part, float* probs, hipStream_t s);
// Accept / resample / bonus.  Rows come from `p` (materialised) or from
// logits + part (fused).  csum is [B][chunks] scratch (2 x uint64 each).
hipError_t launch_reject(int B, int gamma, int vocab, const float* p, const float* logits, const float2* part,
                         float temperature, const float* q, const int32_t* draft, const int32_t* n_draft,
                         const float* u_acc, const float* u_res, int32_t* n_accepted, int32_t* emitted,
                         int32_t* len_commit, unsigned long long* csum, hipStream_t s);

}  // namespace sv
