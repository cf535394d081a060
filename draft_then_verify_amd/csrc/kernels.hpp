// Host-side launchers of the gfx950 kernels (internal to libspecverify).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

// ---- weight-streaming linear ---------------------------------------------------
enum GemvEpi { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_QKV = 3, EPI_PARTIAL = 4, EPI_LMSTAT = 5 };

// y[M][N] (op) x[M][K] . W[N][K]^T for any M (in blocks of rows), x in the
// model dtype.
//  EPI_STORE : y[m][n]  = acc            (float32, ld ldy)
//  EPI_PARTIAL: as EPI_STORE, launch shape of the residual linears; with
//              ksplit > 1 slice s of K writes its partial to y + s * ysplit
//  EPI_RESID : y[m][n] += acc            (float32 residual, ld ldy)
//  EPI_SWIGLU: z[m][n]  = silu(g) * u    g: W rows n, u: rows n + N (dtype, ld ldz)
//  EPI_QKV   : W = [(H + 2 Hkv) hd][K]; q heads rotated into q [M][H hd];
//              k heads rotated and v heads copied into the KV cache of
//              `layer` at position len[b] + i (row = b * m_per_seq + i).
//  EPI_LMSTAT: the LM head without writing logits (bf16, matrix cores
//              only): per (row, 128-column tile) the softmax statistics of
//              lmstat.hpp at temperature `temp` (or, at temp = 0, the tile's
//              (max, lowest argmax as int bits)) into tpart [M][ceil(N/128)],
//              and lx[row] = the logit of the drafted token the row scores
//              (row = b * m_per_seq + i, i < m_per_seq - 1 scores
//              draft[b * (m_per_seq - 1) + i]; ids outside [0, N) are skipped).
// mfma: take the matrix-core kernel even for M <= 8 (its per-element results
// do not depend on M, so a recomputed row matches a larger pass bitwise).
// ldw / ldx: row strides of W and x (0: K).
// hn: when not NULL the activations are not read from x but made from the
// float32 residual rows hn [M][K] as cvt(RMSNorm(hn) * gain) while being
// staged (K = d_model, one K slice, M <= 8).
struct GemvArgs {
  const void* W = nullptr;
  int N = 0, K = 0, M = 0;
  int ldw = 0, ldx = 0;
  int ksplit = 1;
  const void* x = nullptr;
  const float* hn = nullptr;
  const float* gain = nullptr;
  float eps = 0.f;
  float* y = nullptr;
  int ldy = 0;
  size_t ysplit = 0;
  void* z = nullptr;
  int ldz = 0;
  // EPI_QKV
  float* q = nullptr;
  int H = 0, Hkv = 0, hd = 0;
  const float2* cs = nullptr;
  void* kc = nullptr;
  void* vc = nullptr;
  const int32_t* len = nullptr;
  int m_per_seq = 1, row0 = 0, layer = 0, kvB = 0, max_ctx = 0;
  // EPI_LMSTAT
  float2* tpart = nullptr;
  float* lx = nullptr;
  const int32_t* draft = nullptr;
  float temp = 1.f;
  bool mfma = false;
  // x from attention partials (AttnArgs::dpo/dpml of a split pass) instead of
  // x: x[m][h * ahd + j] = the merge of the asplit partials of row m, head h
  const float* apo = nullptr;
  const float2* apml = nullptr;
  int asplit = 1, ahd = 0, aH = 0;
};
hipError_t launch_gemv(bool bf16, int epi, const GemvArgs& a, int M, hipStream_t s);

// K slices the residual linears use for an M-row pass with N outputs: for
// M <= 8, the fewest that let a workgroup stage its block of activation rows
// in LDS; for the matrix-core path, enough slices for about 2 workgroups per
// CU.
int gemv_ksplit(bool bf16, int M, int N, int K);

// h[r][:] += part[0][r][:] + ... + part[ks-1][r][:] (slices summed in order
// first, float32; slice stride pstride floats), then
// x[r][:] = cvt(h[r][:] * rsqrt(mean(h[r][:]^2) + eps) * gain) in the model
// dtype; d % 4 == 0, d <= 4096.
// 1 <= ks <= 8.
hipError_t launch_resid_norm(bool bf16, float* h, const float* part, int ks, size_t pstride, int rows, int d,
                             const float* gain, float eps, void* x, hipStream_t s);

// h[r][:] = embed[tok(r)][:] (float32) and the RoPE table cs[r][j] = (cos, sin)
// of angle pos(r) * theta^(-2j/hd), pos(r) = len[b] + i for row r = b*m + i.
// tok(r) = tokens[r] if tokens, else (i == 0 ? last[b] : draft[b*(m-1) + i-1]).
// x[r][:] = cvt(RMSNorm(h[r][:]) * gain) is the first linear's input.
// Also zeroes the n_ctr tickets of the pass.
hipError_t launch_embed(bool bf16, const void* embed, int vocab, int d, const int32_t* tokens,
                        const int32_t* last, const int32_t* draft, const int32_t* len, int B, int m,
                        int hd, float theta, const float* gain, float eps, float* h, void* x, float2* cs,
                        int* ctr, int n_ctr, hipStream_t s);

// ---- attention -------------------------------------------------------------------
struct AttnArgs {
  const float* q = nullptr;  // [B*m][H*hd] rotated queries
  const void* kc = nullptr;
  const void* vc = nullptr;
  const int32_t* len = nullptr;
  int m = 1, H = 0, Hkv = 0, layer = 0, kvB = 0, max_ctx = 0, n_split = 1, n_qc = 1;
  float* part_o = nullptr;     // [B][H][m][n_split][hd]
  float2* part_ml = nullptr;   // [B][H][m][n_split]
  int* counters = nullptr;     // attn_counters(...) tickets, zero between launches
  void* xo = nullptr;          // [B*m][H*hd] output in the model dtype
  // Short passes with few (sequence, head, row) units split each head's
  // context over dsplit workgroups; each writes its partial (unnormalised
  // output dpo [B*m][H][dsplit][hd], max and weight dpml [B*m][H][dsplit])
  // instead of xo, and the O linear (or launch_attn_merge) merges them.
  int dsplit = 1;
  float* dpo = nullptr;
  float2* dpml = nullptr;
};
// hd 64/128; G = H/Hkv divides the workgroup's waves (16 for hd 128, 8 for
// hd 64) or is a multiple of them
bool attn_supported(int H, int Hkv, int hd);
// The split path's plan (row blocks n_qc, context splits n_split, tickets);
// bf16 passes of head_dim 64 take the matrix-core kernel, whose plan differs.
int attn_row_blocks(bool bf16, int B, int H, int Hkv, int hd, int m);  // n_qc
int attn_num_splits(bool bf16, int B, int H, int Hkv, int hd, int m, int max_ctx);
size_t attn_counters(bool bf16, int B, int H, int Hkv, int hd, int m);  // tickets the launch uses
hipError_t launch_attention(bool bf16, int hd, const AttnArgs& a, int B, hipStream_t s);
// True when launch_attention takes the short-pass kernel (m <= 8 rows,
// max_ctx <= 2048, a K/V row of at most 256 bytes): one workgroup per
// (sequence, query head), no context splits, so n_split, part_* and counters
// are not used.
bool attn_decode_path(bool bf16, int hd, int m, int max_ctx);
// Context splits launch_attention gives a pass (1 unless the short-pass
// kernel runs with few units).
int attn_decode_splits(bool bf16, int hd, int B, int H, int m, int max_ctx);
// xo from the partials of a split pass (rows = B*m), in the merge the O
// linear applies while staging.
hipError_t launch_attn_merge(bool bf16, int hd, const AttnArgs& a, int rows, hipStream_t s);

// Round bookkeeping (see spec_commit_round).
hipError_t launch_commit_round(int B, int gamma, const int32_t* n_acc, const int32_t* emitted, int32_t* tok2,
                               int32_t* last, int32_t* out, int32_t* out_len, int cap, int n_stop, int32_t* kv_len,
                               int32_t* n_rounds, int32_t* n_log, int log_cap, hipStream_t s);

// Prompt lookup (see spec_ngram_propose).
hipError_t launch_ngram(int B, int n_min, int n_max, int gamma, const int32_t* prefix, const int32_t* prefix_len, int P,
                        const int32_t* out, const int32_t* out_len, int cap, const int32_t* fill_off,
                        int32_t* drafts, int32_t* n_draft, int32_t* n_found, hipStream_t s);

// len[b] = (src ? src[b] : len[b]) + add
hipError_t launch_kv_len(int32_t* len, const int32_t* src, int add, int B, hipStream_t s);

// Validation: *flag = 0; then flag |= 1 for an id outside [0, vocab) among
// the first n_valid[r] (or per_row) of each row of ids [rows][per_row], and
// flag |= 2 for a non-finite value among v[0 .. n).
hipError_t launch_check_clear(int* flag, hipStream_t s);
hipError_t launch_check_ids(const int32_t* ids, int rows, int per_row, const int32_t* n_valid, int vocab, int* flag,
                            hipStream_t s);
hipError_t launch_check_finite(const float* v, int64_t n, int* flag, hipStream_t s);

// ---- sampler ----------------------------------------------------------------------
int sampler_chunks(int vocab);
// part[row][c] = (max, sum exp(l/T - max)) over chunk c of each row.
// ld: floats between logit rows (0: vocab).
hipError_t launch_row_partials(const float* logits, int64_t rows, int vocab, float temperature, float2* part,
                               hipStream_t s, int64_t ld = 0);
// probs = exp(l/T - m) / Z with the row statistics combined from part; with
// csum, also each chunk's fixed-point weight sums for a gamma = 0 draw from
// the rows (launch_reject then with have_chunks).
hipError_t launch_softmax_write(const float* logits, int64_t rows, int vocab, float temperature,
                                const float2* part, float* probs, hipStream_t s, int64_t ld_in = 0, int64_t ld_out = 0,
                                unsigned long long* csum = nullptr);
// Temperature 0: part[row][c] = (chunk max, its lowest index as int bits);
// one-hot rows at the row argmax; greedy accept (x_i == argmax_i) with the
// argmax of row n emitted after the accepted drafts.
hipError_t launch_row_argmax(const float* logits, int64_t rows, int vocab, float2* part, hipStream_t s,
                             int64_t ld = 0);
hipError_t launch_onehot_write(int64_t rows, int vocab, const float2* part, float* probs, hipStream_t s,
                               int64_t ld_out = 0);
hipError_t launch_greedy(int B, int gamma, int vocab, const float2* part, const int32_t* draft,
                         const int32_t* n_draft, int32_t* n_accepted, int32_t* emitted, int32_t* len_commit,
                         hipStream_t s, int ld_em = 0);
// Where the sampler's rows come from: materialised probabilities p, or
// logits + chunk statistics part; for passes whose logits were not written,
// lx (the logit at each row's drafted token) and sel ([B][vocab], the
// recomputed logits of the row each sequence samples from).
struct RejectRows {
  const float* p = nullptr;
  const float* logits = nullptr;
  const float2* part = nullptr;
  float temperature = 1.f;
  const float* lx = nullptr;
  const float* sel = nullptr;
  int64_t ld = 0;  // floats between rows of p or logits (0: vocab)
};
// Accept / resample / bonus.  csum is [B][chunks] scratch (2 x uint64 each).
hipError_t launch_reject(const RejectRows& rr, int B, int gamma, int vocab, const float* q, const int32_t* draft,
                         const int32_t* n_draft, const float* u_acc, const float* u_res, int32_t* n_accepted,
                         int32_t* emitted, int32_t* len_commit, unsigned long long* csum, hipStream_t s,
                         int ld_em = 0,               // ints between sequences' emitted rows (0: gamma + 1)
                         bool have_chunks = false);   // csum already holds the chunk sums (gamma = 0)
// Chunk statistics part [rows][chunks] from the LM head's tile statistics
// tpart [rows][ceil(vocab/128)] (EPI_LMSTAT).
hipError_t launch_tile_merge(int64_t rows, int vocab, const float2* tpart, bool greedy, float2* part, hipStream_t s);
// xsel[b] = xn[b * (gamma + 1) + n_b] (bf16 rows of d), n_b from the accept
// scan: the LM head inputs of the rows the sequences sample from.
hipError_t launch_select_rows(const RejectRows& rr, int B, int gamma, int vocab, const float* q, const int32_t* draft,
                              const int32_t* n_draft, const float* u_acc, const void* xn, int d, void* xsel,
                              hipStream_t s);

}  // namespace sv
