/*
 * spec_verify.h -- C ABI of the MI355X verify hot path of speculative
 * (draft-then-verify) decoding.
 *
 * What the library computes, by the pages that define it:
 *   - One round of Algorithm 1 as quoted on "Speculative Decoding Spends
 *     Arithmetic You May Not Have" (section "What one iteration actually
 *     does"): the target scores [last committed token, x_1 .. x_gamma] in ONE
 *     forward pass, giving p_1 .. p_{gamma+1}; drafts are accepted in order
 *     while u_i * q_i(x_i) <= p_i(x_i); the first rejection is replaced by a
 *     draw from norm(max(0, p - q)); when all gamma drafts pass, a bonus token
 *     is drawn from p_{gamma+1}.  One round emits 1 .. gamma+1 tokens.
 *   - The rule's exactness argument ("How Speculative Decoding Works (and When
 *     It Doesn't)", section "Why the output doesn't change") is what the
 *     residual and the bonus preserve.
 *   - The draw t ~ p' is a fixed-point inverse CDF: w_v = floor(r_v * 2^40),
 *     S = sum w, T = floor(k * S / 2^24) with k = u * 2^24, t = the smallest v
 *     whose inclusive prefix sum exceeds T.  Integer sums make the draw
 *     independent of reduction order.
 *
 * Conventions for every call below:
 *   - Array arguments are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or keeps them beyond the call; a model only
 *     borrows its weight pointers for its lifetime.
 *   - Calls are asynchronous on `stream`; results are valid after the stream
 *     is synchronised.  Host-side argument checks run before any launch.
 *   - Return value: SPEC_OK (0) or a negative spec_status; spec_last_error()
 *     returns a thread-local message describing the last failure.
 *   - Identical inputs give bitwise identical outputs (no floating-point
 *     atomics; every reduction has a fixed order).
 *   - Token ids outside [0, vocab) are never used to address memory: they are
 *     clamped for the embedding gather and count as rejected drafts in the
 *     sampler.  A pass whose positions would reach max_ctx writes and reads no
 *     KV row at or beyond max_ctx; its results are then undefined.
 *   - Uniforms are float32 values in [0, 1); the exact draw above assumes they
 *     are multiples of 2^-24 (any other value is truncated to that grid).
 *   - Validation mode: with SPEC_CHECK=1 in the environment,
 *     spec_verify_forward, spec_softmax_pq, spec_reject_sample,
 *     spec_draft_sample and spec_decode_step (and its _static form) also
 *     check their token ids
 *     (input tokens, the last committed tokens, the first n_draft drafts:
 *     inside [0, vocab)) and their float rows (logits, p and q rows: finite),
 *     synchronise the stream and return SPEC_EDEVICE when a check fails; the
 *     outputs are written either way.  In this mode a call blocks until its
 *     work is done (it cannot be captured into a graph), and a decode step
 *     keeps its logits in the workspace so that they can be checked.
 *
 * Data layout:
 *   - Weights are row-major [out][in] in the model dtype (float32 or bf16);
 *     norm gains are float32.
 *   - KV cache: k and v are [n_layers][B][n_kv_heads][max_ctx][head_dim] in the
 *     model dtype; len[B] (int32, device) is the number of committed positions
 *     of each sequence.  A forward pass over m rows writes positions
 *     len[b] .. len[b]+m-1 and does not change len.
 *   - Logits and probabilities are float32, row-major [rows][vocab]; the rows
 *     of a verify pass are ordered [b][i] (sequence-major).
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spec_status {
  SPEC_OK = 0,
  SPEC_EINVAL = -1,        /* invalid argument (checked on the host before any launch) */
  SPEC_ENOMEM = -2,        /* workspace smaller than the matching *_bytes() query */
  SPEC_EHIP = -3,          /* a HIP runtime call or a kernel launch failed */
  SPEC_EUNSUPPORTED = -4,  /* shape the kernels do not handle (see each call) */
  SPEC_EDEVICE = -5        /* no usable gfx950 device; or (SPEC_CHECK=1) the inputs or logits failed validation */
} spec_status;

typedef enum spec_dtype { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;

/* Decoder shape.  Llama-style: pre-norm RMSNorm, rotate-half RoPE, grouped-
 * query attention (query head h reads KV head h / (n_heads / n_kv_heads)),
 * SwiGLU MLP, no biases.  Requirements: head_dim in {64, 128}; n_heads a
 * multiple of n_kv_heads; d_model, d_ff and n_heads*head_dim multiples of 8. */
typedef struct spec_model_cfg {
  int32_t d_model, n_layers, n_heads, n_kv_heads, head_dim, d_ff, vocab;
  int32_t dtype; /* spec_dtype of weights, embedding, LM head and KV cache */
  float rope_theta, rms_eps;
} spec_model_cfg;

/* Device pointers of one model's weights.  The per-layer arrays are HOST
 * arrays of n_layers device pointers; they are copied at spec_model_create. */
typedef struct spec_weights {
  const void* embed;              /* [vocab][d_model] */
  const void* lm_head;            /* [vocab][d_model]; may equal embed (tied) */
  const float* final_norm;        /* [d_model] */
  const float* const* attn_norm;  /* [n_layers] x [d_model] */
  const void* const* wqkv;        /* [n_layers] x [(H + 2 Hkv) hd][d_model]: q rows, k rows, v rows */
  const void* const* wo;          /* [n_layers] x [d_model][H hd] */
  const float* const* mlp_norm;   /* [n_layers] x [d_model] */
  const void* const* wgu;         /* [n_layers] x [2 d_ff][d_model]: gate rows, then up rows */
  const void* const* wd;          /* [n_layers] x [d_model][d_ff] */
} spec_weights;

/* A per-sequence contiguous KV cache (layout above). */
typedef struct spec_kv {
  void* k;
  void* v;
  int32_t* len; /* [B] device */
  int32_t B;
  int32_t max_ctx;
} spec_kv;

typedef struct spec_model spec_model;

/* Create a model handle over borrowed weights.  A self-speculative drafter
 * (the target's first layers, final norm and head) is a second handle with a
 * smaller n_layers over the same pointers.  Errors: SPEC_EINVAL (shape),
 * SPEC_EUNSUPPORTED (head_dim), SPEC_EDEVICE (no gfx950 device current). */
spec_status spec_model_create(const spec_model_cfg* cfg, const spec_weights* w, spec_model** out);
void spec_model_destroy(spec_model* model);

/* Workspace bytes a verify pass / decode step of B sequences x m rows needs,
 * for a KV cache of max_ctx positions (the context split of attention depends
 * on it).  0 on invalid arguments. */
size_t spec_workspace_bytes(const spec_model* model, int32_t B, int32_t m, int32_t max_ctx);

/* Workspace bytes spec_softmax_pq / spec_reject_sample need for `rows`
 * probability rows of `vocab` entries and B sequences. */
size_t spec_sampler_workspace_bytes(int64_t rows, int32_t B, int32_t vocab);

/* The verify pass (first page, Algorithm 1 and the mechanism section: the
 * target scores all gamma + 1 positions of a round in one forward pass):
 * one forward over B sequences x m rows at positions
 * len[b] .. len[b]+m-1, streaming every weight once per block of 8 rows.
 *   tokens  [B][m] int32 input ids.
 *   logits  [B][m][vocab] float32 output, or NULL to skip the LM head
 *           (prefill).
 * Writes the m new K/V rows of every layer; len is unchanged (advance it with
 * spec_kv_set_len).  Errors: SPEC_EINVAL (null/size mismatch,
 * kv->B < B), SPEC_ENOMEM (ws_bytes < spec_workspace_bytes), SPEC_EHIP. */
spec_status spec_verify_forward(const spec_model* model, const spec_kv* kv, int32_t B, int32_t m,
                                const int32_t* tokens, float* logits, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* The values inside a forward pass, per layer, for checking a pass one step
 * at a time.  The verify pass of the first page (section "What one iteration
 * actually does") runs every position through the same layer stack; each
 * member below is the input of the next step in that stack, after its
 * rounding to the model dtype, so a reference can run every step on exactly
 * the inputs the kernels had.  rows = B * m, ordered [b][i].  Members are
 * caller-owned device buffers, each may be NULL (not captured):
 *   h      [n_layers + 1][rows][d_model] float32: the residual rows entering
 *          each layer (entry 0: the embedding rows), then the final rows.
 *   q      [n_layers][rows][n_heads * head_dim] float32: rotated queries.
 *   attn   [n_layers][rows][n_heads * head_dim] model dtype: attention
 *          output, the O linear's input.
 *   h_mid  [n_layers][rows][d_model] float32: residual after the attention
 *          block.
 *   mlp    [n_layers][rows][d_ff] model dtype: SwiGLU output, the down
 *          linear's input.
 * (The new K and V rows are in the cache.) */
typedef struct spec_trace {
  float* h;
  float* q;
  void* attn;
  float* h_mid;
  void* mlp;
} spec_trace;

/* spec_verify_forward with its per-layer values copied out (spec_trace):
 * the same launches and results, plus one device-to-device copy per
 * captured value and layer.  Errors: as spec_verify_forward; trace NULL is
 * SPEC_EINVAL. */
spec_status spec_verify_forward_trace(const spec_model* model, const spec_kv* kv, int32_t B, int32_t m,
                                      const int32_t* tokens, float* logits, const spec_trace* trace, void* ws,
                                      size_t ws_bytes, hipStream_t stream);

/* Target/draft probabilities p = softmax(logits / temperature) over `vocab`
 * entries for `rows` rows (p and q of the acceptance rule are the two
 * models' next-token distributions: "How Speculative Decoding Works (and
 * When It Doesn't)", section "Why the output doesn't change").  float32, max-subtracted; the same row statistics the fused
 * decode step uses, so p is bitwise what spec_decode_step samples from.
 * temperature >= 0 and finite.  temperature = 0 is the T -> 0 limit (same
 * page, section "Exactness is a choice"): a one-hot row at the argmax, the
 * lowest index among equal maxima (NaN entries are never selected).
 * Errors: SPEC_EINVAL, SPEC_ENOMEM, SPEC_EHIP. */
spec_status spec_softmax_pq(const float* logits, int64_t rows, int32_t vocab, float temperature,
                            float* probs, void* ws, size_t ws_bytes, hipStream_t stream);

/* The drafter's sampling step (the last page's draft.sample: a token and the
 * probability row it was drawn from; first page, Algorithm 1: x_i ~ q_i).
 * For b < B, with logit row l_b = logits + b * ld_logits [vocab]:
 *   q + b * ld_q [vocab]   out: q_b = softmax(l_b / temperature), written as
 *                          spec_softmax_pq writes it (one-hot at the lowest
 *                          argmax when temperature = 0);
 *   tokens[b * ld_tokens]  out: a draw from q_b with the uniform u[b], by the
 *                          rule spec_reject_sample applies with gamma = 0
 *                          (the same token for the same row and uniform), or
 *                          the argmax when temperature = 0 (u may be NULL).
 * The strides let one call per draft position write column i of the
 * [B][gamma][vocab] draft rows and [B][gamma] drafts that spec_decode_step
 * reads (q + i * vocab with ld_q = gamma * vocab; tokens + i with
 * ld_tokens = gamma), and read one row per sequence of a multi-row pass's
 * logits (ld_logits = m * vocab).  ld_logits, ld_q >= vocab, ld_tokens >= 1;
 * q must not overlap logits.
 * ws: spec_sampler_workspace_bytes(B, B, vocab) bytes.
 * Errors: SPEC_EINVAL, SPEC_ENOMEM, SPEC_EHIP. */
spec_status spec_draft_sample(const float* logits, int64_t ld_logits, int32_t B, int32_t vocab, float temperature,
                              const float* u, float* q, int64_t ld_q, int32_t* tokens, int32_t ld_tokens, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/* The accept / resample / bonus rule on materialised rows (first page,
 * Algorithm 1: the accepted-prefix count, the residual resample and the
 * bonus draw).
 *   p        [B][gamma+1][vocab] target probabilities.
 *   q        [B][gamma][vocab] draft probabilities, or NULL for a one-hot
 *            draft (q_i(x_i) = 1, e.g. n-gram lookup).
 *   draft    [B][gamma] drafted ids x_1 .. x_gamma.
 *   n_draft  [B] number of valid drafts per sequence (clamped to [0, gamma]),
 *            or NULL for gamma.
 *   u_acc    [B][gamma], u_res [B] uniforms.
 *   n_accepted [B] out: n.   emitted [B][gamma+1] out: x_1 .. x_n, t, then -1.
 * gamma = 0 is a plain draw t ~ p (draft sampling, plain decoding).
 * Limits: gamma <= 63, vocab <= 262144 (64 chunks of 4096).
 * Errors: SPEC_EINVAL, SPEC_ENOMEM, SPEC_EHIP. */
spec_status spec_reject_sample(int32_t B, int32_t gamma, int32_t vocab, const float* p, const float* q,
                               const int32_t* draft, const int32_t* n_draft, const float* u_acc,
                               const float* u_res, int32_t* n_accepted, int32_t* emitted, void* ws,
                               size_t ws_bytes, hipStream_t stream);

/* One whole verify step: assemble [last_tok, draft] (B x (gamma+1) rows),
 * run the verify pass, the fused softmax + accept/resample/bonus without
 * materialising p, and commit the KV cache: len[b] += n[b] + 1 (the last
 * committed token and the n accepted drafts stay cached: a rejection cuts
 * the round's block at that position, first page).  Arguments as in spec_reject_sample;
 * logits_out [B][gamma+1][vocab] receives the logits when non-NULL.
 * temperature = 0 verifies greedily ("How Speculative Decoding Works",
 * section "Exactness is a choice": at temperature zero the target takes its
 * argmax): x_i is accepted while it equals the argmax of row i (lowest index
 * on ties), n is the first mismatch (or n_draft), and the argmax of row n
 * follows the accepted drafts; q, u_acc and u_res are not read and may be
 * NULL.  temperature must be finite and >= 0.
 * Errors: as spec_verify_forward. */
spec_status spec_decode_step(const spec_model* target, const spec_kv* kv, int32_t B, int32_t gamma,
                             float temperature, const int32_t* last_tok, const int32_t* draft,
                             const int32_t* n_draft, const float* q, const float* u_acc,
                             const float* u_res, int32_t* n_accepted, int32_t* emitted,
                             float* logits_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* spec_decode_step for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops or harnesses that forbid hipMalloc):
 * the workspace is a device array inside the library,
 * SPEC_STATIC_WORKSPACE_BYTES per GPU, held by each GPU the library runs on
 * until the process ends.  The caller still owns the KV cache, the inputs
 * and the outputs.  Calls no allocating routine.  Every call on a GPU uses
 * that GPU's one array: calls that overlap on one GPU (other streams, other
 * threads) race and their results are undefined; calls in stream order are
 * safe (nothing in the array carries over from one call to the next).
 * Arguments and results as spec_decode_step.  Errors: as spec_decode_step,
 * and SPEC_EUNSUPPORTED when the step's workspace (spec_workspace_bytes of
 * B sequences x gamma + 1 rows) exceeds the array. */
#define SPEC_STATIC_WORKSPACE_BYTES (64u * 1024u * 1024u)
spec_status spec_decode_step_static(const spec_model* target, const spec_kv* kv, int32_t B, int32_t gamma,
                                    float temperature, const int32_t* last_tok, const int32_t* draft,
                                    const int32_t* n_draft, const float* q, const float* u_acc,
                                    const float* u_res, int32_t* n_accepted, int32_t* emitted, float* logits_out,
                                    hipStream_t stream);

/* The weight-streaming linear of the verify pass on its own: y = x . W^T for
 * M rows, every weight byte read once per block of 8 rows (a verify pass
 * streams the same weight bytes whatever the number of positions it scores,
 * first page, section "The speedup is borrowed").
 *   dtype     SPEC_F32 or SPEC_BF16: type of W, x and z.
 *   epilogue  0: y[M][N] = acc;  1: y[M][N] += acc (float32 residual);
 *             2: z[M][N] = silu(g) * u with g from W rows 0..N-1 and u from
 *                rows N..2N-1 (W is [2N][K]).
 *   W [N or 2N][K], x [M][K], y float32 [M][N] (epilogues 0, 1), z [M][N]
 *   (epilogue 2).  K a multiple of 16 bytes of the dtype; W and x 16-byte
 *   aligned.
 *   hn, gain, eps  optional (hn NULL: x is the input): the input rows are
 *   made from float32 residual rows hn [M][K] as RMSNorm(hn) * gain rounded
 *   to the dtype while they are staged, the form the verify pass uses for
 *   its QKV, gate/up and LM-head linears (x is then not read and may be
 *   NULL).  Needs M <= 8, K <= 4096, gain [K] float32, eps >= 0.
 * Errors: SPEC_EINVAL, SPEC_EHIP. */
spec_status spec_linear(int32_t dtype, int32_t epilogue, const void* W, const void* x, int32_t M, int32_t N,
                        int32_t K, float* y, void* z, const float* hn, const float* gain, float eps,
                        hipStream_t stream);

/* Round bookkeeping on the device, so a whole generation can run as graph
 * replays with no host round trip per round (first page, Algorithm 1: a
 * round emits x_1 .. x_n, t; the next round starts from t).  For b < B:
 * appends emitted[b][0 .. n] (n = n_accepted[b], clamped to [0, gamma]) to
 * out_tokens[b][out_len[b] ...] (positions >= cap are dropped but counted),
 * out_len[b] += n + 1, tok2[b] = (x_n, or the old tok2[b][1] when n = 0; t),
 * and last[b] = t when last is not NULL.
 *   n_accepted [B], emitted [B][gamma+1] as written by spec_decode_step;
 *   tok2 [B][2] in/out; last [B] out or NULL; out_tokens [B][cap];
 *   out_len [B] in/out.
 *   n_stop     0, or a token count: a sequence whose out_len had already
 *              reached n_stop before this round is finished and frozen: the
 *              round's outputs are discarded, and when kv_len is given
 *              (the target cache's len [B]) the decode step's commit is
 *              undone (kv_len[b] -= n + 1), so its cache stops growing.
 *   n_rounds   [B] in/out or NULL: rounds counted for each unfrozen sequence.
 *   n_log      [B][log_cap] out or NULL (needs n_rounds): n of the sequence's
 *              k-th counted round at [b][k] for k < log_cap (the accepted
 *              lengths behind the per-position acceptance counts of the first
 *              page, section "Checking it on a real system").
 * Errors: SPEC_EINVAL, SPEC_EHIP. */
spec_status spec_commit_round(int32_t B, int32_t gamma, const int32_t* n_accepted, const int32_t* emitted,
                              int32_t* tok2, int32_t* last, int32_t* out_tokens, int32_t* out_len, int32_t cap,
                              int32_t n_stop, int32_t* kv_len, int32_t* n_rounds, int32_t* n_log, int32_t log_cap,
                              hipStream_t stream);

/* Prompt lookup on the device: the n-gram drafter ("05 · Speculative
 * Decoding", section "The three proposers"; first page, section "Checking
 * it on a real system", method "ngram").  For sequence b the context is
 * prefix[b][0 .. prefix_len[b]) followed by out[b][0 .. min(out_len[b], cap)).
 * For a match length n, the most recent earlier occurrence of the context's
 * last n tokens (the match may not be the suffix itself) proposes the up to
 * gamma tokens that followed it, stopping at the end of the context.  The
 * lengths n_max, n_max - 1, ..., n_min are tried in that order and the first
 * that occurs is used (the match window prompt_lookup_min/max of "05 ·
 * Speculative Decoding", section "Dial It In"); n_min = n_max is a fixed
 * length.  No occurrence at any length (or a context shorter than n_min + 1)
 * proposes nothing.  The proposal is one-hot: verify it with q = NULL.
 *   prefix     [B][P] ids, row stride P (the prompt, or everything committed
 *              before `out` started); prefix_len [B] or NULL for P.
 *   out, out_len, cap  as maintained by spec_commit_round.
 *   fill_off   [B] or NULL.  When given, a proposal shorter than gamma is
 *              padded with prefix[b][fill_off[b] ...] (indexes clamped into
 *              the row) so that every sequence proposes gamma tokens.
 *   drafts     [B][gamma] out (entries past n_draft[b] are -1);
 *   n_draft    [B] out: tokens proposed (gamma when fill_off is given);
 *   n_found    [B] out or NULL: tokens that came from the lookup.
 * Limits: 1 <= n_min <= n_max <= 16, 0 <= gamma <= 63.  Deterministic.
 * Errors: SPEC_EINVAL, SPEC_EHIP. */
spec_status spec_ngram_propose(int32_t B, int32_t n_min, int32_t n_max, int32_t gamma, const int32_t* prefix,
                               const int32_t* prefix_len, int32_t P, const int32_t* out, const int32_t* out_len,
                               int32_t cap, const int32_t* fill_off, int32_t* drafts, int32_t* n_draft,
                               int32_t* n_found, hipStream_t stream);

/* KV length bookkeeping: len[b] = (src ? src[b] : len[b]) + add for b < B.
 * Used to advance after prefill / draft passes and to rewind a drafter to the
 * target's length.  Errors: SPEC_EINVAL, SPEC_EHIP. */
spec_status spec_kv_set_len(const spec_kv* kv, int32_t B, const int32_t* src, int32_t add,
                            hipStream_t stream);

/* Message of the last failed call on this thread ("" if none). */
const char* spec_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
