// libspecverify C ABI: argument checks, workspace carving, and the launch
// sequence of a verify pass / decode step on one HIP stream.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/spec_verify.h"
#include "kernels.hpp"

#define SPEC_API extern "C" __attribute__((visibility("default")))

struct spec_model {
  spec_model_cfg cfg;
  const void* embed;
  const void* lm_head;
  const float* final_norm;
  std::vector<const float*> attn_norm, mlp_norm;
  std::vector<const void*> wqkv, wo, wgu, wd;
};

namespace {

thread_local std::string g_err;

spec_status fail(spec_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define HIP_TRY(expr)                                                                     \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess) return fail(SPEC_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Layout {
  size_t h, xn, xo, z, q, cs, po, pml, ctr, pt, logits, part, csum, tpart, lx, xsel, dpo, dpml, total;
  int n_split, n_qc, n_ctr, ks_o, ks_d;
  int dsplit;  // context splits of the short-pass attention (1: none)
};

Layout make_layout(const spec_model_cfg& c, int B, int m, int max_ctx) {
  Layout L{};
  const size_t rows = static_cast<size_t>(B) * m;
  const size_t elt = c.dtype == SPEC_BF16 ? 2 : 4;
  const int hq = c.n_heads * c.head_dim;
  const int nch = sv::sampler_chunks(c.vocab);
  const bool bf16 = c.dtype == SPEC_BF16;
  L.n_qc = sv::attn_row_blocks(bf16, B, c.n_heads, c.n_kv_heads, c.head_dim, m);
  L.n_split = sv::attn_num_splits(bf16, B, c.n_heads, c.n_kv_heads, c.head_dim, m, max_ctx);
  L.n_ctr = static_cast<int>(sv::attn_counters(bf16, B, c.n_heads, c.n_kv_heads, c.head_dim, m));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += up(bytes);
    return o;
  };
  L.h = take(rows * c.d_model * 4);
  L.xn = take(rows * c.d_model * elt);
  L.xo = take(rows * hq * elt);
  L.z = take(rows * c.d_ff * elt);
  L.q = take(rows * hq * 4);
  L.cs = take(rows * (c.head_dim / 2) * 8);
  L.po = take(static_cast<size_t>(B) * c.n_heads * m * L.n_split * c.head_dim * 4);
  L.pml = take(static_cast<size_t>(B) * c.n_heads * m * L.n_split * 8);
  L.ctr = take(static_cast<size_t>(L.n_ctr) * 4);  // attention tickets
  L.ks_o = sv::gemv_ksplit(c.dtype == SPEC_BF16, static_cast<int>(rows), c.d_model, hq);
  L.ks_d = sv::gemv_ksplit(c.dtype == SPEC_BF16, static_cast<int>(rows), c.d_model, c.d_ff);
  L.pt = take(static_cast<size_t>(std::max(L.ks_o, L.ks_d)) * rows * c.d_model * 4);  // K-slice partials
  L.logits = take(rows * c.vocab * 4);  // also the recomputed rows [B][vocab] of a fused step
  L.part = take(rows * nch * 8);
  L.csum = take(static_cast<size_t>(B) * nch * 16);
  L.tpart = take(rows * ((c.vocab + 127) / 128) * 8);  // LM-head tile statistics (fused step)
  L.lx = take(rows * 4);
  L.xsel = take(static_cast<size_t>(B) * c.d_model * elt);
  // one-row passes (a drafter's step) split each head's context when the
  // short-pass attention would run few workgroups
  L.dsplit = rows == 1 ? sv::attn_decode_splits(c.dtype == SPEC_BF16, c.head_dim, B, c.n_heads, m, max_ctx) : 1;
  L.dpo = take(rows * c.n_heads * L.dsplit * c.head_dim * 4);
  L.dpml = take(rows * c.n_heads * L.dsplit * 8);
  L.total = off;
  return L;
}

spec_status check_kv(const spec_model* M, const spec_kv* kv, int B, int m) {
  if (!M) return fail(SPEC_EINVAL, "model is NULL");
  if (!kv || !kv->k || !kv->v || !kv->len) return fail(SPEC_EINVAL, "kv cache pointers are NULL");
  if (B <= 0 || m <= 0) return fail(SPEC_EINVAL, "B=%d and m=%d must be positive", B, m);
  if (kv->B < B) return fail(SPEC_EINVAL, "kv cache holds %d sequences, pass needs %d", kv->B, B);
  if (kv->max_ctx <= 0) return fail(SPEC_EINVAL, "kv max_ctx=%d", kv->max_ctx);
  if (static_cast<int64_t>(B) * m > 65535 * 32) return fail(SPEC_EUNSUPPORTED, "B*m=%lld rows too many", (long long)B * m);
  return SPEC_OK;
}

// Whether a decode step runs the LM head without writing its logits (when
// the caller does not ask for them).  That needs the matrix-core LM head
// (bf16, more than 8 rows) and pays one more LM-head pass over the B sampled
// rows; it is taken when the logits' write and read (2 x rows x vocab x 4
// bytes) would move more than that extra pass reads (vocab x d_model x 2
// bytes).  A one-sequence verify pass of the 8B shape writes 3 MB of logits
// against 1.2 GB of LM head, so it keeps them.
bool fused_head(const spec_model_cfg& c, int rows) {
  if (c.dtype != SPEC_BF16 || rows <= 8 || c.d_model % 64) return false;
  return 2.0 * rows * 4 > 2.0 * c.d_model;
}

// Launch sequence of one forward pass over B x m rows.  The embedding kernel
// writes the residual rows h and the first RMSNorm's output; per layer
//   QKV linear (RoPE + KV append) -> attention -> O linear -> h += O,
//   MLP RMSNorm -> gate/up linear (SwiGLU) -> down linear -> h += down,
//   the next RMSNorm;
// then the LM head on the final RMSNorm.  With at most 8 rows the residual
// adds happen in the linears' epilogues and each RMSNorm in the next
// linear's staging; otherwise the linears write K-slice partials that one
// small kernel sums into h before normalising.
// trace (optional): the per-layer values of spec_trace (spec_verify.h).
// stat (optional, instead of logits): the LM head writes its tile statistics
// and the drafted tokens' logits (EPI_LMSTAT) rather than the logits.
struct LmStat {
  float temperature;
  const int32_t* draft;
};
spec_status run_forward(const spec_model* M, const spec_kv* kv, int B, int m, const int32_t* tokens,
                        const int32_t* last, const int32_t* draft, float* logits, const Layout& L, char* ws,
                        hipStream_t s, const spec_trace* trace = nullptr, const LmStat* stat = nullptr) {
  const spec_model_cfg& c = M->cfg;
  const bool bf16 = c.dtype == SPEC_BF16;
  const int rows = B * m;
  const int d = c.d_model, H = c.n_heads, Hkv = c.n_kv_heads, hd = c.head_dim, F = c.d_ff, V = c.vocab;
  float* h = reinterpret_cast<float*>(ws + L.h);
  void* xn = ws + L.xn;
  float2* cs = reinterpret_cast<float2*>(ws + L.cs);
  int* ctr = reinterpret_cast<int*>(ws + L.ctr);

  HIP_TRY(sv::launch_embed(bf16, M->embed, V, d, tokens, last, draft, kv->len, B, m, hd, c.rope_theta,
                           M->attn_norm[0], c.rms_eps, h, xn, cs, ctr, L.n_ctr, s));
  const size_t elt = bf16 ? 2 : 4;
  // per-layer copies of the trace: member dst (or NULL) gets bytes from src
  auto snap = [&](void* dst, int l, const void* src, size_t per_row) -> hipError_t {
    if (!dst) return hipSuccess;
    const size_t bytes = static_cast<size_t>(rows) * per_row;
    return hipMemcpyAsync(static_cast<char*>(dst) + static_cast<size_t>(l) * bytes, src, bytes,
                          hipMemcpyDeviceToDevice, s);
  };
  const spec_trace tr = trace ? *trace : spec_trace{};
  HIP_TRY(snap(tr.h, 0, h, d * sizeof(float)));
  sv::GemvArgs qkv;
  qkv.N = (H + 2 * Hkv) * hd;
  qkv.K = d;
  qkv.x = xn;
  qkv.q = reinterpret_cast<float*>(ws + L.q);
  qkv.H = H;
  qkv.Hkv = Hkv;
  qkv.hd = hd;
  qkv.cs = cs;
  qkv.kc = kv->k;
  qkv.vc = kv->v;
  qkv.len = kv->len;
  qkv.m_per_seq = m;
  qkv.kvB = kv->B;
  qkv.max_ctx = kv->max_ctx;
  sv::AttnArgs at;
  at.q = qkv.q;
  at.kc = kv->k;
  at.vc = kv->v;
  at.len = kv->len;
  at.m = m;
  at.H = H;
  at.Hkv = Hkv;
  at.kvB = kv->B;
  at.max_ctx = kv->max_ctx;
  at.n_split = L.n_split;
  at.n_qc = L.n_qc;
  at.part_o = reinterpret_cast<float*>(ws + L.po);
  at.part_ml = reinterpret_cast<float2*>(ws + L.pml);
  at.counters = ctr;
  at.xo = ws + L.xo;
  at.dsplit = L.dsplit;
  at.dpo = reinterpret_cast<float*>(ws + L.dpo);
  at.dpml = reinterpret_cast<float2*>(ws + L.dpml);
  float* pt = reinterpret_cast<float*>(ws + L.pt);
  const size_t pstride = static_cast<size_t>(rows) * d;
  sv::GemvArgs o;
  o.N = d;
  o.K = H * hd;
  o.ksplit = L.ks_o;
  o.x = ws + L.xo;
  o.y = pt;
  o.ldy = d;
  o.ysplit = pstride;
  sv::GemvArgs gu;
  gu.N = F;
  gu.K = d;
  gu.x = xn;
  gu.z = ws + L.z;
  gu.ldz = F;
  sv::GemvArgs dn = o;
  dn.K = F;
  dn.ksplit = L.ks_d;
  dn.x = ws + L.z;
  // Passes of at most 8 rows add a residual linear's output straight into h
  // (one K slice: every output element has one owner), and the next linear
  // makes its RMSNorm input from h while staging it.  Otherwise the K-slice
  // partials go through the residual-sum + RMSNorm kernel.
  const bool o_direct = rows <= 8 && L.ks_o == 1;
  const bool d_direct = rows <= 8 && L.ks_d == 1;
  for (int l = 0; l < c.n_layers; ++l) {
    qkv.W = M->wqkv[l];
    qkv.layer = l;
    if (l > 0 && d_direct) {
      qkv.hn = h;
      qkv.gain = M->attn_norm[l];
      qkv.eps = c.rms_eps;
    }
    HIP_TRY(sv::launch_gemv(bf16, sv::EPI_QKV, qkv, rows, s));
    HIP_TRY(snap(tr.q, l, qkv.q, static_cast<size_t>(H) * hd * sizeof(float)));
    at.layer = l;
    HIP_TRY(sv::launch_attention(bf16, hd, at, B, s));
    // a split pass's O linear merges the partials while staging; a traced or
    // K-sliced one gets them merged into xo first (the same arithmetic)
    const bool merge_in_o = L.dsplit > 1 && o_direct && !trace;
    if (L.dsplit > 1 && !merge_in_o) HIP_TRY(sv::launch_attn_merge(bf16, hd, at, rows, s));
    HIP_TRY(snap(tr.attn, l, at.xo, static_cast<size_t>(H) * hd * elt));
    o.W = M->wo[l];
    if (o_direct) {
      sv::GemvArgs od = o;
      od.y = h;
      if (merge_in_o) {
        od.x = nullptr;
        od.apo = at.dpo;
        od.apml = at.dpml;
        od.asplit = L.dsplit;
        od.ahd = hd;
        od.aH = H;
      }
      HIP_TRY(sv::launch_gemv(bf16, sv::EPI_RESID, od, rows, s));
      gu.hn = h;
      gu.gain = M->mlp_norm[l];
      gu.eps = c.rms_eps;
    } else {
      HIP_TRY(sv::launch_gemv(bf16, sv::EPI_PARTIAL, o, rows, s));
      HIP_TRY(sv::launch_resid_norm(bf16, h, pt, L.ks_o, pstride, rows, d, M->mlp_norm[l], c.rms_eps, xn, s));
    }
    HIP_TRY(snap(tr.h_mid, l, h, d * sizeof(float)));
    gu.W = M->wgu[l];
    HIP_TRY(sv::launch_gemv(bf16, sv::EPI_SWIGLU, gu, rows, s));
    HIP_TRY(snap(tr.mlp, l, gu.z, static_cast<size_t>(F) * elt));
    dn.W = M->wd[l];
    if (d_direct) {
      sv::GemvArgs dd = dn;
      dd.y = h;
      HIP_TRY(sv::launch_gemv(bf16, sv::EPI_RESID, dd, rows, s));
    } else {
      HIP_TRY(sv::launch_gemv(bf16, sv::EPI_PARTIAL, dn, rows, s));
      HIP_TRY(sv::launch_resid_norm(bf16, h, pt, L.ks_d, pstride, rows, d,
                                    l + 1 < c.n_layers ? M->attn_norm[l + 1] : M->final_norm, c.rms_eps, xn, s));
    }
    HIP_TRY(snap(tr.h, l + 1, h, d * sizeof(float)));
  }
  if (logits || stat) {
    sv::GemvArgs lm;
    lm.W = M->lm_head;
    lm.N = V;
    lm.K = d;
    lm.x = xn;
    if (d_direct) {
      lm.hn = h;
      lm.gain = M->final_norm;
      lm.eps = c.rms_eps;
    }
    if (stat) {
      lm.tpart = reinterpret_cast<float2*>(ws + L.tpart);
      lm.lx = reinterpret_cast<float*>(ws + L.lx);
      lm.draft = stat->draft;
      lm.temp = stat->temperature;
      lm.m_per_seq = m;
      HIP_TRY(sv::launch_gemv(bf16, sv::EPI_LMSTAT, lm, rows, s));
    } else {
      lm.y = logits;
      lm.ldy = V;
      HIP_TRY(sv::launch_gemv(bf16, sv::EPI_STORE, lm, rows, s));
    }
  }
  return SPEC_OK;
}

}  // namespace

SPEC_API const char* spec_last_error(void) { return g_err.c_str(); }

SPEC_API spec_status spec_model_create(const spec_model_cfg* cfg, const spec_weights* w, spec_model** out) {
  if (!cfg || !w || !out) return fail(SPEC_EINVAL, "NULL argument");
  *out = nullptr;
  const spec_model_cfg& c = *cfg;
  if (c.d_model <= 0 || c.n_layers <= 0 || c.n_heads <= 0 || c.n_kv_heads <= 0 || c.d_ff <= 0 || c.vocab <= 0)
    return fail(SPEC_EINVAL, "non-positive dimension in model config");
  if (c.dtype != SPEC_F32 && c.dtype != SPEC_BF16) return fail(SPEC_EINVAL, "dtype %d", c.dtype);
  if (c.head_dim != 64 && c.head_dim != 128) return fail(SPEC_EUNSUPPORTED, "head_dim %d (64 or 128)", c.head_dim);
  if (c.n_heads % c.n_kv_heads) return fail(SPEC_EINVAL, "n_heads %% n_kv_heads != 0");
  if (!sv::attn_supported(c.n_heads, c.n_kv_heads, c.head_dim))
    return fail(SPEC_EUNSUPPORTED, "query heads per KV head %d must divide 8 (16 at head_dim 128) or be a multiple",
                c.n_heads / c.n_kv_heads);
  if (c.d_model > 16 * 256) return fail(SPEC_EUNSUPPORTED, "d_model %d > 4096", c.d_model);
  if (static_cast<size_t>(std::max(c.d_model, std::max(c.d_ff, c.n_heads * c.head_dim))) *
          (c.dtype == SPEC_BF16 ? 2 : 4) > 159 * 1024)
    return fail(SPEC_EUNSUPPORTED, "a linear input row does not fit the 159 KiB of LDS");
  const int vec = c.dtype == SPEC_BF16 ? 8 : 4;
  if (c.d_model % vec || c.d_ff % vec || (c.n_heads * c.head_dim) % vec)
    return fail(SPEC_EINVAL, "d_model, d_ff and n_heads*head_dim must be multiples of %d", vec);
  if (!(c.rope_theta > 0.f) || !(c.rms_eps >= 0.f)) return fail(SPEC_EINVAL, "rope_theta / rms_eps");
  if (!w->embed || !w->lm_head || !w->final_norm || !w->attn_norm || !w->wqkv || !w->wo || !w->mlp_norm || !w->wgu ||
      !w->wd)
    return fail(SPEC_EINVAL, "NULL weight pointer");
  if (!aligned16(w->embed) || !aligned16(w->lm_head)) return fail(SPEC_EINVAL, "embed/lm_head not 16-byte aligned");
  for (int l = 0; l < c.n_layers; ++l) {
    if (!w->attn_norm[l] || !w->wqkv[l] || !w->wo[l] || !w->mlp_norm[l] || !w->wgu[l] || !w->wd[l])
      return fail(SPEC_EINVAL, "NULL weight pointer in layer %d", l);
    if (!aligned16(w->wqkv[l]) || !aligned16(w->wo[l]) || !aligned16(w->wgu[l]) || !aligned16(w->wd[l]))
      return fail(SPEC_EINVAL, "layer %d weights not 16-byte aligned", l);
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SPEC_EDEVICE, "no HIP device: %s", hipGetErrorString(e));
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return fail(SPEC_EDEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (std::string(prop.gcnArchName).rfind("gfx950", 0) != 0)
    return fail(SPEC_EDEVICE, "device %d is %s, this library is built for gfx950", dev, prop.gcnArchName);
  spec_model* M = new spec_model;
  M->cfg = c;
  M->embed = w->embed;
  M->lm_head = w->lm_head;
  M->final_norm = w->final_norm;
  M->attn_norm.assign(w->attn_norm, w->attn_norm + c.n_layers);
  M->mlp_norm.assign(w->mlp_norm, w->mlp_norm + c.n_layers);
  M->wqkv.assign(w->wqkv, w->wqkv + c.n_layers);
  M->wo.assign(w->wo, w->wo + c.n_layers);
  M->wgu.assign(w->wgu, w->wgu + c.n_layers);
  M->wd.assign(w->wd, w->wd + c.n_layers);
  *out = M;
  return SPEC_OK;
}

SPEC_API void spec_model_destroy(spec_model* model) { delete model; }

SPEC_API size_t spec_workspace_bytes(const spec_model* model, int32_t B, int32_t m, int32_t max_ctx) {
  if (!model || B <= 0 || m <= 0 || max_ctx <= 0) return 0;
  return make_layout(model->cfg, B, m, max_ctx).total;
}

SPEC_API size_t spec_sampler_workspace_bytes(int64_t rows, int32_t B, int32_t vocab) {
  if (rows < 0 || B < 0 || vocab <= 0) return 0;
  const int nch = sv::sampler_chunks(vocab);
  return up(static_cast<size_t>(rows) * nch * 8) + up(static_cast<size_t>(B) * nch * 16);
}

// ---- validation mode (SPEC_CHECK=1) -------------------------------------------------
// The checks write one flag word, a device variable of the library looked up
// per device (its host-side name is only a stand-in for the symbol).
namespace {
bool check_mode() {
  const char* e = getenv("SPEC_CHECK");
  return e && e[0] == '1';
}
std::mutex g_flag_mu;
int* g_flag_ptr[64] = {};
}  // namespace

static __device__ int check_flag;

namespace {
spec_status check_begin(int** flag, hipStream_t s) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(SPEC_EDEVICE, "device %d outside 0..63", dev);
  {
    std::lock_guard<std::mutex> lock(g_flag_mu);
    if (!g_flag_ptr[dev]) {
      void* p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(check_flag));
      if (e != hipSuccess || !p) return fail(SPEC_EHIP, "hipGetSymbolAddress(check_flag): %s", hipGetErrorString(e));
      g_flag_ptr[dev] = static_cast<int*>(p);
    }
    *flag = g_flag_ptr[dev];
  }
  HIP_TRY(sv::launch_check_clear(*flag, s));
  return SPEC_OK;
}

// Waits for the stream, then reports what the checks found.
spec_status check_end(int* flag, hipStream_t s, const char* call) {
  HIP_TRY(hipStreamSynchronize(s));
  int h = 0;
  HIP_TRY(hipMemcpy(&h, flag, sizeof(int), hipMemcpyDeviceToHost));
  if (h & 1) return fail(SPEC_EDEVICE, "%s: a token id outside [0, vocab) (SPEC_CHECK)", call);
  if (h & 2) return fail(SPEC_EDEVICE, "%s: a non-finite logit or probability (SPEC_CHECK)", call);
  return SPEC_OK;
}
}  // namespace

SPEC_API spec_status spec_verify_forward(const spec_model* model, const spec_kv* kv, int32_t B, int32_t m,
                                         const int32_t* tokens, float* logits, void* ws, size_t ws_bytes,
                                         hipStream_t stream) {
  spec_status st = check_kv(model, kv, B, m);
  if (st != SPEC_OK) return st;
  if (!tokens) return fail(SPEC_EINVAL, "tokens is NULL");
  const Layout L = make_layout(model->cfg, B, m, kv->max_ctx);
  if (!ws || ws_bytes < L.total) return fail(SPEC_ENOMEM, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  st = run_forward(model, kv, B, m, tokens, nullptr, nullptr, logits, L, static_cast<char*>(ws), stream);
  if (st != SPEC_OK || !check_mode()) return st;
  int* flag = nullptr;
  if ((st = check_begin(&flag, stream)) != SPEC_OK) return st;
  const int V = model->cfg.vocab;
  HIP_TRY(sv::launch_check_ids(tokens, B, m, nullptr, V, flag, stream));
  HIP_TRY(sv::launch_check_finite(logits, static_cast<int64_t>(B) * m * V, flag, stream));
  return check_end(flag, stream, "spec_verify_forward");
}

SPEC_API spec_status spec_verify_forward_trace(const spec_model* model, const spec_kv* kv, int32_t B, int32_t m,
                                               const int32_t* tokens, float* logits, const spec_trace* trace,
                                               void* ws, size_t ws_bytes, hipStream_t stream) {
  spec_status st = check_kv(model, kv, B, m);
  if (st != SPEC_OK) return st;
  if (!tokens || !trace) return fail(SPEC_EINVAL, "tokens/trace is NULL");
  const Layout L = make_layout(model->cfg, B, m, kv->max_ctx);
  if (!ws || ws_bytes < L.total) return fail(SPEC_ENOMEM, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  return run_forward(model, kv, B, m, tokens, nullptr, nullptr, logits, L, static_cast<char*>(ws), stream, trace);
}

namespace {
// T > 0: chunk (max, sum exp) partials, and the probabilities when probs is
// not NULL.  T = 0: chunk (max, argmax) partials, and one-hot rows.
spec_status softmax_rows(const float* logits, int64_t rows, int V, float T, float* probs, float2* part,
                         hipStream_t s) {
  const int nch = sv::sampler_chunks(V);
  for (int64_t r0 = 0; r0 < rows; r0 += 65535) {
    const int64_t nr = std::min<int64_t>(65535, rows - r0);
    if (T == 0.f) {
      HIP_TRY(sv::launch_row_argmax(logits + r0 * V, nr, V, part + r0 * nch, s));
      if (probs) HIP_TRY(sv::launch_onehot_write(nr, V, part + r0 * nch, probs + r0 * V, s));
    } else {
      HIP_TRY(sv::launch_row_partials(logits + r0 * V, nr, V, T, part + r0 * nch, s));
      if (probs) HIP_TRY(sv::launch_softmax_write(logits + r0 * V, nr, V, T, part + r0 * nch, probs + r0 * V, s));
    }
  }
  return SPEC_OK;
}

bool valid_temperature(float T) { return T >= 0.f && T <= 3.0e38f; }
}  // namespace

SPEC_API spec_status spec_softmax_pq(const float* logits, int64_t rows, int32_t vocab, float temperature, float* probs,
                                     void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!logits || !probs) return fail(SPEC_EINVAL, "NULL logits/probs");
  if (rows < 0 || vocab <= 0) return fail(SPEC_EINVAL, "rows=%lld vocab=%d", (long long)rows, vocab);
  if (!valid_temperature(temperature)) return fail(SPEC_EINVAL, "temperature must be finite and >= 0");
  if (rows == 0) return SPEC_OK;
  const size_t need = spec_sampler_workspace_bytes(rows, 0, vocab);
  if (!ws || ws_bytes < need) return fail(SPEC_ENOMEM, "workspace %zu bytes < %zu needed", ws_bytes, need);
  spec_status st = softmax_rows(logits, rows, vocab, temperature, probs, static_cast<float2*>(ws), stream);
  if (st != SPEC_OK || !check_mode()) return st;
  int* flag = nullptr;
  if ((st = check_begin(&flag, stream)) != SPEC_OK) return st;
  HIP_TRY(sv::launch_check_finite(logits, rows * vocab, flag, stream));
  return check_end(flag, stream, "spec_softmax_pq");
}

namespace {
// greedy: the uniforms are not used and may be NULL.
spec_status check_sampler_args(int B, int gamma, int V, const int32_t* draft, const float* u_acc, const float* u_res,
                               const int32_t* n_accepted, const int32_t* emitted, bool greedy = false) {
  if (B <= 0 || B > 65535) return fail(SPEC_EINVAL, "B=%d (1..65535)", B);
  if (gamma < 0 || gamma > 63) return fail(SPEC_EINVAL, "gamma=%d (0..63)", gamma);
  if (V <= 0 || V > 64 * 4096) return fail(SPEC_EINVAL, "vocab=%d (1..262144)", V);
  if (gamma > 0 && !draft) return fail(SPEC_EINVAL, "draft NULL with gamma > 0");
  if (!greedy && ((gamma > 0 && !u_acc) || !u_res)) return fail(SPEC_EINVAL, "u_acc/u_res NULL");
  if (!n_accepted || !emitted) return fail(SPEC_EINVAL, "n_accepted/emitted NULL");
  return SPEC_OK;
}
}  // namespace

SPEC_API spec_status spec_reject_sample(int32_t B, int32_t gamma, int32_t vocab, const float* p, const float* q,
                                        const int32_t* draft, const int32_t* n_draft, const float* u_acc,
                                        const float* u_res, int32_t* n_accepted, int32_t* emitted, void* ws,
                                        size_t ws_bytes, hipStream_t stream) {
  spec_status st = check_sampler_args(B, gamma, vocab, draft, u_acc, u_res, n_accepted, emitted);
  if (st != SPEC_OK) return st;
  if (!p) return fail(SPEC_EINVAL, "p is NULL");
  const size_t need = spec_sampler_workspace_bytes(0, B, vocab);
  if (!ws || ws_bytes < need) return fail(SPEC_ENOMEM, "workspace %zu bytes < %zu needed", ws_bytes, need);
  sv::RejectRows rr;
  rr.p = p;
  HIP_TRY(sv::launch_reject(rr, B, gamma, vocab, q, draft, n_draft, u_acc, u_res, n_accepted, emitted, nullptr,
                            static_cast<unsigned long long*>(ws), stream));
  if (!check_mode()) return SPEC_OK;
  int* flag = nullptr;
  if ((st = check_begin(&flag, stream)) != SPEC_OK) return st;
  HIP_TRY(sv::launch_check_ids(draft, B, gamma, n_draft, vocab, flag, stream));
  HIP_TRY(sv::launch_check_finite(p, static_cast<int64_t>(B) * (gamma + 1) * vocab, flag, stream));
  HIP_TRY(sv::launch_check_finite(q, static_cast<int64_t>(B) * gamma * vocab, flag, stream));
  return check_end(flag, stream, "spec_reject_sample");
}

SPEC_API spec_status spec_draft_sample(const float* logits, int64_t ld_logits, int32_t B, int32_t vocab,
                                       float temperature, const float* u, float* q, int64_t ld_q, int32_t* tokens,
                                       int32_t ld_tokens, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!logits || !q || !tokens) return fail(SPEC_EINVAL, "NULL logits/q/tokens");
  if (B <= 0 || B > 65535) return fail(SPEC_EINVAL, "B=%d (1..65535)", B);
  if (vocab <= 0 || vocab > 64 * 4096) return fail(SPEC_EINVAL, "vocab=%d (1..262144)", vocab);
  if (ld_logits < vocab || ld_q < vocab || ld_tokens < 1)
    return fail(SPEC_EINVAL, "row strides %lld/%lld/%d below vocab/vocab/1", (long long)ld_logits, (long long)ld_q,
                ld_tokens);
  if (!valid_temperature(temperature)) return fail(SPEC_EINVAL, "temperature must be finite and >= 0");
  if (temperature > 0.f && !u) return fail(SPEC_EINVAL, "u is NULL");
  const size_t need = spec_sampler_workspace_bytes(B, B, vocab);
  if (!ws || ws_bytes < need) return fail(SPEC_ENOMEM, "workspace %zu bytes < %zu needed", ws_bytes, need);
  const int nch = sv::sampler_chunks(vocab);
  float2* part = static_cast<float2*>(ws);
  auto* csum = reinterpret_cast<unsigned long long*>(static_cast<char*>(ws) + up(static_cast<size_t>(B) * nch * 8));
  if (temperature == 0.f) {
    HIP_TRY(sv::launch_row_argmax(logits, B, vocab, part, stream, ld_logits));
    HIP_TRY(sv::launch_onehot_write(B, vocab, part, q, stream, ld_q));
    HIP_TRY(sv::launch_greedy(B, 0, vocab, part, nullptr, nullptr, nullptr, tokens, nullptr, stream, ld_tokens));
  } else {
    // the softmax pass also leaves each chunk's weight sums, so the draw is
    // one workgroup per sequence over its chosen chunk
    HIP_TRY(sv::launch_row_partials(logits, B, vocab, temperature, part, stream, ld_logits));
    HIP_TRY(sv::launch_softmax_write(logits, B, vocab, temperature, part, q, stream, ld_logits, ld_q, csum));
    sv::RejectRows rr;
    rr.logits = logits;
    rr.part = part;
    rr.temperature = temperature;
    rr.ld = ld_logits;
    HIP_TRY(sv::launch_reject(rr, B, 0, vocab, nullptr, nullptr, nullptr, nullptr, u, nullptr, tokens, nullptr, csum,
                              stream, ld_tokens, true));
  }
  if (!check_mode()) return SPEC_OK;
  int* flag = nullptr;
  spec_status st;
  if ((st = check_begin(&flag, stream)) != SPEC_OK) return st;
  for (int b = 0; b < B; ++b) HIP_TRY(sv::launch_check_finite(logits + static_cast<int64_t>(b) * ld_logits, vocab, flag, stream));
  return check_end(flag, stream, "spec_draft_sample");
}

SPEC_API spec_status spec_decode_step(const spec_model* target, const spec_kv* kv, int32_t B, int32_t gamma,
                                      float temperature, const int32_t* last_tok, const int32_t* draft,
                                      const int32_t* n_draft, const float* q, const float* u_acc, const float* u_res,
                                      int32_t* n_accepted, int32_t* emitted, float* logits_out, void* ws,
                                      size_t ws_bytes, hipStream_t stream) {
  const int m = gamma + 1;
  spec_status st = check_kv(target, kv, B, m);
  if (st != SPEC_OK) return st;
  if (!valid_temperature(temperature)) return fail(SPEC_EINVAL, "temperature must be finite and >= 0");
  const bool greedy = temperature == 0.f;
  st = check_sampler_args(B, gamma, target->cfg.vocab, draft, u_acc, u_res, n_accepted, emitted, greedy);
  if (st != SPEC_OK) return st;
  if (!last_tok) return fail(SPEC_EINVAL, "last_tok is NULL");
  const Layout L = make_layout(target->cfg, B, m, kv->max_ctx);
  if (!ws || ws_bytes < L.total) return fail(SPEC_ENOMEM, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  char* w = static_cast<char*>(ws);
  const int V = target->cfg.vocab;
  const int rows = B * m;
  float2* part = reinterpret_cast<float2*>(w + L.part);
  unsigned long long* csum = reinterpret_cast<unsigned long long*>(w + L.csum);
  const bool check = check_mode();
  if (!logits_out && !check && fused_head(target->cfg, rows)) {
    // The LM head leaves its softmax statistics and the drafted tokens'
    // logits instead of the [rows][vocab] logits; the row each sequence
    // samples from is recomputed afterwards (same kernel, same bits).
    const LmStat stat{temperature, draft};
    st = run_forward(target, kv, B, m, nullptr, last_tok, draft, nullptr, L, w, stream, nullptr, &stat);
    if (st != SPEC_OK) return st;
    HIP_TRY(sv::launch_tile_merge(rows, V, reinterpret_cast<const float2*>(w + L.tpart), greedy, part, stream));
    if (greedy) {
      HIP_TRY(sv::launch_greedy(B, gamma, V, part, draft, n_draft, n_accepted, emitted, kv->len, stream));
      return SPEC_OK;
    }
    sv::RejectRows rr;
    rr.part = part;
    rr.temperature = temperature;
    rr.lx = reinterpret_cast<const float*>(w + L.lx);
    HIP_TRY(sv::launch_select_rows(rr, B, gamma, V, q, draft, n_draft, u_acc, w + L.xn, target->cfg.d_model,
                                   w + L.xsel, stream));
    float* sel = reinterpret_cast<float*>(w + L.logits);
    sv::GemvArgs lm;
    lm.W = target->lm_head;
    lm.N = V;
    lm.K = target->cfg.d_model;
    lm.x = w + L.xsel;
    lm.y = sel;
    lm.ldy = V;
    lm.mfma = true;
    HIP_TRY(sv::launch_gemv(true, sv::EPI_STORE, lm, B, stream));
    rr.sel = sel;
    HIP_TRY(sv::launch_reject(rr, B, gamma, V, q, draft, n_draft, u_acc, u_res, n_accepted, emitted, kv->len, csum,
                              stream));
    return SPEC_OK;
  }
  float* logits = logits_out ? logits_out : reinterpret_cast<float*>(w + L.logits);
  st = run_forward(target, kv, B, m, nullptr, last_tok, draft, logits, L, w, stream);
  if (st != SPEC_OK) return st;
  st = softmax_rows(logits, static_cast<int64_t>(rows), V, temperature, nullptr, part, stream);
  if (st != SPEC_OK) return st;
  if (greedy) {
    HIP_TRY(sv::launch_greedy(B, gamma, V, part, draft, n_draft, n_accepted, emitted, kv->len, stream));
  } else {
    sv::RejectRows rr;
    rr.logits = logits;
    rr.part = part;
    rr.temperature = temperature;
    HIP_TRY(sv::launch_reject(rr, B, gamma, V, q, draft, n_draft, u_acc, u_res, n_accepted, emitted, kv->len, csum,
                              stream));
  }
  if (!check) return SPEC_OK;
  int* flag = nullptr;
  if ((st = check_begin(&flag, stream)) != SPEC_OK) return st;
  HIP_TRY(sv::launch_check_ids(last_tok, B, 1, nullptr, V, flag, stream));
  HIP_TRY(sv::launch_check_ids(draft, B, gamma, n_draft, V, flag, stream));
  HIP_TRY(sv::launch_check_finite(logits, static_cast<int64_t>(rows) * V, flag, stream));
  if (!greedy) HIP_TRY(sv::launch_check_finite(q, static_cast<int64_t>(B) * gamma * V, flag, stream));
  return check_end(flag, stream, "spec_decode_step");
}

// ---- the decode step with a workspace inside the library ----------------------------
// For callers that cannot allocate: each GPU holds one copy of `scratch` for
// the life of the process.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): the device
// address of each GPU's copy is looked up once, with that device current, and
// kept per device.
namespace {
constexpr size_t kScratchBytes = static_cast<size_t>(SPEC_STATIC_WORKSPACE_BYTES);
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
spec_status scratch_address(void** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(SPEC_EDEVICE, "device %d outside 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(SPEC_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SPEC_OK;
}
}  // namespace

SPEC_API spec_status spec_decode_step_static(const spec_model* target, const spec_kv* kv, int32_t B, int32_t gamma,
                                             float temperature, const int32_t* last_tok, const int32_t* draft,
                                             const int32_t* n_draft, const float* q, const float* u_acc,
                                             const float* u_res, int32_t* n_accepted, int32_t* emitted,
                                             float* logits_out, hipStream_t stream) {
  spec_status st = check_kv(target, kv, B, gamma + 1);
  if (st != SPEC_OK) return st;
  const size_t need = make_layout(target->cfg, B, gamma + 1, kv->max_ctx).total;
  if (need > kScratchBytes)
    return fail(SPEC_EUNSUPPORTED, "this step needs %zu bytes of workspace; the library's holds %zu", need,
                kScratchBytes);
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != SPEC_OK) return st;
  return spec_decode_step(target, kv, B, gamma, temperature, last_tok, draft, n_draft, q, u_acc, u_res, n_accepted,
                          emitted, logits_out, ws, kScratchBytes, stream);
}

SPEC_API spec_status spec_linear(int32_t dtype, int32_t epilogue, const void* W, const void* x, int32_t M, int32_t N,
                                 int32_t K, float* y, void* z, const float* hn, const float* gain, float eps,
                                 hipStream_t stream) {
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return fail(SPEC_EINVAL, "dtype %d", dtype);
  if (epilogue < 0 || epilogue > 2) return fail(SPEC_EINVAL, "epilogue %d", epilogue);
  if (M <= 0 || N <= 0 || K <= 0) return fail(SPEC_EINVAL, "M=%d N=%d K=%d", M, N, K);
  const int vec = dtype == SPEC_BF16 ? 8 : 4;
  if (K % vec) return fail(SPEC_EINVAL, "K=%d not a multiple of %d", K, vec);
  if (!W || !aligned16(W)) return fail(SPEC_EINVAL, "W NULL or not 16-byte aligned");
  if (hn) {
    if (!gain || !aligned16(hn) || !aligned16(gain)) return fail(SPEC_EINVAL, "hn/gain NULL or not 16-byte aligned");
    if (M > 8 || K > 4096 || !(eps >= 0.f))
      return fail(SPEC_EINVAL, "normalised input: M=%d must be <= 8, K=%d <= 4096, eps >= 0", M, K);
  } else if (!x || !aligned16(x)) {
    return fail(SPEC_EINVAL, "x NULL or not 16-byte aligned");
  }
  if (epilogue == 2 ? !z : !y) return fail(SPEC_EINVAL, "output pointer NULL");
  if (static_cast<size_t>(K) * (dtype == SPEC_BF16 ? 2 : 4) > 159 * 1024)
    return fail(SPEC_EINVAL, "K=%d: an input row must fit the 159 KiB of LDS", K);
  sv::GemvArgs a;
  a.W = W;
  a.N = N;
  a.K = K;
  a.x = hn ? nullptr : x;
  a.hn = hn;
  a.gain = gain;
  a.eps = eps;
  a.y = y;
  a.ldy = N;
  a.z = z;
  a.ldz = N;
  HIP_TRY(sv::launch_gemv(dtype == SPEC_BF16, epilogue, a, M, stream));
  return SPEC_OK;
}

SPEC_API spec_status spec_commit_round(int32_t B, int32_t gamma, const int32_t* n_accepted, const int32_t* emitted,
                                       int32_t* tok2, int32_t* last, int32_t* out_tokens, int32_t* out_len,
                                       int32_t cap, int32_t n_stop, int32_t* kv_len, int32_t* n_rounds,
                                       int32_t* n_log, int32_t log_cap, hipStream_t stream) {
  if (B <= 0 || gamma < 0 || cap < 0 || n_stop < 0 || log_cap < 0)
    return fail(SPEC_EINVAL, "B=%d gamma=%d cap=%d n_stop=%d log_cap=%d", B, gamma, cap, n_stop, log_cap);
  if (!n_accepted || !emitted || !tok2 || !out_len || (cap > 0 && !out_tokens))
    return fail(SPEC_EINVAL, "NULL argument");
  if (n_log && (!n_rounds || log_cap == 0)) return fail(SPEC_EINVAL, "n_log needs n_rounds and log_cap > 0");
  HIP_TRY(sv::launch_commit_round(B, gamma, n_accepted, emitted, tok2, last, out_tokens, out_len, cap, n_stop, kv_len,
                                  n_rounds, n_log, log_cap, stream));
  return SPEC_OK;
}

SPEC_API spec_status spec_ngram_propose(int32_t B, int32_t n_min, int32_t n_max, int32_t gamma,
                                        const int32_t* prefix, const int32_t* prefix_len, int32_t P,
                                        const int32_t* out, const int32_t* out_len, int32_t cap,
                                        const int32_t* fill_off, int32_t* drafts, int32_t* n_draft,
                                        int32_t* n_found, hipStream_t stream) {
  if (B <= 0 || B > 65535) return fail(SPEC_EINVAL, "B=%d (1..65535)", B);
  if (n_min < 1 || n_max < n_min || n_max > 16)
    return fail(SPEC_EINVAL, "n_min=%d n_max=%d (1 <= n_min <= n_max <= 16)", n_min, n_max);
  if (gamma < 0 || gamma > 63) return fail(SPEC_EINVAL, "gamma=%d (0..63)", gamma);
  if (P < 0 || cap < 0) return fail(SPEC_EINVAL, "P=%d cap=%d", P, cap);
  if ((P > 0 && !prefix) || (cap > 0 && (!out || !out_len)) || !n_draft || (gamma > 0 && !drafts))
    return fail(SPEC_EINVAL, "NULL argument");
  if (fill_off && P == 0) return fail(SPEC_EINVAL, "fill_off needs a prefix");
  HIP_TRY(sv::launch_ngram(B, n_min, n_max, gamma, prefix, prefix_len, P, out, out_len, cap, fill_off, drafts,
                           n_draft, n_found, stream));
  return SPEC_OK;
}

SPEC_API spec_status spec_kv_set_len(const spec_kv* kv, int32_t B, const int32_t* src, int32_t add,
                                     hipStream_t stream) {
  if (!kv || !kv->len) return fail(SPEC_EINVAL, "kv/len is NULL");
  if (B <= 0 || B > kv->B) return fail(SPEC_EINVAL, "B=%d outside 1..%d", B, kv->B);
  HIP_TRY(sv::launch_kv_len(kv->len, src, add, B, stream));
  return SPEC_OK;
}
