// Vocab-wide softmax and the rejection sampler of a verify round.
//
// The rule (first page, "What one iteration actually does", Algorithm 1; and
// "How Speculative Decoding Works", "Why the output doesn't change"):
//   accept x_i while u_i * q_i(x_i) <= p_i(x_i)  (reject iff u > p/q, written
//   without the division, float32); n = the first failure or n_draft;
//   row j = n: r = max(0, p_j - q_j) after a rejection, r = p_j (bonus) when
//   every draft passed; t ~ r / sum(r).
//
// Rows of 151936 float32 entries (608 KB) do not fit in LDS, so a row is cut
// in 4096-entry chunks:
//   1. row_partials: per (row, chunk) the max and sum of exp(l/T - max),
//      built from 128-column tiles in the order of lmstat.hpp -- the order
//      in which the matrix-core LM head produces them without writing the
//      logits (tile_merge then turns its tiles into the same chunk pairs).
//      Every consumer merges the chunk pairs in chunk order, so the row
//      statistics -- and hence every p(v) = exp(l_v/T - M) / Z -- are bitwise
//      the same wherever they are used (materialised or fused).
//   2. reject_chunks: per (sequence, chunk) the accept scan (one thread), then
//      the chunk sums of w = floor(r * 2^40) for the residual row and for p
//      (the all-zero-residual fallback).  Integer sums are exact, so any
//      reduction order gives the same S.
//   3. reject_final: per sequence, T = floor(k * S / 2^24) from k = u * 2^24;
//      the chunk whose running sum first exceeds T; an in-chunk scan finds the
//      smallest v with inclusive prefix > T.  Then the outputs and the KV
//      commit len += n + 1.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"
#include "lmstat.hpp"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 4096;
constexpr int kPer = kChunk / kThreads;
constexpr float kTwo40 = 1099511627776.0f;  // 2^40
constexpr float kTwo24 = 16777216.0f;       // 2^24
constexpr int kMaxRows = 64;                // gamma + 1 rows per sequence at most
constexpr int kMaxChunks = 64;              // vocab <= 64 * 4096

// Row statistics (M, Z) from the chunk partials, by one whole wave: lane j
// takes chunks j, j + 64, ... in order, then a wave max and a wave sum of
// Z_j = sum over its chunks of Z_c exp(M_c - M).  Every caller (the
// materialised softmax and the fused sampler) uses this same function, so a
// probability is bitwise the same wherever it is computed.
__device__ __forceinline__ float2 wave_stats(const float2* pr, int nch) {
  const int lane = threadIdx.x & (kWave - 1);
  float m = -INFINITY;
  for (int c = lane; c < nch; c += kWave) m = fmaxf(m, pr[c].x);
  const float M = wave_max(m);
  float z = 0.f;
  for (int c = lane; c < nch; c += kWave) z = fmaf(pr[c].y, expf(__fsub_rn(pr[c].x, M)), z);
  return make_float2(M, wave_sum(z));
}

// Where a probability row comes from.
struct RowSrc {
  const float* p;        // materialised rows, or nullptr
  const float* logits;   // logits + partials
  const float2* part;
  float T;
  int nch;
  int V;
  // Large passes whose logits were never written: the LM head gathered the
  // logit of each row's drafted token (lx [rows]) and the row each sequence
  // samples from was recomputed (sel [B][V]; rows per sequence m).
  const float* lx;
  const float* sel;
  int m;
  int64_t ld = 0;  // floats between rows of p or logits (0: V)
  // called by a whole wave
  __device__ __forceinline__ float2 stats(int64_t row) const {
    return p ? make_float2(0.f, 1.f) : wave_stats(part + row * nch, nch);
  }
  __device__ __forceinline__ float from_logit(float l, float2 st) const {
    return __fdiv_rn(expf(__fsub_rn(__fdiv_rn(l, T), st.x)), st.y);
  }
  // p(v) of the row a sequence samples from (the only full row read)
  __device__ __forceinline__ float prob(int64_t row, int v, float2 st) const {
    const int64_t rs = ld > 0 ? ld : V;
    if (p) return p[row * rs + v];
    const float* l = sel ? sel + (row / m) * V : logits + row * rs;
    return from_logit(l[v], st);
  }
  // p(x) at the drafted token x the row scores
  __device__ __forceinline__ float prob_x(int64_t row, int x, float2 st) const {
    return lx ? from_logit(lx[row], st) : prob(row, x, st);
  }
};

__device__ __forceinline__ unsigned long long fixed_weight(float r) {
  return static_cast<unsigned long long>(__fmul_rn(r, kTwo40));
}

// Accept scan for sequence b, by the whole workgroup: the statistics of rows
// 0 .. nd (waves in parallel) go to st_rows, lane i of wave 0 tests draft i,
// and n = the first failing i (a ballot), or nd.  Returns n to every thread.
__device__ int accept_scan(const RowSrc& src, int b, int gamma, int nd, const float* q, const int32_t* draft,
                           const float* u_acc, float2* st_rows, int* n_sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  for (int i = wave; i <= nd; i += kThreads / kWave) {
    const float2 st = src.stats(static_cast<int64_t>(b) * (gamma + 1) + i);
    if (lane == 0) st_rows[i] = st;
  }
  __syncthreads();
  if (wave == 0) {
    bool fail = false;
    if (lane < nd) {
      const int x = draft[b * gamma + lane];
      if (x < 0 || x >= src.V) {
        fail = true;
      } else {
        const int64_t row = static_cast<int64_t>(b) * (gamma + 1) + lane;
        const float px = src.prob_x(row, x, st_rows[lane]);
        const float qx = q ? q[(static_cast<int64_t>(b) * gamma + lane) * src.V + x] : 1.f;
        fail = !(__fmul_rn(u_acc[b * gamma + lane], qx) <= px);
      }
    }
    const unsigned long long m = __ballot(fail);
    if (lane == 0) *n_sh = m ? (__ffsll(static_cast<long long>(m)) - 1) : nd;
  }
  __syncthreads();
  return *n_sh;
}

// Exclusive prefix sums of one value per thread over the workgroup (fixed
// order: wave scans, then the wave totals in index order).
__device__ unsigned long long block_exclusive_scan_u64(unsigned long long v, unsigned long long* wsum) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  unsigned long long incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const unsigned long long t = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += t;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  unsigned long long base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  return base + incl - v;
}

__device__ __forceinline__ int n_valid(const int32_t* n_draft, int b, int gamma) {
  return n_draft ? min(max(n_draft[b], 0), gamma) : gamma;
}

// The sampled row at entry v: residual max(0, p - q) or p itself.
__device__ __forceinline__ float sample_mass(float pv, bool use_p, const float* qrow, int x_rej, int v) {
  if (use_p) return pv;
  const float qv = qrow ? qrow[v] : (v == x_rej ? 1.f : 0.f);
  return fmaxf(0.f, __fsub_rn(pv, qv));
}

// (max, sum exp) of chunk c of a row from materialised logits: 16-lane
// groups take the chunk's 32 tiles (two each) in lmstat.hpp's order, and
// thread 0 merges the tiles in order.
__global__ __launch_bounds__(kThreads) void row_partials_kernel(const float* __restrict__ logits, int64_t ld, int V,
                                                                float T, int nch, float2* __restrict__ part) {
  __shared__ float2 tst[lmstat::kTilesPerChunk];
  const int64_t row = blockIdx.y;
  const int c = blockIdx.x;
  const float* l = logits + row * ld;
  const int col = threadIdx.x & 15, grp = threadIdx.x >> 4;
  constexpr int kGroups = kThreads / 16;
  for (int t = grp; t < lmstat::kTilesPerChunk; t += kGroups) {
    const int c0 = c * kChunk + t * lmstat::kTile + col;
    float v[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int idx = c0 + h * 64 + j * 16;
        v[h][j] = idx < V ? (T == 1.f ? l[idx] : __fdiv_rn(l[idx], T)) : -INFINITY;  // x / 1 rounds to x
        mx = fmaxf(mx, v[h][j]);
      }
    mx = lmstat::group16_max(mx);
    const float z0 = group_sum<16>(lmstat::slot_sum(v[0], mx));
    const float z1 = group_sum<16>(lmstat::slot_sum(v[1], mx));
    if (col == 0) tst[t] = make_float2(mx, z0 + z1);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int tiles = min(lmstat::kTilesPerChunk, (V - c * kChunk + lmstat::kTile - 1) / lmstat::kTile);
    part[row * nch + c] = lmstat::merge_tiles(tst, tiles);
  }
}

// Chunk pairs from the LM head's tile statistics (EPI_LMSTAT): 32 lanes per
// (row, chunk), lane k holding tile k.  At T = 0 the (max, lowest argmax)
// pair is merged across the lanes (any order gives the same pair).  At T > 0
// the maximum is taken across the lanes (exact in any order), each lane
// weighs its tile by exp(M_t - M), and the chunk's weight sum Z_t x weight
// runs in tile order with the fused multiply-adds of lmstat::merge_tiles, so
// the pair is bitwise the one the materialised path builds.
__global__ __launch_bounds__(kThreads) void tile_merge_kernel(int64_t rows, int V, int nch, int nts, bool greedy,
                                                              const float2* __restrict__ tpart,
                                                              float2* __restrict__ part) {
  constexpr int kGroup = lmstat::kTilesPerChunk;  // lanes per (row, chunk)
  static_assert(kGroup == 32 && kThreads % kGroup == 0, "two chunks per wave");
  const int64_t i = static_cast<int64_t>(blockIdx.x) * (kThreads / kGroup) + threadIdx.x / kGroup;
  const int k = threadIdx.x % kGroup;
  const bool live = i < rows * nch;  // every lane stays for the shuffles
  const int64_t row = live ? i / nch : 0;
  const int c = live ? static_cast<int>(i - row * nch) : 0;
  const int n = min(kGroup, nts - c * kGroup);
  const bool mine = live && k < n;
  const float2 t = mine ? tpart[row * nts + c * kGroup + k] : make_float2(-INFINITY, 0.f);
  if (greedy) {
    float m = t.x;
    int ix = mine ? __float_as_int(t.y) : V;
#pragma unroll
    for (int off = kGroup / 2; off > 0; off >>= 1) {
      const float m2 = __shfl_xor(m, off, kWave);
      const int i2 = __shfl_xor(ix, off, kWave);
      lmstat::argmax_merge(m, ix, m2, i2);
    }
    if (live && k == 0) part[i] = make_float2(m, __int_as_float(ix));
    return;
  }
  float M = t.x;
#pragma unroll
  for (int off = kGroup / 2; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, kWave));
  const float w = t.y != 0.f ? expf(__fsub_rn(t.x, M)) : 0.f;
  float Z = 0.f;
#pragma unroll
  for (int j = 0; j < kGroup; ++j) {
    const float y = __shfl(t.y, j, kGroup), wj = __shfl(w, j, kGroup);
    if (y != 0.f) Z = fmaf(y, wj, Z);  // lanes past n hold y = 0
  }
  if (live && k == 0) part[i] = make_float2(M, Z);
}

// probs[row][v] = p(v) over chunk c of the row.  With csum (a row drawn from
// as a bonus row, gamma = 0) it also writes the chunk's fixed-point weight
// sum twice, as reject_chunks_kernel does for such a row, so the draw needs
// only reject_final_kernel.
template <bool SUMS>
__global__ __launch_bounds__(kThreads) void softmax_write_kernel(const float* __restrict__ logits, int64_t ld_in,
                                                                 int V, float T, int nch,
                                                                 const float2* __restrict__ part,
                                                                 float* __restrict__ probs, int64_t ld_out,
                                                                 unsigned long long* __restrict__ csum) {
  __shared__ float2 st_sh;
  __shared__ unsigned long long red[kThreads / kWave];
  const int64_t row = blockIdx.y;
  const int c = blockIdx.x;
  if (threadIdx.x < kWave) {
    const float2 st = wave_stats(part + row * nch, nch);
    if (threadIdx.x == 0) st_sh = st;
  }
  __syncthreads();
  const float2 st = st_sh;
  RowSrc src{nullptr, logits, part, T, nch, V, nullptr, nullptr, 1, ld_in};
  unsigned long long wp = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int v = c * kChunk + e * kThreads + threadIdx.x;
    if (v < V) {
      const float pv = src.prob(row, v, st);
      probs[row * ld_out + v] = pv;
      if (SUMS) wp += fixed_weight(pv);
    }
  }
  if (SUMS) {
    wp = block_sum_u64<kThreads>(wp, red);
    if (threadIdx.x == 0) {
      csum[(row * nch + c) * 2 + 0] = wp;
      csum[(row * nch + c) * 2 + 1] = wp;
    }
  }
}

struct RejectArgs {
  RowSrc src;
  int gamma;
  const float* q;
  const int32_t* draft;
  const int32_t* n_draft;
  const float* u_acc;
  const float* u_res;
  int32_t* n_accepted;
  int32_t* emitted;
  int32_t* len_commit;
  unsigned long long* csum;  // [B][nch][2]: residual sum, p sum
  int ld_em;                 // ints between sequences' emitted rows (0: gamma + 1)
};

__global__ __launch_bounds__(kThreads) void reject_chunks_kernel(RejectArgs a) {
  __shared__ int n_sh;
  __shared__ float2 st_rows[kMaxRows];
  __shared__ unsigned long long red[kThreads / kWave];
  const int c = blockIdx.x, b = blockIdx.y;
  const RowSrc& src = a.src;
  const int nd = n_valid(a.n_draft, b, a.gamma);
  const int n = accept_scan(src, b, a.gamma, nd, a.q, a.draft, a.u_acc, st_rows, &n_sh);
  const float2 st = st_rows[n];
  const bool bonus = n == nd;
  const int64_t row = static_cast<int64_t>(b) * (a.gamma + 1) + n;
  const int x_rej = bonus ? -1 : a.draft[b * a.gamma + n];
  const float* qrow = (!bonus && a.q) ? a.q + (static_cast<int64_t>(b) * a.gamma + n) * src.V : nullptr;
  unsigned long long wr = 0, wp = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int v = c * kChunk + e * kThreads + threadIdx.x;
    if (v < src.V) {
      const float pv = src.prob(row, v, st);
      wr += fixed_weight(sample_mass(pv, bonus, qrow, x_rej, v));
      wp += fixed_weight(pv);
    }
  }
  wr = block_sum_u64<kThreads>(wr, red);
  wp = block_sum_u64<kThreads>(wp, red);
  if (threadIdx.x == 0) {
    a.csum[(static_cast<size_t>(b) * src.nch + c) * 2 + 0] = wr;
    a.csum[(static_cast<size_t>(b) * src.nch + c) * 2 + 1] = wp;
  }
}

__global__ __launch_bounds__(kThreads) void reject_final_kernel(RejectArgs a) {
  __shared__ int n_sh, cstar_sh, use_p_sh, tok_sh;
  __shared__ float2 st_rows[kMaxRows];
  __shared__ unsigned long long base_sh, T_sh;
  __shared__ unsigned long long cs[2 * kMaxChunks];
  __shared__ unsigned long long wsum[kThreads / kWave];
  const int b = blockIdx.x;
  const RowSrc& src = a.src;
  const int nch = src.nch;
  const int nd = n_valid(a.n_draft, b, a.gamma);
  for (int i = threadIdx.x; i < 2 * nch; i += kThreads) cs[i] = a.csum[static_cast<size_t>(b) * nch * 2 + i];
  const int n_all = accept_scan(src, b, a.gamma, nd, a.q, a.draft, a.u_acc, st_rows, &n_sh);
  if (threadIdx.x == 0) {
    const int n = n_all;
    unsigned long long Sr = 0, Sp = 0;
    for (int c = 0; c < nch; ++c) {
      Sr += cs[2 * c];
      Sp += cs[2 * c + 1];
    }
    const int use_p = (n == nd) || Sr == 0;
    const unsigned long long S = use_p ? Sp : Sr;
    float uk = __fmul_rn(a.u_res[b], kTwo24);
    uk = fminf(fmaxf(uk, 0.f), kTwo24 - 1.f);
    const unsigned long long k = static_cast<unsigned long long>(uk);
    const unsigned long long T = (S >> 24) * k + (((S & 0xFFFFFFull) * k) >> 24);
    unsigned long long acc = 0;
    int cstar = nch - 1;
    for (int c = 0; c < nch; ++c) {
      const unsigned long long w = cs[2 * c + (use_p ? 1 : 0)];
      if (acc + w > T) {
        cstar = c;
        break;
      }
      acc += w;
    }
    use_p_sh = use_p;
    cstar_sh = cstar;
    base_sh = acc;
    T_sh = T;
    tok_sh = -1;
  }
  __syncthreads();
  const int n = n_all;
  const bool use_p = use_p_sh;
  const int64_t row = static_cast<int64_t>(b) * (a.gamma + 1) + n;
  const int x_rej = (n == nd) ? -1 : a.draft[b * a.gamma + n];
  const float* qrow = (n != nd && a.q) ? a.q + (static_cast<int64_t>(b) * a.gamma + n) * src.V : nullptr;
  const float2 st = st_rows[n];
  const int v0 = cstar_sh * kChunk + threadIdx.x * kPer;
  unsigned long long w[kPer];
  unsigned long long tsum = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int v = v0 + e;
    w[e] = (v < src.V) ? fixed_weight(sample_mass(src.prob(row, v, st), use_p, qrow, x_rej, v)) : 0ull;
    tsum += w[e];
  }
  const unsigned long long excl = block_exclusive_scan_u64(tsum, wsum);
  const unsigned long long T = T_sh;
  unsigned long long run = base_sh + excl;
  if (run <= T && T < run + tsum) {
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      run += w[e];
      if (run > T) {
        tok_sh = v0 + e;
        break;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int tok = tok_sh;
    if (tok < 0) tok = 0;  // unreachable when S > 0 and k < 2^24
    if (a.n_accepted) a.n_accepted[b] = n;
    const int lde = a.ld_em > 0 ? a.ld_em : a.gamma + 1;
    for (int j = 0; j <= a.gamma; ++j)
      a.emitted[b * lde + j] = j < n ? a.draft[b * a.gamma + j] : (j == n ? tok : -1);
    if (a.len_commit) a.len_commit[b] += n + 1;
  }
}

// The row each sequence samples from (row n after the accept scan) is copied
// from the LM head's input rows xn [rows][d] to xsel [B][d], for the
// recompute of that row's logits.
__global__ __launch_bounds__(kThreads) void select_rows_kernel(RejectArgs a, const uint16_t* __restrict__ xn, int d,
                                                               uint16_t* __restrict__ xsel) {
  __shared__ int n_sh;
  __shared__ float2 st_rows[kMaxRows];
  const int b = blockIdx.x;
  const int nd = n_valid(a.n_draft, b, a.gamma);
  const int n = accept_scan(a.src, b, a.gamma, nd, a.q, a.draft, a.u_acc, st_rows, &n_sh);
  const uint16_t* src = xn + (static_cast<size_t>(b) * (a.gamma + 1) + n) * d;
  for (int k = threadIdx.x; k < d; k += kThreads) xsel[static_cast<size_t>(b) * d + k] = src[k];
}

// ---- temperature 0 ------------------------------------------------------------------
// At T = 0 the target's distribution is its argmax ("How Speculative Decoding
// Works", section "Exactness is a choice"): draft x_i is accepted while it
// equals a_i = argmax of row i, and the round emits a_n after the accepted
// drafts (the replacement at a mismatch, or the bonus).  Ties go to the
// lowest index; a NaN entry is never selected (an all-NaN row selects 0).
// The order (larger value, then lower index) is total on non-NaN values, so
// any reduction tree gives the same (value, index).

using lmstat::argmax_merge;

__device__ __forceinline__ void wave_argmax(float& m, int& i) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off, kWave);
    const int i2 = __shfl_xor(i, off, kWave);
    argmax_merge(m, i, m2, i2);
  }
}

// Row argmax from the chunk partials (value, index bits), by one whole wave.
__device__ __forceinline__ int wave_row_argmax(const float2* pr, int nch, int V) {
  const int lane = threadIdx.x & (kWave - 1);
  float m = -INFINITY;
  int i = V;
  for (int c = lane; c < nch; c += kWave) argmax_merge(m, i, pr[c].x, __float_as_int(pr[c].y));
  wave_argmax(m, i);
  return i < V ? i : 0;
}

// part[row][c] = (max of chunk c, its lowest index as int bits).
__global__ __launch_bounds__(kThreads) void row_argmax_kernel(const float* __restrict__ logits, int64_t ld, int V,
                                                              int nch, float2* __restrict__ part) {
  __shared__ float mred[kThreads / kWave];
  __shared__ int ired[kThreads / kWave];
  const int64_t row = blockIdx.y;
  const int c = blockIdx.x;
  const float* l = logits + row * ld;
  float m = -INFINITY;
  int i = V;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int v = c * kChunk + e * kThreads + threadIdx.x;
    if (v < V) argmax_merge(m, i, l[v], v);
  }
  wave_argmax(m, i);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) {
    mred[wave] = m;
    ired[wave] = i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kThreads / kWave; ++w) argmax_merge(m, i, mred[w], ired[w]);
    part[row * nch + c] = make_float2(m, __int_as_float(i));
  }
}

// probs[row][v] = (v == argmax) ? 1 : 0.
__global__ __launch_bounds__(kThreads) void onehot_write_kernel(int V, int nch, const float2* __restrict__ part,
                                                                float* __restrict__ probs, int64_t ld_out) {
  __shared__ int a_sh;
  const int64_t row = blockIdx.y;
  const int c = blockIdx.x;
  if (threadIdx.x < kWave) {
    const int a = wave_row_argmax(part + row * nch, nch, V);
    if (threadIdx.x == 0) a_sh = a;
  }
  __syncthreads();
  const int a = a_sh;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int v = c * kChunk + e * kThreads + threadIdx.x;
    if (v < V) probs[row * ld_out + v] = (v == a) ? 1.f : 0.f;
  }
}

// One workgroup per sequence: the argmax of rows 0 .. nd (waves in
// parallel), then n and the emitted tokens; len_commit[b] += n + 1.
__global__ __launch_bounds__(kThreads) void greedy_kernel(int V, int nch, int gamma, const float2* __restrict__ part,
                                                          const int32_t* __restrict__ draft,
                                                          const int32_t* __restrict__ n_draft,
                                                          int32_t* __restrict__ n_accepted,
                                                          int32_t* __restrict__ emitted,
                                                          int32_t* __restrict__ len_commit, int ld_em) {
  __shared__ int amax[kMaxRows];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int nd = n_valid(n_draft, b, gamma);
  for (int i = wave; i <= nd; i += kThreads / kWave) {
    const int a = wave_row_argmax(part + (static_cast<int64_t>(b) * (gamma + 1) + i) * nch, nch, V);
    if (lane == 0) amax[i] = a;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    while (n < nd && draft[b * gamma + n] == amax[n]) ++n;
    if (n_accepted) n_accepted[b] = n;
    const int lde = ld_em > 0 ? ld_em : gamma + 1;
    for (int j = 0; j <= gamma; ++j)
      emitted[b * lde + j] = j < n ? draft[b * gamma + j] : (j == n ? amax[n] : -1);
    if (len_commit) len_commit[b] += n + 1;
  }
}

}  // namespace

hipError_t launch_row_argmax(const float* logits, int64_t rows, int vocab, float2* part, hipStream_t s, int64_t ld) {
  const int nch = sampler_chunks(vocab);
  hipLaunchKernelGGL(row_argmax_kernel, dim3(nch, static_cast<unsigned>(rows)), dim3(kThreads), 0, s, logits,
                     ld > 0 ? ld : vocab, vocab, nch, part);
  return hipGetLastError();
}

hipError_t launch_onehot_write(int64_t rows, int vocab, const float2* part, float* probs, hipStream_t s,
                               int64_t ld_out) {
  const int nch = sampler_chunks(vocab);
  hipLaunchKernelGGL(onehot_write_kernel, dim3(nch, static_cast<unsigned>(rows)), dim3(kThreads), 0, s, vocab, nch,
                     part, probs, ld_out > 0 ? ld_out : vocab);
  return hipGetLastError();
}

hipError_t launch_greedy(int B, int gamma, int vocab, const float2* part, const int32_t* draft,
                         const int32_t* n_draft, int32_t* n_accepted, int32_t* emitted, int32_t* len_commit,
                         hipStream_t s, int ld_em) {
  hipLaunchKernelGGL(greedy_kernel, dim3(B), dim3(kThreads), 0, s, vocab, sampler_chunks(vocab), gamma, part, draft,
                     n_draft, n_accepted, emitted, len_commit, ld_em);
  return hipGetLastError();
}

int sampler_chunks(int vocab) { return (vocab + kChunk - 1) / kChunk; }

hipError_t launch_row_partials(const float* logits, int64_t rows, int vocab, float temperature, float2* part,
                               hipStream_t s, int64_t ld) {
  const int nch = sampler_chunks(vocab);
  hipLaunchKernelGGL(row_partials_kernel, dim3(nch, static_cast<unsigned>(rows)), dim3(kThreads), 0, s, logits,
                     ld > 0 ? ld : vocab, vocab, temperature, nch, part);
  return hipGetLastError();
}

hipError_t launch_softmax_write(const float* logits, int64_t rows, int vocab, float temperature, const float2* part,
                                float* probs, hipStream_t s, int64_t ld_in, int64_t ld_out, unsigned long long* csum) {
  const int nch = sampler_chunks(vocab);
  const dim3 grid(nch, static_cast<unsigned>(rows));
  if (csum)
    hipLaunchKernelGGL(softmax_write_kernel<true>, grid, dim3(kThreads), 0, s, logits, ld_in > 0 ? ld_in : vocab,
                       vocab, temperature, nch, part, probs, ld_out > 0 ? ld_out : vocab, csum);
  else
    hipLaunchKernelGGL(softmax_write_kernel<false>, grid, dim3(kThreads), 0, s, logits, ld_in > 0 ? ld_in : vocab,
                       vocab, temperature, nch, part, probs, ld_out > 0 ? ld_out : vocab, csum);
  return hipGetLastError();
}

hipError_t launch_tile_merge(int64_t rows, int vocab, const float2* tpart, bool greedy, float2* part, hipStream_t s) {
  const int nch = sampler_chunks(vocab);
  const int nts = (vocab + lmstat::kTile - 1) / lmstat::kTile;
  const int64_t n = rows * nch;
  constexpr int per = kThreads / lmstat::kTilesPerChunk;  // (row, chunk) pairs per workgroup
  hipLaunchKernelGGL(tile_merge_kernel, dim3(static_cast<unsigned>((n + per - 1) / per)), dim3(kThreads), 0, s, rows,
                     vocab, nch, nts, greedy, tpart, part);
  return hipGetLastError();
}

namespace {
RejectArgs reject_args(const RejectRows& rr, int B, int gamma, int vocab, const float* q, const int32_t* draft,
                       const int32_t* n_draft, const float* u_acc, const float* u_res, int32_t* n_accepted,
                       int32_t* emitted, int32_t* len_commit, unsigned long long* csum) {
  const int nch = sampler_chunks(vocab);
  return RejectArgs{RowSrc{rr.p, rr.logits, rr.part, rr.temperature, nch, vocab, rr.lx, rr.sel, gamma + 1, rr.ld},
                    gamma, q, draft, n_draft, u_acc, u_res, n_accepted, emitted, len_commit, csum, 0};
}
}  // namespace

hipError_t launch_select_rows(const RejectRows& rr, int B, int gamma, int vocab, const float* q, const int32_t* draft,
                              const int32_t* n_draft, const float* u_acc, const void* xn, int d, void* xsel,
                              hipStream_t s) {
  RejectArgs a = reject_args(rr, B, gamma, vocab, q, draft, n_draft, u_acc, nullptr, nullptr, nullptr, nullptr, nullptr);
  hipLaunchKernelGGL(select_rows_kernel, dim3(B), dim3(kThreads), 0, s, a, static_cast<const uint16_t*>(xn), d,
                     static_cast<uint16_t*>(xsel));
  return hipGetLastError();
}

hipError_t launch_reject(const RejectRows& rr, int B, int gamma, int vocab, const float* q, const int32_t* draft,
                         const int32_t* n_draft, const float* u_acc, const float* u_res, int32_t* n_accepted,
                         int32_t* emitted, int32_t* len_commit, unsigned long long* csum, hipStream_t s,
                         int ld_em, bool have_chunks) {
  const int nch = sampler_chunks(vocab);
  RejectArgs a = reject_args(rr, B, gamma, vocab, q, draft, n_draft, u_acc, u_res, n_accepted, emitted, len_commit,
                             csum);
  a.ld_em = ld_em;
  if (!have_chunks) {
    hipLaunchKernelGGL(reject_chunks_kernel, dim3(nch, B), dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(reject_final_kernel, dim3(B), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace sv
