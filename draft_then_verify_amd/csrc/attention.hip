// Attention of the verify pass: m query rows per sequence (the last committed
// token and the gamma drafts) against the sequence's KV cache.
//
// The pages: one read of the cache serves every query position of the block
// (first page, section "The speedup is borrowed"), and decode-time attention
// stays memory-bound, its KV traffic growing with context and batch ("How
// Speculative Decoding Works", section "Prefill and Decode").  So a K/V row is
// fetched from memory once per workgroup and used by every query row that
// shares its KV head (grouped-query attention: G = H / Hkv query heads).
//
// Workgroup = 8 waves = (sequence b, KV head, block of query heads, block of
// query rows, context split).  The waves cover the query heads of the group
// (up to 8) times row sub-blocks: with G = 4, two waves per head, each
// owning MQ = ceil(m / 2) of the rows, so per-wave work stays short.  Per
// 64-key tile:
//  * the workgroup copies the K and V tile into LDS with 16-byte loads, all
//    of a tile's loads in flight at once, the next tile's issued before the
//    current one is used;
//  * scores: lane j holds key j of the tile (float32, from LDS) and dots it
//    with each of its wave's query rows (LDS broadcasts, 8 dimensions of
//    every row at a time so the reads overlap the FMAs);
//  * online softmax per row (wave max / sum);
//  * P.V: lane l takes the 16-byte chunk l % CPR of the V rows of keys
//    l / CPR, l / CPR + 64 / CPR, ... of the tile (one 16-byte LDS read per
//    key), and after the last tile the 64 / CPR key groups of each chunk are
//    summed across lanes in a fixed butterfly.
// At B = 1 the (sequence, head) pairs are few, so the context is cut into
// splits, one workgroup each; the partial (max, sum, output) rows are merged
// by the last workgroup of each (sequence, head block, row block) to finish
// (an atomic ticket), in split order: deterministic, with no combine launch.
//
// Causality inside the new block: query row i sits at position len + i and
// sees keys 0 .. len + i.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace sv {
namespace {

// Waves per workgroup (8: two per query head of a 4-head group; 16 measured
// no faster at B = 1, gamma = 4).
__host__ __device__ constexpr int waves_for(int) { return 8; }
constexpr int KT = 64;  // keys per tile (one per lane)

typedef unsigned int v4u __attribute__((ext_vector_type(4)));  // 16 bytes, kept in registers

template <typename ET> struct Cvt;  // 16 bytes of a K/V row -> floats
template <> struct Cvt<uint16_t> {
  static constexpr int n = 8;
  __device__ __forceinline__ static void run(const v4u& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
};
template <> struct Cvt<float> {
  static constexpr int n = 4;
  __device__ __forceinline__ static void run(const v4u& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
};

// Shape of the work split, shared by the launcher and the kernel.
struct Plan {
  int hpw;  // query heads per workgroup (min(G, waves))
  int nhb;  // head blocks per KV head (G / hpw)
  int rb;   // query rows per workgroup ((waves / hpw) * mq)
  int nqc;  // row blocks (ceil(m / rb))
};
__host__ __device__ inline Plan make_plan(int H, int Hkv, int m, int mq, int waves) {
  Plan p;
  const int G = H / Hkv;
  p.hpw = G < waves ? G : waves;
  p.nhb = G / p.hpw;
  p.rb = (waves / p.hpw) * mq;
  p.nqc = (m + p.rb - 1) / p.rb;
  return p;
}

template <typename ET, int HD> struct Lds {
  static constexpr int kWaves = waves_for(HD);
  static constexpr int kThreadsA = kWaves * kWave;
  static constexpr int KROW = HD * static_cast<int>(sizeof(ET));  // bytes of a K/V row
  static constexpr int KSTR = KROW + 16;                          // padded K row stride (bank spread)
  static constexpr int CPR = KROW / 16;                           // 16-byte chunks per row
  static constexpr int NL = KT * CPR / kThreadsA;                 // chunks per thread per tile (K or V)
  static constexpr size_t k_off = 0;
  static constexpr size_t v_off = k_off + static_cast<size_t>(KT) * KSTR;
  static constexpr size_t q_off = v_off + static_cast<size_t>(KT) * KROW;
  template <int MQ> static constexpr size_t p_off() { return q_off + sizeof(float) * kWaves * MQ * HD; }
  template <int MQ> static constexpr size_t bytes() { return p_off<MQ>() + sizeof(float) * kWaves * MQ * KT; }
};

template <typename ET, int HD>
__device__ __forceinline__ void load_tile(const ET* kc, const ET* vc, size_t kvbase, int k0, int klast,
                                          v4u (&kr)[Lds<ET, HD>::NL], v4u (&vr)[Lds<ET, HD>::NL]) {
  using L = Lds<ET, HD>;
#pragma unroll
  for (int i = 0; i < L::NL; ++i) {
    const int c = threadIdx.x + i * L::kThreadsA;
    const int row = c / L::CPR, col = c - row * L::CPR;
    const size_t g = (kvbase + min(k0 + row, klast)) * HD + static_cast<size_t>(col) * Cvt<ET>::n;
    kr[i] = *reinterpret_cast<const v4u*>(kc + g);
    vr[i] = *reinterpret_cast<const v4u*>(vc + g);
  }
}

template <typename ET, int HD>
__device__ __forceinline__ void store_tile(char* ks, char* vs, const v4u (&kr)[Lds<ET, HD>::NL],
                                           const v4u (&vr)[Lds<ET, HD>::NL]) {
  using L = Lds<ET, HD>;
#pragma unroll
  for (int i = 0; i < L::NL; ++i) {
    const int c = threadIdx.x + i * L::kThreadsA;
    const int row = c / L::CPR, col = c - row * L::CPR;
    *reinterpret_cast<v4u*>(ks + row * L::KSTR + col * 16) = kr[i];
    *reinterpret_cast<v4u*>(vs + row * L::KROW + col * 16) = vr[i];
  }
}

template <typename ET, int HD, int MQ>
__global__ __launch_bounds__(waves_for(HD) * kWave) __attribute__((amdgpu_waves_per_eu(waves_for(HD) / 4))) void attn_kernel(
    AttnArgs a) {
  using L = Lds<ET, HD>;
  constexpr int kThreadsA = L::kThreadsA;
  constexpr int DPL = HD / kWave;  // query dims per lane (staging q)
  constexpr int CE = Cvt<ET>::n;   // elements per 16-byte chunk
  constexpr int VCPR = HD / CE;    // 16-byte chunks per V row
  constexpr int NG = kWave / VCPR; // key groups in P.V
  static_assert(kWave % VCPR == 0 && KT % NG == 0, "P.V lane split");
  static_assert(L::NL * kThreadsA == KT * L::CPR, "tile chunks must split evenly over the threads");

  extern __shared__ uint4 smem_a[];
  char* sm = reinterpret_cast<char*>(smem_a);
  char* ks = sm + L::k_off;
  ET* vs = reinterpret_cast<ET*>(sm + L::v_off);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  float (*qs)[HD] = reinterpret_cast<float (*)[HD]>(sm + L::q_off) + wave * MQ;
  float (*ps)[KT] = reinterpret_cast<float (*)[KT]>(sm + L::template p_off<MQ>()) + wave * MQ;
  __shared__ int last_sh;

  const int H = a.H, Hkv = a.Hkv, m = a.m;
  const Plan pl = make_plan(H, Hkv, m, MQ, L::kWaves);
  const int G = H / Hkv;
  const int hb = blockIdx.x % pl.nhb;
  const int kvh = (blockIdx.x / pl.nhb) % Hkv;
  const int b = blockIdx.x / (pl.nhb * Hkv);
  const int s = blockIdx.y, qc = blockIdx.z;
  const int h = kvh * G + hb * pl.hpw + wave % pl.hpw;
  const int i0 = qc * pl.rb + (wave / pl.hpw) * MQ;
  const int nrows = max(0, min(MQ, m - i0));
  const int Lb = a.len[b];
  const int n_keys = max(0, min(Lb + m, a.max_ctx));
  const int per = (n_keys + a.n_split - 1) / a.n_split;
  const int kbeg = s * per;
  // keys past the workgroup's last visible one are not read
  const int wg_last_row = min(m, (qc + 1) * pl.rb) - 1;
  const int kend = min(min(kbeg + per, n_keys), max(0, Lb + wg_last_row + 1));
  const float scale = 1.0f / sqrtf(static_cast<float>(HD));
  const int qld = H * HD;
  const ET* kc = static_cast<const ET*>(a.kc);
  const ET* vc = static_cast<const ET*>(a.vc);
  const size_t kvbase = ((static_cast<size_t>(a.layer) * a.kvB + b) * Hkv + kvh) * a.max_ctx;

  // tile loads: chunk c = tid + i * 256 -> (row c / CPR, column chunk c % CPR);
  // rows are clamped into [k0, kend) (row 0 for an empty split), so every
  // load is unconditional; a prefetch past the last tile re-reads it
  const int klast = max(kend - 1, 0);
  v4u kr[L::NL], vr[L::NL];
  load_tile<ET, HD>(kc, vc, kvbase, kbeg, klast, kr, vr);
  // this wave's query rows, pre-scaled (rows past nrows repeat the last row;
  // their results are never written)
#pragma unroll
  for (int r = 0; r < MQ; ++r) {
    const float* qr = a.q + static_cast<size_t>(b * m + min(i0 + r, m - 1)) * qld + h * HD + lane * DPL;
#pragma unroll
    for (int k = 0; k < DPL; ++k) qs[r][lane * DPL + k] = qr[k] * scale;
  }
  // P.V accumulators: chunk vch of the V rows, keys vg, vg + NG, ... of each tile
  const int vch = lane % VCPR, vg = lane / VCPR;
  float mrow[MQ], lrow[MQ], o[MQ][CE];
#pragma unroll
  for (int r = 0; r < MQ; ++r) {
    mrow[r] = -INFINITY;
    lrow[r] = 0.f;
#pragma unroll
    for (int k = 0; k < CE; ++k) o[r][k] = 0.f;
  }

  for (int k0 = kbeg; k0 < kend; k0 += KT) {
    const int nt = min(KT, kend - k0);
    __syncthreads();  // previous tile fully consumed
    store_tile<ET, HD>(ks, reinterpret_cast<char*>(vs), kr, vr);
    __syncthreads();
    load_tile<ET, HD>(kc, vc, kvbase, k0 + KT, klast, kr, vr);
    // scores: lane = key; the key row in float32 registers
    float kf[HD];
#pragma unroll
    for (int c = 0; c < L::CPR; ++c)
      Cvt<ET>::run(*reinterpret_cast<const v4u*>(ks + lane * L::KSTR + c * 16), kf + c * CE);
    // 8 dimensions at a time for every row: MQ x 2 independent FMA chains
    float t[MQ][2];
#pragma unroll
    for (int r = 0; r < MQ; ++r) t[r][0] = t[r][1] = 0.f;
#pragma unroll
    for (int c = 0; c < HD; c += 8) {
#pragma unroll
      for (int r = 0; r < MQ; ++r) {
        const float4 qa = *reinterpret_cast<const float4*>(&qs[r][c]);
        const float4 qb = *reinterpret_cast<const float4*>(&qs[r][c + 4]);
        t[r][0] = fmaf(qa.x, kf[c], t[r][0]);
        t[r][1] = fmaf(qa.y, kf[c + 1], t[r][1]);
        t[r][0] = fmaf(qa.z, kf[c + 2], t[r][0]);
        t[r][1] = fmaf(qa.w, kf[c + 3], t[r][1]);
        t[r][0] = fmaf(qb.x, kf[c + 4], t[r][0]);
        t[r][1] = fmaf(qb.y, kf[c + 5], t[r][1]);
        t[r][0] = fmaf(qb.z, kf[c + 6], t[r][0]);
        t[r][1] = fmaf(qb.w, kf[c + 7], t[r][1]);
      }
    }
#pragma unroll
    for (int r = 0; r < MQ; ++r) ps[r][lane] = t[r][0] + t[r][1];
    // online softmax; p overwrites the score (same lane).  All MQ rows run
    // branch-free so their reductions interleave; rows past nrows are never
    // written out.
#pragma unroll
    for (int r = 0; r < MQ; ++r) {
      const bool valid = lane < nt && k0 + lane <= Lb + i0 + r;
      const float sv = valid ? ps[r][lane] : -INFINITY;
      const float mnew = fmaxf(mrow[r], wave_max(sv));
      const bool live = mnew != -INFINITY;
      const float alpha = live ? expf(mrow[r] - mnew) : 1.f;
      const float p = (valid && live) ? expf(sv - mnew) : 0.f;
      lrow[r] = lrow[r] * alpha + wave_sum(p);
      mrow[r] = mnew;
#pragma unroll
      for (int k = 0; k < CE; ++k) o[r][k] *= alpha;
      ps[r][lane] = p;
    }
    __syncthreads();
    // P.V over the tile: this lane's keys vg + NG t (keys past nt have p = 0
    // and finite V rows: the clamped copies of the last one)
#pragma unroll 4
    for (int t = 0; t < KT / NG; ++t) {
      const int j = vg + t * NG;
      float vf[CE];
      Cvt<ET>::run(*reinterpret_cast<const v4u*>(vs + j * HD + vch * CE), vf);
#pragma unroll
      for (int r = 0; r < MQ; ++r) {
        const float pj = ps[r][j];
#pragma unroll
        for (int k = 0; k < CE; ++k) o[r][k] = fmaf(pj, vf[k], o[r][k]);
      }
    }
  }
  // the key groups of each chunk, summed across lanes (every lane of a chunk
  // ends with the same sum)
#pragma unroll
  for (int off = VCPR; off < kWave; off <<= 1)
#pragma unroll
    for (int r = 0; r < MQ; ++r)
#pragma unroll
      for (int k = 0; k < CE; ++k) o[r][k] += __shfl_xor(o[r][k], off, kWave);

  ET* xo = static_cast<ET*>(a.xo);
  if (a.n_split == 1) {
#pragma unroll
    for (int r = 0; r < MQ; ++r) {
      if (r < nrows && vg == 0) {
#pragma unroll
        for (int k = 0; k < CE; ++k)
          xo[static_cast<size_t>(b * m + i0 + r) * qld + h * HD + vch * CE + k] =
              Elt<ET>::from_f(lrow[r] > 0.f ? o[r][k] / lrow[r] : 0.f);
      }
    }
    return;
  }

  const int ns = a.n_split;  // <= 64: one split per lane in the merge
  const size_t prow0 = ((static_cast<size_t>(b) * H + h) * m + i0) * ns;
#pragma unroll
  for (int r = 0; r < MQ; ++r) {
    if (r < nrows) {
      const size_t prow = prow0 + static_cast<size_t>(r) * ns + s;
      if (vg == 0) {
#pragma unroll
        for (int k = 0; k < CE; ++k) a.part_o[prow * HD + vch * CE + k] = o[r][k];
      }
      if (lane == 0) a.part_ml[prow] = make_float2(mrow[r], lrow[r]);
    }
  }
  if (!last_block(a.counters + static_cast<size_t>(blockIdx.x) * gridDim.z + qc, ns, &last_sh)) return;

  // merge the splits of each of this wave's rows, in split order
  for (int r = 0; r < nrows; ++r) {
    const size_t pr = prow0 + static_cast<size_t>(r) * ns;
    const float2 ml = (lane < ns) ? a.part_ml[pr + lane] : make_float2(-INFINITY, 0.f);
    const float M = wave_max(ml.x);
    const float w = (ml.x == -INFINITY) ? 0.f : expf(ml.x - M);
    const float l = wave_sum(ml.y * w);
    ps[0][lane] = w;
    float acc[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
    for (int s0 = 0; s0 < ns; s0 += 16) {
      float v[16][DPL];
#pragma unroll
      for (int t = 0; t < 16; ++t)
#pragma unroll
        for (int k = 0; k < DPL; ++k) v[t][k] = a.part_o[(pr + min(s0 + t, ns - 1)) * HD + lane * DPL + k];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const float ws = (s0 + t < ns) ? ps[0][s0 + t] : 0.f;
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[k] = fmaf(v[t][k], ws, acc[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k)
      xo[static_cast<size_t>(b * m + i0 + r) * qld + h * HD + lane * DPL + k] =
          Elt<ET>::from_f(l > 0.f ? acc[k] / l : 0.f);
  }
}

template <typename ET, int HD, int MQ>
hipError_t launch_mq(const AttnArgs& a, int B, hipStream_t s) {
  using L = Lds<ET, HD>;
  auto kern = attn_kernel<ET, HD, MQ>;
  constexpr size_t lds = L::template bytes<MQ>();
  static bool opt_in = false;
  if (!opt_in) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    opt_in = true;
  }
  const Plan pl = make_plan(a.H, a.Hkv, a.m, MQ, L::kWaves);
  if (pl.nqc != a.n_qc || a.n_split < 1 || a.n_split > kWave) return hipErrorInvalidValue;
  dim3 grid(B * a.Hkv * pl.nhb, a.n_split, pl.nqc);
  hipLaunchKernelGGL(kern, grid, dim3(L::kThreadsA), lds, s, a);
  return hipGetLastError();
}

// ---- matrix cores: bf16 K/V rows of head_dim 64 ---------------------------------
// The split kernel's work with v_mfma_f32_16x16x32_bf16 instead of float32
// FMAs.  With many query rows per KV head (G heads x the block's rows: 20 for
// a gamma = 4 pass of a 4:1 GQA model) the FMA form is bound by issuing its
// multiply-adds, not by the K/V bytes.
//
// Workgroup = (sequence b, KV head, context split, block of rows): its R = G x
// mb query rows (R <= 32, padded to RT x 16) against the keys it sees.  Its
// NW waves take 32-key blocks in turn (wave w: blocks w, w + NW, ...), each
// with its own online softmax, and are merged at the end in wave order; no
// wave waits for another inside the key loop.  Per block:
//  * S^T = K . Q^T: A is K straight from the cache (lane l: key row l % 16,
//    8 dims), B is the wave's queries (lane l: row l % 16, 8 dims), held in
//    registers for the whole pass.  Key tile t's A row i is key
//    8 (i / 4) + 4 t + i % 4 of the block, so that the result leaves lane l
//    with keys 8 (l / 16) .. + 7 of row l % 16;
//  * online softmax per row: the lane's 8 keys, then the 4 lanes of the row
//    (xor 16, xor 32);
//  * O^T += V^T . P^T: B is the lane's 8 probabilities as they are, A is V^T
//    read from a per-wave LDS block where the wave has written the block's V
//    rows transposed (dimension-major), and O^T leaves each row's output in
//    the lanes that hold its softmax state, so rescaling needs no exchange.
// The queries and probabilities enter as bf16 pairs x = hi + lo (hi the bf16
// rounding of x, lo that of the remainder): the pair carries x to within
// 2^-18 relative, and K and V are bf16 already, so the products are those of
// the float32 form to within that, accumulated in float32.
namespace mfa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int NW = 2;        // waves per workgroup (1, 2, 4 and 8 measured; 2 fastest at B = 64 and 256)
constexpr int KB = 32;       // keys per wave block
constexpr int HD = 64;       // head_dim
constexpr int VTS = KB + 8;  // bf16 per dimension row of a wave's V^T block (16-byte aligned)
constexpr int RMAX = 32;     // query rows per workgroup

// Row blocks of a pass: workgroups of at most 32 query rows (G heads x mb
// rows), or of at most 16 when that still leaves fewer than two workgroups
// per CU (more, narrower workgroups with fewer registers each, rather than
// context splits and their merge).
__host__ __device__ inline int row_blocks(int B, int Hkv, int G, int m) {
  const int cap32 = RMAX / G > 1 ? RMAX / G : 1, cap16 = 16 / G > 1 ? 16 / G : 1;
  const int n32 = (m + cap32 - 1) / cap32;
  if (static_cast<long long>(B) * Hkv * n32 >= 512) return n32;
  return (m + cap16 - 1) / cap16;
}
__host__ __device__ inline int rows_per_block(int m, int nqc) { return (m + nqc - 1) / nqc; }

// e^x as 2^(x log2 e) with the hardware exponential (e^-inf = 0)
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(x);
  lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

// bf16 e of a 16-byte chunk of 8
__device__ __forceinline__ uint32_t half_of(const v4u& v, int e) {
  return (e & 1) ? (v[e >> 1] >> 16) : (v[e >> 1] & 0xffffu);
}

template <int RT>
__global__ __launch_bounds__(NW * kWave) void attn_mfma_kernel(AttnArgs a) {
  constexpr int ROWS = RT * 16;
  constexpr int VT_BYTES = NW * HD * VTS * 2;
  constexpr int OB_BYTES = NW * ROWS * HD * 4;
  constexpr int U_BYTES = VT_BYTES > OB_BYTES ? VT_BYTES : OB_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char su[U_BYTES];  // V^T blocks, then the merge
  __shared__ float2 sml[NW][ROWS];  // each wave's (max, weight) per row
  __shared__ float2 sfin[ROWS];     // the workgroup's (max, weight) per row
  __shared__ int last_sh;

  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int g16 = lane >> 4, c16 = lane & 15;
  const int H = a.H, Hkv = a.Hkv, m = a.m, G = H / Hkv;
  const int mb = rows_per_block(m, a.n_qc);
  const int kvh = blockIdx.x % Hkv, b = blockIdx.x / Hkv;
  const int sp = blockIdx.y, qc = blockIdx.z, ns = a.n_split;
  const int i_first = qc * mb;
  const int R = G * mb;
  const int Lb = a.len[b];
  const int n_keys = max(0, min(Lb + m, a.max_ctx));
  const int last_row = min(m, i_first + mb) - 1;
  const int kvis = max(0, min(n_keys, Lb + last_row + 1));  // keys the block's last row sees
  const int nblk = (kvis + KB - 1) / KB;
  const int per = (nblk + ns - 1) / ns;  // blocks per split
  const int kbeg = min(kvis, sp * per * KB);
  const int kend = min(kvis, kbeg + per * KB);
  const int qld = H * HD;
  const uint16_t* kc = static_cast<const uint16_t*>(a.kc);
  const uint16_t* vc = static_cast<const uint16_t*>(a.vc);
  const size_t kvbase = ((static_cast<size_t>(a.layer) * a.kvB + b) * Hkv + kvh) * a.max_ctx;

  // the wave's first block is in flight while the queries are set up
  const int klast = max(kend - 1, 0);
  const int vcq = lane & 7, vkq = lane >> 3;  // V staging: dims 8 vcq .., keys 4 vkq ..
  v4u kf[2][2], vf[4];
  auto load = [&](int kb) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = min(kb + 8 * (c16 >> 2) + 4 * kt + (c16 & 3), klast);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        kf[kt][ks] = *reinterpret_cast<const v4u*>(kc + (kvbase + key) * HD + ks * 32 + g16 * 8);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
      vf[t] = *reinterpret_cast<const v4u*>(vc + (kvbase + min(kb + 4 * vkq + t, klast)) * HD + vcq * 8);
  };
  int kb = kbeg + wave * KB;
  if (kb < kend) load(kb);

  // this lane's query row in each row tile: r = 16 rt + c16 -> (head g, row i)
  int lim[RT];  // last key the row sees (-1: a padding row or one past m)
  bf16x8_t qh[RT][2], ql[RT][2];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = rt * 16 + c16;
    const int g = r / mb, i = i_first + r % mb;
    const bool valid = r < R && i < m;
    lim[rt] = valid ? Lb + i : -1;
    const float* qr = a.q + static_cast<size_t>(b * m + (valid ? i : 0)) * qld + (kvh * G + (valid ? g : 0)) * HD;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const float4 x0 = *reinterpret_cast<const float4*>(qr + ks * 32 + g16 * 8);
      const float4 x1 = *reinterpret_cast<const float4*>(qr + ks * 32 + g16 * 8 + 4);
      const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 hi, lo;
        split_bf16(valid ? xs[e] * 0.125f : 0.f, hi, lo);  // scaled by 1 / sqrt(64)
        qh[rt][ks][e] = hi;
        ql[rt][ks][e] = lo;
      }
    }
  }

  f32x4_t o[RT][4];  // O^T: dims 16 dt + 4 g16 + j of row 16 rt + c16
  float mrow[RT], lrow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    mrow[rt] = -INFINITY;
    lrow[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[rt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  unsigned char* vt = su + wave * (HD * VTS * 2);
  for (; kb < kend; kb += NW * KB) {
    // S^T for the block
    f32x4_t sc[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) sc[rt][0] = sc[rt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8_t ka = __builtin_bit_cast(bf16x8_t, kf[kt][ks]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          sc[rt][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qh[rt][ks], sc[rt][kt], 0, 0, 0);
          sc[rt][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, ql[rt][ks], sc[rt][kt], 0, 0, 0);
        }
      }
    // the block's V rows into the wave's V^T block: dimension 8 vcq + e,
    // keys 4 vkq .. + 3 as one 8-byte write
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint2 w;
      w.x = half_of(vf[0], e) | (half_of(vf[1], e) << 16);
      w.y = half_of(vf[2], e) | (half_of(vf[3], e) << 16);
      *reinterpret_cast<uint2*>(vt + ((vcq * 8 + e) * VTS + 4 * vkq) * 2) = w;
    }
    const int kb_next = kb + NW * KB;
    if (kb_next < kend) load(kb_next);
    // online softmax; the lane's keys are kb + 8 g16 + 4 kt + j
    bf16x8_t ph[RT], pq[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float sv[8];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = kb + 8 * g16 + 4 * kt + j;
          sv[4 * kt + j] = (key < kend && key <= lim[rt]) ? sc[rt][kt][j] : -INFINITY;
        }
      float tm = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) tm = fmaxf(tm, sv[e]);
      tm = fmaxf(tm, __shfl_xor(tm, 16, kWave));
      tm = fmaxf(tm, __shfl_xor(tm, 32, kWave));
      const float mnew = fmaxf(mrow[rt], tm);
      const float mref = mnew == -INFINITY ? 0.f : mnew;  // no key seen yet: everything weighs 0
      const float alpha = exp_hw(mrow[rt] - mref);
      float ls = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = exp_hw(sv[e] - mref);
        ls += p;
        __bf16 hi, lo;
        split_bf16(p, hi, lo);
        ph[rt][e] = hi;
        pq[rt][e] = lo;
      }
      lrow[rt] = lrow[rt] * alpha + ls;
      mrow[rt] = mnew;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[rt][dt] *= alpha;
    }
    // O^T += V^T . P^T
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(vt + ((dt * 16 + c16) * VTS + 8 * g16) * 2);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, ph[rt], o[rt][dt], 0, 0, 0);
        o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pq[rt], o[rt][dt], 0, 0, 0);
      }
    }
  }

  // merge the waves in wave order: (max, weight) per row through LDS, then
  // each wave's rescaled output
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float l = lrow[rt] + __shfl_xor(lrow[rt], 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    if (g16 == 0) sml[wave][rt * 16 + c16] = make_float2(mrow[rt], l);
  }
  __syncthreads();  // also: every wave is done with its V^T block
  float* ob = reinterpret_cast<float*>(su);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + c16;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sml[w][row].x);
    const float Mref = M == -INFINITY ? 0.f : M;
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float2 ml = sml[w][row];
      L = fmaf(ml.y, exp_hw(ml.x - Mref), L);
    }
    const float wown = exp_hw(mrow[rt] - Mref);
    const float sc = ns == 1 ? (L > 0.f ? wown / L : 0.f) : wown;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      *reinterpret_cast<float4*>(ob + (static_cast<size_t>(wave) * ROWS + row) * HD + dt * 16 + g16 * 4) =
          make_float4(o[rt][dt][0] * sc, o[rt][dt][1] * sc, o[rt][dt][2] * sc, o[rt][dt][3] * sc);
    if (wave == 0 && g16 == 0) sfin[row] = make_float2(M, L);
  }
  __syncthreads();
  // rows summed over the waves in wave order: the output (one split) or this
  // split's partial (unnormalised output, max, weight)
  uint16_t* xo = static_cast<uint16_t*>(a.xo);
  constexpr int Q4 = HD / 4;
  for (int idx = threadIdx.x; idx < R * Q4; idx += NW * kWave) {
    const int r = idx / Q4, d4 = idx - r * Q4;
    const int g = r / mb, i = i_first + r % mb;
    if (i >= m) continue;
    float4 acc = *reinterpret_cast<const float4*>(ob + static_cast<size_t>(r) * HD + 4 * d4);
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      const float4 v = *reinterpret_cast<const float4*>(ob + (static_cast<size_t>(w) * ROWS + r) * HD + 4 * d4);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const int h = kvh * G + g;
    if (ns == 1) {
      uint2 pk;
      pk.x = static_cast<uint32_t>(f2bf(acc.x)) | (static_cast<uint32_t>(f2bf(acc.y)) << 16);
      pk.y = static_cast<uint32_t>(f2bf(acc.z)) | (static_cast<uint32_t>(f2bf(acc.w)) << 16);
      *reinterpret_cast<uint2*>(xo + static_cast<size_t>(b * m + i) * qld + h * HD + 4 * d4) = pk;
    } else {
      const size_t prow = ((static_cast<size_t>(b) * H + h) * m + i) * ns + sp;
      *reinterpret_cast<float4*>(a.part_o + prow * HD + 4 * d4) = acc;
      if (d4 == 0) a.part_ml[prow] = sfin[r];
    }
  }
  if (ns == 1) return;
  if (!last_block(a.counters + static_cast<size_t>(blockIdx.x) * gridDim.z + qc, ns, &last_sh)) return;
  // The last workgroup of the row block merges the splits.  A wave per row
  // takes the splits' weights exp(m_s - max) (lane = split) and their sum;
  // then each thread sums its 4 dimensions of a row over the splits in split
  // order, 8 partial loads in flight at a time.
  float* swt = ob;  // [ROWS][64] split weights (the merge area is free again)
  for (int r = wave; r < R; r += NW) {
    const int g = r / mb, i = i_first + r % mb;
    if (i >= m) continue;
    const size_t p0 = ((static_cast<size_t>(b) * H + kvh * G + g) * m + i) * ns;
    const float2 ml = lane < ns ? a.part_ml[p0 + lane] : make_float2(-INFINITY, 0.f);
    const float M = wave_max(ml.x);
    const float w = exp_hw(ml.x - (M == -INFINITY ? 0.f : M));
    const float L = wave_sum(ml.y * w);
    swt[r * kWave + lane] = w;
    if (lane == 0) sfin[r] = make_float2(M, L);
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < R * Q4; idx += NW * kWave) {
    const int r = idx / Q4, d4 = idx - r * Q4;
    const int g = r / mb, i = i_first + r % mb;
    if (i >= m) continue;
    const int h = kvh * G + g;
    const size_t p0 = ((static_cast<size_t>(b) * H + h) * m + i) * ns;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int t0 = 0; t0 < ns; t0 += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = *reinterpret_cast<const float4*>(a.part_o + (p0 + min(t0 + u, ns - 1)) * HD + 4 * d4);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = t0 + u < ns ? swt[r * kWave + t0 + u] : 0.f;
        acc.x = fmaf(v[u].x, w, acc.x);
        acc.y = fmaf(v[u].y, w, acc.y);
        acc.z = fmaf(v[u].z, w, acc.z);
        acc.w = fmaf(v[u].w, w, acc.w);
      }
    }
    const float L = sfin[r].y, inv = L > 0.f ? 1.f / L : 0.f;
    uint2 pk;
    pk.x = static_cast<uint32_t>(f2bf(acc.x * inv)) | (static_cast<uint32_t>(f2bf(acc.y * inv)) << 16);
    pk.y = static_cast<uint32_t>(f2bf(acc.z * inv)) | (static_cast<uint32_t>(f2bf(acc.w * inv)) << 16);
    *reinterpret_cast<uint2*>(xo + static_cast<size_t>(b * m + i) * qld + h * HD + 4 * d4) = pk;
  }
}

template <int RT>
hipError_t launch_rt(const AttnArgs& a, int B, hipStream_t s) {
  hipLaunchKernelGGL((attn_mfma_kernel<RT>), dim3(B * a.Hkv, a.n_split, a.n_qc), dim3(NW * kWave), 0, s, a);
  return hipGetLastError();
}

hipError_t launch(const AttnArgs& a, int B, hipStream_t s) {
  const int G = a.H / a.Hkv;
  if (a.n_qc != row_blocks(B, a.Hkv, G, a.m) || a.n_split < 1 || a.n_split > kWave || !a.counters)
    return hipErrorInvalidValue;
  if (a.n_split > 1 && (!a.part_o || !a.part_ml)) return hipErrorInvalidValue;
  const int R = G * rows_per_block(a.m, a.n_qc);
  if (R > RMAX) return hipErrorInvalidValue;
  return R <= 16 ? launch_rt<1>(a, B, s) : launch_rt<2>(a, B, s);
}

}  // namespace mfa

// The matrix-core kernel takes the split path's bf16 passes of head_dim 64.
bool mfma_attention(bool bf16, int H, int Hkv, int hd) {
  return bf16 && hd == mfa::HD && Hkv > 0 && H % Hkv == 0 && H / Hkv <= mfa::RMAX;
}

// ---- short passes: m <= 8 query rows, contexts up to kDecodeMaxCtx -------------
// One workgroup per (sequence, query head, block of RW query rows): with few
// sequences the rows are split until there are enough workgroups to spread
// over the chip, and each workgroup still sees the whole context, so no
// workgroup waits for another.  Its NWV waves split the keys (wave w takes
// KTD-key tiles w, w + NWV, ...) and merge their partial (max, sum, output)
// rows in LDS at the end, in wave order.
// Lane l of a wave works on 16-byte chunk chi = l % CPR of rows
// rho = l / CPR, rho + RPI, ... of the tile: the K and V loads are coalesced
// (RPI whole rows per load instruction).  Scores: a lane dots its K chunk with
// the same chunk of each query row (held in registers) and the CPR lanes of a
// row add their parts with DPP moves inside the 16-lane row, so every lane of
// the group holds the row's scores.  The softmax update and P.V then need no
// data movement: the lane scales its V chunks by its rows' p; the RPI row
// groups are summed once, after the last tile.
constexpr int kDecWaves = 8;
constexpr int kDecodeMaxCtx = 2048;
// Past this many (sequence, query head, row) units a pass takes the split
// kernel instead: its workgroups serve the query heads of one KV head
// together, where this kernel re-reads the KV head once per query head.
// Measured on MI355X, head_dim 64, 16:4 heads, ~300 keys: B = 64 and 256
// verify passes (5 rows) ran 12% and 34% faster that way, B = 256 one-row
// passes 15% faster; B = 64 one-row passes (1024 units) ran 6% slower, and
// 8 or fewer sequences slower still.
constexpr long long kDecodeMaxUnits = 4096;

template <typename ET, int HD> struct Dec {
  static constexpr int CE = 16 / static_cast<int>(sizeof(ET));        // elements per 16-byte chunk
  static constexpr int CPR = HD / CE;                                 // chunks per K/V row
  static constexpr int RPI = kWave / CPR;                             // rows per load instruction
};


// NWV waves of KTD-key tiles: 8 x 64 by default, 16 x 32 for blocks of at
// most 2 rows (their registers fit the 4 waves per SIMD that 16-wave
// workgroups need; at ~300 keys all 16 waves then hold keys, where 3 of 8
// waves of 64-key tiles sat idle: 8B-shaped step 3.639 -> 3.619 ms,
// 0.6B-shaped drafter rounds 7.45 -> 7.39 ms).
template <typename ET, int HD, int RW, int NWV, int KTD>
__global__ __launch_bounds__(NWV * kWave) __attribute__((amdgpu_waves_per_eu(NWV / 4))) void attn_decode_kernel(
    AttnArgs a, int n_rb) {
  using D = Dec<ET, HD>;
  constexpr int CE = D::CE, CPR = D::CPR, RPI = D::RPI, NI = KTD / RPI, NT = NWV * kWave;
  static_assert(NI >= 1 && KTD % RPI == 0, "keys per tile");
  static_assert(CPR == 8 || CPR == 16, "K/V rows of 8 or 16 chunks");
  static_assert(NWV <= 16, "the merge gives each wave one of 16 lanes");
  __shared__ float mo[NWV][RW][HD];
  __shared__ float2 ml[NWV][RW];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;

  const int H = a.H, Hkv = a.Hkv, m = a.m, S = a.dsplit;
  const int sp = blockIdx.x % S;          // context split of this workgroup
  const int unit = blockIdx.x / S;
  const int rb = unit % n_rb;
  const int h = (unit / n_rb) % H;
  const int b = unit / (n_rb * H);
  const int i0 = rb * RW;                 // first query row of the block
  const int kvh = h / (H / Hkv);
  const int Lb = a.len[b];
  // keys the block's rows may see: positions 0 .. Lb + i0 + RW - 1; split sp
  // takes tiles [t_lo, t_hi) of them
  const int kend = max(0, min(min(Lb + m, Lb + i0 + RW), a.max_ctx));
  const int ntiles_all = (kend + KTD - 1) / KTD;
  const int tps = (ntiles_all + S - 1) / S;
  const int t_lo = min(sp * tps, ntiles_all), t_hi = min(t_lo + tps, ntiles_all);
  const int ntiles = t_hi - t_lo;
  const int trips = (ntiles + NWV - 1) / NWV;
  const int qld = H * HD;
  const ET* kc = static_cast<const ET*>(a.kc);
  const ET* vc = static_cast<const ET*>(a.vc);
  const size_t kvbase = ((static_cast<size_t>(a.layer) * a.kvB + b) * Hkv + kvh) * a.max_ctx;
  const float scale = 1.0f / sqrtf(static_cast<float>(HD));
  const int rho = lane / CPR, chi = lane % CPR;

  // this lane's chunk of each query row of the block, pre-scaled (rows past
  // m repeat row m - 1; their results are never written)
  float qr[RW][CE];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const float* src = a.q + static_cast<size_t>(b * m + min(i0 + r, m - 1)) * qld + h * HD + chi * CE;
#pragma unroll
    for (int e = 0; e < CE; ++e) qr[r][e] = src[e] * scale;
  }
  float mrow[RW], lrow[RW], o[RW][CE];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    mrow[r] = -INFINITY;
    lrow[r] = 0.f;
#pragma unroll
    for (int e = 0; e < CE; ++e) o[r][e] = 0.f;
  }

  for (int it = 0; it < trips; ++it) {
    const int tile = it * NWV + wave;
    const int k0 = (t_lo + tile) * KTD;  // this wave's tile
    // a tile past the split's keys would only load clamped rows and mask them
    // all: skip it (the CU's vector memory pipe is what the waves share)
    if (tile >= ntiles) continue;
    const int klast = max(kend - 1, 0);
    v4u kr[NI], vr[NI];
#pragma unroll
    for (int c = 0; c < NI; ++c) {
      const size_t g = (kvbase + min(k0 + c * RPI + rho, klast)) * HD + chi * CE;
      kr[c] = *reinterpret_cast<const v4u*>(kc + g);
      vr[c] = *reinterpret_cast<const v4u*>(vc + g);
    }
    // scores of keys k0 + c * RPI + rho against each row
    float sc[RW][NI];
#pragma unroll
    for (int c = 0; c < NI; ++c) {
      float kf[CE];
      Cvt<ET>::run(kr[c], kf);
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        float t0 = 0.f, t1 = 0.f;
#pragma unroll
        for (int e = 0; e < CE; e += 2) {
          t0 = fmaf(qr[r][e], kf[e], t0);
          t1 = fmaf(qr[r][e + 1], kf[e + 1], t1);
        }
        sc[r][c] = group_sum<CPR>(t0 + t1);
      }
    }
    // online softmax per row (row i0 + r sees keys 0 .. Lb + i0 + r), then
    // this lane's V chunks weighted by its rows' p
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      float mt = -INFINITY;
#pragma unroll
      for (int c = 0; c < NI; ++c) {
        const int key = k0 + c * RPI + rho;
        if (!(key < kend && key <= Lb + i0 + r)) sc[r][c] = -INFINITY;
        mt = fmaxf(mt, sc[r][c]);
      }
      const float mnew = fmaxf(mrow[r], groups_max<CPR>(mt));
      const bool live = mnew != -INFINITY;
      const float alpha = live ? expf(mrow[r] - mnew) : 1.f;
      float ls = 0.f;
#pragma unroll
      for (int c = 0; c < NI; ++c) {
        sc[r][c] = (live && sc[r][c] != -INFINITY) ? expf(sc[r][c] - mnew) : 0.f;
        ls += sc[r][c];
      }
      lrow[r] = lrow[r] * alpha + groups_sum<CPR>(ls);
      mrow[r] = mnew;
#pragma unroll
      for (int e = 0; e < CE; ++e) o[r][e] *= alpha;
    }
#pragma unroll
    for (int c = 0; c < NI; ++c) {
      float vf[CE];
      Cvt<ET>::run(vr[c], vf);
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int e = 0; e < CE; ++e) o[r][e] = fmaf(sc[r][c], vf[e], o[r][e]);
    }
  }
  // the row groups' parts of each chunk, then the waves, in order
#pragma unroll
  for (int r = 0; r < RW; ++r) {
#pragma unroll
    for (int e = 0; e < CE; ++e) o[r][e] = groups_sum<CPR>(o[r][e]);
    if (rho == 0) {
#pragma unroll
      for (int e = 0; e < CE; ++e) mo[wave][r][chi * CE + e] = o[r][e];
    }
    if (lane == 0) ml[wave][r] = make_float2(mrow[r], lrow[r]);
  }
  __syncthreads();
  // The waves' weights exp(m_w - max) and the row's total weight l, once per
  // row: lanes 16k .. 16k + 15 of wave 0 take row r0 + k, lane w its wave's
  // partial (l summed by a 16-lane butterfly); then every output element is
  // its waves' partials weighted in wave order.
  __shared__ float wts[NWV][RW];
  __shared__ float lsum[RW];
  if (wave == 0) {
    const int w = lane & 15, k = lane >> 4;
#pragma unroll
    for (int r0 = 0; r0 < RW; r0 += 4) {
      const int r = r0 + k < RW ? r0 + k : RW - 1;
      float Mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < NWV; ++j) Mx = fmaxf(Mx, ml[j][r].x);
      float wt = 0.f, lw = 0.f;
      if (w < NWV) {
        const float2 v = ml[w][r];
        wt = (v.x == -INFINITY) ? 0.f : expf(v.x - Mx);
        lw = v.y * wt;
      }
      lw = group_sum<16>(lw);
      if (r0 + k < RW) {
        if (w < NWV) wts[w][r] = wt;
        if (w == 0) lsum[r] = lw;
      }
    }
  }
  __syncthreads();
  ET* xo = static_cast<ET*>(a.xo);
  const int nr = max(0, min(RW, m - i0));
  for (int idx = threadIdx.x; idx < nr * HD; idx += NT) {
    const int r = idx / HD, dd = idx - r * HD;
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) acc = fmaf(mo[w][r][dd], wts[w][r], acc);
    const float l = lsum[r];
    const int row = b * m + i0 + r;
    if (S == 1) {
      xo[static_cast<size_t>(row) * qld + h * HD + dd] = Elt<ET>::from_f(l > 0.f ? acc / l : 0.f);
    } else {
      // this split's partial: the unnormalised output, its max and weight
      const size_t pi = (static_cast<size_t>(row) * H + h) * S + sp;
      a.dpo[pi * HD + dd] = acc;
      if (dd == 0) {
        float Mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < NWV; ++w) Mx = fmaxf(Mx, ml[w][r].x);
        a.dpml[pi] = make_float2(Mx, l);
      }
    }
  }
}

// Output rows from the context splits' partials (a traced pass: the O linear
// otherwise merges them while staging its input).  One workgroup per
// (row, head); thread j takes VE consecutive head dimensions.
template <typename ET, int HD>
__global__ __launch_bounds__(HD) void attn_merge_kernel(AttnArgs a) {
  constexpr int VE = 16 / static_cast<int>(sizeof(ET));
  const int row = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int dd0 = threadIdx.x * VE;
  if (dd0 >= HD) return;
  const size_t pi = (static_cast<size_t>(row) * a.H + h) * a.dsplit;
  AttnPart<VE> part;
  attn_part_load<VE>(a.dpo + pi * HD, a.dpml + pi, a.dsplit, HD, dd0, part);
  float out[VE];
  attn_part_merge<VE>(part, a.dsplit, out);
  ET* xo = static_cast<ET*>(a.xo) + static_cast<size_t>(row) * a.H * HD + h * HD + dd0;
#pragma unroll
  for (int e = 0; e < VE; ++e) xo[e] = Elt<ET>::from_f(out[e]);
}

// Query rows per workgroup: split the m rows until B * H * blocks reaches
// about one workgroup per CU, and to at most rw_max rows (the register budget:
// 3 rows for 16-chunk K/V rows, 5 for 8-chunk rows).
inline int decode_rows_per_block(int B, int H, int m, int rw_max) {
  const int units = B * H;
  int blocks = (256 + units - 1) / units;
  blocks = max(1, min(blocks, m));
  return min((m + blocks - 1) / blocks, rw_max);
}

template <typename ET, int HD, int RW>
hipError_t launch_decode_rw(const AttnArgs& a, int B, hipStream_t s) {
  const int n_rb = (a.m + RW - 1) / RW;
  constexpr int NWV = RW <= 2 ? 16 : kDecWaves, KTD = RW <= 2 ? 32 : KT;
  if (a.dsplit < 1 || a.dsplit > kMaxAttnSplits || (a.dsplit > 1 && (!a.dpo || !a.dpml))) return hipErrorInvalidValue;
  // A split one-row pass gives each workgroup a quarter or half of the
  // context (≈ 75-150 keys at 300): 4 waves of 32-key tiles, where 16 left
  // most waves idle and lengthened the merge (0.6B-shaped drafter round
  // 2.779 -> 2.766 ms, the second workload's 2-layer drafter round 0.3224 ->
  // 0.3201 ms; 8 waves in between).
  if constexpr (RW == 1) {
    if (a.dsplit > 1) {
      constexpr int SW = 4;
      hipLaunchKernelGGL((attn_decode_kernel<ET, HD, RW, SW, KTD>), dim3(B * a.H * n_rb * a.dsplit), dim3(SW * kWave),
                         0, s, a, n_rb);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((attn_decode_kernel<ET, HD, RW, NWV, KTD>), dim3(B * a.H * n_rb * a.dsplit), dim3(NWV * kWave), 0,
                     s, a, n_rb);
  return hipGetLastError();
}

template <typename ET, int HD>
hipError_t launch_decode(const AttnArgs& a, int B, hipStream_t s) {
  constexpr int rw_max = Dec<ET, HD>::CPR == 16 ? 3 : 5;
  switch (decode_rows_per_block(B, a.H, a.m, rw_max)) {
    case 1: return launch_decode_rw<ET, HD, 1>(a, B, s);
    case 2: return launch_decode_rw<ET, HD, 2>(a, B, s);
    case 3: return launch_decode_rw<ET, HD, 3>(a, B, s);
    case 4: return launch_decode_rw<ET, HD, (rw_max >= 4 ? 4 : 3)>(a, B, s);
    default: return launch_decode_rw<ET, HD, (rw_max >= 5 ? 5 : 3)>(a, B, s);
  }
}

template <typename ET, int HD>
constexpr bool decode_fits() {
  return Dec<ET, HD>::CPR == 8 || Dec<ET, HD>::CPR == 16;
}

// Query rows per wave: the rows of a block spread over the waves of a head.
int rows_per_wave(int H, int Hkv, int hd, int m) {
  const int G = H / Hkv, waves = waves_for(hd);
  const int wph = waves / (G < waves ? G : waves);
  const int mq = (m + wph - 1) / wph;
  return mq < 8 ? mq : 8;
}

template <typename ET, int HD>
hipError_t launch_hd(const AttnArgs& a, int B, hipStream_t s) {
  switch (rows_per_wave(a.H, a.Hkv, HD, a.m)) {
    case 1: return launch_mq<ET, HD, 1>(a, B, s);
    case 2: return launch_mq<ET, HD, 2>(a, B, s);
    case 3: return launch_mq<ET, HD, 3>(a, B, s);
    case 4: return launch_mq<ET, HD, 4>(a, B, s);
    case 5: return launch_mq<ET, HD, 5>(a, B, s);
    case 6: return launch_mq<ET, HD, 6>(a, B, s);
    case 7: return launch_mq<ET, HD, 7>(a, B, s);
    default: return launch_mq<ET, HD, 8>(a, B, s);
  }
}

}  // namespace

bool attn_supported(int H, int Hkv, int hd) {
  if (hd != 64 && hd != 128) return false;
  if (Hkv <= 0 || H % Hkv != 0) return false;
  const int G = H / Hkv, waves = waves_for(hd);
  return G <= waves ? (waves % G == 0) : (G % waves == 0);
}

int attn_row_blocks(bool bf16, int B, int H, int Hkv, int hd, int m) {
  if (mfma_attention(bf16, H, Hkv, hd)) return mfa::row_blocks(B, Hkv, H / Hkv, m);
  return make_plan(H, Hkv, m, rows_per_wave(H, Hkv, hd, m), waves_for(hd)).nqc;
}

int attn_num_splits(bool bf16, int B, int H, int Hkv, int hd, int m, int max_ctx) {
  if (mfma_attention(bf16, H, Hkv, hd)) {
    // context splits only while the row blocks leave fewer workgroups than
    // CUs: about one per CU, each split at least two blocks per wave (one
    // block per wave measured slower on 2048-token contexts at B = 1)
    const int units = B * Hkv * mfa::row_blocks(B, Hkv, H / Hkv, m);
    if (units >= 256) return 1;
    int n = (256 + units - 1) / units;
    n = min(n, (max_ctx + 2 * mfa::NW * mfa::KB - 1) / (2 * mfa::NW * mfa::KB));
    return max(1, min(n, kWave));
  }
  const Plan pl = make_plan(H, Hkv, m, rows_per_wave(H, Hkv, hd, m), waves_for(hd));
  const int units = B * Hkv * pl.nhb * pl.nqc;  // workgroups per split
  int n = (512 + units - 1) / units;
  n = min(n, (max_ctx + KT - 1) / KT);
  return max(1, min(n, kWave));
}

size_t attn_counters(bool bf16, int B, int H, int Hkv, int hd, int m) {
  if (mfma_attention(bf16, H, Hkv, hd)) return static_cast<size_t>(B) * Hkv * mfa::row_blocks(B, Hkv, H / Hkv, m);
  const Plan pl = make_plan(H, Hkv, m, rows_per_wave(H, Hkv, hd, m), waves_for(hd));
  return static_cast<size_t>(B) * Hkv * pl.nhb * pl.nqc;
}

int attn_decode_splits(bool bf16, int hd, int B, int H, int m, int max_ctx) {
  if (!attn_decode_path(bf16, hd, m, max_ctx) || static_cast<long long>(B) * H * m >= kDecodeMaxUnits) return 1;
  const int cpr = hd / (bf16 ? 8 : 4);  // 16-byte chunks per K/V row
  const int rw = decode_rows_per_block(B, H, m, cpr == 16 ? 3 : 5);
  const long long units = static_cast<long long>(B) * H * ((m + rw - 1) / rw);
  return units >= 128 ? 1 : units >= 64 ? 2 : kMaxAttnSplits;
}

hipError_t launch_attn_merge(bool bf16, int hd, const AttnArgs& a, int rows, hipStream_t s) {
  if (a.dsplit < 2 || rows <= 0) return hipSuccess;
  const dim3 grid(rows * a.H);
  if (bf16) {
    if (hd == 128) hipLaunchKernelGGL((attn_merge_kernel<uint16_t, 128>), grid, dim3(128), 0, s, a);
    else hipLaunchKernelGGL((attn_merge_kernel<uint16_t, 64>), grid, dim3(64), 0, s, a);
  } else {
    if (hd == 128) hipLaunchKernelGGL((attn_merge_kernel<float, 128>), grid, dim3(128), 0, s, a);
    else hipLaunchKernelGGL((attn_merge_kernel<float, 64>), grid, dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

bool attn_decode_path(bool bf16, int hd, int m, int max_ctx) {
  if (m > 8 || max_ctx > kDecodeMaxCtx) return false;
  if (bf16) return hd == 128 ? decode_fits<uint16_t, 128>() : decode_fits<uint16_t, 64>();
  return hd == 128 ? decode_fits<float, 128>() : decode_fits<float, 64>();
}

hipError_t launch_attention(bool bf16, int hd, const AttnArgs& a, int B, hipStream_t s) {
  if (B <= 0 || a.m <= 0) return hipSuccess;
  if (!attn_supported(a.H, a.Hkv, hd)) return hipErrorInvalidValue;
  const bool decode = attn_decode_path(bf16, hd, a.m, a.max_ctx) && static_cast<long long>(B) * a.H * a.m < kDecodeMaxUnits;
  if (a.dsplit != 1 && (!decode || (!bf16 && hd != 64))) return hipErrorInvalidValue;  // splits: short-pass kernel only
  if (decode) {
    if (bf16) return hd == 128 ? launch_decode<uint16_t, 128>(a, B, s) : launch_decode<uint16_t, 64>(a, B, s);
    if (hd == 64) return launch_decode<float, 64>(a, B, s);
  }
  if (mfma_attention(bf16, a.H, a.Hkv, hd)) return mfa::launch(a, B, s);
  if (bf16) return hd == 128 ? launch_hd<uint16_t, 128>(a, B, s) : launch_hd<uint16_t, 64>(a, B, s);
  return hd == 128 ? launch_hd<float, 128>(a, B, s) : launch_hd<float, 64>(a, B, s);
}

}  // namespace sv
