// Matrix-core linear for the verify pass with more than 8 activation rows:
//   Y[M][N] (op) X[M][K] . W[N][K]^T, bf16 inputs, float32 accumulation.
//
// With B sequences the verify pass has M = B (gamma + 1) rows, and a prefill
// has B (P - 1).  The arithmetic per weight byte grows with M (first page,
// section "The speedup is borrowed, and there is a lender": the batch turns
// the same weight read into more work), so past a few rows the linear is a
// real dense contraction and belongs on MFMA.  The GEMV kernel would stream
// the weights once per 8 rows instead.
//
// Tiles: a workgroup computes BMT rows x BNT weight rows of Y with 2 x
// (BNT / 64) waves; each wave owns BMT/2 x 64 = (BMT/32) x 4 tiles of
// v_mfma_f32_16x16x32_bf16.  The tile is 256 x 256 (8 waves, one workgroup
// per CU) when the launch still has a workgroup per CU with it, else 128 x
// 128 (4 waves, two workgroups per CU), else 64 x 128.  A CU's vector memory
// path moves 64 bytes per clock: a 128 x 128 tile's K blocks take as many
// clocks to load as its MFMAs take to run, a 256 x 256 tile's half as many.
// The K dimension advances in blocks through a ring of LDS stages.  Fragment layouts (gfx950): A lane l holds
// row l % 16, k = 8 (l / 16) .. +7; B lane l holds column l % 16, the same k;
// D lane l holds rows 4 (l / 16) .. +3 of column l % 16.
//
// The epilogues match the GEMV kernel's.  For SwiGLU, a wave's 4 weight tiles
// are 2 gate tiles and the 2 matching up tiles.  For QKV with head_dim 128 a
// workgroup is one head, and a wave's tiles are dims {j, j + 64} pairs; with
// head_dim 64 a workgroup is two heads, one per wave column, and a wave's
// tiles are dims {j, j + 32} pairs.  Either way both halves of a rotated pair
// sit in the same lane.
//
// Tile order: the workgroups of one weight tile run on one XCD, because the
// hardware deals workgroup ids round-robin over the 8 XCDs; the weight tile
// is then read into one L2 and reused there by every row block.
#pragma once

#include "common.hpp"
#include "kernels.hpp"
#include "lmstat.hpp"

namespace sv {
namespace mfma {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int BM = 64;     // rows of X per workgroup (the smaller of the two tile heights)
constexpr int BN = 128;    // weight rows per workgroup
constexpr int KB = 64;     // K per LDS stage
constexpr int LDK = KB + 8;  // LDS row stride in bf16 (16-byte pad spreads the banks)
constexpr int NTH = 256;
constexpr int kXcds = 8;
// K blocks in flight through LDS (gemm_kernel2) for 128- and 64-row tiles;
// 0: the register-staged gemm_kernel
constexpr int kDmaStages = 2;
constexpr int kDmaStages64 = 3;
constexpr int kDmaKB = 64;    // K per LDS stage, 128-row tiles
constexpr int kDmaKB64 = 64;  // 64-row tiles
// 256 x 256 tiles (8 waves, one workgroup per CU); 0: not used
constexpr int kDmaStages256 = 2;
constexpr int kDmaKB256 = 64;

// Weight tiles of a launch whose workgroups hold BNT weight rows (128 or
// 256; QKV only 128).
template <int EPI, int BNT = BN>
__host__ __device__ inline int n_tiles(const GemvArgs& a) {
  if (EPI == EPI_SWIGLU) return (a.N + BNT / 2 - 1) / (BNT / 2);
  if (EPI == EPI_QKV) return a.hd == 128 ? a.H + 2 * a.Hkv : (a.H + 2 * a.Hkv + 1) / 2;
  return (a.N + BNT - 1) / BNT;
}

// Weight row held in local tile row lr (0 .. BNT-1) of weight tile nt.  Each
// 64 rows are one wave column's: for SwiGLU 32 gate rows, then the matching
// 32 up rows.
template <int EPI, int BNT>
__device__ __forceinline__ int w_row(const GemvArgs& a, int nt, int lr) {
  const int wn = lr >> 6, c = lr & 63;
  if constexpr (EPI == EPI_SWIGLU) {
    const int n = min(nt * (BNT / 2) + wn * 32 + (c & 31), a.N - 1);
    return c < 32 ? n : a.N + n;
  } else if constexpr (EPI == EPI_QKV) {
    static_assert(BNT == 128, "QKV tiles are 128 rows");
    if (a.hd == 64) return min((2 * nt + wn) * 64 + c, a.N - 1);  // head 2 nt + wn, dim c
    const int dim = (c < 32) ? wn * 32 + c : 64 + wn * 32 + (c - 32);
    return nt * a.hd + dim;
  } else {
    return min(nt * BNT + lr, a.N - 1);
  }
}

// The epilogue of a workgroup's BMT x BNT tile (acc: the wave's MI x 4
// 16 x 16 tiles; wave column wn holds tile columns wn*64 .. +63).  Lane holds
// rows 4 (lane / 16) + r of each 16-row tile, column lane % 16.
template <int EPI, int BMT, int BNT>
__device__ __forceinline__ void gemm_epilogue(const GemvArgs& a, f32x4_t (&acc)[BMT / 32][4], int mt, int nt,
                                              int slice, int wm, int wn, int lane) {
  constexpr int MI = BMT / 32;
  constexpr int WN = BNT / 64;  // wave columns
  const int M = a.M, m0 = mt * BMT;
  const int col = lane & 15, rb = (lane >> 4) * 4;
  if constexpr (EPI == EPI_LMSTAT) {
    // Row statistics of each 128-column tile in lmstat.hpp's order: wave
    // column wn holds half wn & 1 of statistics tile nt * BNT / 128 + wn / 2,
    // column 64 (wn & 1) + 16 j + col of it in slot j of lane col.  The two
    // halves meet in LDS.
    __shared__ float hmax[WN][BMT];
    __shared__ float hsum[WN][BMT];
    __shared__ int hidx[WN][BMT];
    const float T = a.temp;
    const int N = a.N, nts = (a.N + lmstat::kTile - 1) / lmstat::kTile;
    const int n0 = nt * BNT + wn * 64 + col;
    const int h0 = wn & ~1;  // the statistics tile's first half
    // the drafted token each of this lane's rows scores (-1: none), loaded
    // before the first store
    const int mps = a.m_per_seq;
    int xdr[MI][4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * (BMT / 2) + i * 16 + rb + r;
        const int rg = a.row0 + min(m, M - 1);
        const int b = rg / mps, ii = rg - b * mps;
        xdr[i][r] = (a.lx && m < M && ii < mps - 1) ? a.draft[b * (mps - 1) + ii] : -1;
      }
    auto vals = [&](int i, int r, float (&v)[4]) {
#pragma unroll
      for (int j = 0; j < 4; ++j)  // x / 1 rounds to x: no division at T = 1
        v[j] = (n0 + j * 16 < N) ? (T == 1.f ? acc[i][j][r] : __fdiv_rn(acc[i][j][r], T)) : -INFINITY;
    };
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lr = wm * (BMT / 2) + i * 16 + rb + r;
        if (T > 0.f) {
          float v[4];
          vals(i, r, v);
          const float mx = lmstat::group16_max(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
          if (col == 0) hmax[wn][lr] = mx;
        } else {
          float mx = -INFINITY;
          int ix = N;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (n0 + j * 16 < N) lmstat::argmax_merge(mx, ix, acc[i][j][r], n0 + j * 16);
          lmstat::group16_argmax(mx, ix);
          if (col == 0) {
            hmax[wn][lr] = mx;
            hidx[wn][lr] = ix;
          }
        }
      }
    __syncthreads();
    if (T > 0.f) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lr = wm * (BMT / 2) + i * 16 + rb + r;
          float v[4];
          vals(i, r, v);
          const float z = group_sum<16>(lmstat::slot_sum(v, fmaxf(hmax[h0][lr], hmax[h0 + 1][lr])));
          if (col == 0) hsum[wn][lr] = z;
        }
      __syncthreads();
    }
    const int stile = nt * (BNT / lmstat::kTile) + (wn >> 1);
    if ((wn & 1) == 0 && col == 0 && stile < nts) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lr = wm * (BMT / 2) + i * 16 + rb + r;
          const int m = m0 + lr;
          if (m >= M) continue;
          float2 st;
          if (T > 0.f) {
            st = make_float2(fmaxf(hmax[h0][lr], hmax[h0 + 1][lr]), hsum[h0][lr] + hsum[h0 + 1][lr]);
          } else {
            float mx = hmax[h0][lr];
            int ix = hidx[h0][lr];
            lmstat::argmax_merge(mx, ix, hmax[h0 + 1][lr], hidx[h0 + 1][lr]);
            st = make_float2(mx, __int_as_float(ix));
          }
          a.tpart[static_cast<size_t>(m) * nts + stile] = st;
        }
    }
    // the logit at the drafted token of each row that scores one
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * (BMT / 2) + i * 16 + rb + r;
        const int x = xdr[i][r];
        if (x < 0) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (n0 + j * 16 == x && x < N) a.lx[m] = acc[i][j][r];
      }
    return;
  }
  if constexpr (EPI == EPI_QKV) {
    // RoPE on query and key rows, then the stores: q rows (float32), and K/V
    // rows into the cache at len[b] + i.  Every (cos, sin) pair and cache
    // position this lane needs is loaded before the first store, so their
    // latencies overlap instead of queueing behind the stores.
    static_assert(BNT == 128, "QKV tiles are 128 rows");
    const int H = a.H, Hkv = a.Hkv, hd = a.hd, half = hd / 2;
    const bool two = hd == 64;  // two heads per workgroup
    const int hh = two ? 2 * nt + wn : nt;
    if (hh >= H + 2 * Hkv) return;  // an odd head count's empty half
    const bool rope = hh < H + Hkv;
    float2 cs[MI][4][2];
    int pos[MI][4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rg = a.row0 + min(m0 + wm * (BMT / 2) + i * 16 + rb + r, M - 1);
        const int b = rg / a.m_per_seq, ii = rg - b * a.m_per_seq;
        pos[i][r] = hh >= H ? a.len[b] + ii : 0;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int d = two ? j * 16 + col : wn * 32 + j * 16 + col;  // 0 .. half-1; its pair is d + half
          cs[i][r][j] = rope ? a.cs[static_cast<size_t>(rg) * half + d] : make_float2(0.f, 0.f);
        }
      }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * (BMT / 2) + i * 16 + rb + r;
        if (m >= M) continue;
        const int rg = a.row0 + m;
        const int b = rg / a.m_per_seq;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int d = two ? j * 16 + col : wn * 32 + j * 16 + col;
          const float x0 = acc[i][j][r], y0 = acc[i][j + 2][r];
          if (rope) {
            const float2 c = cs[i][r][j];
            const float r0 = x0 * c.x - y0 * c.y, s0 = y0 * c.x + x0 * c.y;
            if (hh < H) {
              float* qr = a.q + static_cast<size_t>(rg) * (H * hd) + hh * hd;
              qr[d] = r0;
              qr[d + half] = s0;
            } else if (pos[i][r] >= 0 && pos[i][r] < a.max_ctx) {
              uint16_t* dst = static_cast<uint16_t*>(a.kc) +
                              (((static_cast<size_t>(a.layer) * a.kvB + b) * Hkv + (hh - H)) * a.max_ctx + pos[i][r]) * hd;
              dst[d] = f2bf(r0);
              dst[d + half] = f2bf(s0);
            }
          } else if (pos[i][r] >= 0 && pos[i][r] < a.max_ctx) {
            uint16_t* dst = static_cast<uint16_t*>(a.vc) +
                            (((static_cast<size_t>(a.layer) * a.kvB + b) * Hkv + (hh - H - Hkv)) * a.max_ctx + pos[i][r]) * hd;
            dst[d] = f2bf(x0);
            dst[d + half] = f2bf(y0);
          }
        }
      }
    return;
  }
  float* y = a.y ? a.y + static_cast<size_t>(slice) * a.ysplit : nullptr;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    // residual add: the 16-row tile's values added to, loaded before its
    // first store
    float yv[4][4];
    if constexpr (EPI == EPI_RESID) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int m = min(m0 + wm * (BMT / 2) + i * 16 + rb + r, M - 1);
          const int n = min(nt * BNT + wn * 64 + j * 16 + col, a.N - 1);
          yv[r][j] = y[static_cast<size_t>(m) * a.ldy + n];
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * (BMT / 2) + i * 16 + rb + r;
      if (m >= M) continue;
      if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = nt * (BNT / 2) + wn * 32 + j * 16 + col;
          if (n < a.N) {
            const float g = acc[i][j][r], u = acc[i][j + 2][r];
            static_cast<uint16_t*>(a.z)[static_cast<size_t>(m) * a.ldz + n] = f2bf(g / (1.f + expf(-g)) * u);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = nt * BNT + wn * 64 + j * 16 + col;
          if (n < a.N) {
            float* dst = y + static_cast<size_t>(m) * a.ldy + n;
            if constexpr (EPI == EPI_RESID) *dst = yv[r][j] + acc[i][j][r];
            else *dst = acc[i][j][r];
          }
        }
      }
    }
  }
}

template <int EPI, int BMT>
__global__ __launch_bounds__(NTH) void gemm_kernel(GemvArgs a, int mtiles, int ntiles) {
  constexpr int MI = BMT / 32;   // 16-row tiles per wave (a wave covers BMT / 2 rows)
  constexpr int XL = BMT / 32;   // 16-byte X chunks per thread per K block
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BMT][LDK];
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][BN][LDK];
  const int per = gridDim.x / kXcds;
  const int tile = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (tile >= mtiles * ntiles) return;  // padding workgroups leave before any barrier
  const int mt = tile % mtiles, nt = tile / mtiles;
  const int M = a.M, K = a.K, slice = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int wm = wave & 1, wn = wave >> 1;
  const int m0 = mt * BMT;

  // this thread's global chunks: X XL x 16 B, W 4 x 16 B per K block
  const uint16_t* xp[XL];
  const uint16_t* wp[4];
  int xr[XL], xc[XL], wr[4], wc[4];
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int c = threadIdx.x + i * NTH;
    xr[i] = c >> 3;
    xc[i] = (c & 7) * 8;
    xp[i] = static_cast<const uint16_t*>(a.x) + static_cast<size_t>(min(m0 + xr[i], M - 1)) * a.ldx +
            static_cast<size_t>(slice) * K + xc[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = threadIdx.x + i * NTH;
    wr[i] = c >> 3;
    wc[i] = (c & 7) * 8;
    wp[i] = static_cast<const uint16_t*>(a.W) + static_cast<size_t>(w_row<EPI, BN>(a, nt, wr[i])) * a.ldw +
            static_cast<size_t>(slice) * K + wc[i];
  }
  v4u gx[XL], gw[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < XL; ++i) gx[i] = *reinterpret_cast<const v4u*>(xp[i] + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) gw[i] = *reinterpret_cast<const v4u*>(wp[i] + k0);
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XL; ++i) *reinterpret_cast<v4u*>(&xs[buf][xr[i]][xc[i]]) = gx[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<v4u*>(&ws[buf][wr[i]][wc[i]]) = gw[i];
  };

  f32x4_t acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = K / KB;
  load(0);
  store(0);
  __syncthreads();
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  for (int kb = 0; kb < nk; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nk) load((kb + 1) * KB);
#pragma unroll
    for (int ks = 0; ks < KB; ks += 32) {
      bf16x8_t af[MI], bfr[4];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&xs[buf][wm * (BMT / 2) + i * 16 + fr][ks + fk]);
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[j] = *reinterpret_cast<const bf16x8_t*>(&ws[buf][wn * 64 + j * 16 + fr][ks + fk]);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kb + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }

  gemm_epilogue<EPI, BMT, BN>(a, acc, mt, nt, slice, wm, wn, lane);
}

// ---- the same tile with its K blocks moved global -> LDS directly -------------
// global_load_lds_dwordx4 writes lane l's 16 bytes at the instruction's LDS
// base + 16 l, so one instruction fills 64 / CPR tile rows of CPR chunks (one
// K block of KBD bf16, CPR = KBD / 8) and no registers stage the loads: NS
// blocks can be in flight, issued NS - 1 blocks ahead of the one being
// multiplied.  Chunk c of tile row r sits in slot c ^ ((r >> SH) & (CPR - 1))
// of its row (a lane picks the global chunk that belongs in its slot), so
// the 16 rows of a fragment read fall in distinct LDS banks.
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  constexpr int SH = CPR == 8 ? 1 : 2;
  return r * CPR + (c ^ ((r >> SH) & (CPR - 1)));
}

// s_waitcnt vmcnt(n), expcnt and lgkmcnt not waited for (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

template <int EPI, int BMT, int BNT, int NS, int KBD>
__global__ __launch_bounds__(2 * BNT) void gemm_kernel2(GemvArgs a, int mtiles, int ntiles) {
  static_assert(KBD == 32 || KBD == 64, "K block");
  static_assert(BNT == 128 || BNT == 256, "weight tile");
  constexpr int MI = BMT / 32;
  constexpr int NW = BNT / 32;  // waves: 2 rows x BNT / 64 columns of (BMT / 2) x 64 wave tiles
  constexpr int CPR = KBD / 8, RPI = kWave / CPR;  // chunks per row, rows per DMA instruction
  constexpr int XI = BMT / (NW * RPI), WI = BNT / (NW * RPI);  // DMA instructions per wave and block
  static_assert(XI * NW * RPI == BMT && WI * NW * RPI == BNT, "DMA rows");
  constexpr int L = XI + WI;
  constexpr int STAGE = (BMT + BNT) * KBD;  // bf16 per stage
  static_assert(NS >= 2 && NS <= 4 && (NS - 2) * L < 64, "stages");
  __shared__ __attribute__((aligned(16))) uint16_t lds[NS * STAGE];
  const int per = gridDim.x / kXcds;
  const int tile = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (tile >= mtiles * ntiles) return;  // padding workgroups leave before any barrier
  const int mt = tile % mtiles, nt = tile / mtiles;
  const int M = a.M, K = a.K, slice = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int wm = wave & 1, wn = wave >> 1;
  const int m0 = mt * BMT;

  // this lane's global chunk for each of its DMA instructions
  const uint16_t* xp[XI];
  const uint16_t* wp[WI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int r = (wave * XI + i) * RPI + lane / CPR;
    const int c = swz<CPR>(r, lane % CPR) - r * CPR;  // the slot's chunk (the swizzle is its own inverse)
    xp[i] = static_cast<const uint16_t*>(a.x) + static_cast<size_t>(min(m0 + r, M - 1)) * a.ldx +
            static_cast<size_t>(slice) * K + c * 8;
  }
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int r = (wave * WI + i) * RPI + lane / CPR;
    const int c = swz<CPR>(r, lane % CPR) - r * CPR;
    wp[i] = static_cast<const uint16_t*>(a.W) + static_cast<size_t>(w_row<EPI, BNT>(a, nt, r)) * a.ldw +
            static_cast<size_t>(slice) * K + c * 8;
  }
  auto issue = [&](int st, int k0) {
    uint16_t* base = lds + st * STAGE;
#pragma unroll
    for (int i = 0; i < XI; ++i)
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(xp[i] + k0), (lds_ptr_t)(base + (wave * XI + i) * RPI * KBD), 16, 0,
                                       0);
#pragma unroll
    for (int i = 0; i < WI; ++i)
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(wp[i] + k0),
                                       (lds_ptr_t)(base + BMT * KBD + (wave * WI + i) * RPI * KBD), 16, 0, 0);
  };

  f32x4_t acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = K / KBD;
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nk) issue(st, st * KBD);
  const int fr = lane & 15, fc = lane >> 4;
  for (int kb = 0; kb < nk; ++kb) {
    // this wave's block kb is in LDS once at most `later` later blocks are in flight
    const int later = min(NS - 2, nk - 1 - kb);
    if (later >= NS - 2) wait_vm<(NS - 2) * L>();
    else if (later == 1) wait_vm<L>();
    else wait_vm<0>();
    // every wave's block kb is in; every wave is done with block kb - 1 (its
    // LDS reads were consumed by its MFMAs).  A bare s_barrier: the fence of
    // __syncthreads would wait for every block in flight.
    __builtin_amdgcn_s_barrier();
    if (kb + NS - 1 < nk) issue((kb + NS - 1) % NS, (kb + NS - 1) * KBD);
    const uint16_t* xs = lds + (kb % NS) * STAGE;
    const uint16_t* ws = xs + BMT * KBD;
#pragma unroll
    for (int ks = 0; ks < CPR; ks += 4) {  // 32 K per MFMA: chunks ks .. ks + 3
      bf16x8_t af[MI], bfr[4];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r = wm * (BMT / 2) + i * 16 + fr;
        af[i] = *reinterpret_cast<const bf16x8_t*>(xs + swz<CPR>(r, ks + fc) * 8);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wn * 64 + j * 16 + fr;
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(ws + swz<CPR>(r, ks + fc) * 8);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
  gemm_epilogue<EPI, BMT, BNT>(a, acc, mt, nt, slice, wm, wn, lane);
}

}  // namespace mfma
}  // namespace sv
