// Attention of one (sequence, query head, row) unit by a whole workgroup,
// for a kernel that computes attention right after writing q and the new
// K/V rows itself (the persistent pass).
//
// Decode-time attention is bound by reading the cache (first page, section
// "The speedup is borrowed"; "How Speculative Decoding Works", section
// "Prefill and Decode"): the unit's keys 0 .. len + i are split over the
// workgroup's waves, KT per wave per trip; a lane holds a 16-byte chunk of a
// K or V row, the row's lanes add their partial dot products with DPP moves,
// and the waves' (max, sum, output) partials merge in LDS in wave order.
// q and the rows written by the calling launch (positions >= len) are read
// with agent-scope (sc1) loads: another workgroup, on another XCD, wrote
// them with agent-scope stores in the same launch.  Earlier rows use
// ordinary loads.  The output row is stored with agent-scope stores.
#pragma once

#include <math.h>

#include "common.hpp"

namespace sv {
namespace unit {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
constexpr int kSc1 = 16;  // buffer-access cache policy: agent-scope coherent

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}
__device__ __forceinline__ v4u load_sc1(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kSc1);
}
__device__ __forceinline__ void store_sc1(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_sc1(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The unit's inputs.  q [B m][H HD] float32, K/V caches [L][kvB][Hkv][max_ctx][HD]
// bf16, xo [B m][H HD] bf16 output.
struct AttnUnitArgs {
  const float* q;
  const void* kc;
  const void* vc;
  const int32_t* len;
  void* xo;
  int B, m, H, Hkv, kvB, max_ctx, layer;
};

// Bytes of LDS the unit needs with NWV waves.
template <int HD, int NWV>
__host__ __device__ constexpr int attn_unit_lds() {
  return static_cast<int>(sizeof(float)) * NWV * HD + static_cast<int>(sizeof(float2)) * NWV;
}

template <int HD> struct AttnShape {
  static constexpr int CPR = HD / 8;       // 16-byte chunks per K/V row
  static constexpr int RPI = kWave / CPR;  // rows per load instruction
};

// All threads of the workgroup (NWV waves) call it with the same u.
template <int HD, int NWV, int KT>
__device__ __forceinline__ void attn_unit(const AttnUnitArgs& a, int u, char* lds) {
  using S = AttnShape<HD>;
  constexpr int CPR = S::CPR, RPI = S::RPI, NI = KT / RPI;
  static_assert(NI >= 1 && KT % RPI == 0, "keys per wave tile");
  float (*mo)[HD] = reinterpret_cast<float (*)[HD]>(lds);
  float2* ml = reinterpret_cast<float2*>(lds + sizeof(float) * NWV * HD);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int H = a.H, m = a.m;
  const int b = u / (H * m), rem = u - b * H * m, h = rem / m, i = rem - h * m;
  const int kvh = h / (H / a.Hkv);
  const int Lb = a.len[b];
  const int pos = Lb + i;
  const int kend = max(0, min(pos + 1, a.max_ctx));
  const int klast = max(kend - 1, 0);
  const int trips = (kend + NWV * KT - 1) / (NWV * KT);
  const size_t kvbase = ((static_cast<size_t>(a.layer) * a.kvB + b) * a.Hkv + kvh) * a.max_ctx;
  const uint16_t* kc = static_cast<const uint16_t*>(a.kc) + kvbase * HD;
  const uint16_t* vc = static_cast<const uint16_t*>(a.vc) + kvbase * HD;
  const uint32_t kvbytes = static_cast<uint32_t>(a.max_ctx) * HD * 2;
  const __amdgpu_buffer_rsrc_t rk = rsrc(kc, kvbytes), rv = rsrc(vc, kvbytes);
  const int rho = lane / CPR, chi = lane % CPR;
  const int row = b * m + i;
  const float scale = 1.0f / sqrtf(static_cast<float>(HD));
  float qr[8];
  {
    const __amdgpu_buffer_rsrc_t rq = rsrc(a.q, static_cast<uint32_t>(a.B) * m * H * HD * 4);
    const uint32_t off = static_cast<uint32_t>(row * H * HD + h * HD + chi * 8) * 4;
    const v4u q0 = load_sc1(rq, off), q1 = load_sc1(rq, off + 16);
    qr[0] = __uint_as_float(q0.x) * scale;
    qr[1] = __uint_as_float(q0.y) * scale;
    qr[2] = __uint_as_float(q0.z) * scale;
    qr[3] = __uint_as_float(q0.w) * scale;
    qr[4] = __uint_as_float(q1.x) * scale;
    qr[5] = __uint_as_float(q1.y) * scale;
    qr[6] = __uint_as_float(q1.z) * scale;
    qr[7] = __uint_as_float(q1.w) * scale;
  }
  float mrow = -INFINITY, lrow = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;

  for (int it = 0; it < trips; ++it) {
    const int k0 = (it * NWV + wave) * KT;
    v4u kr[NI], vr[NI];
#pragma unroll
    for (int c = 0; c < NI; ++c) {
      const int key = min(k0 + c * RPI + rho, klast);
      const uint32_t off = static_cast<uint32_t>(key * HD + chi * 8) * 2;
      if (key >= Lb) {  // written by this pass: agent-scope loads
        kr[c] = load_sc1(rk, off);
        vr[c] = load_sc1(rv, off);
      } else {
        kr[c] = *reinterpret_cast<const v4u*>(reinterpret_cast<const char*>(kc) + off);
        vr[c] = *reinterpret_cast<const v4u*>(reinterpret_cast<const char*>(vc) + off);
      }
    }
    float sc[NI];
    float mt = -INFINITY;
#pragma unroll
    for (int c = 0; c < NI; ++c) {
      float t0 = 0.f, t1 = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        t0 = fmaf(qr[2 * e], __uint_as_float(kr[c][e] << 16), t0);
        t1 = fmaf(qr[2 * e + 1], __uint_as_float(kr[c][e] & 0xffff0000u), t1);
      }
      float s = group_sum<CPR>(t0 + t1);
      const int key = k0 + c * RPI + rho;
      if (!(key < kend)) s = -INFINITY;
      sc[c] = s;
      mt = fmaxf(mt, s);
    }
    const float mnew = fmaxf(mrow, groups_max<CPR>(mt));
    const bool live = mnew != -INFINITY;
    const float alpha = live ? expf(mrow - mnew) : 1.f;
    float ls = 0.f;
#pragma unroll
    for (int c = 0; c < NI; ++c) {
      sc[c] = (live && sc[c] != -INFINITY) ? expf(sc[c] - mnew) : 0.f;
      ls += sc[c];
    }
    lrow = lrow * alpha + groups_sum<CPR>(ls);
    mrow = mnew;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
    for (int c = 0; c < NI; ++c) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] = fmaf(sc[c], __uint_as_float(vr[c][e] << 16), o[2 * e]);
        o[2 * e + 1] = fmaf(sc[c], __uint_as_float(vr[c][e] & 0xffff0000u), o[2 * e + 1]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = groups_sum<CPR>(o[e]);
  if (rho == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) mo[wave][chi * 8 + e] = o[e];
  }
  if (lane == 0) ml[wave] = make_float2(mrow, lrow);
  __syncthreads();
  uint16_t* xo = static_cast<uint16_t*>(a.xo);
  if (static_cast<int>(threadIdx.x) < HD) {
    const int dd = threadIdx.x;
    float Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) Mx = fmaxf(Mx, ml[w].x);
    float l = 0.f, accv = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const float2 v = ml[w];
      const float wt = (v.x == -INFINITY) ? 0.f : expf(v.x - Mx);
      l = fmaf(v.y, wt, l);
      accv = fmaf(mo[w][dd], wt, accv);
    }
    store_sc1(xo + static_cast<size_t>(row) * H * HD + h * HD + dd, f2bf(l > 0.f ? accv / l : 0.f));
  }
  __syncthreads();  // the scratch is reused by the next unit
}

}  // namespace unit
}  // namespace sv
