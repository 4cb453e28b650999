// Device helpers shared by the fused SGMM kernels (decode and prefill).
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace rp {

// Layout of the workspace's reserved counter region (int32 words; words that
// atomics hit from many workgroups sit on cache lines of their own).
//   kCtlEpoch      decode launches completed on this workspace.  Launch n uses
//                  control set n & 1; the last workgroup to arrive clears the
//                  other set for launch n + 1 and then advances the epoch, so
//                  no launch ends with a serialised "who finished last" count.
//   kCtlWaitOverflow  sticky flag: a wait gave up after its spin limit.
//   kCtlSegErr     out-of-range router indices seen by a fused launch's
//                  segmentation (always 0 for indices the router wrote).
// In a control set, per group g of the launch (g < kMaxGroups):
//   kSetShrinkDone + 32 g          pair-chunk shrink units finished
//   kSetGroupDone + 256 g + 32 c   output tiles finished, counted per tile % 8
//   kSetQueue                      items claimed after every workgroup's first (item = grid + count)
constexpr int kCtlEpoch = 0;
constexpr int kCtlWaitOverflow = 32;
constexpr int kCtlSegErr = 64;
constexpr int kCtlSet0 = 1024;
constexpr int kCtlSetStride = 4096;
constexpr int kSetShrinkDone = 0;
constexpr int kSetRouteDone = 32 * kMaxGroups;  // router tiles finished
constexpr int kSetSegDone = kSetRouteDone + 32;  // segmentation finished
constexpr int kSetArrive = kSetSegDone + 32;     // + 32 * (blockIdx % 8): workgroups that read the epoch
constexpr int kSetArriveAll = kSetArrive + 8 * 32;
constexpr int kSetGroupDone = kSetArriveAll + 64;
constexpr int kSetQueue = kSetGroupDone + 256 * kMaxGroups;  // items handed out after each workgroup's first
constexpr int kSetWords = kSetQueue + 32;
static_assert(kCtlSet0 + 2 * kCtlSetStride <= kPrefillCounterWord, "control sets overlap the prefill counters");
static_assert(kCtlSegErr < kRouteCounterWord && kRouteCounterWord + kRouteCounterWords <= kCtlSet0,
              "router counters overlap the control words");
static_assert(kSetWords <= kCtlSetStride, "control set overflow");
static_assert(kActPairWords * kMaxGroups <= kPrefillCounterWords, "activation pair counters overflow");

// Device-scope (sc1) loads of routing data another workgroup of the same
// launch may have written; plain loads when it was written by an earlier launch.
template <bool COH>
__device__ __forceinline__ int ld_route(const int* p) {
  if (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}
template <bool COH>
__device__ __forceinline__ float ld_route(const float* p) {
  if (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}

// Projection that owns output-row tile `tile` of the packed row space.
__device__ __forceinline__ int proj_of_tile(const SgmmArgs& a, int tile) {
  int p = 0;
  if (a.n_proj > 1 && tile >= a.proj[1].tile_begin) p = 1;
  if (a.n_proj > 2 && tile >= a.proj[2].tile_begin) p = 2;
  if (a.n_proj > 3 && tile >= a.proj[3].tile_begin) p = 3;
  return p;
}

// Field-wise select of projection p's descriptor (keeps the kernel argument
// block out of private memory).
template <typename F>
__device__ __forceinline__ F pick4(int p, F f0, F f1, F f2, F f3) {
  return p == 0 ? f0 : p == 1 ? f1 : p == 2 ? f2 : f3;
}
#define RP_PICK(a, p, field) pick4(p, a.proj[0].field, a.proj[1].field, a.proj[2].field, a.proj[3].field)

__device__ __forceinline__ ProjDesc proj_at(const SgmmArgs& a, int p) {
  ProjDesc d;
  d.W0 = RP_PICK(a, p, W0);
  d.A = RP_PICK(a, p, A);
  d.B = RP_PICK(a, p, B);
  d.y = RP_PICK(a, p, y);
  d.d_out = RP_PICK(a, p, d_out);
  d.ld_y = RP_PICK(a, p, ld_y);
  d.tile_begin = RP_PICK(a, p, tile_begin);
  d.tiled = RP_PICK(a, p, tiled);
  d.residual = RP_PICK(a, p, residual);
  return d;
}

__device__ __forceinline__ uint4 sel4(bool ok, uint4 v) { return ok ? v : zero4(); }

// True when some slot of token t chose adapter e.
__device__ __forceinline__ bool chose(const int* idx, int t, int k, int e) {
  bool any = false;
  for (int j = 0; j < k; ++j) any |= idx[t * k + j] == e;
  return any;
}

// Gated u rows [c, c+8) summed over every slot of token t that chose adapter e
// (a token may name one adapter in several slots), as hi/lo bf16 operands;
// zero when !ok or no slot matches.
__device__ __forceinline__ void u_operand(const float* u, const int* idx, int r, int t, int k, int e, int c, bool ok,
                                          uint4& hi, uint4& lo) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.f;
  if (ok) {
    for (int j = 0; j < k; ++j) {
      if (idx[t * k + j] != e) continue;
      const float* p = u + (size_t)(t * k + j) * r + c;
      const float4 a = *reinterpret_cast<const float4*>(p);
      const float4 b = *reinterpret_cast<const float4*>(p + 4);
      v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w; v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
    }
  }
  split_hi_lo(v, hi, lo);
}

// Shrink chunks are numbered segment by segment, ceil(n_e / nch) per segment.
// Run by one full wave; returns (segment, chunk) or segment -1 past the end.
template <bool COH = false>
__device__ __forceinline__ void locate_chunk(const SgmmArgs& a, int unit, int nch, int lane, int* seg,
                                             int* chunk) {
  int carry = 0, fe = -1, fc = 0;
  for (int e0 = 0; e0 < a.E; e0 += 64) {
    const int e = e0 + lane;
    const int n = (e < a.E) ? (ld_route<COH>(&a.seg_offsets[e + 1]) - ld_route<COH>(&a.seg_offsets[e])) : 0;
    const int c = (n + nch - 1) / nch;
    const int incl = wave_inclusive_scan(c, lane);
    const int excl = carry + incl - c;
    const uint64_t m = __ballot(c > 0 && unit >= excl && unit < excl + c);
    if (m) {
      const int src = __ffsll((unsigned long long)m) - 1;
      fe = e0 + src;
      fc = unit - __shfl(excl, src, 64);
      break;
    }
    carry += __shfl(incl, 63, 64);
  }
  *seg = fe;
  *chunk = fc;
}

// One shrink unit: u[p, :] = g_p * A_e x_t for the pairs p of chunk `chunk`
// (16*NCT pairs) of segment e, with bf16 MFMA 16x16x32 (A_e rows as M, pairs
// as N).  WAVES waves split d_in; their partial sums are added in wave order in
// LDS (`red`: MTR*NCT*4*64 floats), so the result does not depend on timing.
// Must be called by all WAVES*64 threads of the workgroup.
template <int MTR, int NCT, int WAVES, int U>
__device__ __forceinline__ void shrink_unit(const SgmmArgs& a, int proj, int e, int chunk, float* red) {
  constexpr int NCH = 16 * NCT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const ProjDesc pd = proj_at(a, proj);
  const int slot0 = a.seg_offsets[e] + chunk * NCH;
  const int slot_end = min(a.seg_offsets[e + 1], slot0 + NCH);
  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  const bf16_t* Ae = static_cast<const bf16_t*>(pd.A) + (size_t)e * a.r * a.d_in;
  const int lr = lane & 15, kg = lane >> 4;

  const bf16_t* xp[NCT];
#pragma unroll
  for (int nt = 0; nt < NCT; ++nt) {
    const int slot = min(slot0 + nt * 16 + lr, slot_end - 1);
    xp[nt] = x + (size_t)(a.pair_perm[slot] / a.k) * a.ld_x;
  }
  const bf16_t* ap[MTR];
  bool aok[MTR];
#pragma unroll
  for (int mt = 0; mt < MTR; ++mt) {
    const int c = mt * 16 + lr;
    aok[mt] = c < a.r;
    ap[mt] = Ae + (size_t)min(c, a.r - 1) * a.d_in;
  }

  const int nsteps = (a.d_in + 31) >> 5;
  const int sb = nsteps * wave / WAVES, se = nsteps * (wave + 1) / WAVES;
  f32x4_t acc[MTR][NCT];
#pragma unroll
  for (int mt = 0; mt < MTR; ++mt)
#pragma unroll
    for (int nt = 0; nt < NCT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // batches of U K steps, two in flight: the loads of the next batch go out
  // before the MFMAs of the current one (batches and steps still summed in
  // ascending K)
  uint4 av[2][U][MTR], bv[2][U][NCT];
  auto load = [&](int buf, int s) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s + u) * 32 + kg * 8;
      const bool ok = (s + u < se) && (k < a.d_in);
      const int kc = min(k, a.d_in - 8);
#pragma unroll
      for (int mt = 0; mt < MTR; ++mt) av[buf][u][mt] = sel4(ok && aok[mt], ld16(ap[mt] + kc));
#pragma unroll
      for (int nt = 0; nt < NCT; ++nt) bv[buf][u][nt] = sel4(ok, ld16(xp[nt] + kc));
    }
  };
  auto math = [&](int buf) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MTR; ++mt)
#pragma unroll
        for (int nt = 0; nt < NCT; ++nt) acc[mt][nt] = mfma16(av[buf][u][mt], bv[buf][u][nt], acc[mt][nt]);
  };
  int s = sb;
  if (s < se) load(0, s);
  while (s < se) {
    if (s + U < se) load(1, s + U);
    math(0);
    s += U;
    if (s >= se) break;
    if (s + U < se) load(0, s + U);
    math(1);
    s += U;
  }

  // fixed-order sum over waves (wave 0 first), accumulated in LDS
  for (int w = 0; w < WAVES; ++w) {
    if (wave == w) {
#pragma unroll
      for (int mt = 0; mt < MTR; ++mt)
#pragma unroll
        for (int nt = 0; nt < NCT; ++nt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float* dst = red + ((mt * NCT + nt) * 4 + v) * 64 + lane;
            *dst = (w == 0) ? acc[mt][nt][v] : *dst + acc[mt][nt][v];
          }
    }
    __syncthreads();
  }

  // D layout: lane -> pair lane%16, rank row 4*(lane/16)+v
  float* u_out = a.u + (size_t)proj * a.T * a.k * a.r;
  for (int q = tid; q < MTR * NCT * 4 * 64; q += WAVES * 64) {
    const int l = q & 63, f = q >> 6;
    const int v = f & 3, nt = (f >> 2) % NCT, mt = (f >> 2) / NCT;
    const int slot = slot0 + nt * 16 + (l & 15);
    const int c = mt * 16 + 4 * (l >> 4) + v;
    if (slot < slot_end && c < a.r) {
      const int p = a.pair_perm[slot];
      u_out[(size_t)p * a.r + c] = a.topk_gate[p] * red[q];
    }
  }
}

}  // namespace rp
