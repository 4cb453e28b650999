// Device functions for token-level pre-gating and segmentation (AdaFuse,
// technical summary §2.A; §2.B decoding steps 1-2), shared by the standalone
// rp_pregate / rp_segment kernels and by the fused launch that routes and then
// projects (so both paths give bit-identical results).
//
// Outputs are written with device-scope (sc1) stores and routing inputs read
// with device-scope loads, so other workgroups of the same launch may consume
// them once a counter says they are complete.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace rp {

__device__ __forceinline__ int ldc_i32(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ldc_f32(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc_i32(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc_f32(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// router
// ---------------------------------------------------------------------------
constexpr int kRouteThreads = 128;     // threads per router tile for E <= 64 (both launch forms)
constexpr int kRouteThreadsWide = 1024;  // threads per router tile for E > 64 (router launch only)
constexpr int kRouteCB = 8;         // router columns per thread

template <typename Tin>
struct Vec8;
template <>
struct Vec8<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float (&v)[8]) {
    const uint4 q = ld16(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ float one(const bf16_t* p) { return bf16_to_f32(*p); }
};
template <>
struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ float one(const float* p) { return *p; }
};

// Eight consecutive elements as raw loaded data (unpacked to fp32 later).
template <typename Tin>
struct Raw8;
template <>
struct Raw8<bf16_t> {
  typedef uint4 type;
  static __device__ __forceinline__ type fetch(const bf16_t* p) { return ld16(p); }
  static __device__ __forceinline__ void unpack(const type& q, float (&v)[8]) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
struct F32x8 {
  float4 a, b;
};
template <>
struct Raw8<float> {
  typedef F32x8 type;
  static __device__ __forceinline__ type fetch(const float* p) {
    return F32x8{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
  }
  static __device__ __forceinline__ void unpack(const type& q, float (&v)[8]) {
    v[0] = q.a.x; v[1] = q.a.y; v[2] = q.a.z; v[3] = q.a.w; v[4] = q.b.x; v[5] = q.b.y; v[6] = q.b.z; v[7] = q.b.w;
  }
};
constexpr int kRouteNB = 2;  // groups of 8 k per router load batch

// (value, index) order of the router: larger logit first, lower index on ties.
__device__ __forceinline__ bool route_better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

struct RoutePlan {
  int NCBp;   // column blocks rounded up to a power of two
  int slice;  // k per k-slice
  bool vec_cols;
  int TT;     // tokens per tile
  int NT;     // threads per tile
  int KR;     // partial sums per column left after the in-wave butterfly
};

// Top-k of tokens [t0, t0 + nt) from their logits lg[t][E] (LDS, t relative
// to t0) and the softmax gates over the chosen logits: one wave per token,
// waves w, w + n_waves, ... of the caller's thread group.  Larger logit first,
// lower index on ties.  Results go out with device-scope stores (and as tagged
// pairs when `tagged` is set).
__device__ __forceinline__ void route_select(const PregateArgs& a, const float* lg, int t0, int nt, int wave,
                                             int n_waves, unsigned long long* tagged, uint32_t tag) {
  const int lane = threadIdx.x & 63;
  const int E = a.E;
  for (int tt = wave; tt < nt; tt += n_waves) {
    const float* row = lg + tt * E;
    uint32_t taken = 0;  // bit m: this lane's m-th candidate (e = lane + 64 m) is chosen
    float selv[kMaxK];
    int seli[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j >= a.k) break;
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int m = 0, e = lane; e < E; ++m, e += 64) {
        if (!((taken >> m) & 1u)) {
          const float v = row[e];
          if (bi == 0x7fffffff || route_better(v, e, bv, bi)) { bv = v; bi = e; }
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (oi != 0x7fffffff && (bi == 0x7fffffff || route_better(ov, oi, bv, bi))) { bv = ov; bi = oi; }
      }
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
      selv[j] = bv;
      seli[j] = bi;
    }
    if (lane < a.k) {
      // softmax over the chosen logits, shifted by the largest
      float s = 0.f, mine = 0.f;
      int mine_i = 0;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (j >= a.k) break;
        const float z = expf(selv[j] - selv[0]);
        s += z;
        if (j == lane) { mine = z; mine_i = seli[j]; }
      }
      const size_t base = (size_t)(t0 + tt) * a.k;
      const float g = mine / s;
      stc_i32(&a.topk_idx[base + lane], mine_i);
      stc_f32(&a.topk_gate[base + lane], g);
      if (tagged) {
        const unsigned long long hi = (unsigned long long)tag << 32;
        __hip_atomic_store(&tagged[(base + lane) * 2], hi | (uint32_t)mine_i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&tagged[(base + lane) * 2 + 1], hi | __float_as_uint(g), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// The k-slices (and with them the summation order of a logit) depend on E and
// d_in only, never on T or on which launch runs the router: with E <= 64 a
// tile has 128 threads (the decode launch runs two tiles per workgroup), with
// more adapters 1024 (at most two tokens a tile), so a thread's k-slice stays
// short.
__host__ __device__ inline RoutePlan route_plan(int E, int d_in, int elem_bytes) {
  RoutePlan p;
  const int ncb = (E + kRouteCB - 1) / kRouteCB;
  p.NCBp = 1;
  while (p.NCBp < ncb) p.NCBp <<= 1;
  p.NT = E <= 64 ? kRouteThreads : kRouteThreadsWide;
  const int KS = p.NT / p.NCBp > 0 ? p.NT / p.NCBp : 1;
  p.slice = ((d_in + KS - 1) / KS + 7) / 8 * 8;
  p.vec_cols = (E * elem_bytes) % 16 == 0;
  const int L = p.NCBp >= 64 ? 1 : 64 / p.NCBp;
  p.KR = KS / L > 1 ? KS / L : 1;
  p.TT = E <= 64 || (p.NT <= 512 && (p.KR + 1) * 4 * E * 4 <= 65536) ? 4 : 2;
  return p;
}

// LDS floats a router tile needs: KR partial sums and the logits per (token, column).
__host__ __device__ inline int route_lds_floats(const RoutePlan& p, int E, int TT) { return (p.KR + 1) * TT * E; }

// Score tokens [t0, t0 + TT) against all E router columns, choose the top k
// and their softmax gates.  Threads are (block of 8 columns, k-slice); a thread
// walks its k-slice in ascending k with one fp32 sum per (token, column); the
// slices are combined with a fixed butterfly inside each wave and then in wave
// order, so equal router columns give bit-equal logits.
// NCBp <= 128 (E <= 1024).  Must be called by all NT threads of a
// group (every group of a wider workgroup calls it, with its own smem and t0).
// With `tagged` set, each (token, slot) result is also written as two tagged
// 8-byte pairs (index, tag) and (gate bits, tag) for readers in the same launch.
template <typename Tin, int TT, int NT = kRouteThreads>
__device__ __forceinline__ void route_tile(const PregateArgs& a, int t0, const RoutePlan& rp_, float* smem,
                                           unsigned long long* tagged = nullptr, uint32_t tag = 0) {
  const int NCBp = rp_.NCBp;
  // a wider workgroup runs one tile per group of NT threads
  const int tid = threadIdx.x & (NT - 1), lane = tid & 63, wave = tid >> 6;
  const int nt = min(TT, a.T - t0);
  const int E = a.E;
  const Tin* x = static_cast<const Tin*>(a.x);
  const Tin* Wg = static_cast<const Tin*>(a.Wg);
  const int ncb = (E + kRouteCB - 1) / kRouteCB;
  const int cb = tid % NCBp, ks = tid / NCBp;
  const int L = NCBp >= 64 ? 1 : 64 / NCBp;          // lanes of a wave sharing a column block
  const int KR = max(1, (NT / NCBp) / L);  // partial sums left per column after the butterfly
  float* red = smem;
  float* lg = smem + (size_t)KR * TT * E;

  // loads per batch: as many as the registers of a thread hold (fewer threads
  // per CU and fewer tokens per tile leave more)
  constexpr int NB = NT <= 512 ? (TT == 1 ? 2 * kRouteNB : kRouteNB) : (TT == 1 ? kRouteNB : 1);
  float acc[TT][kRouteCB];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int c = 0; c < kRouteCB; ++c) acc[t][c] = 0.f;
  const int c0 = cb * kRouteCB;
  const bool active = cb < ncb && ks * NCBp + cb < NT;
  if (active) {
    const Tin* xr[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) xr[t] = x + (size_t)(t0 + min(t, nt - 1)) * a.ld_x;
    const int kb = ks * rp_.slice, ke = min(a.d_in, kb + rp_.slice);
    const int ke8 = kb + max(0, ke - kb) / 8 * 8;  // full groups of 8; fp32 rows may end in a group of 4
    int k0 = kb;
    if (rp_.vec_cols && c0 + kRouteCB <= E) {
      // batches of NB groups: every load of a batch is issued before its
      // arithmetic, so a batch costs one memory round trip; the sums still run
      // over k in ascending order
      for (; k0 + 8 * NB <= ke8; k0 += 8 * NB) {
        typename Raw8<Tin>::type xq[NB][TT], wq[NB][8];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
          for (int t = 0; t < TT; ++t) xq[b][t] = Raw8<Tin>::fetch(xr[t] + k0 + 8 * b);
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) wq[b][kk] = Raw8<Tin>::fetch(Wg + (size_t)(k0 + 8 * b + kk) * E + c0);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          float xv[TT][8], wv[8][kRouteCB];
#pragma unroll
          for (int t = 0; t < TT; ++t) Raw8<Tin>::unpack(xq[b][t], xv[t]);
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) Raw8<Tin>::unpack(wq[b][kk], wv[kk]);
#pragma unroll
          for (int kk = 0; kk < 8; ++kk)
#pragma unroll
            for (int t = 0; t < TT; ++t)
#pragma unroll
              for (int c = 0; c < kRouteCB; ++c) acc[t][c] = fmaf(xv[t][kk], wv[kk][c], acc[t][c]);
        }
      }
    }
    for (; k0 < ke8; k0 += 8) {
      float xv[TT][8];
#pragma unroll
      for (int t = 0; t < TT; ++t) Vec8<Tin>::load(xr[t] + k0, xv[t]);
      float wv[8][kRouteCB];
      if (rp_.vec_cols && c0 + kRouteCB <= E) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) Vec8<Tin>::load(Wg + (size_t)(k0 + kk) * E + c0, wv[kk]);
      } else {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
#pragma unroll
          for (int c = 0; c < kRouteCB; ++c)
            wv[kk][c] = (c0 + c < E) ? Vec8<Tin>::one(Wg + (size_t)(k0 + kk) * E + c0 + c) : 0.f;
      }
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
          for (int c = 0; c < kRouteCB; ++c) acc[t][c] = fmaf(xv[t][kk], wv[kk][c], acc[t][c]);
    }
    for (int k = ke8; k < ke; ++k) {
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const float xs = Vec8<Tin>::one(xr[t] + k);
#pragma unroll
        for (int c = 0; c < kRouteCB; ++c)
          if (c0 + c < E) acc[t][c] = fmaf(xs, Vec8<Tin>::one(Wg + (size_t)k * E + c0 + c), acc[t][c]);
      }
    }
  }
  // butterfly over the L lanes of this wave that hold the same columns
  for (int o = NCBp; o < 64; o <<= 1) {
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int c = 0; c < kRouteCB; ++c) acc[t][c] += __shfl_xor(acc[t][c], o, 64);
  }
  if (active && (lane / NCBp) % L == 0) {
    const int kr = ks / L;
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int c = 0; c < kRouteCB; ++c)
        if (c0 + c < E) red[((size_t)kr * TT + t) * E + c0 + c] = acc[t][c];
  }
  __syncthreads();
  for (int q = tid; q < TT * E; q += NT) {
    float s = 0.f;
    for (int j = 0; j < KR; ++j) s += red[(size_t)j * TT * E + q];
    lg[q] = s;
  }
  __syncthreads();

  if (a.logits) {
    for (int q = tid; q < nt * E; q += NT) a.logits[(size_t)t0 * E + q] = lg[q];
  }
  route_select(a, lg, t0, nt, wave, NT / 64, tagged, tag);
}

// ---------------------------------------------------------------------------
// segmentation
// ---------------------------------------------------------------------------
// Stable counting sort of the pairs p = t*k + j by adapter, run by one
// workgroup of NW waves; `hist` is NW*E ints of LDS, `wave_tot` NW ints,
// `bad` one int.  Wave w owns a contiguous run of pairs:
//   1. per-wave histogram of adapter ids
//   2. exclusive scan over (adapter, wave): seg_offsets[e] and the first output
//      slot of every (wave, adapter) run
//   3. each wave walks its run in 64-pair chunks; lanes with equal ids are
//      matched with ballots and ranked by lane order, so a segment lists its
//      pairs in ascending id.
// Out-of-range ids are counted into *err_count and left out.
template <int NW>
__device__ __forceinline__ void segment_block(const SegmentArgs& a, int* hist, int* wave_tot, int* bad) {
  constexpr int NT = NW * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, n = a.n_pairs;
  for (int q = tid; q < NW * E; q += NT) hist[q] = 0;
  if (tid == 0) *bad = 0;
  __syncthreads();

  const int run = (n + NW - 1) / NW;
  const int beg = min(n, wave * run), end = min(n, beg + run);

  int my_bad = 0;
  for (int p = beg + lane; p < end; p += 64) {
    const int e = ldc_i32(&a.topk_idx[p]);
    if (e >= 0 && e < E)
      atomicAdd(&hist[wave * E + e], 1);
    else
      ++my_bad;
  }
  my_bad = wave_sum_int(my_bad);
  if (lane == 0 && my_bad) atomicAdd(bad, my_bad);
  __syncthreads();

  int carry = 0;
  for (int e0 = 0; e0 < E; e0 += NT) {
    const int e = e0 + tid;
    int tot = 0;
    if (e < E)
      for (int w = 0; w < NW; ++w) tot += hist[w * E + e];
    const int incl = wave_inclusive_scan(tot, lane);
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int wave_base = 0, block_total = 0;
    for (int w = 0; w < NW; ++w) {
      if (w < wave) wave_base += wave_tot[w];
      block_total += wave_tot[w];
    }
    const int excl = carry + wave_base + incl - tot;
    if (e < E) {
      stc_i32(&a.seg_offsets[e], excl);
      int s = excl;
      for (int w = 0; w < NW; ++w) {
        const int c = hist[w * E + e];
        hist[w * E + e] = s;
        s += c;
      }
    }
    carry += block_total;
    __syncthreads();
  }
  if (tid == 0) {
    stc_i32(&a.seg_offsets[E], carry);
    stc_i32(a.err_count, *bad);
  }
  __syncthreads();

  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  for (int c0 = beg; c0 < end; c0 += 64) {
    const int p = c0 + lane;
    const bool in = p < end;
    const int e = in ? ldc_i32(&a.topk_idx[p]) : -1;
    const bool valid = in && e >= 0 && e < E;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(valid && bit);
      peers &= bit ? m : ~m;
    }
    if (valid) {
      const int rank = __popcll(peers & lanemask_lt(lane));
      stc_i32(&a.pair_perm[hist[wave * E + e] + rank], p);
    }
    // the last lane of each group advances the group's cursor; reads above
    // happen before any of these writes (lockstep wave, in-order LDS)
    __builtin_amdgcn_wave_barrier();
    if (valid && (peers >> lane) == 1ull) hist[wave * E + e] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace rp
