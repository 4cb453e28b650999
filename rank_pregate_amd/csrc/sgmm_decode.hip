// Decode-shaped fused SGMM (T <= 64 tokens): one launch per projection group
// computes, for every projection sharing x,
//
//     y[t] = W0 x[t] + sum_j g[t,j] * B_e (A_e x[t]),   e = idx[t,j]
//
// (AdaFuse technical summary §2.B: the chosen adapters are applied with the
// backbone in a single kernel call).  Decode is bound by HBM: every byte of W0
// is read once.  A fused launch also runs the router and the segmentation
// first (§2.A pre-gating; §2.B decoding steps 1-2), so routing overlaps the
// weight stream instead of preceding it.
//
// Work items, numbered in this order; workgroup b runs items b, b + G, ...:
//   0. (fused) router tiles, then one segmentation item.
//   1. shrink units: for one adapter e and one of KP parts of K, either every
//      token (`dense`, small E) or one chunk of <= 16 pairs of e's segment:
//      unscaled partial products A_e x[t] in fp32.
//   2. base items (32 output rows, one of S splits of K), two waves, each
//      owning 16 rows: bf16 MFMA 16x16x32 with the tokens as M and W0 rows as
//      N.  The tokens' activations for each 256-wide K chunk are staged in LDS
//      with coalesced loads two chunks ahead; W0 rows stream from HBM straight
//      into registers one chunk ahead, in a pinned issue order that keeps the
//      loads in flight behind the math.  Then the adapter deltas: the KP
//      partials of the lane's (token, slot) pairs are summed in part order and
//      scaled by the gate, and each touched adapter adds a (hi, lo) pair of
//      MFMAs on B_e's rows.
// An item only ever waits for items with smaller numbers, and the grid never
// exceeds what the chip holds at once, so every wait ends: the smallest
// unfinished item always has its workgroup running and nothing to wait for.
//
// Data crossing workgroups (routing results, u, split-K partial tiles) is
// written and read with device-scope (sc1) accesses; a writer waits for its
// stores before it bumps a counter, so no cache-wide fence is needed.  The
// split-K partials of a tile are summed in split order by the tile's last
// split, so the output does not depend on timing.
#include "route_common.h"
#include "sgmm_common.h"

namespace rp {
namespace {

constexpr int kSpinLimit = 1 << 22;  // ~seconds; a wait this long flags kCtlWaitOverflow and gives up
constexpr int kWV = 2;               // waves per item
constexpr int kThreads = 64 * kWV;
constexpr int kTileRows = 16 * kWV;
constexpr int kKC = 256;             // K per LDS chunk
constexpr int kSteps = kKC / 32;     // MFMA k-steps per chunk
constexpr int kLD = kKC + 8;         // padded LDS row (elements)
static_assert(kThreads == kRouteThreads, "router tiles run on the decode workgroup shape");

typedef unsigned int u32x4_v __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, CDNA
constexpr int kSc1 = 1 << 4;            // device-scope coherence bit of the cache policy

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ void st_coh16(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_v, v), r, off, 0, kSc1);
}
__device__ __forceinline__ f32x4_t ld_coh16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1));
}

template <int MT, bool FUSED>
constexpr size_t smem_bytes() {
  constexpr size_t xs = 2ull * 16 * MT * kLD * sizeof(bf16_t);
  constexpr size_t red = 8ull * MT * 64 * 4 * sizeof(float);             // shrink: up to 8 rank tiles x MT token tiles
  constexpr size_t route = FUSED ? 3ull * 2 * kMaxE * sizeof(float) : 0;  // router tile, E = 1024
  constexpr size_t seg = FUSED ? 2ull * kMaxE * sizeof(int) : 0;          // two-wave segmentation histograms
  size_t m = xs;
  if (red > m) m = red;
  if (route > m) m = route;
  if (seg > m) m = seg;
  return m;
}

// Per-wave wait until *p >= target (uniform across the wave).
__device__ __forceinline__ void wait_geq(int* ctl, const int* p, int target) {
  int spins = 0;
  while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    __builtin_amdgcn_s_sleep(2);
    if (++spins > kSpinLimit) {
      if ((threadIdx.x & 63) == 0) atomicOr(&ctl[kCtlWaitOverflow], 1);
      break;
    }
  }
}

__device__ __forceinline__ int* ctl_set(int* ctl, int ep) { return ctl + kCtlSet0 + (ep & 1) * kCtlSetStride; }

// Thread 0, once per workgroup: record that this workgroup has read the epoch.
__device__ __forceinline__ int arrive(int* ctl, int ep) {
  return atomicAdd(&ctl_set(ctl, ep)[kSetArrive + 32 * (blockIdx.x & 7)], 1);
}

// u partials of projection `proj`, part kp: [slots][r] fp32 with
// slots = dense ? E * t_pad (adapter-major, then token) : T * k (pair id).
__device__ __forceinline__ size_t upart_slots(const SgmmArgs& a, const DecodeArgs& d) {
  return d.dense ? (size_t)a.E * d.t_pad : (size_t)a.T * a.k;
}

// ---------------------------------------------------------------------------
// shrink units, 2 waves
// ---------------------------------------------------------------------------
// One unit: rank rows of A_e (MTR tiles of 16) against NT tiles of 16 columns
// (tokens when dense, pairs of one segment chunk otherwise) over K part kp;
// the two waves split the part and are added in wave order.
template <int MTR, int NT, bool DENSE, bool COH>
__device__ __forceinline__ void shrink_item(const SgmmArgs& a, const DecodeArgs& d, int proj, int unit, int kp, float* red,
                            int* s_loc) {
  constexpr int U = MTR * NT >= 8 ? 1 : 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int e, slot0 = 0, slot_end = 0;
  if (DENSE) {
    e = unit;
    // adapters no token chose have no consumer (known before the launch only)
    if (!COH && a.seg_offsets[e + 1] == a.seg_offsets[e]) return;
  } else {
    if (tid < 64) {
      int ee, c;
      locate_chunk<COH>(a, unit, 16, tid, &ee, &c);
      if (tid == 0) { s_loc[0] = ee; s_loc[1] = c; }
    }
    __syncthreads();
    e = s_loc[0];
    if (e < 0) return;
    slot0 = ld_route<COH>(&a.seg_offsets[e]) + s_loc[1] * 16;
    slot_end = min(ld_route<COH>(&a.seg_offsets[e + 1]), slot0 + 16);
  }

  const ProjDesc pd = proj_at(a, proj);
  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  const bf16_t* Ae = static_cast<const bf16_t*>(pd.A) + (size_t)e * a.r * a.d_in;
  const int lr = lane & 15, kg = lane >> 4;
  const bf16_t* xp[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int t;
    if (DENSE)
      t = min(nt * 16 + lr, a.T - 1);
    else
      t = ld_route<COH>(&a.pair_perm[min(slot0 + nt * 16 + lr, slot_end - 1)]) / a.k;
    xp[nt] = x + (size_t)t * a.ld_x;
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
  const int pb = nsteps * kp / d.KP, pe = nsteps * (kp + 1) / d.KP;
  const int sb = pb + (pe - pb) * wave / kWV, se = pb + (pe - pb) * (wave + 1) / kWV;
  f32x4_t acc[MTR][NT];
#pragma unroll
  for (int mt = 0; mt < MTR; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s = sb; s < se; s += U) {
    uint4 av[U][MTR], bv[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s + u) * 32 + kg * 8;
      const bool ok = (s + u < se) && (k < a.d_in);
      const int kc = min(k, a.d_in - 8);
#pragma unroll
      for (int mt = 0; mt < MTR; ++mt) av[u][mt] = sel4(ok && aok[mt], ld16(ap[mt] + kc));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) bv[u][nt] = sel4(ok, ld16(xp[nt] + kc));
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MTR; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma16(av[u][mt], bv[u][nt], acc[mt][nt]);
  }
  // wave 0 + wave 1, in that order; D layout: lane -> column nt*16 + lane%16,
  // rank rows mt*16 + 4*(lane/16) + 0..3
  if (wave == 1) {
#pragma unroll
    for (int mt = 0; mt < MTR; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        *reinterpret_cast<f32x4_t*>(&red[((mt * NT + nt) * 64 + lane) * 4]) = acc[mt][nt];
  }
  __syncthreads();
  if (wave == 0) {
    const size_t slots = upart_slots(a, d);
    const float* ub = a.u + ((size_t)proj * d.KP + kp) * slots * a.r;
    const __amdgpu_buffer_rsrc_t r = rsrc(ub, (uint32_t)(slots * a.r * sizeof(float)));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      int slot;
      bool ok;
      if (DENSE) {
        const int t = nt * 16 + lr;
        ok = t < a.T;
        slot = e * d.t_pad + t;
      } else {
        const int s = slot0 + nt * 16 + lr;
        ok = s < slot_end;
        slot = ok ? ld_route<COH>(&a.pair_perm[s]) : 0;
      }
      if (!ok) continue;
#pragma unroll
      for (int mt = 0; mt < MTR; ++mt) {
        const int c = mt * 16 + 4 * kg;
        if (c < a.r) {
          const f32x4_t o = *reinterpret_cast<const f32x4_t*>(&red[((mt * NT + nt) * 64 + lane) * 4]);
          st_coh16(r, (uint32_t)(((size_t)slot * a.r + c) * sizeof(float)), acc[mt][nt] + o);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// base item
// ---------------------------------------------------------------------------
template <int MT, bool TILED, bool FUSED>
__device__ __forceinline__ void base_item(const SgmmArgs& a, const DecodeArgs& d, int bi, bf16_t* xs, int* ctl, int* s_ep,
                          bool first, int ep_in, int* arrive_old, int* s_flag) {
  constexpr int TP = 16 * MT;
  constexpr int XCH = TP * kKC / 8 / kThreads;  // 16-byte x pieces per thread per chunk
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = bi / a.S, split = bi % a.S;
  const int proj = proj_of_tile(a, tile);
  const ProjDesc pd = proj_at(a, proj);
  const int row0 = (tile - pd.tile_begin) * kTileRows + wave * 16;
  const int lr = lane & 15, kg = lane >> 4;
  const int row = min(row0 + lr, pd.d_out - 1);
  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  // row-major: this lane's row at column 8*kg; tiled: this wave's run of 1 KB blocks
  const bf16_t* wrow = TILED
      ? static_cast<const bf16_t*>(pd.W0) + (size_t)(row0 / 16) * (a.d_in / 32) * 512 + lane * 8
      : static_cast<const bf16_t*>(pd.W0) + (size_t)row * a.d_in + kg * 8;
  const int nch = (a.d_in + kKC - 1) / kKC;
  const int cb = (int)((long long)nch * split / a.S), ce = (int)((long long)nch * (split + 1) / a.S);

  f32x4_t acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Loads in the loop are never masked (a select would force a wait right
  // after the load): W0 addresses are clamped into the row, and whatever they
  // read past d_in meets activations that store_x wrote as zero.
  auto load_w = [&](uint4 (&w)[kSteps], int c) {
    const int cc = min(c, ce - 1);
    if (TILED) {
#pragma unroll
      for (int st = 0; st < kSteps; ++st) w[st] = ld16(wrow + (size_t)min(cc * kSteps + st, a.d_in / 32 - 1) * 512);
    } else {
#pragma unroll
      for (int st = 0; st < kSteps; ++st) w[st] = ld16(wrow + min(cc * kKC + st * 32, a.d_in - 8 - kg * 8));
    }
  };
  auto load_x = [&](uint4 (&xr)[XCH], int c) {
    const int cc = min(c, ce - 1);
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int q = tid + i * kThreads;
      const int tok = q / (kKC / 8), kc = (q % (kKC / 8)) * 8;
      xr[i] = ld16(x + (size_t)min(tok, a.T - 1) * a.ld_x + min(cc * kKC + kc, a.d_in - 8));
    }
  };
  auto store_x = [&](const uint4 (&xr)[XCH], int buf, int c) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int q = tid + i * kThreads;
      const int tok = q / (kKC / 8), kc = (q % (kKC / 8)) * 8;
      *reinterpret_cast<uint4*>(&xs[((size_t)buf * TP + tok) * kLD + kc]) =
          sel4(tok < a.T && c < ce && c * kKC + kc < a.d_in, xr[i]);
    }
  };
  auto compute = [&](const uint4 (&w)[kSteps], int buf) {
#pragma unroll
    for (int st = 0; st < kSteps; ++st)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint4 xf = *reinterpret_cast<const uint4*>(&xs[((size_t)buf * TP + m * 16 + lr) * kLD + st * 32 + kg * 8]);
        acc[m] = mfma16(xf, w[st], acc[m]);
      }
  };

  // the lane's tokens' choices; known before the launch unless routing runs in it
  int sel[MT][kMaxK];
  if (!FUSED) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int t = min(m * 16 + lr, a.T - 1);
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) sel[m][j] = (j < a.k && m * 16 + lr < a.T) ? a.topk_idx[t * a.k + j] : -1;
    }
  }

  {
    uint4 wA[kSteps], wB[kSteps], XA[XCH], XB[XCH];
    load_w(wA, cb);
    load_x(XA, cb);
    load_x(XB, cb + 1);
    if (first && tid == 0) {
      *s_ep = ep_in;
      *arrive_old = arrive(ctl, ep_in);
    }
    store_x(XA, 0, cb);
    __syncthreads();
    // chunk pairs, no exit between the two halves; an odd last chunk follows
    int c = cb;
    for (; c + 2 <= ce; c += 2) {
      // chunk c: x in LDS buffer 0, W0 in wA; XB holds chunk c+1
      __builtin_amdgcn_sched_barrier(0);
      load_w(wB, c + 1);
      load_x(XA, c + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(wA, 0);
      __builtin_amdgcn_sched_barrier(0);
      store_x(XB, 1, c + 1);
      __syncthreads();
      // chunk c+1: x in buffer 1, W0 in wB; XA holds chunk c+2
      __builtin_amdgcn_sched_barrier(0);
      load_w(wA, c + 2);
      load_x(XB, c + 3);
      __builtin_amdgcn_sched_barrier(0);
      compute(wB, 1);
      __builtin_amdgcn_sched_barrier(0);
      store_x(XA, 0, c + 2);
      __syncthreads();
    }
    if (c < ce) compute(wA, 0);
  }
  const int ep = *s_ep;
  int* set = ctl_set(ctl, ep);

  // adapter deltas for this wave's 16 rows: adapters e = split, split + S, ...
  // A lane's tokens chose at most k adapters, so it needs u only for its own
  // (token, slot) pairs: their KP partials are loaded two slots per pass,
  // summed in part order and scaled by the gate; the operand for adapter e is
  // then picked in registers.  B rows are loaded eight adapters at a time.
  if (a.k > 0) {
    if (FUSED) wait_geq(ctl, &set[kSetRouteDone], d.n_route);
    wait_geq(ctl, &set[kSetShrinkDone], d.n_shrink);
    if (FUSED) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int t = min(m * 16 + lr, a.T - 1);
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
          sel[m][j] = (j < a.k && m * 16 + lr < a.T) ? ld_route<true>(&a.topk_idx[t * a.k + j]) : -1;
      }
    }
    const bf16_t* Bm = static_cast<const bf16_t*>(pd.B);
    const size_t slots = upart_slots(a, d);
    const float* ub = a.u + (size_t)proj * d.KP * slots * a.r;
    const __amdgpu_buffer_rsrc_t ur = rsrc(ub, (uint32_t)((size_t)d.KP * slots * a.r * sizeof(float)));
    constexpr uint32_t kOob = 0x80000000u;  // past any buffer: the load returns zero
    constexpr int G = 8;                    // adapters per batch of B loads
    for (int c0 = 0; c0 < a.r; c0 += 32) {
      const int c = c0 + kg * 8;
      const int cc = min(c, a.r - 8);
      for (int jp = 0; jp < a.k; jp += 2) {
        f32x4_t uu[MT][2][2];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int j = min(jp + q, kMaxK - 1);
            const int t = m * 16 + lr;
            const bool ok = jp + q < a.k && c < a.r && sel[m][j] >= 0;
            const size_t slot = d.dense ? (size_t)max(sel[m][j], 0) * d.t_pad + t : (size_t)t * a.k + j;
            const uint32_t off = ok ? (uint32_t)((slot * a.r + cc) * sizeof(float)) : kOob;
            const uint32_t part = (uint32_t)(slots * a.r * sizeof(float));
            f32x4_t s0 = ld_coh16(ur, off), s1 = ld_coh16(ur, ok ? off + 16 : kOob);
            for (int kp = 1; kp < d.KP; ++kp) {
              s0 += ld_coh16(ur, ok ? off + kp * part : kOob);
              s1 += ld_coh16(ur, ok ? off + kp * part + 16 : kOob);
            }
            const float g = ok ? ld_route<FUSED>(&a.topk_gate[min(t, a.T - 1) * a.k + j]) : 0.f;
            uu[m][q][0] = g * s0;
            uu[m][q][1] = g * s1;
          }
        for (int e0 = split; e0 < a.E; e0 += G * a.S) {
          int js[G][MT];  // slot (jp or jp+1) of the lane's token that chose adapter e, else -1
          bool any[G];
          bool group = false;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const int e = e0 + g * a.S;
            any[g] = false;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              js[g][m] = -1;
#pragma unroll
              for (int q = 0; q < 2; ++q)
                if (jp + q < kMaxK && sel[m][min(jp + q, kMaxK - 1)] == e) js[g][m] = q;
              any[g] |= __ballot(js[g][m] >= 0) != 0;
            }
            group |= any[g];
          }
          if (!group) continue;
          uint4 bo[G];
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const int e = min(e0 + g * a.S, a.E - 1);
            bo[g] = ld16(Bm + ((size_t)e * pd.d_out + row) * a.r + cc);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            if (!any[g]) continue;
            const uint4 b = sel4(c < a.r, bo[g]);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              const int q = js[g][m];
              float v[8];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                v[i] = q == 0 ? uu[m][0][0][i] : (q == 1 ? uu[m][1][0][i] : 0.f);
                v[4 + i] = q == 0 ? uu[m][0][1][i] : (q == 1 ? uu[m][1][1][i] : 0.f);
              }
              uint4 hi, lo;
              split_hi_lo(v, hi, lo);
              acc[m] = mfma16(hi, b, acc[m]);
              acc[m] = mfma16(lo, b, acc[m]);
            }
          }
        }
      }
    }
  }

  if (a.S > 1) {
    // split-K: splits 0..S-2 publish their partial tiles and count in; the
    // last split waits for them and sums all S in split order
    constexpr int kWaveBytes = MT * 64 * 16;
    const size_t tile_bytes = (size_t)a.S * kWV * kWaveBytes;
    const __amdgpu_buffer_rsrc_t pr = rsrc(reinterpret_cast<char*>(a.partial) + tile * tile_bytes, (uint32_t)tile_bytes);
    int* tc = &ctl[kCtlTiles + tile];
    if (split != a.S - 1) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
        st_coh16(pr, (uint32_t)((split * kWV + wave) * kWaveBytes + (m * 64 + lane) * 16), acc[m]);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) __hip_atomic_fetch_add(tc, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    wait_geq(ctl, tc, a.S - 1);
    __syncthreads();
    if (tid == 0) __hip_atomic_store(tc, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    f32x4_t tot[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) tot[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < a.S; ++s) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
        tot[m] += (s == split) ? acc[m] : ld_coh16(pr, (uint32_t)((s * kWV + wave) * kWaveBytes + (m * 64 + lane) * 16));
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = tot[m];
  }

  // store: lane -> output row row0 + lane%16; accumulator v -> token m*16 + 4*(lane/16) + v
  if (row0 + lr < pd.d_out) {
    bf16_t* y = static_cast<bf16_t*>(pd.y);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = m * 16 + 4 * kg + v;
        if (t < a.T) y[(size_t)t * pd.ld_y + row0 + lr] = f32_to_bf16(acc[m][v]);
      }
  }
}

// ---------------------------------------------------------------------------
// kernel
// ---------------------------------------------------------------------------
template <int MT, bool FUSED>
__global__ __launch_bounds__(kThreads) void decode_kernel(SgmmArgs a, DecodeArgs d) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[smem_bytes<MT, FUSED>()];
  __shared__ int s_ep, s_loc[2], s_flag, s_wave_tot[2], s_bad;
  int* ctl = a.counters;
  const int tid = threadIdx.x;
  // the epoch is read once per workgroup; base items publish it after their
  // first loads are in flight, other items right away
  int ep_in = 0, arrive_old = 0;
  if (tid == 0) ep_in = __hip_atomic_load(&ctl[kCtlEpoch], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int n_base0 = d.n_pre + d.n_shrink;
  bool first = true;
  for (int item = blockIdx.x; item < d.n_items; item += gridDim.x) {
    if (item < n_base0 && first) {
      if (tid == 0) {
        s_ep = ep_in;
        arrive_old = arrive(ctl, ep_in);
      }
      __syncthreads();
      first = false;
    }
    if (FUSED && item < d.n_route) {
      // router tile: top-k and gates of TT tokens
      int* set = ctl_set(ctl, s_ep);
      const RoutePlan rpl = route_plan(d.pg.E, d.pg.d_in, (int)sizeof(bf16_t));
      float* f = reinterpret_cast<float*>(smem);
      if (rpl.TT == 4)
        route_tile<bf16_t, 4>(d.pg, item * 4, rpl, f);
      else
        route_tile<bf16_t, 2>(d.pg, item * 2, rpl, f);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) atomicAdd(&set[kSetRouteDone], 1);
    } else if (FUSED && item < d.n_pre) {
      int* set = ctl_set(ctl, s_ep);
      wait_geq(ctl, &set[kSetRouteDone], d.n_route);
      segment_block<kWV>(d.sg, reinterpret_cast<int*>(smem), s_wave_tot, &s_bad);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) atomicAdd(&set[kSetSegDone], 1);
    } else if (item < n_base0) {
      int* set = ctl_set(ctl, s_ep);
      const int si = item - d.n_pre;
      const int proj = si / d.units_per_proj, w = si % d.units_per_proj;
      const int unit = w / d.KP, kp = w % d.KP;
      float* red = reinterpret_cast<float*>(smem);
      if (d.dense) {
        switch ((a.r + 15) >> 4) {
          case 1: shrink_item<1, MT, true, FUSED>(a, d, proj, unit, kp, red, s_loc); break;
          case 2: shrink_item<2, MT, true, FUSED>(a, d, proj, unit, kp, red, s_loc); break;
          case 4: shrink_item<4, MT, true, FUSED>(a, d, proj, unit, kp, red, s_loc); break;
          default: shrink_item<8, MT, true, FUSED>(a, d, proj, unit, kp, red, s_loc); break;
        }
      } else {
        if (FUSED) wait_geq(ctl, &set[kSetSegDone], 1);
        switch ((a.r + 15) >> 4) {
          case 1: shrink_item<1, 1, false, FUSED>(a, d, proj, unit, kp, red, s_loc); break;
          case 2: shrink_item<2, 1, false, FUSED>(a, d, proj, unit, kp, red, s_loc); break;
          case 4: shrink_item<4, 1, false, FUSED>(a, d, proj, unit, kp, red, s_loc); break;
          default: shrink_item<8, 1, false, FUSED>(a, d, proj, unit, kp, red, s_loc); break;
        }
      }
      // the u stores are device-coherent; wait for them before counting this unit done
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) atomicAdd(&set[kSetShrinkDone], 1);
    } else {
      const int bi = item - n_base0;
      const int bp = proj_of_tile(a, bi / a.S);
      if (RP_PICK(a, bp, tiled))
        base_item<MT, true, FUSED>(a, d, bi, reinterpret_cast<bf16_t*>(smem), ctl, &s_ep, first, ep_in, &arrive_old,
                                   &s_flag);
      else
        base_item<MT, false, FUSED>(a, d, bi, reinterpret_cast<bf16_t*>(smem), ctl, &s_ep, first, ep_in, &arrive_old,
                                    &s_flag);
      first = false;
    }
    __syncthreads();  // LDS is reused by the next item
  }
  // The last workgroup to have read the epoch clears the other control set
  // for the next launch and advances the epoch.  Arrivals are counted per
  // blockIdx % 8 class first, so no single counter takes every workgroup.
  if (tid == 0) {
    const int G = gridDim.x, cls = blockIdx.x & 7;
    const int count_c = (G - 1 - cls) / 8 + 1;
    if (arrive_old == count_c - 1) {
      const int n_classes = G < 8 ? G : 8;
      int* set = ctl_set(ctl, s_ep);
      if (atomicAdd(&set[kSetArriveAll], 1) == n_classes - 1) {
        int* other = ctl_set(ctl, s_ep + 1);
        for (int w = 0; w < kSetWords; w += 32) __hip_atomic_store(&other[w], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ctl[kCtlEpoch], s_ep + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

template <int MT, bool FUSED>
int resident_per_cu() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  if (cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<MT, FUSED>, kThreads, 0) != hipSuccess || n < 1)
    n = 1;
  cache[dev] = n;
  return n;
}

template <bool FUSED>
hipError_t launch_t(const SgmmArgs& a, const DecodeArgs& d, const SgmmPlan& plan, hipStream_t s) {
  const dim3 grid(plan.grid);
  switch (decode_mt(a.T)) {
    case 1: decode_kernel<1, FUSED><<<grid, kThreads, 0, s>>>(a, d); break;
    case 2: decode_kernel<2, FUSED><<<grid, kThreads, 0, s>>>(a, d); break;
    default: decode_kernel<4, FUSED><<<grid, kThreads, 0, s>>>(a, d); break;
  }
  return hipGetLastError();
}

}  // namespace

int decode_mt(int T) { return T <= 16 ? 1 : T <= 32 ? 2 : 4; }
int decode_chunk_k(int T) { (void)T; return kKC; }
int decode_tile_rows() { return kTileRows; }

int decode_resident_per_cu(int T, bool fused) {
  switch (decode_mt(T)) {
    case 1: return fused ? resident_per_cu<1, true>() : resident_per_cu<1, false>();
    case 2: return fused ? resident_per_cu<2, true>() : resident_per_cu<2, false>();
    default: return fused ? resident_per_cu<4, true>() : resident_per_cu<4, false>();
  }
}

static DecodeArgs decode_args(const SgmmArgs& a, const SgmmPlan& plan) {
  DecodeArgs d{};
  d.n_route = plan.n_route;
  d.n_pre = plan.n_pre;
  d.units_per_proj = plan.units_per_proj;
  d.n_shrink = plan.units_per_proj * a.n_proj;
  d.n_items = plan.n_items;
  d.KP = plan.KP;
  d.dense = plan.dense;
  d.t_pad = plan.t_pad;
  return d;
}

hipError_t launch_decode(const SgmmArgs& a, const SgmmPlan& plan, hipStream_t s) {
  DecodeArgs d = decode_args(a, plan);
  d.fused = 0;
  return launch_t<false>(a, d, plan, s);
}

hipError_t launch_route_sgmm(const SgmmArgs& a, const PregateArgs& pg, const SegmentArgs& sg, const SgmmPlan& plan,
                             hipStream_t s) {
  DecodeArgs d = decode_args(a, plan);
  d.fused = 1;
  d.pg = pg;
  d.sg = sg;
  return launch_t<true>(a, d, plan, s);
}

}  // namespace rp
