// Decode-shaped fused SGMM (T <= 64 tokens): one launch per projection group
// computes, for every projection sharing x,
//
//     y[t] = W0 x[t] + sum_j g[t,j] * B_e (A_e x[t]),   e = idx[t,j]
//
// (AdaFuse technical summary §2.B: the chosen adapters are applied with the
// backbone in a single kernel call).  Decode is bound by HBM: every byte of W0
// is read once.
//
// Work items, handed out in launch order through a ticket counter:
//   1. shrink units (projection, chunk of <= 16 pairs of one adapter segment):
//      u[pair] = g * A_e x[t] in fp32; each chosen A_e is streamed once.
//   2. base items (32 output rows, one of S splits of K), two waves, each
//      owning 16 rows: bf16 MFMA 16x16x32 with the tokens as M and W0 rows as
//      N.  The tokens' activations for each 256-wide K chunk are staged in LDS
//      with coalesced loads two chunks ahead; W0 rows stream from HBM straight
//      into registers one chunk ahead.  The issue order of loads and MFMAs is
//      pinned so the loads stay in flight behind the math.  Then the adapter
//      deltas: per touched adapter and 16-token tile, a (hi, lo) pair of MFMAs
//      on B_e's rows and the gathered u.
// Tickets go out in order, so every shrink unit is taken by a running
// workgroup before any base item: a base item only waits for workgroups that
// are already running, and the wait always ends.
//
// Data crossing workgroups (u, split-K partial tiles) is written and read with
// device-scope (sc1) 16-byte buffer accesses, and a writer waits for its
// stores to complete before it bumps a counter, so no cache-wide fence is
// needed.  Split-K partials are summed in split order by the last of the S
// workgroups: the output does not depend on timing.
#include "sgmm_common.h"

namespace rp {
namespace {

constexpr int kSpinLimit = 1 << 24;  // ~seconds; a wait this long flags kCtlWaitOverflow and gives up
constexpr int kWV = 2;               // waves per base item
constexpr int kThreads = 64 * kWV;
constexpr int kTileRows = 16 * kWV;
constexpr int kKC = 256;             // K per LDS chunk
constexpr int kSteps = kKC / 32;     // MFMA k-steps per chunk
constexpr int kLD = kKC + 8;         // padded LDS row (elements)

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

// ---------------------------------------------------------------------------
// shrink unit, 2 waves
// ---------------------------------------------------------------------------
template <int MTR>
__device__ void shrink_item(const SgmmArgs& a, int proj, int unit, float* red, int* s_loc) {
  constexpr int U = MTR >= 4 ? 2 : 16 / MTR;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 64) {
    int e, c;
    locate_chunk(a, unit, 16, tid, &e, &c);
    if (tid == 0) { s_loc[0] = e; s_loc[1] = c; }
  }
  __syncthreads();
  const int e = s_loc[0], chunk = s_loc[1];
  if (e < 0) return;

  const ProjDesc pd = proj_at(a, proj);
  const int slot0 = a.seg_offsets[e] + chunk * 16;
  const int slot_end = min(a.seg_offsets[e + 1], slot0 + 16);
  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  const bf16_t* Ae = static_cast<const bf16_t*>(pd.A) + (size_t)e * a.r * a.d_in;
  const int lr = lane & 15, kg = lane >> 4;
  const bf16_t* xp = x + (size_t)(a.pair_perm[min(slot0 + lr, slot_end - 1)] / a.k) * a.ld_x;
  const bf16_t* ap[MTR];
  bool aok[MTR];
#pragma unroll
  for (int mt = 0; mt < MTR; ++mt) {
    const int c = mt * 16 + lr;
    aok[mt] = c < a.r;
    ap[mt] = Ae + (size_t)min(c, a.r - 1) * a.d_in;
  }
  const int nsteps = (a.d_in + 31) >> 5;
  const int sb = nsteps * wave / kWV, se = nsteps * (wave + 1) / kWV;
  f32x4_t acc[MTR];
#pragma unroll
  for (int mt = 0; mt < MTR; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s = sb; s < se; s += U) {
    uint4 av[U][MTR], bv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s + u) * 32 + kg * 8;
      const bool ok = (s + u < se) && (k < a.d_in);
      const int kc = min(k, a.d_in - 8);
#pragma unroll
      for (int mt = 0; mt < MTR; ++mt) av[u][mt] = sel4(ok && aok[mt], ld16(ap[mt] + kc));
      bv[u] = sel4(ok, ld16(xp + kc));
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MTR; ++mt) acc[mt] = mfma16(av[u][mt], bv[u], acc[mt]);
  }
  // fixed-order sum of the two waves in LDS; D layout: lane -> pair lane%16,
  // rank rows mt*16 + 4*(lane/16) + 0..3 (four consecutive ranks)
  if (wave == 1) {
#pragma unroll
    for (int mt = 0; mt < MTR; ++mt) *reinterpret_cast<f32x4_t*>(&red[(mt * 64 + lane) * 4]) = acc[mt];
  }
  __syncthreads();
  if (wave == 0) {
    const int slot = slot0 + lr;
    if (slot < slot_end) {
      const int p = a.pair_perm[slot];
      const float g = a.topk_gate[p];
      const float* ubase = a.u + (size_t)proj * a.T * a.k * a.r;
      const __amdgpu_buffer_rsrc_t r = rsrc(ubase, (uint32_t)((size_t)a.T * a.k * a.r * sizeof(float)));
#pragma unroll
      for (int mt = 0; mt < MTR; ++mt) {
        const int c = mt * 16 + 4 * kg;
        if (c < a.r) {
          const f32x4_t o = *reinterpret_cast<const f32x4_t*>(&red[(mt * 64 + lane) * 4]);
          f32x4_t v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = g * (acc[mt][i] + o[i]);
          st_coh16(r, (uint32_t)(((size_t)p * a.r + c) * sizeof(float)), v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// base item
// ---------------------------------------------------------------------------
// Per-wave wait for the shrink units of this launch (uniform across the wave).
__device__ __forceinline__ void wait_shrink(int* ctl, int n_shrink) {
  int spins = 0;
  while (__hip_atomic_load(&ctl[kCtlShrinkDone], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < n_shrink) {
    __builtin_amdgcn_s_sleep(2);
    if (++spins > kSpinLimit) {
      if ((threadIdx.x & 63) == 0) atomicOr(&ctl[kCtlWaitOverflow], 1);
      break;
    }
  }
}

template <int MT, bool TILED>
__device__ void base_item(const SgmmArgs& a, int item, bf16_t* xs, int* ctl, int n_shrink, int* s_flag) {
  constexpr int TP = 16 * MT;
  constexpr int XCH = TP * kKC / 8 / kThreads;  // 16-byte x pieces per thread per chunk
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = item / a.S, split = item % a.S;
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

  // the lane's tokens' choices (for the adapter deltas), read before the stream starts
  int sel[MT][kMaxK];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int t = min(m * 16 + lr, a.T - 1);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) sel[m][j] = (j < a.k && m * 16 + lr < a.T) ? a.topk_idx[t * a.k + j] : -1;
  }

  if (cb < ce) {
    uint4 wA[kSteps], wB[kSteps], XA[XCH], XB[XCH];
    load_w(wA, cb);
    load_x(XA, cb);
    load_x(XB, cb + 1);
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

  // adapter deltas for this wave's 16 rows: adapters e = split, split + S, ...
  // A lane's tokens chose at most k adapters, so it needs u only for its own
  // (token, slot) pairs: those are loaded once, two slots per pass, right after
  // the shrink units finish (one round trip of device-coherent loads), and the
  // operand for adapter e is picked from them in registers.  The tokens'
  // choices are read before the wait; B rows are loaded eight adapters at a
  // time, together.
  if (a.k > 0) {
    const bf16_t* Bm = static_cast<const bf16_t*>(pd.B);
    const float* ub = a.u + (size_t)proj * a.T * a.k * a.r;
    const __amdgpu_buffer_rsrc_t ur = rsrc(ub, (uint32_t)((size_t)a.T * a.k * a.r * sizeof(float)));
    constexpr uint32_t kOob = 0x80000000u;  // past any buffer: the load returns zero
    constexpr int G = 8;                    // adapters per batch of B loads
    wait_shrink(ctl, n_shrink);
    for (int c0 = 0; c0 < a.r; c0 += 32) {
      const int c = c0 + kg * 8;
      const int cc = min(c, a.r - 8);
      for (int jp = 0; jp < a.k; jp += 2) {
        f32x4_t uu[MT][2][2];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int j = jp + q;
            const bool ok = j < a.k && c < a.r && sel[m][min(j, kMaxK - 1)] >= 0;
            const uint32_t off =
                ok ? (uint32_t)((((size_t)(m * 16 + lr) * a.k + j) * a.r + cc) * sizeof(float)) : kOob;
            uu[m][q][0] = ld_coh16(ur, off);
            uu[m][q][1] = ld_coh16(ur, ok ? off + 16 : kOob);
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
    // split-K: publish this partial; the last of the S workgroups sums all S
    // partials in split order and writes the tile
    constexpr int kWaveBytes = MT * 64 * 16;
    const size_t tile_bytes = (size_t)a.S * kWV * kWaveBytes;
    const __amdgpu_buffer_rsrc_t pr = rsrc(reinterpret_cast<char*>(a.partial) + tile * tile_bytes, (uint32_t)tile_bytes);
#pragma unroll
    for (int m = 0; m < MT; ++m)
      st_coh16(pr, (uint32_t)((split * kWV + wave) * kWaveBytes + (m * 64 + lane) * 16), acc[m]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) *s_flag = (atomicAdd(&ctl[kCtlTiles + tile], 1) == a.S - 1);
    __syncthreads();
    if (!*s_flag) return;
    if (tid == 0) __hip_atomic_store(&ctl[kCtlTiles + tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

template <int MT>
__global__ __launch_bounds__(kThreads) void decode_fused(SgmmArgs a, int units_per_proj, int n_shrink, int n_items) {
  constexpr size_t kXsBytes = 2ull * 16 * MT * kLD * sizeof(bf16_t);
  __shared__ __attribute__((aligned(16))) unsigned char smem[kXsBytes > 8192 ? kXsBytes : 8192];
  __shared__ int s_ticket, s_loc[2], s_flag;
  int* ctl = a.counters;
  const int tid = threadIdx.x;
  if (tid == 0) s_ticket = atomicAdd(&ctl[kCtlTicket], 1);
  __syncthreads();
  const int item = s_ticket;

  if (item < n_shrink) {
    float* red = reinterpret_cast<float*>(smem);
    const int proj = item / units_per_proj, unit = item % units_per_proj;
    switch ((a.r + 15) >> 4) {
      case 1: shrink_item<1>(a, proj, unit, red, s_loc); break;
      case 2: shrink_item<2>(a, proj, unit, red, s_loc); break;
      case 4: shrink_item<4>(a, proj, unit, red, s_loc); break;
      default: shrink_item<8>(a, proj, unit, red, s_loc); break;
    }
    // the u stores are device-coherent; wait for them before counting this unit done
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) atomicAdd(&ctl[kCtlShrinkDone], 1);
  } else {
    const int bi = item - n_shrink;
    const int bp = proj_of_tile(a, bi / a.S);
    if (RP_PICK(a, bp, tiled))
      base_item<MT, true>(a, bi, reinterpret_cast<bf16_t*>(smem), ctl, n_shrink, &s_flag);
    else
      base_item<MT, false>(a, bi, reinterpret_cast<bf16_t*>(smem), ctl, n_shrink, &s_flag);
  }
  // the last workgroup to finish clears the launch's control words
  if (tid == 0) {
    if (atomicAdd(&ctl[kCtlFinished], 1) == n_items - 1) {
      ctl[kCtlTicket] = 0;
      ctl[kCtlShrinkDone] = 0;
      ctl[kCtlFinished] = 0;
    }
  }
}

}  // namespace

int decode_mt(int T) { return T <= 16 ? 1 : T <= 32 ? 2 : 4; }
int decode_chunk_k(int T) { (void)T; return kKC; }
int decode_tile_rows() { return kTileRows; }

hipError_t launch_decode(const SgmmArgs& a, const SgmmPlan& plan, hipStream_t s) {
  const int units = a.k > 0 ? a.E + (a.T * a.k + 15) / 16 : 0;
  const int n_shrink = units * a.n_proj;
  const int n_items = n_shrink + plan.n_tiles * plan.S;
  const dim3 grid(n_items);
  switch (decode_mt(a.T)) {
    case 1: decode_fused<1><<<grid, kThreads, 0, s>>>(a, units, n_shrink, n_items); break;
    case 2: decode_fused<2><<<grid, kThreads, 0, s>>>(a, units, n_shrink, n_items); break;
    default: decode_fused<4><<<grid, kThreads, 0, s>>>(a, units, n_shrink, n_items); break;
  }
  return hipGetLastError();
}

}  // namespace rp
