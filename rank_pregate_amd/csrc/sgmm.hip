// Fused pre-gated segmented gather matrix multiply (AdaFuse, technical summary
// §2.B): for every projection p sharing the token activations x,
//
//     y[t] = W0 x[t] + sum_j g[t,j] * B_e (A_e x[t]),   e = idx[t,j].
//
// Stage 1 (shrink): per adapter segment, u[pair] = g * A_e x[t] (rank r, fp32).
//   The segment's tokens are gathered so each chosen A_e is streamed once per
//   chunk of up to 16*NCT pairs.  bf16 MFMA 16x16x32, fp32 accumulation.
// Stage 2 (base + expand): output rows are tiled; each tile streams its W0 rows
//   once for all tokens (bf16 MFMA) and adds the chosen adapters' deltas as
//   extra MFMA steps whose operands are B_e's rows and the gathered u (split
//   into a high and a low bf16 part, so the delta keeps ~16 bits).
//   decode (T <= 256): 32-row tiles over all tokens, K split over the 4 waves
//     of a workgroup and over S workgroups; the partial tiles are summed in a
//     fixed order by the last workgroup to arrive, so results are
//     deterministic.
//   prefill (T > 256): 128-token x 128-row LDS-tiled MFMA GEMM; tokens taken
//     in segment order (top-1) so a tile meets few adapters.
// fp32 inputs use plain VALU kernels of the same structure.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace rp {
namespace {

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
  return d;
}

__device__ __forceinline__ uint4 sel4(bool ok, uint4 v) { return ok ? v : zero4(); }

// Slot j of token t chose adapter e?  (-1 if none)
__device__ __forceinline__ int match_slot(const int* idx, int t, int k, int e) {
  int js = -1;
  for (int j = 0; j < k; ++j)
    if (idx[t * k + j] == e) js = j;
  return js;
}

// Gated u row chunk [c, c+8) of pair p as hi/lo bf16 operands (zero if !ok).
__device__ __forceinline__ void u_operand(const float* u, int r, int p, int c, bool ok, uint4& hi,
                                          uint4& lo) {
  float v[8];
  if (ok) {
    const float4 a = *reinterpret_cast<const float4*>(u + (size_t)p * r + c);
    const float4 b = *reinterpret_cast<const float4*>(u + (size_t)p * r + c + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
  }
  split_hi_lo(v, hi, lo);
}

// ============================================================================
// Stage 1: shrink, bf16.  One workgroup per (projection, segment chunk).
// ============================================================================
template <int MT, int NCT, int WAVES, int U>
__global__ __launch_bounds__(WAVES * 64) void shrink_bf16(SgmmArgs a, int units_per_proj) {
  constexpr int NCH = 16 * NCT;
  __shared__ int s_e, s_chunk;
  __shared__ float red[MT * NCT * 4][64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int proj = blockIdx.x / units_per_proj;
  const int unit = blockIdx.x % units_per_proj;

  // locate (segment, chunk) of this unit: chunks are numbered segment by segment
  if (wave == 0) {
    int carry = 0, fe = -1, fc = 0;
    for (int e0 = 0; e0 < a.E; e0 += 64) {
      const int e = e0 + lane;
      const int n = (e < a.E) ? (a.seg_offsets[e + 1] - a.seg_offsets[e]) : 0;
      const int c = (n + NCH - 1) / NCH;
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
    if (lane == 0) { s_e = fe; s_chunk = fc; }
  }
  __syncthreads();
  const int e = s_e;
  if (e < 0) return;

  const ProjDesc pd = proj_at(a, proj);
  const int slot0 = a.seg_offsets[e] + s_chunk * NCH;
  const int slot_end = min(a.seg_offsets[e + 1], slot0 + NCH);
  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  const bf16_t* Ae = static_cast<const bf16_t*>(pd.A) + (size_t)e * a.r * a.d_in;
  const int lr = lane & 15, kg = lane >> 4;

  const bf16_t* xp[NCT];
#pragma unroll
  for (int nt = 0; nt < NCT; ++nt) {
    const int slot = min(slot0 + nt * 16 + lr, slot_end - 1);
    const int t = a.pair_perm[slot] / a.k;
    xp[nt] = x + (size_t)t * a.ld_x;
  }
  const bf16_t* ap[MT];
  bool aok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int c = mt * 16 + lr;
    aok[mt] = c < a.r;
    ap[mt] = Ae + (size_t)min(c, a.r - 1) * a.d_in;
  }

  const int nsteps = (a.d_in + 31) >> 5;
  const int sb = nsteps * wave / WAVES, se = nsteps * (wave + 1) / WAVES;
  f32x4_t acc[MT][NCT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NCT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int s = sb; s < se; s += U) {
    uint4 av[U][MT], bv[U][NCT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s + u) * 32 + kg * 8;
      const bool ok = (s + u < se) && (k < a.d_in);
      const int kc = min(k, a.d_in - 8);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) av[u][mt] = sel4(ok && aok[mt], ld16(ap[mt] + kc));
#pragma unroll
      for (int nt = 0; nt < NCT; ++nt) bv[u][nt] = sel4(ok, ld16(xp[nt] + kc));
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NCT; ++nt) acc[mt][nt] = mfma16(av[u][mt], bv[u][nt], acc[mt][nt]);
  }

  // fixed-order sum over waves (wave 0 first), accumulated in LDS
  for (int w = 0; w < WAVES; ++w) {
    if (wave == w) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NCT; ++nt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float& dst = red[(mt * NCT + nt) * 4 + v][lane];
            dst = (w == 0) ? acc[mt][nt][v] : dst + acc[mt][nt][v];
          }
    }
    __syncthreads();
  }

  // D layout: lane -> pair lane%16, rank row 4*(lane/16)+v
  float* u_out = a.u + (size_t)proj * a.T * a.k * a.r;
  for (int q = tid; q < MT * NCT * 4 * 64; q += WAVES * 64) {
    const int l = q & 63, f = q >> 6;
    const int v = f & 3, nt = (f >> 2) % NCT, mt = (f >> 2) / NCT;
    const float sum = red[f][l];
    const int slot = slot0 + nt * 16 + (l & 15);
    const int c = mt * 16 + 4 * (l >> 4) + v;
    if (slot < slot_end && c < a.r) {
      const int p = a.pair_perm[slot];
      u_out[(size_t)p * a.r + c] = a.topk_gate[p] * sum;
    }
  }
}

// ============================================================================
// Stage 2, decode: base + expand, bf16, 32 output rows x all T (<= 32*NT) tokens.
// MFMA 32x32x16 with A = token activations (M = tokens) and B = W0^T (N = rows),
// so a lane's accumulators share one output row.
// ============================================================================
template <int NT, int U>
__device__ __forceinline__ void decode_load(uint4 (&wv)[U], uint4 (&xv)[U][NT], const bf16_t* wrow,
                                            const bf16_t* const (&xrow)[NT], int s, int se, int kg,
                                            int d_in) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int k = (s + u) * 16 + kg * 8;
    const bool ok = (s + u < se) && (k < d_in);
    const int kc = min(k, d_in - 8);
    wv[u] = sel4(ok, ld16_stream(wrow + kc));
#pragma unroll
    for (int n = 0; n < NT; ++n) xv[u][n] = sel4(ok, ld16(xrow[n] + kc));
  }
}

template <int NT, int U>
__device__ __forceinline__ void decode_mma(f32x16_t (&acc)[NT], const uint4 (&wv)[U],
                                           const uint4 (&xv)[U][NT]) {
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = mfma32(xv[u][n], wv[u], acc[n]);
}

template <int NT, int U>
__global__ __launch_bounds__(256) void decode_bf16(SgmmArgs a) {
  __shared__ float red[3][NT * 16][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x / a.S, split = blockIdx.x % a.S;
  const int proj = proj_of_tile(a, tile);
  const ProjDesc pd = proj_at(a, proj);
  const int row0 = (tile - pd.tile_begin) * 32;
  const int lr = lane & 31, kg = lane >> 5;
  const int row = min(row0 + lr, pd.d_out - 1);
  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  const bf16_t* wrow = static_cast<const bf16_t*>(pd.W0) + (size_t)row * a.d_in;
  const bf16_t* xrow[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) xrow[n] = x + (size_t)min(n * 32 + lr, a.T - 1) * a.ld_x;

  const int nsteps = (a.d_in + 15) >> 4;
  const int H = a.S * 4, h = split * 4 + wave;
  const int sb = (int)((long long)nsteps * h / H), se = (int)((long long)nsteps * (h + 1) / H);

  f32x16_t acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[n][v] = 0.f;

  // software pipeline: the next batch of U k-steps is in flight while the
  // current one feeds the MFMAs (loads past the end re-read the last batch and
  // are not used)
  const int nb = (se - sb + U - 1) / U;
  if (nb > 0) {
    uint4 w0[U], x0[U][NT], w1[U], x1[U][NT];
    decode_load<NT, U>(w0, x0, wrow, xrow, sb, se, kg, a.d_in);
    for (int b = 0; b < nb; b += 2) {
      decode_load<NT, U>(w1, x1, wrow, xrow, sb + min(b + 1, nb - 1) * U, se, kg, a.d_in);
      decode_mma<NT, U>(acc, w0, x0);
      decode_load<NT, U>(w0, x0, wrow, xrow, sb + min(b + 2, nb - 1) * U, se, kg, a.d_in);
      if (b + 1 < nb) decode_mma<NT, U>(acc, w1, x1);
    }
  }

  // expand: adapters e = h, h+H, ... are this wave's share of the deltas
  if (a.k > 0) {
    const bf16_t* Bm = static_cast<const bf16_t*>(pd.B);
    const float* ub = a.u + (size_t)proj * a.T * a.k * a.r;
    for (int e = h; e < a.E; e += H) {
      const int o0 = a.seg_offsets[e], o1 = a.seg_offsets[e + 1];
      if (o0 == o1) continue;
      int ntm = 0;
      for (int q = o0 + lane; q < o1; q += 64) ntm |= 1 << ((a.pair_perm[q] / a.k) >> 5);
      ntm = wave_or(ntm);
      const bf16_t* Be = Bm + ((size_t)e * pd.d_out + row) * a.r;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if (!((ntm >> n) & 1)) continue;
        const int t = n * 32 + lr;
        const int js = (t < a.T) ? match_slot(a.topk_idx, t, a.k, e) : -1;
        for (int c0 = 0; c0 < a.r; c0 += 16) {
          const int c = c0 + kg * 8;
          const bool cok = c < a.r;
          const uint4 bo = sel4(cok, ld16(Be + min(c, a.r - 8)));
          uint4 hi, lo;
          u_operand(ub, a.r, t * a.k + max(js, 0), min(c, a.r - 8), cok && js >= 0, hi, lo);
          acc[n] = mfma32(hi, bo, acc[n]);
          acc[n] = mfma32(lo, bo, acc[n]);
        }
      }
    }
  }

  // fixed-order reduction over the 4 waves
  if (wave > 0) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int v = 0; v < 16; ++v) red[wave - 1][n * 16 + v][lane] = acc[n][v];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[n][v] += red[w][n * 16 + v][lane];

  if (a.S > 1) {
    // split-K: publish this partial; the last of the S workgroups sums all S
    // partials in split order and writes the tile
    constexpr int kTileFloats = NT * 16 * 64;
    float* P = a.partial + (size_t)tile * a.S * kTileFloats;
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int v = 0; v < 16; ++v) P[(size_t)split * kTileFloats + (n * 16 + v) * 64 + lane] = acc[n][v];
    __threadfence();
    int prev = 0;
    if (lane == 0) prev = atomicAdd(&a.counters[tile], 1);
    prev = __shfl(prev, 0, 64);
    if (prev != a.S - 1) return;
    __threadfence();
    if (lane == 0) __hip_atomic_store(&a.counters[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    f32x16_t tot[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int v = 0; v < 16; ++v) tot[n][v] = 0.f;
    for (int s = 0; s < a.S; ++s) {
      if (s == split) {
#pragma unroll
        for (int n = 0; n < NT; ++n) tot[n] += acc[n];
      } else {
        const float* Ps = P + (size_t)s * kTileFloats;
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            tot[n][v] += __hip_atomic_load(Ps + (n * 16 + v) * 64 + lane, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = tot[n];
  }

  // store: lane -> output row row0 + lr; accumulator v -> token 8*(v/4) + 4*kg + v%4
  if (row0 + lr < pd.d_out) {
    bf16_t* y = static_cast<bf16_t*>(pd.y);
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = n * 32 + 8 * (v >> 2) + 4 * kg + (v & 3);
        if (t < a.T) y[(size_t)t * pd.ld_y + row0 + lr] = f32_to_bf16(acc[n][v]);
      }
  }
}

// ============================================================================
// Stage 2, prefill: 128 tokens x 128 rows per workgroup, LDS-tiled MFMA GEMM.
// ============================================================================
constexpr int kPB = 128;       // tile edge (tokens and rows)
constexpr int kPK = 32;        // K per LDS stage
constexpr int kPLd = kPK + 8;  // padded LDS row (elements)

__device__ __forceinline__ int token_at(const SgmmArgs& a, int i) {
  // top-1: walk tokens in segment order so a tile meets few adapters
  return (a.k == 1) ? a.pair_perm[i] : i;
}

__global__ __launch_bounds__(256) void prefill_bf16(SgmmArgs a, int n_tok_tiles) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][kPB][kPLd];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][kPB][kPLd];
  __shared__ uint32_t amask[kMaxEWords];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tt = blockIdx.x % n_tok_tiles, tile = blockIdx.x / n_tok_tiles;
  const int proj = proj_of_tile(a, tile);
  const ProjDesc pd = proj_at(a, proj);
  const int row0 = (tile - pd.tile_begin) * kPB;
  const int i0 = tt * kPB;  // position in token order
  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  const bf16_t* W0 = static_cast<const bf16_t*>(pd.W0);

  // global -> LDS: 512 16-byte chunks per operand tile, two per thread each
  const bf16_t* gA[2];
  const bf16_t* gB[2];
  int lrow[2], lk[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + i * 256;
    lrow[i] = q >> 2;
    lk[i] = (q & 3) * 8;
    const int pos = min(i0 + lrow[i], a.T - 1);
    gA[i] = x + (size_t)token_at(a, pos) * a.ld_x;
    gB[i] = W0 + (size_t)min(row0 + lrow[i], pd.d_out - 1) * a.d_in;
  }
  const int nk = (a.d_in + kPK - 1) / kPK;
  uint4 ra[2], rb[2];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int k = kt * kPK + lk[i];
      const bool ok = k < a.d_in;
      const int kc = min(k, a.d_in - 8);
      ra[i] = sel4(ok, ld16(gA[i] + kc));
      rb[i] = sel4(ok, ld16_stream(gB[i] + kc));
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *reinterpret_cast<uint4*>(&As[buf][lrow[i]][lk[i]]) = ra[i];
      *reinterpret_cast<uint4*>(&Bs[buf][lrow[i]][lk[i]]) = rb[i];
    }
  };

  const int wm = wave & 1, wn = wave >> 1;  // wave tile: tokens wm*64.., rows wn*64..
  const int lr = lane & 31, kg = lane >> 5;
  f32x16_t acc[2][2];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[f][g][v] = 0.f;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < kPK; kk += 16) {
      uint4 af[2], bfr[2];
#pragma unroll
      for (int f = 0; f < 2; ++f)
        af[f] = *reinterpret_cast<const uint4*>(&As[cur][wm * 64 + f * 32 + lr][kk + kg * 8]);
#pragma unroll
      for (int g = 0; g < 2; ++g)
        bfr[g] = *reinterpret_cast<const uint4*>(&Bs[cur][wn * 64 + g * 32 + lr][kk + kg * 8]);
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int g = 0; g < 2; ++g) acc[f][g] = mfma32(af[f], bfr[g], acc[f][g]);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // expand: the adapters met by this tile's tokens
  if (a.k > 0) {
    const int nw = (a.E + 31) >> 5;
    for (int q = tid; q < nw; q += 256) amask[q] = 0u;
    __syncthreads();
    for (int q = tid; q < kPB * a.k; q += 256) {
      const int pos = i0 + q / a.k;
      if (pos < a.T) {
        const int e = a.topk_idx[token_at(a, pos) * a.k + q % a.k];
        if ((unsigned)e < (unsigned)a.E) atomicOr(&amask[e >> 5], 1u << (e & 31));
      }
    }
    __syncthreads();
    const bf16_t* Bm = static_cast<const bf16_t*>(pd.B);
    const float* ub = a.u + (size_t)proj * a.T * a.k * a.r;
    int tok[2];
    bool tok_ok[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int pos = i0 + wm * 64 + f * 32 + lr;
      tok_ok[f] = pos < a.T;
      tok[f] = token_at(a, min(pos, a.T - 1));
    }
    for (int w = 0; w < nw; ++w) {
      uint32_t bits = amask[w];
      while (bits) {
        const int e = w * 32 + __ffs(bits) - 1;
        bits &= bits - 1;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int js = tok_ok[f] ? match_slot(a.topk_idx, tok[f], a.k, e) : -1;
          if (__ballot(js >= 0) == 0) continue;
          for (int c0 = 0; c0 < a.r; c0 += 16) {
            const int c = c0 + kg * 8;
            const bool cok = c < a.r;
            uint4 hi, lo;
            u_operand(ub, a.r, tok[f] * a.k + max(js, 0), min(c, a.r - 8), cok && js >= 0, hi, lo);
#pragma unroll
            for (int g = 0; g < 2; ++g) {
              const int row = min(row0 + wn * 64 + g * 32 + lr, pd.d_out - 1);
              const uint4 bo = sel4(cok, ld16(Bm + ((size_t)e * pd.d_out + row) * a.r + min(c, a.r - 8)));
              acc[f][g] = mfma32(hi, bo, acc[f][g]);
              acc[f][g] = mfma32(lo, bo, acc[f][g]);
            }
          }
        }
      }
    }
  }

  bf16_t* y = static_cast<bf16_t*>(pd.y);
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int row = row0 + wn * 64 + g * 32 + lr;
    if (row >= pd.d_out) continue;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int pos = i0 + wm * 64 + f * 32 + 8 * (v >> 2) + 4 * kg + (v & 3);
        if (pos < a.T) y[(size_t)token_at(a, pos) * pd.ld_y + row] = f32_to_bf16(acc[f][g][v]);
      }
  }
}

// ============================================================================
// fp32 inputs: VALU kernels.
// ============================================================================

// u[pair] = g * A_e x[t]: one wave per (projection, pair).
__global__ __launch_bounds__(256) void shrink_f32(SgmmArgs a) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int npairs = a.T * a.k;
  if (gw >= a.n_proj * npairs) return;
  const int proj = gw / npairs, p = gw % npairs;
  const ProjDesc pd = proj_at(a, proj);
  const int t = p / a.k, e = a.topk_idx[p];
  if ((unsigned)e >= (unsigned)a.E) return;
  const float* xr = static_cast<const float*>(a.x) + (size_t)t * a.ld_x;
  const float* Ae = static_cast<const float*>(pd.A) + (size_t)e * a.r * a.d_in;
  float* u_out = a.u + ((size_t)proj * npairs + p) * a.r;
  const float g = a.topk_gate[p];
  for (int c = 0; c < a.r; ++c) {
    float s = 0.f;
    for (int i = lane; i < a.d_in; i += 64) s = fmaf(Ae[(size_t)c * a.d_in + i], xr[i], s);
    s = wave_sum_f32(s);
    if (lane == 0) u_out[c] = g * s;
  }
}

// 64 rows x 64 tokens per workgroup; thread = 4 rows (strided by 16) x 4 tokens.
__global__ __launch_bounds__(256) void base_expand_f32(SgmmArgs a, int n_tok_tiles) {
  __shared__ float xs[16][64 + 1];
  __shared__ float wsm[16][64 + 1];
  const int tid = threadIdx.x;
  const int tt = blockIdx.x % n_tok_tiles, tile = blockIdx.x / n_tok_tiles;
  const int proj = proj_of_tile(a, tile);
  const ProjDesc pd = proj_at(a, proj);
  const int row0 = (tile - pd.tile_begin) * 64, t0 = tt * 64;
  const float* x = static_cast<const float*>(a.x);
  const float* W0 = static_cast<const float*>(pd.W0);
  const int tr = tid & 15, tc = tid >> 4;  // rows tr + 16 i, tokens tc*4 + j
  float acc[4][4] = {};
  for (int k0 = 0; k0 < a.d_in; k0 += 16) {
    __syncthreads();
    for (int q = tid; q < 16 * 64; q += 256) {
      const int kk = q & 15, m = q >> 4;
      const int k = k0 + kk;
      const int t = t0 + m, rw = row0 + m;
      xs[kk][m] = (k < a.d_in && t < a.T) ? x[(size_t)t * a.ld_x + k] : 0.f;
      wsm[kk][m] = (k < a.d_in && rw < pd.d_out) ? W0[(size_t)rw * a.d_in + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float wv[4], xv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[i] = wsm[kk][tr + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) xv[j] = xs[kk][tc * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(wv[i], xv[j], acc[i][j]);
    }
  }
  const float* Bm = static_cast<const float*>(pd.B);
  const float* ub = a.u + (size_t)proj * a.T * a.k * a.r;
  float* y = static_cast<float*>(pd.y);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + tc * 4 + j;
    if (t >= a.T) continue;
    for (int s = 0; s < a.k; ++s) {
      const int e = a.topk_idx[t * a.k + s];
      if ((unsigned)e >= (unsigned)a.E) continue;
      const float* up = ub + (size_t)(t * a.k + s) * a.r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rw = row0 + tr + 16 * i;
        if (rw >= pd.d_out) continue;
        const float* br = Bm + ((size_t)e * pd.d_out + rw) * a.r;
        float d = 0.f;
        for (int c = 0; c < a.r; ++c) d = fmaf(br[c], up[c], d);
        acc[i][j] += d;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rw = row0 + tr + 16 * i;
      if (rw < pd.d_out) y[(size_t)t * pd.ld_y + rw] = acc[i][j];
    }
  }
}

template <int MT>
hipError_t launch_shrink_bf16(const SgmmArgs& a, bool big, hipStream_t s) {
  const int npairs = a.T * a.k;
  if (!big) {
    constexpr int NCT = 1, W = 16;
    const int units = a.E + (npairs + 16 * NCT - 1) / (16 * NCT);
    shrink_bf16<MT, NCT, W, 2><<<a.n_proj * units, W * 64, 0, s>>>(a, units);
  } else {
    constexpr int NCT = 4, W = 4;
    const int units = a.E + (npairs + 16 * NCT - 1) / (16 * NCT);
    shrink_bf16<MT, NCT, W, (MT >= 4 ? 1 : 2)><<<a.n_proj * units, W * 64, 0, s>>>(a, units);
  }
  return hipGetLastError();
}

hipError_t launch_shrink(const SgmmArgs& a, bool big, hipStream_t s) {
  switch ((a.r + 15) / 16) {
    case 1: return launch_shrink_bf16<1>(a, big, s);
    case 2: return launch_shrink_bf16<2>(a, big, s);
    case 4: return launch_shrink_bf16<4>(a, big, s);
    default: return launch_shrink_bf16<8>(a, big, s);
  }
}

}  // namespace

static constexpr size_t kCounterBytes = 65536;
static constexpr int kMaxCounters = (int)(kCounterBytes / sizeof(int));

static int decode_nt(int T) { return T <= 32 ? 1 : T <= 64 ? 2 : T <= 128 ? 4 : 8; }

SgmmPlan plan_sgmm(Dtype dt, int n_proj, const int* d_out, int T, int d_in, int E, int r, int k, int n_cu) {
  SgmmPlan p{};
  p.path = (dt == kF32) ? 0 : (T <= 256 ? 1 : 2);
  p.tile_rows = p.path == 0 ? 64 : p.path == 1 ? 32 : kPB;
  p.n_tiles = 0;
  for (int i = 0; i < n_proj; ++i) p.n_tiles += (d_out[i] + p.tile_rows - 1) / p.tile_rows;
  p.S = 1;
  p.t_pad = 0;
  auto align = [](size_t v) { return (v + 255) & ~(size_t)255; };
  // the arrival counters live in a fixed region at the start of every
  // workspace that no other data ever uses, so calls of any shape can share one
  // workspace and the counters stay zero between calls
  p.off_counters = 0;
  size_t off = kCounterBytes;
  if (p.path == 1) {
    const int nt = decode_nt(T);
    p.t_pad = 32 * nt;
    const int nsteps = (d_in + 15) / 16;
    const int s_cap = T <= 64 ? 8 : T <= 128 ? 4 : 2;
    int S = (n_cu + p.n_tiles - 1) / p.n_tiles;
    S = std::max(1, std::min(S, std::min(s_cap, nsteps / 16)));
    if (p.n_tiles > kMaxCounters) S = 1;  // no arrival counters beyond the reserved region
    p.S = S;
  }
  p.off_u = off;
  off = align(off + (size_t)n_proj * T * k * r * sizeof(float));
  p.off_partial = off;
  if (p.path == 1 && p.S > 1) off = align(off + (size_t)p.n_tiles * p.S * p.t_pad * 32 * sizeof(float));
  p.bytes = off;
  return p;
}

size_t sgmm_workspace_upper_bound(Dtype dt, int n_proj, int T, int d_in, long long sum_d_out, int E, int r,
                                  int k) {
  // largest S the planner can pick, tiles rounded up per projection
  auto align = [](size_t v) { return (v + 255) & ~(size_t)255; };
  size_t b = kCounterBytes;
  b = align(b + (size_t)n_proj * T * k * r * sizeof(float));
  if (dt == kBF16 && T <= 256) {
    const int s_cap = T <= 64 ? 8 : T <= 128 ? 4 : 2;
    b = align(b + (size_t)(sum_d_out / 32 + n_proj) * s_cap * 32 * decode_nt(T) * 32 * sizeof(float));
  }
  return b;
}

hipError_t launch_sgmm(const SgmmArgs& a, const SgmmPlan& plan, Dtype dt, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  hipError_t err;
  if (plan.path == 0) {
    if (a.k > 0) {
      const int waves = a.n_proj * a.T * a.k;
      shrink_f32<<<(waves + 3) / 4, 256, 0, s>>>(a);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    const int ntt = (a.T + 63) / 64;
    base_expand_f32<<<plan.n_tiles * ntt, 256, 0, s>>>(a, ntt);
    return hipGetLastError();
  }
  if (a.k > 0) {
    if ((err = launch_shrink(a, plan.path == 2, s)) != hipSuccess) return err;
  }
  if (plan.path == 1) {
    const dim3 grid(plan.n_tiles * plan.S);
    switch (decode_nt(a.T)) {
      case 1: decode_bf16<1, 8><<<grid, 256, 0, s>>>(a); break;
      case 2: decode_bf16<2, 6><<<grid, 256, 0, s>>>(a); break;
      case 4: decode_bf16<4, 4><<<grid, 256, 0, s>>>(a); break;
      default: decode_bf16<8, 2><<<grid, 256, 0, s>>>(a); break;
    }
    return hipGetLastError();
  }
  const int ntt = (a.T + kPB - 1) / kPB;
  prefill_bf16<<<plan.n_tiles * ntt, 256, 0, s>>>(a, ntt);
  return hipGetLastError();
}

}  // namespace rp
