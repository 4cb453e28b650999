// Prefill-shaped fused SGMM (T > 256 tokens): the base projection is a dense
// GEMM (bf16 MFMA, 128 tokens x 128 rows per workgroup, LDS-tiled), so it is
// bound by matrix throughput rather than HBM.  The adapter deltas (AdaFuse
// technical summary §2.B) are folded in as extra MFMA steps: for every adapter
// the tile's tokens chose, B_e's rows times the gathered rank-r intermediates.
// With top-1 the tokens are visited in segment order, so a tile meets one or
// two adapters.  The intermediates come from a separate shrink launch, one
// workgroup per (projection, chunk of 64 pairs of a segment).
#include "sgmm_common.h"

namespace rp {
namespace {

template <int MTR>
__global__ __launch_bounds__(256) void shrink_bf16(SgmmArgs a, int units_per_proj) {
  __shared__ __attribute__((aligned(16))) float red[MTR * 4 * 4 * 64];
  __shared__ int s_loc[2];
  const int proj = blockIdx.x / units_per_proj, unit = blockIdx.x % units_per_proj;
  if (threadIdx.x < 64) {
    int e, c;
    locate_chunk(a, unit, 64, threadIdx.x, &e, &c);
    if (threadIdx.x == 0) { s_loc[0] = e; s_loc[1] = c; }
  }
  __syncthreads();
  if (s_loc[0] < 0) return;
  shrink_unit<MTR, 4, 4, (MTR >= 4 ? 1 : 2)>(a, proj, s_loc[0], s_loc[1], red);
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
  // A (tokens): chunk q -> token row q/4, columns 8*(q%4).  B (W0 rows):
  // row-major the same; tiled, chunk q is lane q%64 of 16-row block q/64, which
  // holds row 16*(q/64) + (q%64)%16, columns 8*((q%64)/16).
  const bf16_t* gA[2];
  const bf16_t* gB[2];
  int lrow[2], lk[2], brow[2], bk[2], tblk[2];
  const int nkb = a.d_in / 32, n_rb = pd.d_out / 16;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + i * 256;
    lrow[i] = q >> 2;
    lk[i] = (q & 3) * 8;
    const int pos = min(i0 + lrow[i], a.T - 1);
    gA[i] = x + (size_t)token_at(a, pos) * a.ld_x;
    if (pd.tiled) {
      tblk[i] = min(row0 / 16 + q / 64, n_rb - 1);
      brow[i] = (q / 64) * 16 + (q % 64) % 16;
      bk[i] = ((q % 64) / 16) * 8;
      gB[i] = W0 + (q % 64) * 8;
    } else {
      brow[i] = lrow[i];
      bk[i] = lk[i];
      tblk[i] = 0;
      gB[i] = W0 + (size_t)min(row0 + lrow[i], pd.d_out - 1) * a.d_in;
    }
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
      if (pd.tiled)
        rb[i] = ld16(gB[i] + w0_block_offset(tblk[i], min(kt, nkb - 1), n_rb, nkb));  // d_in % 32 == 0: whole blocks
      else
        rb[i] = sel4(k < a.d_in, ld16(gB[i] + min(kt * kPK + lk[i], a.d_in - 8)));
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *reinterpret_cast<uint4*>(&As[buf][lrow[i]][lk[i]]) = ra[i];
      *reinterpret_cast<uint4*>(&Bs[buf][brow[i]][bk[i]]) = rb[i];
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
          const bool mine = tok_ok[f] && chose(a.topk_idx, tok[f], a.k, e);
          if (__ballot(mine) == 0) continue;
          for (int c0 = 0; c0 < a.r; c0 += 16) {
            const int c = c0 + kg * 8;
            const bool cok = c < a.r;
            uint4 hi, lo;
            u_operand(ub, a.topk_idx, a.r, tok[f], a.k, e, min(c, a.r - 8), cok && mine, hi, lo);
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

}  // namespace

hipError_t launch_prefill(const SgmmArgs& a, const SgmmPlan& plan, hipStream_t s) {
  if (a.k > 0) {
    const int units = a.E + (a.T * a.k + 63) / 64;
    const dim3 g(units * a.n_proj);
    switch ((a.r + 15) >> 4) {
      case 1: shrink_bf16<1><<<g, 256, 0, s>>>(a, units); break;
      case 2: shrink_bf16<2><<<g, 256, 0, s>>>(a, units); break;
      case 4: shrink_bf16<4><<<g, 256, 0, s>>>(a, units); break;
      default: shrink_bf16<8><<<g, 256, 0, s>>>(a, units); break;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int ntt = (a.T + kPB - 1) / kPB;
  prefill_bf16<<<plan.n_tiles * ntt, 256, 0, s>>>(a, ntt);
  return hipGetLastError();
}

}  // namespace rp
