// fp32 inputs: plain VALU kernels (the reference-precision path).
//   shrink_f32:      u[pair] = g * A_e x[t], one wave per (projection, pair)
//   base_expand_f32: 64 rows x 64 tokens per workgroup, W0 and x staged in LDS,
//                    then the adapter deltas B_e u added per (token, slot).
#include "sgmm_common.h"

namespace rp {
namespace {

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

}  // namespace

hipError_t launch_f32(const SgmmArgs& a, const SgmmPlan& plan, hipStream_t s) {
  if (a.k > 0) {
    const int waves = a.n_proj * a.T * a.k;
    shrink_f32<<<(waves + 3) / 4, 256, 0, s>>>(a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int ntt = (a.T + 63) / 64;
  base_expand_f32<<<plan.n_tiles * ntt, 256, 0, s>>>(a, ntt);
  return hipGetLastError();
}

}  // namespace rp
