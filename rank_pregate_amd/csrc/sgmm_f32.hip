// fp32 inputs: VALU kernels (the reference-precision path).
//   shrink_f32:      u[pair] = g * A_e x[t], one wave per (projection, pair)
//   base_expand_f32: 16 output rows x 32 tokens per workgroup; the four waves
//                    split K in quarters and their partial tiles are added in
//                    wave order, then the adapter deltas B_e u are added per
//                    (token, slot).
// Every fp32 sum over K is blocked: a lane sums 64 columns into a fresh
// partial and adds the partial to its running total, so no rounding chain is
// longer than a few dozen terms even at d_in = 12288 (a single chain over K
// grows the error with the square root of K).  Orders are fixed, so results
// do not depend on timing.
#include "sgmm_common.h"

namespace rp {
namespace {

constexpr int kF32Rows = 16;        // output rows per workgroup (8 per half wave)
constexpr int kF32Tokens = 32;      // tokens per workgroup (lane % 32)
constexpr int kF32Waves = 4;        // waves per workgroup, one K quarter each
constexpr int kF32Block4 = 16;      // 4-column steps per partial sum (64 columns)

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }

__device__ __forceinline__ float dot4(float4 a, float4 b, float s) {
  s = fmaf(a.x, b.x, s);
  s = fmaf(a.y, b.y, s);
  s = fmaf(a.z, b.z, s);
  return fmaf(a.w, b.w, s);
}

// u[pair] = g * A_e x[t]: one wave per (projection, pair).  Lane l sums
// columns 4l + 256i .. +3 over i in blocks of 64 columns, then the 64 lane
// sums are combined by a fixed butterfly.
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
  const int n4 = a.d_in >> 2;
  for (int c = 0; c < a.r; ++c) {
    const float* ar = Ae + (size_t)c * a.d_in;
    float tot = 0.f;
    for (int q0 = lane; q0 < n4; q0 += 64 * kF32Block4) {
      float part = 0.f;
#pragma unroll 4
      for (int i = 0; i < kF32Block4; ++i) {
        const int q = q0 + 64 * i;
        if (q < n4) part = dot4(ld4(ar + 4 * q), ld4(xr + 4 * q), part);
      }
      tot += part;
    }
    tot = wave_sum_f32(tot);
    if (lane == 0) u_out[c] = g * tot;
  }
}

// One workgroup: output rows row0 .. row0+15 of one projection for tokens
// t0 .. t0+31.  Lane l of every wave owns token t0 + l%32 and rows
// row0 + 8*(l/32) .. +7; wave w sums K quarter w (4-column steps
// [n4*w/4, n4*(w+1)/4)) in 64-column partials.  Waves 1..3 hand their tiles
// to wave 0 through LDS, which adds them in wave order, applies the adapters
// and stores.
__global__ __launch_bounds__(256) void base_expand_f32(SgmmArgs a, int n_tok_tiles) {
  __shared__ float red[kF32Waves - 1][8][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tt = blockIdx.x % n_tok_tiles, tile = blockIdx.x / n_tok_tiles;
  const int proj = proj_of_tile(a, tile);
  const ProjDesc pd = proj_at(a, proj);
  const int t = tt * kF32Tokens + (lane & 31);
  const int row0 = (tile - pd.tile_begin) * kF32Rows + 8 * (lane >> 5);
  const bool row_ok = row0 < pd.d_out;  // d_out % 8 == 0: the lane's 8 rows are all in or all out
  const float* xr = static_cast<const float*>(a.x) + (size_t)min(t, a.T - 1) * a.ld_x;
  const float* W0 = static_cast<const float*>(pd.W0) + (size_t)min(row0, pd.d_out - 8) * a.d_in;
  const int n4 = a.d_in >> 2;
  const int qb = (int)((long long)n4 * wave / kF32Waves), qe = (int)((long long)n4 * (wave + 1) / kF32Waves);

  float tot[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) tot[i] = 0.f;
  for (int q0 = qb; q0 < qe; q0 += kF32Block4) {
    float part[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) part[i] = 0.f;
    const int qn = min(kF32Block4, qe - q0);
#pragma unroll 4
    for (int q = 0; q < qn; ++q) {
      const int col = 4 * (q0 + q);
      const float4 xv = ld4(xr + col);
#pragma unroll
      for (int i = 0; i < 8; ++i) part[i] = dot4(ld4(W0 + (size_t)i * a.d_in + col), xv, part[i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) tot[i] += part[i];
  }
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red[wave - 1][i][lane] = tot[i];
  }
  __syncthreads();
  if (wave > 0 || t >= a.T || !row_ok) return;
#pragma unroll
  for (int w = 0; w < kF32Waves - 1; ++w)
#pragma unroll
    for (int i = 0; i < 8; ++i) tot[i] += red[w][i][lane];

  // adapter deltas: per slot, delta = B_e (g u) over the rank, then added
  const float* Bm = static_cast<const float*>(pd.B);
  const float* ub = a.u + (size_t)proj * a.T * a.k * a.r;
  for (int j = 0; j < a.k; ++j) {
    const int e = a.topk_idx[t * a.k + j];
    if ((unsigned)e >= (unsigned)a.E) continue;
    const float* up = ub + (size_t)(t * a.k + j) * a.r;
    const float* br = Bm + ((size_t)e * pd.d_out + row0) * a.r;
    float d[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = 0.f;
    for (int c = 0; c < a.r; c += 4) {
      const float4 uv = ld4(up + c);
#pragma unroll
      for (int i = 0; i < 8; ++i) d[i] = dot4(ld4(br + (size_t)i * a.r + c), uv, d[i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) tot[i] += d[i];
  }
  if (pd.residual) {  // added before the output is stored (the one rounding of fp32 is the last add)
    const float* rr = static_cast<const float*>(pd.residual) + (size_t)t * pd.ld_y + row0;
    const float4 r0 = ld4(rr), r1 = ld4(rr + 4);
    tot[0] += r0.x; tot[1] += r0.y; tot[2] += r0.z; tot[3] += r0.w;
    tot[4] += r1.x; tot[5] += r1.y; tot[6] += r1.z; tot[7] += r1.w;
  }
  float* y = static_cast<float*>(pd.y) + (size_t)t * pd.ld_y + row0;
  *reinterpret_cast<float4*>(y) = make_float4(tot[0], tot[1], tot[2], tot[3]);
  *reinterpret_cast<float4*>(y + 4) = make_float4(tot[4], tot[5], tot[6], tot[7]);
}

}  // namespace

int f32_tile_rows() { return kF32Rows; }

hipError_t launch_f32(const SgmmArgs& a, const SgmmPlan& plan, hipStream_t s) {
  if (a.k > 0) {
    const int waves = a.n_proj * a.T * a.k;
    shrink_f32<<<(waves + 3) / 4, 256, 0, s>>>(a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int ntt = (a.T + kF32Tokens - 1) / kF32Tokens;
  base_expand_f32<<<plan.n_tiles * ntt, 256, 0, s>>>(a, ntt);
  return hipGetLastError();
}

}  // namespace rp
