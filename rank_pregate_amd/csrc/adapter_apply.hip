// One adapter's gated low-rank delta, added in place to the outputs of the
// tokens in its segment (the unfused form: a base projection launch followed
// by one launch per adapter).  This is the "simple fusion" that the AdaFuse
// page's ablation (technical summary §4) sets against SGMM, and the per-adapter
// kernel fragmentation its problem statement (§1) blames for dynamic-adapter
// latency; it serves as a measured baseline next to the fused kernels.
//
//   y[t] += g[t,j] * B_e (A_e x[t])   for every pair (t, j) of segment e
//
// One workgroup per 256 output rows of one projection.  The segment's pairs go
// in chunks of 16: the four waves compute the chunk's rank-r intermediates
// (one pair per wave at a time, lanes across d_in and eight rank rows at once,
// fp32, a fixed butterfly over lanes) into LDS, then each thread adds the gated deltas of its row for
// the chunk's pairs in segment order (a token named twice gets both terms, one
// after the other) with a read-modify-write of y (one rounding per pair).
#include "sgmm_common.h"

namespace rp {
namespace {

constexpr int kApplyRows = 256;   // output rows per workgroup (one per thread)
constexpr int kApplyPairs = 16;   // pairs per chunk
constexpr int kApplyMaxR = 128;
constexpr int kApplyRankGroup = 8;  // rank rows a lane sums at once (r is a multiple of 8)

template <typename Tin>
struct Elem;
template <>
struct Elem<bf16_t> {
  static constexpr int kVec = 8;  // elements per 16-byte load
  static __device__ __forceinline__ void load(const bf16_t* p, float (&v)[8]) {
    const uint4 q = ld16(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void load8(const bf16_t* p, float (&v)[8]) { load(p, v); }
  static __device__ __forceinline__ float get(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void put(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};
template <>
struct Elem<float> {
  static constexpr int kVec = 4;
  static __device__ __forceinline__ void load(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  }
  static __device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ float get(const float* p) { return *p; }
  static __device__ __forceinline__ void put(float* p, float v) { *p = v; }
};

template <typename Tin>
__global__ __launch_bounds__(256) void adapter_apply_kernel(SgmmArgs a, int e) {
  using El = Elem<Tin>;
  constexpr int V = El::kVec;
  __shared__ float su[kApplyPairs][kApplyMaxR];
  __shared__ int s_t[kApplyPairs];
  __shared__ float s_g[kApplyPairs];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x;
  const int proj = proj_of_tile(a, tile);
  const ProjDesc pd = proj_at(a, proj);
  const int row = (tile - pd.tile_begin) * kApplyRows + tid;
  const Tin* x = static_cast<const Tin*>(a.x);
  const Tin* Ae = static_cast<const Tin*>(pd.A) + (size_t)e * a.r * a.d_in;
  const Tin* Br = static_cast<const Tin*>(pd.B) + ((size_t)e * pd.d_out + min(row, pd.d_out - 1)) * a.r;
  Tin* y = static_cast<Tin*>(pd.y);
  const int s0 = a.seg_offsets[e], s1 = a.seg_offsets[e + 1];
  for (int c0 = s0; c0 < s1; c0 += kApplyPairs) {
    const int n = min(kApplyPairs, s1 - c0);
    if (tid < n) {
      const int p = a.pair_perm[c0 + tid];
      s_t[tid] = p / a.k;
      s_g[tid] = a.topk_gate[p];
    }
    __syncthreads();
    // rank-r intermediates of the chunk's pairs: wave w takes pairs w, w+4, ..;
    // a lane sums its columns (lane*V + 64*V*i) for 8 rank rows at once, so the
    // loads of a whole rank group are in flight together, then a butterfly per
    // rank row combines the lanes
    for (int q = wave; q < n; q += 4) {
      const Tin* xr = x + (size_t)s_t[q] * a.ld_x;
      for (int rc = 0; rc < a.r; rc += kApplyRankGroup) {
        float s[kApplyRankGroup];
#pragma unroll
        for (int c = 0; c < kApplyRankGroup; ++c) s[c] = 0.f;
        for (int i = lane * V; i < a.d_in; i += 64 * V) {
          float xv[8];
          El::load(xr + i, xv);
#pragma unroll
          for (int c = 0; c < kApplyRankGroup; ++c) {
            float av[8];
            El::load(Ae + (size_t)(rc + c) * a.d_in + i, av);
#pragma unroll
            for (int j = 0; j < V; ++j) s[c] = fmaf(av[j], xv[j], s[c]);
          }
        }
#pragma unroll
        for (int c = 0; c < kApplyRankGroup; ++c) {
          const float v = wave_sum_f32(s[c]);
          if (lane == 0) su[q][rc + c] = v;
        }
      }
    }
    __syncthreads();
    if (row < pd.d_out) {
      for (int q = 0; q < n; ++q) {
        float d = 0.f;
        for (int c = 0; c < a.r; c += 8) {
          float bv[8];
          El::load8(Br + c, bv);
#pragma unroll
          for (int j = 0; j < 8; ++j) d = fmaf(bv[j], su[q][c + j], d);
        }
        Tin* yp = y + (size_t)s_t[q] * pd.ld_y + row;
        El::put(yp, El::get(yp) + s_g[q] * d);
      }
    }
    __syncthreads();  // s_t, s_g and su are rewritten by the next chunk
  }
}

}  // namespace

int adapter_apply_tile_rows() { return kApplyRows; }

hipError_t launch_adapter_apply(const SgmmArgs& a, int e, Dtype dt, hipStream_t s) {
  if (a.T == 0 || a.k == 0) return hipSuccess;
  if (dt == kBF16)
    adapter_apply_kernel<bf16_t><<<a.n_tiles, 256, 0, s>>>(a, e);
  else
    adapter_apply_kernel<float><<<a.n_tiles, 256, 0, s>>>(a, e);
  return hipGetLastError();
}

}  // namespace rp
