// In-place merge of a weighted set of adapters into a backbone weight, and the
// inverse: the AdaFuse page's literal decoding steps 3 and 5 (technical summary
// §2.B: fold the chosen experts into the backbone, run the backbone, unfold
// them again), kept as a measured alternative to the factorised fused path.
//
//   W0[o, i] <- round(W0[o, i] + sign * sum_j w_j sum_c B[e_j, o, c] A[e_j, c, i])
//
// One workgroup per 64 rows x 128 columns of W0: the gated rank columns of the
// selected adapters go through LDS 32 at a time (A as [32][128] fp32, B as
// [64][32] fp32), each thread accumulates 4 rows x 8 columns in fp32 over all
// k*r rank columns in (adapter, rank) order, then adds them to W0 in fp32 and
// rounds the sum to W0's type.  Both W0 storage orders are supported.
#include "sgmm_common.h"

namespace rp {
namespace {

constexpr int kMRows = 64;
constexpr int kMCols = 128;
constexpr int kMRank = 32;  // rank columns per LDS stage

template <typename Tin>
struct MergeIO;
template <>
struct MergeIO<bf16_t> {
  static __device__ __forceinline__ void load8(const bf16_t* p, float (&v)[8]) {
    const uint4 q = ld16(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store8(bf16_t* p, const float (&v)[8]) {
    uint4 q;
    q.x = f32x2_to_bf16x2(v[0], v[1]);
    q.y = f32x2_to_bf16x2(v[2], v[3]);
    q.z = f32x2_to_bf16x2(v[4], v[5]);
    q.w = f32x2_to_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = q;
  }
  static __device__ __forceinline__ float one(const bf16_t* p) { return bf16_to_f32(*p); }
};
template <>
struct MergeIO<float> {
  static __device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  static __device__ __forceinline__ float one(const float* p) { return *p; }
};

// Element offset of W0[o][i .. i+7] (i a multiple of 8) in the given order.
__device__ __forceinline__ size_t w0_offset(const MergeArgs& m, int o, int i) {
  if (!m.tiled) return (size_t)o * m.d_in + i;
  const int rb = o >> 4, cb = i >> 5;
  const int q = (o & 15) + 16 * ((i & 31) >> 3);
  return w0_block_offset(rb, cb, m.d_out >> 4, m.d_in >> 5) + (size_t)q * 8;
}

template <typename Tin>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs m, int n_col_tiles) {
  using IO = MergeIO<Tin>;
  __shared__ float sA[kMRank][kMCols];
  __shared__ float sB[kMRows][kMRank + 1];
  const int tid = threadIdx.x;
  const int ct = blockIdx.x % n_col_tiles, rt = blockIdx.x / n_col_tiles;
  const int o0 = rt * kMRows, i0 = ct * kMCols;
  const int cg = tid & 15, rg = tid >> 4;  // columns i0 + 8*cg .. +7; rows o0 + rg + 16*q
  const Tin* A = static_cast<const Tin*>(m.A);
  const Tin* B = static_cast<const Tin*>(m.B);
  float acc[4][8];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[q][c] = 0.f;
  const int KR = m.n_sel * m.r;  // concatenated rank columns (adapter-major)
  for (int k0 = 0; k0 < KR; k0 += kMRank) {
    __syncthreads();
    // A rows k0 .. k0+31 (scaled by their adapter's weight) over the tile's columns
    for (int f = tid; f < kMRank * (kMCols / 8); f += 256) {
      const int kr = f / (kMCols / 8), c8 = (f % (kMCols / 8)) * 8;
      const int kk = k0 + kr, col = i0 + c8;
      float v[8];
      if (kk < KR && col < m.d_in) {
        const int j = kk / m.r, c = kk % m.r;
        const int e = m.sel[j];
        const float w = m.weights[j];
        if ((unsigned)e < (unsigned)m.E) {  // an index outside [0, E) adds nothing
          IO::load8(A + ((size_t)e * m.r + c) * m.d_in + col, v);
#pragma unroll
          for (int z = 0; z < 8; ++z) v[z] *= w;
        } else {
#pragma unroll
          for (int z = 0; z < 8; ++z) v[z] = 0.f;
        }
      } else {
#pragma unroll
        for (int z = 0; z < 8; ++z) v[z] = 0.f;
      }
#pragma unroll
      for (int z = 0; z < 8; ++z) sA[kr][c8 + z] = v[z];
    }
    // B rows o0 .. o0+63, rank columns k0 .. k0+31
    for (int f = tid; f < kMRows * kMRank; f += 256) {
      const int ro = f / kMRank, kr = f % kMRank;
      const int kk = k0 + kr, o = o0 + ro;
      float v = 0.f;
      if (kk < KR && o < m.d_out) {
        const int j = kk / m.r, c = kk % m.r;
        const int e = m.sel[j];
        if ((unsigned)e < (unsigned)m.E) v = IO::one(B + ((size_t)e * m.d_out + o) * m.r + c);
      }
      sB[ro][kr] = v;
    }
    __syncthreads();
#pragma unroll 4
    for (int kr = 0; kr < kMRank; ++kr) {
      float a8[8];
#pragma unroll
      for (int z = 0; z < 8; ++z) a8[z] = sA[kr][cg * 8 + z];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float b = sB[rg + 16 * q][kr];
#pragma unroll
        for (int z = 0; z < 8; ++z) acc[q][z] = fmaf(b, a8[z], acc[q][z]);
      }
    }
  }
  Tin* W0 = static_cast<Tin*>(m.W0);
  const int col = i0 + cg * 8;
  if (col >= m.d_in) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int o = o0 + rg + 16 * q;
    if (o >= m.d_out) continue;
    Tin* p = W0 + w0_offset(m, o, col);
    float v[8];
    IO::load8(p, v);
#pragma unroll
    for (int z = 0; z < 8; ++z) v[z] += m.sign * acc[q][z];
    IO::store8(p, v);
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& m, Dtype dt, hipStream_t s) {
  const int nct = (m.d_in + kMCols - 1) / kMCols, nrt = (m.d_out + kMRows - 1) / kMRows;
  if (dt == kBF16)
    merge_kernel<bf16_t><<<nct * nrt, 256, 0, s>>>(m, nct);
  else
    merge_kernel<float><<<nct * nrt, 256, 0, s>>>(m, nct);
  return hipGetLastError();
}

}  // namespace rp
