// Token-level pre-gating (AdaFuse, technical summary §2.A; §2.B decoding steps
// 1-2): one linear router scores each token once, the k best adapters are
// kept (ties to the lower index) and weighted by a softmax over the k chosen
// logits.
//
// One workgroup scores TT tokens against all E router columns.  Threads are
// laid out as (block of 8 columns, k-slice).  A thread walks its k-slice in
// ascending k, reading 8 consecutive router columns per row with one 16-byte
// load and 8 consecutive activations per token with another, and keeps one
// fp32 sum per (token, column).  The slices are then added with a fixed
// butterfly inside each wave and in wave order across waves.  Every logit is
// therefore summed in the same order, so two equal router columns give
// bit-equal logits and the tie rule holds exactly.  Top-k runs per
// token on one wave with shuffles.
#include "device_common.h"
#include "kernels.h"

namespace rp {
namespace {

constexpr int kThreads = 256;
constexpr int kCB = 8;  // router columns per thread

template <typename Tin>
struct Vec8;
template <>
struct Vec8<bf16_t> {
  // 8 consecutive bf16 -> fp32
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

// (value, index) ordering of the router: larger logit first, lower index on ties.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

template <typename Tin, int TT>
__global__ __launch_bounds__(kThreads) void pregate_kernel(PregateArgs a, int NCBp, int slice, bool vec_cols) {
  extern __shared__ float smem[];  // red[KR][TT][E] then lg[TT][E]
  const int tid = threadIdx.x, lane = tid & 63;
  const int t0 = blockIdx.x * TT;
  const int nt = min(TT, a.T - t0);
  const int E = a.E;
  const Tin* x = static_cast<const Tin*>(a.x);
  const Tin* Wg = static_cast<const Tin*>(a.Wg);
  const int ncb = (E + kCB - 1) / kCB;
  const int cb = tid % NCBp, ks = tid / NCBp;
  // lanes of one wave that share a column block (L of them) are summed with a
  // butterfly; the KR partial sums left per column go through LDS
  const int L = NCBp >= 64 ? 1 : 64 / NCBp;
  const int KR = (kThreads / NCBp) / L;
  float* red = smem;
  float* lg = smem + (size_t)KR * TT * E;

  float acc[TT][kCB];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int c = 0; c < kCB; ++c) acc[t][c] = 0.f;
  const int c0 = cb * kCB;
  if (cb < ncb) {
    const Tin* xr[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) xr[t] = x + (size_t)(t0 + min(t, nt - 1)) * a.ld_x;
    const int kb = ks * slice, ke = min(a.d_in, kb + slice);
    const int ke8 = kb + max(0, ke - kb) / 8 * 8;  // full groups of 8; fp32 rows may end in a group of 4
    for (int k0 = kb; k0 < ke8; k0 += 8) {
      float xv[TT][8];
#pragma unroll
      for (int t = 0; t < TT; ++t) Vec8<Tin>::load(xr[t] + k0, xv[t]);
      float wv[8][kCB];
      if (vec_cols && c0 + kCB <= E) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) Vec8<Tin>::load(Wg + (size_t)(k0 + kk) * E + c0, wv[kk]);
      } else {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
#pragma unroll
          for (int c = 0; c < kCB; ++c)
            wv[kk][c] = (c0 + c < E) ? Vec8<Tin>::one(Wg + (size_t)(k0 + kk) * E + c0 + c) : 0.f;
      }
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
          for (int c = 0; c < kCB; ++c) acc[t][c] = fmaf(xv[t][kk], wv[kk][c], acc[t][c]);
    }
    for (int k = ke8; k < ke; ++k) {
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const float xs = Vec8<Tin>::one(xr[t] + k);
#pragma unroll
        for (int c = 0; c < kCB; ++c)
          if (c0 + c < E) acc[t][c] = fmaf(xs, Vec8<Tin>::one(Wg + (size_t)k * E + c0 + c), acc[t][c]);
      }
    }
  }
  // butterfly over the L lanes of this wave that hold the same columns
  for (int o = NCBp; o < 64; o <<= 1) {
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int c = 0; c < kCB; ++c) acc[t][c] += __shfl_xor(acc[t][c], o, 64);
  }
  if (cb < ncb && (lane / NCBp) % L == 0) {
    const int kr = ks / L;
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int c = 0; c < kCB; ++c)
        if (c0 + c < E) red[((size_t)kr * TT + t) * E + c0 + c] = acc[t][c];
  }
  __syncthreads();
  // the remaining partial sums, in order
  for (int q = tid; q < TT * E; q += kThreads) {
    float s = 0.f;
    for (int j = 0; j < KR; ++j) s += red[(size_t)j * TT * E + q];
    lg[q] = s;
  }
  __syncthreads();

  if (a.logits) {
    for (int q = tid; q < nt * E; q += kThreads) a.logits[(size_t)t0 * E + q] = lg[q];
  }

  // top-k per token: wave w handles tokens w, w+4, ...
  const int wave = tid >> 6;
  for (int tt = wave; tt < nt; tt += kThreads / 64) {
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
          if (bi == 0x7fffffff || better(v, e, bv, bi)) { bv = v; bi = e; }
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (oi != 0x7fffffff && (bi == 0x7fffffff || better(ov, oi, bv, bi))) { bv = ov; bi = oi; }
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
      a.topk_idx[base + lane] = mine_i;
      a.topk_gate[base + lane] = mine / s;
    }
  }
}

template <typename Tin>
hipError_t launch_t(const PregateArgs& a, hipStream_t s) {
  const int ncb = (a.E + kCB - 1) / kCB;
  int NCBp = 1;
  while (NCBp < ncb) NCBp <<= 1;
  const int KS = kThreads / NCBp;
  const int L = NCBp >= 64 ? 1 : 64 / NCBp;
  const int KR = KS / L;
  const int slice = ((a.d_in + KS - 1) / KS + 7) / 8 * 8;
  const bool vec_cols = (a.E * (int)sizeof(Tin)) % 16 == 0;  // every router row starts 16-byte aligned
  if (a.E <= 64) {
    constexpr int TT = 4;
    const size_t lds = sizeof(float) * ((size_t)KR * TT * a.E + (size_t)TT * a.E);
    pregate_kernel<Tin, TT><<<(a.T + TT - 1) / TT, kThreads, lds, s>>>(a, NCBp, slice, vec_cols);
  } else {
    constexpr int TT = 2;
    const size_t lds = sizeof(float) * ((size_t)KR * TT * a.E + (size_t)TT * a.E);
    pregate_kernel<Tin, TT><<<(a.T + TT - 1) / TT, kThreads, lds, s>>>(a, NCBp, slice, vec_cols);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pregate(const PregateArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  return a.dt == kBF16 ? launch_t<bf16_t>(a, s) : launch_t<float>(a, s);
}

}  // namespace rp
