// Token-level pre-gating (AdaFuse, technical summary §2.A; §2.B decoding steps
// 1-2): one linear router scores each token once, the k best adapters are
// kept (ties to the lower index) and weighted by a softmax over the k chosen
// logits.
//
// One workgroup scores TT tokens against all E router columns.  Threads are
// laid out as (column, k-slice); every logit is summed in the same order
// (k-slice by k-slice over the d_in chunks, then a fixed-order sum over the
// slices), so two equal router columns produce bit-equal logits and the tie
// rule holds exactly.  Top-k runs per token on one wave with shuffles.
#include "device_common.h"
#include "kernels.h"

namespace rp {
namespace {

constexpr int kThreads = 256;
constexpr int kTT = 8;      // tokens per workgroup
constexpr int kKC = 512;    // d_in chunk staged in LDS

template <typename Tin>
__device__ __forceinline__ float load_elem(const Tin* p);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_elem<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

// (value, index) ordering of the router: larger logit first, lower index on ties.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

template <typename Tin>
__global__ __launch_bounds__(kThreads) void pregate_kernel(PregateArgs a, int EC, int KS) {
  __shared__ float xs[kTT][kKC];
  __shared__ float red[kThreads * kTT];
  extern __shared__ float lg[];  // [kTT][E] logits of this tile

  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kTT;
  const int nt = min(kTT, a.T - t0);
  const Tin* x = static_cast<const Tin*>(a.x);
  const Tin* Wg = static_cast<const Tin*>(a.Wg);
  const int ec = tid % EC;   // column inside the block
  const int ks = tid / EC;   // k-slice
  const int E = a.E;

  for (int cb = 0; cb < E; cb += EC) {
    const int e = cb + ec;
    const bool col_ok = e < E;
    float acc[kTT];
#pragma unroll
    for (int i = 0; i < kTT; ++i) acc[i] = 0.f;

    for (int k0 = 0; k0 < a.d_in; k0 += kKC) {
      const int kc = min(kKC, a.d_in - k0);
      __syncthreads();
      for (int q = tid; q < kTT * kc; q += kThreads) {
        const int tt = q / kc, kk = q % kc;
        xs[tt][kk] = (tt < nt) ? load_elem<Tin>(x + (size_t)(t0 + tt) * a.ld_x + k0 + kk) : 0.f;
      }
      __syncthreads();
      const int slice = (kc + KS - 1) / KS;
      const int kb = ks * slice, ke = min(kc, kb + slice);
      if (col_ok) {
        const Tin* wp = Wg + (size_t)(k0 + kb) * E + e;
        for (int kk = kb; kk < ke; ++kk, wp += E) {
          const float w = load_elem<Tin>(wp);
#pragma unroll
          for (int tt = 0; tt < kTT; ++tt) acc[tt] = fmaf(xs[tt][kk], w, acc[tt]);
        }
      }
    }
    // fixed-order sum over the k-slices
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) red[(ks * kTT + tt) * EC + ec] = acc[tt];
    __syncthreads();
    for (int q = tid; q < kTT * EC; q += kThreads) {
      const int tt = q / EC, c = q % EC;
      float s = 0.f;
      for (int j = 0; j < KS; ++j) s += red[(j * kTT + tt) * EC + c];
      if (cb + c < E) lg[tt * E + cb + c] = s;
    }
    __syncthreads();
  }

  if (a.logits) {
    for (int q = tid; q < nt * E; q += kThreads) a.logits[(size_t)t0 * E + q] = lg[q];
  }

  // top-k per token: wave w handles tokens w, w+4, ...
  const int lane = tid & 63, wave = tid >> 6;
  for (int tt = wave; tt < nt; tt += kThreads / 64) {
    const float* row = lg + tt * E;
    uint32_t taken = 0;  // bit m: this lane's m-th candidate (e = lane + 64 m) is chosen
    float selv[kMaxK];
    int seli[kMaxK];
    for (int j = 0; j < a.k; ++j) {
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
    if (lane == 0) {
      const size_t base = (size_t)(t0 + tt) * a.k;
      float z[kMaxK];
      float s = 0.f;
      for (int j = 0; j < a.k; ++j) { z[j] = expf(selv[j] - selv[0]); s += z[j]; }
      for (int j = 0; j < a.k; ++j) {
        a.topk_idx[base + j] = seli[j];
        a.topk_gate[base + j] = z[j] / s;
      }
    }
  }
}

}  // namespace

hipError_t launch_pregate(const PregateArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  int EC = 1;
  while (EC < a.E && EC < kThreads) EC <<= 1;
  const int KS = kThreads / EC;
  const dim3 grid((a.T + kTT - 1) / kTT);
  const size_t lds = sizeof(float) * kTT * a.E;
  if (a.dt == kBF16)
    pregate_kernel<bf16_t><<<grid, kThreads, lds, s>>>(a, EC, KS);
  else
    pregate_kernel<float><<<grid, kThreads, lds, s>>>(a, EC, KS);
  return hipGetLastError();
}

}  // namespace rp
