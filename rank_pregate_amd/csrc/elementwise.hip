// The base model's own per-token operations between the adapted projections
// of a Llama-style decoder layer (AdaFuse technical summary §2.B decoding step
// 4 runs the base model; §4 measures 7B Llama-family models): RMSNorm and the
// gated MLP activation silu(g) * u.  Both are small next to the projections;
// the activation also runs fused into the (gate, up) group's decode launch.
#include "device_common.h"
#include "kernels.h"

namespace rp {
namespace {

constexpr int kNormThreads = 256;

template <typename T>
struct Io;
template <>
struct Io<bf16_t> {
  static constexpr int kVec = 8;
  static __device__ __forceinline__ void load(const bf16_t* p, float (&v)[8]) {
    const uint4 q = ld16(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float (&v)[8]) {
    uint4 q;
    q.x = f32x2_to_bf16x2(v[0], v[1]);
    q.y = f32x2_to_bf16x2(v[2], v[3]);
    q.z = f32x2_to_bf16x2(v[4], v[5]);
    q.w = f32x2_to_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = q;
  }
};
template <>
struct Io<float> {
  static constexpr int kVec = 4;
  static __device__ __forceinline__ void load(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  }
  static __device__ __forceinline__ void store(float* p, const float (&v)[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// One workgroup per token row.  Thread i sums the squares of its vectors
// i, i + 256, ... in order; the 256 partial sums are combined by a fixed wave
// butterfly and then in wave order, so the result does not depend on timing.
template <typename T>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const T* x, int d, int ld_x, const T* gamma, float eps,
                                                               T* y, int ld_y) {
  using IO = Io<T>;
  constexpr int V = IO::kVec;
  __shared__ float s_part[kNormThreads / 64];
  const int t = blockIdx.x, tid = threadIdx.x;
  const T* xr = x + (size_t)t * ld_x;
  T* yr = y + (size_t)t * ld_y;
  float ss = 0.f;
  for (int i = tid * V; i < d; i += kNormThreads * V) {
    float v[8];
    IO::load(xr + i, v);
#pragma unroll
    for (int j = 0; j < V; ++j) ss = fmaf(v[j], v[j], ss);
  }
  ss = wave_sum_f32(ss);
  if ((tid & 63) == 0) s_part[tid >> 6] = ss;
  __syncthreads();
  float tot = s_part[0];
#pragma unroll
  for (int w = 1; w < kNormThreads / 64; ++w) tot += s_part[w];
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
  // every thread has read s_part before any output is written (y may be x)
  for (int i = tid * V; i < d; i += kNormThreads * V) {
    float v[8], gm[8];
    IO::load(xr + i, v);
    IO::load(gamma + i, gm);
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] = v[j] * inv * gm[j];
    IO::store(yr + i, v);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void silu_mul_kernel(const T* g, int ld_g, const T* u, int ld_u, int T_, int d, T* m,
                                                       int ld_m) {
  using IO = Io<T>;
  constexpr int V = IO::kVec;
  const int per_row = d / V;
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)T_ * per_row) return;
  const int t = (int)(i / per_row), c = (int)(i % per_row) * V;
  float gv[8], uv[8];
  IO::load(g + (size_t)t * ld_g + c, gv);
  IO::load(u + (size_t)t * ld_u + c, uv);
#pragma unroll
  for (int j = 0; j < V; ++j) gv[j] = silu_mul_f32(gv[j], uv[j]);
  IO::store(m + (size_t)t * ld_m + c, gv);
}

}  // namespace

hipError_t launch_rmsnorm(const void* x, int T, int d, int ld_x, const void* gamma, float eps, void* y, int ld_y,
                          Dtype dt, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dt == kBF16)
    rmsnorm_kernel<bf16_t><<<T, kNormThreads, 0, s>>>(static_cast<const bf16_t*>(x), d, ld_x,
                                                      static_cast<const bf16_t*>(gamma), eps, static_cast<bf16_t*>(y),
                                                      ld_y);
  else
    rmsnorm_kernel<float><<<T, kNormThreads, 0, s>>>(static_cast<const float*>(x), d, ld_x,
                                                     static_cast<const float*>(gamma), eps, static_cast<float*>(y),
                                                     ld_y);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const void* g, int ld_g, const void* u, int ld_u, int T, int d, void* m, int ld_m,
                           Dtype dt, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int V = dt == kBF16 ? 8 : 4;
  const long long n = (long long)T * (d / V);
  const int blocks = (int)((n + 255) / 256);
  if (dt == kBF16)
    silu_mul_kernel<bf16_t><<<blocks, 256, 0, s>>>(static_cast<const bf16_t*>(g), ld_g, static_cast<const bf16_t*>(u),
                                                   ld_u, T, d, static_cast<bf16_t*>(m), ld_m);
  else
    silu_mul_kernel<float><<<blocks, 256, 0, s>>>(static_cast<const float*>(g), ld_g, static_cast<const float*>(u),
                                                  ld_u, T, d, static_cast<float*>(m), ld_m);
  return hipGetLastError();
}

}  // namespace rp
