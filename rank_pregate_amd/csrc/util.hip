// Measurement helpers: an HBM stream-read kernel (achievable read bandwidth)
// and a plain copy kernel (known traffic, for scaling hardware byte counters).
#include "device_common.h"
#include "kernels.h"

namespace rp {
namespace {

constexpr int kThreads = 256;
constexpr int kBlocks = 1024;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* src, size_t n16, float* sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = ld16_stream(src + i), b = ld16_stream(src + i + stride);
    const uint4 c = ld16_stream(src + i + 2 * stride), d = ld16_stream(src + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = ld16_stream(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  acc = (uint32_t)wave_or((int)acc);
  __shared__ uint32_t s[kThreads / 64];
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = (float)(s[0] ^ s[1] ^ s[2] ^ s[3]);
}

__global__ __launch_bounds__(kThreads) void copy_kernel(uint4* dst, const uint4* src, size_t n16) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) dst[i] = ld16_stream(src + i);
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t n_bytes, float* sink, hipStream_t s) {
  stream_read_kernel<<<kBlocks, kThreads, 0, s>>>(static_cast<const uint4*>(src), n_bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_copy(void* dst, const void* src, size_t n_bytes, hipStream_t s) {
  copy_kernel<<<kBlocks, kThreads, 0, s>>>(static_cast<uint4*>(dst), static_cast<const uint4*>(src), n_bytes / 16);
  return hipGetLastError();
}

}  // namespace rp
