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

// One 16-byte piece per thread: piece o is lane o%64 of block o/64, block
// (rb, cb) = (o/64 / nb, o/64 % nb); lane g holds row 16*rb + g%16, columns
// 32*cb + 8*(g/16) .. +7 of the row-major source, and the block lands where
// w0_block_offset puts it.
__global__ __launch_bounds__(kThreads) void pack_w0_kernel(const uint4* src, uint4* dst, int d_out, int d_in) {
  const size_t n = (size_t)d_out * d_in / 8;
  const int nb = d_in / 32, n_rb = d_out / 16;
  for (size_t o = (size_t)blockIdx.x * kThreads + threadIdx.x; o < n; o += (size_t)gridDim.x * kThreads) {
    const size_t blk = o / 64;
    const int g = (int)(o % 64);
    const int rb = (int)(blk / nb), cb = (int)(blk % nb);
    const size_t row = (size_t)rb * 16 + (g % 16), col = (size_t)cb * 32 + (g / 16) * 8;
    dst[(w0_block_offset(rb, cb, n_rb, nb) + (size_t)g * 8) / 8] = src[(row * d_in + col) / 8];
  }
}

}  // namespace

hipError_t launch_pack_w0(const void* src, void* dst, int d_out, int d_in, hipStream_t s) {
  pack_w0_kernel<<<2048, kThreads, 0, s>>>(static_cast<const uint4*>(src), static_cast<uint4*>(dst), d_out, d_in);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, size_t n_bytes, float* sink, hipStream_t s) {
  stream_read_kernel<<<kBlocks, kThreads, 0, s>>>(static_cast<const uint4*>(src), n_bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_copy(void* dst, const void* src, size_t n_bytes, hipStream_t s) {
  copy_kernel<<<kBlocks, kThreads, 0, s>>>(static_cast<uint4*>(dst), static_cast<const uint4*>(src), n_bytes / 16);
  return hipGetLastError();
}

}  // namespace rp
