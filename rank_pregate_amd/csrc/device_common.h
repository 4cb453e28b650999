// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace rp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kMaxK = 8;   // largest top-k
constexpr int kMaxE = 1024;  // largest adapter count
constexpr int kMaxEWords = kMaxE / 32;

// bfloat16 values travel as raw 16-bit patterns.
typedef uint16_t bf16_t;

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time (for
// register arrays indexed by a loop position).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Packed backbone weights (RP_W0_TILED): 16-row x 32-column blocks of 1 KB,
// grouped in chunks of four block columns (128 columns).  Chunk g stores its
// blocks row block by row block, nbg = min(4, nb - 4g) blocks each, so the
// blocks a decode launch reads at one moment (the same chunk of every row
// block) sit together in memory.  Element offset of block (rb, cb), for n_rb
// row blocks and nb block columns:
__host__ __device__ inline size_t w0_block_offset(int rb, int cb, int n_rb, int nb) {
  const int g = cb >> 2;
  const int nbg = nb - 4 * g < 4 ? nb - 4 * g : 4;
  return ((size_t)g * 4 * n_rb + (size_t)rb * nbg + (cb & 3)) * 512;
}

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two bfloat16 packed in one word (a in the low half), rounded to
// nearest even by the hardware conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Round-to-nearest-even float -> bfloat16 (inputs are finite by contract).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return static_cast<bf16_t>(f32x2_to_bf16x2(f, f) & 0xffffu); }

// Eight packed bf16 (one 16-byte vector) as the MFMA operand type.
__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Streaming 16-byte load for data read exactly once (backbone weights).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Split eight fp32 values into a high and a low bf16 part, hi + lo ~= v to
// about 16 significant bits, so a bf16 MFMA on (hi, lo) keeps close to fp32
// precision for the small rank-r operand.
__device__ __forceinline__ void split_hi_lo(const float* v, uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = f32x2_to_bf16x2(v[2 * i], v[2 * i + 1]);
    const float r0 = v[2 * i] - __uint_as_float(h[i] << 16);
    const float r1 = v[2 * i + 1] - __uint_as_float(h[i] & 0xffff0000u);
    l[i] = f32x2_to_bf16x2(r0, r1);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

__device__ __forceinline__ f32x16_t mfma32(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Gated MLP activation on one element: silu(g) * u in fp32 (the fused epilogue
// and the separate launch both use this, so they give the same bits).
__device__ __forceinline__ float silu_mul_f32(float g, float u) { return g / (1.0f + expf(-g)) * u; }

__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int n = __shfl_up(v, o, kWave);
    if (lane >= o) v += n;
  }
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace rp
