// Token-level pre-gating with the router product on the matrix cores (bf16
// inputs, more than 64 adapters, E a multiple of 8; AdaFuse technical summary
// §2.A, and §2.B decoding steps 1-2).  The logits of a tile of 16 tokens are
// the MFMA product x[16, d] . Wg[d, E] with fp32 accumulation.  Wg is stored
// column-contiguous ([d][E]) while the matrix cores take K-contiguous
// operands, so a lane loads eight consecutive router rows at eight consecutive
// columns and transposes that 8 x 8 block in registers: MFMA c of a 32-wide
// k-step then covers columns 8n + c of a 128-column chunk (n = lane % 16).
//
// Summation order of a logit, the same in both launch forms and for every
// column (equal router columns give bit-equal logits, and ties go to the lower
// index): the 32-wide k-steps are cut into 16 contiguous parts; part q is one
// MFMA chain from zero in ascending k; a group of four parts is added in order,
// ((P0 + P1) + P2) + P3, and the four group sums in order again.
//
// Launch forms:
//   tile form  (rp_pregate, no workspace): one workgroup per token tile runs
//              every column chunk and part group, then selects the top k;
//   split form (inside a step): one workgroup per (token tile, column chunk,
//              part group) stores its group sum in the workspace; the last
//              workgroup of a tile to finish adds the sums, selects the top k,
//              and the last tile to finish runs the segmentation, so routing
//              and segmentation take one launch.
#include "route_common.h"

namespace rp {
namespace {

constexpr int kRmTok = 16;     // tokens per tile (MFMA rows)
constexpr int kRmCols = 128;   // router columns per chunk (16 lanes x 8)
constexpr int kRmParts = 16;   // K parts, each one MFMA chain
constexpr int kRmWaves = 4;    // waves per workgroup = parts per group
constexpr int kRmGroups = kRmParts / kRmWaves;
constexpr int kRmRing = 4;     // k-steps whose loads are in flight
constexpr int kRmThreads = 64 * kRmWaves;
constexpr int kRmChunkFloats = kRmTok * kRmCols;

__device__ __forceinline__ uint4 pick4(bool ok, uint4 v) { return ok ? v : make_uint4(0u, 0u, 0u, 0u); }

// Group sums cross workgroups through device-coherent (sc1) buffer accesses:
// a writer's stores have completed (s_waitcnt) before its arrival is counted,
// and the last arriver reads them from the coherence point, so no cache-wide
// write-back or invalidate is needed.
typedef unsigned int rm_u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kRmRsrcWord3 = 0x00020000;  // raw buffer, CDNA
constexpr int kRmSc1 = 1 << 4;            // device-scope coherence bit of the cache policy
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rm_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRmRsrcWord3);
}

// Part q of the logits of tokens t0 .. t0+15 at columns chunk*128 .. +127:
// acc[c][v] is the partial of token t0 + 4*(lane/16) + v at column
// chunk*128 + 8*(lane%16) + c.  Tokens past T repeat the last one.
__device__ __forceinline__ void logit_part(const PregateArgs& a, int t0, int chunk, int q, f32x4_t (&acc)[8]) {
  const int lane = threadIdx.x & 63, n = lane & 15, kg = lane >> 4;
  const bf16_t* xr = static_cast<const bf16_t*>(a.x) + (size_t)min(t0 + n, a.T - 1) * a.ld_x;
  const int col = chunk * kRmCols + 8 * n;  // E % 8 == 0: the lane's eight columns are all in or all out
  const bf16_t* wc = static_cast<const bf16_t*>(a.Wg) + min(col, a.E - 8);
  const int nks = (a.d_in + 31) >> 5;
  const int s0 = (int)((long long)nks * q / kRmParts), s1 = (int)((long long)nks * (q + 1) / kRmParts);
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 xa[kRmRing], wr[kRmRing][8];
  // k-step s: columns k = 32 s + 8 kg .. +7 of x (this lane's token) and router
  // rows k .. k+7 (this lane's columns); d_in % 8 == 0, so a group of eight is
  // all in or all out
  // loads go to clamped addresses and are masked where they are used, not as
  // they arrive (a select on loaded data waits for the load right there)
  auto issue = [&](int slot, int s) {
    const int kk = min(s * 32 + 8 * kg, a.d_in - 8);
    xa[slot] = ld16(xr + kk);
#pragma unroll
    for (int i = 0; i < 8; ++i) wr[slot][i] = ld16(wc + (size_t)(kk + i) * a.E);
  };
  auto consume = [&](int slot, int s) {
    // K columns past d_in contribute zero (the token operand is zeroed there);
    // router columns past E read a real column and are never stored
    const bool ok = s * 32 + 8 * kg < a.d_in;
    xa[slot] = pick4(ok, xa[slot]);
    // bt[c] = column col + c at rows k .. k+7 (element i = row k + i)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 lo4 = wr[slot][2 * j], hi4 = wr[slot][2 * j + 1];
        const uint32_t lo = (c >> 1) == 0 ? lo4.x : (c >> 1) == 1 ? lo4.y : (c >> 1) == 2 ? lo4.z : lo4.w;
        const uint32_t hi = (c >> 1) == 0 ? hi4.x : (c >> 1) == 1 ? hi4.y : (c >> 1) == 2 ? hi4.z : hi4.w;
        w[j] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      acc[c] = mfma16(xa[slot], make_uint4(w[0], w[1], w[2], w[3]), acc[c]);
    }
  };
  static_for<0, kRmRing>([&](auto I) {
    constexpr int i = decltype(I)::value;
    if (s0 + i < s1) issue(i, s0 + i);
  });
  int s = s0;
  for (; s + kRmRing <= s1; s += kRmRing) {
    static_for<0, kRmRing>([&](auto I) {
      constexpr int i = decltype(I)::value;
      consume(i, s + i);
      if (s + i + kRmRing < s1) issue(i, s + i + kRmRing);
    });
  }
  static_for<0, kRmRing>([&](auto I) {
    constexpr int i = decltype(I)::value;
    if (s + i < s1) consume(i, s + i);
  });
}

// Group g of (tile t0, chunk): wave w computes part 4g + w; wave 0 adds the
// four parts in order.  Returns true in wave 0, whose gs[c][v] then holds the
// group sum at the acc positions of logit_part.  `red` is 3 * 2048 floats.
__device__ __forceinline__ bool group_sum(const PregateArgs& a, int t0, int chunk, int g, float* red,
                                          f32x4_t (&gs)[8]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  logit_part(a, t0, chunk, g * kRmWaves + wave, gs);
  if (wave > 0) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[(wave - 1) * kRmChunkFloats + (c * 4 + v) * 64 + lane] = gs[c][v];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < kRmWaves - 1; ++w)
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int v = 0; v < 4; ++v) gs[c][v] += red[w * kRmChunkFloats + (c * 4 + v) * 64 + lane];
  }
  __syncthreads();  // red is free again
  return wave == 0;
}

// Logit position (token in tile, column) of entry (c, v) of `lane`.
__device__ __forceinline__ int pos_tok(int lane, int v) { return 4 * (lane >> 4) + v; }
__device__ __forceinline__ int pos_col(int lane, int chunk, int c) { return chunk * kRmCols + 8 * (lane & 15) + c; }

__global__ __launch_bounds__(kRmThreads) void route_mfma_tile_kernel(PregateArgs a) {
  __shared__ float lg[kRmTok * kMaxE];
  __shared__ float red[(kRmWaves - 1) * kRmChunkFloats];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kRmTok, nt = min(kRmTok, a.T - t0);
  const int n_chunks = (a.E + kRmCols - 1) / kRmCols;
  for (int chunk = 0; chunk < n_chunks; ++chunk)
    for (int g = 0; g < kRmGroups; ++g) {
      f32x4_t gs[8];
      if (group_sum(a, t0, chunk, g, red, gs)) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int col = pos_col(lane, chunk, c);
            if (col < a.E) {
              float* p = &lg[pos_tok(lane, v) * a.E + col];
              *p = g == 0 ? gs[c][v] : *p + gs[c][v];
            }
          }
      }
    }
  __syncthreads();
  if (a.logits)
    for (int i = threadIdx.x; i < nt * a.E; i += kRmThreads) a.logits[(size_t)t0 * a.E + i] = lg[i];
  route_select(a, lg, t0, nt, wave, kRmWaves, nullptr, 0);
}

struct RouteSplitArgs {
  PregateArgs a;
  SegmentArgs sg;
  float* sums;     // [tile][group][16][E] group sums
  int* counters;   // [0]: tiles finished; [1 + tile]: arrivals of the tile
  int n_chunks;
  int n_tiles;
};

__global__ __launch_bounds__(kRmThreads) void route_mfma_split_kernel(RouteSplitArgs ra) {
  __shared__ float lg[kRmTok * kMaxE];
  __shared__ float red[(kRmWaves - 1) * kRmChunkFloats];  // also the segmentation's histograms
  __shared__ int s_last, s_wave_tot[kRmWaves], s_bad;
  static_assert((kRmWaves - 1) * kRmChunkFloats >= kRmWaves * kMaxE, "histograms fit the reduction buffer");
  const PregateArgs& a = ra.a;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.x % kRmGroups, chunk = (blockIdx.x / kRmGroups) % ra.n_chunks;
  const int tile = blockIdx.x / (kRmGroups * ra.n_chunks);
  const int t0 = tile * kRmTok, nt = min(kRmTok, a.T - t0);
  const uint32_t tile_bytes = (uint32_t)(kRmGroups * kRmTok * a.E * sizeof(float));
  const __amdgpu_buffer_rsrc_t rs = rm_rsrc(ra.sums + (size_t)tile * kRmGroups * kRmTok * a.E, tile_bytes);
  f32x4_t gs[8];
  if (group_sum(a, t0, chunk, g, red, gs)) {
    const int col = pos_col(lane, chunk, 0);
    if (col < a.E) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t off = (uint32_t)(((g * kRmTok + pos_tok(lane, v)) * a.E + col) * sizeof(float));
        const f32x4_t lo = {gs[0][v], gs[1][v], gs[2][v], gs[3][v]};
        const f32x4_t hi = {gs[4][v], gs[5][v], gs[6][v], gs[7][v]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(rm_u32x4_t, lo), rs, off, 0, kRmSc1);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(rm_u32x4_t, hi), rs, off + 16, 0, kRmSc1);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // the group sum is at the coherence point before the arrival is counted
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&ra.counters[1 + tile], 1) == ra.n_chunks * kRmGroups - 1;
  __syncthreads();
  if (!s_last) return;
  if (tid == 0) stc_i32(&ra.counters[1 + tile], 0);  // ready for the next launch
  const int n4 = kRmTok * a.E / 4;
#pragma unroll 4
  for (int i = tid; i < n4; i += kRmThreads) {
    f32x4_t t[kRmGroups];
#pragma unroll
    for (int gg = 0; gg < kRmGroups; ++gg)
      t[gg] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                  rs, (uint32_t)((gg * n4 + i) * 16), 0, kRmSc1));
    f32x4_t s = t[0];
#pragma unroll
    for (int gg = 1; gg < kRmGroups; ++gg) s += t[gg];
    *reinterpret_cast<f32x4_t*>(&lg[4 * i]) = s;
  }
  __syncthreads();
  if (a.logits)
    for (int i = tid; i < nt * a.E; i += kRmThreads) a.logits[(size_t)t0 * a.E + i] = lg[i];
  route_select(a, lg, t0, nt, wave, kRmWaves, nullptr, 0);
  __builtin_amdgcn_s_waitcnt(0);  // the tile's routing (device-scope stores) is out before the tile is counted
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&ra.counters[0], 1) == ra.n_tiles - 1;
  __syncthreads();
  if (!s_last) return;
  if (tid == 0) stc_i32(&ra.counters[0], 0);
  segment_block<kRmWaves>(ra.sg, reinterpret_cast<int*>(red), s_wave_tot, &s_bad);
}

}  // namespace

bool mfma_router_supported(Dtype dt, int E) { return dt == kBF16 && E > 64 && E <= kMaxE && E % 8 == 0; }

int route_split_tiles(int T) { return (T + kRmTok - 1) / kRmTok; }

size_t route_split_bytes(int T, int E) {
  return (size_t)route_split_tiles(T) * kRmGroups * kRmTok * E * sizeof(float);
}

hipError_t launch_route_mfma(const PregateArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  route_mfma_tile_kernel<<<route_split_tiles(a.T), kRmThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_route_segment_mfma(const PregateArgs& a, const SegmentArgs& sg, void* sums, int* counters,
                                     hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  RouteSplitArgs ra;
  ra.a = a;
  ra.sg = sg;
  ra.sums = static_cast<float*>(sums);
  ra.counters = counters;
  ra.n_chunks = (a.E + kRmCols - 1) / kRmCols;
  ra.n_tiles = route_split_tiles(a.T);
  route_mfma_split_kernel<<<ra.n_tiles * ra.n_chunks * kRmGroups, kRmThreads, 0, s>>>(ra);
  return hipGetLastError();
}

}  // namespace rp
