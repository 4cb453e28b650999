// Segmentation of the (token, slot) pairs by adapter: the segments of the
// segmented gather matrix multiply (AdaFuse, technical summary §2.B).
//
// One workgroup of 16 waves.  Wave w owns a contiguous run of pairs.
//   1. per-wave histogram of adapter ids in LDS
//   2. exclusive scan over (adapter, wave): seg_offsets[e] and the first output
//      slot of every (wave, adapter) run
//   3. each wave walks its run in 64-pair chunks; lanes with equal adapter ids
//      are matched with ballots, ranked by lane order, and scattered, so the
//      order inside a segment is ascending pair id (stable).
// Out-of-range ids are counted into *err_count and left out.
#include "device_common.h"
#include "kernels.h"

namespace rp {
namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;

__global__ __launch_bounds__(kThreads) void segment_kernel(SegmentArgs a) {
  __shared__ int hist[kWaves][kMaxE];  // counts, then running output slots
  __shared__ int wave_tot[kWaves];
  __shared__ int bad;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, n = a.n_pairs;
  for (int q = tid; q < kWaves * E; q += kThreads) hist[q / E][q % E] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();

  const int run = (n + kWaves - 1) / kWaves;
  const int beg = min(n, wave * run), end = min(n, beg + run);

  // 1. histogram
  int my_bad = 0;
  for (int p = beg + lane; p < end; p += 64) {
    const int e = a.topk_idx[p];
    if (e >= 0 && e < E)
      atomicAdd(&hist[wave][e], 1);
    else
      ++my_bad;
  }
  my_bad = wave_sum_int(my_bad);
  if (lane == 0 && my_bad) atomicAdd(&bad, my_bad);
  __syncthreads();

  // 2. scan: per adapter e, counts of waves 0..15 in order; then across adapters.
  //    Thread e (looping for E > kThreads) holds the adapter's total.
  int carry = 0;
  for (int e0 = 0; e0 < E; e0 += kThreads) {
    const int e = e0 + tid;
    int tot = 0;
    if (e < E)
      for (int w = 0; w < kWaves; ++w) tot += hist[w][e];
    // block-wide exclusive scan of tot over e (in e order)
    const int incl = wave_inclusive_scan(tot, lane);
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int wave_base = 0;
    for (int w = 0; w < wave; ++w) wave_base += wave_tot[w];
    int block_total = 0;
    for (int w = 0; w < kWaves; ++w) block_total += wave_tot[w];
    const int excl = carry + wave_base + incl - tot;
    if (e < E) {
      a.seg_offsets[e] = excl;
      int s = excl;
      for (int w = 0; w < kWaves; ++w) {
        const int c = hist[w][e];
        hist[w][e] = s;
        s += c;
      }
    }
    carry += block_total;
    __syncthreads();
  }
  if (tid == 0) {
    a.seg_offsets[E] = carry;
    *a.err_count = bad;
  }
  __syncthreads();

  // 3. stable scatter
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  for (int c0 = beg; c0 < end; c0 += 64) {
    const int p = c0 + lane;
    const bool in = p < end;
    const int e = in ? a.topk_idx[p] : -1;
    const bool valid = in && e >= 0 && e < E;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(valid && bit);
      peers &= bit ? m : ~m;
    }
    if (valid) {
      const int rank = __popcll(peers & lanemask_lt(lane));
      a.pair_perm[hist[wave][e] + rank] = p;
    }
    // the last lane of each group advances the group's cursor; reads above
    // happen before any of these writes (lockstep wave, in-order LDS)
    __builtin_amdgcn_wave_barrier();
    if (valid && (peers >> lane) == 1ull) hist[wave][e] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

hipError_t launch_segment(const SegmentArgs& a, hipStream_t s) {
  segment_kernel<<<1, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace rp
