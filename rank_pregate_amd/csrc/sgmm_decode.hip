// Decode-shaped fused SGMM (T <= 64 tokens): one launch per projection group
// computes, for every projection sharing x,
//
//     y[t] = W0 x[t] + sum_j g[t,j] * B_e (A_e x[t]),   e = idx[t,j]
//
// (AdaFuse technical summary §2.B: the chosen adapters are applied with the
// backbone in a single kernel call).  Decode is bound by HBM: every byte of W0
// is read once.  A fused launch also runs the router and the segmentation
// first (§2.A pre-gating; §2.B decoding steps 1-2), so routing overlaps the
// weight stream instead of preceding it.
//
// Work items, numbered in this order; a workgroup's first item is its block
// index, each later one is claimed from a launch-wide counter:
//   0. (fused) router items (two two-token tiles, one per half workgroup),
//      then one segmentation item.
//   1. shrink items, for every group whose input comes from the call first:
//      with E <= 32, 64-row tiles of the stacked [A_0; ..; A_{E-1}] through
//      the backbone's streaming loop over every token, split along K (`dense`
//      u as tagged fp32 pairs); with more adapters, chunks of <= 16 pairs of
//      one segment over one of KP parts of K (unscaled fp32 partials).
//   2. backbone items: 16 output rows per wave (four waves, or eight for 64
//      tokens) over one of S splits of K, bf16 MFMA 16x16x32 with the tokens as M and W0 rows as N.
//      K goes in 128-column chunks; each thread issues a chunk's activation
//      pieces and then its wave's four 1 KB weight blocks NR chunks ahead of
//      the math into register rings (NR = 4 for T <= 32, 2 for T = 64); the
//      next chunk's activations move to an LDS double buffer in MFMA fragment
//      order one chunk before use.  The last split adds the other splits'
//      partial tiles in split order and applies the adapter deltas: the
//      chosen adapters' gated u as a (hi, lo) bf16 token operand against B_e's
//      rows, its operands requested inside the last two rings.
// An item only ever waits for items with smaller numbers, and the grid never
// exceeds what the chip holds at once, so every wait ends: the smallest
// unfinished item always has its workgroup running and nothing to wait for.
//
// Data crossing workgroups is written and read with device-scope (sc1)
// accesses, so no cache-wide fence is needed.  Routing results and pair-chunk
// u are announced by counters (a writer waits for its stores first); dense u
// and split-K partial tiles travel as tagged pairs that the reader validates.
// The split-K partials of a tile are summed in split order by the tile's last
// split, so the output does not depend on timing.
#include "route_common.h"
#include "sgmm_common.h"

namespace rp {
namespace {

constexpr int kSpinLimit = 1 << 22;  // ~seconds; a wait this long flags kCtlWaitOverflow and gives up
constexpr int kKC = 128;             // K per chunk
constexpr int kKS = kKC / 32;        // MFMA k-steps per chunk
// Waves per item (16 output rows each).  A workgroup stages each chunk's
// activations once for all its waves, so the activation bytes per weight byte
// of a workgroup are T / (16 * waves): with 64 tokens, eight waves (128-row
// tiles) halve them against four (measured with a stream probe of this loop on
// 128 MiB: 4.6 -> 5.9 TB/s); with 32 tokens or fewer four waves stream as fast.
template <int MT>
constexpr int kWavesOf = MT >= 4 ? 8 : 4;
template <int MT>
constexpr int kThreadsOf = 64 * kWavesOf<MT>;
template <int MT>
constexpr int kTileRowsOf = 16 * kWavesOf<MT>;
template <int MT>
constexpr int kBlocksPerCuOf = kWavesOf<MT> == 8 ? 1 : 2;  // launch bound: workgroups one CU holds
// Chunks whose loads are in flight ahead of the math.  A load returns about
// that many chunk times after issue (returns are in order behind the stream),
// so the ring is no deeper than the bandwidth needs: with 64 tokens the
// activation bytes equal the weight bytes and two chunks suffice.
template <int MT>
constexpr int kRingOf = MT >= 4 ? 2 : 4;
static_assert(kThreadsOf<2> == 2 * kRouteThreads, "a fused workgroup runs two router tiles side by side");
static_assert(sizeof(StepArgs) <= 4096, "kernel argument block too large");
constexpr int kFusedRouteTokens = 2;  // tokens per router tile of a fused launch
constexpr int kMaxFusedE = 64;        // adapters a fused launch routes over (two partial sums per column)
constexpr int kUPiecesPerItem = 1024;  // u pieces (two tagged values each) the staged expand holds per item

typedef unsigned int u32x4_v __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, CDNA
constexpr int kSc1 = 1 << 4;            // device-scope coherence bit of the cache policy

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ void st_coh16(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_v, v), r, off, 0, kSc1);
}
__device__ __forceinline__ f32x4_t ld_coh16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1));
}

// Tagged hand-offs: a value crossing workgroups travels as an 8-byte pair
// (fp32 bits, tag), where the tag names the launch that wrote it (a NaN bit
// pattern carrying the low 20 bits of the workspace's launch epoch; finite
// data never has it).  A reader loads the pairs directly and retries while
// any tag is stale, so no separate "ready" counter costs it a round trip.
// Each pair is written by one 8-byte-aligned piece of a store and checked on
// its own, so a store seen half-done is simply retried.
__device__ __forceinline__ uint32_t launch_tag(int ep) { return 0xFFF00000u | ((uint32_t)ep & 0xFFFFFu); }

__device__ __forceinline__ void st_tagged4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4_t v, uint32_t tag) {
  const u32x4_v a = {__float_as_uint(v[0]), tag, __float_as_uint(v[1]), tag};
  const u32x4_v b = {__float_as_uint(v[2]), tag, __float_as_uint(v[3]), tag};
  __builtin_amdgcn_raw_buffer_store_b128(a, r, off, 0, kSc1);
  __builtin_amdgcn_raw_buffer_store_b128(b, r, off + 16, 0, kSc1);
}

// Four tagged values at byte offset off (32 bytes); true when all four carry `tag`.
__device__ __forceinline__ bool ld_tagged4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t tag, f32x4_t& v) {
  const u32x4_v a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1);
  const u32x4_v b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, kSc1);
  v = f32x4_t{__uint_as_float(a.x), __uint_as_float(a.z), __uint_as_float(b.x), __uint_as_float(b.z)};
  return a.y == tag && a.w == tag && b.y == tag && b.w == tag;
}

// Per-wave retry bookkeeping of a tagged read: true while it should go on.
__device__ __forceinline__ bool retry_tagged(int* ctl, bool lane_ok, int* spins) {
  if (__ballot(!lane_ok) == 0) return false;
  __builtin_amdgcn_s_sleep(2);
  if (++*spins > kSpinLimit) {
    if ((threadIdx.x & 63) == 0) atomicOr(&ctl[kCtlWaitOverflow], 1);
    return false;
  }
  return true;
}

template <int MT, bool FUSED>
constexpr size_t smem_bytes() {
  constexpr size_t WV = kWavesOf<MT>;
  // activation chunks (double-buffered), the expand's routing, its token operand (hi, lo)
  constexpr size_t xs = 2ull * MT * kKS * 512 * sizeof(bf16_t) + 16ull * MT * kMaxK * 8 + MT * 4 * 64 * 16 * 2;
  constexpr size_t red = (WV - 1) * 8 * 64 * 4 * sizeof(float);         // pair shrink: waves 1.., 8 rank tiles
  constexpr size_t route = FUSED ? 2ull * 3 * kFusedRouteTokens * kMaxFusedE * sizeof(float) : 0;  // two router tiles
  constexpr size_t seg = FUSED ? WV * kMaxE * sizeof(int) : 0;           // segmentation histograms
  size_t m = xs;
  if (red > m) m = red;
  if (route > m) m = route;
  if (seg > m) m = seg;
  return m;
}

// Per-wave wait until *p >= target (uniform across the wave).
__device__ __forceinline__ void wait_geq(int* ctl, const int* p, int target) {
  int spins = 0;
  while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    __builtin_amdgcn_s_sleep(2);
    if (++spins > kSpinLimit) {
      if ((threadIdx.x & 63) == 0) atomicOr(&ctl[kCtlWaitOverflow], 1);
      break;
    }
  }
}

__device__ __forceinline__ int* ctl_set(int* ctl, int ep) { return ctl + kCtlSet0 + (ep & 1) * kCtlSetStride; }

// Before reading an input that earlier groups of the launch write, an item of
// group g waits until every output tile of groups 0..g-1 is written (tiles are
// counted per group and tile % 8, so no single counter takes every workgroup;
// lane 8*h + c reads group h's class c); wave 0 polls, the workgroup then
// proceeds.  No cache-wide fence follows: those tiles were stored
// device-coherent before they were counted, and the group reads its input with
// device-coherent loads (an agent-scope acquire would wait for the weight
// loads already in flight and invalidate the XCD's L2).
__device__ __forceinline__ void wait_prev_group(int* ctl, int ep, const DecodeArgs& d) {
  static_assert(8 * kMaxGroups <= 64, "one counter per lane");
  if ((threadIdx.x >> 6) == 0) {
    const int lane = threadIdx.x & 63;
    const int* p = ctl + kCtlSet0 + (ep & 1) * kCtlSetStride + kSetGroupDone + 256 * (lane >> 3) + 32 * (lane & 7);
    const bool mine = lane < 8 * d.group;
    int spins = 0;
    while (true) {
      const int v = mine ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
      if (wave_sum_int(v) >= d.prev_target) break;
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kSpinLimit) {
        if (lane == 0) atomicOr(&ctl[kCtlWaitOverflow], 1);
        break;
      }
    }
  }
  __syncthreads();
}

// Thread 0, once per workgroup, after reading the epoch: count in per
// blockIdx % 8 class (no single counter takes every workgroup); the last of a
// class counts into the launch total, and the last of those (every workgroup
// has now read the epoch) clears the other control set for the next launch and
// advances the epoch, early in the launch rather than after its last item.
__device__ __forceinline__ void arrive(int* ctl, int ep) {
  int* set = ctl_set(ctl, ep);
  const int G = gridDim.x, cls = blockIdx.x & 7;
  const int count_c = (G - 1 - cls) / 8 + 1;
  if (atomicAdd(&set[kSetArrive + 32 * cls], 1) != count_c - 1) return;
  const int n_classes = G < 8 ? G : 8;
  if (atomicAdd(&set[kSetArriveAll], 1) != n_classes - 1) return;
  int* other = ctl_set(ctl, ep + 1);
  for (int w = 0; w < kSetWords; w += 32) __hip_atomic_store(&other[w], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&ctl[kCtlEpoch], ep + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// u partials of projection `proj`, part kp: [slots][r] fp32 with
// slots = dense ? E * t_pad (adapter-major, then token) : T * k (pair id).
__device__ __forceinline__ size_t upart_slots(const SgmmArgs& a, const DecodeArgs& d) {
  return d.dense ? (size_t)a.E * d.t_pad : (size_t)a.T * a.k;
}

// ---------------------------------------------------------------------------
// pair-chunk shrink units, 2 waves
// ---------------------------------------------------------------------------
// One unit (adapters beyond the dense limit): rank rows of A_e (MTR tiles of
// 16) against one chunk of <= 16 pairs of e's segment, over K part kp; the
// two waves split the part and are added in wave order.  COH: the segments
// were written by this launch.
template <int MTR, bool COH, int WV>
__device__ __forceinline__ void shrink_item(const SgmmArgs& a, const DecodeArgs& d, int proj, int unit, int kp,
                                            float* red, int* s_loc, int* ctl, int ep) {
  // k-steps per batch: all loads of a batch are issued before its MFMAs, so a
  // unit costs about one memory round trip per batch
  constexpr int U = MTR <= 2 ? 8 : (MTR <= 8 ? 2 : 1);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (d.prev_target > 0) wait_prev_group(ctl, ep, d);
  if (tid < 64) {
    int ee, c;
    locate_chunk<COH>(a, unit, 16, tid, &ee, &c);
    if (tid == 0) { s_loc[0] = ee; s_loc[1] = c; }
  }
  __syncthreads();
  const int e = s_loc[0];
  if (e < 0) return;
  const int slot0 = ld_route<COH>(&a.seg_offsets[e]) + s_loc[1] * 16;
  const int slot_end = min(ld_route<COH>(&a.seg_offsets[e + 1]), slot0 + 16);

  const ProjDesc pd = proj_at(a, proj);
  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  const bf16_t* Ae = static_cast<const bf16_t*>(pd.A) + (size_t)e * a.r * a.d_in;
  const int lr = lane & 15, kg = lane >> 4;
  const bf16_t* xp = x + (size_t)(ld_route<COH>(&a.pair_perm[min(slot0 + lr, slot_end - 1)]) / a.k) * a.ld_x;
  const __amdgpu_buffer_rsrc_t rx = rsrc(x, (uint32_t)((size_t)a.T * a.ld_x * sizeof(bf16_t)));
  const bf16_t* ap[MTR];
  bool aok[MTR];
#pragma unroll
  for (int mt = 0; mt < MTR; ++mt) {
    const int c = mt * 16 + lr;
    aok[mt] = c < a.r;
    ap[mt] = Ae + (size_t)min(c, a.r - 1) * a.d_in;
  }
  const int nsteps = (a.d_in + 31) >> 5;
  const int pb = nsteps * kp / d.KP, pe = nsteps * (kp + 1) / d.KP;
  const int sb = pb + (pe - pb) * wave / WV, se = pb + (pe - pb) * (wave + 1) / WV;
  f32x4_t acc[MTR];
#pragma unroll
  for (int mt = 0; mt < MTR; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s = sb; s < se; s += U) {
    uint4 av[U][MTR], bv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s + u) * 32 + kg * 8;
      const bool ok = (s + u < se) && (k < a.d_in);
      const int kc = min(k, a.d_in - 8);
#pragma unroll
      for (int mt = 0; mt < MTR; ++mt) av[u][mt] = sel4(ok && aok[mt], ld16(ap[mt] + kc));
      // an input written earlier in this launch is read device-coherent
      bv[u] = sel4(ok, d.x_acquire ? __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                         rx, (uint32_t)((xp + kc - x) * sizeof(bf16_t)), 0, kSc1))
                                   : ld16(xp + kc));
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MTR; ++mt) acc[mt] = mfma16(av[u][mt], bv[u], acc[mt]);
  }
  // waves 0, 1, .. added in that order; D layout: lane -> pair slot0 +
  // lane%16, rank rows mt*16 + 4*(lane/16) + 0..3
  if (wave > 0) {
#pragma unroll
    for (int mt = 0; mt < MTR; ++mt)
      *reinterpret_cast<f32x4_t*>(&red[(((wave - 1) * 8 + mt) * 64 + lane) * 4]) = acc[mt];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 1; w < WV; ++w)
#pragma unroll
      for (int mt = 0; mt < MTR; ++mt) acc[mt] += *reinterpret_cast<const f32x4_t*>(&red[(((w - 1) * 8 + mt) * 64 + lane) * 4]);
    const size_t slots = upart_slots(a, d);
    const float* ub = a.u + ((size_t)proj * d.KP + kp) * slots * a.r;
    const __amdgpu_buffer_rsrc_t r = rsrc(ub, (uint32_t)(slots * a.r * sizeof(float)));
    const int s = slot0 + lr;
    if (s < slot_end) {
      const int p = ld_route<COH>(&a.pair_perm[s]);
#pragma unroll
      for (int mt = 0; mt < MTR; ++mt) {
        const int c = mt * 16 + 4 * kg;
        if (c < a.r) st_coh16(r, (uint32_t)(((size_t)p * a.r + c) * sizeof(float)), acc[mt]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// base item
// ---------------------------------------------------------------------------
// One output tile of 64 rows (16 per wave) over one K split.  With ATILE the
// rows are those of the stacked adapter down-projections [A_0; ..; A_{E-1}]
// of one projection and the result is the rank-r intermediate u[e][t] (fp32,
// every token) instead of y.  The last of a tile's S splits applies the
// adapter deltas and sums the other splits' partial tiles.
//
// The stream: K goes in chunks of 128 columns.  For every chunk each thread
// issues its activation pieces first, then its wave's four 1 KB weight blocks,
// NR chunks ahead of the math, into register rings; the activations of the
// next chunk move to an LDS double buffer (in MFMA fragment order) one chunk
// before use.  Loads retire in issue order, so waiting for a chunk's
// activations leaves the weight loads of the NR chunks issued after them in
// flight.  The expand's operands (routing, u, B) are requested inside the last
// two rings at fixed positions, each before the weights it must not wait for,
// so only the expand's MFMAs and the stores follow the last chunk.
template <int MT, bool TILED, bool FUSED, bool ATILE, bool LANEX>
__device__ __forceinline__ void base_item(const SgmmArgs& a, const DecodeArgs& d, int bi, bf16_t* xs, int* ctl, int* s_ep,
                          bool first, int ep_in) {
  constexpr int G = 8;                          // adapters per batch of B loads
  constexpr uint32_t kOob = 0x80000000u;        // past any buffer: a buffer load returns zero
  constexpr int XB = MT * kKS;                  // 1 KB activation fragment blocks per chunk
  constexpr int NR = kRingOf<MT>;               // chunks in flight ahead of the math
  constexpr int WV = kWavesOf<MT>;              // waves of the item, 16 output rows each
  constexpr int NTH = 64 * WV;
  constexpr int TR = 16 * WV;                   // output rows of the item
  constexpr int MP = XB / WV;                   // activation fragment blocks a thread stages per chunk
  static_assert(XB % WV == 0, "every wave stages the same number of fragment blocks");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = ATILE ? d.SA : a.S;
  const int tile = bi / S, split = bi % S;
  const bool last = split == S - 1;
  const bool expand = !ATILE && a.k > 0 && last;
  const int proj = ATILE ? tile / d.atiles_per_proj : proj_of_tile(a, tile);
  const ProjDesc pd = proj_at(a, proj);
  const int n_rows = ATILE ? a.E * a.r : pd.d_out;
  const int row0 = (ATILE ? tile % d.atiles_per_proj : tile - pd.tile_begin) * TR + wave * 16;
  const int lr = lane & 15, kg = lane >> 4;
  const int row = min(row0 + lr, n_rows - 1);
  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  const bf16_t* Bm = static_cast<const bf16_t*>(pd.B);
  const bf16_t* w0 = static_cast<const bf16_t*>(ATILE ? pd.A : pd.W0);
  // tiled: this wave's row block; row-major: this lane's row at column 8*kg of each k-step
  const int nb = a.d_in / 32, n_rb = pd.d_out / 16;
  const int rblk = min(row0 / 16, n_rb - 1);
  const bf16_t* wrow = w0 + (size_t)row * a.d_in + kg * 8;
  const int nch = (a.d_in + kKC - 1) / kKC;
  const int cbeg = (int)((long long)nch * split / S);
  const int nc = (int)((long long)nch * (split + 1) / S) - cbeg;  // >= 1: the plan keeps S <= nch
  // activation piece p of this thread: fragment block b = wave + WV*p of the
  // chunk, i.e. token tile b / 4 (token (b/4)*16 + lane%16) and k-step b % 4
  // = wave % 4 (columns 32*(wave%4) + 8*kg .. +7 of the chunk)
  const int xcol = (wave & 3) * 32 + kg * 8;
  const bf16_t* xq[MP];
#pragma unroll
  for (int p = 0; p < MP; ++p) xq[p] = x + (size_t)min(((wave + WV * p) >> 2) * 16 + lr, a.T - 1) * a.ld_x;
  // an input written earlier in this launch is read device-coherent
  const bool x_coh = d.x_acquire != 0;
  const __amdgpu_buffer_rsrc_t rx = rsrc(x, (uint32_t)((size_t)a.T * a.ld_x * sizeof(bf16_t)));

  f32x4_t acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint4 wr[NR][kKS];
  uint4 xr[NR][MP];

  // The split's nc chunks are preceded by `pad` empty ones so that their count
  // V is a multiple of NR: chunk v then always sits in ring slot v % NR
  // and the last chunks at fixed positions of the code.  An empty chunk stages
  // zero activations; its weight slot loads activation bytes (cache-resident)
  // in place of weights, except in a group whose x an earlier group of the
  // launch writes: there the weight slots fill before the wait, when x may
  // still hold anything (a NaN times the zero activations would poison the
  // sums), so they load the split's first weight block instead.  Loads are
  // never masked (a select would force a wait right after them); weight
  // blocks past d_in are clamped to a real block and meet activations that
  // store_x wrote as zero.
  const int pad = (NR - nc % NR) % NR;
  const int V = nc + pad;
  const bool pad_reads_w = d.prev_target > 0;
  auto issue_w = [&](int slot, int v) {
    const int c = v - pad;
    const int cc = cbeg + max(c, 0);
    const bf16_t* xa = xq[0] + min(cc * kKC + xcol, a.d_in - 8);
    const bool real = c >= 0 || pad_reads_w;
    if (TILED) {
      const int nbg = min(4, nb - 4 * cc);
      const bf16_t* blk = w0 + ((size_t)cc * 4 * n_rb + (size_t)rblk * nbg) * 512 + lane * 8;
#pragma unroll
      for (int s = 0; s < kKS; ++s) wr[slot][s] = ld16_stream(real ? blk + (size_t)min(s, nbg - 1) * 512 : xa);
    } else {
#pragma unroll
      for (int s = 0; s < kKS; ++s)
        wr[slot][s] = ld16_stream(real ? wrow + min(cc * kKC + s * 32, a.d_in - 8 - kg * 8) : xa);
    }
  };
  auto issue_x = [&](int slot, int v) {
    const int col = min((cbeg + max(v - pad, 0)) * kKC + xcol, a.d_in - 8);
    if (x_coh) {
#pragma unroll
      for (int p = 0; p < MP; ++p)
        xr[slot][p] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)((xq[p] + col - x) * sizeof(bf16_t)), 0, kSc1));
    } else {
#pragma unroll
      for (int p = 0; p < MP; ++p) xr[slot][p] = ld16(xq[p] + col);
    }
  };
  auto issue = [&](int slot, int v) {  // activations first, then weights
    issue_x(slot, v);
    issue_w(slot, v);
  };
  // piece p of thread tid goes to fragment block wave + WV*p, lane `lane`
  auto store_x = [&](int slot, int buf, int v) {
    const int c = v - pad;
    const bool ok = c >= 0 && (cbeg + c) * kKC + xcol < a.d_in;
#pragma unroll
    for (int p = 0; p < MP; ++p)
      *reinterpret_cast<uint4*>(&xs[(buf * XB + WV * p) * 512 + tid * 8]) = sel4(ok, xr[slot][p]);
  };
  auto compute = [&](int slot, int buf) {
#pragma unroll
    for (int s = 0; s < kKS; ++s)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint4 xf = *reinterpret_cast<const uint4*>(&xs[((buf * XB + m * kKS + s) * 64 + lane) * 8]);
        acc[m] = mfma16(xf, wr[slot][s], acc[m]);
      }
  };

  // dense u as tagged pairs [proj][e][t_pad][r]
  const __amdgpu_buffer_rsrc_t ru =
      rsrc(reinterpret_cast<const char*>(a.u) + (size_t)proj * a.E * d.t_pad * a.r * 8,
           (uint32_t)((size_t)a.E * d.t_pad * a.r * 8));
  auto load_u4 = [&](u32x4_v (&w)[4], uint32_t off) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = __builtin_amdgcn_raw_buffer_load_b128(ru, off == kOob ? kOob : off + 16 * i, 0, kSc1);
  };
  // routing of the tile's tokens for the expand: pair p = tid + j * NTH
  // as (index, tag, gate bits, tag) when this launch's router tiles wrote it,
  // else (index, -, gate bits, -) from the inputs
  constexpr int kRP = (16 * MT * kMaxK + NTH - 1) / NTH;
  const int n_pairs = a.T * a.k;
  const __amdgpu_buffer_rsrc_t rt = rsrc(d.route_tagged, (uint32_t)((size_t)n_pairs * 16));
  u32x4_v rraw[kRP];
  auto route_load = [&](int j) {
    const int p = tid + j * NTH;
    if (FUSED) {
      rraw[j] = __builtin_amdgcn_raw_buffer_load_b128(rt, p < n_pairs ? (uint32_t)(p * 16) : kOob, 0, kSc1);
    } else {
      const int q = min(p, n_pairs - 1);
      rraw[j] = u32x4_v{(uint32_t)a.topk_idx[q], 0u, __float_as_uint(a.topk_gate[q]), 0u};
    }
  };
  auto route_issue = [&]() {
#pragma unroll
    for (int j = 0; j < kRP; ++j) route_load(j);
  };
  // LDS after the activation buffers: adapter and gate of every (token, slot)
  // pair, then the expand's token operand in MFMA fragment order
  int* s_sel = reinterpret_cast<int*>(xs + 2 * XB * 512);
  float* s_gate = reinterpret_cast<float*>(s_sel + 16 * MT * kMaxK);
  uint4* fhi = reinterpret_cast<uint4*>(s_gate + 16 * MT * kMaxK);
  uint4* flo = fhi + MT * 4 * 64;
  auto stage_route = [&](uint32_t tg) {
#pragma unroll
    for (int j = 0; j < kRP; ++j) {
      const int p = tid + j * NTH;
      if (FUSED) {
        // written by this launch's router tiles, validated by tag
        // first check outside the retry loop: waiting for this load then
        // leaves the weight loads issued after it in flight (a loop header
        // would wait for every load)
        int spins = 0;
        if (retry_tagged(ctl, p >= n_pairs || (rraw[j].y == tg && rraw[j].w == tg), &spins)) do
            route_load(j);
          while (retry_tagged(ctl, p >= n_pairs || (rraw[j].y == tg && rraw[j].w == tg), &spins));
      }
      if (p < n_pairs) {
        s_sel[p] = (int)rraw[j].x;
        s_gate[p] = __uint_as_float(rraw[j].z);
      }
    }
  };

  // The expand with every adapter's rank columns side by side along K (dense
  // u, E*r <= 128, the tile's u pieces fitting kUP per thread): column e*r + c
  // of the token operand is sum_j [idx(t,j) = e] g(t,j) u_e[t][c], split into
  // bf16 (hi, lo); each wave adds two MFMAs per 32 columns against its rows of
  // the B_e placed side by side the same way.  u pieces are scattered straight
  // into fragment order; B fragments go straight to registers.
  const int kcat = a.E * a.r;
  const int half_r = a.r >> 1;
  const int lg_r = __builtin_ctz(a.r);  // r is a power of two >= 8
  constexpr int kUP = kUPiecesPerItem / NTH;  // per thread
  const bool px = expand && d.dense && kcat <= 128 && n_pairs * half_r <= kUP * NTH;
  // with two rings or more, the expand's operands are requested and placed
  // while the last chunks stream, so only its MFMAs follow the last chunk
  const bool early = !LANEX && px && V >= 2 * NR;
  uint4 bfr[4];
  auto b_issue = [&]() {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kcol = min(st * 32 + kg * 8, kcat - 8);
      bfr[st] = ld16(Bm + ((size_t)(kcol >> lg_r) * pd.d_out + row) * a.r + (kcol & (a.r - 1)));
    }
  };
  // piece q: pair q / (r/2), values 2 * (q % (r/2)) and the next
  u32x4_v uraw[kUP];
  auto u_piece = [&](int q) -> uint32_t {
    if (q >= n_pairs * half_r) return kOob;
    const int p = q / half_r, c = 2 * (q % half_r);
    return (uint32_t)((((size_t)s_sel[p] * d.t_pad + p / a.k) * a.r + c) * 8);
  };
  auto u_issue = [&]() {
#pragma unroll
    for (int i = 0; i < kUP; ++i) uraw[i] = __builtin_amdgcn_raw_buffer_load_b128(ru, u_piece(tid + i * NTH), 0, kSc1);
  };
  auto frag_zero = [&]() {
#pragma unroll
    for (int i = 0; i < 512 * MT / NTH; ++i) fhi[tid + i * NTH] = zero4();  // fhi and flo, MT * 512 entries
  };
  auto u_scatter = [&](uint32_t tg) {
#pragma unroll
    for (int i = 0; i < kUP; ++i) {
      const int q = tid + i * NTH;
      const uint32_t off = u_piece(q);
      int spins = 0;  // first check outside the retry loop (as in stage_route)
      if (retry_tagged(ctl, off == kOob || (uraw[i].y == tg && uraw[i].w == tg), &spins)) do
          uraw[i] = __builtin_amdgcn_raw_buffer_load_b128(ru, off, 0, kSc1);
        while (retry_tagged(ctl, off == kOob || (uraw[i].y == tg && uraw[i].w == tg), &spins));
      if (off != kOob) {
        const int p = q / half_r, c = 2 * (q % half_r);
        const int t = p / a.k, j = p - t * a.k, e = s_sel[p];
        // a token naming e in several slots: the first of them carries the
        // gates of all of them (summed in slot order), the others add nothing
        float g = 0.f;
        bool lead = true;
        for (int jj = 0; jj < a.k; ++jj)
          if (s_sel[t * a.k + jj] == e) {
            g += s_gate[t * a.k + jj];
            lead &= jj >= j;
          }
        if (lead && (unsigned)e < (unsigned)a.E) {
          const float v0 = g * __uint_as_float(uraw[i].x), v1 = g * __uint_as_float(uraw[i].z);
          const uint32_t h = f32x2_to_bf16x2(v0, v1);
          const uint32_t l = f32x2_to_bf16x2(v0 - __uint_as_float(h << 16), v1 - __uint_as_float(h & 0xffff0000u));
          const int kcol = e * a.r + c;
          const int w = ((((t >> 4) * 4 + (kcol >> 5)) * 64 + (t & 15) + 16 * ((kcol & 31) >> 3)) << 2) + ((kcol & 7) >> 1);
          reinterpret_cast<uint32_t*>(fhi)[w] = h;
          reinterpret_cast<uint32_t*>(flo)[w] = l;
        }
      }
    }
  };

  {
    if (d.prev_target > 0) {
      // weights do not depend on the earlier groups: they are in flight during the wait
      static_for<0, NR>([&](auto I) { issue_w(decltype(I)::value, decltype(I)::value); });
      wait_prev_group(ctl, first ? __builtin_amdgcn_readfirstlane(ep_in) : *s_ep, d);
      static_for<0, NR>([&](auto I) { issue_x(decltype(I)::value, decltype(I)::value); });
    } else {
      static_for<0, NR>([&](auto I) { issue(decltype(I)::value, decltype(I)::value); });
    }
    if (first && tid == 0) {
      *s_ep = ep_in;
      arrive(ctl, ep_in);
    }
    store_x(0, 0, 0);
    __syncthreads();
    // full rings while the chunks after them fill the end section (the last
    // ring, or the last two when the expand's operands are prepared early)
    const int v_end = V - (early ? 2 : 1) * NR;
    int v0 = 0;
    for (; v0 < v_end; v0 += NR) {
      static_for<0, NR>([&](auto I) {
        constexpr int i = decltype(I)::value;
        const int v = v0 + i;
        __builtin_amdgcn_sched_barrier(0);
        compute(i, v & 1);
        __builtin_amdgcn_sched_barrier(0);
        issue(i, v + NR);
        __builtin_amdgcn_sched_barrier(0);
        store_x((i + 1) % NR, (v + 1) & 1, v + 1);
        __syncthreads();
      });
    }
    const uint32_t tag_r = launch_tag(*s_ep);
    if (early) {
      // chunks V-6 .. V-4: the routing is requested before the weights of
      // chunk V-3 and staged after chunk V-4; the u pieces it selects are
      // requested before the weights of chunk V-1, so waiting for them never
      // waits for those weights
      static_for<0, NR>([&](auto I) {
        constexpr int i = decltype(I)::value;
        const int v = v0 + i;
        __builtin_amdgcn_sched_barrier(0);
        compute(i, v & 1);
        __builtin_amdgcn_sched_barrier(0);
        if (i == 0) route_issue();
        if (i == NR - 1) {
          stage_route(tag_r);
          frag_zero();
          __syncthreads();
          u_issue();
        }
        __builtin_amdgcn_sched_barrier(0);
        issue(i, v + NR);
        __builtin_amdgcn_sched_barrier(0);
        store_x((i + 1) % NR, (v + 1) & 1, v + 1);
        __syncthreads();
      });
      v0 += NR;
      // chunks V-3 .. V-1: B fragments are requested after chunk V-3 (their
      // registers free by then), the u pieces land in fragment order after
      // chunk V-2
      static_for<0, NR>([&](auto I) {
        constexpr int i = decltype(I)::value;
        const int v = v0 + i;
        __builtin_amdgcn_sched_barrier(0);
        compute(i, v & 1);
        if (i == 0) b_issue();
        if (i == NR - 2) u_scatter(tag_r);
        if (i + 1 < NR) {
          store_x(i + 1, (v + 1) & 1, v + 1);
          __syncthreads();
        }
      });
    } else {
      // the last ring, already issued; an expand's routing (and B fragments)
      // are requested now and staged after its first chunk
      if (expand) route_issue();
      static_for<0, NR>([&](auto I) {
        constexpr int i = decltype(I)::value;
        const int v = v0 + i;
        __builtin_amdgcn_sched_barrier(0);
        compute(i, v & 1);
        if (i + 1 < NR) store_x(i + 1, (v + 1) & 1, v + 1);
        if (i == 0 && expand) {
          stage_route(tag_r);
          if (px) frag_zero();
        }
        if (i + 1 < NR) __syncthreads();
        if (i == 0 && px) u_issue();
      });
    }
  }
  const int ep = *s_ep;
  int* set = ctl_set(ctl, ep);
  const uint32_t tag = launch_tag(ep);

  if (px) {
    if (!early) {
      b_issue();
      u_scatter(tag);
      __syncthreads();
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      if (st * 32 < kcat) {
        const uint4 b = sel4(st * 32 + kg * 8 < kcat, bfr[st]);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          acc[m] = mfma16(fhi[(m * 4 + st) * 64 + lane], b, acc[m]);
          acc[m] = mfma16(flo[(m * 4 + st) * 64 + lane], b, acc[m]);
        }
      }
    }
  } else if (LANEX && expand) {
    // adapter deltas for this wave's 16 rows, lane by lane: the routing of
    // the tile's tokens (adapter and gate of every (token, slot) pair) is in
    // LDS.  A lane's tokens chose at most k adapters, so it needs u only for
    // its own (token, slot) pairs, two slots per pass, scaled by the gate;
    // the operand for adapter e is then picked in registers.  B rows are
    // loaded eight adapters at a time.
    {
      if (!d.dense) wait_geq(ctl, &set[kSetShrinkDone + 32 * d.group], d.shrink_target);
      const size_t slots = upart_slots(a, d);
      const size_t pbytes = (size_t)d.KP * slots * a.r * sizeof(float);  // pair-chunk partials (E > 32)
      const __amdgpu_buffer_rsrc_t rp = rsrc(reinterpret_cast<const char*>(a.u) + proj * pbytes, (uint32_t)pbytes);
      for (int c0 = 0; c0 < a.r; c0 += 32) {
        const int c = c0 + kg * 8;
        const int cc = min(c, a.r - 8);
        for (int jp = 0; jp < a.k; jp += 2) {
          // the lane's adapters and gates of slots jp, jp + 1 (-1: none)
          int sa[MT][2];
          float ga[MT][2];
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const int t = m * 16 + lr, j = jp + q;
              const bool v = j < a.k && t < a.T;
              sa[m][q] = v ? s_sel[t * a.k + j] : -1;
              ga[m][q] = v ? s_gate[t * a.k + j] : 0.f;
            }
          f32x4_t uu[MT][2][2];
          if (d.dense) {
            // tagged pairs [e][t][c] from this launch's A tiles, MU token tiles
            // at a time (all their loads out before any is checked)
            constexpr int MU = 1;
#pragma unroll
            for (int m0 = 0; m0 < MT; m0 += MU) {
              u32x4_v w[MU][2][4];
              uint32_t offv[MU][2];
#pragma unroll
              for (int mm = 0; mm < MU; ++mm)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                  const int e = sa[m0 + mm][q];
                  offv[mm][q] = e >= 0 && c < a.r
                      ? (uint32_t)((((size_t)e * d.t_pad + (m0 + mm) * 16 + lr) * a.r + c) * 8) : kOob;
                  load_u4(w[mm][q], offv[mm][q]);
                }
              int spins = 0;
              while (true) {
                bool good = true;
#pragma unroll
                for (int mm = 0; mm < MU; ++mm)
#pragma unroll
                  for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                      const u32x4_v& lo4 = w[mm][q][2 * i];
                      const u32x4_v& hi4 = w[mm][q][2 * i + 1];
                      uu[m0 + mm][q][i] = f32x4_t{__uint_as_float(lo4.x), __uint_as_float(lo4.z), __uint_as_float(hi4.x),
                                                  __uint_as_float(hi4.z)};
                      if (offv[mm][q] != kOob) good &= lo4.y == tag && lo4.w == tag && hi4.y == tag && hi4.w == tag;
                    }
                if (!retry_tagged(ctl, good, &spins)) break;
#pragma unroll
                for (int mm = 0; mm < MU; ++mm)
#pragma unroll
                  for (int q = 0; q < 2; ++q) load_u4(w[mm][q], offv[mm][q]);
              }
            }
          } else {
            const uint32_t part = (uint32_t)(slots * a.r * sizeof(float));
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
              for (int q = 0; q < 2; ++q) {
                const int t = m * 16 + lr, j = jp + q;
                const bool ok = c < a.r && sa[m][q] >= 0;
                const uint32_t off = ok ? (uint32_t)((((size_t)t * a.k + j) * a.r + cc) * sizeof(float)) : kOob;
                uu[m][q][0] = ld_coh16(rp, off);
                uu[m][q][1] = ld_coh16(rp, ok ? off + 16 : kOob);
                for (int kp = 1; kp < d.KP; ++kp) {
                  uu[m][q][0] += ld_coh16(rp, ok ? off + kp * part : kOob);
                  uu[m][q][1] += ld_coh16(rp, ok ? off + kp * part + 16 : kOob);
                }
              }
          }
          // a token that chose one adapter in both slots gets both gated terms in slot 0
          bool dup[MT];
#pragma unroll
          for (int m = 0; m < MT; ++m) dup[m] = sa[m][0] >= 0 && sa[m][0] == sa[m][1];
          // gated operands of the two slots, split once into (hi, lo) bf16 parts
          uint4 uhi[MT][2], ulo[MT][2];
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const float g0 = ga[m][0], g1 = ga[m][1];
            float v0[8], v1[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              v0[i] = g0 * uu[m][0][0][i];
              v0[4 + i] = g0 * uu[m][0][1][i];
              v1[i] = g1 * uu[m][1][0][i];
              v1[4 + i] = g1 * uu[m][1][1][i];
            }
            if (dup[m]) {
#pragma unroll
              for (int i = 0; i < 8; ++i) v0[i] += v1[i], v1[i] = 0.f;
              sa[m][1] = -1;
            }
            split_hi_lo(v0, uhi[m][0], ulo[m][0]);
            split_hi_lo(v1, uhi[m][1], ulo[m][1]);
          }
          for (int e0 = 0; e0 < a.E; e0 += G) {
            // skip a batch no token of the tile chose; with many adapters, skip
            // single adapters too (with few, all of them are applied branch-free)
            bool any[G];
            bool group = false;
#pragma unroll
            for (int g = 0; g < G; ++g) {
              bool mine = false;
#pragma unroll
              for (int m = 0; m < MT; ++m) mine |= sa[m][0] == e0 + g || sa[m][1] == e0 + g;
              any[g] = __ballot(mine) != 0;
              group |= any[g];
            }
            if (!group) continue;
            uint4 bo[G];
#pragma unroll
            for (int g = 0; g < G; ++g) bo[g] = ld16(Bm + ((size_t)min(e0 + g, a.E - 1) * pd.d_out + row) * a.r + cc);
#pragma unroll
            for (int g = 0; g < G; ++g) {
              if (!d.dense && !any[g]) continue;
              const uint4 b = sel4(c < a.r && e0 + g < a.E, bo[g]);
#pragma unroll
              for (int m = 0; m < MT; ++m) {
                // operand of the slot that chose e0 + g (zero if none), by masks
                const uint32_t k0 = sa[m][0] == e0 + g ? ~0u : 0u, k1 = sa[m][1] == e0 + g ? ~0u : 0u;
                const uint4 hi = make_uint4((uhi[m][0].x & k0) | (uhi[m][1].x & k1), (uhi[m][0].y & k0) | (uhi[m][1].y & k1),
                                            (uhi[m][0].z & k0) | (uhi[m][1].z & k1), (uhi[m][0].w & k0) | (uhi[m][1].w & k1));
                const uint4 lo = make_uint4((ulo[m][0].x & k0) | (ulo[m][1].x & k1), (ulo[m][0].y & k0) | (ulo[m][1].y & k1),
                                            (ulo[m][0].z & k0) | (ulo[m][1].z & k1), (ulo[m][0].w & k0) | (ulo[m][1].w & k1));
                acc[m] = mfma16(hi, b, acc[m]);
                acc[m] = mfma16(lo, b, acc[m]);
              }
            }
          }
        }
      }
    }
  }

  if (S > 1) {
    // split-K: splits 0..S-2 publish their partial tiles as tagged pairs; the
    // last split reads them as they land and sums all S in split order
    constexpr int kWaveBytes = MT * 64 * 32;
    const size_t tile_bytes = (size_t)S * WV * kWaveBytes;
    const __amdgpu_buffer_rsrc_t pr =
        rsrc(reinterpret_cast<char*>(ATILE ? d.partial_a : a.partial) + tile * tile_bytes, (uint32_t)tile_bytes);
    if (!last) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
        st_tagged4(pr, (uint32_t)((split * WV + wave) * kWaveBytes + (m * 64 + lane) * 32), acc[m], tag);
      return;
    }
    // SU splits at a time: all their loads go out before any is checked (a
    // split past S, and this split itself, read zero from past the buffer);
    // a batch with a stale tag is read again; the sums run in split order
    constexpr int SU = MT <= 2 ? 4 : 2;
    f32x4_t tot[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) tot[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += SU) {
      f32x4_t part[SU][MT];
      int spins = 0;
      while (true) {
        u32x4_v raw[SU][MT][2];
#pragma unroll
        for (int i = 0; i < SU; ++i)
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const int s = s0 + i;
            const uint32_t off = s < S && s != split ? (uint32_t)((s * WV + wave) * kWaveBytes + (m * 64 + lane) * 32) : kOob;
            raw[i][m][0] = __builtin_amdgcn_raw_buffer_load_b128(pr, off, 0, kSc1);
            raw[i][m][1] = __builtin_amdgcn_raw_buffer_load_b128(pr, off == kOob ? kOob : off + 16, 0, kSc1);
          }
        bool good = true;
#pragma unroll
        for (int i = 0; i < SU; ++i)
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const u32x4_v& lo4 = raw[i][m][0];
            const u32x4_v& hi4 = raw[i][m][1];
            part[i][m] = f32x4_t{__uint_as_float(lo4.x), __uint_as_float(lo4.z), __uint_as_float(hi4.x), __uint_as_float(hi4.z)};
            const int s = s0 + i;
            if (s < S && s != split) good &= lo4.y == tag && lo4.w == tag && hi4.y == tag && hi4.w == tag;
          }
        if (!retry_tagged(ctl, good, &spins)) break;
      }
#pragma unroll
      for (int i = 0; i < SU; ++i)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const int s = s0 + i;
          if (s < S) tot[m] += s == split ? acc[m] : part[i][m];
        }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = tot[m];
  }

  if (ATILE) {
    // u[proj][e][t][c] for row e*r + c, as tagged pairs (one 8-byte store each)
    if (row0 + lr < n_rows) {
      const int e = (row0 + lr) / a.r, c = (row0 + lr) % a.r;
      unsigned long long* u = reinterpret_cast<unsigned long long*>(a.u) + (((size_t)proj * a.E + e) * d.t_pad) * a.r + c;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t = m * 16 + 4 * kg + v;
          const unsigned long long pair = ((unsigned long long)tag << 32) | __float_as_uint(acc[m][v]);
          if (t < a.T) __hip_atomic_store(&u[(size_t)t * a.r], pair, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    return;
  }

  // store through LDS: lane holds output row row0 + lane%16 of tokens
  // m*16 + 4*(lane/16) + v; the tile goes to the activation buffer the last
  // chunk did not use (free since the barrier of chunk V-2) as [token][TR
  // rows], then each thread writes 16 bytes (8 rows of one token; d_out and
  // ld_y are multiples of 8).  With a residual the tile stays fp32 (both
  // activation buffers, once every wave is done with them) and the residual
  // is added before the one rounding.  A group with an activation stores its
  // tiles device-coherent: the partner tile's item reads them.
  const int tile_row0 = row0 - wave * 16;
  bf16_t* y = static_cast<bf16_t*>(pd.y);
  auto put16 = [&](bf16_t* p, uint4 v) {
    if (d.act || d.release) {
      unsigned long long* q = reinterpret_cast<unsigned long long*>(p);
      __hip_atomic_store(q, (unsigned long long)v.x | ((unsigned long long)v.y << 32), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(q + 1, (unsigned long long)v.z | ((unsigned long long)v.w << 32), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    } else {
      *reinterpret_cast<uint4*>(p) = v;
    }
  };
  if (pd.residual) {
    static_assert(16 * MT * TR * 4 <= 2 * XB * 512 * 2, "an fp32 output tile fits both activation buffers");
    float* yf = reinterpret_cast<float*>(xs);
    const bf16_t* res = static_cast<const bf16_t*>(pd.residual);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int v = 0; v < 4; ++v) yf[(m * 16 + 4 * kg + v) * TR + wave * 16 + lr] = acc[m][v];
    __syncthreads();
    // a group that waited for earlier groups may add one of their outputs:
    // read device-coherent, as its x
    const __amdgpu_buffer_rsrc_t rres = rsrc(res, (uint32_t)((size_t)a.T * pd.ld_y * sizeof(bf16_t)));
    for (int q = tid; q < a.T * (TR / 8); q += NTH) {
      const int t = q / (TR / 8), c8 = (q % (TR / 8)) * 8;
      if (tile_row0 + c8 < pd.d_out) {
        const size_t ro = (size_t)t * pd.ld_y + tile_row0 + c8;
        const uint4 rv = x_coh ? __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                     rres, (uint32_t)(ro * sizeof(bf16_t)), 0, kSc1))
                               : ld16(res + ro);
        const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
        const float* f = &yf[t * TR + c8];
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = f32x2_to_bf16x2(f[2 * i] + __uint_as_float(rw[i] << 16), f[2 * i + 1] + __uint_as_float(rw[i] & 0xffff0000u));
        put16(y + (size_t)t * pd.ld_y + tile_row0 + c8, make_uint4(o[0], o[1], o[2], o[3]));
      }
    }
  } else {
    bf16_t* ys = xs + (size_t)(V & 1) * XB * 512;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int v = 0; v < 4; ++v) ys[(m * 16 + 4 * kg + v) * TR + wave * 16 + lr] = f32_to_bf16(acc[m][v]);
    __syncthreads();
    for (int q = tid; q < a.T * (TR / 8); q += NTH) {
      const int t = q / (TR / 8), c8 = (q % (TR / 8)) * 8;
      if (tile_row0 + c8 < pd.d_out)
        put16(y + (size_t)t * pd.ld_y + tile_row0 + c8, *reinterpret_cast<const uint4*>(&ys[t * TR + c8]));
    }
  }
  int n_done = 1;  // output tiles this item completes
  if (d.act) {
    // (gate, up) pair: the item that finishes second computes m = silu(g) * u
    // for the tile from both rounded tiles and writes it over the gate tile
    __builtin_amdgcn_s_waitcnt(0);  // this tile is at the coherence point before the arrival
    __syncthreads();
    __shared__ int s_pair;
    const int lt = tile - pd.tile_begin;
    if (tid == 0) s_pair = atomicAdd(&d.pair_cnt[lt], 1);
    __syncthreads();
    if (s_pair == 0) return;  // the partner's item completes the pair
    if (tid == 0) __hip_atomic_store(&d.pair_cnt[lt], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const ProjDesc pg = proj_at(a, 0), pu = proj_at(a, 1);
    bf16_t* gy = static_cast<bf16_t*>(pg.y);
    const bf16_t* uy = static_cast<const bf16_t*>(pu.y);
    for (int q = tid; q < a.T * (TR / 8); q += NTH) {
      const int t = q / (TR / 8), c8 = (q % (TR / 8)) * 8;
      if (tile_row0 + c8 < pd.d_out) {
        const unsigned long long* gp = reinterpret_cast<const unsigned long long*>(gy + (size_t)t * pg.ld_y + tile_row0 + c8);
        const unsigned long long* up = reinterpret_cast<const unsigned long long*>(uy + (size_t)t * pu.ld_y + tile_row0 + c8);
        const unsigned long long g0 = __hip_atomic_load(gp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned long long g1 = __hip_atomic_load(gp + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned long long u0 = __hip_atomic_load(up, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned long long u1 = __hip_atomic_load(up + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t gw[4] = {(uint32_t)g0, (uint32_t)(g0 >> 32), (uint32_t)g1, (uint32_t)(g1 >> 32)};
        const uint32_t uw[4] = {(uint32_t)u0, (uint32_t)(u0 >> 32), (uint32_t)u1, (uint32_t)(u1 >> 32)};
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = f32x2_to_bf16x2(silu_mul_f32(__uint_as_float(gw[i] << 16), __uint_as_float(uw[i] << 16)),
                                 silu_mul_f32(__uint_as_float(gw[i] & 0xffff0000u), __uint_as_float(uw[i] & 0xffff0000u)));
        put16(gy + (size_t)t * pg.ld_y + tile_row0 + c8, make_uint4(o[0], o[1], o[2], o[3]));
      }
    }
    n_done = 2;  // both tiles of the pair are final now
  }
  if (d.count_done) {
    // a later group of this launch waits for this tile (and, with release, reads
    // it: then the tile was stored device-coherent, and waiting for the stores
    // puts it at the coherence point before it is counted -- no L2 write-back)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) atomicAdd(&set[kSetGroupDone + 256 * d.group + 32 * (tile & 7)], n_done);
  }
}

// ---------------------------------------------------------------------------
// kernel
// ---------------------------------------------------------------------------
// The view of group gi that the item functions take.
__device__ __forceinline__ DecodeArgs group_view(const StepArgs& st, int gi) {
  const GroupPlan& gp = st.gp[gi];
  DecodeArgs d;
  d.n_route = st.n_route;
  d.n_pre = st.n_pre;
  d.n_shrink = gp.n_shrink;
  d.n_items = gp.n_items;
  d.units_per_proj = gp.units_per_proj;
  d.KP = gp.KP;
  d.dense = st.dense;
  d.atiles_per_proj = gp.atiles_per_proj;
  d.n_atiles = gp.n_atiles;
  d.SA = gp.SA;
  d.shrink_target = gp.shrink_target;
  d.t_pad = st.t_pad;
  d.fused = st.fused;
  d.group = gi;
  d.prev_target = gp.wait_target;
  d.x_acquire = gp.x_acquire;
  d.count_done = gp.count_done;
  d.release = gp.release;
  d.partial_a = gp.partial_a;
  d.act = gp.act;
  d.pair_cnt = gp.pair_cnt;
  d.route_tagged = st.route_tagged;
  return d;
}

// LANEX: the launch has items whose expand cannot take the staged form (more
// than 32 adapters, E*r > 128, or more u pieces than the threads hold); only
// then is the lane-by-lane expand compiled in (its registers would otherwise
// crowd the stream).
template <int MT, bool FUSED, bool LANEX>
__global__ __launch_bounds__(kThreadsOf<MT>, kBlocksPerCuOf<MT>) void decode_kernel(StepArgs st) {
  constexpr int WV = kWavesOf<MT>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[smem_bytes<MT, FUSED>()];
  __shared__ int s_ep, s_loc[2], s_wave_tot[WV], s_bad;
  int* ctl = st.g[0].counters;
  const int tid = threadIdx.x;
  // the epoch is read once per workgroup; backbone items publish it after
  // their first loads are in flight, other items right away
  int ep_in = 0;
  if (tid == 0) ep_in = __hip_atomic_load(&ctl[kCtlEpoch], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  bool first = true;
  // Items in claim order: a workgroup's first item is its block index, each
  // later one comes from a launch-wide counter claimed at the start of the
  // item before (its latency overlaps that item).  Claims are in increasing
  // order, so every item an item waits for has been claimed by a running
  // workgroup -- with static first items, as long as every workgroup of the
  // launch is running, which a launch sharing the GPU with another cannot
  // count on (workgroups go to the XCDs by index, and one XCD may be full);
  // such launches claim every item (claim_all).
  __shared__ int s_next[2];
  int item = blockIdx.x;
  if (st.claim_all) {
    // the workgroup may start after later-numbered ones (another launch holds
    // CUs): it reads the epoch and arrives now, then claims its first item
    if (tid == 0) {
      s_ep = ep_in;
      arrive(ctl, ep_in);
      s_next[1] = atomicAdd(ctl_set(ctl, ep_in) + kSetQueue, 1);
    }
    __syncthreads();
    item = s_next[1];
    first = false;
  }
  for (int iter = 0; item < st.n_items; ++iter) {
    int nxt = st.n_items;  // a launch with no more items than workgroups claims nothing
    if (tid == 0 && (st.claim_all || st.n_items > (int)gridDim.x))
      nxt = (st.claim_all ? 0 : (int)gridDim.x) + atomicAdd(ctl_set(ctl, ep_in) + kSetQueue, 1);
    if (FUSED && item < st.n_pre) {
      if (first) {
        if (tid == 0) {
          s_ep = ep_in;
          arrive(ctl, ep_in);
        }
        __syncthreads();
        first = false;
      }
      int* set = ctl_set(ctl, s_ep);
      if (item < st.n_route) {
        // two router tiles, one per half of the workgroup: top-k and gates of
        // kFusedRouteTokens tokens each (the sums do not depend on the tile size)
        const int half = tid / kRouteThreads;
        const RoutePlan rpl = route_plan(st.pg.E, st.pg.d_in, (int)sizeof(bf16_t));
        route_tile<bf16_t, kFusedRouteTokens>(st.pg, (item * 2 + half) * kFusedRouteTokens, rpl,
                                              reinterpret_cast<float*>(smem) + half * route_lds_floats(rpl, st.pg.E, kFusedRouteTokens),
                                              reinterpret_cast<unsigned long long*>(st.route_tagged), launch_tag(s_ep));
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) atomicAdd(&set[kSetRouteDone], 1);
      } else {
        wait_geq(ctl, &set[kSetRouteDone], st.n_route);
        segment_block<WV>(st.sg, reinterpret_cast<int*>(smem), s_wave_tot, &s_bad);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) atomicAdd(&set[kSetSegDone], 1);
      }
    } else {
      // the group owning this item: li < n_shrink is shrink item li, else
      // backbone item li - n_shrink
      int gi = 0, li = 0;
      for (int g = 0; g < st.n_groups; ++g) {
        const GroupPlan& q = st.gp[g];
        if (item >= q.shrink_begin && item < q.shrink_begin + q.n_shrink) gi = g, li = item - q.shrink_begin;
        if (item >= q.base_begin && item < q.base_begin + q.n_items - q.n_shrink) gi = g, li = q.n_shrink + item - q.base_begin;
      }
      const SgmmArgs& a = st.g[gi];
      const DecodeArgs d = group_view(st, gi);
      if (li < d.n_shrink && d.dense) {
        base_item<MT, false, FUSED, true, LANEX>(a, d, li, reinterpret_cast<bf16_t*>(smem), ctl, &s_ep, first, ep_in);
        first = false;
      } else if (li < d.n_shrink) {
        if (first) {
          if (tid == 0) {
            s_ep = ep_in;
            arrive(ctl, ep_in);
          }
          __syncthreads();
          first = false;
        }
        int* set = ctl_set(ctl, s_ep);
        const int proj = li / d.units_per_proj, w = li % d.units_per_proj;
        const int unit = w / d.KP, kp = w % d.KP;
        float* red = reinterpret_cast<float*>(smem);
        if (FUSED) wait_geq(ctl, &set[kSetSegDone], 1);
        switch ((a.r + 15) >> 4) {
          case 1: shrink_item<1, FUSED, WV>(a, d, proj, unit, kp, red, s_loc, ctl, s_ep); break;
          case 2: shrink_item<2, FUSED, WV>(a, d, proj, unit, kp, red, s_loc, ctl, s_ep); break;
          case 4: shrink_item<4, FUSED, WV>(a, d, proj, unit, kp, red, s_loc, ctl, s_ep); break;
          default: shrink_item<8, FUSED, WV>(a, d, proj, unit, kp, red, s_loc, ctl, s_ep); break;
        }
        // the u stores are device-coherent; wait for them before counting this unit done
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) atomicAdd(&set[kSetShrinkDone + 32 * gi], 1);
      } else {
        const int bi = li - d.n_shrink;
        const int bp = proj_of_tile(a, bi / a.S);
        if (RP_PICK(a, bp, tiled))
          base_item<MT, true, FUSED, false, LANEX>(a, d, bi, reinterpret_cast<bf16_t*>(smem), ctl, &s_ep, first, ep_in);
        else
          base_item<MT, false, FUSED, false, LANEX>(a, d, bi, reinterpret_cast<bf16_t*>(smem), ctl, &s_ep, first, ep_in);
        first = false;
      }
    }
    if (tid == 0) s_next[iter & 1] = nxt;
    __syncthreads();  // LDS is reused by the next item
    item = s_next[iter & 1];
  }
}

template <int MT, bool FUSED>
int resident_per_cu() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  if (cache[dev] > 0) return cache[dev];
  int n = 0;
  int n2 = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<MT, FUSED, false>, kThreadsOf<MT>, 0) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&n2, decode_kernel<MT, FUSED, true>, kThreadsOf<MT>, 0) != hipSuccess)
    n = 1;
  n = std::max(1, std::min(n, n2));
  cache[dev] = n;
  return n;
}

template <bool LANEX>
hipError_t launch_lx(const StepArgs& st, const StepPlan& plan, hipStream_t s) {
  const dim3 grid(plan.grid);
  const int T = st.g[0].T;
  if (st.fused) {
    // routing inside the launch is built for up to two token tiles (T <= 32)
    switch (decode_mt(T)) {
      case 1: decode_kernel<1, true, LANEX><<<grid, kThreadsOf<1>, 0, s>>>(st); break;
      case 2: decode_kernel<2, true, LANEX><<<grid, kThreadsOf<2>, 0, s>>>(st); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (decode_mt(T)) {
      case 1: decode_kernel<1, false, LANEX><<<grid, kThreadsOf<1>, 0, s>>>(st); break;
      case 2: decode_kernel<2, false, LANEX><<<grid, kThreadsOf<2>, 0, s>>>(st); break;
      default: decode_kernel<4, false, LANEX><<<grid, kThreadsOf<4>, 0, s>>>(st); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_t(const StepArgs& st, const StepPlan& plan, hipStream_t s) {
  // the staged expand's conditions (base_item's px), uniform over the launch
  const SgmmArgs& a = st.g[0];
  const bool staged = a.k == 0 || (st.dense && a.E * a.r <= 128 && a.T * a.k * (a.r / 2) <= kUPiecesPerItem);
  return staged ? launch_lx<false>(st, plan, s) : launch_lx<true>(st, plan, s);
}

}  // namespace

int decode_mt(int T) { return T <= 16 ? 1 : T <= 32 ? 2 : 4; }
int decode_chunk_k(int T) { (void)T; return kKC; }
int decode_tile_rows(int T) { return decode_mt(T) >= 4 ? kTileRowsOf<4> : kTileRowsOf<1>; }
int fused_route_tile_tokens() { return 2 * kFusedRouteTokens; }  // tokens per router item

int decode_resident_per_cu(int T, bool fused) {
  switch (decode_mt(T)) {
    case 1: return fused ? resident_per_cu<1, true>() : resident_per_cu<1, false>();
    case 2: return fused ? resident_per_cu<2, true>() : resident_per_cu<2, false>();
    default: return resident_per_cu<4, false>();
  }
}

bool decode_fused_route_supported(int T, int E) { return decode_mt(T) <= 2 && E <= 64; }

hipError_t launch_step(const StepArgs& st, const StepPlan& plan, hipStream_t s) { return launch_t(st, plan, s); }

}  // namespace rp
