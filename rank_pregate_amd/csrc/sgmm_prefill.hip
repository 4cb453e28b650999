// Prefill-shaped fused SGMM (bf16, T > 64 tokens): the base projection is a
// dense GEMM (bf16 MFMA, 128 or 256 tokens x 128 rows per workgroup,
// LDS-tiled), bound by matrix throughput at thousands of tokens.  The adapter
// deltas (AdaFuse technical summary §2.B) are folded in as extra MFMA steps:
// for every adapter the tile's tokens chose, B_e's rows times the gathered
// rank-r intermediates.  With top-1 the tokens are visited in segment order,
// so a tile meets one or two adapters.  The intermediates come from a separate
// shrink launch, one workgroup per (projection, segment) when segments hold a
// few tokens, else per (projection, chunk of 64 pairs of a segment).
#include <cstdlib>

#include "sgmm_common.h"

namespace rp {
namespace {

// Group of block b among cumulative block counts end[0..n).
__device__ __forceinline__ int group_of_block(const int* end, int n, int b) {
  int g = 0;
  while (g + 1 < n && b >= end[g]) ++g;
  return g;
}

// Shrink blocks go to the groups in order of decreasing d_in (ties: lower
// group first), so the longest blocks are dispatched first and the launch
// does not end on them.  Returns the group; *b = the block's index in it.
__device__ __forceinline__ int shrink_group_of_block(const PrefillStep& ps, int bid, int* b) {
  uint32_t done = 0;
  int g = 0;
  for (int n = 0; n < ps.n_groups; ++n) {
    g = -1;
    for (int h = 0; h < ps.n_groups; ++h)
      if (!((done >> h) & 1u) && (g < 0 || ps.g[h].d_in > ps.g[g].d_in)) g = h;
    done |= 1u << g;
    const int cnt = ps.shrink_end[g] - (g > 0 ? ps.shrink_end[g - 1] : 0);
    if (bid < cnt) break;
    bid -= cnt;
  }
  *b = bid;
  return g;
}

// Waves of a shrink block: chunks of 64 pairs (long segments, few blocks)
// split K eight ways while rank <= 64 leaves the registers for it, other
// blocks four ways.
template <int MTR, int NCT>
constexpr int kShrinkWaves = NCT == 4 && MTR <= 4 ? 8 : 4;

// One shrink block: a chunk of 16*NCT pairs of one segment.  Small segments
// (a few tokens each) take NCT = 1 and keep more K steps of A_e in flight.
template <int MTR, int NCT>
__global__ __launch_bounds__(64 * (kShrinkWaves<MTR, NCT>)) void shrink_bf16(PrefillStep ps) {
  __shared__ __attribute__((aligned(16))) float red[MTR * NCT * 4 * 64];
  __shared__ int s_loc[2];
  int b;
  const int g = shrink_group_of_block(ps, blockIdx.x, &b);
  const SgmmArgs& a = ps.g[g];
  const int proj = b / ps.units, unit = b % ps.units;
  constexpr int U = NCT == 1 ? (MTR == 1 ? 4 : MTR == 2 ? 4 : 2) : (MTR <= 2 ? 2 : 1);  // K steps per load batch
  constexpr int W = kShrinkWaves<MTR, NCT>;
  if (NCT == 1) {
    // small segments: block e takes segment e whole, chunk by chunk (no scan
    // over the segment table to find its work)
    const int n = a.seg_offsets[unit + 1] - a.seg_offsets[unit];
    for (int c = 0; c * 16 < n; ++c) {
      shrink_unit<MTR, NCT, W, U>(a, proj, unit, c, red);
      __syncthreads();  // `red` is read out before the next chunk reduces into it
    }
    return;
  }
  if (threadIdx.x < 64) {
    int e, c;
    locate_chunk(a, unit, 16 * NCT, threadIdx.x, &e, &c);
    if (threadIdx.x == 0) { s_loc[0] = e; s_loc[1] = c; }
  }
  __syncthreads();
  if (s_loc[0] < 0) return;
  shrink_unit<MTR, NCT, W, U>(a, proj, s_loc[0], s_loc[1], red);
}

// ============================================================================
// Stage 2, prefill: 128 or 256 tokens x 128 rows per workgroup, LDS-tiled MFMA GEMM.
// ============================================================================
constexpr int kPB = 128;       // W0 rows per tile
constexpr int kPK = 64;        // K per LDS stage
constexpr int kPLd = kPK + 8;  // padded LDS row (elements)
constexpr int kPR = 2;         // stages whose loads are in flight ahead of the math
constexpr int kPCB = kPK / 32;  // tiled W0 block columns per stage
constexpr int kPBigT = 256;     // from this many tokens, 256-token tiles of eight waves
constexpr int kPNB = 4;        // adapters per batch of B loads in the expand
constexpr int kPUJ = 4;        // slots of a token whose u a lane holds at once (k > 2)
constexpr int kNoAdapter = 0x7fffffff;
// expand as a launch of its own (expand_gather_bf16)
constexpr int kGRows = 64;  // output rows per block
constexpr int kGWaves = 4;
constexpr int kGTok = 64;   // tokens per block
constexpr int kGMaxK = 4;   // top-k the launch serves
constexpr int kCThreads = 256;  // combine: threads per block
constexpr int kCRowsPerBlock = kCThreads / (kPB / 8);  // ... and the (tile, token) rows it takes
static_assert(sizeof(PrefillStep) <= 4096, "kernel argument block too large");

__device__ __forceinline__ int token_at(const SgmmArgs& a, int i) {
  // top-1: walk tokens in segment order so a tile meets few adapters
  return (a.k == 1) ? a.pair_perm[i] : i;
}

// Minimum over the 64 lanes of a wave (all lanes active), with DPP moves
// instead of LDS permutes: within quads, half rows, rows, then row 0 into
// row 1, row 2 into row 3, rows 0-1 into rows 2-3; lane 63 holds the result.
__device__ __forceinline__ int wave_min_int(int v) {
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false));  // row_mirror
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

// Split-K hand-over of an NW-wave GEMM block whose accumulators are acc[2][2]
// (64 floats a lane): every split publishes its fp32 partial tile with
// device-scope stores (chunk c of lane l at ((wave*16 + c)*64 + l)*16 bytes),
// counts its arrival, and the last to arrive sums all S in split order (the
// result does not depend on which finishes last).  Returns false in the splits
// that are not last.  `slot0` numbers the tile's first partial.
template <int NW>
__device__ __forceinline__ bool splitk_reduce(const SgmmArgs& a, size_t slot0, int split, int S, int* cnt,
                                              f32x16_t (&acc)[2][2]) {
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr size_t tile_floats = NW * 64 * 64;
  const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
      a.partial + slot0 * tile_floats, 0, (int)(S * tile_floats * sizeof(float)), 0x00020000);
  constexpr int kSc1 = 1 << 4;
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int c = (f * 2 + g) * 4 + v4;
        const f32x4_t val = {acc[f][g][4 * v4], acc[f][g][4 * v4 + 1], acc[f][g][4 * v4 + 2], acc[f][g][4 * v4 + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, val), pr,
                                               (uint32_t)((split * tile_floats + ((wave * 16 + c) * 64 + lane) * 4) * 4), 0, kSc1);
      }
  __builtin_amdgcn_s_waitcnt(0);  // the partial is in memory before the arrival is counted
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(cnt, 1) == S - 1;
  __syncthreads();
  if (!s_last) return false;
  if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
  f32x16_t tot[2][2];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) tot[f][g][v] = 0.f;
  for (int sp = 0; sp < S; ++sp) {
    if (sp == split) {
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int g = 0; g < 2; ++g) tot[f][g] += acc[f][g];
      continue;
    }
    f32x4_t pv[16];
#pragma unroll
    for (int c = 0; c < 16; ++c)
      pv[c] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                  pr, (uint32_t)((sp * tile_floats + ((wave * 16 + c) * 64 + lane) * 4) * 4), 0, kSc1));
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
#pragma unroll
          for (int e = 0; e < 4; ++e) tot[f][g][4 * v4 + e] += pv[(f * 2 + g) * 4 + v4][e];
  }
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g) acc[f][g] = tot[f][g];
  return true;
}

// Expand: per 32-token block, the distinct adapters its tokens chose, in
// ascending order (found with wave minimums, no memory round trip); a lane
// holds its token's gated u for every slot, so an adapter's token operand is
// picked in registers (slots naming the same adapter summed in slot order)
// and split into bf16 (hi, lo).  B rows go out a batch of kPNB adapters ahead
// of the batch whose MFMAs run.
// The wave's tokens are positions pos0 .. pos0+63 (two 32-token blocks), its
// rows rowb .. rowb+63 (two 32-row blocks); acc[f][g] as the GEMM left it.
template <int PUJ>
__device__ __forceinline__ void expand_adapters(const SgmmArgs& a, const ProjDesc& pd, int proj, int pos0, int rowb,
                                                f32x16_t (&acc)[2][2], uint32_t* emask) {
  const int lane = threadIdx.x & 63, lr = lane & 31, kg = lane >> 5;
  const bf16_t* Bm = static_cast<const bf16_t*>(pd.B);
  const float* ub = a.u + (size_t)proj * a.T * a.k * a.r;
  const int kk = a.k;
  int brow_g[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) brow_g[g] = min(rowb + g * 32 + lr, pd.d_out - 1);
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int pos = pos0 + f * 32 + lr;
    const bool tok_ok = pos < a.T;
    const int t = token_at(a, min(pos, a.T - 1));
    // slots in groups of PUJ (a token naming one adapter in two groups
    // gets its two terms from two passes)
    for (int j0 = 0; j0 < kk; j0 += PUJ) {
      int ej[PUJ];
#pragma unroll
      for (int j = 0; j < PUJ; ++j) {
        const int e = (j0 + j < kk && tok_ok) ? a.topk_idx[t * kk + j0 + j] : -1;
        ej[j] = (e >= 0 && e < a.E) ? e : kNoAdapter;
      }
      // the wave's distinct adapters as a bit mask in LDS (one word per 32
      // adapters); LDS operations of one wave complete in issue order
      const int n_words = (a.E + 31) >> 5;
      for (int w = lane; w < n_words; w += 64) emask[w] = 0u;
#pragma unroll
      for (int j = 0; j < PUJ; ++j)
        if (ej[j] != kNoAdapter) atomicOr(&emask[ej[j] >> 5], 1u << (ej[j] & 31));
    for (int c0 = 0; c0 < a.r; c0 += 16) {
      const int c = c0 + kg * 8;
      const bool cok = c < a.r;
      const int cc = min(c, a.r - 8);
      f32x4_t uj[PUJ][2];
#pragma unroll
      for (int j = 0; j < PUJ; ++j) {
        const bool ok = ej[j] != kNoAdapter && cok;
        const float* p = ub + (size_t)(t * kk + min(j0 + j, kk - 1)) * a.r + cc;
        uj[j][0] = ok ? *reinterpret_cast<const f32x4_t*>(p) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        uj[j][1] = ok ? *reinterpret_cast<const f32x4_t*>(p + 4) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
      // ascending walk over the mask (wave-uniform, scalar)
      int wi = 0;
      uint32_t cur = __builtin_amdgcn_readfirstlane(emask[0]);
      auto next_e = [&]() -> int {
        while (cur == 0u && wi + 1 < n_words) cur = __builtin_amdgcn_readfirstlane(emask[++wi]);
        if (cur == 0u) return kNoAdapter;
        const int e = wi * 32 + __builtin_ctz(cur);
        cur &= cur - 1u;
        return e;
      };
      int beA[kPNB], beB[kPNB];
      uint4 bA[kPNB][2], bB[kPNB][2];
      auto collect = [&](int (&be)[kPNB], uint4 (&bo)[kPNB][2]) -> bool {
#pragma unroll
        for (int i = 0; i < kPNB; ++i) be[i] = next_e();
#pragma unroll
        for (int i = 0; i < kPNB; ++i) {
          const int e = be[i] == kNoAdapter ? 0 : be[i];
#pragma unroll
          for (int g = 0; g < 2; ++g) bo[i][g] = ld16(Bm + ((size_t)e * pd.d_out + brow_g[g]) * a.r + cc);
        }
        return be[0] != kNoAdapter;
      };
      auto apply = [&](const int (&be)[kPNB], const uint4 (&bo)[kPNB][2]) {
#pragma unroll
        for (int i = 0; i < kPNB; ++i) {
          if (be[i] == kNoAdapter) continue;
          float v[8];
#pragma unroll
          for (int m = 0; m < 8; ++m) v[m] = 0.f;
#pragma unroll
          for (int j = 0; j < PUJ; ++j)
            if (ej[j] == be[i]) {
#pragma unroll
              for (int m = 0; m < 4; ++m) v[m] += uj[j][0][m], v[4 + m] += uj[j][1][m];
            }
          uint4 hi, lo;
          split_hi_lo(v, hi, lo);
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const uint4 b = sel4(cok, bo[i][g]);
            acc[f][g] = mfma32(hi, b, acc[f][g]);
            acc[f][g] = mfma32(lo, b, acc[f][g]);
          }
        }
      };
      bool haveA = collect(beA, bA);
      while (haveA) {
        const bool haveB = collect(beB, bB);
        apply(beA, bA);
        if (!haveB) break;
        haveA = collect(beA, bA);
        apply(beB, bB);
      }
    }
    }
  }
}

// Expand for top-1 with r <= 64 (RC = r/16 rank-column pieces): a token has
// one adapter, so a lane loads its token's gated u for every rank column at
// once, and for each distinct adapter of the 32-token block (ascending, by
// wave minimums) the B rows of every rank column in one batch; the next
// adapter's B rows are in flight while the current one's MFMAs run.  Rank
// columns past r are zero on both sides.
template <int RC>
__device__ __forceinline__ void expand_top1(const SgmmArgs& a, const ProjDesc& pd, int proj, int pos0, int rowb,
                                            f32x16_t (&acc)[2][2]) {
  const int lane = threadIdx.x & 63, lr = lane & 31, kg = lane >> 5;
  const bf16_t* Bm = static_cast<const bf16_t*>(pd.B);
  const float* ub = a.u + (size_t)proj * a.T * a.r;
  int brow_g[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) brow_g[g] = min(rowb + g * 32 + lr, pd.d_out - 1);
  bool cok[RC];
  int cc[RC];
#pragma unroll
  for (int q = 0; q < RC; ++q) {
    const int c = q * 16 + kg * 8;
    cok[q] = c < a.r;
    cc[q] = min(c, a.r - 8);
  }
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    __builtin_amdgcn_sched_barrier(0);  // keeps the second block's loads after the first's MFMAs
    const int pos = pos0 + f * 32 + lr;
    const int t = token_at(a, min(pos, a.T - 1));
    const int e0 = pos < a.T ? a.topk_idx[t] : -1;
    const int mine = (e0 >= 0 && e0 < a.E) ? e0 : kNoAdapter;
    f32x4_t u[RC][2];
#pragma unroll
    for (int q = 0; q < RC; ++q) {
      const float* p = ub + (size_t)t * a.r + cc[q];
      u[q][0] = *reinterpret_cast<const f32x4_t*>(p);
      u[q][1] = *reinterpret_cast<const f32x4_t*>(p + 4);
    }
    bool todo = mine != kNoAdapter;
    auto next_e = [&]() -> int {
      const int e = wave_min_int(todo ? mine : kNoAdapter);
      if (mine == e) todo = false;
      return e;
    };
    uint4 bA[RC][2], bB[RC][2];
    auto load_b = [&](int e, uint4 (&bo)[RC][2]) {
      const int ee = e == kNoAdapter ? 0 : e;
#pragma unroll
      for (int q = 0; q < RC; ++q)
#pragma unroll
        for (int g = 0; g < 2; ++g) bo[q][g] = ld16(Bm + ((size_t)ee * pd.d_out + brow_g[g]) * a.r + cc[q]);
    };
    auto apply = [&](int e, const uint4 (&bo)[RC][2]) {
#pragma unroll
      for (int q = 0; q < RC; ++q) {
        float v[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          v[m] = (mine == e && cok[q]) ? u[q][0][m] : 0.f;
          v[4 + m] = (mine == e && cok[q]) ? u[q][1][m] : 0.f;
        }
        uint4 hi, lo;
        split_hi_lo(v, hi, lo);
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const uint4 b = sel4(cok[q], bo[q][g]);
          acc[f][g] = mfma32(hi, b, acc[f][g]);
          acc[f][g] = mfma32(lo, b, acc[f][g]);
        }
      }
    };
    int eA = next_e();
    if (eA == kNoAdapter) continue;
    load_b(eA, bA);
    while (true) {
      const int eB = next_e();
      if (eB != kNoAdapter) load_b(eB, bB);
      apply(eA, bA);
      if (eB == kNoAdapter) break;
      eA = next_e();
      if (eA != kNoAdapter) load_b(eA, bA);
      apply(eB, bB);
      if (eA == kNoAdapter) break;
    }
  }
}

// Blocks b and b + 8 share an XCD (b % 8).  With K split, the splits and
// token tiles of a row tile are blocks q*8 + x for consecutive q, so they run
// on one XCD at about the same time and all but the first read of the W0 tile
// hit its L2.  Without splits, an XCD's 32 CUs take 8 of its row tiles x 4
// token tiles at a time: each weight tile is read by 4 of them and each token
// tile by 8, so a phase fetches 8 weight tiles and 4 token tiles (one row
// tile x all 16 token tiles of 4096 tokens fetched 2 weight and 16 token
// tiles per 32 blocks: prefill_mlp 1.56 -> 1.34 ms).
// FAST: every projection of the launch is in the tiled W0 order and every
// d_in is a multiple of kPK, so a stage never reaches past d_in (no clamps or
// selects) and a wave's W0 block row is wave-uniform: its block offsets are
// scalar arithmetic.
// BM: tokens per tile, 128 (four waves, two blocks a CU) or 256 (eight waves,
// one block a CU; each W0 byte fetched serves twice the tokens).  Waves are
// BM/64 x 2 tiles of 64 tokens x 64 rows.
// EXP: the expand form: 1 top-1 routing with r <= 64 (expand_top1), 2 two
// slots per token, 4 up to four slots per pass.
template <bool FAST, int BM, int EXP>
__global__ __launch_bounds__(2 * BM, BM == 128 ? 2 : 1) void prefill_bf16(PrefillStep ps) {
  constexpr int NT = 2 * BM, NW = NT / 64;
  constexpr int kPPA = BM * kPK / 8 / NT;   // 16-byte pieces per thread and stage: A
  constexpr int kPPB = kPB * kPK / 8 / NT;  // and B
  // operand double buffers, reused for the output tile at the end
  __shared__ __attribute__((aligned(16))) bf16_t smem_p[2 * (BM + kPB) * kPLd];
  constexpr bool TOP1 = EXP == 1;
  __shared__ uint32_t s_emask[TOP1 ? 1 : NW][TOP1 ? 1 : kMaxEWords];  // expand: a wave's adapters
  auto As = reinterpret_cast<bf16_t(*)[BM][kPLd]>(smem_p);
  auto Bs = reinterpret_cast<bf16_t(*)[kPB][kPLd]>(smem_p + 2 * BM * kPLd);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = group_of_block(ps.block_end, ps.n_groups, blockIdx.x);
  const SgmmArgs& a = ps.g[grp];
  const int n_tok_tiles = ps.n_tok_tiles, S = a.S;
  // block q*8 + x of the group: row tile (q / (ntt*S))*8 + x, K split and
  // token tile from q % (ntt*S), so every split and token tile of a row tile
  // shares an XCD
  const int q = (blockIdx.x - (grp > 0 ? ps.block_end[grp - 1] : 0)) >> 3;  // groups start at multiples of 8
  const int per = n_tok_tiles * S;
  int tile = (q / per) * 8 + (blockIdx.x & 7);
  int split = (q % per) / n_tok_tiles, tt = q % n_tok_tiles;
  if (S == 1 && n_tok_tiles > 1) {
    // super-blocks of RB row tiles of this XCD; inside one, phases of TB token
    // tiles x the super-block's row tiles run together (RB * TB = 32 blocks, one
    // per CU of the XCD), so a phase fetches RB weight tiles and TB token tiles
    constexpr int RB = 8, TB = 4;
    const int n_rt = (a.n_tiles + 7) / 8;
    const int sb = q / (RB * n_tok_tiles), within = q % (RB * n_tok_tiles);
    const int rb_cnt = min(RB, n_rt - sb * RB);
    const int phase = within / (rb_cnt * TB), in_phase = within - phase * rb_cnt * TB;
    tile = (sb * RB + in_phase % rb_cnt) * 8 + (blockIdx.x & 7);
    tt = phase * TB + in_phase / rb_cnt;
    split = 0;
  }
  if (tile >= a.n_tiles) return;
  const int proj = proj_of_tile(a, tile);
  const ProjDesc pd = proj_at(a, proj);
  const int row0 = (tile - pd.tile_begin) * kPB;
  const int i0 = tt * BM;  // position in token order
  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  const bf16_t* W0 = static_cast<const bf16_t*>(pd.W0);

  // global -> LDS, 16-byte pieces.  A (tokens): piece c -> token row
  // c/(kPK/8), columns 8*(c%(kPK/8)).  B (W0 rows): row-major the same; tiled,
  // piece c is lane c%64 of block c/64 = (row block (c/64)%8, block column
  // (c/64)/8), which holds row 16*((c/64)%8) + (c%64)%16, columns
  // 32*((c/64)/8) + 8*((c%64)/16).  Block c/64 = wave + NW*i is uniform over a
  // wave.
  const bf16_t* gA[kPPA];
  const bf16_t* gB[kPPB];
  int lrow[kPPA], lk[kPPA], brow[kPPB], bk[kPPB], tblk[kPPB];
  const int nkb = a.d_in / 32, n_rb = pd.d_out / 16;
#pragma unroll
  for (int i = 0; i < kPPA; ++i) {
    const int c = tid + i * NT;
    lrow[i] = c / (kPK / 8);
    lk[i] = (c % (kPK / 8)) * 8;
    const int pos = min(i0 + lrow[i], a.T - 1);
    gA[i] = x + (size_t)token_at(a, pos) * a.ld_x + lk[i];
  }
#pragma unroll
  for (int i = 0; i < kPPB; ++i) {
    const int c = tid + i * NT;
    if (pd.tiled) {
      const int blk = c / 64;
      tblk[i] = min(row0 / 16 + blk % 8, n_rb - 1);
      brow[i] = (blk % 8) * 16 + (c % 64) % 16;
      bk[i] = (blk / 8) * 32 + ((c % 64) / 16) * 8;
      gB[i] = W0 + (c % 64) * 8;
    } else {
      brow[i] = c / (kPK / 8);
      bk[i] = (c % (kPK / 8)) * 8;
      tblk[i] = 0;
      gB[i] = W0 + (size_t)min(row0 + brow[i], pd.d_out - 1) * a.d_in + bk[i];
    }
  }
  const int nk_all = (a.d_in + kPK - 1) / kPK;
  const int kb = (int)((long long)nk_all * split / S);
  const int nk = (int)((long long)nk_all * (split + 1) / S) - kb;  // this split's stages, >= 1
  // Stages go global -> registers kPR stages ahead of the math, then to the
  // LDS double buffer one stage ahead.  Loads are never masked (stages past
  // the end re-read the last one); columns past d_in are zeroed on the way to
  // LDS.  Stage j of the split is stage kb + j of K.
  uint4 ra[kPR][kPPA], rb[kPR][kPPB];
  // FAST: tiled block row of piece i, scalar
  int rbw[kPPB];
#pragma unroll
  for (int i = 0; i < kPPB; ++i)
    rbw[i] = __builtin_amdgcn_readfirstlane(min(row0 / 16 + (wave + NW * i) % 8, n_rb - 1));
  const bf16_t* Wl = W0 + lane * 8;
  auto gload = [&](int slot, int j) {
    const int kt = kb + min(j, nk - 1);
    if (FAST) {
#pragma unroll
      for (int i = 0; i < kPPA; ++i) ra[slot][i] = ld16(gA[i] + kt * kPK);
#pragma unroll
      for (int i = 0; i < kPPB; ++i) rb[slot][i] = ld16(Wl + w0_block_offset(rbw[i], kt * kPCB + NW * i / 8, n_rb, nkb));
      return;
    }
#pragma unroll
    for (int i = 0; i < kPPA; ++i) ra[slot][i] = ld16(gA[i] + min(kt * kPK, a.d_in - 8 - lk[i]));
#pragma unroll
    for (int i = 0; i < kPPB; ++i) {
      if (pd.tiled)
        rb[slot][i] = ld16(gB[i] + w0_block_offset(tblk[i], min(kt * kPCB + bk[i] / 32, nkb - 1), n_rb, nkb));
      else
        rb[slot][i] = ld16(gB[i] + min(kt * kPK, a.d_in - 8 - bk[i]));
    }
  };
  auto lstore = [&](int slot, int buf, int j) {
#pragma unroll
    for (int i = 0; i < kPPA; ++i) {
      const bool ok = FAST || (kb + j) * kPK + lk[i] < a.d_in;
      *reinterpret_cast<uint4*>(&As[buf][lrow[i]][lk[i]]) = sel4(ok, ra[slot][i]);
    }
#pragma unroll
    for (int i = 0; i < kPPB; ++i) {
      const bool ok = FAST || (kb + j) * kPK + bk[i] < a.d_in;
      *reinterpret_cast<uint4*>(&Bs[buf][brow[i]][bk[i]]) = sel4(ok, rb[slot][i]);
    }
  };

  const int wm = wave % (BM / 64), wn = wave / (BM / 64);  // wave tile: tokens wm*64.., rows wn*64..
  const int lr = lane & 31, kg = lane >> 5;
  f32x16_t acc[2][2];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[f][g][v] = 0.f;
  // MFMA fragments, double-buffered: those of the next 16 columns of the
  // stage are read from LDS while the MFMAs of the current ones run
  uint4 fa[2][2], fb[2][2];
  auto fragload = [&](int buf, int kk, int p) {
#pragma unroll
    for (int f = 0; f < 2; ++f) fa[p][f] = *reinterpret_cast<const uint4*>(&As[buf][wm * 64 + f * 32 + lr][kk + kg * 8]);
#pragma unroll
    for (int g = 0; g < 2; ++g) fb[p][g] = *reinterpret_cast<const uint4*>(&Bs[buf][wn * 64 + g * 32 + lr][kk + kg * 8]);
  };
  auto compute = [&](int cur) {
    fragload(cur, 0, 0);
    static_for<0, kPK / 16>([&](auto Q) {
      constexpr int q = decltype(Q)::value;
      if (q + 1 < kPK / 16) fragload(cur, (q + 1) * 16, (q + 1) & 1);
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int g = 0; g < 2; ++g) acc[f][g] = mfma32(fa[q & 1][f], fb[q & 1][g], acc[f][g]);
    });
  };

  static_for<0, kPR>([&](auto I) { gload(decltype(I)::value, decltype(I)::value); });
  lstore(0, 0, 0);
  __syncthreads();
  // full rings while every stage has kPR successors, ring slots by static index
  int kt0 = 0;
  for (; kt0 + kPR < nk; kt0 += kPR) {
    static_for<0, kPR>([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int kt = kt0 + i;
      compute(kt & 1);
      gload(i, kt + kPR);
      lstore((i + 1) % kPR, (kt + 1) & 1, kt + 1);
      __syncthreads();
    });
  }
  // the last 1..kPR stages, already issued
  static_for<0, kPR>([&](auto I) {
    constexpr int i = decltype(I)::value;
    const int kt = kt0 + i;
    if (kt < nk) {
      compute(kt & 1);
      if (kt + 1 < nk) lstore((i + 1) % kPR, (kt + 1) & 1, kt + 1);
      __syncthreads();
    }
  });

  if (S > 1 && !splitk_reduce<NW>(a, ((size_t)tile * n_tok_tiles + tt) * S, split, S,
                              a.counters + (size_t)tile * n_tok_tiles + tt, acc))
    return;
  if (EXP == 0) {
    // the expand runs as a launch of its own: store the fp32 base tile as
    // [token][128 rows] (token positions in the tile's order, T <= BM)
    float* bt = a.base + (size_t)tile * a.T * kPB;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int pos = i0 + wm * 64 + f * 32 + 8 * (v >> 2) + 4 * kg + (v & 3);
          if (pos < a.T) bt[(size_t)pos * kPB + wn * 64 + g * 32 + lr] = acc[f][g][v];
        }
    return;
  }
  if (TOP1)
    expand_top1<4>(a, pd, proj, i0 + wm * 64, row0 + wn * 64, acc);
  else if (a.k > 0)
    expand_adapters<EXP == 2 ? 2 : kPUJ>(a, pd, proj, i0 + wm * 64, row0 + wn * 64, acc, s_emask[wave]);

  // a residual is added in fp32 before the one rounding: lane entry v of
  // acc[f][g] is token position wm*64 + f*32 + 8*(v/4) + 4*kg + v%4, row
  // wn*64 + g*32 + lr of the tile
  if (pd.residual) {
    const bf16_t* res = static_cast<const bf16_t*>(pd.residual);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int row = row0 + wn * 64 + g * 32 + lr;
      if (row >= pd.d_out) continue;
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int pos = i0 + wm * 64 + f * 32 + 8 * (v >> 2) + 4 * kg + (v & 3);
          if (pos < a.T) acc[f][g][v] += bf16_to_f32(res[(size_t)token_at(a, pos) * pd.ld_y + row]);
        }
    }
  }
  // store through LDS: the tile as [token][128 rows] bf16, then 16-byte row
  // pieces per (token, 8 rows); d_out and ld_y are multiples of 8
  bf16_t* ys = smem_p;
  static_assert(2 * (BM + kPB) * kPLd >= BM * kPB, "output tile must fit the operand buffers");
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        ys[(wm * 64 + f * 32 + 8 * (v >> 2) + 4 * kg + (v & 3)) * kPB + wn * 64 + g * 32 + lr] = f32_to_bf16(acc[f][g][v]);
  __syncthreads();
  bf16_t* y = static_cast<bf16_t*>(pd.y);
  for (int c = tid; c < BM * (kPB / 8); c += NT) {
    const int tl = c / (kPB / 8), r8 = (c % (kPB / 8)) * 8;
    const int pos = i0 + tl;
    if (pos < a.T && row0 + r8 < pd.d_out)
      *reinterpret_cast<uint4*>(y + (size_t)token_at(a, pos) * pd.ld_y + row0 + r8) = *reinterpret_cast<const uint4*>(&ys[tl * kPB + r8]);
  }
}

}  // namespace

int prefill_tile_rows(int T) { (void)T; return kPB; }
int prefill_tile_tokens(int T) { return T >= kPBigT ? 256 : 128; }
// (row tile, token tile) units of one group's GEMM, the blocks of one K split
int prefill_units(int n_tiles, int T) {
  const int bm = prefill_tile_tokens(T);
  return (n_tiles + 7) / 8 * 8 * ((T + bm - 1) / bm);
}
int prefill_group_blocks(int n_tiles, int T) { return prefill_units(n_tiles, T); }
int prefill_shrink_nct(int T, int E, int k) { return (long long)T * k <= 16LL * E ? 1 : 4; }
bool prefill_split_expand(int T, int E, int r, int k) {
  return k >= 2 && k <= kGMaxK && r <= 32 && T <= kPBigT && prefill_shrink_nct(T, E, k) == 1;
}
size_t prefill_base_bytes(int n_tiles, int T) { return 2 * (size_t)n_tiles * T * kPB * sizeof(float); }
int prefill_expand_blocks(int n_tiles, int T) {
  // 64-row blocks rounded up to whole sets of 8 (one per XCD), times the token blocks
  return (2 * n_tiles + 7) / 8 * 8 * ((T + kGTok - 1) / kGTok);
}
int prefill_combine_blocks(int n_tiles, int T) {
  return (int)(((long long)n_tiles * T + kCRowsPerBlock - 1) / kCRowsPerBlock);
}
int prefill_shrink_units(int T, int E, int k) {
  if (prefill_shrink_nct(T, E, k) == 1) return E;  // one block per segment
  return E + (T * k + 63) / 64;
}

template <int BM>
void launch_gemm(const PrefillStep& ps, bool fast, int exp, dim3 grid, hipStream_t s) {
  if (fast) {
    if (exp == 0) prefill_bf16<true, BM, 0><<<grid, 2 * BM, 0, s>>>(ps);
    else if (exp == 1) prefill_bf16<true, BM, 1><<<grid, 2 * BM, 0, s>>>(ps);
    else if (exp == 2) prefill_bf16<true, BM, 2><<<grid, 2 * BM, 0, s>>>(ps);
    else prefill_bf16<true, BM, 4><<<grid, 2 * BM, 0, s>>>(ps);
  } else {
    if (exp == 0) prefill_bf16<false, BM, 0><<<grid, 2 * BM, 0, s>>>(ps);
    else if (exp == 1) prefill_bf16<false, BM, 1><<<grid, 2 * BM, 0, s>>>(ps);
    else if (exp == 2) prefill_bf16<false, BM, 2><<<grid, 2 * BM, 0, s>>>(ps);
    else prefill_bf16<false, BM, 4><<<grid, 2 * BM, 0, s>>>(ps);
  }
}

// ----------------------------------------------------------------------------
// The expand as a launch of its own, for top-k >= 2 over many adapters (most
// segments one to three tokens long): per token, not per segment.  A block
// takes 64 output rows (lane = row) of one projection and kGTok tokens; each
// of its waves walks its own tokens and, for token t, sums the k terms
// B_e(t,j)[rows, :] . u[t*k + j, :] (u already carries the gate; slots in
// order j = 0..k-1, each rank sum in rank order) into the fp32 delta tile,
// laid out as the GEMM's base tile.  It needs the routing and u but not the
// GEMM, so it can run beside it; combine_bf16 then rounds base + delta
// (+ residual) once to bf16.  There is no segment walk, no staging and no
// barrier after the first: a pair's 64 B rows are 64 x r contiguous bf16 that
// its wave reads straight from memory, G tokens' worth at a time.  The
// kGTok-token blocks of one 64-row block run on one XCD one after another
// (blockIdx % 8 picks the XCD), so a B chunk that several of them read comes
// from that XCD's L2 after the first.  Every output has one owner, so the
// result does not depend on timing.
// ----------------------------------------------------------------------------
template <int R, int KK>
__global__ __launch_bounds__(64 * kGWaves) void expand_gather_bf16(PrefillStep ps) {
  constexpr int TW = kGTok / kGWaves;                       // tokens per wave
  constexpr int G = 128 / (KK * R) > 0 ? 128 / (KK * R) : 1;  // tokens whose B rows are in flight at once
  static_assert(TW % G == 0, "token groups must tile a wave's tokens");
  __shared__ __attribute__((aligned(16))) float U[kGTok * KK * R];
  __shared__ int I[kGTok * KK];
  const int tid = threadIdx.x, rr = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = group_of_block(ps.expand_end, ps.n_groups, blockIdx.x);
  const SgmmArgs& a = ps.g[grp];
  const int b = blockIdx.x - (grp > 0 ? ps.expand_end[grp - 1] : 0);
  const int T = a.T, k = a.k;
  const int n_tc = (T + kGTok - 1) / kGTok;
  const int tc = (b >> 3) % n_tc, rb = ((b >> 3) / n_tc) * 8 + (b & 7);
  if (rb >= 2 * a.n_tiles) return;
  const int tile = rb >> 1;
  const int proj = proj_of_tile(a, tile);
  const ProjDesc pd = proj_at(a, proj);
  const int row0 = (tile - pd.tile_begin) * kPB + (rb & 1) * kGRows;
  if (row0 >= pd.d_out) return;  // the second half of a ragged last tile
  const int row = row0 + rr, prow = min(row, pd.d_out - 1);
  const int t0 = tc * kGTok, nt = min(kGTok, T - t0);

  // gated u and adapter indices of the block's tokens
  const float4* ug = reinterpret_cast<const float4*>(a.u + ((size_t)proj * T + t0) * k * R);
  for (int i = tid; i < nt * k * R / 4; i += 64 * kGWaves) reinterpret_cast<float4*>(U)[i] = ug[i];
  for (int i = tid; i < nt * k; i += 64 * kGWaves) I[i] = a.topk_idx[(size_t)t0 * k + i];
  __syncthreads();

  const bf16_t* Bm = static_cast<const bf16_t*>(pd.B);
  float* dt = a.delta + (size_t)tile * T * kPB + (rb & 1) * kGRows + rr;
  const int tw_end = min((w + 1) * TW, nt);
  for (int g0 = w * TW; g0 < tw_end; g0 += G) {
    // loads of G tokens first (a token past the wave's last repeats its last,
    // and is never stored), then their sums
    int ev[G][KK];
    uint4 bq[G][KK][R / 8];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int tl = min(g0 + i, tw_end - 1);
#pragma unroll
      for (int j = 0; j < KK; ++j) {
        ev[i][j] = -1;
        if (j < k) {
          const int e = __builtin_amdgcn_readfirstlane(I[tl * k + j]);
          if (e >= 0 && e < a.E) {  // out-of-range indices add nothing (no segment holds them)
            ev[i][j] = e;
            const bf16_t* src = Bm + ((size_t)e * pd.d_out + prow) * R;
#pragma unroll
            for (int c = 0; c < R / 8; ++c) bq[i][j][c] = ld16(src + 8 * c);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int tl = g0 + i;
      if (tl >= tw_end) break;
      float v = 0.f;
#pragma unroll
      for (int j = 0; j < KK; ++j) {
        if (ev[i][j] < 0) continue;
        const float4* up = reinterpret_cast<const float4*>(&U[(tl * k + j) * R]);
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < R / 8; ++c) {
          const uint32_t wv[4] = {bq[i][j][c].x, bq[i][j][c].y, bq[i][j][c].z, bq[i][j][c].w};
          const float4 u0 = up[2 * c], u1 = up[2 * c + 1];
          const float uv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc = fmaf(__uint_as_float(wv[q] << 16), uv[2 * q], acc);
            acc = fmaf(__uint_as_float(wv[q] & 0xffff0000u), uv[2 * q + 1], acc);
          }
        }
        v += acc;
      }
      dt[(size_t)(t0 + tl) * kPB] = v;
    }
  }
}

// y[t, rows] = bf16(base + delta (+ residual)) for the tiles of the split
// expand: a thread takes 8 rows of one (tile, token), 16-byte loads and stores.
__global__ __launch_bounds__(kCThreads) void combine_bf16(PrefillStep ps) {
  const int grp = group_of_block(ps.combine_end, ps.n_groups, blockIdx.x);
  const SgmmArgs& a = ps.g[grp];
  const int b = blockIdx.x - (grp > 0 ? ps.combine_end[grp - 1] : 0);
  const int q = b * kCRowsPerBlock + (int)threadIdx.x / (kPB / 8);  // tile * T + token
  if (q >= a.n_tiles * a.T) return;
  const int tile = q / a.T, t = q % a.T;
  const int proj = proj_of_tile(a, tile);
  const ProjDesc pd = proj_at(a, proj);
  const int c = ((int)threadIdx.x % (kPB / 8)) * 8;
  const int row = (tile - pd.tile_begin) * kPB + c;
  if (row >= pd.d_out) return;  // d_out % 8 == 0: a thread's 8 rows are all in or all out
  const float* bp = a.base + (size_t)q * kPB + c;
  const float* dp = a.delta + (size_t)q * kPB + c;
  const float4 b0 = *reinterpret_cast<const float4*>(bp), b1 = *reinterpret_cast<const float4*>(bp + 4);
  const float4 d0 = *reinterpret_cast<const float4*>(dp), d1 = *reinterpret_cast<const float4*>(dp + 4);
  float v[8] = {b0.x + d0.x, b0.y + d0.y, b0.z + d0.z, b0.w + d0.w, b1.x + d1.x, b1.y + d1.y, b1.z + d1.z, b1.w + d1.w};
  const size_t o = (size_t)t * pd.ld_y + row;
  if (pd.residual) {
    const uint4 rq = ld16(static_cast<const bf16_t*>(pd.residual) + o);
    const uint32_t rw[4] = {rq.x, rq.y, rq.z, rq.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] += __uint_as_float(rw[i] << 16);
      v[2 * i + 1] += __uint_as_float(rw[i] & 0xffff0000u);
    }
  }
  uint32_t ow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    ow[i] = f32x2_to_bf16x2(v[2 * i], v[2 * i + 1]);
  *reinterpret_cast<uint4*>(static_cast<bf16_t*>(pd.y) + o) = uint4{ow[0], ow[1], ow[2], ow[3]};
}

hipError_t launch_prefill_shrink(const PrefillStep& ps, hipStream_t s) {
  const SgmmArgs& a0 = ps.g[0];
  if (a0.T == 0) return hipSuccess;
  if (a0.k > 0) {
    const dim3 g(ps.shrink_end[ps.n_groups - 1]);
    const bool small = prefill_shrink_nct(a0.T, a0.E, a0.k) == 1;
    static_assert(kShrinkWaves<4, 4> == 8 && kShrinkWaves<8, 4> == 4 && kShrinkWaves<1, 1> == 4, "launch sizes");
    switch ((a0.r + 15) >> 4) {
      case 1: small ? shrink_bf16<1, 1><<<g, 256, 0, s>>>(ps) : shrink_bf16<1, 4><<<g, 512, 0, s>>>(ps); break;
      case 2: small ? shrink_bf16<2, 1><<<g, 256, 0, s>>>(ps) : shrink_bf16<2, 4><<<g, 512, 0, s>>>(ps); break;
      case 4: small ? shrink_bf16<4, 1><<<g, 256, 0, s>>>(ps) : shrink_bf16<4, 4><<<g, 512, 0, s>>>(ps); break;
      default: small ? shrink_bf16<8, 1><<<g, 256, 0, s>>>(ps) : shrink_bf16<8, 4><<<g, 256, 0, s>>>(ps); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_prefill_gemm(const PrefillStep& ps, hipStream_t s) {
  const SgmmArgs& a0 = ps.g[0];
  if (a0.T == 0) return hipSuccess;
  bool fast = true;  // every projection tiled, every d_in a multiple of kPK
  for (int g = 0; g < ps.n_groups; ++g) {
    fast = fast && ps.g[g].d_in % kPK == 0;
    for (int p = 0; p < ps.g[g].n_proj; ++p) fast = fast && ps.g[g].proj[p].tiled;
  }
  const dim3 grid(ps.block_end[ps.n_groups - 1]);
  if (ps.n_tok_tiles != (a0.T + prefill_tile_tokens(a0.T) - 1) / prefill_tile_tokens(a0.T))
    return hipErrorInvalidValue;  // token tiles planned for another tile size
  const int exp = ps.split_expand ? 0 : a0.k == 1 && a0.r <= 64 ? 1 : a0.k <= 2 ? 2 : 4;
  if (prefill_tile_tokens(a0.T) == 256)
    launch_gemm<256>(ps, fast, exp, grid, s);
  else
    launch_gemm<128>(ps, fast, exp, grid, s);
  return hipGetLastError();
}

hipError_t launch_prefill_expand(const PrefillStep& ps, hipStream_t s) {
  const SgmmArgs& a0 = ps.g[0];
  if (a0.T == 0) return hipSuccess;
  if (ps.split_expand) {
    const dim3 xg(ps.expand_end[ps.n_groups - 1]);
    const bool k2 = a0.k <= 2;  // k <= kGMaxK (prefill_split_expand)
    switch (a0.r) {             // r in {8, 16, 32} (prefill_split_expand)
      case 8: k2 ? expand_gather_bf16<8, 2><<<xg, 64 * kGWaves, 0, s>>>(ps) : expand_gather_bf16<8, 4><<<xg, 64 * kGWaves, 0, s>>>(ps); break;
      case 16: k2 ? expand_gather_bf16<16, 2><<<xg, 64 * kGWaves, 0, s>>>(ps) : expand_gather_bf16<16, 4><<<xg, 64 * kGWaves, 0, s>>>(ps); break;
      default: k2 ? expand_gather_bf16<32, 2><<<xg, 64 * kGWaves, 0, s>>>(ps) : expand_gather_bf16<32, 4><<<xg, 64 * kGWaves, 0, s>>>(ps); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_prefill_combine(const PrefillStep& ps, hipStream_t s) {
  if (ps.g[0].T == 0 || !ps.split_expand) return hipSuccess;
  combine_bf16<<<dim3(ps.combine_end[ps.n_groups - 1]), kCThreads, 0, s>>>(ps);
  return hipGetLastError();
}

hipError_t launch_prefill_step(const PrefillStep& ps, hipStream_t s) {
  hipError_t e = launch_prefill_shrink(ps, s);
  if (e == hipSuccess) e = launch_prefill_gemm(ps, s);
  if (e == hipSuccess) e = launch_prefill_expand(ps, s);
  if (e == hipSuccess) e = launch_prefill_combine(ps, s);
  return e;
}

hipError_t launch_prefill(const SgmmArgs& a, const SgmmPlan& plan, hipStream_t s) {
  PrefillStep ps{};
  ps.g[0] = a;
  ps.g[0].n_tiles = plan.n_tiles;
  ps.n_groups = 1;
  ps.n_tok_tiles = (a.T + prefill_tile_tokens(a.T) - 1) / prefill_tile_tokens(a.T);
  ps.units = prefill_shrink_units(a.T, a.E, a.k);
  ps.shrink_end[0] = ps.units * a.n_proj;
  ps.block_end[0] = prefill_group_blocks(plan.n_tiles, a.T);
  return launch_prefill_step(ps, s);
}

}  // namespace rp
