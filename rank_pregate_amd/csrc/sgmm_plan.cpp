// Launch planning for the SGMM entry points: which kernel family serves a
// call, output-row tiling, K splits, grid and workspace layout.
#include <algorithm>
#include <functional>
#include <queue>
#include <vector>

#include "kernels.h"

namespace rp {

namespace {
constexpr size_t kCounterBytes = kWorkspaceCounterBytes;
constexpr int kDecodeMaxT = 64;
constexpr int kDenseMaxE = 32;           // decode shrink covers every token per adapter up to this many adapters
constexpr int kMaxSplits = 8;            // decode split-K
constexpr int kMaxKParts = 8;            // decode pair-chunk shrink K parts
constexpr int kShrinkPartBytes = 16384;  // target A bytes per decode pair-chunk shrink unit
constexpr int kSplitCols = 4096;         // decode backbone: about this many K columns per item
constexpr int kMaxSplitsWide = 4;        // decode split-K of 128-row tiles (T > 32): their partial tiles are
                                         // summed two splits per round trip, so more splits cost more than
                                         // their shorter streams save

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int shrink_kparts(int d_in, int r) {
  const int nsteps = (d_in + 31) / 32;
  const long long bytes = (long long)r * d_in * 2;
  int kp = (int)((bytes + kShrinkPartBytes / 2) / kShrinkPartBytes);
  kp = std::max(1, std::min(kp, kMaxKParts));
  while (kp > 1 && nsteps / kp < 2) --kp;  // at least one k-step per wave
  return kp;
}

// dense u and split-K partials are (fp32, tag) pairs: 8 bytes per value
size_t decode_u_bytes(int n_proj, int T, int E, int r, int k, int KP, bool dense) {
  const size_t t_pad = (size_t)16 * decode_mt(T);
  if (dense) return (size_t)n_proj * E * t_pad * r * 8;
  return (size_t)n_proj * KP * T * k * r * sizeof(float);
}

size_t decode_partial_bytes(int n_tiles, int S, int T) {
  return S > 1 ? (size_t)n_tiles * S * 16 * decode_mt(T) * decode_tile_rows(T) * 8 : 0;
}

int a_tiles_per_proj(int E, int r, int T) { return (E * r + decode_tile_rows(T) - 1) / decode_tile_rows(T); }

int decode_tiles(int n_proj, const int* d_out, int T) {
  int n = 0;
  for (int i = 0; i < n_proj; ++i) n += (d_out[i] + decode_tile_rows(T) - 1) / decode_tile_rows(T);
  return n;
}

// One decode group: tiling, splits, items, and its workspace starting at `off`.
// `launch_tiles` counts the backbone tiles of every group sharing the launch.
SgmmPlan plan_decode_group(int n_proj, const int* d_out, int T, int d_in, int E, int r, int k, int n_cu,
                           int launch_tiles, size_t off, int s_mult = 1, int s_fill = 0) {
  SgmmPlan p{};
  p.path = 1;
  p.tile_rows = decode_tile_rows(T);
  p.n_tiles = decode_tiles(n_proj, d_out, T);
  p.t_pad = 16 * decode_mt(T);
  p.dense = E <= kDenseMaxE;
  const int nchunks = (d_in + decode_chunk_k(T) - 1) / decode_chunk_k(T);
  const int s_max = std::max(1, std::min(decode_tile_rows(T) >= 128 ? kMaxSplitsWide : kMaxSplits, nchunks / 2));
  p.KP = 1;
  p.SA = 1;
  int n_shrink = 0;
  if (k > 0 && p.dense) {
    // the shrink as row tiles of [A_0; ..; A_{E-1}], split along K more finely
    // than the backbone so its results are ready before the backbone's
    p.atiles_per_proj = a_tiles_per_proj(E, r, T);
    p.n_atiles = p.atiles_per_proj * n_proj;
    // (up to eight splits at every T: the backbone's cap for 128-row tiles does
    // not apply, the shrink is what the expand waits for)
    p.SA = std::max(1, std::min(kMaxSplits, nchunks / 2));
    n_shrink = p.n_atiles * p.SA;
  } else if (k > 0) {
    p.KP = shrink_kparts(d_in, r);
    p.units_per_proj = (E + (T * k + 15) / 16) * p.KP;
    n_shrink = p.units_per_proj * n_proj;
  }
  // one whole-K item per tile streams best (no partial tiles to hand over);
  // long K is split to about kSplitCols columns per item so items stay alike,
  // and a launch with fewer tiles than CUs splits until every CU has an item
  int S = (d_in + kSplitCols / 2) / kSplitCols;
  S = std::max(S, (n_cu + launch_tiles - 1) / std::max(1, launch_tiles));
  if (s_fill > 0) S = s_fill;
  p.S = std::max(1, std::min(S * s_mult, s_max));
  p.n_shrink = n_shrink;
  p.n_items = n_shrink + p.n_tiles * p.S;
  p.off_u = off;
  off = align256(off + decode_u_bytes(n_proj, T, E, r, k, p.KP, p.dense));
  p.off_partial = off;
  off = align256(off + decode_partial_bytes(p.n_tiles, p.S, T));
  p.off_partial_a = off;
  off = align256(off + decode_partial_bytes(p.n_atiles, p.SA, T));
  p.bytes = off;
  return p;
}
// Estimated duration of one phase of a launch of 128-row tiles, in chunk times
// (one CU streaming one 128 x 128 weight chunk alone): the phase's items handed
// out in claim order to `cap` workgroups, each to the first one free (the
// launch's counter does the same), stretched when more workgroups stream at
// once than the chip's bandwidth feeds at one CU's rate.  Constants from
// single-group launches at 64 tokens, in chunk times: starting an item costs
// about 2, each partial tile its last split reads 2.5, the adapter expand 2,
// and the chip streams about 156 chunks while one CU streams one.
constexpr double kItemStart = 2.0, kPerPartial = 2.5, kExpand = 2.0, kChipChunks = 156.0;

struct PhaseGroup {
  int tiles, nch, S, SA, n_atiles, n_pair_units, KP;
  bool dense, expand;
};

double phase_estimate(const PhaseGroup* pg, int n, int cap) {
  std::vector<double> items;
  double total = 0;
  auto splits = [&](int count, int nch, int S, double last_extra) {
    for (int t = 0; t < count; ++t)
      for (int s = 0; s < S; ++s) {
        const int nc = (int)((long long)nch * (s + 1) / S - (long long)nch * s / S);
        items.push_back(kItemStart + nc + (s == S - 1 ? kPerPartial * (S - 1) + last_extra : 0.0));
        total += nc;
      }
  };
  for (int g = 0; g < n; ++g) {  // shrink items are claimed first
    if (pg[g].dense) splits(pg[g].n_atiles, pg[g].nch, pg[g].SA, 0.0);
    for (int u = 0; u < pg[g].n_pair_units; ++u) items.push_back(kItemStart + 0.25 * pg[g].nch / pg[g].KP);
  }
  for (int g = 0; g < n; ++g) splits(pg[g].tiles, pg[g].nch, pg[g].S, pg[g].expand ? kExpand : 0.0);
  std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
  for (int i = 0; i < cap; ++i) free_at.push(0.0);
  double end = 0;
  for (double d : items) {
    const double t = free_at.top() + d;
    free_at.pop();
    free_at.push(t);
    end = std::max(end, t);
  }
  const double busy = (double)std::min<size_t>(items.size(), (size_t)cap);
  return std::max(end * std::max(1.0, busy / kChipChunks), total / kChipChunks);
}
}  // namespace

SgmmPlan plan_sgmm(Dtype dt, int n_proj, const int* d_out, int T, int d_in, int E, int r, int k, int n_cu,
                   bool fused_route) {
  (void)fused_route;
  if (dt == kBF16 && T <= kDecodeMaxT)
    return plan_decode_group(n_proj, d_out, T, d_in, E, r, k, n_cu, decode_tiles(n_proj, d_out, T), kCounterBytes);
  SgmmPlan p{};
  p.path = (dt == kF32) ? 0 : 2;
  p.tile_rows = p.path == 0 ? f32_tile_rows() : prefill_tile_rows(T);
  p.n_tiles = 0;
  for (int i = 0; i < n_proj; ++i) p.n_tiles += (d_out[i] + p.tile_rows - 1) / p.tile_rows;
  p.S = 1;
  p.off_counters = 0;
  p.off_u = kCounterBytes;
  p.off_partial = align256(p.off_u + (size_t)n_proj * T * k * r * sizeof(float));
  p.bytes = p.off_partial;
  return p;
}

StepPlan plan_step(const StepGroupDesc* groups, int n_groups, int T, int E, int r, int k, int n_cu, bool fused_route) {
  StepPlan sp{};
  sp.n_groups = n_groups;
  sp.n_route = fused_route ? (T + fused_route_tile_tokens() - 1) / fused_route_tile_tokens() : 0;
  sp.n_pre = fused_route ? sp.n_route + 1 : 0;
  size_t off = kCounterBytes;
  int items = sp.n_pre;
  int launch_tiles = 0;
  for (int g = 0; g < n_groups; ++g) launch_tiles += decode_tiles(groups[g].n_proj, groups[g].d_out, T);
  // A launch with more items than its workgroups hands them out in item
  // order, so it ends on the last group's items: that group's K splits are
  // doubled, so the workgroups that run out of work first wait for items of
  // half the length.
  int n_all = sp.n_pre;
  for (int g = 0; g < n_groups; ++g)
    n_all += plan_decode_group(groups[g].n_proj, groups[g].d_out, T, groups[g].d_in, E, r, k, n_cu, launch_tiles,
                               off).n_items;
  const int cap = std::max(1, decode_resident_per_cu(T, fused_route) * n_cu);
  // 128-row tiles (T > 32, one workgroup per CU): a phase -- a group that
  // reads an earlier group's output and the independent groups after it --
  // runs by itself.  When its tiles leave CUs free, its K splits are the
  // candidate with the shortest estimated phase (a few items past the grid
  // would add a round; many splits add partial tiles to sum): group g splits
  // max(its long-K count, m) ways for m = 1 .. the cap, the same m for the
  // whole phase, the fewest splits on a tie.
  int s_fill[kMaxGroups] = {0};
  if (decode_tile_rows(T) >= 128) {
    for (int g0 = 0; g0 < n_groups;) {
      int g1 = g0 + 1;
      while (g1 < n_groups && !groups[g1].x_acquire) ++g1;
      int tiles = 0;
      PhaseGroup pg[kMaxGroups];
      int s_cols[kMaxGroups], s_top[kMaxGroups], m_max = 1;
      for (int g = g0; g < g1; ++g) {
        const SgmmPlan q = plan_decode_group(groups[g].n_proj, groups[g].d_out, T, groups[g].d_in, E, r, k, n_cu,
                                             launch_tiles, off, 1, 1);
        const int nch = (groups[g].d_in + decode_chunk_k(T) - 1) / decode_chunk_k(T);
        tiles += q.n_tiles;
        s_top[g] = std::max(1, std::min(kMaxSplitsWide, nch / 2));
        s_cols[g] = std::min(s_top[g], std::max(1, (groups[g].d_in + kSplitCols / 2) / kSplitCols));
        m_max = std::max(m_max, s_top[g]);
        pg[g - g0] = PhaseGroup{q.n_tiles, nch, 1, q.SA, q.dense ? q.n_atiles : 0,
                                q.dense ? 0 : q.n_shrink, q.KP, q.dense && k > 0, k > 0};
      }
      if (tiles < n_cu) {
        double best = 0;
        int best_m = 0;
        for (int m = 1; m <= m_max; ++m) {
          for (int g = g0; g < g1; ++g) pg[g - g0].S = std::min(s_top[g], std::max(s_cols[g], m));
          const double est = phase_estimate(pg, g1 - g0, cap);
          if (best_m == 0 || est < best) best = est, best_m = m;
        }
        for (int g = g0; g < g1; ++g) s_fill[g] = std::min(s_top[g], std::max(s_cols[g], best_m));
      }
      g0 = g1;
    }
  }
  for (int g = 0; g < n_groups; ++g) {
    const int s_mult = (s_fill[g] == 0 && n_groups > 1 && g == n_groups - 1 && n_all > cap) ? 2 : 1;
    sp.gp[g] = plan_decode_group(groups[g].n_proj, groups[g].d_out, T, groups[g].d_in, E, r, k, n_cu, launch_tiles,
                                 off, s_mult, s_fill[g]);
    off = sp.gp[g].bytes;
  }
  // Item order: routing; the shrink items of every group whose input comes
  // from the call (short, so a CU holding two workgroups pairs a backbone tile
  // with one of them); then group by group, a dependent group's shrink items
  // and every group's backbone items.  An item still only waits for items
  // numbered below it.
  for (int g = 0; g < n_groups; ++g)
    if (!groups[g].x_acquire) {
      sp.shrink_begin[g] = items;
      items += sp.gp[g].n_shrink;
    }
  for (int g = 0; g < n_groups; ++g) {
    if (groups[g].x_acquire) {
      sp.shrink_begin[g] = items;
      items += sp.gp[g].n_shrink;
    }
    sp.base_begin[g] = items;
    items += sp.gp[g].n_items - sp.gp[g].n_shrink;
  }
  sp.off_route = off;
  if (fused_route) off = align256(off + (size_t)T * k * 16);
  sp.bytes = off;
  sp.n_items = items;
  sp.grid = std::min(sp.n_items, cap);
  return sp;
}

size_t step_workspace_upper_bound(const StepGroupDesc* groups, int n_groups, int T, int E, int r, int k) {
  size_t b = kCounterBytes;
  for (int g = 0; g < n_groups; ++g) {
    long long sum_d_out = 0;
    for (int i = 0; i < groups[g].n_proj; ++i) sum_d_out += groups[g].d_out[i];
    const bool dense = E <= kDenseMaxE;
    const int KP = (k > 0 && !dense) ? shrink_kparts(groups[g].d_in, r) : 1;
    b = align256(b + decode_u_bytes(groups[g].n_proj, T, E, r, k, KP, dense));
    const int tiles = (int)(sum_d_out / decode_tile_rows(T) + groups[g].n_proj);
    b = align256(b + decode_partial_bytes(tiles, kMaxSplits, T));
    if (k > 0 && dense) b = align256(b + decode_partial_bytes(a_tiles_per_proj(E, r, T) * groups[g].n_proj, kMaxSplits, T));
  }
  return align256(b + (size_t)T * k * 16);
}

size_t sgmm_workspace_upper_bound(Dtype dt, int n_proj, int T, int d_in, long long sum_d_out, int E, int r, int k) {
  if (dt == kBF16 && T <= kDecodeMaxT) {
    // one group whose widths sum to sum_d_out (the bound only depends on the sum)
    int d_out[kMaxProj];
    for (int i = 0; i < n_proj; ++i) d_out[i] = (int)(sum_d_out / n_proj) + (i < sum_d_out % n_proj ? 1 : 0);
    StepGroupDesc g{n_proj, d_out, d_in, 0};
    return step_workspace_upper_bound(&g, 1, T, E, r, k);
  }
  size_t b = align256(kCounterBytes + (size_t)n_proj * T * k * r * sizeof(float));
  if (dt == kBF16) {  // the prefill GEMM's split-K partials (and fp32 base tiles when the expand runs apart)
    const int tiles_bound = (int)(sum_d_out / prefill_tile_rows(T) + n_proj);
    b += prefill_partial_bytes(tiles_bound, T, prefill_max_splits(d_in));
    if (prefill_split_expand(T, E, r, k)) b += prefill_base_bytes(tiles_bound, T);
  }
  return b;
}

// Long K on few blocks splits the GEMM tiles along K (about 4096 columns a
// split) so their blocks stay short next to the other groups'; a group with
// blocks enough for the chip keeps whole tiles.
int prefill_max_splits(int d_in) { return std::max(1, std::min(8, (d_in + 4095) / 4096)); }
int prefill_splits(int d_in, int n_tiles, int T, int n_cu) {
  if (prefill_units(n_tiles, T) >= 2 * n_cu) return 1;
  return prefill_max_splits(d_in);
}
size_t prefill_partial_bytes(int n_tiles, int T, int S) {  // a tile's partial: its fp32 outputs
  const size_t tile_floats = (size_t)prefill_tile_tokens(T) * prefill_tile_rows(T);
  return S > 1 ? align256((size_t)prefill_units(n_tiles, T) * S * tile_floats * sizeof(float)) : 0;
}

size_t prefill_u_bytes(int n_proj, int T, int r, int k) {
  return align256((size_t)n_proj * T * k * r * sizeof(float));
}

hipError_t launch_sgmm(const SgmmArgs& a, const SgmmPlan& plan, Dtype dt, hipStream_t s) {
  (void)dt;
  if (a.T == 0) return hipSuccess;
  switch (plan.path) {
    case 0: return launch_f32(a, plan, s);
    case 2: return launch_prefill(a, plan, s);
    default: return hipErrorInvalidValue;  // decode groups launch through launch_step
  }
}

}  // namespace rp
