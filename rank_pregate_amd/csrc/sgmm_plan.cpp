// Launch planning for rp_sgmm_fused / rp_route_sgmm_fused: which kernel family
// serves a call, its output-row tiling, K splits, grid and workspace layout.
#include <algorithm>
#include <cstdlib>

#include "kernels.h"

namespace rp {

namespace {
constexpr size_t kCounterBytes = 65536;  // reserved control region at the start of the workspace
constexpr int kCtlTilesOffset = 4096;    // control words before the split-K tile counters
constexpr int kMaxTileCounters = (int)(kCounterBytes / sizeof(int)) - kCtlTilesOffset;
constexpr int kDecodeTileRows = 32;
constexpr int kDecodeMaxT = 64;
constexpr int kPrefillTileRows = 128;
constexpr int kF32TileRows = 64;
constexpr int kDenseMaxE = 32;      // decode shrink covers every token per adapter up to this many adapters
constexpr int kMaxSplits = 8;       // decode split-K
constexpr int kMaxKParts = 8;       // decode shrink K parts
constexpr int kShrinkPartBytes = 32768;  // target A bytes per decode shrink unit

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int shrink_kparts(int d_in, int r) {
  const int nsteps = (d_in + 31) / 32;
  const long long bytes = (long long)r * d_in * 2;
  int kp = (int)((bytes + kShrinkPartBytes / 2) / kShrinkPartBytes);
  kp = std::max(1, std::min(kp, kMaxKParts));
  while (kp > 1 && nsteps / kp < 2) --kp;  // at least one k-step per wave
  return kp;
}

size_t decode_u_bytes(int n_proj, int T, int E, int r, int k, int KP, bool dense) {
  const size_t t_pad = (size_t)16 * decode_mt(T);
  const size_t slots = dense ? (size_t)E * t_pad : (size_t)T * k;
  return (size_t)n_proj * KP * slots * r * sizeof(float);
}

size_t decode_partial_bytes(int n_tiles, int S, int T) {
  return S > 1 ? (size_t)n_tiles * S * 16 * decode_mt(T) * kDecodeTileRows * sizeof(float) : 0;
}
}  // namespace

SgmmPlan plan_sgmm(Dtype dt, int n_proj, const int* d_out, int T, int d_in, int E, int r, int k, int n_cu,
                   bool fused_route) {
  SgmmPlan p{};
  p.path = (dt == kF32) ? 0 : (T <= kDecodeMaxT ? 1 : 2);
  p.tile_rows = p.path == 0 ? kF32TileRows : p.path == 1 ? kDecodeTileRows : kPrefillTileRows;
  p.n_tiles = 0;
  for (int i = 0; i < n_proj; ++i) p.n_tiles += (d_out[i] + p.tile_rows - 1) / p.tile_rows;
  p.S = 1;
  p.off_counters = 0;
  size_t off = kCounterBytes;
  p.off_u = off;
  if (p.path != 1) {
    off = align256(off + (size_t)n_proj * T * k * r * sizeof(float));
    p.off_partial = off;
    p.bytes = off;
    return p;
  }
  // decode: every item of the launch is resident at once when it fits; the
  // row tiles are split along K until the chip holds about as many items as
  // it can run together
  p.t_pad = 16 * decode_mt(T);
  p.dense = E <= kDenseMaxE;
  p.KP = k > 0 ? shrink_kparts(d_in, r) : 1;
  p.units_per_proj = k > 0 ? (p.dense ? E : E + (T * k + 15) / 16) * p.KP : 0;
  p.n_route = fused_route ? (T + route_tile_tokens(E) - 1) / route_tile_tokens(E) : 0;
  p.n_pre = fused_route ? p.n_route + 1 : 0;
  const int n_shrink = p.units_per_proj * n_proj;
  const int cap = std::max(1, decode_resident_per_cu(T, fused_route) * n_cu);
  const int nchunks = (d_in + decode_chunk_k(T) - 1) / decode_chunk_k(T);
  int s_max = std::max(1, std::min(kMaxSplits, nchunks / 2));
  if (p.n_tiles > kMaxTileCounters) s_max = 1;
  int S = (cap - p.n_pre - n_shrink) / p.n_tiles;
  if (const char* env = std::getenv("RP_DECODE_SPLITS")) {  // tuning override
    const int v = std::atoi(env);
    if (v > 0) S = v;
  }
  p.S = std::max(1, std::min(S, s_max));
  p.n_items = p.n_pre + n_shrink + p.n_tiles * p.S;
  p.grid = std::min(p.n_items, cap);
  off = align256(off + decode_u_bytes(n_proj, T, E, r, k, p.KP, p.dense));
  p.off_partial = off;
  off = align256(off + decode_partial_bytes(p.n_tiles, p.S, T));
  p.bytes = off;
  return p;
}

size_t sgmm_workspace_upper_bound(Dtype dt, int n_proj, int T, int d_in, long long sum_d_out, int E, int r, int k) {
  size_t b = kCounterBytes;
  if (dt == kBF16 && T <= kDecodeMaxT) {
    const int KP = k > 0 ? shrink_kparts(d_in, r) : 1;
    b = align256(b + decode_u_bytes(n_proj, T, E, r, k, KP, E <= kDenseMaxE));
    const int tiles = (int)(sum_d_out / kDecodeTileRows + n_proj);
    b = align256(b + decode_partial_bytes(tiles, kMaxSplits, T));
  } else {
    b = align256(b + (size_t)n_proj * T * k * r * sizeof(float));
  }
  return b;
}

hipError_t launch_sgmm(const SgmmArgs& a, const SgmmPlan& plan, Dtype dt, hipStream_t s) {
  (void)dt;
  if (a.T == 0) return hipSuccess;
  switch (plan.path) {
    case 0: return launch_f32(a, plan, s);
    case 1: return launch_decode(a, plan, s);
    default: return launch_prefill(a, plan, s);
  }
}

}  // namespace rp
