// Launch planning for rp_sgmm_fused: which kernel family serves a call, its
// output-row tiling, K splits and workspace layout.
#include <algorithm>

#include "kernels.h"

namespace rp {

namespace {
constexpr size_t kCounterBytes = 65536;                       // reserved, zero between calls
constexpr int kCtlTilesOffset = 16;                           // control words before the tile counters
constexpr int kMaxTileCounters = (int)(kCounterBytes / sizeof(int)) - kCtlTilesOffset;
constexpr int kDecodeTileRows = 32;
constexpr int kDecodeMaxT = 64;
constexpr int kPrefillTileRows = 128;
constexpr int kF32TileRows = 64;

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int split_cap(int T) { return T <= 32 ? 8 : 4; }
}  // namespace

SgmmPlan plan_sgmm(Dtype dt, int n_proj, const int* d_out, int T, int d_in, int E, int r, int k, int n_cu) {
  (void)E;
  SgmmPlan p{};
  p.path = (dt == kF32) ? 0 : (T <= kDecodeMaxT ? 1 : 2);
  p.tile_rows = p.path == 0 ? kF32TileRows : p.path == 1 ? kDecodeTileRows : kPrefillTileRows;
  p.n_tiles = 0;
  for (int i = 0; i < n_proj; ++i) p.n_tiles += (d_out[i] + p.tile_rows - 1) / p.tile_rows;
  p.S = 1;
  p.t_pad = 0;
  p.off_counters = 0;
  if (p.path == 1) {
    // split K only when the row tiles alone do not cover the chip, keeping at
    // least two LDS chunks of K per split
    p.t_pad = 16 * decode_mt(T);
    const int nchunks = (d_in + decode_chunk_k(T) - 1) / decode_chunk_k(T);
    int S = (n_cu + p.n_tiles - 1) / p.n_tiles;
    S = std::max(1, std::min(S, std::min(split_cap(T), nchunks / 2)));
    if (p.n_tiles > kMaxTileCounters) S = 1;
    p.S = S;
  }
  size_t off = kCounterBytes;
  p.off_u = off;
  off = align256(off + (size_t)n_proj * T * k * r * sizeof(float));
  p.off_partial = off;
  if (p.path == 1 && p.S > 1) off = align256(off + (size_t)p.n_tiles * p.S * p.t_pad * kDecodeTileRows * sizeof(float));
  p.bytes = off;
  return p;
}

size_t sgmm_workspace_upper_bound(Dtype dt, int n_proj, int T, int d_in, long long sum_d_out, int E, int r, int k) {
  (void)d_in;
  (void)E;
  size_t b = kCounterBytes;
  b = align256(b + (size_t)n_proj * T * k * r * sizeof(float));
  if (dt == kBF16 && T <= kDecodeMaxT) {
    const size_t tiles = (size_t)(sum_d_out / kDecodeTileRows + n_proj);
    b = align256(b + tiles * split_cap(T) * 16 * decode_mt(T) * kDecodeTileRows * sizeof(float));
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
