// C ABI of the library: argument validation, launch planning and dispatch.
// Every check runs on the host before anything is queued; no exception leaves
// this file.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/rank_pregate.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

rp_status fail(rp_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

rp_status hip_fail(const char* where, hipError_t e) {
  return fail(RP_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t dsize(rp_dtype dt) { return dt == RP_BF16 ? 2 : 4; }

bool valid_dtype(rp_dtype dt) { return dt == RP_F32 || dt == RP_BF16; }

// Compute units of the current device, cached per device id.
int cu_count(int* out) {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= 0 && dev < 64 && cache[dev] > 0) {
    *out = cache[dev];
    return 0;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
  if (dev >= 0 && dev < 64) cache[dev] = n;
  *out = n;
  return 0;
}

constexpr int64_t kIntMax = 0x7fffffff;

}  // namespace

extern "C" {

const char* rp_last_error(void) { return g_last_error.c_str(); }

int rp_abi_version(void) { return RP_ABI_VERSION; }

rp_status rp_pregate(const void* x, int64_t T, int64_t d_in, int64_t ld_x, const void* Wg, int64_t E, int32_t k,
                     rp_dtype dt, int32_t* topk_idx, float* topk_gate, float* logits_or_null, hipStream_t stream) {
  g_last_error.clear();
  if (!valid_dtype(dt)) return fail(RP_ERR_INVALID_ARG, "rp_pregate: unknown dtype %d", (int)dt);
  if (T < 0 || T > kIntMax) return fail(RP_ERR_INVALID_ARG, "rp_pregate: T=%lld out of range", (long long)T);
  if (E < 1 || E > RP_MAX_E) return fail(RP_ERR_INVALID_ARG, "rp_pregate: E=%lld not in [1, %d]", (long long)E, RP_MAX_E);
  if (k < 1 || k > RP_MAX_K || k > E)
    return fail(RP_ERR_INVALID_ARG, "rp_pregate: k=%d not in [1, min(E, %d)]", k, RP_MAX_K);
  const int64_t vec = dt == RP_BF16 ? 8 : 4;
  if (d_in < 1 || d_in % vec != 0 || d_in > kIntMax)
    return fail(RP_ERR_INVALID_ARG, "rp_pregate: d_in=%lld must be a positive multiple of %lld", (long long)d_in,
                (long long)vec);
  if (ld_x < d_in || (ld_x * (int64_t)dsize(dt)) % 16 != 0 || ld_x > kIntMax)
    return fail(RP_ERR_INVALID_ARG, "rp_pregate: ld_x=%lld must be >= d_in with ld_x*elem a multiple of 16 bytes",
                (long long)ld_x);
  if (T * E > (int64_t)1 << 40) return fail(RP_ERR_INVALID_ARG, "rp_pregate: T*E too large");
  if (T == 0) return RP_OK;
  if (!x || !Wg || !topk_idx || !topk_gate) return fail(RP_ERR_INVALID_ARG, "rp_pregate: null pointer");
  if (!aligned(x, 16) || !aligned(Wg, 16)) return fail(RP_ERR_INVALID_ARG, "rp_pregate: x and Wg must be 16-byte aligned");
  if (!aligned(topk_idx, 4) || !aligned(topk_gate, 4) || (logits_or_null && !aligned(logits_or_null, 4)))
    return fail(RP_ERR_INVALID_ARG, "rp_pregate: outputs must be 4-byte aligned");
  rp::PregateArgs a;
  a.x = x;
  a.T = (int)T;
  a.d_in = (int)d_in;
  a.ld_x = (int)ld_x;
  a.Wg = Wg;
  a.E = (int)E;
  a.k = k;
  a.dt = dt == RP_BF16 ? rp::kBF16 : rp::kF32;
  a.topk_idx = topk_idx;
  a.topk_gate = topk_gate;
  a.logits = logits_or_null;
  hipError_t e = rp::launch_pregate(a, stream);
  return e == hipSuccess ? RP_OK : hip_fail("rp_pregate launch", e);
}

size_t rp_segment_workspace_size(int64_t T, int32_t k, int64_t E) {
  (void)T;
  (void)k;
  (void)E;
  return 256;
}

rp_status rp_segment(const int32_t* topk_idx, int64_t T, int32_t k, int64_t E, int32_t* seg_offsets,
                     int32_t* pair_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  if (T < 0 || k < 0 || k > RP_MAX_K) return fail(RP_ERR_INVALID_ARG, "rp_segment: T=%lld / k=%d out of range", (long long)T, k);
  if (E < 1 || E > RP_MAX_E) return fail(RP_ERR_INVALID_ARG, "rp_segment: E=%lld not in [1, %d]", (long long)E, RP_MAX_E);
  if (T * (int64_t)k > kIntMax) return fail(RP_ERR_INVALID_ARG, "rp_segment: T*k must be < 2^31");
  if (!seg_offsets || !ws) return fail(RP_ERR_INVALID_ARG, "rp_segment: null pointer");
  if (T * k > 0 && (!topk_idx || !pair_perm)) return fail(RP_ERR_INVALID_ARG, "rp_segment: null pointer");
  if (!aligned(seg_offsets, 4) || (topk_idx && !aligned(topk_idx, 4)) || (pair_perm && !aligned(pair_perm, 4)))
    return fail(RP_ERR_INVALID_ARG, "rp_segment: pointers must be 4-byte aligned");
  if (!aligned(ws, 4)) return fail(RP_ERR_WORKSPACE, "rp_segment: workspace must be 4-byte aligned");
  if (ws_bytes < rp_segment_workspace_size(T, k, E))
    return fail(RP_ERR_WORKSPACE, "rp_segment: workspace %zu bytes, need %zu", ws_bytes, rp_segment_workspace_size(T, k, E));
  rp::SegmentArgs a;
  a.topk_idx = topk_idx;
  a.n_pairs = (int)(T * k);
  a.k = k;
  a.E = (int)E;
  a.seg_offsets = seg_offsets;
  a.pair_perm = pair_perm;
  a.err_count = static_cast<int*>(ws);
  hipError_t e = rp::launch_segment(a, stream);
  return e == hipSuccess ? RP_OK : hip_fail("rp_segment launch", e);
}

size_t rp_sgmm_workspace_size(int32_t n_proj, int64_t T, int64_t d_in, int64_t sum_d_out, int64_t E, int64_t r,
                              int32_t k, rp_dtype dt) {
  if (!valid_dtype(dt) || n_proj < 1 || n_proj > RP_MAX_PROJ || T < 0 || T > kIntMax || d_in < 1 || sum_d_out < 1 ||
      E < 1 || E > RP_MAX_E || k < 0 || k > RP_MAX_K || k > E)
    return 0;
  if (!(r == 8 || r == 16 || r == 32 || r == 64 || r == 128)) return 0;
  if (T * k * r * n_proj > ((int64_t)1 << 34)) return 0;
  return rp::sgmm_workspace_upper_bound(dt == RP_BF16 ? rp::kBF16 : rp::kF32, n_proj, (int)T, (int)d_in,
                                        (long long)sum_d_out, (int)E, (int)r, k);
}

}  // extern "C"

namespace {

// Argument checks shared by rp_sgmm_fused and rp_route_sgmm_fused (no device calls).
rp_status check_sgmm(const char* fn, const rp_proj* projs, int32_t n_proj, const void* x, int64_t T, int64_t d_in,
                     int64_t ld_x, int64_t E, int64_t r, int32_t k, rp_dtype dt, void* ws) {
  if (!valid_dtype(dt)) return fail(RP_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
  if (!projs || n_proj < 1 || n_proj > RP_MAX_PROJ)
    return fail(RP_ERR_INVALID_ARG, "%s: n_proj=%d not in [1, %d]", fn, n_proj, RP_MAX_PROJ);
  if (T < 0 || T > kIntMax) return fail(RP_ERR_INVALID_ARG, "%s: T=%lld out of range", fn, (long long)T);
  if (E < 1 || E > RP_MAX_E) return fail(RP_ERR_INVALID_ARG, "%s: E=%lld not in [1, %d]", fn, (long long)E, RP_MAX_E);
  if (k < 0 || k > RP_MAX_K || k > E)
    return fail(RP_ERR_INVALID_ARG, "%s: k=%d not in [0, min(E, %d)]", fn, k, RP_MAX_K);
  if (!(r == 8 || r == 16 || r == 32 || r == 64 || r == 128))
    return fail(RP_ERR_UNSUPPORTED, "%s: rank r=%lld not in {8,16,32,64,128}", fn, (long long)r);
  const int64_t es = (int64_t)dsize(dt);
  const int64_t vec = dt == RP_BF16 ? 8 : 4;
  if (d_in < 1 || d_in % vec != 0 || d_in > kIntMax)
    return fail(RP_ERR_INVALID_ARG, "%s: d_in=%lld must be a positive multiple of %lld", fn, (long long)d_in,
                (long long)vec);
  if (ld_x < d_in || (ld_x * es) % 16 != 0 || ld_x > kIntMax)
    return fail(RP_ERR_INVALID_ARG, "%s: ld_x=%lld must be >= d_in with ld_x*elem a multiple of 16 bytes", fn,
                (long long)ld_x);
  if (T * k * r * n_proj > ((int64_t)1 << 34)) return fail(RP_ERR_INVALID_ARG, "%s: T*k*r too large", fn);
  for (int p = 0; p < n_proj; ++p) {
    const rp_proj& q = projs[p];
    if (q.d_out < 8 || q.d_out % 8 != 0 || q.d_out > kIntMax)
      return fail(RP_ERR_INVALID_ARG, "%s: projection %d: d_out=%lld must be a positive multiple of 8", fn, p,
                  (long long)q.d_out);
    if (q.ld_y < q.d_out || (q.ld_y * es) % 16 != 0 || q.ld_y > kIntMax)
      return fail(RP_ERR_INVALID_ARG, "%s: projection %d: ld_y=%lld must be >= d_out with ld_y*elem a "
                  "multiple of 16 bytes", fn, p, (long long)q.ld_y);
    if (T > 0 && (!q.W0 || !q.y || (k > 0 && (!q.A || !q.B))))
      return fail(RP_ERR_INVALID_ARG, "%s: projection %d: null pointer", fn, p);
    if (!aligned(q.W0, 16) || !aligned(q.A, 16) || !aligned(q.B, 16) || !aligned(q.y, 16))
      return fail(RP_ERR_INVALID_ARG, "%s: projection %d: W0, A, B, y must be 16-byte aligned", fn, p);
    if ((int64_t)q.d_out * d_in > ((int64_t)1 << 40) || E * r * std::max<int64_t>(d_in, q.d_out) > ((int64_t)1 << 40))
      return fail(RP_ERR_INVALID_ARG, "%s: projection %d too large", fn, p);
    if (q.reserved != 0 || (q.w0_layout != RP_W0_ROWS && q.w0_layout != RP_W0_TILED))
      return fail(RP_ERR_INVALID_ARG, "%s: projection %d: unknown w0_layout %d / reserved %d", fn, p,
                  q.w0_layout, q.reserved);
    if (q.w0_layout == RP_W0_TILED && (dt != RP_BF16 || q.d_out % 16 != 0 || d_in % 32 != 0))
      return fail(RP_ERR_UNSUPPORTED, "%s: projection %d: the tiled W0 layout needs bf16, d_out %% 16 == 0 "
                  "and d_in %% 32 == 0", fn, p);
  }
  if (T == 0) return RP_OK;
  if (!x || !aligned(x, 16)) return fail(RP_ERR_INVALID_ARG, "%s: x must be non-null and 16-byte aligned", fn);
  if (!ws) return fail(RP_ERR_WORKSPACE, "%s: null workspace", fn);
  if (!aligned(ws, 256)) return fail(RP_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  return RP_OK;
}

// Kernel view of one projection group (routing pointers and workspace views
// are filled by the caller).
void fill_group(rp::SgmmArgs* a, const rp_proj* projs, int n_proj, const void* x, int64_t T, int64_t d_in,
                int64_t ld_x, int64_t E, int64_t r, int32_t k, int tile_rows) {
  int tile = 0;
  for (int p = 0; p < RP_MAX_PROJ; ++p) {
    const int q = p < n_proj ? p : n_proj - 1;  // unused slots repeat the last projection
    a->proj[p].W0 = projs[q].W0;
    a->proj[p].A = projs[q].A;
    a->proj[p].B = projs[q].B;
    a->proj[p].y = projs[q].y;
    a->proj[p].d_out = (int)projs[q].d_out;
    a->proj[p].ld_y = (int)projs[q].ld_y;
    a->proj[p].tile_begin = tile;
    a->proj[p].tiled = projs[q].w0_layout == RP_W0_TILED;
    if (p < n_proj) tile += ((int)projs[p].d_out + tile_rows - 1) / tile_rows;
  }
  a->n_proj = n_proj;
  a->x = x;
  a->T = (int)T;
  a->d_in = (int)d_in;
  a->ld_x = (int)ld_x;
  a->E = (int)E;
  a->r = (int)r;
  a->k = k;
}

// Word of the workspace's control region that receives the count of
// out-of-range router indices when a call computes the routing.
constexpr size_t kSegErrWord = 64;

struct Routing {
  const void* Wg;  // non-null: compute the routing from the first group's x
  int32_t* idx;
  float* gate;
  int32_t* off;
  int32_t* perm;
};

bool decode_shape(rp_dtype dt, int64_t T) { return dt == RP_BF16 && T <= 64; }

// Workspace bytes a validated call needs.
size_t groups_workspace_bytes(const rp_group* gs, int n_groups, int64_t T, int64_t E, int64_t r, int32_t k,
                              rp_dtype dt) {
  size_t need = 0;
  if (decode_shape(dt, T)) {
    for (int g0 = 0; g0 < n_groups; g0 += rp::kMaxGroups) {
      const int ng = std::min(rp::kMaxGroups, n_groups - g0);
      rp::StepGroupDesc desc[rp::kMaxGroups];
      int d_out[rp::kMaxGroups][RP_MAX_PROJ];
      for (int i = 0; i < ng; ++i) {
        for (int p = 0; p < gs[g0 + i].n_proj; ++p) d_out[i][p] = (int)gs[g0 + i].projs[p].d_out;
        desc[i] = rp::StepGroupDesc{gs[g0 + i].n_proj, d_out[i], (int)gs[g0 + i].d_in, 0};
      }
      need = std::max(need, rp::step_workspace_upper_bound(desc, ng, (int)T, (int)E, (int)r, k));
    }
  } else if (dt == RP_BF16) {
    // every group's u side by side (a launch pair runs several groups)
    need = rp::kWorkspaceCounterBytes;
    for (int g = 0; g < n_groups; ++g) {
      int64_t sum = 0;
      for (int p = 0; p < gs[g].n_proj; ++p) sum += gs[g].projs[p].d_out;
      const int tiles_bound = (int)(sum / rp::prefill_tile_rows((int)T) + gs[g].n_proj);
      need += rp::prefill_u_bytes(gs[g].n_proj, (int)T, (int)r, k) +
              rp::prefill_partial_bytes(tiles_bound, (int)T, rp::prefill_max_splits((int)gs[g].d_in));
    }
  } else {
    for (int g = 0; g < n_groups; ++g) {
      int64_t sum = 0;
      for (int p = 0; p < gs[g].n_proj; ++p) sum += gs[g].projs[p].d_out;
      need = std::max(need, rp::sgmm_workspace_upper_bound(rp::kF32, gs[g].n_proj, (int)T, (int)gs[g].d_in, sum,
                                                           (int)E, (int)r, k));
    }
  }
  return need;
}

// Runs the groups of a validated call in order on `stream`.  Decode shapes go
// through the multi-group decode kernel, up to kMaxGroups groups per launch;
// routing to compute runs inside the first launch when T <= 32, otherwise as
// router and segmentation launches of its own first.
rp_status run_groups(const char* fn, const rp_group* gs, int n_groups, int64_t T, int64_t E, int64_t r, int32_t k,
                     rp_dtype dt, const Routing& rt, void* ws, size_t ws_bytes, hipStream_t stream) {
  int n_cu = 0;
  if (cu_count(&n_cu) != 0) return fail(RP_ERR_HIP, "%s: cannot query the current device", fn);
  const rp::Dtype rdt = dt == RP_BF16 ? rp::kBF16 : rp::kF32;
  const bool decode = decode_shape(dt, T);
  char* w = static_cast<char*>(ws);
  rp::PregateArgs pg{};
  rp::SegmentArgs sg{};
  const bool route = rt.Wg != nullptr;
  if (route) {
    pg.x = gs[0].x;
    pg.T = (int)T;
    pg.d_in = (int)gs[0].d_in;
    pg.ld_x = (int)gs[0].ld_x;
    pg.Wg = rt.Wg;
    pg.E = (int)E;
    pg.k = k;
    pg.dt = rdt;
    pg.topk_idx = rt.idx;
    pg.topk_gate = rt.gate;
    pg.logits = nullptr;
    sg.topk_idx = rt.idx;
    sg.n_pairs = (int)(T * k);
    sg.k = k;
    sg.E = (int)E;
    sg.seg_offsets = rt.off;
    sg.pair_perm = rt.perm;
    sg.err_count = reinterpret_cast<int*>(ws) + kSegErrWord;
  }
  const bool fuse_route = route && decode && rp::decode_fused_route_supported((int)T, (int)E);
  if (route && !fuse_route) {
    hipError_t e = rp::launch_pregate(pg, stream);
    if (e == hipSuccess) e = rp::launch_segment(sg, stream);
    if (e != hipSuccess) return hip_fail(fn, e);
  }
  if (!decode && dt == RP_BF16) {
    // groups batched into launch pairs (shrink, then GEMM); a group that reads
    // an earlier group's output starts a new batch, so the launch boundary
    // orders the data
    for (int g0 = 0; g0 < n_groups;) {
      int ng = 1;
      while (g0 + ng < n_groups && ng < rp::kMaxGroups && !gs[g0 + ng].x_from_call) ++ng;
      rp::PrefillStep ps{};
      ps.n_groups = ng;
      ps.n_tok_tiles = (int)((T + rp::prefill_tile_tokens((int)T) - 1) / rp::prefill_tile_tokens((int)T));
      ps.units = rp::prefill_shrink_units((int)T, (int)E, k);
      size_t off = rp::kWorkspaceCounterBytes;
      int shrink_blocks = 0, gemm_blocks = 0, counters = 0;
      for (int i = 0; i < ng; ++i) {
        const rp_group& g = gs[g0 + i];
        int d_out[RP_MAX_PROJ];
        for (int p = 0; p < g.n_proj; ++p) d_out[p] = (int)g.projs[p].d_out;
        const rp::SgmmPlan plan =
            rp::plan_sgmm(rdt, g.n_proj, d_out, (int)T, (int)g.d_in, (int)E, (int)r, k, n_cu, false);
        rp::SgmmArgs& a = ps.g[i];
        fill_group(&a, g.projs, g.n_proj, g.x, T, g.d_in, g.ld_x, E, r, k, plan.tile_rows);
        a.topk_idx = rt.idx;
        a.topk_gate = rt.gate;
        a.seg_offsets = rt.off;
        a.pair_perm = rt.perm;
        a.u = reinterpret_cast<float*>(w + off);
        a.n_tiles = plan.n_tiles;
        off += rp::prefill_u_bytes(g.n_proj, (int)T, (int)r, k);
        // split-K needs one arrival counter per (tile, token tile)
        int S = rp::prefill_splits((int)g.d_in, plan.n_tiles, (int)T, n_cu);
        const int n_cnt = rp::prefill_units(plan.n_tiles, (int)T);
        if (S > 1 && counters + n_cnt > rp::kPrefillCounterWords) S = 1;
        a.S = S;
        a.counters = reinterpret_cast<int*>(w) + rp::kPrefillCounterWord + counters;
        a.partial = reinterpret_cast<float*>(w + off);
        if (S > 1) counters += n_cnt;
        off += rp::prefill_partial_bytes(plan.n_tiles, (int)T, S);
        shrink_blocks += ps.units * g.n_proj;
        gemm_blocks += rp::prefill_group_blocks(plan.n_tiles, (int)T) * S;
        ps.shrink_end[i] = shrink_blocks;
        ps.block_end[i] = gemm_blocks;
      }
      if (ws_bytes < off) return fail(RP_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, off);
      hipError_t e = rp::launch_prefill_step(ps, stream);
      if (e != hipSuccess) return hip_fail(fn, e);
      g0 += ng;
    }
    return RP_OK;
  }
  if (!decode) {
    for (int g = 0; g < n_groups; ++g) {
      int d_out[RP_MAX_PROJ];
      for (int p = 0; p < gs[g].n_proj; ++p) d_out[p] = (int)gs[g].projs[p].d_out;
      const rp::SgmmPlan plan =
          rp::plan_sgmm(rdt, gs[g].n_proj, d_out, (int)T, (int)gs[g].d_in, (int)E, (int)r, k, n_cu, false);
      if (ws_bytes < plan.bytes)
        return fail(RP_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, plan.bytes);
      rp::SgmmArgs a{};
      fill_group(&a, gs[g].projs, gs[g].n_proj, gs[g].x, T, gs[g].d_in, gs[g].ld_x, E, r, k, plan.tile_rows);
      a.topk_idx = rt.idx;
      a.topk_gate = rt.gate;
      a.seg_offsets = rt.off;
      a.pair_perm = rt.perm;
      a.counters = reinterpret_cast<int*>(w);
      a.u = reinterpret_cast<float*>(w + plan.off_u);
      a.partial = reinterpret_cast<float*>(w + plan.off_partial);
      a.n_tiles = plan.n_tiles;
      a.S = plan.S;
      hipError_t e = rp::launch_sgmm(a, plan, rdt, stream);
      if (e != hipSuccess) return hip_fail(fn, e);
    }
    return RP_OK;
  }
  for (int g0 = 0; g0 < n_groups; g0 += rp::kMaxGroups) {
    const int ng = std::min(rp::kMaxGroups, n_groups - g0);
    rp::StepGroupDesc desc[rp::kMaxGroups];
    int d_out[rp::kMaxGroups][RP_MAX_PROJ];
    for (int i = 0; i < ng; ++i) {
      const rp_group& g = gs[g0 + i];
      for (int p = 0; p < g.n_proj; ++p) d_out[i][p] = (int)g.projs[p].d_out;
      // across launches the kernel boundary orders the data already
      desc[i] = rp::StepGroupDesc{g.n_proj, d_out[i], (int)g.d_in, i > 0 && g.x_from_call ? 1 : 0};
    }
    const bool fused_here = fuse_route && g0 == 0;
    const rp::StepPlan sp = rp::plan_step(desc, ng, (int)T, (int)E, (int)r, k, n_cu, fused_here);
    if (ws_bytes < sp.bytes)
      return fail(RP_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, sp.bytes);
    rp::StepArgs st{};
    for (int i = 0; i < ng; ++i) {
      const rp_group& g = gs[g0 + i];
      const rp::SgmmPlan& gp = sp.gp[i];
      rp::SgmmArgs& a = st.g[i];
      fill_group(&a, g.projs, g.n_proj, g.x, T, g.d_in, g.ld_x, E, r, k, gp.tile_rows);
      a.topk_idx = rt.idx;
      a.topk_gate = rt.gate;
      a.seg_offsets = rt.off;
      a.pair_perm = rt.perm;
      a.counters = reinterpret_cast<int*>(w);
      a.u = reinterpret_cast<float*>(w + gp.off_u);
      a.partial = reinterpret_cast<float*>(w + gp.off_partial);
      a.n_tiles = gp.n_tiles;
      a.S = gp.S;
      rp::GroupPlan& q = st.gp[i];
      q.shrink_begin = sp.shrink_begin[i];
      q.base_begin = sp.base_begin[i];
      q.n_shrink = gp.n_shrink;
      q.n_items = gp.n_items;
      q.shrink_target = gp.dense ? 0 : q.n_shrink;
      q.units_per_proj = gp.units_per_proj;
      q.KP = gp.KP;
      q.atiles_per_proj = gp.atiles_per_proj;
      q.n_atiles = gp.n_atiles;
      q.SA = gp.SA;
      // only a group whose x an earlier group writes waits, and it waits for
      // all of them; the others stream as soon as they are scheduled
      bool later_reads = false;
      for (int j = i + 1; j < ng; ++j) later_reads = later_reads || desc[j].x_acquire;
      q.x_acquire = desc[i].x_acquire;
      q.count_done = later_reads;
      q.release = later_reads;
      q.wait_target = 0;
      if (desc[i].x_acquire)
        for (int j = 0; j < i; ++j) q.wait_target += sp.gp[j].n_tiles;
      q.partial_a = reinterpret_cast<float*>(w + gp.off_partial_a);
    }
    st.n_groups = ng;
    st.n_items = sp.n_items;
    st.n_route = sp.n_route;
    st.n_pre = sp.n_pre;
    st.fused = fused_here;
    st.dense = sp.gp[0].dense;
    st.t_pad = sp.gp[0].t_pad;
    st.route_tagged = reinterpret_cast<unsigned int*>(w + sp.off_route);
    st.pg = pg;
    st.sg = sg;
    hipError_t e = rp::launch_step(st, sp, stream);
    if (e != hipSuccess) return hip_fail(fn, e);
  }
  return RP_OK;
}

// Checks of a call's routing pointers; `compute` when the call writes them.
rp_status check_routing(const char* fn, const Routing& rt, int64_t T, int64_t E, int32_t k, bool compute) {
  if (compute) {
    if (k < 1) return fail(RP_ERR_INVALID_ARG, "%s: k=%d, routing needs k >= 1", fn, k);
    if (!rt.Wg || !aligned(rt.Wg, 16)) return fail(RP_ERR_INVALID_ARG, "%s: Wg must be non-null and 16-byte aligned", fn);
    if (T * E > (int64_t)1 << 40) return fail(RP_ERR_INVALID_ARG, "%s: T*E too large", fn);
  }
  if (k > 0 && (!rt.idx || !rt.gate || !rt.off || !rt.perm))
    return fail(RP_ERR_INVALID_ARG, "%s: k>0 needs topk_idx, topk_gate, seg_offsets and pair_perm", fn);
  if ((rt.idx && !aligned(rt.idx, 4)) || (rt.gate && !aligned(rt.gate, 4)) || (rt.off && !aligned(rt.off, 4)) ||
      (rt.perm && !aligned(rt.perm, 4)))
    return fail(RP_ERR_INVALID_ARG, "%s: routing arrays must be 4-byte aligned", fn);
  return RP_OK;
}

}  // namespace

extern "C" {

rp_status rp_sgmm_fused(const rp_proj* projs, int32_t n_proj, const void* x, int64_t T, int64_t d_in, int64_t ld_x,
                        int64_t E, int64_t r, int32_t k, const int32_t* topk_idx, const float* topk_gate,
                        const int32_t* seg_offsets, const int32_t* pair_perm, rp_dtype dt, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  g_last_error.clear();
  const char* fn = "rp_sgmm_fused";
  rp_status st = check_sgmm(fn, projs, n_proj, x, T, d_in, ld_x, E, r, k, dt, ws);
  if (st != RP_OK || T == 0) return st;
  const Routing rt{nullptr, const_cast<int32_t*>(topk_idx), const_cast<float*>(topk_gate),
                   const_cast<int32_t*>(seg_offsets), const_cast<int32_t*>(pair_perm)};
  st = check_routing(fn, rt, T, E, k, false);
  if (st != RP_OK) return st;
  const rp_group g{projs, n_proj, 0, x, d_in, ld_x};
  return run_groups(fn, &g, 1, T, E, r, k, dt, rt, ws, ws_bytes, stream);
}

rp_status rp_route_sgmm_fused(const rp_proj* projs, int32_t n_proj, const void* x, int64_t T, int64_t d_in,
                              int64_t ld_x, const void* Wg, int64_t E, int64_t r, int32_t k, rp_dtype dt,
                              int32_t* topk_idx, float* topk_gate, int32_t* seg_offsets, int32_t* pair_perm,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  const char* fn = "rp_route_sgmm_fused";
  if (k < 1) return fail(RP_ERR_INVALID_ARG, "%s: k=%d, routing needs k >= 1", fn, k);
  rp_status st = check_sgmm(fn, projs, n_proj, x, T, d_in, ld_x, E, r, k, dt, ws);
  if (st != RP_OK || T == 0) return st;
  const Routing rt{Wg, topk_idx, topk_gate, seg_offsets, pair_perm};
  st = check_routing(fn, rt, T, E, k, true);
  if (st != RP_OK) return st;
  const rp_group g{projs, n_proj, 0, x, d_in, ld_x};
  return run_groups(fn, &g, 1, T, E, r, k, dt, rt, ws, ws_bytes, stream);
}

size_t rp_sgmm_step_workspace_size(const rp_group* groups, int32_t n_groups, int64_t T, int64_t E, int64_t r,
                                   int32_t k, rp_dtype dt) {
  if (!groups || n_groups < 1 || n_groups > RP_MAX_GROUPS || !valid_dtype(dt) || T < 0 || T > kIntMax || E < 1 ||
      E > RP_MAX_E || k < 0 || k > RP_MAX_K || k > E || !(r == 8 || r == 16 || r == 32 || r == 64 || r == 128))
    return 0;
  for (int g = 0; g < n_groups; ++g) {
    if (!groups[g].projs || groups[g].n_proj < 1 || groups[g].n_proj > RP_MAX_PROJ || groups[g].d_in < 1) return 0;
    for (int p = 0; p < groups[g].n_proj; ++p)
      if (groups[g].projs[p].d_out < 8 || groups[g].projs[p].d_out > kIntMax) return 0;
  }
  return groups_workspace_bytes(groups, n_groups, T, E, r, k, dt);
}

rp_status rp_sgmm_step(const rp_group* groups, int32_t n_groups, int64_t T, int64_t E, int64_t r, int32_t k,
                       const void* Wg_or_null, int32_t* topk_idx, float* topk_gate, int32_t* seg_offsets,
                       int32_t* pair_perm, rp_dtype dt, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  const char* fn = "rp_sgmm_step";
  if (!groups || n_groups < 1 || n_groups > RP_MAX_GROUPS)
    return fail(RP_ERR_INVALID_ARG, "%s: n_groups=%d not in [1, %d]", fn, n_groups, RP_MAX_GROUPS);
  for (int g = 0; g < n_groups; ++g) {
    char name[64];
    snprintf(name, sizeof name, "%s: group %d", fn, g);
    rp_status st = check_sgmm(name, groups[g].projs, groups[g].n_proj, groups[g].x, T, groups[g].d_in,
                              groups[g].ld_x, E, r, k, dt, ws);
    if (st != RP_OK) return st;
    if (groups[g].x_from_call != 0 && groups[g].x_from_call != 1)
      return fail(RP_ERR_INVALID_ARG, "%s: x_from_call must be 0 or 1", name);
  }
  if (T == 0) return RP_OK;
  const Routing rt{Wg_or_null, topk_idx, topk_gate, seg_offsets, pair_perm};
  rp_status st = check_routing(fn, rt, T, E, k, Wg_or_null != nullptr);
  if (st != RP_OK) return st;
  const size_t need = groups_workspace_bytes(groups, n_groups, T, E, r, k, dt);
  if (ws_bytes < need) return fail(RP_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
  return run_groups(fn, groups, n_groups, T, E, r, k, dt, rt, ws, ws_bytes, stream);
}

rp_status rp_pack_w0(const void* src, void* dst, int64_t d_out, int64_t d_in, rp_dtype dt, hipStream_t stream) {
  g_last_error.clear();
  if (dt != RP_BF16) return fail(RP_ERR_UNSUPPORTED, "rp_pack_w0: the tiled layout is bf16 only");
  if (d_out < 16 || d_in < 32 || d_out % 16 != 0 || d_in % 32 != 0 || d_out * d_in > ((int64_t)1 << 40))
    return fail(RP_ERR_INVALID_ARG, "rp_pack_w0: need d_out %% 16 == 0 and d_in %% 32 == 0 (got %lld x %lld)",
                (long long)d_out, (long long)d_in);
  if (!src || !dst || !aligned(src, 16) || !aligned(dst, 16))
    return fail(RP_ERR_INVALID_ARG, "rp_pack_w0: src and dst must be non-null and 16-byte aligned");
  const char* s0 = static_cast<const char*>(src);
  const char* d0 = static_cast<const char*>(dst);
  const int64_t bytes = d_out * d_in * 2;
  if (s0 < d0 + bytes && d0 < s0 + bytes) return fail(RP_ERR_INVALID_ARG, "rp_pack_w0: src and dst overlap");
  if (d_out > kIntMax || d_in > kIntMax) return fail(RP_ERR_INVALID_ARG, "rp_pack_w0: sizes too large");
  hipError_t e = rp::launch_pack_w0(src, dst, (int)d_out, (int)d_in, stream);
  return e == hipSuccess ? RP_OK : hip_fail("rp_pack_w0 launch", e);
}

rp_status rp_util_stream_read(const void* src, size_t n_bytes, float* sink, hipStream_t stream) {
  g_last_error.clear();
  if (!src || !sink || !aligned(src, 16) || n_bytes % 16 != 0 || n_bytes == 0)
    return fail(RP_ERR_INVALID_ARG, "rp_util_stream_read: need non-null 16-byte aligned src and n_bytes %% 16 == 0");
  hipError_t e = rp::launch_stream_read(src, n_bytes, sink, stream);
  return e == hipSuccess ? RP_OK : hip_fail("rp_util_stream_read launch", e);
}

rp_status rp_util_copy(void* dst, const void* src, size_t n_bytes, hipStream_t stream) {
  g_last_error.clear();
  if (!src || !dst || !aligned(src, 16) || !aligned(dst, 16) || n_bytes % 16 != 0 || n_bytes == 0)
    return fail(RP_ERR_INVALID_ARG, "rp_util_copy: need non-null 16-byte aligned buffers and n_bytes %% 16 == 0");
  hipError_t e = rp::launch_copy(dst, src, n_bytes, stream);
  return e == hipSuccess ? RP_OK : hip_fail("rp_util_copy launch", e);
}

}  // extern "C"
