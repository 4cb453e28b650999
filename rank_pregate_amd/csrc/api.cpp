// C ABI of the library: argument validation, launch planning and dispatch.
// Every check runs on the host before anything is queued; no exception leaves
// this file.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdarg>
#include <cmath>
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

// A second stream per device, with the events that fork work from a caller's
// stream onto it and join it back; created on first use outside stream
// capture (default priority), kept until the process ends.  Callers hold
// side_mu from the fork to the join, so the records and waits of calls from
// several host threads do not interleave.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex side_mu;
SideStream* side_stream(bool may_create) {
  static SideStream cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  SideStream& ss = cache[dev];
  if (ss.join) return &ss;
  if (!may_create) return nullptr;
  if (!ss.s && hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess) ss.s = nullptr;
  if (ss.s && !ss.fork && hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess) ss.fork = nullptr;
  if (ss.fork && hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) ss.join = nullptr;
  return ss.join ? &ss : nullptr;
}

}  // namespace

namespace rp {
// Records a status message for rp_last_error() from another source file of the library.
rp_status record_error(rp_status st, const char* msg) { return fail(st, "%s", msg); }
}  // namespace rp

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
  const rp::Dtype rdt = dt == RP_BF16 ? rp::kBF16 : rp::kF32;
  size_t b = rp::sgmm_workspace_upper_bound(rdt, n_proj, (int)T, (int)d_in, (long long)sum_d_out, (int)E, (int)r, k);
  // routing computed by the call (rp_route_sgmm_fused) may run the split-form router first
  if (rp::mfma_router_supported(rdt, (int)E) && rp::route_split_tiles((int)T) + 1 <= rp::kRouteCounterWords)
    b = std::max(b, rp::kWorkspaceCounterBytes + rp::route_split_bytes((int)T, (int)E));
  return b;
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
    if (!aligned(q.W0, 16) || !aligned(q.A, 16) || !aligned(q.B, 16) || !aligned(q.y, 16) || !aligned(q.residual, 16))
      return fail(RP_ERR_INVALID_ARG, "%s: projection %d: W0, A, B, y, residual must be 16-byte aligned", fn, p);
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
    a->proj[p].residual = projs[q].residual;
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

// Words of the workspace's control region: the count of out-of-range router
// indices when a call computes the routing, and the sticky flag a kernel sets
// when a cross-workgroup wait gives up (the device side's kCtlSegErr and
// kCtlWaitOverflow).
constexpr size_t kSegErrWord = 64;
constexpr size_t kWaitOverflowWord = 32;

struct Routing {
  const void* Wg;  // non-null: compute the routing from the first group's x
  int32_t* idx;
  float* gate;
  int32_t* off;
  int32_t* perm;
};

bool decode_shape(rp_dtype dt, int64_t T) { return dt == RP_BF16 && T <= 64; }

// Routing computed in a step by the split-form matrix-core router (routing and
// segmentation in one launch); its workspace need, 0 if it does not apply.
bool split_router(rp_dtype dt, int64_t T, int64_t E) {
  return rp::mfma_router_supported(dt == RP_BF16 ? rp::kBF16 : rp::kF32, (int)E) &&
         rp::route_split_tiles((int)T) + 1 <= rp::kRouteCounterWords;
}
size_t split_router_bytes(rp_dtype dt, int64_t T, int64_t E) {
  return split_router(dt, T, E) ? rp::kWorkspaceCounterBytes + rp::route_split_bytes((int)T, (int)E) : 0;
}

// Prefill batches whose shrink (and routing) can run beside the base GEMM:
// bf16, the expand as a launch of its own, every group in one launch pair.
bool overlap_shrink(const rp_group* gs, int n_groups, int64_t T, int64_t E, int64_t r, int32_t k, rp_dtype dt) {
  if (decode_shape(dt, T) || dt != RP_BF16 || n_groups > rp::kMaxGroups ||
      !rp::prefill_split_expand((int)T, (int)E, (int)r, k))
    return false;
  for (int g = 1; g < n_groups; ++g)
    if (gs[g].x_from_call) return false;
  return true;
}

// Workspace bytes a validated call needs.
size_t groups_workspace_bytes(const rp_group* gs, int n_groups, int64_t T, int64_t E, int64_t r, int32_t k,
                              rp_dtype dt) {
  size_t need = split_router_bytes(dt, T, E);  // routing, if the call computes it (before any group runs)
  if (decode_shape(dt, T)) {
    // launches alternate between two workspace halves when no group reads
    // another's output and there are more than two (see run_groups)
    bool alt = n_groups > 2 * rp::kMaxGroups;
    for (int g = 0; g < n_groups; ++g) alt = alt && !gs[g].x_from_call;
    size_t m = 0;
    for (int g0 = 0; g0 < n_groups; g0 += rp::kMaxGroups) {
      const int ng = std::min(rp::kMaxGroups, n_groups - g0);
      rp::StepGroupDesc desc[rp::kMaxGroups];
      int d_out[rp::kMaxGroups][RP_MAX_PROJ];
      for (int i = 0; i < ng; ++i) {
        for (int p = 0; p < gs[g0 + i].n_proj; ++p) d_out[i][p] = (int)gs[g0 + i].projs[p].d_out;
        desc[i] = rp::StepGroupDesc{gs[g0 + i].n_proj, d_out[i], (int)gs[g0 + i].d_in, 0};
      }
      m = std::max(m, rp::step_workspace_upper_bound(desc, ng, (int)T, (int)E, (int)r, k));
    }
    m = (m + 255) & ~(size_t)255;
    need = std::max(need, alt ? 2 * m : m);
  } else if (dt == RP_BF16) {
    // every group's u side by side (a launch pair runs several groups)
    size_t b = rp::kWorkspaceCounterBytes;
    for (int g = 0; g < n_groups; ++g) {
      int64_t sum = 0;
      for (int p = 0; p < gs[g].n_proj; ++p) sum += gs[g].projs[p].d_out;
      const int tiles_bound = (int)(sum / rp::prefill_tile_rows((int)T) + gs[g].n_proj);
      b += rp::prefill_u_bytes(gs[g].n_proj, (int)T, (int)r, k) +
           rp::prefill_partial_bytes(tiles_bound, (int)T, rp::prefill_max_splits((int)gs[g].d_in));
      if (rp::prefill_split_expand((int)T, (int)E, (int)r, k)) b += rp::prefill_base_bytes(tiles_bound, (int)T);
    }
    // routing beside the groups: its partial sums after their buffers
    need = overlap_shrink(gs, n_groups, T, E, r, k, dt) ? b + 256 + split_router_bytes(dt, T, E) : std::max(need, b);
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

// A group's activation as its own launch after the group (paths without the
// fused epilogue): projs[0].y <- silu(projs[0].y) * projs[1].y.
hipError_t launch_act(const rp_group& g, int64_t T, rp::Dtype dt, hipStream_t stream) {
  return rp::launch_silu_mul(g.projs[0].y, (int)g.projs[0].ld_y, g.projs[1].y, (int)g.projs[1].ld_y, (int)T,
                             (int)g.projs[0].d_out, g.projs[0].y, (int)g.projs[0].ld_y, dt, stream);
}

// Runs the groups of a validated call in order on `stream`.  Decode shapes go
// through the multi-group decode kernel, up to kMaxGroups groups per launch;
// routing to compute runs inside the first launch when T <= 32, otherwise as
// router and segmentation launches of its own first.  With `dry_need` set it
// only plans: *dry_need receives the workspace bytes the largest launch of the
// call uses on the current device, and nothing is launched.
rp_status run_groups(const char* fn, const rp_group* gs, int n_groups, int64_t T, int64_t E, int64_t r, int32_t k,
                     rp_dtype dt, const Routing& rt, void* ws, size_t ws_bytes, hipStream_t stream,
                     size_t* dry_need = nullptr) {
  int n_cu = 0;
  if (cu_count(&n_cu) != 0) return fail(RP_ERR_HIP, "%s: cannot query the current device", fn);
  const bool dry = dry_need != nullptr;
  if (dry) {
    *dry_need = rp::kWorkspaceCounterBytes;
    ws_bytes = SIZE_MAX;
  }
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
  // prefill with the expand in a launch of its own and every group in one
  // batch: the routing, the shrink and the expand run on a second stream
  // beside the base GEMM, which needs none of them; a last launch adds the
  // two
  const bool overlap = overlap_shrink(gs, n_groups, T, E, r, k, dt);
  if (overlap) {
    // launched with the groups below
  } else if (route && !fuse_route && split_router(dt, T, E)) {
    // router and segmentation in one launch; its partial sums sit where the
    // groups' buffers go (the groups' launches are queued after it)
    const size_t need = split_router_bytes(dt, T, E);
    if (ws_bytes < need) return fail(RP_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
    if (dry) {
      *dry_need = std::max(*dry_need, need);
    } else {
      hipError_t e = rp::launch_route_segment_mfma(pg, sg, w + rp::kWorkspaceCounterBytes,
                                                   reinterpret_cast<int*>(w) + rp::kRouteCounterWord, stream);
      if (e != hipSuccess) return hip_fail(fn, e);
    }
  } else if (route && !fuse_route && !dry) {
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
      ps.split_expand = rp::prefill_split_expand((int)T, (int)E, (int)r, k) ? 1 : 0;
      size_t off = rp::kWorkspaceCounterBytes;
      int shrink_blocks = 0, gemm_blocks = 0, counters = 0, expand_blocks = 0, combine_blocks = 0;
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
        if (ps.split_expand) {
          a.base = reinterpret_cast<float*>(w + off);
          a.delta = a.base + (size_t)plan.n_tiles * T * rp::prefill_tile_rows((int)T);
          off += rp::prefill_base_bytes(plan.n_tiles, (int)T);
          expand_blocks += rp::prefill_expand_blocks(plan.n_tiles, (int)T);
          combine_blocks += rp::prefill_combine_blocks(plan.n_tiles, (int)T);
          ps.expand_end[i] = expand_blocks;
          ps.combine_end[i] = combine_blocks;
        }
        shrink_blocks += ps.units * g.n_proj;
        gemm_blocks += rp::prefill_group_blocks(plan.n_tiles, (int)T) * S;
        ps.shrink_end[i] = shrink_blocks;
        ps.block_end[i] = gemm_blocks;
      }
      // the split-form router's partial sums go after the groups' buffers
      // when it runs beside the GEMM
      const bool split_rt = overlap && route && split_router(dt, T, E);
      const size_t rbase = (off + 255) & ~(size_t)255;
      const size_t need = split_rt ? rbase + rp::route_split_bytes((int)T, (int)E) : off;
      if (ws_bytes < need) return fail(RP_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
      g0 += ng;
      if (dry) {
        *dry_need = std::max(*dry_need, need);
        continue;
      }
      hipError_t e = hipSuccess;
      if (overlap) {
        std::lock_guard<std::mutex> lock(side_mu);
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(stream, &cs);
        SideStream* ss = e == hipSuccess ? side_stream(cs == hipStreamCaptureStatusNone) : nullptr;
        const hipStream_t side = ss ? ss->s : stream;  // without one, the same order on the caller's stream
        if (e == hipSuccess && ss) e = hipEventRecord(ss->fork, stream);
        if (e == hipSuccess && ss) e = hipStreamWaitEvent(side, ss->fork, 0);
        if (e == hipSuccess && split_rt)
          e = rp::launch_route_segment_mfma(pg, sg, w + rbase, reinterpret_cast<int*>(w) + rp::kRouteCounterWord,
                                            side);
        else if (e == hipSuccess && route)
          e = rp::launch_pregate(pg, side);
        if (e == hipSuccess && route && !split_rt) e = rp::launch_segment(sg, side);
        if (e == hipSuccess) e = rp::launch_prefill_shrink(ps, side);
        if (e == hipSuccess) e = rp::launch_prefill_expand(ps, side);
        if (e == hipSuccess && ss) e = hipEventRecord(ss->join, side);
        if (e == hipSuccess) e = rp::launch_prefill_gemm(ps, stream);
        if (e == hipSuccess && ss) e = hipStreamWaitEvent(stream, ss->join, 0);
        if (e == hipSuccess) e = rp::launch_prefill_combine(ps, stream);
      } else {
        e = rp::launch_prefill_step(ps, stream);
      }
      for (int i = 0; e == hipSuccess && i < ng; ++i)
        if (gs[g0 - ng + i].act == RP_ACT_SILU_MUL) e = launch_act(gs[g0 - ng + i], T, rdt, stream);
      if (e != hipSuccess) return hip_fail(fn, e);
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
      if (dry) {
        *dry_need = std::max(*dry_need, plan.bytes);
        continue;
      }
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
      if (e == hipSuccess && gs[g].act == RP_ACT_SILU_MUL) e = launch_act(gs[g], T, rdt, stream);
      if (e != hipSuccess) return hip_fail(fn, e);
    }
    return RP_OK;
  }
  // Launches of kMaxGroups groups.  When no group reads another group's
  // output, launches after the first (which writes the routing when it runs
  // inside) depend on nothing but it: odd launches then go to the second
  // stream with the second half of the workspace, so the last items of one
  // launch run beside the first items of the next instead of leaving CUs idle.
  const int n_batches = (n_groups + rp::kMaxGroups - 1) / rp::kMaxGroups;
  bool alt = n_batches > 2;
  for (int g = 0; g < n_groups; ++g) alt = alt && !gs[g].x_from_call;
  auto batch_plan = [&](int g0, rp::StepGroupDesc* desc, int (*d_out)[RP_MAX_PROJ]) {
    const int ng = std::min(rp::kMaxGroups, n_groups - g0);
    for (int i = 0; i < ng; ++i) {
      const rp_group& g = gs[g0 + i];
      for (int p = 0; p < g.n_proj; ++p) d_out[i][p] = (int)g.projs[p].d_out;
      // across launches the kernel boundary orders the data already
      desc[i] = rp::StepGroupDesc{g.n_proj, d_out[i], (int)g.d_in, i > 0 && g.x_from_call ? 1 : 0};
    }
    return rp::plan_step(desc, ng, (int)T, (int)E, (int)r, k, n_cu, fuse_route && g0 == 0);
  };
  size_t half = 0;  // workspace bytes of one launch (the largest)
  for (int g0 = 0; g0 < n_groups; g0 += rp::kMaxGroups) {
    rp::StepGroupDesc desc[rp::kMaxGroups];
    int d_out[rp::kMaxGroups][RP_MAX_PROJ];
    half = std::max(half, batch_plan(g0, desc, d_out).bytes);
  }
  half = (half + 255) & ~(size_t)255;
  const size_t need_all = alt ? 2 * half : half;
  if (ws_bytes < need_all) return fail(RP_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need_all);
  if (dry) {
    *dry_need = std::max(*dry_need, need_all);
    return RP_OK;
  }
  std::unique_lock<std::mutex> side_lock(side_mu, std::defer_lock);
  SideStream* ss = nullptr;
  if (alt) {
    side_lock.lock();
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return hip_fail(fn, hipGetLastError());
    ss = side_stream(cs == hipStreamCaptureStatusNone);
    if (!ss) alt = false;  // no second stream: every launch in order on the caller's
  }
  char* const w_main = w;
  for (int g0 = 0, b = 0; g0 < n_groups; g0 += rp::kMaxGroups, ++b) {
    const int ng = std::min(rp::kMaxGroups, n_groups - g0);
    rp::StepGroupDesc desc[rp::kMaxGroups];
    int d_out[rp::kMaxGroups][RP_MAX_PROJ];
    const bool fused_here = fuse_route && g0 == 0;
    const rp::StepPlan sp = batch_plan(g0, desc, d_out);
    const bool on_side = alt && (b & 1);
    w = on_side ? w_main + half : w_main;
    int* const ctl = reinterpret_cast<int*>(w_main + (on_side ? rp::kCounterBlockBytes : 0));
    const hipStream_t bs = on_side ? ss->s : stream;
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
      a.counters = ctl;
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
      q.act = g.act;
      q.pair_cnt = ctl + rp::kPrefillCounterWord + i * rp::kActPairWords;
      // such a group reads x and its residuals through buffer resources: 32-bit byte ranges
      bool wide = (uint64_t)T * (uint64_t)g.ld_x * 2u > 0xFFFFFFFFull;
      for (int p = 0; p < g.n_proj; ++p) wide = wide || (uint64_t)T * (uint64_t)g.projs[p].ld_y * 2u > 0xFFFFFFFFull;
      if (desc[i].x_acquire && wide)
        return fail(RP_ERR_UNSUPPORTED, "%s: group %d reads an earlier group's output of more than 4 GiB (T * ld)",
                    fn, g0 + i);
      if (g.act == RP_ACT_SILU_MUL && (g.projs[0].d_out + gp.tile_rows - 1) / gp.tile_rows > rp::kActPairWords)
        return fail(RP_ERR_UNSUPPORTED, "%s: group %d: RP_ACT_SILU_MUL supports at most %d output tiles", fn,
                    g0 + i, rp::kActPairWords);
    }
    st.n_groups = ng;
    st.n_items = sp.n_items;
    st.n_route = sp.n_route;
    st.n_pre = sp.n_pre;
    st.fused = fused_here;
    st.claim_all = alt ? 1 : 0;
    st.dense = sp.gp[0].dense;
    st.t_pad = sp.gp[0].t_pad;
    st.route_tagged = reinterpret_cast<unsigned int*>(w + sp.off_route);
    st.pg = pg;
    st.sg = sg;
    hipError_t e = rp::launch_step(st, sp, bs);
    if (e == hipSuccess && alt && b == 0) {
      // the second stream starts after the first launch
      e = hipEventRecord(ss->fork, stream);
      if (e == hipSuccess) e = hipStreamWaitEvent(ss->s, ss->fork, 0);
    }
    if (e != hipSuccess) return hip_fail(fn, e);
  }
  if (alt) {
    hipError_t e = hipEventRecord(ss->join, ss->s);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, ss->join, 0);
    if (e != hipSuccess) return hip_fail(fn, e);
  }
  return RP_OK;
}

// Workspace bytes a validated call uses on the current device (0 if the
// device cannot be queried).
size_t exact_need(const rp_group* gs, int n_groups, int64_t T, int64_t E, int64_t r, int32_t k, rp_dtype dt,
                  bool route) {
  size_t need = 0;
  const Routing rt{route ? reinterpret_cast<const void*>(16) : nullptr, nullptr, nullptr, nullptr, nullptr};
  const std::string saved = g_last_error;
  if (run_groups("plan", gs, n_groups, T, E, r, k, dt, rt, nullptr, 0, nullptr, &need) != RP_OK) need = 0;
  g_last_error = saved;
  return need;
}

// Checks that the workspace covers every launch of a validated call before
// anything is queued.
rp_status check_need(const char* fn, const rp_group* gs, int n_groups, int64_t T, int64_t E, int64_t r, int32_t k,
                     rp_dtype dt, bool route, size_t ws_bytes) {
  size_t need = exact_need(gs, n_groups, T, E, r, k, dt, route);
  if (need == 0) need = groups_workspace_bytes(gs, n_groups, T, E, r, k, dt);  // no device: the bound
  if (ws_bytes < need) return fail(RP_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
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
  st = check_need(fn, &g, 1, T, E, r, k, dt, false, ws_bytes);
  if (st != RP_OK) return st;
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
  st = check_need(fn, &g, 1, T, E, r, k, dt, true, ws_bytes);
  if (st != RP_OK) return st;
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
  // the exact need of the call on the current device, taking the routing as
  // computed when k > 0 (its split-form router may need more than the
  // groups; given routing never needs more); the device-independent bound if
  // the device cannot be queried
  const size_t need = exact_need(groups, n_groups, T, E, r, k, dt, k > 0);
  return need ? need : groups_workspace_bytes(groups, n_groups, T, E, r, k, dt);
}

}  // extern "C"

namespace rp {
// Every argument check of rp_sgmm_step except the workspace's (no device call).
rp_status validate_step(const char* fn, const rp_group* groups, int32_t n_groups, int64_t T, int64_t E, int64_t r,
                        int32_t k, const void* Wg_or_null, int32_t* topk_idx, float* topk_gate, int32_t* seg_offsets,
                        int32_t* pair_perm, rp_dtype dt) {
  if (!groups || n_groups < 1 || n_groups > RP_MAX_GROUPS)
    return fail(RP_ERR_INVALID_ARG, "%s: n_groups=%d not in [1, %d]", fn, n_groups, RP_MAX_GROUPS);
  void* const ws_stub = reinterpret_cast<void*>(256);  // the workspace is checked by the caller
  for (int g = 0; g < n_groups; ++g) {
    char name[96];
    snprintf(name, sizeof name, "%s: group %d", fn, g);
    rp_status st = check_sgmm(name, groups[g].projs, groups[g].n_proj, groups[g].x, T, groups[g].d_in,
                              groups[g].ld_x, E, r, k, dt, ws_stub);
    if (st != RP_OK) return st;
    if (groups[g].x_from_call != 0 && groups[g].x_from_call != 1)
      return fail(RP_ERR_INVALID_ARG, "%s: x_from_call must be 0 or 1", name);
    if (groups[g].reserved != 0 || (groups[g].act != RP_ACT_NONE && groups[g].act != RP_ACT_SILU_MUL))
      return fail(RP_ERR_INVALID_ARG, "%s: unknown act %d / reserved %d", name, groups[g].act, groups[g].reserved);
    if (groups[g].act == RP_ACT_SILU_MUL &&
        (groups[g].n_proj != 2 || groups[g].projs[0].d_out != groups[g].projs[1].d_out))
      return fail(RP_ERR_INVALID_ARG, "%s: RP_ACT_SILU_MUL needs two projections of equal d_out", name);
  }
  if (T == 0) return RP_OK;
  const Routing rt{Wg_or_null, topk_idx, topk_gate, seg_offsets, pair_perm};
  return check_routing(fn, rt, T, E, k, Wg_or_null != nullptr);
}
}  // namespace rp

extern "C" {

rp_status rp_sgmm_step(const rp_group* groups, int32_t n_groups, int64_t T, int64_t E, int64_t r, int32_t k,
                       const void* Wg_or_null, int32_t* topk_idx, float* topk_gate, int32_t* seg_offsets,
                       int32_t* pair_perm, rp_dtype dt, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  const char* fn = "rp_sgmm_step";
  rp_status st = rp::validate_step(fn, groups, n_groups, T, E, r, k, Wg_or_null, topk_idx, topk_gate, seg_offsets,
                                   pair_perm, dt);
  if (st != RP_OK || T == 0) return st;
  if (!ws) return fail(RP_ERR_WORKSPACE, "%s: null workspace", fn);
  if (!aligned(ws, 256)) return fail(RP_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  st = check_need(fn, groups, n_groups, T, E, r, k, dt, Wg_or_null != nullptr, ws_bytes);
  if (st != RP_OK) return st;
  const Routing rt{Wg_or_null, topk_idx, topk_gate, seg_offsets, pair_perm};
  return run_groups(fn, groups, n_groups, T, E, r, k, dt, rt, ws, ws_bytes, stream);
}

rp_status rp_adapter_apply(const rp_proj* projs, int32_t n_proj, const void* x, int64_t T, int64_t d_in,
                           int64_t ld_x, int64_t E, int64_t r, int32_t k, int32_t adapter, const float* topk_gate,
                           const int32_t* seg_offsets, const int32_t* pair_perm, rp_dtype dt, hipStream_t stream) {
  g_last_error.clear();
  const char* fn = "rp_adapter_apply";
  // the projection checks of rp_sgmm_fused (W0 is not read; no workspace is used)
  rp_status st = check_sgmm(fn, projs, n_proj, x, T, d_in, ld_x, E, r, k, dt, reinterpret_cast<void*>(256));
  for (int p = 0; st == RP_OK && p < n_proj; ++p)
    if (projs[p].residual)
      st = fail(RP_ERR_INVALID_ARG, "%s: projection %d: residual must be NULL (y already holds the base projection)",
                fn, p);
  if (st != RP_OK) return st;
  if (k < 1) return fail(RP_ERR_INVALID_ARG, "%s: k=%d, an adapter delta needs k >= 1", fn, k);
  if (adapter < 0 || adapter >= E) return fail(RP_ERR_INVALID_ARG, "%s: adapter %d not in [0, E)", fn, adapter);
  if (T == 0) return RP_OK;
  if (!topk_gate || !seg_offsets || !pair_perm || !aligned(topk_gate, 4) || !aligned(seg_offsets, 4) ||
      !aligned(pair_perm, 4))
    return fail(RP_ERR_INVALID_ARG, "%s: topk_gate, seg_offsets and pair_perm must be non-null and 4-byte aligned", fn);
  rp::SgmmArgs a{};
  fill_group(&a, projs, n_proj, x, T, d_in, ld_x, E, r, k, rp::adapter_apply_tile_rows());
  int tiles = 0;
  for (int p = 0; p < n_proj; ++p)
    tiles += (int)((projs[p].d_out + rp::adapter_apply_tile_rows() - 1) / rp::adapter_apply_tile_rows());
  a.n_tiles = tiles;
  a.topk_gate = topk_gate;
  a.seg_offsets = seg_offsets;
  a.pair_perm = pair_perm;
  hipError_t e = rp::launch_adapter_apply(a, adapter, dt == RP_BF16 ? rp::kBF16 : rp::kF32, stream);
  return e == hipSuccess ? RP_OK : hip_fail("rp_adapter_apply launch", e);
}

rp_status rp_merge_adapters(void* W0, int32_t w0_layout, int64_t d_out, int64_t d_in, const void* A, const void* B,
                            int64_t E, int64_t r, const int32_t* sel, const float* weights, int32_t n_sel, float sign,
                            rp_dtype dt, hipStream_t stream) {
  g_last_error.clear();
  const char* fn = "rp_merge_adapters";
  if (!valid_dtype(dt)) return fail(RP_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
  if (w0_layout != RP_W0_ROWS && w0_layout != RP_W0_TILED)
    return fail(RP_ERR_INVALID_ARG, "%s: unknown w0_layout %d", fn, w0_layout);
  if (d_out < 1 || d_in < 8 || d_in % 8 != 0 || d_out > kIntMax || d_in > kIntMax || d_out * d_in > ((int64_t)1 << 40))
    return fail(RP_ERR_INVALID_ARG, "%s: need d_out >= 1 and d_in a positive multiple of 8 (got %lld x %lld)", fn,
                (long long)d_out, (long long)d_in);
  if (w0_layout == RP_W0_TILED && (dt != RP_BF16 || d_out % 16 != 0 || d_in % 32 != 0))
    return fail(RP_ERR_UNSUPPORTED, "%s: the tiled W0 layout needs bf16, d_out %% 16 == 0 and d_in %% 32 == 0", fn);
  if (E < 1 || E > RP_MAX_E) return fail(RP_ERR_INVALID_ARG, "%s: E=%lld not in [1, %d]", fn, (long long)E, RP_MAX_E);
  if (!(r == 8 || r == 16 || r == 32 || r == 64 || r == 128))
    return fail(RP_ERR_UNSUPPORTED, "%s: rank r=%lld not in {8,16,32,64,128}", fn, (long long)r);
  if (n_sel < 0 || n_sel > RP_MAX_K) return fail(RP_ERR_INVALID_ARG, "%s: n_sel=%d not in [0, %d]", fn, n_sel, RP_MAX_K);
  if (E * r * std::max(d_in, d_out) > ((int64_t)1 << 40)) return fail(RP_ERR_INVALID_ARG, "%s: sizes too large", fn);
  if (n_sel == 0) return RP_OK;
  if (!W0 || !A || !B || !aligned(W0, 16) || !aligned(A, 16) || !aligned(B, 16))
    return fail(RP_ERR_INVALID_ARG, "%s: W0, A, B must be non-null and 16-byte aligned", fn);
  if (!sel || !weights || !aligned(sel, 4) || !aligned(weights, 4))
    return fail(RP_ERR_INVALID_ARG, "%s: sel and weights must be non-null and 4-byte aligned", fn);
  rp::MergeArgs m;
  m.W0 = W0;
  m.tiled = w0_layout == RP_W0_TILED;
  m.d_out = (int)d_out;
  m.d_in = (int)d_in;
  m.A = A;
  m.B = B;
  m.E = (int)E;
  m.r = (int)r;
  m.sel = sel;
  m.weights = weights;
  m.n_sel = n_sel;
  m.sign = sign;
  hipError_t e = rp::launch_merge(m, dt == RP_BF16 ? rp::kBF16 : rp::kF32, stream);
  return e == hipSuccess ? RP_OK : hip_fail("rp_merge_adapters launch", e);
}

// Shared checks of the per-token elementwise calls: rows of d elements with
// leading dimensions `lds` (n of them), pointers `ps`.
static rp_status check_rows(const char* fn, int64_t T, int64_t d, const int64_t* lds, const void* const* ps, int n,
                            rp_dtype dt) {
  if (!valid_dtype(dt)) return fail(RP_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
  if (T < 0 || T > kIntMax) return fail(RP_ERR_INVALID_ARG, "%s: T=%lld out of range", fn, (long long)T);
  const int64_t vec = dt == RP_BF16 ? 8 : 4, es = (int64_t)dsize(dt);
  if (d < vec || d % vec != 0 || d > 65536)
    return fail(RP_ERR_INVALID_ARG, "%s: d=%lld must be a positive multiple of %lld, at most 65536", fn, (long long)d,
                (long long)vec);
  for (int i = 0; i < n; ++i)
    if (lds[i] < d || (lds[i] * es) % 16 != 0 || lds[i] > kIntMax)
      return fail(RP_ERR_INVALID_ARG, "%s: leading dimension %lld must be >= d with ld*elem a multiple of 16 bytes",
                  fn, (long long)lds[i]);
  if (T == 0) return RP_OK;
  for (int i = 0; i < n; ++i)
    if (!ps[i] || !aligned(ps[i], 16)) return fail(RP_ERR_INVALID_ARG, "%s: pointers must be non-null and 16-byte aligned", fn);
  if (T * std::max(lds[0], d) > ((int64_t)1 << 40)) return fail(RP_ERR_INVALID_ARG, "%s: T*d too large", fn);
  return RP_OK;
}

rp_status rp_rmsnorm(const void* x, int64_t T, int64_t d, int64_t ld_x, const void* gamma, float eps, void* y,
                     int64_t ld_y, rp_dtype dt, hipStream_t stream) {
  g_last_error.clear();
  const char* fn = "rp_rmsnorm";
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(RP_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
  const int64_t lds[3] = {ld_x, ld_y, d};
  const void* ps[3] = {x, y, gamma};
  rp_status st = check_rows(fn, T, d, lds, ps, 3, dt);
  if (st != RP_OK || T == 0) return st;
  hipError_t e = rp::launch_rmsnorm(x, (int)T, (int)d, (int)ld_x, gamma, eps, y, (int)ld_y,
                                    dt == RP_BF16 ? rp::kBF16 : rp::kF32, stream);
  return e == hipSuccess ? RP_OK : hip_fail(fn, e);
}

rp_status rp_silu_mul(const void* g, int64_t ld_g, const void* u, int64_t ld_u, int64_t T, int64_t d, void* m,
                      int64_t ld_m, rp_dtype dt, hipStream_t stream) {
  g_last_error.clear();
  const char* fn = "rp_silu_mul";
  const int64_t lds[3] = {ld_g, ld_u, ld_m};
  const void* ps[3] = {g, u, m};
  rp_status st = check_rows(fn, T, d, lds, ps, 3, dt);
  if (st != RP_OK || T == 0) return st;
  hipError_t e = rp::launch_silu_mul(g, (int)ld_g, u, (int)ld_u, (int)T, (int)d, m, (int)ld_m,
                                     dt == RP_BF16 ? rp::kBF16 : rp::kF32, stream);
  return e == hipSuccess ? RP_OK : hip_fail(fn, e);
}

rp_status rp_workspace_status(void* ws, size_t ws_bytes, int32_t clear, int32_t* wait_overflow,
                              int32_t* bad_indices, hipStream_t stream) {
  g_last_error.clear();
  if (!ws || !aligned(ws, 256) || ws_bytes < rp::kWorkspaceCounterBytes)
    return fail(RP_ERR_WORKSPACE, "rp_workspace_status: need a 256-byte aligned workspace of at least %zu bytes",
                rp::kWorkspaceCounterBytes);
  // the two words sit in one 256-byte span of the control region
  static_assert(kSegErrWord > kWaitOverflowWord && kSegErrWord - kWaitOverflowWord < 64, "status span");
  // both control blocks (launches on the second stream flag theirs)
  constexpr int kBlockWords = (int)(rp::kCounterBlockBytes / 4);
  int32_t span[2][64];
  int32_t wo = 0, bad = 0;
  hipError_t e = hipSuccess;
  for (int blk = 0; blk < 2 && e == hipSuccess; ++blk)
    e = hipMemcpyAsync(span[blk], static_cast<int32_t*>(ws) + blk * kBlockWords + kWaitOverflowWord, sizeof span[blk],
                       hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail("rp_workspace_status", e);
  for (int blk = 0; blk < 2; ++blk) {
    wo |= span[blk][0];
    bad += span[blk][kSegErrWord - kWaitOverflowWord];
  }
  if (wait_overflow) *wait_overflow = wo;
  if (bad_indices) *bad_indices = bad;
  if (clear && (wo != 0 || bad != 0)) {
    for (int blk = 0; blk < 2 && e == hipSuccess; ++blk) {
      int32_t* b0 = static_cast<int32_t*>(ws) + blk * kBlockWords;
      e = hipMemsetAsync(b0 + kWaitOverflowWord, 0, sizeof(int32_t), stream);
      if (e == hipSuccess) e = hipMemsetAsync(b0 + kSegErrWord, 0, sizeof(int32_t), stream);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail("rp_workspace_status clear", e);
  }
  if (wo != 0 || bad != 0)
    return fail(RP_ERR_DEVICE, "rp_workspace_status: wait overflow flag %d, out-of-range adapter indices %d%s", wo,
                bad, wo ? " (a cross-workgroup wait gave up: outputs since the last clear are not valid)" : "");
  return RP_OK;
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
