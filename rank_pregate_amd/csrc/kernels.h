// Host-side launch interface between the C ABI layer (api.cpp) and the kernels.
// Everything here has already been validated by api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rp {

enum Dtype { kF32 = 0, kBF16 = 1 };

struct PregateArgs {
  const void* x;
  int T, d_in, ld_x;
  const void* Wg;
  int E, k;
  Dtype dt;
  int* topk_idx;
  float* topk_gate;
  float* logits;  // may be null
};
hipError_t launch_pregate(const PregateArgs& a, hipStream_t s);

// Router on the matrix cores (bf16, 64 < E <= kMaxE, E % 8 == 0).  The tile
// form needs no workspace (rp_pregate); the split form also runs the
// segmentation, with route_split_bytes(T, E) of workspace for its partial sums
// and 1 + route_split_tiles(T) arrival counters (zero before, zero after).
bool mfma_router_supported(Dtype dt, int E);
int route_split_tiles(int T);
size_t route_split_bytes(int T, int E);
hipError_t launch_route_mfma(const PregateArgs& a, hipStream_t s);

struct SegmentArgs {
  const int* topk_idx;
  int n_pairs;  // T * k
  int k;
  int E;
  int* seg_offsets;
  int* pair_perm;
  int* err_count;  // first word of the workspace
};
hipError_t launch_segment(const SegmentArgs& a, hipStream_t s);
hipError_t launch_route_segment_mfma(const PregateArgs& a, const SegmentArgs& sg, void* sums, int* counters,
                                     hipStream_t s);

constexpr int kMaxProj = 4;

struct ProjDesc {
  const void* W0;
  const void* A;
  const void* B;
  void* y;
  int d_out;
  int ld_y;
  int tile_begin;  // first output-row tile of this projection in the packed row space
  int tiled;       // W0 in the 16x32-block order of rp_pack_w0
  const void* residual;  // null, or [T, d_out] (leading dimension ld_y) added before the output rounding
};

struct SgmmArgs {
  ProjDesc proj[kMaxProj];
  int n_proj;
  const void* x;
  int T, d_in, ld_x;
  int E, r, k;
  const int* topk_idx;
  const float* topk_gate;
  const int* seg_offsets;
  const int* pair_perm;
  // workspace views
  float* u;          // [n_proj][T*k][r] gated rank-r intermediates
  float* partial;    // split-K partial tiles (decode path)
  int* counters;     // reserved counter region (decode path): epoch, control sets, split-K counters
  int n_tiles;       // output-row tiles over all projections
  int S;             // K splits per output tile (decode path)
  float* base;       // prefill with the expand in its own launch: fp32 base tiles [tile][T][128 rows]
  float* delta;      // ... and the adapter terms' sums, same layout
};

// Per-group launch constants of the decode kernel (the view its item
// functions take).  Items of a group are numbered
//   [0, n_shrink)          shrink: A-row tiles x SA splits (dense) or pair-chunk units
//   [n_shrink, n_items)    backbone tiles x S splits
struct DecodeArgs {
  int n_route, n_pre;  // routing items at the start of a fused launch
  int n_shrink, n_items;
  int units_per_proj;  // pair-chunk shrink units per projection (E > 32)
  int KP;              // K parts of a pair-chunk shrink unit (partial sums added in the expand)
  int dense;           // 1: the shrink runs as row tiles of the stacked A_e over every token (E <= 32);
                       // 0: pair-chunk shrink units of <= 16 pairs of one segment
  int atiles_per_proj, n_atiles, SA;  // dense: 32-row tiles of [A_0; ..; A_{E-1}] and their K splits
  int shrink_target;                  // shrink_done count that means every u is written (pair chunks)
  int t_pad;                          // tokens padded to whole 16-token tiles
  int fused;                          // routing runs inside the launch
  int group;                          // position of the group in its launch
  int prev_target;                    // > 0: wait until groups 0..group-1 have written this many tiles
  int x_acquire;                      // x was written earlier in this launch: acquire before reading it
  int count_done;                     // a later group waits for this one: count finished tiles
  int release;                        // ... and reads what this one wrote: release before counting
  float* partial_a;                   // dense: split-K partial tiles of the A tiles
  int act;                            // rp_act of the group (RP_ACT_SILU_MUL: projections 0, 1 pair up)
  int* pair_cnt;                      // act: arrival counter per output tile of projection 0
  unsigned int* route_tagged;         // fused: (index, tag, gate, tag) per (token, slot)
  PregateArgs pg;                     // fused: router arguments (outputs topk_idx, topk_gate)
  SegmentArgs sg;                     // fused: segmentation arguments
};

// Projection groups run in order inside one decode launch (a decode step or
// part of one); group g's items start reading their input only after every
// output tile of group g-1 is written.
constexpr int kMaxGroups = 8;
struct GroupPlan {
  int shrink_begin, base_begin;  // first shrink item and first backbone item of the group in the launch
  int n_shrink, n_items, shrink_target, units_per_proj, KP, atiles_per_proj, n_atiles, SA;
  int x_acquire, count_done, release;
  int wait_target;  // x_acquire: output tiles of every earlier group of the launch, else 0
  float* partial_a;
  int act;          // rp_act: with RP_ACT_SILU_MUL the second tile of a (gate, up) pair writes silu(g)*u
  int* pair_cnt;    // act: one arrival counter per output tile of projection 0 (zero before and after)
};
struct StepArgs {
  SgmmArgs g[kMaxGroups];
  GroupPlan gp[kMaxGroups];
  int n_groups, n_items;  // groups and items of the launch (routing items included)
  int n_route, n_pre, fused, dense, t_pad;
  int claim_all;  // every item, a workgroup's first too, is claimed from the launch's queue (launches that may
                  // run beside another: a waited-on item then always belongs to a running workgroup)
  unsigned int* route_tagged;
  PregateArgs pg;
  SegmentArgs sg;
};

// Which kernel family serves a call, and the workspace it needs.
struct SgmmPlan {
  int path;          // 0: fp32 VALU, 1: bf16 decode (T <= 64), 2: bf16 prefill
  int tile_rows;     // output rows per tile
  int n_tiles;
  int S;
  int t_pad;         // tokens padded to the decode token tiles
  int KP;            // decode: K parts per pair-chunk shrink unit
  int dense;         // decode: shrink as row tiles of the stacked A_e over all tokens
  int units_per_proj;
  int atiles_per_proj, n_atiles, SA;
  size_t off_partial_a, off_route;
  int n_pre, n_route;  // decode: routing items of a fused launch
  int n_items, grid;   // decode: work items and workgroups (grid <= resident capacity)
  int n_shrink;        // decode: shrink items among n_items
  size_t off_u, off_partial, off_counters, bytes;
};
// fused_route: the launch also runs the router and segmentation (decode path only)
SgmmPlan plan_sgmm(Dtype dt, int n_proj, const int* d_out, int T, int d_in, int E, int r, int k, int n_cu,
                   bool fused_route);

// A decode launch over several projection groups (bf16, T <= 64).
struct StepGroupDesc {
  int n_proj;
  const int* d_out;  // n_proj widths
  int d_in;
  int x_acquire;     // x is written by an earlier group of the same launch
};
struct StepPlan {
  int n_groups;
  SgmmPlan gp[kMaxGroups];  // per group: tiling, splits and its workspace offsets (absolute)
  int shrink_begin[kMaxGroups], base_begin[kMaxGroups];
  int n_route, n_pre, n_items, grid;
  size_t off_route, bytes;
};
StepPlan plan_step(const StepGroupDesc* groups, int n_groups, int T, int E, int r, int k, int n_cu, bool fused_route);
size_t step_workspace_upper_bound(const StepGroupDesc* groups, int n_groups, int T, int E, int r, int k);
hipError_t launch_step(const StepArgs& st, const StepPlan& plan, hipStream_t s);
int decode_mt(int T);       // 16-token tiles of the decode kernel
int decode_tile_rows(int T);  // output rows per decode item (16 per wave)
int decode_chunk_k(int T);  // K per LDS chunk of the decode kernel
int decode_resident_per_cu(int T, bool fused);  // workgroups of the decode kernel one CU holds at once
int fused_route_tile_tokens();                  // tokens per router tile of a fused decode launch
bool decode_fused_route_supported(int T, int E);  // routing can run inside a decode launch of T tokens

hipError_t launch_prefill(const SgmmArgs& a, const SgmmPlan& plan, hipStream_t s);
// Several bf16 prefill-shaped groups (T > 64) in one shrink launch and one
// GEMM launch; group g owns blocks [end[g-1], end[g]) of each.  Groups of one
// launch pair must not read each other's outputs.
struct PrefillStep {
  SgmmArgs g[kMaxGroups];
  int n_groups;
  int n_tok_tiles;                 // token tiles of prefill_tile_tokens(T) tokens
  int units;                       // shrink units per projection (same for every group)
  int shrink_end[kMaxGroups];      // cumulative shrink blocks
  int block_end[kMaxGroups];       // cumulative GEMM blocks (multiples of 8)
  int split_expand;                // 1: the GEMM stores fp32 base tiles and the expand runs as a launch of its own
  int expand_end[kMaxGroups];      // cumulative blocks of that expand launch
  int combine_end[kMaxGroups];     // cumulative blocks of the launch that adds base, delta and residual
};
hipError_t launch_prefill_step(const PrefillStep& ps, hipStream_t s);  // the three below, in order
hipError_t launch_prefill_shrink(const PrefillStep& ps, hipStream_t s);  // u of every group (needs the routing)
hipError_t launch_prefill_gemm(const PrefillStep& ps, hipStream_t s);    // W0 x (+ the expand unless split_expand)
hipError_t launch_prefill_expand(const PrefillStep& ps, hipStream_t s);  // split_expand: delta = B u (needs u)
hipError_t launch_prefill_combine(const PrefillStep& ps, hipStream_t s);  // split_expand: y = base + delta (+ residual)
// Reserved control region at the start of every workspace: two control blocks
// of kCounterBlockBytes; the second serves decode launches queued on the
// library's second stream.  Word offsets below are within a block.
constexpr size_t kCounterBlockBytes = 65536;
constexpr size_t kWorkspaceCounterBytes = 2 * kCounterBlockBytes;
// words [kPrefillCounterWord, + kPrefillCounterWords) of a block: split-K
// arrival counters of prefill GEMM tiles (each returns to zero when its tile
// completes); the decode control sets sit below
constexpr int kPrefillCounterWord = 9216;
// words [kRouteCounterWord, + kRouteCounterWords) of that region: arrival
// counters of the split-form router (below the decode control sets)
constexpr int kRouteCounterWord = 128;
constexpr int kRouteCounterWords = 1024 - kRouteCounterWord;
// decode launches leave the prefill counters unused: the (gate, up) tile-pair
// counters of groups with an activation take kActPairWords words per group
// there (each returns to zero when its pair completes)
constexpr int kActPairWords = 896;
constexpr int kPrefillCounterWords = (int)(kCounterBlockBytes / 4) - kPrefillCounterWord;
int prefill_splits(int d_in, int n_tiles, int T, int n_cu);          // K splits of one group's GEMM tiles
size_t prefill_partial_bytes(int n_tiles, int T, int S);            // its split-K partial tiles
int prefill_max_splits(int d_in);                                     // bound on prefill_splits for any device
size_t prefill_u_bytes(int n_proj, int T, int r, int k);  // one group's gated u, 256-byte aligned
int prefill_group_blocks(int n_tiles, int T);  // GEMM blocks of one group (one K split)
int prefill_units(int n_tiles, int T);         // (row tile, token tile) units of one group
int prefill_tile_rows(int T);                  // output rows per GEMM tile
int prefill_tile_tokens(int T);                // tokens per GEMM tile
int prefill_shrink_units(int T, int E, int k);  // shrink units per projection
// Many small segments (top-k >= 2 over many adapters, T <= 256): the GEMM stores
// its fp32 base tiles and a separate expand launch adds the adapters' deltas.
bool prefill_split_expand(int T, int E, int r, int k);
size_t prefill_base_bytes(int n_tiles, int T);  // one group's fp32 base and delta tiles
int prefill_expand_blocks(int n_tiles, int T);  // expand blocks of one group (a multiple of 8)
int prefill_combine_blocks(int n_tiles, int T); // combine blocks of one group
hipError_t launch_f32(const SgmmArgs& a, const SgmmPlan& plan, hipStream_t s);
int f32_tile_rows();  // output rows per fp32 workgroup
size_t sgmm_workspace_upper_bound(Dtype dt, int n_proj, int T, int d_in, long long sum_d_out, int E, int r,
                                  int k);
hipError_t launch_sgmm(const SgmmArgs& a, const SgmmPlan& plan, Dtype dt, hipStream_t s);


// One adapter's gated delta added in place to its segment's outputs (tiles of
// adapter_apply_tile_rows() rows over the group's projections).
hipError_t launch_adapter_apply(const SgmmArgs& a, int e, Dtype dt, hipStream_t s);
int adapter_apply_tile_rows();

// In-place merge (sign +1) or unmerge (sign -1) of n_sel weighted adapters into W0.
struct MergeArgs {
  void* W0;
  int tiled;  // W0 in the rp_pack_w0 order
  int d_out, d_in;
  const void* A;  // [E, r, d_in]
  const void* B;  // [E, d_out, r]
  int E, r;
  const int* sel;        // device: n_sel adapter indices
  const float* weights;  // device: n_sel weights
  int n_sel;
  float sign;
};
hipError_t launch_merge(const MergeArgs& m, Dtype dt, hipStream_t s);

hipError_t launch_pack_w0(const void* src, void* dst, int d_out, int d_in, hipStream_t s);
hipError_t launch_rmsnorm(const void* x, int T, int d, int ld_x, const void* gamma, float eps, void* y, int ld_y,
                          Dtype dt, hipStream_t s);
hipError_t launch_silu_mul(const void* g, int ld_g, const void* u, int ld_u, int T, int d, void* m, int ld_m,
                           Dtype dt, hipStream_t s);
hipError_t launch_stream_read(const void* src, size_t n_bytes, float* sink, hipStream_t s);
hipError_t launch_copy(void* dst, const void* src, size_t n_bytes, hipStream_t s);

}  // namespace rp
