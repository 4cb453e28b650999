/*
 * rank_pregate.h -- C ABI of the pre-gated multi-adapter low-rank projection
 * library for AMD Instinct MI355X (gfx950).
 *
 * The operation (AdaFuse, "Accelerating Dynamic Adapter Inference via
 * Token-Level Pre-Gating and Fused Kernel Optimization", technical summary §2):
 *
 *   rp_pregate    -- §2.A token-level pre-gating and §2.B decoding steps 1-2: a
 *                    light linear router scores every token once and keeps its
 *                    top-k adapters; the choice then holds for every layer.
 *   rp_segment    -- groups the (token, slot) pairs by adapter, giving the
 *                    segments the segmented gather matrix multiply runs over.
 *   rp_sgmm_fused -- §2.B SGMM and decoding step 3: base projection plus the
 *                    gated low-rank deltas of the chosen adapters, in one pass:
 *                       y[t] = W0 x[t] + sum_j g[t,j] B_e (A_e x[t]),  e = idx[t,j]
 *                    for up to four projections that share x and the gate.
 *   rp_route_sgmm_fused -- the three steps above for the first adapted layer
 *                    of a step, whose input is also the router input: one
 *                    launch for decode shapes, so routing overlaps the weights.
 *   rp_sgmm_step  -- a decode step: many projection groups in dependency
 *                    order (q|k|v, o, gate|up, down, layer after layer), the
 *                    routing optionally computed first, as few launches as
 *                    possible ("FlashSVD v1.5: Making Low-Rank Transformers
 *                    Inference Actually Fast", La Solución: gate and up
 *                    packed into one wide operation, and the per-token
 *                    routine recorded once and replayed as a unit).
 *
 * Conventions shared by every entry point
 *   - Every data pointer is DEVICE memory owned by the caller.  The library
 *     allocates no device memory and keeps no state besides a per-device
 *     property cache and a thread-local error message.
 *   - Matrices are row-major.  Sizes and leading dimensions count elements.
 *   - Work is queued on `stream` (0 = the null stream) and returns at once;
 *     results are valid once the stream is synchronised or ordered after.
 *   - Argument checks happen on the host, before any launch; a failing check
 *     returns a non-OK status, launches nothing and records a message readable
 *     through rp_last_error().  No C++ exception crosses this boundary.
 *   - Calls are thread-safe on distinct streams with distinct workspaces.
 *   - Inputs must be finite; behaviour on NaN or Inf is unspecified.
 */
#ifndef RANK_PREGATE_H
#define RANK_PREGATE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RP_ABI_VERSION 7
#define RP_MAX_K 8          /* largest top-k */
#define RP_MAX_E 1024       /* largest adapter count */
#define RP_MAX_PROJ 4       /* projections per rp_sgmm_fused call (per group) */
#define RP_MAX_GROUPS 4096  /* projection groups per rp_sgmm_step call */

typedef enum {
  RP_OK = 0,
  RP_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, size or count out of range */
  RP_ERR_UNSUPPORTED = 2,   /* well-formed but outside what the kernels implement */
  RP_ERR_WORKSPACE = 3,     /* workspace missing, misaligned or too small */
  RP_ERR_HIP = 4,           /* a HIP runtime call or kernel launch failed */
  RP_ERR_DEVICE = 5         /* rp_workspace_status: a kernel flagged a fault in the workspace */
} rp_status;

typedef enum { RP_F32 = 0, RP_BF16 = 1 } rp_dtype;

/* Storage order of a backbone weight W0.
 *   RP_W0_ROWS   dense row-major [d_out, d_in]
 *   RP_W0_TILED  the order rp_pack_w0 writes (bf16 only): blocks of 16 rows x 32
 *                columns (nb = d_in/32 block columns, n_rb = d_out/16 row
 *                blocks), grouped in chunks of four block columns.  Chunk g
 *                (block columns 4g .. 4g+nbg-1, nbg = min(4, nb - 4g)) starts at
 *                element 4g * n_rb * 512 and holds its blocks row block by row
 *                block: block (rb, cb) at element offset
 *                (4g * n_rb + rb * nbg + cb - 4g) * 512, g = cb / 4.  Inside a
 *                block, 64 groups of 8 consecutive columns, group q holding row
 *                16*rb + q%16, columns 32*cb + 8*(q/16) .. +7.  A decode launch
 *                reads the same chunk of every row block at about the same
 *                time, and those blocks are contiguous. */
typedef enum { RP_W0_ROWS = 0, RP_W0_TILED = 1 } rp_w0_layout;

/* One adapted projection (one linear layer with its adapter bank).
 *   W0 [d_out, d_in]     backbone weight, in the storage order w0_layout names
 *   A  [E, r, d_in]      adapter down-projections, dense, one block per adapter
 *   B  [E, d_out, r]     adapter up-projections, dense, one block per adapter
 *   y  [T, d_out]        output, leading dimension ld_y (>= d_out)
 *   residual [T, d_out]  NULL, or a tensor added to the output before its one
 *                        rounding (a decoder layer's residual stream), with the
 *                        leading dimension ld_y; it may be y itself (updated
 *                        in place) but must not otherwise overlap y
 * All have the call's dtype.  y must not alias any other input.
 * RP_W0_TILED needs bf16, d_out % 16 == 0 and d_in % 32 == 0; reserved must be 0. */
typedef struct {
  const void* W0;
  const void* A;
  const void* B;
  void* y;
  int64_t d_out;
  int64_t ld_y;
  int32_t w0_layout;
  int32_t reserved;
  const void* residual;
} rp_proj;

/* Token-level pre-gating (AdaFuse §2.A; §2.B decoding steps 1-2).
 *
 *   logits[t,e] = sum_i x[t,i] * Wg[i,e]            fp32 accumulation
 *   topk_idx[t,0..k-1]  = the k adapters with the largest logits, best first;
 *                         an exact tie goes to the lower adapter index
 *   topk_gate[t,j]      = exp(l_j - l_0) / sum_j' exp(l_j' - l_0) over the k
 *                         chosen logits (softmax over the selection; 1.0 when k=1)
 *
 *   x       [T, d_in], leading dimension ld_x, dtype dt
 *   Wg      [d_in, E], dense, dtype dt
 *   topk_idx  int32 [T, k], dense          (output)
 *   topk_gate fp32  [T, k], dense          (output)
 *   logits_or_null  fp32 [T, E], dense, or NULL to skip (output)
 *
 * The sum over i runs in the same order for every adapter column, so equal
 * router columns give bit-equal logits and the tie rule is exact.
 * Limits: 1 <= k <= min(E, RP_MAX_K), 1 <= E <= RP_MAX_E, d_in >= 1 and a
 * multiple of 8 (bf16) or 4 (fp32); x, Wg 16-byte aligned, ld_x*sizeof(dt) a
 * multiple of 16; T = 0 is a no-op. */
rp_status rp_pregate(const void* x, int64_t T, int64_t d_in, int64_t ld_x, const void* Wg, int64_t E,
                     int32_t k, rp_dtype dt, int32_t* topk_idx, float* topk_gate, float* logits_or_null,
                     hipStream_t stream);

/* Segmentation: group the pairs p = t*k + j by adapter (the segments of the
 * segmented gather matrix multiply, AdaFuse §2.B).
 *
 *   seg_offsets int32 [E+1] (output): segment e is pair_perm[seg_offsets[e] ..
 *                                     seg_offsets[e+1]); seg_offsets[0] = 0
 *   pair_perm   int32 [T*k] (output): pair ids grouped by ascending adapter and,
 *                                     inside a segment, by ascending pair id
 *   ws          device workspace of at least rp_segment_workspace_size() bytes,
 *               4-byte aligned; its first int32 receives the number of pairs
 *               whose index was outside [0, E).  Such pairs are left out of
 *               every segment (seg_offsets[E] counts only the valid pairs) and
 *               the tail of pair_perm is then left unwritten.
 * Runs as one workgroup.  Limits: 0 <= k <= RP_MAX_K, 1 <= E <= RP_MAX_E,
 * T*k < 2^31.  T = 0 or k = 0 writes all-zero offsets. */
rp_status rp_segment(const int32_t* topk_idx, int64_t T, int32_t k, int64_t E, int32_t* seg_offsets,
                     int32_t* pair_perm, void* ws, size_t ws_bytes, hipStream_t stream);
size_t rp_segment_workspace_size(int64_t T, int32_t k, int64_t E);

/* Fused pre-gated SGMM (AdaFuse §2.B): for each of the n_proj projections,
 *
 *   y[t,:] = W0 x[t,:] + sum_{j<k} topk_gate[t,j] * B_e (A_e x[t,:]),  e = topk_idx[t,j]
 *
 * with fp32 accumulation and one rounding to dt on the final store.  The
 * adapter work follows the segments of rp_segment (each chosen adapter's A
 * and B are read once per output tile).  k = 0 computes the base projection
 * only (topk_*, seg_offsets, pair_perm may then be NULL).
 *
 *   projs      host array of n_proj (1..RP_MAX_PROJ) descriptors sharing x and
 *              the gate, e.g. q|k|v or gate|up (the descriptor array itself is
 *              read during the call and not kept)
 *   x          [T, d_in], leading dimension ld_x
 *   topk_idx, topk_gate, seg_offsets, pair_perm   as produced above
 *   ws         device workspace of at least rp_sgmm_workspace_size() bytes,
 *              256-byte aligned.  Its first 64 KiB are a control region that
 *              must be zero before the first call (zero-fill the buffer once)
 *              and is then kept consistent by the calls themselves: do not
 *              write it between calls.  One workspace serves calls of any
 *              shape in sequence; calls that may overlap in time need distinct
 *              workspaces.
 * Limits: r in {8,16,32,64,128}; 0 <= k <= min(E, RP_MAX_K); 1 <= E <=
 * RP_MAX_E; d_in a multiple of 8 (bf16) / 4 (fp32); d_out a multiple of 8;
 * all matrix pointers 16-byte aligned and ld_x*sizeof(dt), ld_y*sizeof(dt)
 * multiples of 16; T = 0 is a no-op. */
rp_status rp_sgmm_fused(const rp_proj* projs, int32_t n_proj, const void* x, int64_t T, int64_t d_in,
                        int64_t ld_x, int64_t E, int64_t r, int32_t k, const int32_t* topk_idx,
                        const float* topk_gate, const int32_t* seg_offsets, const int32_t* pair_perm,
                        rp_dtype dt, void* ws, size_t ws_bytes, hipStream_t stream);

/* Pre-gating, segmentation and the fused SGMM in one call (AdaFuse §2.A-§2.B),
 * for the first adapted projection group of a step: x is both the router input
 * and the input of the projections.  Equivalent to
 *
 *   rp_pregate(x, T, d_in, ld_x, Wg, E, k, dt, topk_idx, topk_gate, NULL)
 *   rp_segment(topk_idx, T, k, E, seg_offsets, pair_perm, ...)
 *   rp_sgmm_fused(projs, n_proj, x, ..., topk_idx, topk_gate, seg_offsets, pair_perm, ...)
 *
 * with bit-identical routing outputs, which later groups of the same step then
 * pass to rp_sgmm_fused.  For decode shapes (bf16, T <= 32, E <= 64)
 * everything runs in one kernel launch whose router and segmentation finish
 * while the backbone weights stream; bf16 with 64 < E (E a multiple of 8)
 * routes and segments in one launch of its own on the matrix cores (the
 * routing is bit-identical to rp_pregate's); other shapes issue the three
 * launches in order.
 *
 *   Wg        [d_in, E], dense, dtype dt (the router weight)
 *   topk_idx  int32 [T, k], topk_gate fp32 [T, k], seg_offsets int32 [E+1],
 *   pair_perm int32 [T*k]  (outputs, as rp_pregate / rp_segment define them)
 *   ws        as for rp_sgmm_fused, rp_sgmm_workspace_size() bytes
 * Limits: those of rp_pregate and rp_sgmm_fused, and k >= 1. */
rp_status rp_route_sgmm_fused(const rp_proj* projs, int32_t n_proj, const void* x, int64_t T, int64_t d_in,
                              int64_t ld_x, const void* Wg, int64_t E, int64_t r, int32_t k, rp_dtype dt,
                              int32_t* topk_idx, float* topk_gate, int32_t* seg_offsets, int32_t* pair_perm,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* Activation a group applies to its outputs (rp_group.act).
 *   RP_ACT_NONE       the projections' outputs as they are
 *   RP_ACT_SILU_MUL   gated MLP input: the group has two projections of equal
 *                     d_out (gate, then up; packed as in "FlashSVD v1.5", La
 *                     Solución) and projs[0].y receives
 *                        m = round(silu(g) * u),  silu(g) = g / (1 + exp(-g)),
 *                     from the rounded outputs g (projection 0) and u
 *                     (projection 1), in fp32 -- the values rp_silu_mul gives
 *                     on them -- while projs[1].y keeps u. */
typedef enum { RP_ACT_NONE = 0, RP_ACT_SILU_MUL = 1 } rp_act;

/* One group of projections that share their input x (see rp_sgmm_fused). */
typedef struct {
  const rp_proj* projs;  /* host array of n_proj (1..RP_MAX_PROJ) descriptors */
  int32_t n_proj;
  int32_t x_from_call;   /* 1 if x is written by an earlier group of the same call */
  const void* x;         /* [T, d_in], leading dimension ld_x */
  int64_t d_in;
  int64_t ld_x;
  int32_t act;           /* rp_act */
  int32_t reserved;      /* must be 0 */
} rp_group;

/* A decode step (AdaFuse §2.B decoding steps 1-3 over every adapted layer).
 * A group marked x_from_call reads its x (and its projections' residuals)
 * only after every output of the groups before it is written, so its x and
 * residuals may be any earlier group's y.  A group without the mark does not
 * wait and may run concurrently with earlier groups: neither its x nor its
 * residuals may be written by this call.  No y may overlap another
 * y or any group's x.  All groups use one routing:
 *
 *   Wg_or_null non-null: the routing is computed first from groups[0].x, as
 *                        rp_route_sgmm_fused does; topk_idx, topk_gate,
 *                        seg_offsets, pair_perm are outputs
 *   Wg_or_null NULL:     they are inputs (as for rp_sgmm_fused)
 *
 * For decode shapes (bf16, T <= 64) the groups run inside multi-group
 * launches (up to eight groups each): a group's first weight chunk is already
 * streaming while it waits for the previous group, and no launch boundary
 * separates them.  Other shapes run group by group.
 *   ws   rp_sgmm_step_workspace_size() bytes, same rules as rp_sgmm_fused
 * Limits: 1 <= n_groups <= RP_MAX_GROUPS, each group as for rp_sgmm_fused; E, r,
 * k shared by all groups; k >= 1 when the routing is computed. */
rp_status rp_sgmm_step(const rp_group* groups, int32_t n_groups, int64_t T, int64_t E, int64_t r, int32_t k,
                       const void* Wg_or_null, int32_t* topk_idx, float* topk_gate, int32_t* seg_offsets,
                       int32_t* pair_perm, rp_dtype dt, void* ws, size_t ws_bytes, hipStream_t stream);
size_t rp_sgmm_step_workspace_size(const rp_group* groups, int32_t n_groups, int64_t T, int64_t E, int64_t r,
                                   int32_t k, rp_dtype dt);

/* rp_sgmm_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments without ws / ws_bytes, the same kernels and results.  The
 * workspace is a static device array of 64 MiB (64 << 20 bytes) that each GPU
 * the library runs on holds until the process ends; a call whose
 * rp_sgmm_step_workspace_size exceeds it returns RP_ERR_WORKSPACE and launches
 * nothing.  The first call on a device looks up that device's array and
 * clears its control region with a kernel on `stream`; that first call must
 * not be recorded into a graph (RP_ERR_INVALID_ARG), later ones may be.  All
 * calls on one GPU share the array: calls that may overlap in time on one GPU
 * (other streams, other host threads) race and give undefined results.  No
 * hipMalloc, hipFree or other allocating routine is called. */
rp_status rp_sgmm_step_noalloc(const rp_group* groups, int32_t n_groups, int64_t T, int64_t E, int64_t r,
                               int32_t k, const void* Wg_or_null, int32_t* topk_idx, float* topk_gate,
                               int32_t* seg_offsets, int32_t* pair_perm, rp_dtype dt, hipStream_t stream);

/* Repack a dense row-major bf16 W0 [d_out, d_in] into RP_W0_TILED order (a
 * one-time weight preparation; the result serves every later call).
 * d_out % 16 == 0, d_in % 32 == 0, src and dst 16-byte aligned and disjoint. */
rp_status rp_pack_w0(const void* src, void* dst, int64_t d_out, int64_t d_in, rp_dtype dt, hipStream_t stream);

/* Workspace bytes rp_sgmm_fused needs for these sizes, an upper bound valid on
 * any device; sum_d_out is the sum of
 * the projections' d_out.  Returns 0 for sizes the call would reject.
 * Besides the rank-r intermediates (T*k*r per projection), the workspace holds
 * the split-K partial tiles of long-K or few-tile calls: their count follows
 * the output tiles over all projections (sum_d_out) and the K splits (d_in). */
size_t rp_sgmm_workspace_size(int32_t n_proj, int64_t T, int64_t d_in, int64_t sum_d_out, int64_t E,
                              int64_t r, int32_t k, rp_dtype dt);

/* One adapter's gated low-rank delta added in place to the outputs of the
 * tokens in its segment, for every projection of a group (the unfused form:
 * a base projection, e.g. rp_sgmm_fused with k = 0, then one call per adapter;
 * the "simple fusion" that AdaFuse's ablation, technical summary §4, measures
 * against SGMM, and the per-adapter launches its §1 blames for latency):
 *
 *   y[t,:] += topk_gate[t,j] * B_e (A_e x[t,:])   for every pair p = t*k + j
 *                                                 in pair_perm[seg_offsets[e] ..
 *                                                 seg_offsets[e+1]),  e = adapter
 *
 * y is read and written (it must already hold the base projection); each
 * pair's delta is accumulated in fp32 and added with one rounding to dt, pairs
 * of the segment in order.  W0 is not read.  projs, x, T, d_in, ld_x, E, r, k,
 * dt as for rp_sgmm_fused; 0 <= adapter < E; k >= 1; seg_offsets / pair_perm
 * as rp_segment writes them, topk_gate as rp_pregate writes it.  No workspace.
 * The segment's size is read on the device, so a call can be recorded into a
 * graph before the routing is known; an empty segment launches a no-op. */
rp_status rp_adapter_apply(const rp_proj* projs, int32_t n_proj, const void* x, int64_t T, int64_t d_in,
                           int64_t ld_x, int64_t E, int64_t r, int32_t k, int32_t adapter, const float* topk_gate,
                           const int32_t* seg_offsets, const int32_t* pair_perm, rp_dtype dt, hipStream_t stream);

/* In-place merge of weighted adapters into a backbone weight, or its inverse
 * (AdaFuse technical summary §2.B, decoding steps 3 and 5: the selected
 * experts are folded into the backbone, the backbone runs, and they are
 * unfolded for the next token):
 *
 *   W0[o,i] <- round_dt(W0[o,i] + sign * sum_{j<n_sel} weights[j] * sum_c B[e_j,o,c] A[e_j,c,i]),
 *   e_j = sel[j]
 *
 * The rank sum runs in fp32 in (j, c) order and is added to W0 in fp32, then
 * rounded to dt.  With bf16 a merge followed by an unmerge does not in general
 * restore W0 bit for bit (each rounds): the factorised path (rp_sgmm_fused)
 * never writes W0.
 *
 *   W0       [d_out, d_in] in w0_layout order (read and written)
 *   A, B     [E, r, d_in], [E, d_out, r], dtype dt
 *   sel      device int32 [n_sel]: adapter indices (e.g. one token's topk_idx
 *            row); an index outside [0, E) contributes nothing
 *   weights  device fp32 [n_sel] (e.g. that token's topk_gate row)
 *   sign     +1 to merge, -1 to unmerge (any finite value scales the delta)
 * Limits: d_in a multiple of 8; RP_W0_TILED as for rp_proj; r in
 * {8,16,32,64,128}; 0 <= n_sel <= RP_MAX_K (0 is a no-op).  No workspace. */
rp_status rp_merge_adapters(void* W0, int32_t w0_layout, int64_t d_out, int64_t d_in, const void* A, const void* B,
                            int64_t E, int64_t r, const int32_t* sel, const float* weights, int32_t n_sel, float sign,
                            rp_dtype dt, hipStream_t stream);

/* Device-side health of an SGMM workspace (one used by rp_sgmm_fused,
 * rp_route_sgmm_fused or rp_sgmm_step).  Kernels that hand data between
 * workgroups of one launch wait for it with bounded polls; a wait that runs
 * out (possible only if the launch's workgroups are not all resident at once,
 * e.g. another program occupies the device's compute units) gives up and sets
 * a sticky word in the workspace, and the outputs of that call are then not
 * valid.  Routing computed by these calls also counts, in a second word,
 * pairs whose adapter index was outside [0, E) (always 0 for indices the
 * router wrote).
 *
 *   ws, ws_bytes     the workspace (at least 64 KiB, 256-byte aligned)
 *   wait_overflow    host int32 out, or NULL: nonzero if a wait gave up
 *   bad_indices      host int32 out, or NULL: out-of-range indices counted
 *   clear            nonzero: reset both words after reading them
 *
 * Orders after the work queued on `stream`: queues a copy of the two words,
 * then waits for the stream (so it cannot be recorded into a graph).  Returns
 * RP_ERR_DEVICE when either word is nonzero, RP_OK when both are zero. */
rp_status rp_workspace_status(void* ws, size_t ws_bytes, int32_t clear, int32_t* wait_overflow,
                              int32_t* bad_indices, hipStream_t stream);

/* RMSNorm of each token row: the normalisation in front of the attention and
 * MLP projections of a Llama-style decoder layer (the 7B models AdaFuse
 * measures latency on, technical summary §4), part of the base model's
 * standard inference that decoding step 4 of §2.B runs between the adapted
 * projections:
 *
 *   y[t,i] = round(x[t,i] * inv[t] * gamma[i]),
 *   inv[t] = 1 / sqrt(sum_i x[t,i]^2 / d + eps)      fp32, fixed summation order
 *
 *   x [T, d] (ld_x), gamma [d], y [T, d] (ld_y), dtype dt; y may be x.
 * Limits: d a multiple of 8 (bf16) / 4 (fp32), d <= 65536; pointers 16-byte
 * aligned, ld*sizeof(dt) multiples of 16; eps >= 0 finite; T = 0 is a no-op. */
rp_status rp_rmsnorm(const void* x, int64_t T, int64_t d, int64_t ld_x, const void* gamma, float eps, void* y,
                     int64_t ld_y, rp_dtype dt, hipStream_t stream);

/* Gated MLP activation as its own launch (what RP_ACT_SILU_MUL fuses):
 *   m[t,i] = round(silu(g[t,i]) * u[t,i]),  silu(g) = g / (1 + exp(-g)), fp32.
 *   g, u, m [T, d] with leading dimensions ld_g, ld_u, ld_m; m may be g or u.
 * Limits as for rp_rmsnorm. */
rp_status rp_silu_mul(const void* g, int64_t ld_g, const void* u, int64_t ld_u, int64_t T, int64_t d, void* m,
                      int64_t ld_m, rp_dtype dt, hipStream_t stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* rp_last_error(void);

/* RP_ABI_VERSION of the built library. */
int rp_abi_version(void);

/* ---- measurement helpers (not part of the method) ------------------------
 * rp_util_stream_read: reads n_bytes (multiple of 16, 16-byte aligned) from
 * src with coalesced 16-byte loads and writes one fp32 checksum per workgroup
 * to sink[0..1023]; gives the achievable HBM read bandwidth of the device.
 * rp_util_copy: copies n_bytes (multiple of 16, both 16-byte aligned) from src
 * to dst; a kernel of known traffic for scaling hardware byte counters. */
rp_status rp_util_stream_read(const void* src, size_t n_bytes, float* sink, hipStream_t stream);
rp_status rp_util_copy(void* dst, const void* src, size_t n_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* RANK_PREGATE_H */
