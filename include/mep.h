/*
 * mep.h - C ABI of the balanced expert-parallel MoE hot path (MI355X, gfx950).
 *
 * One GPU computes, for a logical expert-parallel world of R ranks:
 *   - the global plan that every rank would compute identically
 *     (mep_plan), and this rank's send and receive maps;
 *   - the EPLB logical-to-physical expert remap with score pruning
 *     (mep_remap_prune);
 *   - this rank's pack into per-destination send segments and the grouping
 *     of received rows by expert instance (mep_dispatch);
 *   - the score-weighted K-way reduction of returned expert outputs
 *     (mep_combine).
 *
 * Sources, cited by page title and section:
 *   [MoonEP-TD]  "MoonEP" technical overview (twodots.gr), architecture and
 *                memory-contract sections: every EP rank processes exactly
 *                S*K routed rows; temporary redundant expert copies planned
 *                online on the GPU from the router output; tokens land at
 *                their final position grouped by expert; planner-made
 *                cu_seqlens; static S*K buffers so no per-layer host sync.
 *   [MoonEP-API] "MoonEP API完全参考" (stapisi.com), sections 2.2 (planning)
 *                and 3.1 (dispatch and combine).
 *   [UpdExp]     "aclnnMoeUpdateExpert" op doc: "功能说明" (remap and pruning
 *                formulas), "函数原型"/"参数说明" (two-phase API, parameters),
 *                "返回值" (status codes), "约束说明" (constraints).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked (host). The caller owns
 *     every buffer; the library never allocates device memory and keeps
 *     no state between calls, except mep_plan_noalloc's static device
 *     array (see there), which holds its workspace.
 *   - bf16 data is passed as raw 16-bit patterns (uint16_t); ids, tables
 *     and maps are int32_t; masks are uint8_t holding 0 or 1.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream). Calls
 *     only enqueue work: no host synchronisation, no host read of device
 *     data. Outputs are complete when the stream reaches that point.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     an error status nothing has been enqueued. Device-side VALUES (ids in
 *     range, table entries valid, maps forming the stated permutations) are
 *     the caller's responsibility, as in [UpdExp] "参数说明" (the table's
 *     values must be correct); kernels clamp their own reads so that bad
 *     values give wrong results, not out-of-bounds accesses (an
 *     out-of-range row index skips that row).
 *   - Row pointers (x, send_buf, recv_raw, recv_grouped, y_ret, out_bf16,
 *     out_f32) must be 16-byte aligned and H a multiple of 8.
 *   - Every output is a pure function of the inputs (no order-dependent
 *     atomics), as [UpdExp] "约束说明" asks (deterministic by default).
 *   - Calls are reentrant; concurrent calls must not share output buffers
 *     (nor, for mep_plan_noalloc, overlap on one GPU).
 */
#ifndef MEP_H
#define MEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. The three argument errors mirror the op doc's
 * ACLNN_ERR_PARAM_NULLPTR, ACLNN_ERR_PARAM_INVALID and
 * ACLNN_ERR_INNER_TILING_ERROR ([UpdExp] "返回值"). */
typedef enum {
    MEP_OK = 0,
    MEP_ERR_NULLPTR = 1, /* a required pointer is NULL */
    MEP_ERR_PARAM = 2,   /* bad mode, unpaired optional arguments, rank out
                            of range, workspace too small, K > E */
    MEP_ERR_SHAPE = 3,   /* a size out of the supported range, H % 8 != 0,
                            a row pointer not 16-byte aligned */
    MEP_ERR_HIP = 4      /* the HIP runtime reported an error at launch */
} mep_status;

/* Human-readable name of a status (static string, never NULL). */
const char* mep_status_str(int status);

/* Library version as major*10000 + minor*100 + patch. */
int mep_version(void);

/* ------------------------------------------------------------------ plan */

/* Supported plan sizes: 1 <= R <= 1024, 1 <= E <= 1024, 1 <= K <= E,
 * S >= 1, R*S*K <= 2^30. */

/*
 * Bytes of device workspace mep_plan needs for these sizes (host-only, pure
 * function; [UpdExp] "函数原型": size query before execution). Returns 0 if
 * the sizes are unsupported.
 */
size_t mep_plan_workspace_size(int R, int E, int S, int K);

/*
 * mep_plan - global balanced plan and rank `my_rank`'s maps.
 *
 * [MoonEP-TD] invariant: each of the R ranks receives exactly C = S*K
 * routed rows. With home(e) = floor(e*R/E), native loads
 * L[r] = sum of cnt[e] over home(e) = r, and routes f = g*K + k
 * (g = src*S + s) taken in (expert, g, k) order:
 *   - each rank keeps the first C of its routes at slots 0..C-1 in order;
 *   - the remaining routes of over-loaded ranks, in the same global order,
 *     fill the under-loaded ranks in ascending rank order, rank u taking
 *     C - L[u] routes at slots L[u], L[u]+1, ...; each (expert, rank != home)
 *     pair so created is a redundant instance.
 * Rank u's local layout (its grouped receive buffer; the row offsets are the
 * cu_seqlens of [MoonEP-TD]): native experts in ascending e (zero-row
 * natives keep their place), then redundant instances in ascending e. A
 * global instance id (gid) numbers instances in (rank, local index) order.
 *
 * Inputs:
 *   topk_ids   [R*S*K] int32, row-major [R][S][K]: the whole routing table;
 *              values in [0, E).
 *   workspace  device buffer of at least mep_plan_workspace_size() bytes,
 *              256-byte aligned; contents on entry do not matter; clobbered.
 * Outputs (all int32, all overwritten):
 *   expert_count  [E]      routes per expert.
 *   rank_load     [R]      native loads L[r] (before balancing).
 *   route_dest    [R*S*K]  destination rank of each route   (may be NULL).
 *   route_slot    [R*S*K]  slot on that rank, in [0, C)      (may be NULL;
 *                          NULL together with route_dest).
 *   inst_count    [R]      instances per rank (natives + redundant).
 *   inst_expert   [R][E]   expert of local instance i; -1 past inst_count.
 *   inst_cu       [R][E+1] row offset of local instance i; entries past
 *                          inst_count hold C.
 *   inst_gid_base [R+1]    exclusive prefix of inst_count.
 *   send_pos      [S*K]    row of route (my_rank, s, k) in the send buffer,
 *                          ordered by (destination, destination slot).
 *   send_count    [R]      rows sent to each destination.
 *   recv_pos      [C]      for grouped slot t of my_rank, the row of the
 *                          source-major arrival buffer (sources ascending,
 *                          each source's rows in slot order) holding it.
 *   recv_count    [R]      rows received from each source.
 * Errors: MEP_ERR_NULLPTR (required pointer NULL), MEP_ERR_SHAPE (sizes),
 *   MEP_ERR_PARAM (my_rank out of range, K > E, workspace too small or
 *   misaligned, only one of route_dest/route_slot given), MEP_ERR_HIP.
 */
int mep_plan(int R, int E, int S, int K, int my_rank,
             const int32_t* topk_ids, void* workspace, size_t workspace_bytes,
             int32_t* expert_count, int32_t* rank_load,
             int32_t* route_dest, int32_t* route_slot,
             int32_t* inst_count, int32_t* inst_expert, int32_t* inst_cu,
             int32_t* inst_gid_base,
             int32_t* send_pos, int32_t* send_count,
             int32_t* recv_pos, int32_t* recv_count,
             void* stream);

/*
 * mep_plan_noalloc - mep_plan with no workspace argument and no allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Computes exactly what mep_plan computes (same kernels, same outputs, same
 * argument meaning and errors), with the workspace taken from a static
 * device array of MEP_PLAN_NOALLOC_SCRATCH_BYTES inside the library. Each
 * GPU the library runs on holds its own copy of that array until the
 * process ends; its device address is looked up on the first call on each
 * device. Nothing is allocated (no hipMalloc, no library allocation) at any
 * call. The device current at the call must be the stream's device.
 *
 * Limit: sizes whose mep_plan_workspace_size() exceeds
 * MEP_PLAN_NOALLOC_SCRATCH_BYTES (4 MiB) return MEP_ERR_SHAPE and enqueue
 * nothing. For scale: R=8, E=256, S=4096, K=8 needs 0.28 MB and R=64,
 * E=256, S=8192, K=8 0.61 MB; R = E = 1024 needs 8.5 MB and is refused.
 *
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (on different streams, or from several threads) race on it and give
 * undefined outputs; serialize them (one stream, or events between them).
 * The plan's outputs do not depend on what the array holds on entry, so it
 * needs no clearing between calls.
 * Errors: as mep_plan (no workspace errors), plus MEP_ERR_SHAPE for sizes
 * beyond the array and MEP_ERR_HIP if the array's address cannot be found.
 */
#define MEP_PLAN_NOALLOC_SCRATCH_BYTES (4u << 20)
int mep_plan_noalloc(int R, int E, int S, int K, int my_rank,
                     const int32_t* topk_ids,
                     int32_t* expert_count, int32_t* rank_load,
                     int32_t* route_dest, int32_t* route_slot,
                     int32_t* inst_count, int32_t* inst_expert, int32_t* inst_cu,
                     int32_t* inst_gid_base,
                     int32_t* send_pos, int32_t* send_count,
                     int32_t* recv_pos, int32_t* recv_count,
                     void* stream);

/* ---------------------------------------------------------- remap / prune */

/* Scale element types accepted by mep_remap_prune ([UpdExp] "参数说明":
 * FLOAT, BFLOAT16, FLOAT16). */
enum { MEP_SCALE_F32 = 0, MEP_SCALE_BF16 = 1, MEP_SCALE_F16 = 2 };

/*
 * mep_remap_prune - EPLB logical -> physical instance remap and pruning
 * ([UpdExp] "功能说明").
 *
 * Remap, for token t and slot k, e = expert_ids[t*K+k],
 * count = eplb_table[e*F] (instances of e, in [1, F-1]):
 *   count == 1        -> column 1
 *   balance_mode == 0 -> column local_rank_id / ceil(world_size/count) + 1
 *   balance_mode == 1 -> column (t mod count) + 1
 *   balanced_ids[t*K+k] = eplb_table[e*F + column]
 * Pruning (only with expert_scales and pruning_threshold), scales widened
 * exactly to fp32:
 *   thr_sum[t] = sum over k = 0..K-1 of fl(scale[t,k] * threshold[k]),
 *                accumulated in k order from +0.0f, each step rounded to fp32
 *   balanced_mask[t*K+k] = active[t] && !(scale[t,k] < thr_sum[t])
 * (a route below the token's sum is pruned; a tie is kept; every route of
 * an inactive token is pruned). Without scales and threshold the mask is
 * all ones. Pruned routes still receive a remapped id.
 * Send map (when send_pos is given): kept routes ordered by (card, instance,
 * t, k), where card = instance / place_per_rank;
 *   send_pos[t*K+k] = row in that order, or -1 if pruned;
 *   send_count[card] = kept routes per card ([world_size] entries).
 *
 * Inputs:
 *   expert_ids        [BS*K] int32 in [0, E).
 *   eplb_table        [E*F]  int32; column 0 the count, columns 1..count
 *                     instance ids in [0, world_size*place_per_rank).
 *   expert_scales     [BS*K] of scale_dtype (MEP_SCALE_*), sorted
 *                     descending per token; may be NULL.
 *   pruning_threshold [K] fp32 ((K,) and (1,K) alike); NULL iff scales NULL.
 *   active_mask       [BS] uint8, ones before zeros; may be NULL (= all
 *                     active); needs scales and threshold.
 * Outputs: balanced_ids [BS*K] int32, balanced_mask [BS*K] uint8,
 *   send_pos [BS*K] int32 and send_count [world_size] int32 (both NULL or
 *   both given).
 * Limits ([UpdExp] "约束说明"): 1 <= BS <= 512, 1 <= K <= 16, K <= E,
 *   1 <= E <= 1024, 2 <= F <= world_size+1, 1 <= world_size <= 1024,
 *   world_size*place_per_rank <= 1024, balance_mode in {0,1};
 *   mode 0 needs 0 <= local_rank_id < world_size.
 * Errors: MEP_ERR_NULLPTR, MEP_ERR_PARAM (mode, unpaired optionals, rank,
 *   dtype), MEP_ERR_SHAPE (limits), MEP_ERR_HIP.
 */
int mep_remap_prune(int BS, int K, int E, int F, int world_size,
                    int place_per_rank, int local_rank_id, int balance_mode,
                    const int32_t* expert_ids, const int32_t* eplb_table,
                    const void* expert_scales, int scale_dtype,
                    const float* pruning_threshold, const uint8_t* active_mask,
                    int32_t* balanced_ids, uint8_t* balanced_mask,
                    int32_t* send_pos, int32_t* send_count,
                    void* stream);

/* ---------------------------------------------------------------- dispatch */

/*
 * mep_dispatch - pack this rank's token rows into per-destination send
 * segments, and/or group received rows by expert instance ([MoonEP-API]
 * 3.1; [MoonEP-TD]: rows land grouped by expert at the destination).
 *
 * Pack (runs when x != NULL):
 *   send_buf[send_pos[t*K+k], :] = x[t, :] for every 0 <= send_pos < n_send.
 *   x [T,H] bf16; send_pos [T*K] int32 (a row index, or negative to skip
 *   the route); send_buf [n_send, H] bf16, n_send its row count (T*K for
 *   the plan's map, the dedup send count for mep_plan_dedup's dpack_pos);
 *   an entry >= n_send is skipped, rows not named are left untouched.
 * Group (runs when recv_raw != NULL):
 *   recv_grouped[t, :] = recv_raw[recv_pos[t], :] for t in [0, n_recv).
 *   recv_raw [n_raw,H] bf16 in arrival (source-major) order, n_raw its row
 *   count; recv_pos [n_recv] int32; recv_grouped [n_recv,H] bf16. With the
 *   plan's own recv_pos, n_raw = n_recv; with mep_plan_dedup's drecv_pos the
 *   arrival buffer is shorter (n_raw = the dedup arrival count) and rows
 *   fan out. An entry outside [0, n_raw) leaves row t untouched.
 * The two buffer sizes bound every access, so a map paired with a buffer
 * too short for it (say a plan map with a dedup-sized buffer) writes and
 * reads nothing out of bounds; the rows it names past the end are skipped.
 * At least one of the two must run, unless T == 0 and n_recv == 0 (then
 * the call does nothing and may pass NULL buffers). Sizes: T >= 0,
 * n_send >= 0, n_recv >= 0, n_raw >= 0, 1 <= K <= 64, 8 <= H <= 65536 with
 * H % 8 == 0, T*K < 2^31 and T*(H/8) < 2^31 (x below 32 GiB).
 * Errors: MEP_ERR_NULLPTR, MEP_ERR_PARAM (neither phase requested),
 *   MEP_ERR_SHAPE, MEP_ERR_HIP.
 */
int mep_dispatch(int T, int K, int H,
                 const uint16_t* x, const int32_t* send_pos, uint16_t* send_buf, int n_send,
                 int n_recv, const int32_t* recv_pos, const uint16_t* recv_raw, int n_raw,
                 uint16_t* recv_grouped,
                 void* stream);

/* ----------------------------------------------------------------- combine */

/*
 * mep_combine - score-weighted K-way reduction of the returned expert
 * outputs in fixed k order ([MoonEP-API] 3.1 combine; the op doc's combine
 * takes the same per-route expert scales).
 *   acc = +0.0f
 *   for k = 0..K-1 with send_pos[t*K+k] >= 0:
 *       acc = fl(acc + fl(scores[t*K+k] * float(y_ret[send_pos[t*K+k], h])))
 *   out_f32[t,h] = acc; out_bf16[t,h] = acc rounded to nearest even.
 * Scores are used as given (no renormalisation).
 *   y_ret [n_y,H] bf16 in this rank's send order; send_pos [T*K] int32
 *   (a row < n_y; a negative or out-of-range entry skips the route);
 *   scores [T*K] fp32; out_bf16 [T,H] bf16
 *   and out_f32 [T,H] fp32, either may be NULL but not both.
 * Sizes: T >= 0, 1 <= K <= 64, 8 <= H <= 65536, H % 8 == 0, T*K < 2^31,
 * T*(H/8) < 2^31. With T == 0
 * the call does nothing (buffers may be NULL).
 * Errors: MEP_ERR_NULLPTR, MEP_ERR_SHAPE, MEP_ERR_HIP.
 */
int mep_combine(int T, int K, int H, const uint16_t* y_ret, int n_y,
                const int32_t* send_pos, const float* scores,
                uint16_t* out_bf16, float* out_f32,
                void* stream);

/* ------------------------------------------------ zero-copy and return */

/*
 * mep_dispatch_to_peers - zero-copy dispatch ([MoonEP-TD] architecture
 * section: tokens are written directly to their final position on the
 * receiving rank, grouped by expert, and used in place). Each of this rank's
 * routes writes its token row straight into the destination's grouped
 * receive buffer, with no send buffer and no receive-side grouping:
 *   peer_bufs[route_dest[t*K+k]][route_slot[t*K+k], :] = x[t, :]
 *   x          [T,H] bf16, this rank's tokens;
 *   route_dest, route_slot [T*K] int32: this rank's slice of mep_plan's
 *              route maps (routes (my_rank, t, k)); entries outside
 *              [0,R) x [0,C) are skipped;
 *   peer_bufs  DEVICE array of R device pointers, peer_bufs[d] the grouped
 *              receive buffer [C,H] bf16 of rank d, 16-byte aligned (memory
 *              of other GPUs mapped into this process on a multi-GPU system;
 *              slices of one allocation on one GPU).
 * Run by every rank, this fills each rank's grouped buffer with exactly what
 * pack -> exchange -> group produces. Sizes as mep_dispatch's pack,
 * 1 <= R <= 1024 (mep_plan's rank limit; the pointer table is staged in
 * on-chip memory), C >= 1; T == 0 does nothing.
 * Errors: MEP_ERR_NULLPTR, MEP_ERR_SHAPE, MEP_ERR_HIP.
 */
int mep_dispatch_to_peers(int T, int K, int H, int R, int C, const uint16_t* x,
                          const int32_t* route_dest, const int32_t* route_slot,
                          uint16_t* const* peer_bufs, void* stream);

/*
 * mep_combine_from_peers - zero-copy combine: the K expert outputs of each
 * token are read where the experts wrote them, in the destinations' grouped
 * output buffers, and reduced exactly as mep_combine does (fp32, fixed k
 * order, from +0; bf16 round-to-nearest-even):
 *   out[t,h] = sum over k of scores[t*K+k] * peer_bufs[dest][slot, h]
 * with (dest, slot) = (route_dest, route_slot)[t*K+k] of this rank's routes;
 * out-of-range entries are skipped. peer_bufs: DEVICE array of R device
 * pointers to [C,H] bf16 grouped expert outputs, 1 <= R <= 1024, C >= 1.
 * Outputs and errors as mep_combine. With the same values it gives the same
 * bits as mep_combine on the returned rows.
 */
int mep_combine_from_peers(int T, int K, int H, int R, int C,
                           const uint16_t* const* peer_bufs,
                           const int32_t* route_dest, const int32_t* route_slot,
                           const float* scores, uint16_t* out_bf16,
                           float* out_f32, void* stream);

/*
 * mep_ungroup - the return step of the non-zero-copy path: expert outputs
 * in grouped order go back to arrival (source-major) order, the inverse of
 * mep_dispatch's grouping:
 *   y_arrival[recv_pos[t], :] = y_grouped[t, :] for t in [0, n)
 * (recv_pos from mep_plan; entries outside [0, n) are skipped). The source
 * segments of y_arrival are then what each source rank receives back, in
 * its send order. n >= 0 (0 does nothing), H as mep_dispatch.
 * Errors: MEP_ERR_NULLPTR, MEP_ERR_SHAPE, MEP_ERR_HIP.
 */
int mep_ungroup(int n, int H, const int32_t* recv_pos, const uint16_t* y_grouped,
                uint16_t* y_arrival, void* stream);

/*
 * mep_combine_add_rmsnorm - the combine fused with the residual add and RMS
 * normalisation that follow it ([UpdExp] call example: the combine variant
 * taking the residual x and gamma and returning y, rstd and the summed x;
 * the pages give no formula, the usual add + RMSNorm is computed):
 *   a[t,h]  = the fp32 accumulator of mep_combine (same k order and skips)
 *   x[t,h]  = fl(a[t,h] + float(residual[t,h]))
 *   rstd[t] = 1 / sqrt(sum over h of x[t,h]^2 / H + eps), fp32
 *   y[t,h]  = fl(fl(x[t,h] * rstd[t]) * float(gamma[h])), bf16 nearest even
 *   x_out[t,h] = x[t,h] rounded to bf16 nearest even
 *   y_ret [n_y,H], send_pos [T*K], scores [T*K] as mep_combine;
 *   residual [T,H] bf16; gamma [H] bf16; eps >= 0;
 *   outputs: y_out [T,H] bf16 (required), x_out [T,H] bf16 and
 *   rstd_out [T] fp32 (either may be NULL). Row pointers 16-byte aligned.
 * x_out is bit-identical to mep_combine's out_bf16 of a + residual; the sum
 * of squares is reduced in fp32 in a tree order, so rstd and y carry fp32
 * rounding of that sum (relative error well under 1e-5 for H <= 16384).
 * Sizes: T >= 0 (0 does nothing), 1 <= K <= 64, 8 <= H <= 16384,
 * H % 8 == 0, n_y >= 0 (y_ret may be NULL only if n_y == 0).
 * Errors: MEP_ERR_NULLPTR, MEP_ERR_PARAM (eps negative or not finite),
 * MEP_ERR_SHAPE, MEP_ERR_HIP.
 */
int mep_combine_add_rmsnorm(int T, int K, int H, const uint16_t* y_ret, int n_y,
                            const int32_t* send_pos, const float* scores,
                            const uint16_t* residual, const uint16_t* gamma, float eps,
                            uint16_t* x_out, uint16_t* y_out, float* rstd_out,
                            void* stream);

/*
 * mep_plan_weight_rows - the weight row each planned instance's expert GEMM
 * reads under a cap of B prefetch slots per rank ("MoonEP" technical
 * overview, memory contract: weights are one [E+B, H, H'] tensor, rows
 * 0..E-1 the experts of all ranks, rows E..E+B-1 a rank's prefetch slots;
 * B = E/R for training, 3-4 for inference, redundant experts beyond the
 * slots served from their home rank). For rank u and local index i of
 * mep_plan's instance tables:
 *   inst_wrow[u*E+i] = e        for a native instance (home(e) == u)
 *                    = E + j    for the j-th redundant instance, j < B
 *                    = e        for the j-th redundant instance, j >= B
 *                    = -1       for i >= inst_count[u]
 *   inst_count [R], inst_expert [R*E] from mep_plan (the plan's local
 *   layout, natives first, is assumed); inst_wrow [R*E] int32 out.
 * Sizes: 1 <= R, E <= 1024, B >= 0.
 * Errors: MEP_ERR_NULLPTR, MEP_ERR_PARAM (B < 0), MEP_ERR_SHAPE, MEP_ERR_HIP.
 */
int mep_plan_weight_rows(int R, int E, int B, const int32_t* inst_count,
                         const int32_t* inst_expert, int32_t* inst_wrow, void* stream);

/*
 * mep_plan_dedup_workspace_size - device workspace bytes mep_plan_dedup
 * needs for (R, S, K); 0 if unsupported. Host only.
 */
size_t mep_plan_dedup_workspace_size(int R, int S, int K);

/*
 * mep_plan_dedup - per-destination token dedup of rank my_rank's dispatch
 * ("MoonEP API完全参考", §5.2 communication performance, which names a dedup
 * encoding of sent tokens; the reading: a token with several routes to one
 * rank is sent there once and fanned out to its grouped slots on arrival).
 * From mep_plan's global route maps, with D(g) the destinations of global
 * token g = src*S + t:
 *   dpack_pos [S*K]: for the first route (t,k) of t to a destination d, the
 *     row of (t, d) in the send buffer, ordered by (d, t); -1 for t's later
 *     routes to d. mep_dispatch's pack with dpack_pos writes each (t, d) row
 *     once.
 *   dsend_count [R]: rows for each destination.
 *   drecv_pos [S*K]: for each grouped slot on my_rank, the arrival row of
 *     the token whose route occupies it; the arrival buffer holds the rows
 *     reaching my_rank, sources ascending, each in token order.
 *     mep_dispatch's grouping with drecv_pos fills recv_grouped exactly as
 *     the plan's own recv_pos does on the full arrival buffer.
 *   drecv_count [R]: rows arriving from each source.
 *   route_dest, route_slot [R*S*K]: mep_plan outputs (a valid plan: every
 *     slot of my_rank is occupied by exactly one route).
 *   workspace: mep_plan_dedup_workspace_size bytes, 256-byte aligned.
 * Sizes: 1 <= R <= 64, S, K >= 1, R*S*K <= 2^30.
 * Errors: MEP_ERR_NULLPTR, MEP_ERR_PARAM (my_rank outside [0,R), workspace
 * too small), MEP_ERR_SHAPE, MEP_ERR_HIP.
 */
int mep_plan_dedup(int R, int S, int K, int my_rank, const int32_t* route_dest,
                   const int32_t* route_slot, void* workspace, size_t workspace_bytes,
                   int32_t* dpack_pos, int32_t* dsend_count, int32_t* drecv_pos,
                   int32_t* drecv_count, void* stream);

/* -------------------------------------------------------- int8 dispatch */

/*
 * mep_quant_msg_bytes - size of one int8 token message: Align512(Align32(H)
 * + 4) bytes ("aclnnMoeDistributeDispatchSetup" op doc, parameter notes:
 * message size in the quantized case). Host only; 0 for H < 1.
 */
size_t mep_quant_msg_bytes(int H);

/*
 * mep_dispatch_quant - the pack with dynamic int8 quantization of every
 * routed row ("aclnnMoeDistributeDispatchSetup" op doc, interface
 * description: token data may be quantized before sending; parameter notes:
 * optional smoothing scales for dynamic quantization; the message layout).
 * The pages give no formula; this computes, per route (t,k) with
 * 0 <= send_pos[t*K+k] < n_rows:
 *   v[h] = float(x[t,h]), or fl(float(x[t,h]) * smooth[e*H + h]) with
 *          e = route_expert[t*K+k] when smooth is given
 *   s    = fl(max_h |v[h]| / 127)          (fp32, correctly rounded)
 *   q[h] = rint(fl(v[h] / s)), ties to even, clamped to [-127, 127];
 *          q = 0 when s == 0
 * and writes message row p = send_pos[t*K+k] of send_msgs: int8 q[0..H) in
 * bytes [0, H), s (fp32) at byte Align32(H). Other bytes of the row are not
 * written. With smoothing, a route whose expert id is outside [0, E) is
 * skipped.
 *   x [T,H] bf16; smooth [E,H] fp32 or NULL; route_expert [T*K] int32
 *   (required with smooth); send_pos [T*K] int32 (this rank's send map);
 *   send_msgs [n_rows, msg_bytes] bytes, msg_bytes >= Align32(H) + 4 and a
 *   multiple of 16 (mep_quant_msg_bytes(H) is the pages' size).
 * The received messages are grouped with mep_dispatch's grouping as rows of
 * msg_bytes / 2 bf16-sized units (the grouping copies bytes).
 * Sizes: T >= 0, 1 <= K <= 64, 8 <= H <= 16384, H % 8 == 0, T*K < 2^31;
 * T == 0 or n_rows == 0 does nothing. x, send_msgs and smooth 16-byte
 * aligned; values of x (and smooth) finite.
 * Errors: MEP_ERR_NULLPTR, MEP_ERR_PARAM (smooth without route_expert or
 * E < 1), MEP_ERR_SHAPE, MEP_ERR_HIP.
 */
int mep_dispatch_quant(int T, int K, int H, const uint16_t* x, const float* smooth, int E,
                       const int32_t* route_expert, const int32_t* send_pos, int n_rows,
                       int msg_bytes, uint8_t* send_msgs, void* stream);

/*
 * mep_group_quant - receive side of the int8 dispatch: the arrival buffer
 * of messages becomes the expert-side layout, int8 rows grouped by expert
 * instance plus one fp32 scale per row ("aclnnMoeDistributeDispatchSetup"
 * call example: received tokens come back as an int8 matrix and a vector of
 * dynamic scales):
 *   x_q[t, 0:H] = bytes [0, H) of recv_msgs[recv_pos[t]]
 *   scales[t]   = fp32 at byte Align32(H) of recv_msgs[recv_pos[t]]
 * for t in [0, n); an entry of recv_pos outside [0, n_msgs) leaves row t
 * untouched.
 *   recv_msgs [n_msgs, msg_bytes] (16-byte aligned, msg_bytes as in
 *   mep_dispatch_quant); recv_pos [n] int32 (mep_plan's recv_pos);
 *   x_q [n, H] int8 (8-byte aligned); scales [n] fp32.
 * Sizes: n >= 0 (0 does nothing), 8 <= H <= 65536, H % 8 == 0,
 * n*(H/8) < 2^31. Errors: MEP_ERR_NULLPTR, MEP_ERR_SHAPE, MEP_ERR_HIP.
 */
int mep_group_quant(int n, int H, int msg_bytes, const int32_t* recv_pos, int n_msgs,
                    const uint8_t* recv_msgs, uint8_t* x_q, float* scales, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MEP_H */
