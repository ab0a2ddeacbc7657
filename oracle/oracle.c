/*
 * CPU oracle for the balanced expert-parallel MoE hot path.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, single-threaded
 * definition that the GPU library is checked against. Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it. It shares
 * no code, header, table or helper with the GPU library.
 *
 * Sources (web pages on the method; cited by title and section):
 *  [MoonEP-TD]  "MoonEP" technical overview (twodots.gr): the invariant that
 *               every EP rank processes exactly S*K routed rows; redundant
 *               expert instances planned online from the router output;
 *               tokens written grouped by expert at the destination;
 *               planner-produced cu_seqlens; expert rows 0..E-1, then
 *               prefetch slots; static S*K buffers.
 *  [UpdExp]     "aclnnMoeUpdateExpert" op doc, sections "功能说明"
 *               (function description: load-balance remap and pruning
 *               formulas), "参数说明" (parameter table) and "约束说明"
 *               (constraints).
 *  [MoonEP-API] "MoonEP API完全参考" (stapisi.com), sections 2.2 and 3.1:
 *               planning, dispatch and combine entry points.
 * The exact planning rule (native home rank floor(e*R/E), keep the first S*K
 * routes of a rank in (expert, global token, k) order, spill the rest in that
 * order to under-loaded ranks in ascending rank order) is the plainest rule
 * that meets the [MoonEP-TD] invariant; the readings are listed with the
 * design notes of this repository.
 *
 * [DispSetup] "aclnnMoeDistributeDispatchSetup" op doc: quantized token
 *             messages and their size; the call example's outputs.
 *
 * Pins. Every function is checked by the test suite against something other
 * than itself (the op doc's worked example, closed forms, invariants, brute
 * force, textbook special cases, equivalence with already pinned functions),
 * and each pin fails for a planted mistake in the function it covers; no
 * function here is without a pin. Where the pages leave a point open, the
 * function follows a stated reading (listed with the design notes of this
 * repository) and its pins fix that reading: the remap columns for instance
 * counts above one (the printed formula is garbled; structural pins for
 * every count up to 12: mode 0's columns split the ranks into groups of
 * ceil(ws/count), mode 1's cycle over tokens); the precision and order of
 * the prune threshold sum (fp32 in k order with each product rounded,
 * pinned by tokens whose mask flips under fp64, a reversed order or a fused
 * multiply-add); the combine + add + RMSNorm formula
 * (oracle_combine_add_rmsnorm: the textbook RMSNorm, pinned by a hand
 * example and closed forms); the int8 quantization formula
 * (oracle_dispatch_quant: symmetric per-row scaling to +-127, pinned by its
 * defining properties); the prefetch-slot order (oracle_weight_rows) and
 * the dedup orders (oracle_plan_dedup), pinned by layout properties and by
 * equivalence with the plain dispatch chain.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no FMA contraction, so
 * every fp32 multiply and add is rounded on its own).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_OK = 0, OR_ERR_ARG = 1, OR_ERR_ALLOC = 2, OR_ERR_INTERNAL = 3 };

/* ---------------------------------------------------------------- helpers */

/* Native home rank of expert e: floor(e*R/E), in 64-bit integers. */
static int home_rank(int e, int R, int E) {
    return (int)(((int64_t)e * (int64_t)R) / (int64_t)E);
}

/* bf16 bit pattern -> float (exact widening: bf16 is the top half of fp32). */
static float bf16_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* float -> bf16, round to nearest, ties to even, from the bit layout.
 * NaN maps to a quiet NaN with the same sign. */
static uint16_t float_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* IEEE binary16 bit pattern -> float, decoded field by field (exact). */
static float fp16_to_float(uint16_t h) {
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    uint32_t ex = (h >> 10) & 0x1fu;
    uint32_t man = h & 0x3ffu;
    uint32_t u;
    if (ex == 0) {
        if (man == 0) {
            u = sign;
        } else { /* subnormal: value = man * 2^-24 */
            int shift = 0;
            while ((man & 0x400u) == 0) { man <<= 1; shift++; }
            man &= 0x3ffu;
            u = sign | ((uint32_t)(127 - 15 - shift + 1) << 23) | (man << 13);
        }
    } else if (ex == 31) {
        u = sign | 0x7f800000u | (man << 13);
    } else {
        u = sign | ((ex - 15 + 127) << 23) | (man << 13);
    }
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* qsort keys: (primary, secondary) pairs compared lexicographically. */
typedef struct { int64_t a; int64_t b; int32_t idx; } key2;

static int cmp_key2(const void* x, const void* y) {
    const key2* p = (const key2*)x;
    const key2* q = (const key2*)y;
    if (p->a != q->a) return p->a < q->a ? -1 : 1;
    if (p->b != q->b) return p->b < q->b ? -1 : 1;
    return 0;
}

/* ------------------------------------------------------------------- plan */

/*
 * oracle_plan: global plan over the R x S x K routing table, plus the send
 * and receive maps of rank m.
 *
 * [MoonEP-TD] invariant: every rank ends with exactly C = S*K routed rows.
 * Steps:
 *  1. cnt[e] and native loads L[r] = sum of cnt[e] over home(e) = r.
 *  2. Order all routes f = g*K + k (g = src*S + s) by (expert, f): a stable
 *     sort by expert, which is the (expert, global token, k) order.
 *  3. Each rank's routes form one block of that order (home is monotone in
 *     e). The first C of a block stay on the home rank at slots 0..C-1; the
 *     rest are that rank's excess.
 *  4. The excess of all over-loaded ranks, concatenated in ascending rank
 *     (= the same global order), is handed out in order to the under-loaded
 *     ranks in ascending rank; rank u takes C - L[u] routes at slots
 *     L[u], L[u]+1, ...
 *  5. Local instance layout of rank u ([MoonEP-TD]: rows grouped by expert,
 *     expert rows first, prefetch slots after): native experts of u in
 *     ascending e (zero-row natives keep their place), then redundant
 *     instances (experts with home != u that received rows on u) in
 *     ascending e. inst_cu holds the row offsets (the cu_seqlens).
 *  6. send_pos: rank m's routes ordered by (dest, dest slot).
 *     recv_pos: rank m's slots ordered by (source rank, slot); recv_pos[t]
 *     is the row of the source-major arrival buffer that feeds slot t.
 *
 * Outputs beyond inst_count[u]: inst_expert = -1, inst_cu = C.
 * Returns OR_ERR_INTERNAL if the slot assignment does not match the layout
 * of step 5 (a self-check; never expected).
 */
int oracle_plan(int R, int E, int S, int K, int m, const int32_t* ids,
                int32_t* expert_count, int32_t* rank_load,
                int32_t* route_dest, int32_t* route_slot,
                int32_t* inst_count, int32_t* inst_expert, int32_t* inst_cu,
                int32_t* inst_gid_base,
                int32_t* send_pos, int32_t* send_count,
                int32_t* recv_pos, int32_t* recv_count) {
    if (R < 1 || E < 1 || S < 1 || K < 1 || K > E || m < 0 || m >= R)
        return OR_ERR_ARG;
    const int64_t C = (int64_t)S * K;
    const int64_t N = (int64_t)R * C;
    int rc = OR_OK;

    /* step 1 */
    int64_t* cnt = calloc((size_t)E, sizeof(int64_t));
    int64_t* L = calloc((size_t)R, sizeof(int64_t));
    key2* order = malloc((size_t)N * sizeof(key2));
    int32_t* slot_route = malloc((size_t)N * sizeof(int32_t));
    int64_t* rcount = calloc((size_t)R * E, sizeof(int64_t));
    key2* tmp = malloc((size_t)C * sizeof(key2));
    if (!cnt || !L || !order || !slot_route || !rcount || !tmp) {
        rc = OR_ERR_ALLOC;
        goto done;
    }
    for (int64_t f = 0; f < N; f++) {
        int e = ids[f];
        if (e < 0 || e >= E) { rc = OR_ERR_ARG; goto done; }
        cnt[e]++;
    }
    for (int e = 0; e < E; e++) L[home_rank(e, R, E)] += cnt[e];
    for (int e = 0; e < E; e++) expert_count[e] = (int32_t)cnt[e];
    for (int r = 0; r < R; r++) rank_load[r] = (int32_t)L[r];

    /* step 2 */
    for (int64_t f = 0; f < N; f++) {
        order[f].a = ids[f];
        order[f].b = f;
        order[f].idx = (int32_t)f;
    }
    qsort(order, (size_t)N, sizeof(key2), cmp_key2);

    /* step 3: walk each rank's block, keep the first C, list the rest */
    int32_t* excess = malloc((size_t)N * sizeof(int32_t));
    if (!excess) { rc = OR_ERR_ALLOC; goto done; }
    int64_t n_excess = 0;
    {
        int64_t p = 0;
        for (int r = 0; r < R; r++) {
            for (int64_t q = 0; q < L[r]; q++, p++) {
                int32_t f = order[p].idx;
                if (home_rank(ids[f], R, E) != r) { rc = OR_ERR_INTERNAL; free(excess); goto done; }
                if (q < C) {
                    route_dest[f] = r;
                    route_slot[f] = (int32_t)q;
                } else {
                    excess[n_excess++] = f;
                }
            }
        }
    }
    /* step 4: hand the excess out to under-loaded ranks in ascending order */
    {
        int64_t j = 0;
        for (int u = 0; u < R; u++) {
            for (int64_t slot = L[u]; slot < C; slot++) {
                if (j >= n_excess) { rc = OR_ERR_INTERNAL; free(excess); goto done; }
                int32_t f = excess[j++];
                route_dest[f] = u;
                route_slot[f] = (int32_t)slot;
            }
        }
        if (j != n_excess) { rc = OR_ERR_INTERNAL; free(excess); goto done; }
    }
    free(excess);

    /* inverse map: which route sits in (dest, slot) */
    for (int64_t i = 0; i < N; i++) slot_route[i] = -1;
    for (int64_t f = 0; f < N; f++) {
        int64_t at = (int64_t)route_dest[f] * C + route_slot[f];
        if (slot_route[at] != -1) { rc = OR_ERR_INTERNAL; goto done; }
        slot_route[at] = (int32_t)f;
    }

    /* step 5: instance tables */
    for (int64_t f = 0; f < N; f++) rcount[(int64_t)route_dest[f] * E + ids[f]]++;
    {
        int64_t gid = 0;
        for (int u = 0; u < R; u++) {
            int32_t* ie = inst_expert + (int64_t)u * E;
            int32_t* cu = inst_cu + (int64_t)u * (E + 1);
            int n = 0;
            int64_t row = 0;
            for (int e = 0; e < E; e++) {           /* natives */
                if (home_rank(e, R, E) != u) continue;
                ie[n] = e;
                cu[n] = (int32_t)row;
                row += rcount[(int64_t)u * E + e];
                n++;
            }
            for (int e = 0; e < E; e++) {           /* redundant instances */
                if (home_rank(e, R, E) == u || rcount[(int64_t)u * E + e] == 0) continue;
                ie[n] = e;
                cu[n] = (int32_t)row;
                row += rcount[(int64_t)u * E + e];
                n++;
            }
            if (row != C || n > E) { rc = OR_ERR_INTERNAL; goto done; }
            cu[n] = (int32_t)C;
            for (int i = n; i < E; i++) ie[i] = -1;
            for (int i = n + 1; i <= E; i++) cu[i] = (int32_t)C;
            inst_count[u] = n;
            inst_gid_base[u] = (int32_t)gid;
            gid += n;
            /* self-check: the slots of instance i hold exactly its expert */
            for (int i = 0; i < n; i++)
                for (int64_t t = cu[i]; t < cu[i + 1]; t++)
                    if (ids[slot_route[(int64_t)u * C + t]] != ie[i]) {
                        rc = OR_ERR_INTERNAL;
                        goto done;
                    }
        }
        inst_gid_base[R] = (int32_t)gid;
    }

    /* step 6a: send map of rank m, ordered by (dest, dest slot) */
    for (int r = 0; r < R; r++) send_count[r] = 0;
    for (int64_t i = 0; i < C; i++) {
        int64_t f = (int64_t)m * C + i;
        tmp[i].a = route_dest[f];
        tmp[i].b = route_slot[f];
        tmp[i].idx = (int32_t)i;
        send_count[route_dest[f]]++;
    }
    qsort(tmp, (size_t)C, sizeof(key2), cmp_key2);
    for (int64_t i = 0; i < C; i++) send_pos[tmp[i].idx] = (int32_t)i;

    /* step 6b: arrival order on rank m, ordered by (source rank, slot) */
    for (int r = 0; r < R; r++) recv_count[r] = 0;
    for (int64_t t = 0; t < C; t++) {
        int64_t f = slot_route[(int64_t)m * C + t];
        int64_t src = f / C;
        tmp[t].a = src;
        tmp[t].b = t;
        tmp[t].idx = (int32_t)t;
        recv_count[src]++;
    }
    qsort(tmp, (size_t)C, sizeof(key2), cmp_key2);
    for (int64_t i = 0; i < C; i++) recv_pos[tmp[i].idx] = (int32_t)i;

done:
    free(cnt);
    free(L);
    free(order);
    free(slot_route);
    free(rcount);
    free(tmp);
    return rc;
}

/* --------------------------------------------------------- remap / prune */

/*
 * oracle_remap_prune: [UpdExp] "功能说明" load-balance remap and pruning.
 *
 * Remap, per (t, k) with e = expert_ids[t,k] and count = table[e*F]:
 *   count == 1        -> column 1
 *   balance_mode == 0 -> column local_rank_id / ceil(world_size / count) + 1
 *   balance_mode == 1 -> column (t mod count) + 1  (t = token index)
 *   balanced_ids[t,k] = table[e*F + column]
 * Pruning, with scales widened exactly to fp32:
 *   thr_sum[t] = sum over k = 0..K-1 of fl(scale[t,k] * threshold[k]),
 *               added in k order from +0.0f, each step rounded to fp32
 *   mask[t,k]  = active[t] and not (scale[t,k] < thr_sum[t])
 *   (a route whose scale falls below the sum is pruned; a tie is kept)
 *   Without scales and threshold every mask entry is 1.
 * Send map (dispatch after remap): kept routes ordered by (destination card,
 * instance id, t, k), the card of an instance being id / place_per_rank;
 * send_pos[t*K+k] = row, -1 when pruned; send_count[card] = kept routes.
 *
 * scale_dtype: 0 = fp32, 1 = bf16, 2 = fp16. scales/thr/active may be NULL
 * (scales and thr together; active only with them). send_pos and
 * send_count may be NULL (together).
 */
int oracle_remap_prune(int BS, int K, int E, int F, int world_size,
                       int place_per_rank, int local_rank_id, int balance_mode,
                       const int32_t* expert_ids, const int32_t* eplb_table,
                       const void* scales, int scale_dtype, const float* thr,
                       const uint8_t* active,
                       int32_t* balanced_ids, uint8_t* balanced_mask,
                       int32_t* send_pos, int32_t* send_count) {
    if (BS < 1 || K < 1 || E < 1 || F < 2 || world_size < 1 || place_per_rank < 1)
        return OR_ERR_ARG;
    if (balance_mode != 0 && balance_mode != 1) return OR_ERR_ARG;
    if ((scales == NULL) != (thr == NULL)) return OR_ERR_ARG;
    if (active != NULL && scales == NULL) return OR_ERR_ARG;
    const int n_inst = world_size * place_per_rank;

    for (int t = 0; t < BS; t++) {
        for (int k = 0; k < K; k++) {
            int e = expert_ids[t * K + k];
            if (e < 0 || e >= E) return OR_ERR_ARG;
            int count = eplb_table[(int64_t)e * F];
            int col;
            if (count == 1) {
                col = 1;
            } else if (balance_mode == 0) {
                int mode_value = (world_size + count - 1) / count;
                col = local_rank_id / mode_value + 1;
            } else {
                col = t % count + 1;
            }
            if (col < 1 || col >= F) return OR_ERR_ARG;
            balanced_ids[t * K + k] = eplb_table[(int64_t)e * F + col];
        }
    }

    for (int t = 0; t < BS; t++) {
        if (scales == NULL) {
            for (int k = 0; k < K; k++) balanced_mask[t * K + k] = 1;
            continue;
        }
        float s[64];
        if (K > 64) return OR_ERR_ARG;
        for (int k = 0; k < K; k++) {
            int64_t i = (int64_t)t * K + k;
            if (scale_dtype == 0) s[k] = ((const float*)scales)[i];
            else if (scale_dtype == 1) s[k] = bf16_to_float(((const uint16_t*)scales)[i]);
            else if (scale_dtype == 2) s[k] = fp16_to_float(((const uint16_t*)scales)[i]);
            else return OR_ERR_ARG;
        }
        float thr_sum = 0.0f;
        for (int k = 0; k < K; k++) {
            float prod = s[k] * thr[k];
            thr_sum = thr_sum + prod;
        }
        int act = active == NULL ? 1 : (active[t] != 0);
        for (int k = 0; k < K; k++)
            balanced_mask[t * K + k] = (uint8_t)(act && !(s[k] < thr_sum));
    }

    if (send_pos != NULL || send_count != NULL) {
        if (send_pos == NULL || send_count == NULL) return OR_ERR_ARG;
        key2* tmp = malloc((size_t)BS * K * sizeof(key2));
        if (!tmp) return OR_ERR_ALLOC;
        int64_t n = 0;
        for (int c = 0; c < world_size; c++) send_count[c] = 0;
        for (int64_t i = 0; i < (int64_t)BS * K; i++) {
            send_pos[i] = -1;
            if (!balanced_mask[i]) continue;
            int inst = balanced_ids[i];
            if (inst < 0 || inst >= n_inst) { free(tmp); return OR_ERR_ARG; }
            int card = inst / place_per_rank;
            tmp[n].a = (int64_t)card * n_inst + inst;
            tmp[n].b = i;
            tmp[n].idx = (int32_t)i;
            n++;
            send_count[card]++;
        }
        qsort(tmp, (size_t)n, sizeof(key2), cmp_key2);
        for (int64_t r = 0; r < n; r++) send_pos[tmp[r].idx] = (int32_t)r;
        free(tmp);
    }
    return OR_OK;
}

/* --------------------------------------------------------------- dispatch */

/*
 * oracle_pack: send_buf[send_pos[t*K+k], :] = x[t, :] for every route whose
 * send_pos is >= 0 (per-destination send segments; [MoonEP-API] 3.1).
 */
int oracle_pack(int T, int K, int H, const uint16_t* x, const int32_t* send_pos,
                uint16_t* send_buf) {
    if (T < 0 || K < 1 || H < 1) return OR_ERR_ARG;
    for (int64_t t = 0; t < T; t++)
        for (int k = 0; k < K; k++) {
            int32_t row = send_pos[t * K + k];
            if (row < 0) continue;
            for (int64_t h = 0; h < H; h++)
                send_buf[(int64_t)row * H + h] = x[t * H + h];
        }
    return OR_OK;
}

/*
 * oracle_group: recv_grouped[t, :] = recv_raw[recv_pos[t], :], turning the
 * source-major arrival buffer into rows grouped by expert instance
 * ([MoonEP-TD]: tokens land grouped by expert at the destination).
 */
int oracle_group(int n_recv, int H, const int32_t* recv_pos,
                 const uint16_t* recv_raw, uint16_t* recv_grouped) {
    if (n_recv < 0 || H < 1) return OR_ERR_ARG;
    for (int64_t t = 0; t < n_recv; t++) {
        int64_t src = recv_pos[t];
        for (int64_t h = 0; h < H; h++)
            recv_grouped[t * H + h] = recv_raw[src * H + h];
    }
    return OR_OK;
}

/* ---------------------------------------------------------------- combine */

/*
 * oracle_combine: score-weighted K-way reduction in fixed k order.
 *   acc = +0.0f
 *   for k = 0..K-1 with send_pos[t*K+k] >= 0:
 *       acc = fl(acc + fl(score[t,k] * float(y_ret[send_pos[t*K+k], h])))
 *   out_f32[t,h] = acc, out_bf16[t,h] = round-to-nearest-even(acc)
 * Either output may be NULL.
 */
int oracle_combine(int T, int K, int H, const uint16_t* y_ret,
                   const int32_t* send_pos, const float* scores,
                   uint16_t* out_bf16, float* out_f32) {
    if (T < 0 || K < 1 || H < 1) return OR_ERR_ARG;
    for (int64_t t = 0; t < T; t++)
        for (int64_t h = 0; h < H; h++) {
            float acc = 0.0f;
            for (int k = 0; k < K; k++) {
                int32_t row = send_pos[t * K + k];
                if (row < 0) continue;
                float y = bf16_to_float(y_ret[(int64_t)row * H + h]);
                float prod = scores[t * K + k] * y;
                acc = acc + prod;
            }
            if (out_f32) out_f32[t * H + h] = acc;
            if (out_bf16) out_bf16[t * H + h] = float_to_bf16_rne(acc);
        }
    return OR_OK;
}

/*
 * oracle_combine_add_rmsnorm: the combine, then a residual add and an RMS
 * normalisation of the sum ([UpdExp] call example: the combine variant that
 * also takes the residual x and a gamma vector and returns y, rstd and the
 * summed x). The pages name those tensors but print no formula; the reading
 * taken is the usual add + RMSNorm, normalising the unrounded sum:
 *   a[t,h]  = the fp32 accumulator of oracle_combine (same k order)
 *   x[t,h]  = fl(a[t,h] + float(residual[t,h]))          fp32, one rounding
 *   x_out   = round-to-nearest-even bf16 of x
 *   rstd[t] = 1 / sqrt(sum_h x[t,h]^2 / H + eps)          in fp64
 *   y[t,h]  = x[t,h] * rstd[t] * float(gamma[h])          in fp64
 * The squares of fp32 values are exact in fp64, so rstd and y are the
 * definition up to fp64 rounding. x_f32 may be NULL.
 */
int oracle_combine_add_rmsnorm(int T, int K, int H, const uint16_t* y_ret, int n_y,
                               const int32_t* send_pos, const float* scores,
                               const uint16_t* residual, const uint16_t* gamma, double eps,
                               uint16_t* x_out, float* x_f32, double* rstd, double* y) {
    if (T < 0 || K < 1 || H < 1 || n_y < 0 || !(eps >= 0.0)) return OR_ERR_ARG;
    float* xs = (float*)malloc(sizeof(float) * (size_t)(H > 0 ? H : 1));
    if (!xs) return OR_ERR_ALLOC;
    for (int64_t t = 0; t < T; t++) {
        double ss = 0.0;
        for (int64_t h = 0; h < H; h++) {
            float acc = 0.0f;
            for (int k = 0; k < K; k++) {
                int32_t row = send_pos[t * K + k];
                if (row < 0 || row >= n_y) continue;
                float prod = scores[t * K + k] * bf16_to_float(y_ret[(int64_t)row * H + h]);
                acc = acc + prod;
            }
            float x = acc + bf16_to_float(residual[t * H + h]);
            xs[h] = x;
            ss += (double)x * (double)x;
            x_out[t * H + h] = float_to_bf16_rne(x);
            if (x_f32) x_f32[t * H + h] = x;
        }
        double r = 1.0 / sqrt(ss / (double)H + eps);
        rstd[t] = r;
        for (int64_t h = 0; h < H; h++)
            y[t * H + h] = (double)xs[h] * r * (double)bf16_to_float(gamma[h]);
    }
    free(xs);
    return OR_OK;
}

/*
 * oracle_dispatch_quant: the pack with int8 dynamic quantization of each
 * routed row ([DispSetup] interface description: token data may be
 * quantized before it is sent; parameter notes: dynamic quantization may
 * take optional per-expert smoothing scales; message size
 * Align512(Align32(H) + 4): H int8 values, padding to a multiple of 32, one
 * 4-byte scale). The pages give no formula; the reading taken is symmetric
 * per-route int8 quantization in fp32:
 *   v[h]  = float(x[t,h])                            (no smoothing), or
 *   v[h]  = fl(float(x[t,h]) * smooth[e,h])          e = route_expert[t*K+k]
 *   amax  = max over h of |v[h]|
 *   s     = fl(amax / 127)
 *   q[h]  = rint(fl(v[h] / s)) clamped to [-127, 127] (ties to even);
 *           q = 0 everywhere when s == 0
 * written to message row send_pos[t*K+k]: bytes [0, H) hold q, bytes
 * [Align32(H), Align32(H)+4) hold s (fp32, little endian). Other bytes of
 * the row are not written. Routes with send_pos outside [0, n_rows), or
 * (with smoothing) an expert id outside [0, E), are skipped.
 */
int oracle_dispatch_quant(int T, int K, int H, const uint16_t* x, const float* smooth, int E,
                          const int32_t* route_expert, const int32_t* send_pos, int n_rows,
                          int msg_bytes, uint8_t* msgs) {
    const int64_t hq = ((int64_t)H + 31) / 32 * 32;
    if (T < 0 || K < 1 || H < 1 || n_rows < 0 || msg_bytes < hq + 4) return OR_ERR_ARG;
    if (smooth && (!route_expert || E < 1)) return OR_ERR_ARG;
    float* v = (float*)malloc(sizeof(float) * (size_t)H);
    if (!v) return OR_ERR_ALLOC;
    for (int64_t t = 0; t < T; t++)
        for (int k = 0; k < K; k++) {
            const int32_t row = send_pos[t * K + k];
            if (row < 0 || row >= n_rows) continue;
            int32_t e = smooth ? route_expert[t * K + k] : 0;
            if (smooth && (e < 0 || e >= E)) continue; /* no such expert: skipped */
            float amax = 0.0f;
            for (int64_t h = 0; h < H; h++) {
                float a = bf16_to_float(x[t * H + h]);
                if (smooth) a = a * smooth[(int64_t)e * H + h];
                v[h] = a;
                const float m = fabsf(a);
                if (m > amax) amax = m;
            }
            const float sc = amax / 127.0f;
            uint8_t* out = msgs + (int64_t)row * msg_bytes;
            for (int64_t h = 0; h < H; h++) {
                float q = 0.0f;
                if (sc > 0.0f) {
                    q = rintf(v[h] / sc);
                    if (q > 127.0f) q = 127.0f;
                    if (q < -127.0f) q = -127.0f;
                }
                out[h] = (uint8_t)(int8_t)q;
            }
            memcpy(out + hq, &sc, 4);
        }
    free(v);
    return OR_OK;
}

/*
 * oracle_group_quant: receive-side grouping of int8 messages into the
 * expert-side layout ([DispSetup] call example: the dispatch returns the
 * received tokens as an int8 matrix plus one fp32 dynamic scale per token):
 *   x_q[t, 0:H] = msgs[recv_pos[t], 0:H]
 *   scales[t]   = the fp32 at byte Align32(H) of msgs[recv_pos[t]]
 * for t in [0, n); entries outside [0, n_msgs) leave row t untouched.
 */
int oracle_group_quant(int n, int H, int msg_bytes, const int32_t* recv_pos, int n_msgs,
                       const uint8_t* msgs, uint8_t* x_q, float* scales) {
    const int64_t hq = ((int64_t)H + 31) / 32 * 32;
    if (n < 0 || H < 1 || n_msgs < 0 || msg_bytes < hq + 4) return OR_ERR_ARG;
    for (int64_t t = 0; t < n; t++) {
        const int32_t from = recv_pos[t];
        if (from < 0 || from >= n_msgs) continue;
        const uint8_t* m = msgs + (int64_t)from * msg_bytes;
        memcpy(x_q + t * H, m, (size_t)H);
        memcpy(scales + t, m + hq, 4);
    }
    return OR_OK;
}

/*
 * oracle_weight_rows: the weight row each planned instance's expert GEMM
 * reads, under a cap of B prefetch slots per rank ([MoonEP-TD] memory
 * contract: the group GEMM's weights are one [E+B, H, H'] tensor, rows
 * 0..E-1 the experts of all ranks, rows E..E+B-1 local prefetch slots;
 * B = E/R for training, a smaller B (3-4) for inference, with instances
 * beyond the slots served from the home rank). Reading: walk rank u's
 * instances in local order; an instance whose expert is native to u
 * (home(e) == u) reads row e; the j-th non-native (redundant) instance reads
 * prefetch row E + j while j < B, else row e (the home rank's copy).
 * Entries past inst_count[u] are -1.
 */
int oracle_weight_rows(int R, int E, int B, const int32_t* inst_count,
                       const int32_t* inst_expert, int32_t* wrow) {
    if (R < 1 || E < 1 || B < 0) return OR_ERR_ARG;
    for (int u = 0; u < R; u++) {
        int j = 0;
        for (int i = 0; i < E; i++) {
            int32_t* out = wrow + (int64_t)u * E + i;
            if (i >= inst_count[u]) {
                *out = -1;
                continue;
            }
            const int e = inst_expert[(int64_t)u * E + i];
            if (home_rank(e, R, E) == u) {
                *out = e;
            } else {
                *out = j < B ? E + j : e;
                j++;
            }
        }
    }
    return OR_OK;
}

/*
 * oracle_plan_dedup: per-destination token dedup of rank m's dispatch
 * ("MoonEP API完全参考", §5.2 communication performance: a check of the
 * dedup encoding of sent tokens is named there, nothing more). Reading: a token with several routes to one destination rank is
 * sent there once; the receiver fans the row out to each of the token's
 * grouped slots on that rank. From the global plan's route maps:
 *   D(g)             = { route_dest[g*K + k] : k < K } for global token
 *                      g = src*S + t
 *   send buffer of m : one row per (t, d) with d in D(m*S + t), ordered by
 *                      (d ascending, t ascending); dsend_count[d] = rows
 *                      for d
 *   dpack_pos[t*K+k] = that row for the first k of t with destination d,
 *                      -1 for t's later routes to the same d
 *   arrival on m     : sources ascending, each source's rows to m in token
 *                      order; drecv_count[src] = rows from src
 *   drecv_pos[slot]  = arrival row of the token whose route occupies
 *                      grouped slot `slot` on m
 * Pack with dpack_pos, exchange the segments, group with drecv_pos: the
 * grouped buffer equals the one of the plan's own maps.
 */
int oracle_plan_dedup(int R, int S, int K, int m, const int32_t* route_dest,
                      const int32_t* route_slot, int32_t* dpack_pos, int32_t* dsend_count,
                      int32_t* drecv_pos, int32_t* drecv_count) {
    if (R < 1 || S < 1 || K < 1 || m < 0 || m >= R) return OR_ERR_ARG;
    const int64_t C = (int64_t)S * K;
    /* sender side: count per destination, then rows in (d, t) order */
    for (int d = 0; d < R; d++) dsend_count[d] = 0;
    for (int64_t t = 0; t < S; t++)
        for (int k = 0; k < K; k++) {
            const int32_t d = route_dest[((int64_t)m * S + t) * K + k];
            int first = 1;
            for (int k2 = 0; k2 < k; k2++)
                if (route_dest[((int64_t)m * S + t) * K + k2] == d) first = 0;
            if (first && d >= 0 && d < R) dsend_count[d]++;
        }
    int64_t* base = (int64_t*)malloc(sizeof(int64_t) * (size_t)R);
    int64_t* next = (int64_t*)malloc(sizeof(int64_t) * (size_t)R);
    int64_t* arr = (int64_t*)malloc(sizeof(int64_t) * (size_t)R * S);
    if (!base || !next || !arr) {
        free(base);
        free(next);
        free(arr);
        return OR_ERR_ALLOC;
    }
    int64_t run = 0;
    for (int d = 0; d < R; d++) {
        base[d] = run;
        next[d] = 0;
        run += dsend_count[d];
    }
    for (int64_t t = 0; t < S; t++)
        for (int k = 0; k < K; k++) {
            const int32_t d = route_dest[((int64_t)m * S + t) * K + k];
            int first = 1;
            for (int k2 = 0; k2 < k; k2++)
                if (route_dest[((int64_t)m * S + t) * K + k2] == d) first = 0;
            if (first && d >= 0 && d < R) dpack_pos[t * K + k] = (int32_t)(base[d] + next[d]++);
            else dpack_pos[t * K + k] = -1;
        }
    /* receiver side: arrival row of every global token that reaches m */
    run = 0;
    for (int src = 0; src < R; src++) {
        int64_t cnt = 0;
        for (int64_t t = 0; t < S; t++) {
            const int64_t g = (int64_t)src * S + t;
            int reaches = 0;
            for (int k = 0; k < K; k++)
                if (route_dest[g * K + k] == m) reaches = 1;
            arr[g] = reaches ? run + cnt : -1;
            cnt += reaches;
        }
        drecv_count[src] = (int32_t)cnt;
        run += cnt;
    }
    for (int64_t s2 = 0; s2 < C; s2++) drecv_pos[s2] = -1;
    for (int64_t f = 0; f < (int64_t)R * C; f++)
        if (route_dest[f] == m) {
            const int32_t sl = route_slot[f];
            if (sl >= 0 && sl < C) drecv_pos[sl] = (int32_t)arr[f / K];
        }
    free(base);
    free(next);
    free(arr);
    return OR_OK;
}

/* Exposed for pinning the conversions in tests. */
void oracle_bf16_from_float(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; i++) out[i] = float_to_bf16_rne(in[i]);
}

void oracle_float_from_fp16(const uint16_t* in, float* out, int64_t n) {
    for (int64_t i = 0; i < n; i++) out[i] = fp16_to_float(in[i]);
}

/* ------------------------------------------------ zero-copy and return */

/*
 * oracle_push: zero-copy dispatch ([MoonEP-TD]: rows written straight to
 * their grouped position on the receiving rank). All R grouped buffers are
 * one host array [R*C][H]: for every route (t,k) of this rank,
 *   grouped[route_dest*C + route_slot] = x[t]   (out-of-range maps skipped).
 */
int oracle_push(int T, int K, int H, int R, int C, const uint16_t* x,
                const int32_t* route_dest, const int32_t* route_slot, uint16_t* grouped) {
    if (T < 0 || K < 1 || H < 1 || R < 1 || C < 1) return OR_ERR_ARG;
    for (int64_t t = 0; t < T; t++)
        for (int k = 0; k < K; k++) {
            int32_t d = route_dest[t * K + k], s = route_slot[t * K + k];
            if (d < 0 || d >= R || s < 0 || s >= C) continue;
            for (int64_t h = 0; h < H; h++)
                grouped[((int64_t)d * C + s) * H + h] = x[t * H + h];
        }
    return OR_OK;
}

/*
 * oracle_pull_combine: zero-copy combine, the same reduction as
 * oracle_combine with each route's expert output read from its grouped
 * position: y = grouped[route_dest*C + route_slot].
 */
int oracle_pull_combine(int T, int K, int H, int R, int C, const uint16_t* grouped,
                        const int32_t* route_dest, const int32_t* route_slot,
                        const float* scores, uint16_t* out_bf16, float* out_f32) {
    if (T < 0 || K < 1 || H < 1 || R < 1 || C < 1) return OR_ERR_ARG;
    for (int64_t t = 0; t < T; t++)
        for (int64_t h = 0; h < H; h++) {
            float acc = 0.0f;
            for (int k = 0; k < K; k++) {
                int32_t d = route_dest[t * K + k], s = route_slot[t * K + k];
                if (d < 0 || d >= R || s < 0 || s >= C) continue;
                float y = bf16_to_float(grouped[((int64_t)d * C + s) * H + h]);
                float prod = scores[t * K + k] * y;
                acc = acc + prod;
            }
            if (out_f32) out_f32[t * H + h] = acc;
            if (out_bf16) out_bf16[t * H + h] = float_to_bf16_rne(acc);
        }
    return OR_OK;
}

/*
 * oracle_ungroup: y_arrival[recv_pos[t]] = y_grouped[t], the inverse of
 * oracle_group (entries outside [0, n) skipped).
 */
int oracle_ungroup(int n, int H, const int32_t* recv_pos, const uint16_t* y_grouped,
                   uint16_t* y_arrival) {
    if (n < 0 || H < 1) return OR_ERR_ARG;
    for (int64_t t = 0; t < n; t++) {
        int32_t to = recv_pos[t];
        if (to < 0 || to >= n) continue;
        for (int64_t h = 0; h < H; h++)
            y_arrival[(int64_t)to * H + h] = y_grouped[t * H + h];
    }
    return OR_OK;
}
