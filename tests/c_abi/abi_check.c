/*
 * A C consumer of libmep.so: no Python, no PyTorch. Runs the plan (with a
 * workspace and allocation-free), the EPLB remap/prune with its send map,
 * the pack, the receive grouping and the combine through the C ABI
 * (include/mep.h) on device buffers from the HIP runtime, and checks every
 * output bit for bit against the C oracle (oracle/oracle.c, test
 * infrastructure) on the host.
 * Also checks a few argument errors. Prints one line; exit status 0 on
 * success.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mep.h"

/* the oracle's entry points */
int oracle_plan(int R, int E, int S, int K, int m, const int32_t* ids, int32_t* expert_count,
                int32_t* rank_load, int32_t* route_dest, int32_t* route_slot,
                int32_t* inst_count, int32_t* inst_expert, int32_t* inst_cu,
                int32_t* inst_gid_base, int32_t* send_pos, int32_t* send_count,
                int32_t* recv_pos, int32_t* recv_count);
int oracle_pack(int T, int K, int H, const uint16_t* x, const int32_t* send_pos,
                uint16_t* send_buf);
int oracle_group(int n_recv, int H, const int32_t* recv_pos, const uint16_t* recv_raw,
                 uint16_t* recv_grouped);
int oracle_combine(int T, int K, int H, const uint16_t* y_ret, const int32_t* send_pos,
                   const float* scores, uint16_t* out_bf16, float* out_f32);
int oracle_remap_prune(int BS, int K, int E, int F, int world_size, int place_per_rank,
                       int local_rank_id, int balance_mode, const int32_t* expert_ids,
                       const int32_t* eplb_table, const void* scales, int scale_dtype,
                       const float* thr, const uint8_t* active, int32_t* balanced_ids,
                       uint8_t* balanced_mask, int32_t* send_pos, int32_t* send_count);

#define CHECK_HIP(x)                                                          \
    do {                                                                      \
        hipError_t e_ = (x);                                                  \
        if (e_ != hipSuccess) {                                               \
            printf("c abi: HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            exit(2);                                                          \
        }                                                                     \
    } while (0)

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) { /* splitmix64 */
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (uint32_t)((z ^ (z >> 31)) >> 32);
}
static float next_unit(void) { return (next_u32() >> 8) * (1.0f / 16777216.0f); }
static uint16_t bf16_trunc(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static void* dev_copy(const void* h, size_t n) {
    void* d = NULL;
    CHECK_HIP(hipMalloc(&d, n ? n : 16));
    if (n) CHECK_HIP(hipMemcpy(d, h, n, hipMemcpyHostToDevice));
    return d;
}
static void* dev_alloc(size_t n) {
    void* d = NULL;
    CHECK_HIP(hipMalloc(&d, n ? n : 16));
    return d;
}
static int same(const char* what, const void* d, const void* h, size_t n) {
    void* t = malloc(n);
    CHECK_HIP(hipMemcpy(t, d, n, hipMemcpyDeviceToHost));
    const int ok = memcmp(t, h, n) == 0;
    if (!ok) printf("c abi: %s differs from the oracle\n", what);
    free(t);
    return ok;
}

/* A small EPLB workload: a table of instance counts in [1,8] and distinct
 * instance ids, K distinct experts per token, bf16 scales sorted
 * descending, fp32 thresholds, an active mask with a tail of inactive
 * tokens. Both modes at one rank, every output compared with the oracle. */
static int check_remap(void) {
    const int E = 96, F = 9, ws = 40, ppr = 2, BS = 200, K = 8, rank = 13;
    const int n_inst = ws * ppr, n = BS * K;
    int32_t* table = malloc(4 * (size_t)E * F);
    for (int e = 0; e < E; e++) {
        const int cnt = 1 + (int)(next_u32() % 8);
        table[e * F] = cnt;
        for (int c = 1; c < F; c++) {
            int id, dup;
            do {
                id = (int)(next_u32() % n_inst);
                dup = 0;
                for (int j = 1; j < c; j++) dup |= table[e * F + j] == id;
            } while (dup);
            table[e * F + c] = id;
        }
    }
    int32_t* ids = malloc(4 * (size_t)n);
    uint16_t* sc = malloc(2 * (size_t)n);
    for (int t = 0; t < BS; t++) {
        float prev = 1.0f;
        for (int k = 0; k < K; k++) {
            int e, dup;
            do {
                e = (int)(next_u32() % E);
                dup = 0;
                for (int j = 0; j < k; j++) dup |= ids[t * K + j] == e;
            } while (dup);
            ids[t * K + k] = e;
            prev = prev * (0.3f + 0.7f * next_unit());
            sc[t * K + k] = bf16_trunc(prev);
        }
    }
    float thr[8];
    for (int k = 0; k < K; k++) thr[k] = 0.2f * next_unit();
    uint8_t* act = malloc((size_t)BS);
    for (int t = 0; t < BS; t++) act[t] = t < BS - 25;
    int32_t *bid = malloc(4 * (size_t)n), *spos = malloc(4 * (size_t)n), *scnt = malloc(4 * ws);
    uint8_t* bmask = malloc((size_t)n);
    int32_t* d_tab = dev_copy(table, 4 * (size_t)E * F);
    int32_t* d_ids = dev_copy(ids, 4 * (size_t)n);
    uint16_t* d_sc = dev_copy(sc, 2 * (size_t)n);
    float* d_thr = dev_copy(thr, 4 * K);
    uint8_t* d_act = dev_copy(act, (size_t)BS);
    int32_t *d_bid = dev_alloc(4 * (size_t)n), *d_spos = dev_alloc(4 * (size_t)n),
            *d_scnt = dev_alloc(4 * ws);
    uint8_t* d_bmask = dev_alloc((size_t)n);
    int ok = 1;
    for (int mode = 0; mode < 2; mode++) {
        if (oracle_remap_prune(BS, K, E, F, ws, ppr, rank, mode, ids, table, sc, MEP_SCALE_BF16, thr,
                               act, bid, bmask, spos, scnt) != 0) {
            printf("c abi: oracle_remap_prune failed\n");
            return 0;
        }
        const int st = mep_remap_prune(BS, K, E, F, ws, ppr, rank, mode, d_ids, d_tab, d_sc,
                                       MEP_SCALE_BF16, d_thr, d_act, d_bid, d_bmask, d_spos,
                                       d_scnt, NULL);
        if (st != MEP_OK) {
            printf("c abi: mep_remap_prune returned %d (%s)\n", st, mep_status_str(st));
            return 0;
        }
        CHECK_HIP(hipDeviceSynchronize());
        ok &= same(mode ? "remap mode 1 ids" : "remap mode 0 ids", d_bid, bid, 4 * (size_t)n);
        ok &= same(mode ? "remap mode 1 mask" : "remap mode 0 mask", d_bmask, bmask, (size_t)n);
        ok &= same(mode ? "remap mode 1 send_pos" : "remap mode 0 send_pos", d_spos, spos,
                   4 * (size_t)n);
        ok &= same(mode ? "remap mode 1 send_count" : "remap mode 0 send_count", d_scnt, scnt,
                   4 * (size_t)ws);
    }
    /* unpaired optional arguments are refused */
    ok &= mep_remap_prune(BS, K, E, F, ws, ppr, rank, 0, d_ids, d_tab, d_sc, MEP_SCALE_BF16, NULL,
                          NULL, d_bid, d_bmask, NULL, NULL, NULL) == MEP_ERR_PARAM;
    return ok;
}

int main(void) {
    const int R = 8, E = 64, S = 1024, K = 4, H = 2048, m = 3;
    const int C = S * K, N = R * C;
    /* skewed routing: K distinct experts per token, low ids more likely */
    int32_t* ids = malloc(sizeof(int32_t) * N);
    for (int g = 0; g < R * S; g++)
        for (int k = 0; k < K; k++) {
            int e, dup;
            do {
                const float u = next_unit();
                e = (int)(E * u * u);
                if (e >= E) e = E - 1;
                dup = 0;
                for (int j = 0; j < k; j++) dup |= ids[g * K + j] == e;
            } while (dup);
            ids[g * K + k] = e;
        }
    uint16_t* x = malloc(sizeof(uint16_t) * S * H);
    uint16_t* raw = malloc(sizeof(uint16_t) * C * H);
    for (int i = 0; i < S * H; i++) x[i] = bf16_trunc(4.0f * next_unit() - 2.0f);
    for (int i = 0; i < C * H; i++) raw[i] = bf16_trunc(4.0f * next_unit() - 2.0f);
    float* scores = malloc(sizeof(float) * C);
    for (int i = 0; i < C; i++) scores[i] = next_unit();

    /* oracle on the host */
    int32_t *ec = malloc(4 * E), *rl = malloc(4 * R), *rd = malloc(4 * (size_t)N),
            *rs = malloc(4 * (size_t)N), *ic = malloc(4 * R), *ie = malloc(4 * R * E),
            *icu = malloc(4 * R * (E + 1)), *igb = malloc(4 * (R + 1)), *sp = malloc(4 * C),
            *sc = malloc(4 * R), *rp = malloc(4 * C), *rc = malloc(4 * R);
    if (oracle_plan(R, E, S, K, m, ids, ec, rl, rd, rs, ic, ie, icu, igb, sp, sc, rp, rc) != 0) {
        printf("c abi: oracle_plan failed\n");
        return 1;
    }

    /* the library on the GPU */
    const size_t wsb = mep_plan_workspace_size(R, E, S, K);
    void* ws = dev_alloc(wsb);
    int32_t* d_ids = dev_copy(ids, 4 * (size_t)N);
    int32_t *d_ec = dev_alloc(4 * E), *d_rl = dev_alloc(4 * R), *d_rd = dev_alloc(4 * (size_t)N),
            *d_rs = dev_alloc(4 * (size_t)N), *d_ic = dev_alloc(4 * R), *d_ie = dev_alloc(4 * R * E),
            *d_icu = dev_alloc(4 * R * (E + 1)), *d_igb = dev_alloc(4 * (R + 1)),
            *d_sp = dev_alloc(4 * C), *d_sc = dev_alloc(4 * R), *d_rp = dev_alloc(4 * C),
            *d_rc = dev_alloc(4 * R);
    int st = mep_plan(R, E, S, K, m, d_ids, ws, wsb, d_ec, d_rl, d_rd, d_rs, d_ic, d_ie, d_icu,
                      d_igb, d_sp, d_sc, d_rp, d_rc, NULL);
    if (st != MEP_OK) {
        printf("c abi: mep_plan returned %d (%s)\n", st, mep_status_str(st));
        return 1;
    }
    CHECK_HIP(hipDeviceSynchronize());
    int ok = 1;
    ok &= same("expert_count", d_ec, ec, 4 * E);
    ok &= same("rank_load", d_rl, rl, 4 * R);
    ok &= same("route_dest", d_rd, rd, 4 * (size_t)N);
    ok &= same("route_slot", d_rs, rs, 4 * (size_t)N);
    ok &= same("inst_count", d_ic, ic, 4 * R);
    ok &= same("inst_expert", d_ie, ie, 4 * R * E);
    ok &= same("inst_cu", d_icu, icu, 4 * R * (E + 1));
    ok &= same("inst_gid_base", d_igb, igb, 4 * (R + 1));
    ok &= same("send_pos", d_sp, sp, 4 * C);
    ok &= same("send_count", d_sc, sc, 4 * R);
    ok &= same("recv_pos", d_rp, rp, 4 * C);
    ok &= same("recv_count", d_rc, rc, 4 * R);

    /* the allocation-free plan: same outputs, no workspace argument */
    CHECK_HIP(hipMemset(d_rd, 0xFF, 4 * (size_t)N));
    CHECK_HIP(hipMemset(d_sp, 0xFF, 4 * C));
    st = mep_plan_noalloc(R, E, S, K, m, d_ids, d_ec, d_rl, d_rd, d_rs, d_ic, d_ie, d_icu, d_igb,
                          d_sp, d_sc, d_rp, d_rc, NULL);
    if (st != MEP_OK) {
        printf("c abi: mep_plan_noalloc returned %d (%s)\n", st, mep_status_str(st));
        return 1;
    }
    CHECK_HIP(hipDeviceSynchronize());
    ok &= same("noalloc route_dest", d_rd, rd, 4 * (size_t)N);
    ok &= same("noalloc route_slot", d_rs, rs, 4 * (size_t)N);
    ok &= same("noalloc inst_cu", d_icu, icu, 4 * R * (E + 1));
    ok &= same("noalloc send_pos", d_sp, sp, 4 * C);
    ok &= same("noalloc recv_pos", d_rp, rp, 4 * C);

    /* EPLB remap + prune with its send map, both balance modes, bf16 scales */
    ok &= check_remap();

    /* pack, group, combine */
    uint16_t *send = calloc((size_t)C * H, 2), *grouped = calloc((size_t)C * H, 2);
    uint16_t* ob = malloc(2 * (size_t)S * H);
    float* of = malloc(4 * (size_t)S * H);
    oracle_pack(S, K, H, x, sp, send);
    oracle_group(C, H, rp, raw, grouped);
    oracle_combine(S, K, H, send, sp, scores, ob, of);
    uint16_t* d_x = dev_copy(x, 2 * (size_t)S * H);
    uint16_t* d_raw = dev_copy(raw, 2 * (size_t)C * H);
    float* d_scores = dev_copy(scores, 4 * (size_t)C);
    uint16_t *d_send = dev_alloc(2 * (size_t)C * H), *d_grouped = dev_alloc(2 * (size_t)C * H),
             *d_ob = dev_alloc(2 * (size_t)S * H);
    float* d_of = dev_alloc(4 * (size_t)S * H);
    CHECK_HIP(hipMemset(d_send, 0, 2 * (size_t)C * H));
    st = mep_dispatch(S, K, H, d_x, d_sp, d_send, C, C, d_rp, d_raw, C, d_grouped, NULL);
    st = st ? st : mep_combine(S, K, H, d_send, C, d_sp, d_scores, d_ob, d_of, NULL);
    if (st != MEP_OK) {
        printf("c abi: dispatch/combine returned %d (%s)\n", st, mep_status_str(st));
        return 1;
    }
    CHECK_HIP(hipDeviceSynchronize());
    ok &= same("send_buf", d_send, send, 2 * (size_t)C * H);
    ok &= same("recv_grouped", d_grouped, grouped, 2 * (size_t)C * H);
    ok &= same("combine bf16", d_ob, ob, 2 * (size_t)S * H);
    ok &= same("combine fp32", d_of, of, 4 * (size_t)S * H);

    /* argument errors are reported, nothing is launched */
    ok &= mep_plan(R, E, S, K, R, d_ids, ws, wsb, d_ec, d_rl, d_rd, d_rs, d_ic, d_ie, d_icu,
                   d_igb, d_sp, d_sc, d_rp, d_rc, NULL) == MEP_ERR_PARAM;
    ok &= mep_dispatch(S, K, 12, d_x, d_sp, d_send, C, 0, NULL, NULL, 0, NULL, NULL) == MEP_ERR_SHAPE;
    ok &= mep_combine(S, K, H, NULL, C, d_sp, d_scores, d_ob, NULL, NULL) == MEP_ERR_NULLPTR;
    ok &= mep_version() > 0 && strlen(mep_status_str(MEP_ERR_SHAPE)) > 0;

    printf(ok ? "c abi ok: plan, allocation-free plan, remap/prune, pack, group, combine "
                "bit-exact against the oracle\n"
              : "c abi: FAILED\n");
    return ok ? 0 : 1;
}
