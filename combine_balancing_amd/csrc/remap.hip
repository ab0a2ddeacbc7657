// mep_remap_prune: EPLB logical -> physical instance remap, score pruning
// and the send map of the remapped routes.
//
// Method ("aclnnMoeUpdateExpert" op doc, section "功能说明"): each (token,
// k) expert id is replaced by one of the instances its eplb_table row lists
// (by rank in balance_mode 0, rotating over tokens in mode 1); a route whose
// scale falls below the token's sum of scale x threshold is pruned, and an
// inactive token loses all its routes. The send map orders the kept routes
// by destination card and instance, so that a following dispatch writes one
// contiguous segment per card.
//
// One work-group does the whole call (BS*K is at most a few thousand
// entries, so this is latency-bound). Each wave owns a contiguous range of
// entries. One pass computes their ids and masks and, for the send map,
// each kept route's rank among the wave's earlier routes to the same
// instance (a ballot multi-split per 64 entries and a running per-wave
// count in LDS). A block scan over the (instance, wave) counts then gives
// every wave's base per instance. No atomics decide an order, so the
// output is deterministic.
#include "mep_device.h"

namespace mep {
namespace {

constexpr int kRemapThreads = 1024;
constexpr int kRemapWaves = kRemapThreads / kWave;
constexpr int kMaxInst = 1024;
constexpr int kMaxE = 1024;
constexpr int kMaxBS = 512;
constexpr int kMaxK = 16;
constexpr int kMaxEntries = kMaxBS * kMaxK;
constexpr int kMaxBatches = kMaxEntries / kRemapThreads;  // 64-entry batches per wave, at most
constexpr int kStageTable = 9216;  // eplb_table entries kept in LDS (36 KiB)

struct RemapArgs {
    int BS, K, E, F, ws, ppr, rank, mode, scale_dtype;
    const int* __restrict__ ids;
    const int* __restrict__ table;
    const void* __restrict__ scales;
    const float* __restrict__ thr;
    const uint8_t* __restrict__ active;
    int* __restrict__ out_ids;
    uint8_t* __restrict__ out_mask;
    int* __restrict__ send_pos;
    int* __restrict__ send_count;
};

// A scale's bit pattern widened exactly to fp32.
__device__ __forceinline__ float scale_value(uint32_t raw, int dtype) {
    if (dtype == MEP_SCALE_F32) return __uint_as_float(raw);
    if (dtype == MEP_SCALE_BF16) return __uint_as_float(raw << 16);
    return (float)__builtin_bit_cast(_Float16, (uint16_t)raw);
}

// Entry i = t*K + k of the thread's r-th slot: i = lo + r * 64 + lane, where
// wave w owns entries [lo, hi) = [w*seg, w*seg + seg) clipped to n and seg
// is n/16 rounded up to a multiple of 64, at most NB batches (every access
// of a wave covers 64 consecutive entries). Token and column indices use
// exact multiply-shift reciprocals instead of integer divisions:
// t = (i*kmag) >> 21 for i < 8192 and K <= 16, and t / count = (t*m) >> 20
// for t < 512 and count <= 1024, with kmag = ceil(2^21/K) and
// m = ceil(2^20/count).
// TAB_STAGED: the table fits the LDS stage (E*F <= kStageTable) and is read
// from LDS; otherwise from global memory. A compile-time choice keeps the
// table reads plain LDS loads (a pointer chosen at run time between the two
// made them generic loads, which wait on both memory counters).
template <bool TAB_STAGED, int NB>
__global__ __launch_bounds__(kRemapThreads) void remap_prune_kernel(RemapArgs a) {
    // The send-map counters have their own space, so they are cleared while
    // the first loads are in flight.
    __shared__ int s_tab[kStageTable];                // eplb_table, when it fits
    __shared__ int s_cnt[kRemapWaves * kMaxInst];     // [wave][n_inst] send-map counts, then bases
    __shared__ float s_sc[kMaxK * (kMaxBS + 1)];      // scales as fp32, [k][t] skewed by one
    __shared__ float s_sum[kMaxBS];                   // per-token threshold sums
    __shared__ uint8_t s_act[kMaxBS];
    __shared__ float s_thr[kMaxK];
    __shared__ int s_col[kMaxE];                      // mode 0: column; mode 1: reciprocal of count
    __shared__ int s_tot[kMaxInst];
    __shared__ int scratch[kRemapThreads / kWave + 1];
    const int n = a.BS * a.K;
    const int tid = threadIdx.x;
    const int n_inst = a.ws * a.ppr;
    const bool pruning = a.scales != nullptr;
    const int tab_n = a.E * a.F;
    const unsigned kmag = ((1u << 21) + a.K - 1) / a.K;
    const int S1 = a.BS + 1;
    const int wave = tid / kWave;
    const int lane = tid & (kWave - 1);
    const int seg = (((n + kRemapWaves - 1) / kRemapWaves) + kWave - 1) & ~(kWave - 1);
    const int lo = min(wave * seg, n);
    const int hi = min(lo + seg, n);

    // 1. one round trip: the table (when it fits), ids, scales, thresholds
    //    and the active mask are all requested before any is used.
    //  - The table goes straight from global memory into LDS (gfx950's
    //    global_load_lds; each wave instruction fills 64 consecutive ints
    //    at a wave-uniform LDS address), so it holds no registers.
    //  - Ids and scales: NB batches per wave, unconditionally, at indices
    //    clamped into range (a lane past the wave's entries reloads its last
    //    one and never uses it). A load under a lane condition made the
    //    compiler wait for it where the branches join.
    if (TAB_STAGED)
        for (int b = wave * kWave; b < tab_n; b += kRemapThreads)
            if (b + lane < tab_n) __builtin_amdgcn_global_load_lds(a.table + b + lane, s_tab + b, 4, 0, 0);
    const int last = max(hi - 1, 0);
    int e[NB];
    uint32_t raw[NB];  // scale bit patterns
#pragma unroll
    for (int r = 0; r < NB; ++r) e[r] = a.ids[min(lo + r * kWave + lane, last)];
    if (pruning) {
        if (a.scale_dtype == MEP_SCALE_F32) {
#pragma unroll
            for (int r = 0; r < NB; ++r)
                raw[r] = ((const uint32_t*)a.scales)[min(lo + r * kWave + lane, last)];
        } else {
#pragma unroll
            for (int r = 0; r < NB; ++r)
                raw[r] = ((const uint16_t*)a.scales)[min(lo + r * kWave + lane, last)];
        }
    }
    float thr = 0.0f;
    if (pruning) thr = a.thr[min(tid, a.K - 1)];
    uint32_t act = 1u;
    if (pruning && a.active) act = a.active[min(tid, a.BS - 1)];
    // the send-map counters are cleared while the loads above are in flight
    if (a.send_pos)
        for (int i = tid; i < kRemapWaves * n_inst; i += kRemapThreads) s_cnt[i] = 0;
    if (pruning && tid < a.K) s_thr[tid] = thr;
    // opaque here, so the test below is not moved up to the load and its
    // wait with it
    asm volatile("" : "+v"(act));
    if (tid < a.BS) s_act[tid] = act != 0;
    if (pruning) {
#pragma unroll
        for (int r = 0; r < NB; ++r) {
            const int i = lo + r * kWave + lane;
            const int t = (int)(((unsigned)i * kmag) >> 21);
            if (i < hi) s_sc[(i - t * a.K) * S1 + t] = scale_value(raw[r], a.scale_dtype);
        }
    }
    // the table's LDS writes count on vmcnt: every wave's must be done
    // before the barrier
    if (TAB_STAGED) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    const int* tab = TAB_STAGED ? s_tab : a.table;

    // 2. per expert: the mode-0 column (it depends on the rank and the
    //    expert's count only) or the count's reciprocal for mode 1; per
    //    token: sum of scale x threshold in k order from +0 (fp32, no FMA)
    if (tid < a.E) {
        const int count = tab[(size_t)tid * a.F];
        if (a.mode == 0) s_col[tid] = count > 1 ? a.rank / ((a.ws + count - 1) / count) + 1 : 1;
        else s_col[tid] = count > 1 ? (int)(((1u << 20) + count - 1) / count) : 0;
    }
    if (pruning && tid < a.BS) {
        float sum = 0.0f;
        for (int k = 0; k < a.K; ++k) {
            const float prod = s_sc[k * S1 + tid] * s_thr[k];
            sum = sum + prod;
        }
        s_sum[tid] = sum;
    }
    lds_barrier();

    // 3. remap and mask every entry; outputs. With a send map, each kept
    //    route's rank among this wave's earlier routes to its instance: the
    //    lowest lane of each equal-key group advances the wave's count.
    const bool mapping = a.send_pos != nullptr;
    int* my_cnt = s_cnt + wave * n_inst;
    int inst[NB];
    int rank[NB];
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        const int b0 = lo + r * kWave;
        if (b0 >= hi) break;  // wave-uniform
        const int i = b0 + lane;
        int ins = -1;
        if (i < hi) {
            const int t = (int)(((unsigned)i * kmag) >> 21);
            int bal = -1;
            if ((unsigned)e[r] < (unsigned)a.E) {
                const int* row = tab + (size_t)e[r] * a.F;
                int col;
                if (a.mode == 0) {
                    col = s_col[e[r]];
                } else {
                    const int count = row[0];
                    col = count > 1
                              ? t - count * (int)(((unsigned)t * (unsigned)s_col[e[r]]) >> 20) + 1
                              : 1;
                }
                bal = row[clampi(col, 1, a.F - 1)];
            }
            const uint8_t keep =
                pruning ? (uint8_t)(s_act[t] && !(scale_value(raw[r], a.scale_dtype) < s_sum[t]))
                        : (uint8_t)1;
            a.out_ids[i] = bal;
            a.out_mask[i] = keep;
            if (keep && (unsigned)bal < (unsigned)n_inst) ins = bal;
        }
        inst[r] = ins;
        if (mapping) {
            const bool valid = ins >= 0;
            const int key = valid ? ins : 0;
            const uint64_t peers = match_peers(key, valid);
            const int below = count_below(peers);
            rank[r] = my_cnt[key] + below;
            if (valid && below == 0) my_cnt[key] += __popcll(peers);
        }
    }
    if (!mapping) return;

    // 4. send map: per-instance totals, then each wave's base per instance
    //    in (instance, wave) order; an instance's wave counts are read once
    //    and kept for the bases
    lds_barrier();
    int tot = 0;
    int wc[kRemapWaves];
#pragma unroll
    for (int v = 0; v < kRemapWaves; ++v) {
        wc[v] = tid < n_inst ? s_cnt[v * n_inst + tid] : 0;
        tot += wc[v];
    }
    int all;
    const int base = block_exclusive_sum<false>(tot, scratch, &all);  // scratch is not reused
    if (tid < n_inst) {
        s_tot[tid] = tot;
        int run = base;
#pragma unroll
        for (int v = 0; v < kRemapWaves; ++v) {
            s_cnt[v * n_inst + tid] = run;
            run += wc[v];
        }
    }
    lds_barrier();
    for (int card = tid; card < a.ws; card += kRemapThreads) {
        int c = 0;
        for (int j = 0; j < a.ppr; ++j) c += s_tot[card * a.ppr + j];
        a.send_count[card] = c;
    }
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        const int b0 = lo + r * kWave;
        if (b0 >= hi) break;
        const int i = b0 + lane;
        if (i < hi) a.send_pos[i] = inst[r] >= 0 ? my_cnt[inst[r]] + rank[r] : -1;
    }
}

}  // namespace
}  // namespace mep

using namespace mep;

extern "C" int mep_remap_prune(int BS, int K, int E, int F, int world_size, int place_per_rank,
                               int local_rank_id, int balance_mode, const int32_t* expert_ids,
                               const int32_t* eplb_table, const void* expert_scales,
                               int scale_dtype, const float* pruning_threshold,
                               const uint8_t* active_mask, int32_t* balanced_ids,
                               uint8_t* balanced_mask, int32_t* send_pos, int32_t* send_count,
                               void* stream) {
    if (!expert_ids || !eplb_table || !balanced_ids || !balanced_mask) return MEP_ERR_NULLPTR;
    if (balance_mode != 0 && balance_mode != 1) return MEP_ERR_PARAM;
    if ((expert_scales == nullptr) != (pruning_threshold == nullptr)) return MEP_ERR_PARAM;
    if (active_mask && !expert_scales) return MEP_ERR_PARAM;
    if ((send_pos == nullptr) != (send_count == nullptr)) return MEP_ERR_PARAM;
    if (expert_scales && scale_dtype != MEP_SCALE_F32 && scale_dtype != MEP_SCALE_BF16 &&
        scale_dtype != MEP_SCALE_F16)
        return MEP_ERR_PARAM;
    if (BS < 1 || BS > kMaxBS || K < 1 || K > kMaxK || E < 1 || E > 1024 || world_size < 1 ||
        world_size > 1024 || place_per_rank < 1 || F < 2 || F > world_size + 1 ||
        (long long)world_size * place_per_rank > kMaxInst)
        return MEP_ERR_SHAPE;
    if (K > E) return MEP_ERR_PARAM;
    if (balance_mode == 0 && (local_rank_id < 0 || local_rank_id >= world_size))
        return MEP_ERR_PARAM;
    RemapArgs a{BS, K, E, F, world_size, place_per_rank, local_rank_id, balance_mode, scale_dtype,
                (const int*)expert_ids, (const int*)eplb_table, expert_scales, pruning_threshold,
                active_mask, (int*)balanced_ids, balanced_mask, (int*)send_pos, (int*)send_count};
    // batches per wave (the kernel's seg / 64), rounded up to a power of two
    const int n = BS * K;
    const int nbat = ((n + kRemapWaves - 1) / kRemapWaves + kWave - 1) / kWave;
    const int nb = nbat <= 1 ? 1 : nbat <= 2 ? 2 : nbat <= 4 ? 4 : kMaxBatches;
    const bool staged = (long long)E * F <= kStageTable;
    const dim3 g(1), b(kRemapThreads);
    hipStream_t st = (hipStream_t)stream;
    if (staged && nb == 1) hipLaunchKernelGGL((remap_prune_kernel<true, 1>), g, b, 0, st, a);
    else if (staged && nb == 2) hipLaunchKernelGGL((remap_prune_kernel<true, 2>), g, b, 0, st, a);
    else if (staged && nb == 4) hipLaunchKernelGGL((remap_prune_kernel<true, 4>), g, b, 0, st, a);
    else if (staged) hipLaunchKernelGGL((remap_prune_kernel<true, kMaxBatches>), g, b, 0, st, a);
    else if (nb == 1) hipLaunchKernelGGL((remap_prune_kernel<false, 1>), g, b, 0, st, a);
    else if (nb == 2) hipLaunchKernelGGL((remap_prune_kernel<false, 2>), g, b, 0, st, a);
    else if (nb == 4) hipLaunchKernelGGL((remap_prune_kernel<false, 4>), g, b, 0, st, a);
    else hipLaunchKernelGGL((remap_prune_kernel<false, kMaxBatches>), g, b, 0, st, a);
    MEP_LAUNCH_CHECK();
    return MEP_OK;
}
