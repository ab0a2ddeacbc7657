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
// entries, so this is latency-bound): a strided pass computes ids and
// masks; the send map is a stable counting sort by instance built from
// per-wave LDS counts and a ballot multi-split (no atomics decide an
// order, so the output is deterministic).
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
constexpr int kPerThread = kMaxEntries / kRemapThreads;
constexpr int kCountWaves = kRemapWaves;  // waves that build the send map
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

// Entry i = t*K + k of the thread's r-th slot: i = tid + r * kRemapThreads
// (coalesced loads and stores). Token and column indices use exact
// multiply-shift reciprocals instead of integer divisions: t = (i*kmag) >> 21
// for i < 8192 and K <= 16, and t / count = (t*m) >> 20 for t < 512 and
// count <= 1024, with kmag = ceil(2^21/K) and m = ceil(2^20/count).
// TAB_STAGED: the table fits the LDS stage (E*F <= kStageTable) and is read
// from LDS; otherwise from global memory. A compile-time choice keeps the
// table reads plain LDS loads (a pointer chosen at run time between the two
// made them generic loads, which wait on both memory counters).
template <bool TAB_STAGED>
__global__ __launch_bounds__(kRemapThreads) void remap_prune_kernel(RemapArgs a) {
    // The send-map counters have their own space, so they are cleared while
    // the first loads are in flight.
    __shared__ int s_tab[kStageTable];                // eplb_table, when it fits
    __shared__ int s_cnt[kCountWaves * kMaxInst];     // [kCountWaves][n_inst] send-map counts
    __shared__ int16_t s_inst[kMaxEntries];           // kept route's instance, else -1
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

    // 1. one round trip: ids, scales, thresholds, the active mask and (when
    //    it fits) the whole table
    int e[kPerThread];
    uint32_t raw[kPerThread];  // scale bit patterns; converted after every load is issued
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
        const int i = tid + r * kRemapThreads;
        e[r] = i < n ? a.ids[i] : -1;
    }
    if (pruning) {
        if (a.scale_dtype == MEP_SCALE_F32) {
#pragma unroll
            for (int r = 0; r < kPerThread; ++r) {
                const int i = tid + r * kRemapThreads;
                raw[r] = i < n ? ((const uint32_t*)a.scales)[i] : 0u;
            }
        } else {
#pragma unroll
            for (int r = 0; r < kPerThread; ++r) {
                const int i = tid + r * kRemapThreads;
                raw[r] = i < n ? ((const uint16_t*)a.scales)[i] : 0u;
            }
        }
    }
    // the send-map counters are cleared while the loads above are in flight
    if (a.send_pos)
        for (int i = tid; i < kCountWaves * n_inst; i += kRemapThreads) s_cnt[i] = 0;
    if (TAB_STAGED) stage<kRemapThreads, kStageTable / kRemapThreads>(s_tab, a.table, tab_n);
    if (pruning && tid < a.K) s_thr[tid] = a.thr[tid];
    if (tid < a.BS) s_act[tid] = (pruning && a.active) ? (a.active[tid] != 0) : 1;
    if (pruning) {
#pragma unroll
        for (int r = 0; r < kPerThread; ++r) {
            const int i = tid + r * kRemapThreads;
            const int t = (int)(((unsigned)i * kmag) >> 21);
            if (i < n) s_sc[(i - t * a.K) * S1 + t] = scale_value(raw[r], a.scale_dtype);
        }
    }
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

    // 3. remap and mask every entry; outputs
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
        const int i = tid + r * kRemapThreads;
        if (i >= n) continue;
        const int t = (int)(((unsigned)i * kmag) >> 21);
        int bal = -1;
        if ((unsigned)e[r] < (unsigned)a.E) {
            const int* row = tab + (size_t)e[r] * a.F;
            int col;
            if (a.mode == 0) {
                col = s_col[e[r]];
            } else {
                const int count = row[0];
                col = count > 1 ? t - count * (int)(((unsigned)t * (unsigned)s_col[e[r]]) >> 20) + 1
                                : 1;
            }
            bal = row[clampi(col, 1, a.F - 1)];
        }
        const uint8_t keep =
            pruning ? (uint8_t)(s_act[t] && !(s_sc[(i - t * a.K) * S1 + t] < s_sum[t])) : (uint8_t)1;
        a.out_ids[i] = bal;
        a.out_mask[i] = keep;
        s_inst[i] = (int16_t)(keep && (unsigned)bal < (unsigned)n_inst ? bal : -1);
    }
    if (!a.send_pos) return;

    // 4. send map: stable counting sort of kept routes by instance; the
    //    first kCountWaves waves each own a contiguous range of entries
    lds_barrier();
    const int wave = tid / kWave;
    const int lane = tid & (kWave - 1);
    const int seg = (((n + kCountWaves - 1) / kCountWaves) + kWave - 1) & ~(kWave - 1);
    const int lo = wave < kCountWaves ? min(wave * seg, n) : n;
    const int hi = wave < kCountWaves ? min(lo + seg, n) : n;
    int* my_cnt = s_cnt + min(wave, kCountWaves - 1) * n_inst;
    for (int i = lo + lane; i < hi; i += kWave) {
        const int inst = s_inst[i];
        if (inst >= 0) atomicAdd(&my_cnt[inst], 1);
    }
    lds_barrier();
    // per-instance totals, then exclusive offsets in (instance, wave) order;
    // an instance's wave counts are read once and kept for the offsets
    int tot = 0;
    int wc[kCountWaves];
#pragma unroll
    for (int v = 0; v < kCountWaves; ++v) {
        wc[v] = tid < n_inst ? s_cnt[v * n_inst + tid] : 0;
        tot += wc[v];
    }
    int all;
    const int base = block_exclusive_sum<false>(tot, scratch, &all);  // scratch is not reused
    if (tid < n_inst) {
        s_tot[tid] = tot;
        int run = base;
#pragma unroll
        for (int v = 0; v < kCountWaves; ++v) {
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
    for (int b0 = lo; b0 < hi; b0 += kWave) {
        const int i = b0 + lane;
        bool valid = i < hi;
        int inst = valid ? s_inst[i] : -1;
        valid = inst >= 0;
        if (!valid) inst = 0;
        const uint64_t peers = match_peers(inst, valid);
        const int below = count_below(peers);
        const int r = my_cnt[inst] + below;
        if (valid && below == 0) my_cnt[inst] += __popcll(peers);  // the group's lowest lane
        if (i < hi) a.send_pos[i] = valid ? r : -1;
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
    if ((long long)E * F <= kStageTable)
        hipLaunchKernelGGL(remap_prune_kernel<true>, dim3(1), dim3(kRemapThreads), 0,
                           (hipStream_t)stream, a);
    else
        hipLaunchKernelGGL(remap_prune_kernel<false>, dim3(1), dim3(kRemapThreads), 0,
                           (hipStream_t)stream, a);
    MEP_LAUNCH_CHECK();
    return MEP_OK;
}
