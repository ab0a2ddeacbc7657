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
constexpr int kMaxBS = 512;
constexpr int kMaxK = 16;
constexpr int kMaxEntries = kMaxBS * kMaxK;
constexpr int kPerThread = kMaxEntries / kRemapThreads;

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

__device__ __forceinline__ float load_scale(const void* p, int dtype, int i) {
    if (dtype == MEP_SCALE_F32) return ((const float*)p)[i];
    const uint16_t h = ((const uint16_t*)p)[i];
    if (dtype == MEP_SCALE_BF16) return __uint_as_float((uint32_t)h << 16);
    return (float)__builtin_bit_cast(_Float16, h);
}

// Entry i = t*K + k of the thread's r-th slot: i = tid + r * kRemapThreads.
__global__ __launch_bounds__(kRemapThreads) void remap_prune_kernel(RemapArgs a) {
    __shared__ float s_sc[kMaxEntries];               // scales widened to fp32
    __shared__ int s_bal[kMaxEntries];                // remapped ids
    __shared__ uint8_t s_keep[kMaxEntries];           // prune mask
    __shared__ float s_sum[kMaxBS];                   // per-token threshold sums
    __shared__ int s_cnt[kRemapWaves * kMaxInst];     // send-map counts
    __shared__ int s_tot[kMaxInst];
    __shared__ int scratch[kRemapThreads / kWave + 1];
    const int n = a.BS * a.K;
    const int tid = threadIdx.x;
    const int n_inst = a.ws * a.ppr;
    const bool pruning = a.scales != nullptr;

    // 1. ids, their table rows' counts and (for pruning) the scales: the
    //    loads of all of a thread's entries are issued together.
    int e[kPerThread], cnt[kPerThread];
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
        const int i = tid + r * kRemapThreads;
        e[r] = i < n ? a.ids[i] : -1;
        if (pruning && i < n) s_sc[i] = load_scale(a.scales, a.scale_dtype, i);
    }
#pragma unroll
    for (int r = 0; r < kPerThread; ++r)
        cnt[r] = (unsigned)e[r] < (unsigned)a.E ? a.table[(size_t)e[r] * a.F] : 1;
    int bal[kPerThread];
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
        const int i = tid + r * kRemapThreads;
        const int t = i / a.K;
        int col = 1;
        if (cnt[r] > 1) {
            if (a.mode == 0) col = a.rank / ((a.ws + cnt[r] - 1) / cnt[r]) + 1;
            else col = t % cnt[r] + 1;
        }
        col = clampi(col, 1, a.F - 1);
        bal[r] = (unsigned)e[r] < (unsigned)a.E ? a.table[(size_t)e[r] * a.F + col] : -1;
    }
    __syncthreads();

    // 2. per-token sum of scale x threshold, in k order from +0 (fp32, no FMA)
    if (pruning && tid < a.BS) {
        float sum = 0.0f;
        for (int k = 0; k < a.K; ++k) {
            const float prod = s_sc[tid * a.K + k] * a.thr[k];
            sum = sum + prod;
        }
        s_sum[tid] = sum;
    }
    __syncthreads();

    // 3. masks; outputs
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
        const int i = tid + r * kRemapThreads;
        if (i >= n) continue;
        const int t = i / a.K;
        uint8_t keep = 1;
        if (pruning) {
            const bool act = a.active ? a.active[t] != 0 : true;
            keep = (uint8_t)(act && !(s_sc[i] < s_sum[t]));
        }
        a.out_ids[i] = bal[r];
        a.out_mask[i] = keep;
        s_bal[i] = bal[r];
        s_keep[i] = keep;
    }
    if (!a.send_pos) return;

    // 4. send map: stable counting sort of kept routes by instance
    for (int i = tid; i < kRemapWaves * n_inst; i += kRemapThreads) s_cnt[i] = 0;
    __syncthreads();
    const int wave = tid / kWave;
    const int lane = tid & (kWave - 1);
    const int seg = (((n + kRemapWaves - 1) / kRemapWaves) + kWave - 1) & ~(kWave - 1);
    const int lo = min(wave * seg, n);
    const int hi = min(lo + seg, n);
    int* my_cnt = s_cnt + wave * n_inst;
    for (int i = lo + lane; i < hi; i += kWave) {
        const int inst = s_bal[i];
        if (s_keep[i] && (unsigned)inst < (unsigned)n_inst) atomicAdd(&my_cnt[inst], 1);
    }
    __syncthreads();
    // per-instance totals, then exclusive offsets in (instance, wave) order
    int tot = 0;
    if (tid < n_inst)
        for (int v = 0; v < kRemapWaves; ++v) tot += s_cnt[v * n_inst + tid];
    int all;
    const int base = block_exclusive_sum(tot, scratch, &all);
    if (tid < n_inst) {
        s_tot[tid] = tot;
        int run = base;
        for (int v = 0; v < kRemapWaves; ++v) {
            const int c = s_cnt[v * n_inst + tid];
            s_cnt[v * n_inst + tid] = run;
            run += c;
        }
    }
    __syncthreads();
    for (int card = tid; card < a.ws; card += kRemapThreads) {
        int c = 0;
        for (int j = 0; j < a.ppr; ++j) c += s_tot[card * a.ppr + j];
        a.send_count[card] = c;
    }
    int nbits = 0;
    while ((1 << nbits) < n_inst) ++nbits;
    for (int b0 = lo; b0 < hi; b0 += kWave) {
        const int i = b0 + lane;
        bool valid = i < hi;
        int inst = valid ? s_bal[i] : 0;
        valid = valid && s_keep[i] && (unsigned)inst < (unsigned)n_inst;
        if (!valid) inst = 0;
        const uint64_t peers = match_peers(inst, valid, nbits);
        const int r = my_cnt[inst] + count_below(peers);
        if (valid && is_group_leader(peers)) my_cnt[inst] += __popcll(peers);
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
    hipLaunchKernelGGL(remap_prune_kernel, dim3(1), dim3(kRemapThreads), 0, (hipStream_t)stream,
                       a);
    MEP_LAUNCH_CHECK();
    return MEP_OK;
}
