// Per-destination token dedup of this rank's dispatch.
//
// Method ("MoonEP API完全参考", §5.2 communication performance, which names a
// dedup encoding of sent tokens): a token with several routes to one
// destination rank is sent there once, and the receiver fans the row out to
// each of the token's grouped slots. From the global plan's route maps:
//   D(g)         destinations of global token g = src*S + t
//   Q[g][d]      number of global tokens g' < g with d in D(g')
// this rank m's send buffer holds one row per (t, d), d in D(m*S+t), in
// (d, t) order:
//   dpack_pos[t*K+k] = segbase[d] + Q[m*S+t][d] - Q[m*S][d] for the first
//                      route of t to d (-1 for t's later routes to d)
//   dsend_count[d]   = Q[(m+1)*S][d] - Q[m*S][d]
// and its arrival buffer holds the rows reaching m, sources ascending, each
// in token order, which is global token order, so
//   drecv_pos[slot]  = Q[g][m] for the route of g occupying slot on m
//   drecv_count[src] = Q[(src+1)*S][m] - Q[src*S][m].
//
// Two or three launches (latency-bound, like the plan):
//   dedup_count  one 1024-thread work-group per chunk of 1024 tokens (chunks
//                never straddle a source): each token's destination bit
//                mask, then per-destination counts by wave ballots
//   dedup_scan   one work-group: per destination, exclusive scan of the
//                chunk counts (16 threads per destination, DPP-free: a
//                16-lane shuffle scan), plus the send/receive counts and
//                segment bases of rank m
//   dedup_maps   per chunk: the token's routes loaded once (destinations
//                and slots together), Q of every token for its destinations
//                from the chunk base, the wave bases and the token's rank in
//                its wave's ballot (kept in LDS); writes the three maps
// When the chunk counts are small (nchunks * R <= kDedupFusedInts, 1 KiB at
// R = 8, S = 4096), dedup_scan is left out: every dedup_maps work-group
// copies the whole count table to LDS and sums the columns it needs itself
// (its chunk's base, and Q at rank m's first and last chunk), and work-group
// 0 writes the two count outputs.
// R <= 64 (a token's destinations fit one 64-bit mask).
#include "mep_device.h"

namespace mep {
namespace {

constexpr int kDedupThreads = 1024;
constexpr int kDedupChunk = kDedupThreads;  // tokens per chunk
constexpr int kDedupWaves = kDedupThreads / kWave;
constexpr int kDedupMaxR = 64;
constexpr int kDedupFusedInts = 8192;  // count table held in LDS by dedup_maps

struct DedupDims {
    int R, S, K, m, cps, nchunks;
    int vec;  // K % 4 == 0 and both route maps 16-byte aligned: read them as vectors
};

struct DedupWs {
    int* cnt;        // [nchunks][R]
    int* base;       // [nchunks][R] exclusive over chunks
    int* segbase;    // [R]: rank m's send segment bases
    int* q0;         // [R]: Q[m*S][d]
};

// Calls f(k, d) for each route k of global token g with destination d. A
// token's K destinations are contiguous: with vec (K % 4 == 0, aligned maps)
// they are read as 16-byte vectors (a lane's routes in K/4 loads, not K),
// else 8 scalar loads at a time; either way the loads of a batch are in
// flight together.
template <typename F>
__device__ __forceinline__ void for_routes(const int* __restrict__ route_dest, size_t g, int K,
                                           int vec, F f) {
    if (vec) {
        const i32x4* p = (const i32x4*)(route_dest + g * K);
        for (int k0 = 0; k0 < K; k0 += 16) {
            i32x4 v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (k0 + 4 * j < K) v[j] = p[k0 / 4 + j];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (k0 + 4 * j < K)
#pragma unroll
                    for (int i = 0; i < 4; ++i) f(k0 + 4 * j + i, v[j][i]);
        }
        return;
    }
    for (int k0 = 0; k0 < K; k0 += 8) {
        int d[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) d[j] = k0 + j < K ? route_dest[g * K + k0 + j] : -1;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (k0 + j < K) f(k0 + j, d[j]);
    }
}

__device__ __forceinline__ uint64_t token_mask(const int* __restrict__ route_dest, size_t g, int K,
                                               int vec, int R) {
    uint64_t mk = 0;
    for_routes(route_dest, g, K, vec, [&](int, int d) {
        if ((unsigned)d < (unsigned)R) mk |= 1ull << d;
    });
    return mk;
}

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

__global__ __launch_bounds__(kDedupThreads) void dedup_count(DedupDims dd, DedupWs w,
                                                             const int* __restrict__ route_dest) {
    __shared__ int s_cnt[kDedupWaves][kDedupMaxR];
    const int c = blockIdx.x;
    const int src = c / dd.cps, sub = c - src * dd.cps;
    const int t = sub * kDedupChunk + threadIdx.x;
    const bool valid = t < dd.S;
    const size_t g = (size_t)src * dd.S + (valid ? t : 0);
    const uint64_t mk = valid ? token_mask(route_dest, g, dd.K, dd.vec, dd.R) : 0ull;
    const int wave = threadIdx.x / kWave;
    for (int d = 0; d < dd.R; ++d) {
        const uint64_t b = ballot64((mk >> d) & 1ull);
        if (lane_id() == 0) s_cnt[wave][d] = __popcll(b);
    }
    lds_barrier();
    for (int d = threadIdx.x; d < dd.R; d += kDedupThreads) {
        int run = 0;
        for (int v = 0; v < kDedupWaves; ++v) run += s_cnt[v][d];
        w.cnt[(size_t)c * dd.R + d] = run;
    }
}

// 16 threads per destination, destinations in groups of 64 (16 * 64 = 1024)
__global__ __launch_bounds__(kDedupThreads) void dedup_scan(DedupDims dd, DedupWs w,
                                                            int* __restrict__ dsend_count,
                                                            int* __restrict__ drecv_count) {
    __shared__ int s_q0[kDedupMaxR], s_q1[kDedupMaxR];
    const int d = threadIdx.x >> 4;  // 0..63
    const int part = threadIdx.x & 15;
    const int per = (dd.nchunks + 15) / 16;
    const int c0 = min(part * per, dd.nchunks), c1 = min(c0 + per, dd.nchunks);
    int sum = 0;
    if (d < dd.R) {
#pragma unroll 8
        for (int c = c0; c < c1; ++c) sum += w.cnt[(size_t)c * dd.R + d];
    }
    // exclusive scan of the 16 part sums of this destination (16 adjacent lanes)
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
        const int y = __shfl_up(incl, o, 16);
        if (part >= o) incl += y;
    }
    int run = incl - sum;
    if (d < dd.R) {
        for (int c = c0; c < c1; ++c) {
            w.base[(size_t)c * dd.R + d] = run;
            run += w.cnt[(size_t)c * dd.R + d];
        }
    }
    // the bases just stored (global memory) are read back below by other
    // threads of this work-group: a full barrier, which waits for the stores
    __syncthreads();
    // rank m's counts: Q at the source boundaries
    if (threadIdx.x < dd.R) {
        const int dst = threadIdx.x;
        const int cm0 = dd.m * dd.cps, cm1 = cm0 + dd.cps;
        s_q0[dst] = w.base[(size_t)cm0 * dd.R + dst];
        s_q1[dst] = cm1 < dd.nchunks ? w.base[(size_t)cm1 * dd.R + dst]
                                     : w.base[(size_t)(dd.nchunks - 1) * dd.R + dst] +
                                           w.cnt[(size_t)(dd.nchunks - 1) * dd.R + dst];
    }
    lds_barrier();
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int dst = 0; dst < dd.R; ++dst) {
            const int n = s_q1[dst] - s_q0[dst];
            w.segbase[dst] = acc;
            w.q0[dst] = s_q0[dst];
            dsend_count[dst] = n;
            acc += n;
        }
    }
    // tokens of each source reaching m
    for (int src = threadIdx.x; src < dd.R; src += kDedupThreads) {
        int n = 0;
#pragma unroll 8
        for (int c = src * dd.cps; c < (src + 1) * dd.cps; ++c) n += w.cnt[(size_t)c * dd.R + dd.m];
        drecv_count[src] = n;
    }
}

// Sum over chunks [lo, hi) of the count table's column d, held in LDS
// ([nchunks][R]), by the 16 lanes of one destination group (lane part of 16
// takes every 16th chunk); every lane of the group returns the total.
__device__ __forceinline__ int group16_sum(const int* s_all, int R, int d, int part, int lo,
                                           int hi) {
    int sum = 0;
    for (int ch = lo + part; ch < hi; ch += 16) sum += s_all[ch * R + d];
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 16);
    return sum;
}

template <bool FUSED>
__global__ __launch_bounds__(kDedupThreads) void dedup_maps(DedupDims dd, DedupWs w,
                                                            const int* __restrict__ route_dest,
                                                            const int* __restrict__ route_slot,
                                                            int* __restrict__ dpack_pos,
                                                            int* __restrict__ drecv_pos,
                                                            int* __restrict__ dsend_count,
                                                            int* __restrict__ drecv_count) {
    __shared__ int s_all[FUSED ? kDedupFusedInts : 1];  // fused: the count table [nchunks][R]
    __shared__ int s_q0[kDedupMaxR], s_q1[kDedupMaxR];
    __shared__ uint64_t s_bal[kDedupWaves][kDedupMaxR];
    __shared__ int s_wbase[kDedupWaves][kDedupMaxR];
    __shared__ int s_cbase[kDedupMaxR];
    __shared__ int s_seg[kDedupMaxR];  // segbase - q0: send row = s_seg[d] + Q
    const int c = blockIdx.x;
    const int src = c / dd.cps, sub = c - src * dd.cps;
    const int t = sub * kDedupChunk + threadIdx.x;
    const bool valid = t < dd.S;
    const size_t g = (size_t)src * dd.S + (valid ? t : 0);
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();
    if constexpr (FUSED) {
        // the count table straight into LDS (gfx950's global_load_lds: each
        // wave instruction fills 64 consecutive ints), issued first
        const int n_all = dd.nchunks * dd.R;
        for (int b = wave * kWave; b < n_all; b += kDedupThreads)
            if (b + lane < n_all) __builtin_amdgcn_global_load_lds(w.cnt + b + lane, s_all + b, 4, 0, 0);
    }
    // the token's first kRegRoutes destinations are loaded up front and
    // reused for every map
    constexpr int kRegRoutes = 16;
    int rd[kRegRoutes];
#pragma unroll
    for (int k = 0; k < kRegRoutes; ++k) rd[k] = -1;
    uint64_t mk = 0;
    if (valid)
        for_routes(route_dest, g, dd.K, dd.vec, [&](int k, int d) {
            if (k < kRegRoutes) rd[k] = d;
            if ((unsigned)d < (unsigned)dd.R) mk |= 1ull << d;
        });
    for (int d = 0; d < dd.R; ++d) {
        const uint64_t b = ballot64((mk >> d) & 1ull);
        if (lane == 0) s_bal[wave][d] = b;
    }
    if constexpr (FUSED) {
        // the table's LDS writes count on vmcnt: done in every wave before
        // the barrier
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
        // per destination (16 lanes each): Q below this chunk and at rank
        // m's first chunk and one past its last
        const int d = threadIdx.x >> 4, part = threadIdx.x & 15;
        const int cm0 = dd.m * dd.cps, cm1 = cm0 + dd.cps;
        if (d < dd.R) {
            const int below = group16_sum(s_all, dd.R, d, part, 0, c);
            const int q0 = group16_sum(s_all, dd.R, d, part, 0, cm0);
            const int q1 = q0 + group16_sum(s_all, dd.R, d, part, cm0, cm1);
            if (part == 0) {
                s_cbase[d] = below;
                s_q0[d] = q0;
                s_q1[d] = q1;
            }
        }
        lds_barrier();
        // rank m's send segments: exclusive scan of its counts over the
        // destinations (R <= 64: the first wave)
        if (threadIdx.x < kWave) {
            const int n = threadIdx.x < dd.R ? s_q1[threadIdx.x] - s_q0[threadIdx.x] : 0;
            const int seg = wave_inclusive_sum(n) - n;
            if (threadIdx.x < dd.R) {
                s_seg[threadIdx.x] = seg - s_q0[threadIdx.x];
                if (c == 0) dsend_count[threadIdx.x] = n;
            }
        }
        // the tokens of each source reaching m
        if (c == 0)
            for (int s2 = threadIdx.x; s2 < dd.R; s2 += kDedupThreads) {
                int n = 0;
                for (int ch = s2 * dd.cps; ch < (s2 + 1) * dd.cps; ++ch) n += s_all[ch * dd.R + dd.m];
                drecv_count[s2] = n;
            }
    } else if (threadIdx.x < dd.R) {
        s_cbase[threadIdx.x] = w.base[(size_t)c * dd.R + threadIdx.x];
        s_seg[threadIdx.x] = w.segbase[threadIdx.x] - w.q0[threadIdx.x];
    }
    lds_barrier();
    for (int d = threadIdx.x; d < dd.R; d += kDedupThreads) {
        int run = 0;
        for (int v = 0; v < kDedupWaves; ++v) {
            s_wbase[v][d] = run;
            run += __popcll(s_bal[v][d]);
        }
    }
    lds_barrier();
    if (!valid) return;
    const uint64_t below = (1ull << lane) - 1ull;
    auto q_of = [&](int d) {
        return s_cbase[d] + s_wbase[wave][d] + __popcll(s_bal[wave][d] & below);
    };
    const bool reaches_m = (mk >> dd.m) & 1ull;
    if (src != dd.m && !reaches_m) return;
    const int row_m = reaches_m ? q_of(dd.m) : 0;
    const int C = dd.S * dd.K;
    // the token's slots, loaded together before any map is written: loaded
    // in the route loop below, each route to m cost a round trip
    int sl_r[kRegRoutes];
#pragma unroll
    for (int k = 0; k < kRegRoutes; ++k) sl_r[k] = -1;
    if (reaches_m) {
        if (dd.vec) {
            const i32x4* p = (const i32x4*)(route_slot + g * dd.K);
#pragma unroll
            for (int j = 0; j < kRegRoutes / 4; ++j)
                if (4 * j < dd.K) {
                    const i32x4 v = p[j];
#pragma unroll
                    for (int i = 0; i < 4; ++i) sl_r[4 * j + i] = v[i];
                }
        } else {
#pragma unroll
            for (int k = 0; k < kRegRoutes; ++k)
                if (k < dd.K) sl_r[k] = route_slot[g * dd.K + k];
        }
    }
    uint64_t seen = 0;
    auto visit = [&](int k, int d, int sl) {
        if (src == dd.m) {
            int p = -1;
            if ((unsigned)d < (unsigned)dd.R && !((seen >> d) & 1ull)) {
                seen |= 1ull << d;
                p = s_seg[d] + q_of(d);
            }
            dpack_pos[(size_t)t * dd.K + k] = p;
        }
        if (d == dd.m && (unsigned)sl < (unsigned)C) drecv_pos[sl] = row_m;
    };
#pragma unroll
    for (int k = 0; k < kRegRoutes; ++k)
        if (k < dd.K) visit(k, rd[k], sl_r[k]);
    for (int k = kRegRoutes; k < dd.K; ++k) {
        const int d = route_dest[g * dd.K + k];
        visit(k, d, d == dd.m ? route_slot[g * dd.K + k] : -1);
    }
}

bool dedup_dims(int R, int S, int K, int m, DedupDims* d) {
    if (R < 1 || R > kDedupMaxR || S < 1 || K < 1 || m < 0 || m >= R) return false;
    if ((long long)R * S * K > (1ll << 30)) return false;
    d->R = R;
    d->S = S;
    d->K = K;
    d->m = m;
    d->cps = (S + kDedupChunk - 1) / kDedupChunk;
    d->nchunks = R * d->cps;
    d->vec = 0;
    return true;
}

size_t ws_bytes(const DedupDims& d, size_t* off_cnt, size_t* off_base, size_t* off_seg,
                size_t* off_q0) {
    auto up = [](size_t b) { return (b + 255) & ~size_t(255); };
    size_t at = 0;
    *off_cnt = at;
    at += up((size_t)d.nchunks * d.R * sizeof(int));
    *off_base = at;
    at += up((size_t)d.nchunks * d.R * sizeof(int));
    *off_seg = at;
    at += up((size_t)d.R * sizeof(int));
    *off_q0 = at;
    at += up((size_t)d.R * sizeof(int));
    return at;
}

}  // namespace
}  // namespace mep

using namespace mep;

extern "C" size_t mep_plan_dedup_workspace_size(int R, int S, int K) {
    DedupDims d;
    if (!dedup_dims(R, S, K, 0, &d)) return 0;
    size_t a, b, c, e;
    return ws_bytes(d, &a, &b, &c, &e);
}

extern "C" int mep_plan_dedup(int R, int S, int K, int my_rank, const int32_t* route_dest,
                              const int32_t* route_slot, void* workspace, size_t workspace_bytes,
                              int32_t* dpack_pos, int32_t* dsend_count, int32_t* drecv_pos,
                              int32_t* drecv_count, void* stream) {
    DedupDims d;
    if (my_rank < 0 || my_rank >= R) return MEP_ERR_PARAM;
    if (!dedup_dims(R, S, K, my_rank, &d)) return MEP_ERR_SHAPE;
    if (!route_dest || !route_slot || !workspace || !dpack_pos || !dsend_count || !drecv_pos ||
        !drecv_count)
        return MEP_ERR_NULLPTR;
    size_t oc, ob, os, oq;
    if (workspace_bytes < ws_bytes(d, &oc, &ob, &os, &oq)) return MEP_ERR_PARAM;
    if ((uintptr_t)workspace & 255u) return MEP_ERR_SHAPE;
    d.vec = (K % 4) == 0 && ((uintptr_t)route_dest & 15u) == 0 && ((uintptr_t)route_slot & 15u) == 0;
    char* base = (char*)workspace;
    DedupWs w{(int*)(base + oc), (int*)(base + ob), (int*)(base + os), (int*)(base + oq)};
    hipStream_t s = (hipStream_t)stream;
    const int* rd = (const int*)route_dest;
    hipLaunchKernelGGL(dedup_count, dim3(d.nchunks), dim3(kDedupThreads), 0, s, d, w, rd);
    MEP_LAUNCH_CHECK();
    if ((long long)d.nchunks * d.R <= kDedupFusedInts) {
        hipLaunchKernelGGL(dedup_maps<true>, dim3(d.nchunks), dim3(kDedupThreads), 0, s, d, w, rd,
                           (const int*)route_slot, (int*)dpack_pos, (int*)drecv_pos,
                           (int*)dsend_count, (int*)drecv_count);
    } else {
        hipLaunchKernelGGL(dedup_scan, dim3(1), dim3(kDedupThreads), 0, s, d, w,
                           (int*)dsend_count, (int*)drecv_count);
        MEP_LAUNCH_CHECK();
        hipLaunchKernelGGL(dedup_maps<false>, dim3(d.nchunks), dim3(kDedupThreads), 0, s, d, w, rd,
                           (const int*)route_slot, (int*)dpack_pos, (int*)drecv_pos, nullptr,
                           nullptr);
    }
    MEP_LAUNCH_CHECK();
    return MEP_OK;
}
