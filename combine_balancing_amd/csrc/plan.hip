// mep_plan: the global balanced plan and one rank's send/receive maps.
//
// Method ("MoonEP" technical overview, architecture section): every EP rank
// processes exactly C = S*K routed rows; hot experts get temporary redundant
// instances on other ranks, planned on the GPU from the router output each
// step. The rule computed here: expert e lives natively on rank
// floor(e*R/E); in (expert, global token, k) order each rank keeps its first
// C routes; the rest spill, in the same order, to the under-loaded ranks in
// ascending rank order, filling each to exactly C.
//
// GPU design (four launches, all deterministic, no host sync):
//   plan_hist    one block per chunk of T routes (chunks never straddle a
//                source rank): per-chunk expert histogram in LDS.
//   plan_scan    one block per expert: exclusive scan of its column over the
//                chunks, so chunk c knows how many routes of expert e precede
//                it in (expert, f) order.
//   plan_global  one block: expert offsets, native loads, surplus/deficit
//                scans, the redundant instances (the pieces that the ordered
//                excess list forms against the ordered deficit list, found by
//                a merge-path style co-rank with binary searches), instance
//                tables, and per-instance bases for this rank's send and
//                receive maps.
//   plan_routes  one block per chunk: stable within-chunk rank of each route
//                among equal experts (per-wave ballot multi-split plus
//                cross-wave offsets), then the closed-form destination and
//                slot and the send/receive positions.
// Closed forms used by plan_routes. With p the route's position in
// (expert, f) order, r its home rank and rb[r] the first position of rank r:
//   q = p - rb[r];  q < C  -> (r, q)
//   else j = Uex[r] + q - C is the route's index in the global excess list;
//   the piece holding j gives the host u and slot L[u] + j - Dex[u].
// Within one instance, the routes of one source rank are contiguous and in
// position order, so a route's send (receive) row is a per-instance base
// plus its rank among the same source's routes of that expert.
#include <algorithm>

#include "mep_device.h"

namespace mep {
namespace {

constexpr int kHistThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int kScanItems = 4;
constexpr int kMaxChunks = kScanThreads * kScanItems;
constexpr int kGlobalThreads = 1024;
constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kMaxR = 1024;
constexpr int kMaxE = 1024;

enum { SC_NP = 0, SC_EFIRST_M = 1, SC_NAT_M = 2, SC_FP_M = 3, SC_COUNT = 16 };

struct PlanDims {
    int R, E, S, K, m;
    int C;        // S*K: rows per rank
    int N;        // R*C: routes
    int T;        // routes per chunk
    int cps;      // chunks per source rank
    int nchunks;  // R*cps
    int nbits;    // bits needed for E-1
};

struct PlanWs {
    int* chunk;     // [nchunks][E] counts, then exclusive prefix over chunks
    int* cnt;       // [E]
    int* eex;       // [E+1] exclusive prefix of cnt
    int* rb;        // [R+1] first position of each rank's block
    int* load;      // [R]   native loads
    int* uex;       // [R+1] exclusive prefix of surplus
    int* dex;       // [R+1] exclusive prefix of deficit
    int* kept;      // [E]   routes of e kept on its home rank
    int* js;        // [E]   excess-list index of e's first spilled route
    int* pstart;    // [E+R+1] excess index where each piece starts (sorted)
    int* phost;     // [E+R]
    int* pexpert;   // [E+R]
    int* ppos;      // [E+R] position of the piece's first route
    int* pn;        // [E+R] rows in the piece
    int* psend;     // [E+R] send base of each piece (this rank)
    int* nsend;     // [E]   send base of each native instance (this rank)
    int* sendscan;  // [2E+R+1]
    int* recvbase;  // [E][R] receive base per (local instance, source)
    int* scal;      // [SC_COUNT]
};

struct PlanOut {
    int32_t *expert_count, *rank_load, *route_dest, *route_slot;
    int32_t *inst_count, *inst_expert, *inst_cu, *inst_gid_base;
    int32_t *send_pos, *send_count, *recv_pos, *recv_count;
};

__device__ __forceinline__ int home_of(int e, int R, int E) {
    return (int)(((unsigned)e * (unsigned)R) / (unsigned)E);  // e*R < 2^20
}

__device__ __forceinline__ int efirst_of(int r, int R, int E) {
    return (int)(((unsigned)r * (unsigned)E + (unsigned)R - 1u) / (unsigned)R);
}

// ---------------------------------------------------------------- plan_hist
__global__ __launch_bounds__(kHistThreads) void plan_hist(PlanDims d, const int* __restrict__ ids,
                                                          int* __restrict__ chunk) {
    extern __shared__ int s_hist[];
    const int c = blockIdx.x;
    const int src = c / d.cps, sub = c - src * d.cps;
    const int f0 = src * d.C + sub * d.T;
    const int f1 = min(f0 + d.T, (src + 1) * d.C);
    for (int e = threadIdx.x; e < d.E; e += blockDim.x) s_hist[e] = 0;
    __syncthreads();
    for (int f = f0 + threadIdx.x; f < f1; f += blockDim.x) {
        const int e = ids[f];
        if ((unsigned)e < (unsigned)d.E) atomicAdd(&s_hist[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < d.E; e += blockDim.x) chunk[c * d.E + e] = s_hist[e];
}

// ---------------------------------------------------------------- plan_scan
__global__ __launch_bounds__(kScanThreads) void plan_scan(PlanDims d, int* __restrict__ chunk,
                                                          int* __restrict__ cnt) {
    __shared__ int scratch[kScanThreads / kWave + 1];
    const int e = blockIdx.x;
    const int c0 = threadIdx.x * kScanItems;
    int v[kScanItems];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        const int c = c0 + i;
        v[i] = c < d.nchunks ? chunk[c * d.E + e] : 0;
        sum += v[i];
    }
    int total;
    int ex = block_exclusive_sum(sum, scratch, &total);
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        const int c = c0 + i;
        if (c < d.nchunks) chunk[c * d.E + e] = ex;
        ex += v[i];
    }
    if (threadIdx.x == 0) cnt[e] = total;
}

// -------------------------------------------------------------- plan_global
// Routes of source rank `src` of expert e that precede the source's first
// chunk (src == R gives the expert's total).
__device__ __forceinline__ int pre_of(const PlanDims& d, const int* chunk, const int* s_cnt, int src,
                                      int e) {
    return src >= d.R ? s_cnt[e] : chunk[(src * d.cps) * d.E + e];
}

__global__ __launch_bounds__(kGlobalThreads) void plan_global(PlanDims d, PlanWs w, PlanOut o) {
    extern __shared__ int lds[];
    const int E = d.E, R = d.R, C = d.C;
    const int tid = threadIdx.x, NT = blockDim.x;
    int* s_eex = lds;               // E+1
    int* s_cnt = s_eex + E + 1;     // E
    int* s_cjs = s_cnt + E;         // E  excess starts of spilling experts
    int* s_cje = s_cjs + E;         // E  their experts
    int* s_rb = s_cje + E;          // R+1
    int* s_L = s_rb + R + 1;        // R
    int* s_uex = s_L + R;           // R+1
    int* s_dex = s_uex + R + 1;     // R+1
    int* s_cdl = s_dex + R + 1;     // R  deficit starts of under-loaded ranks
    int* s_cdu = s_cdl + R;         // R  their ranks
    int* s_coin = s_cdu + R;        // R+1 prefix count of shared starts
    int* s_fp = s_coin + R + 1;     // R+1 first piece of each under-loaded rank
    int* s_np = s_fp + R + 1;       // R  pieces per rank
    int* s_gid = s_np + R;          // R+1 instance gid base per rank
    int* scratch = s_gid + R + 1;   // NT/64+1

    // 1. expert offsets in (expert, f) order
    int c = tid < E ? w.cnt[tid] : 0;
    int total;
    int ex = block_exclusive_sum(c, scratch, &total);
    if (tid < E) {
        s_cnt[tid] = c;
        s_eex[tid] = ex;
        w.eex[tid] = ex;
        o.expert_count[tid] = c;
    }
    if (tid == 0) {
        s_eex[E] = total;
        w.eex[E] = total;
    }
    __syncthreads();

    // 2. rank blocks, native loads, surplus and deficit prefixes
    for (int r = tid; r <= R; r += NT) {  // R may equal the block size
        const int rb = s_eex[efirst_of(r, R, E)];
        s_rb[r] = rb;
        w.rb[r] = rb;
    }
    __syncthreads();
    int L = 0, U = 0, D = 0;
    if (tid < R) {
        L = s_rb[tid + 1] - s_rb[tid];
        U = max(L - C, 0);
        D = max(C - L, 0);
        s_L[tid] = L;
        w.load[tid] = L;
        o.rank_load[tid] = L;
    }
    int totU, totD;
    const int uex = block_exclusive_sum(U, scratch, &totU);
    const int dex = block_exclusive_sum(D, scratch, &totD);
    if (tid < R) {
        s_uex[tid] = uex;
        s_dex[tid] = dex;
        w.uex[tid] = uex;
        w.dex[tid] = dex;
    }
    if (tid == 0) {
        s_uex[R] = totU;
        s_dex[R] = totD;
        w.uex[R] = totU;
        w.dex[R] = totD;
    }
    __syncthreads();

    // 3. per expert: rows kept at home and the start of its excess
    int spill = 0, kept = 0, js = 0;
    if (tid < E) {
        const int h = home_of(tid, R, E);
        const int rb = s_rb[h];
        kept = clampi(rb + C - s_eex[tid], 0, s_cnt[tid]);
        js = s_uex[h] + max(0, s_eex[tid] + kept - rb - C);
        spill = kept < s_cnt[tid];
        w.kept[tid] = kept;
        w.js[tid] = js;
    }
    int NS;
    const int si = block_exclusive_sum(spill, scratch, &NS);
    if (spill) {
        s_cjs[si] = js;
        s_cje[si] = tid;
    }
    const int under = tid < R && s_L[tid] < C;
    int NU;
    const int ui = block_exclusive_sum(under, scratch, &NU);
    if (under) {
        s_cdl[ui] = s_dex[tid];
        s_cdu[ui] = tid;
    }
    __syncthreads();
    int coin = 0;
    if (tid < NU) {
        const int s = s_cdl[tid];
        const int lb = lower_bound(s_cjs, NS, s);
        coin = lb < NS && s_cjs[lb] == s;
    }
    int NC;
    const int ci = block_exclusive_sum(coin, scratch, &NC);
    if (tid < NU) s_coin[tid] = ci;
    if (tid == 0) s_coin[NU] = NC;
    __syncthreads();
    const int NP = NS + NU - NC;

    // 4. pieces (redundant instances): the excess list [0, totU) cut at every
    //    expert boundary and every under-loaded rank boundary, in order.
    if (tid < NS) {
        const int s = s_cjs[tid];
        const int e = s_cje[tid];
        const int lb = lower_bound(s_cdl, NU, s);
        const int pi = tid + lb - s_coin[lb];
        const int k = upper_bound(s_cdl, NU, s) - 1;
        const int u = s_cdu[k];
        const int kp = w.kept[e];
        const int end = min(s + s_cnt[e] - kp, s_dex[u] + (C - s_L[u]));
        w.pstart[pi] = s;
        w.phost[pi] = u;
        w.pexpert[pi] = e;
        w.pn[pi] = end - s;
        w.ppos[pi] = s_eex[e] + kp;
    }
    if (tid < NU && !coin) {
        const int s = s_cdl[tid];
        const int u = s_cdu[tid];
        const int lb = lower_bound(s_cjs, NS, s);
        const int pi = tid + lb - s_coin[tid];
        const int e = s_cje[lb - 1];
        const int jse = w.js[e];
        const int kp = w.kept[e];
        const int end = min(jse + s_cnt[e] - kp, s + (C - s_L[u]));
        w.pstart[pi] = s;
        w.phost[pi] = u;
        w.pexpert[pi] = e;
        w.pn[pi] = end - s;
        w.ppos[pi] = s_eex[e] + kp + (s - jse);
    }
    if (tid < NU) {
        const int s = s_cdl[tid];
        s_fp[s_cdu[tid]] = tid + lower_bound(s_cjs, NS, s) - s_coin[tid];
    }
    if (tid < R) s_np[tid] = 0;
    if (tid == 0) w.pstart[NP] = totU;
    __syncthreads();
    if (tid < NU) {
        const int u = s_cdu[tid];
        const int nxt = tid + 1 < NU ? s_fp[s_cdu[tid + 1]] : NP;
        s_np[u] = nxt - s_fp[u];
    }
    __syncthreads();

    // 5. instance counts and gid bases
    int ic = 0;
    if (tid < R) {
        ic = efirst_of(tid + 1, R, E) - efirst_of(tid, R, E) + s_np[tid];
        o.inst_count[tid] = ic;
    }
    int NI;
    const int gb = block_exclusive_sum(ic, scratch, &NI);
    if (tid < R) {
        s_gid[tid] = gb;
        o.inst_gid_base[tid] = gb;
    }
    if (tid == 0) {
        s_gid[R] = NI;
        o.inst_gid_base[R] = NI;
    }
    __syncthreads();

    // 6. instance tables
    const int E1 = E + 1;
    for (int idx = tid; idx < R * E1; idx += NT) {
        const int u = idx / E1;
        const int i = idx - u * E1;
        const int ef = efirst_of(u, R, E);
        const int nat = efirst_of(u + 1, R, E) - ef;
        const int n = nat + s_np[u];
        int cu;
        if (i < nat) {
            cu = min(s_eex[ef + i] - s_rb[u], C);
        } else if (i < n) {
            cu = s_L[u] + w.pstart[s_fp[u] + i - nat] - s_dex[u];
        } else {
            cu = C;
        }
        o.inst_cu[idx] = cu;
        if (i < E) {
            const int ie = i < nat ? ef + i : (i < n ? w.pexpert[s_fp[u] + i - nat] : -1);
            o.inst_expert[u * E + i] = ie;
        }
    }

    // 7. send bases of this rank: instances in gid order = (dest, slot) order
    const int m = d.m;
    int carry = 0;
    for (int base = 0; base < NI; base += NT) {
        const int gid = base + tid;
        int cm = 0, qP = 0, e = 0, pi = -1;
        if (gid < NI) {
            const int u = upper_bound(s_gid, R + 1, gid) - 1;
            const int i = gid - s_gid[u];
            const int ef = efirst_of(u, R, E);
            const int nat = efirst_of(u + 1, R, E) - ef;
            int P, n;
            if (i < nat) {
                e = ef + i;
                P = s_eex[e];
                n = w.kept[e];
            } else {
                pi = s_fp[u] + i - nat;
                e = w.pexpert[pi];
                P = w.ppos[pi];
                n = w.pn[pi];
            }
            const int pre = pre_of(d, w.chunk, s_cnt, m, e);
            const int Hm = pre_of(d, w.chunk, s_cnt, m + 1, e) - pre;
            qP = clampi(P - s_eex[e] - pre, 0, Hm);
            cm = clampi(P + n - s_eex[e] - pre, 0, Hm) - qP;
        }
        int tot;
        const int sx = block_exclusive_sum(cm, scratch, &tot) + carry;
        if (gid < NI) {
            w.sendscan[gid] = sx;
            if (pi < 0) w.nsend[e] = sx - qP;
            else w.psend[pi] = sx - qP;
        }
        carry += tot;
    }
    if (tid == 0) w.sendscan[NI] = carry;
    __syncthreads();
    for (int dd = tid; dd < R; dd += NT) o.send_count[dd] = w.sendscan[s_gid[dd + 1]] - w.sendscan[s_gid[dd]];

    // 8. receive bases of this rank: per (local instance i, source), the
    //    source's rows in earlier instances minus the instance's start rank
    const int ef_m = efirst_of(m, R, E);
    const int nat_m = efirst_of(m + 1, R, E) - ef_m;
    const int nim = nat_m + s_np[m];
    const int fp_m = s_fp[m];
    int acc = 0;
    const int src = tid;
    if (src < R) {
        for (int i = 0; i < nim; ++i) {
            int e, P, n;
            if (i < nat_m) {
                e = ef_m + i;
                P = s_eex[e];
                n = w.kept[e];
            } else {
                const int pi = fp_m + i - nat_m;
                e = w.pexpert[pi];
                P = w.ppos[pi];
                n = w.pn[pi];
            }
            const int pre = pre_of(d, w.chunk, s_cnt, src, e);
            const int Hs = pre_of(d, w.chunk, s_cnt, src + 1, e) - pre;
            const int q0 = clampi(P - s_eex[e] - pre, 0, Hs);
            const int q1 = clampi(P + n - s_eex[e] - pre, 0, Hs);
            w.recvbase[i * R + src] = acc - q0;
            acc += q1 - q0;
        }
        o.recv_count[src] = acc;
    }
    int totr;
    const int roff = block_exclusive_sum(src < R ? acc : 0, scratch, &totr);
    if (src < R) {
        for (int i = 0; i < nim; ++i) w.recvbase[i * R + src] += roff;
    }
    if (tid == 0) {
        w.scal[SC_NP] = NP;
        w.scal[SC_EFIRST_M] = ef_m;
        w.scal[SC_NAT_M] = nat_m;
        w.scal[SC_FP_M] = fp_m;
    }
}

// -------------------------------------------------------------- plan_routes
__global__ __launch_bounds__(kRouteThreads) void plan_routes(PlanDims d, PlanWs w,
                                                             const int* __restrict__ ids,
                                                             PlanOut o) {
    extern __shared__ int lds[];
    const int E = d.E, R = d.R, C = d.C;
    const int tid = threadIdx.x;
    int* s_cnt = lds;                      // [waves][E]
    int* s_off = s_cnt + kRouteWaves * E;  // [E]
    int* s_pre = s_off + E;                // [E]
    int* s_eex = s_pre + E;                // [E]
    int* s_rb = s_eex + E;                 // [R+1]
    int* s_uex = s_rb + R + 1;             // [R]
    int* s_L = s_uex + R;                  // [R]
    int* s_dex = s_L + R;                  // [R]
    int* s_ps = s_dex + R;                 // [NP+1]

    const int c = blockIdx.x;
    const int src = c / d.cps, sub = c - src * d.cps;
    const int f0 = src * C + sub * d.T;
    const int f1 = min(f0 + d.T, (src + 1) * C);
    const int NP = w.scal[SC_NP];

    for (int e = tid; e < E; e += kRouteThreads) {
        s_off[e] = w.chunk[c * E + e];
        s_pre[e] = w.chunk[(src * d.cps) * E + e];
        s_eex[e] = w.eex[e];
    }
    for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) s_cnt[i] = 0;
    for (int r = tid; r <= R; r += kRouteThreads) s_rb[r] = w.rb[r];
    for (int r = tid; r < R; r += kRouteThreads) {
        s_uex[r] = w.uex[r];
        s_L[r] = w.load[r];
        s_dex[r] = w.dex[r];
    }
    for (int i = tid; i <= NP; i += kRouteThreads) s_ps[i] = w.pstart[i];
    __syncthreads();

    const int wave = tid / kWave;
    const int lane = tid & (kWave - 1);
    const int len = f1 - f0;
    const int seg = (((len + kRouteWaves - 1) / kRouteWaves) + kWave - 1) & ~(kWave - 1);
    const int a = min(f0 + wave * seg, f1);
    const int b = min(a + seg, f1);
    int* my_cnt = s_cnt + wave * E;

    // pass 1: per-wave expert counts
    for (int f = a + lane; f < b; f += kWave) {
        const int e = ids[f];
        if ((unsigned)e < (unsigned)E) atomicAdd(&my_cnt[e], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += kRouteThreads) {
        int run = 0;
        for (int v = 0; v < kRouteWaves; ++v) {
            const int t = s_cnt[v * E + e];
            s_cnt[v * E + e] = run;
            run += t;
        }
    }
    __syncthreads();

    // pass 2: stable rank within the chunk, then placement
    const int m = d.m;
    const int ef_m = w.scal[SC_EFIRST_M];
    const int nat_m = w.scal[SC_NAT_M];
    const int fp_m = w.scal[SC_FP_M];
    for (int base = a; base < b; base += kWave) {
        const int f = base + lane;
        bool valid = f < b;
        int e = valid ? ids[f] : 0;
        valid = valid && (unsigned)e < (unsigned)E;
        if (!valid) e = 0;
        const uint64_t peers = match_peers(e, valid, d.nbits);
        const int rin = my_cnt[e] + count_below(peers);
        if (valid && is_group_leader(peers)) my_cnt[e] += __popcll(peers);
        if (!valid) {
            if (f < b && o.route_dest) {
                o.route_dest[f] = -1;
                o.route_slot[f] = -1;
            }
            continue;
        }
        const int qs = s_off[e] - s_pre[e] + rin;  // rank among src's routes of e
        const int p = s_eex[e] + s_off[e] + rin;   // position in (expert, f) order
        const int h = home_of(e, R, E);
        const int q = p - s_rb[h];
        int dest, slot, pi = -1;
        if (q < C) {
            dest = h;
            slot = q;
        } else {
            const int j = s_uex[h] + q - C;
            pi = upper_bound(s_ps, NP, j) - 1;
            dest = pi >= 0 ? w.phost[pi] : -1;
            if ((unsigned)dest >= (unsigned)R) {  // only for inconsistent inputs
                if (o.route_dest) {
                    o.route_dest[f] = -1;
                    o.route_slot[f] = -1;
                }
                continue;
            }
            slot = s_L[dest] + j - s_dex[dest];
        }
        if (o.route_dest) {
            o.route_dest[f] = dest;
            o.route_slot[f] = slot;
        }
        if (src == m) o.send_pos[f - m * C] = (pi < 0 ? w.nsend[e] : w.psend[pi]) + qs;
        if (dest == m && (unsigned)slot < (unsigned)C) {
            const int i = pi < 0 ? e - ef_m : nat_m + pi - fp_m;
            o.recv_pos[slot] = w.recvbase[i * R + src] + qs;
        }
    }
}

// ------------------------------------------------------------------- host
bool plan_dims(int R, int E, int S, int K, int m, PlanDims* d) {
    if (R < 1 || R > kMaxR || E < 1 || E > kMaxE || S < 1 || K < 1) return false;
    const long long C = (long long)S * K;
    const long long N = C * R;
    if (N > (1ll << 30)) return false;
    d->R = R;
    d->E = E;
    d->S = S;
    d->K = K;
    d->m = m;
    d->C = (int)C;
    d->N = (int)N;
    long long T = 1024;
    while ((long long)R * ((C + T - 1) / T) > kMaxChunks) T *= 2;
    d->T = (int)std::min<long long>(T, C);
    d->cps = (int)((C + d->T - 1) / d->T);
    d->nchunks = R * d->cps;
    int nb = 0;
    while ((1 << nb) < E) ++nb;
    d->nbits = nb;
    return true;
}

struct WsOffsets {
    size_t chunk, cnt, eex, rb, load, uex, dex, kept, js, pstart, phost, pexpert, ppos, pn, psend,
        nsend, sendscan, recvbase, scal, total;
};

WsOffsets ws_offsets(const PlanDims& d) {
    WsOffsets o{};
    size_t at = 0;
    auto take = [&](size_t ints) {
        const size_t here = at;
        at += (ints * sizeof(int) + 255) & ~size_t(255);
        return here;
    };
    const size_t E = d.E, R = d.R;
    o.chunk = take((size_t)d.nchunks * E);
    o.cnt = take(E);
    o.eex = take(E + 1);
    o.rb = take(R + 1);
    o.load = take(R);
    o.uex = take(R + 1);
    o.dex = take(R + 1);
    o.kept = take(E);
    o.js = take(E);
    o.pstart = take(E + R + 1);
    o.phost = take(E + R);
    o.pexpert = take(E + R);
    o.ppos = take(E + R);
    o.pn = take(E + R);
    o.psend = take(E + R);
    o.nsend = take(E);
    o.sendscan = take(2 * E + R + 1);
    o.recvbase = take(E * R);
    o.scal = take(SC_COUNT);
    o.total = at;
    return o;
}

size_t global_lds_bytes(const PlanDims& d) {
    const size_t ints = (size_t)4 * d.E + 1 + (size_t)10 * d.R + 6 + kGlobalThreads / kWave + 1;
    return ints * sizeof(int);
}

size_t routes_lds_bytes(const PlanDims& d) {
    const size_t ints = (size_t)(kRouteWaves + 3) * d.E + (size_t)4 * d.R + 1 + (size_t)d.E + d.R + 1;
    return ints * sizeof(int);
}

bool lds_ready() {
    // Allow the two single-pass kernels to use more than 64 KiB of LDS when
    // the sizes call for it (gfx950 has 160 KiB per CU).
    static const bool ok = [] {
        const int lim = 160 * 1024;
        bool good = hipFuncSetAttribute((const void*)plan_global,
                                        hipFuncAttributeMaxDynamicSharedMemorySize,
                                        lim) == hipSuccess;
        good = hipFuncSetAttribute((const void*)plan_routes,
                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                   lim) == hipSuccess && good;
        (void)hipGetLastError();
        return good;
    }();
    return ok;
}

}  // namespace
}  // namespace mep

using namespace mep;

extern "C" size_t mep_plan_workspace_size(int R, int E, int S, int K) {
    PlanDims d;
    if (!plan_dims(R, E, S, K, 0, &d) || K > E) return 0;
    return ws_offsets(d).total;
}

extern "C" int mep_plan(int R, int E, int S, int K, int my_rank, const int32_t* topk_ids,
                        void* workspace, size_t workspace_bytes, int32_t* expert_count,
                        int32_t* rank_load, int32_t* route_dest, int32_t* route_slot,
                        int32_t* inst_count, int32_t* inst_expert, int32_t* inst_cu,
                        int32_t* inst_gid_base, int32_t* send_pos, int32_t* send_count,
                        int32_t* recv_pos, int32_t* recv_count, void* stream) {
    if (!topk_ids || !workspace || !expert_count || !rank_load || !inst_count || !inst_expert ||
        !inst_cu || !inst_gid_base || !send_pos || !send_count || !recv_pos || !recv_count)
        return MEP_ERR_NULLPTR;
    PlanDims d;
    if (!plan_dims(R, E, S, K, my_rank, &d)) return MEP_ERR_SHAPE;
    if (K > E || my_rank < 0 || my_rank >= R) return MEP_ERR_PARAM;
    if ((route_dest == nullptr) != (route_slot == nullptr)) return MEP_ERR_PARAM;
    const WsOffsets off = ws_offsets(d);
    if (workspace_bytes < off.total || ((uintptr_t)workspace & 255u) != 0) return MEP_ERR_PARAM;
    const size_t glds = global_lds_bytes(d), rlds = routes_lds_bytes(d);
    if ((glds > 64 * 1024 || rlds > 64 * 1024) && !lds_ready()) return MEP_ERR_HIP;

    char* ws = (char*)workspace;
    PlanWs w;
    w.chunk = (int*)(ws + off.chunk);
    w.cnt = (int*)(ws + off.cnt);
    w.eex = (int*)(ws + off.eex);
    w.rb = (int*)(ws + off.rb);
    w.load = (int*)(ws + off.load);
    w.uex = (int*)(ws + off.uex);
    w.dex = (int*)(ws + off.dex);
    w.kept = (int*)(ws + off.kept);
    w.js = (int*)(ws + off.js);
    w.pstart = (int*)(ws + off.pstart);
    w.phost = (int*)(ws + off.phost);
    w.pexpert = (int*)(ws + off.pexpert);
    w.ppos = (int*)(ws + off.ppos);
    w.pn = (int*)(ws + off.pn);
    w.psend = (int*)(ws + off.psend);
    w.nsend = (int*)(ws + off.nsend);
    w.sendscan = (int*)(ws + off.sendscan);
    w.recvbase = (int*)(ws + off.recvbase);
    w.scal = (int*)(ws + off.scal);
    PlanOut o{expert_count, rank_load, route_dest, route_slot, inst_count, inst_expert,
              inst_cu, inst_gid_base, send_pos, send_count, recv_pos, recv_count};
    hipStream_t s = (hipStream_t)stream;

    hipLaunchKernelGGL(plan_hist, dim3(d.nchunks), dim3(kHistThreads), d.E * sizeof(int), s, d,
                       (const int*)topk_ids, w.chunk);
    MEP_LAUNCH_CHECK();
    hipLaunchKernelGGL(plan_scan, dim3(d.E), dim3(kScanThreads), 0, s, d, w.chunk, w.cnt);
    MEP_LAUNCH_CHECK();
    hipLaunchKernelGGL(plan_global, dim3(1), dim3(kGlobalThreads), glds, s, d, w, o);
    MEP_LAUNCH_CHECK();
    hipLaunchKernelGGL(plan_routes, dim3(d.nchunks), dim3(kRouteThreads), rlds, s, d, w,
                       (const int*)topk_ids, o);
    MEP_LAUNCH_CHECK();
    return MEP_OK;
}
