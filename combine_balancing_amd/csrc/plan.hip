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
// GPU design (three launches, all deterministic, no host sync):
//   plan_hist    one block per chunk of T routes (chunks never straddle a
//                source rank): per-chunk expert histogram in LDS.
//   plan_scan    one block per 8 experts: exclusive scan of each expert's
//                column over the chunks, so chunk c knows how many routes of
//                expert e precede it in (expert, f) order.
//   plan_fused   one block per chunk. First the global phases, in the
//                block's own LDS: expert offsets, native loads,
//                surplus/deficit scans, the redundant instances (the pieces
//                that the ordered excess list forms against the ordered
//                deficit list, found by a merge-path style co-rank with
//                binary searches), instance tables, and per-instance bases
//                for this rank's send and receive maps. Then the chunk's
//                routes: stable within-chunk rank of each route among equal
//                experts (per-wave ballot multi-split plus cross-wave
//                offsets), the closed-form destination and slot and the
//                send/receive positions.
// Where the fused block's LDS does not fit, the two halves run as separate
// launches: plan_global (one block, tables to the workspace) and
// plan_routes (one block per chunk).
// Closed forms used by the route passes. With p the route's position in
// (expert, f) order, r its home rank and rb[r] the first position of rank r:
//   q = p - rb[r];  q < C  -> (r, q)
//   else j = Uex[r] + q - C is the route's index in the global excess list;
//   the piece holding j gives the host u and slot L[u] + j - Dex[u].
// Within one instance, the routes of one source rank are contiguous and in
// position order, so a route's send (receive) row is a per-instance base
// plus its rank among the same source's routes of that expert.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "mep_device.h"

namespace mep {
namespace {

constexpr int kHistThreads = 256;
constexpr int kMaxChunks = 1024;  // column length of the expert scan (>= the rank limit)
// Chunks grow until there are at most 256 while they stay short enough to
// stage their ids (2048 routes), then until there are at most 512 (or one
// per source rank when R is larger). Measured on the fused plan: a
// 524288-route plan (R=8, E=384) took 24.4 us with 256 chunks of 2048
// routes against 25.3 us with 512 of 1024; a 4M-route plan 43.4 us with
// 512 chunks of 8192 routes against 49.7 us with 256 of 16384 (and, in the
// four-launch form, 45.2 against 48.0 us with 1024 of 4096).
constexpr int kTargetChunks = 256;
constexpr int kTargetChunksLong = 512;
constexpr int kBuckets = 1024;  // piece lookup: excess index >> shift -> first piece
constexpr size_t kMaxLds = 160 * 1024;  // LDS a gfx950 work-group may allocate
constexpr int kGlobalThreads = 1024;
constexpr int kItemCache = 4;  // plan_global: per-thread items kept between two passes
constexpr int kRouteThreads = 1024;  // work-group of plan_routes
constexpr int kMinChunk = 1024;      // routes per chunk (at least)
constexpr int kRouteWaves = kRouteThreads / kWave;
// plan_fused work-group: 1024 threads, or 512 when there are more chunks
// than CUs and the chunks are short (see fused_threads)
constexpr int kFusedThreadsSmall = 512;
constexpr int kMaxR = 1024;
static_assert(kMaxChunks >= kMaxR, "a source rank holds at least one chunk");
static_assert(kTargetChunksLong <= kMaxChunks, "chunk target within the scan's capacity");
constexpr int kMaxE = 1024;
constexpr int kStageIds = 2048;  // chunk sizes up to this keep their ids in LDS (plan_routes)

enum { SC_NP = 0, SC_EFIRST_M = 1, SC_NAT_M = 2, SC_FP_M = 3, SC_NIM = 4, SC_SHIFT = 5, SC_COUNT = 16 };

struct PlanDims {
    int R, E, S, K, m;
    int C;        // S*K: rows per rank
    int N;        // R*C: routes
    int T;        // routes per chunk
    int cps;      // chunks per source rank
    int nchunks;  // R*cps
};

struct PlanWs {
    int* chunk;     // [nchunks][E] counts, then exclusive prefix over chunks
    int* cnt;       // [E]
    int* eex;       // [E+1] exclusive prefix of cnt
    int* rb;        // [R+1] first position of each rank's block
    int* load;      // [R]   native loads
    int* uex;       // [R+1] exclusive prefix of surplus
    int* dex;       // [R+1] exclusive prefix of deficit
    int* pstart;    // [E+R+1] excess index where each piece starts (sorted)
    int4* prec;     // [E+R+1] per piece: host rank, slot of excess index 0 on
                    //         the host, send base (this rank), expert
    int* bucket;    // [kBuckets] piece holding excess index b << shift
    int* nsend;     // [E]     send base of each native instance (this rank)
    int* recvbase;  // [R][E]  receive base per (source, local instance)
    int4* rinfo;    // [R]     per rank: first native expert, natives, pieces, first piece
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
// The kernel's arguments are requested as one batch of scalar loads, and the
// first batch of ids is loaded before the histogram is cleared: the compiler
// had issued the arguments' loads next to their first uses (three cold
// scalar round trips before the first id load, the block size among them),
// and the ids only after the clearing barrier.
__global__ __launch_bounds__(kHistThreads) void plan_hist(PlanDims d, const int* __restrict__ ids,
                                                          int* __restrict__ chunk) {
    asm volatile("" ::"s"(ids), "s"(chunk), "s"(d.E), "s"(d.C), "s"(d.T), "s"(d.cps));
    extern __shared__ int s_hist[];
    constexpr int U = 8;  // ids in flight per thread
    const int c = blockIdx.x;
    const int src = c / d.cps, sub = c - src * d.cps;
    const int f0 = src * d.C + sub * d.T;
    const int f1 = min(f0 + d.T, (src + 1) * d.C);
    int e[U];
    auto load = [&](int base) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int f = base + u * kHistThreads + (int)threadIdx.x;
            e[u] = f < f1 ? ids[f] : -1;
        }
    };
    auto count = [&]() {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if ((unsigned)e[u] < (unsigned)d.E) atomicAdd(&s_hist[e[u]], 1);
    };
    load(f0);
    for (int i = threadIdx.x; i < d.E; i += kHistThreads) s_hist[i] = 0;
    lds_barrier();
    count();
    for (int base = f0 + kHistThreads * U; base < f1; base += kHistThreads * U) {
        load(base);
        count();
    }
    lds_barrier();
    for (int i = threadIdx.x; i < d.E; i += kHistThreads) chunk[c * d.E + i] = s_hist[i];
}

// ---------------------------------------------------------------- plan_scan
// Exclusive scan of every expert's column of chunk counts. A work-group
// takes 8 experts (a 32-byte segment of each chunk row) and cuts the column
// into 128 ranges of at most kScanItems chunks: lane l of wave w holds
// expert l % 8 over range 8w + l / 8. Each load instruction of a wave then
// touches eight 32-byte segments, where one wave per expert with
// lane-strided chunks touched 64 lines per load. Range sums are scanned
// across the wave's ranges with shuffles and across the 16 waves through
// LDS. Measured on MI355X (warm): 8 experts per group beat 4, 16 and 32,
// and the whole plan went from 63 to 56 us on a 1024-chunk plan.
// PER (1, 2, 4 or 8) is the range length rounded up to a power of two. The
// loads are unconditional, at indices clamped into the table, and masked
// where they are used: loads under lane conditions made the compiler wait
// for the earlier ones before each of the later ones.
constexpr int kScanExperts = 8;
constexpr int kScanSubs = kWave / kScanExperts;                   // ranges per wave
constexpr int kScanThreads = 1024;
constexpr int kScanRanges = (kScanThreads / kWave) * kScanSubs;  // 128
constexpr int kScanItems = kMaxChunks / kScanRanges;             // 8
static_assert(kScanItems * kScanRanges == kMaxChunks, "chunk ranges must cover kMaxChunks");

template <int PER>
__global__ __launch_bounds__(kScanThreads) void plan_scan(PlanDims d, int* __restrict__ chunk,
                                                          int* __restrict__ cnt) {
    __shared__ int s_wave[kScanThreads / kWave][kScanExperts];
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();
    const int el = lane % kScanExperts, sub = lane / kScanExperts;
    const int e = blockIdx.x * kScanExperts + el;
    const bool live = e < d.E;
    const int per = (d.nchunks + kScanRanges - 1) / kScanRanges;  // <= PER
    const int c0 = (wave * kScanSubs + sub) * per;
    const int ec = min(e, d.E - 1);
    int v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) v[i] = chunk[min(c0 + i, d.nchunks - 1) * d.E + ec];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if (!(live && i < per && c0 + i < d.nchunks)) v[i] = 0;
        sum += v[i];
    }
    // inclusive sum over this wave's ranges of the same expert (lanes el + 8k)
    int incl = sum;
#pragma unroll
    for (int k = 1; k < kScanSubs; k *= 2) {
        const int t = __shfl_up(incl, k * kScanExperts);
        if (sub >= k) incl += t;
    }
    if (sub == kScanSubs - 1) s_wave[wave][el] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += s_wave[w][el];
    int ex = before + incl - sum;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int c = c0 + i;
        if (live && i < per && c < d.nchunks) chunk[c * d.E + e] = ex;
        ex += v[i];
    }
    if (live && wave == kScanThreads / kWave - 1 && sub == kScanSubs - 1) cnt[e] = before + incl;
}

// -------------------------------------------------------------- plan_global
// Everything this single work-group touches more than once lives in LDS
// (gfx950 gives a work-group up to 160 KiB); global memory is read in one
// round trip at the start and written at the end.
struct GlobalLds {
    int *cnt, *eex, *kept, *js, *prem, *prem1, *cjs, *cje;
    int *rb, *ef, *L, *uex, *dex, *cdl, *cdu, *coin, *fp, *np, *gid, *sbase, *roff;
    int *pst, *phost, *pexp, *ppos, *pn;
    int* scratch;
};

__host__ __device__ inline size_t global_lds_ints(int E, int R) {
    return (size_t)8 * E + 1 + (size_t)13 * R + 10 + (size_t)5 * (E + R) + 1 +
           4 * (kGlobalThreads / kWave + 1);
}

__device__ inline GlobalLds carve_global(int* p, int E, int R) {
    GlobalLds g;
    g.cnt = p; p += E;
    g.eex = p; p += E + 1;
    g.kept = p; p += E;
    g.js = p; p += E;
    g.prem = p; p += E;
    g.prem1 = p; p += E;
    g.cjs = p; p += E;
    g.cje = p; p += E;
    g.rb = p; p += R + 1;
    g.ef = p; p += R + 1;
    g.L = p; p += R;
    g.uex = p; p += R + 1;
    g.dex = p; p += R + 1;
    g.cdl = p; p += R;
    g.cdu = p; p += R;
    g.coin = p; p += R + 1;
    g.fp = p; p += R + 1;
    g.np = p; p += R;
    g.gid = p; p += R + 1;
    g.sbase = p; p += R + 1;
    g.roff = p; p += R + 1;
    g.pst = p; p += E + R + 1;
    g.phost = p; p += E + R;
    g.pexp = p; p += E + R;
    g.ppos = p; p += E + R;
    g.pn = p; p += E + R;
    g.scratch = p;
    return g;
}

// Local instance i of rank u: its expert, first position in (expert, f)
// order and row count.
__device__ __forceinline__ void inst_of(const GlobalLds& g, int u, int i, int* e, int* P, int* n,
                                        int* pi) {
    const int ef = g.ef[u];
    const int nat = g.ef[u + 1] - ef;
    if (i < nat) {
        *e = ef + i;
        *P = g.eex[*e];
        *n = g.kept[*e];
        *pi = -1;
    } else {
        *pi = g.fp[u] + i - nat;
        *e = g.pexp[*pi];
        *P = g.ppos[*pi];
        *n = g.pn[*pi];
    }
}

// Routes of expert e from source ranks below `src` (src == R: all of them).
// Both reads are made and one is kept: selecting the pointer instead (LDS
// counts or global chunk prefixes) compiled to a generic load, which waits
// on the LDS counter too.
__device__ __forceinline__ int pre_of(const PlanDims& d, const int* chunk, const int* cnt, int src,
                                      int e) {
    const int from_chunks = chunk[(min(src, d.R - 1) * d.cps) * d.E + e];
    const int total = cnt[e];
    return src >= d.R ? total : from_chunks;
}

// Exclusive sum when only the first wave holds values (R <= 64 for the
// per-rank scans): that wave scans alone, with no barrier; the total goes to
// that wave, and the caller publishes it through LDS at its next barrier.
// Call with the whole first wave.
__device__ __forceinline__ int wave0_exclusive_sum(int v, int* total) {
    const int inc = wave_inclusive_sum(v);
    *total = __builtin_amdgcn_readlane(inc, kWave - 1);
    return inc - v;
}

// Tables that the fused kernel (plan_fused) keeps in its own LDS where the
// two-kernel form passes them through the workspace.
struct FusedLds {
    int* pre0;    // [E] routes of expert e from source ranks below this block's source
    int* pre1;    // [E] the same below the next source rank
    int4* prec;   // [E+R+1] piece records, as PlanWs::prec
    int* nsend;   // [E] send base of each native instance (this rank)
    int* rcv;     // [E] receive base of this block's source per local instance of this rank
    int* bkt;     // [kBuckets]
};

// What the per-route passes need from the global phases (block-uniform).
struct PhaseScalars {
    int NP, ef_m, nat_m, fp_m, nim, shift;
};

// F. instance counts and gid bases (written to the outputs when `out`).
// Returns the instance total NI, after a closing barrier.
__device__ __forceinline__ int instance_bases(const GlobalLds& g, const PlanOut& o, int R, bool out,
                                              int* scr) {
    const int tid = threadIdx.x;
    int ic = 0;
    if (tid < R) {
        ic = g.ef[tid + 1] - g.ef[tid] + g.np[tid];
        if (out) o.inst_count[tid] = ic;
    }
    int NI, gb = 0;
    if (R <= kWave) {
        if (tid < kWave) gb = wave0_exclusive_sum(ic, &NI);
    } else {
        gb = block_exclusive_sum<false>(ic, scr, &NI);
    }
    if (tid < R) {
        g.gid[tid] = gb;
        if (out) o.inst_gid_base[tid] = gb;
    }
    if (tid == 0) {
        g.gid[R] = NI;
        if (out) o.inst_gid_base[R] = NI;
    }
    lds_barrier();
    return g.gid[R];
}

// H. send bases of this rank: instances in gid order = (dest, slot) order;
// c_m(I) = this rank's routes inside instance I. Writes each native
// instance's base to nsend, each piece's record to prec and each
// destination's first row to g.sbase (no closing barrier). A thread's items
// (at most 3: NI <= 2E + R - 1) keep what the first pass found for the
// second, which would otherwise repeat the dependent LDS lookups after the
// scan's barriers.
__device__ __forceinline__ void send_bases(const GlobalLds& g, int R, int NI, int* nsend,
                                           int4* prec, int* scr) {
    const int tid = threadIdx.x, NT = blockDim.x;
    const int ipt = (NI + NT - 1) / NT;
    const int g0 = min(tid * ipt, NI), g1 = min(g0 + ipt, NI);
    int hq0[kItemCache], hcm[kItemCache], hpi[kItemCache], he[kItemCache], hfirst[kItemCache];
    auto counts = [&](int gi, int* q0, int* cm, int* pi_out, int* e_out, int* first) {
        const int u = upper_bound(g.gid, R + 1, gi) - 1;
        int e, P, n, pi;
        inst_of(g, u, gi - g.gid[u], &e, &P, &n, &pi);
        const int Hm = g.prem1[e] - g.prem[e];
        *q0 = clampi(P - g.eex[e] - g.prem[e], 0, Hm);
        *cm = clampi(P + n - g.eex[e] - g.prem[e], 0, Hm) - *q0;
        *pi_out = pi;
        *e_out = e;
        *first = gi == g.gid[u] ? u : -1;
    };
    int sum = 0;
#pragma unroll
    for (int k = 0; k < kItemCache; ++k) {
        hcm[k] = 0;
        if (g0 + k < g1) counts(g0 + k, &hq0[k], &hcm[k], &hpi[k], &he[k], &hfirst[k]);
        sum += hcm[k];
    }
    for (int gi = g0 + kItemCache; gi < g1; ++gi) {
        int q0, cm, pi, e, first;
        counts(gi, &q0, &cm, &pi, &e, &first);
        sum += cm;
    }
    int tot;
    int run = block_exclusive_sum<false>(sum, scr, &tot);
    auto place = [&](int q0, int cm, int pi, int e, int first) {
        if (pi < 0) {
            nsend[e] = run - q0;
        } else {
            const int host = g.phost[pi];
            prec[pi] = make_int4(host, g.L[host] - g.dex[host], run - q0, g.pexp[pi]);
        }
        if (first >= 0) g.sbase[first] = run;
        run += cm;
    };
#pragma unroll
    for (int k = 0; k < kItemCache; ++k)
        if (g0 + k < g1) place(hq0[k], hcm[k], hpi[k], he[k], hfirst[k]);
    for (int gi = g0 + kItemCache; gi < g1; ++gi) {
        int q0, cm, pi, e, first;
        counts(gi, &q0, &cm, &pi, &e, &first);
        place(q0, cm, pi, e, first);
    }
    if (tid == 0) g.sbase[R] = tot;
}

// J. bucket table: bkt[b] = the piece holding excess index b << shift, so
// that a route finds its piece with one lookup and a short walk. Returns
// shift.
__device__ __forceinline__ int bucket_table(const GlobalLds& g, int NP, int totU, int* bkt) {
    int shift = 0;
    while (((long long)kBuckets << shift) < totU) ++shift;
    for (int b = threadIdx.x; b < kBuckets; b += blockDim.x) {
        const long long start = (long long)b << shift;
        bkt[b] = start < totU ? upper_bound(g.pst, NP, (int)start) - 1 : max(NP - 1, 0);
    }
    return shift;
}

// Phases F to J of a plan_fused work-group (see global_phases). Only this
// rank's own chunks place routes with the send bases of phase H; the
// others take the piece records' host, slot base and expert alone. Phase I
// covers the work-group's own source. Returns before a closing barrier:
// f.rcv, f.bkt, f.nsend and f.prec are read after the caller's next one.
// (Run in one epoch, F, I and J measured 0.4 us slower on a 262144-route
// plan than in this order.)
__device__ __forceinline__ PhaseScalars fused_tail(const PlanDims& d, const PlanOut& o,
                                                   const GlobalLds& g, const FusedLds& f, int NP,
                                                   int totU, int src, int sub) {
    const int R = d.R, m = d.m;
    const int tid = threadIdx.x, NT = blockDim.x;
    const bool out_block = blockIdx.x == 0;
    int* scr0 = g.scratch;
    int* scr1 = g.scratch + 2 * (kGlobalThreads / kWave + 1);

    const int NI = instance_bases(g, o, R, out_block, scr0);  // F

    // H. send bases (this rank's own chunks); elsewhere the piece records
    //    without them
    if (src != m) {
        for (int pi = tid; pi < NP; pi += NT) {
            const int host = g.phost[pi];
            f.prec[pi] = make_int4(host, g.L[host] - g.dex[host], 0, g.pexp[pi]);
        }
    } else {
        send_bases(g, R, NI, f.nsend, f.prec, scr1);
    }

    // I. one source: local instance i of m (thread i; nim <= E <= NT)
    //    covers positions [P', P' + n) of its expert, and this source's
    //    routes of that expert are [pre0, pre1). The rows that earlier
    //    sources send to the instance are its overlap with [0, pre0); the
    //    rows before the item are those of every instance plus this
    //    source's rows in the instances before it.
    const int ef_m = g.ef[m];
    const int nat_m = g.ef[m + 1] - ef_m;
    const int nim = nat_m + g.np[m];
    int q0 = 0, cs = 0, before = 0;
    if (tid < nim) {
        int e, P, n, pi;
        inst_of(g, m, tid, &e, &P, &n, &pi);
        const int pre = f.pre0[e];
        const int Hs = f.pre1[e] - pre;
        const int Pl = P - g.eex[e];
        q0 = clampi(Pl - pre, 0, Hs);
        cs = clampi(Pl + n - pre, 0, Hs) - q0;
        before = clampi(pre - Pl, 0, n);
    }
    int xcs, xbefore, tcs, tbefore;
    block_exclusive_sum2<false>(cs, before, scr0, &xcs, &xbefore, &tcs, &tbefore);
    if (tid < nim) f.rcv[tid] = tbefore + xcs - q0;
    if (sub == 0 && tid == 0) o.recv_count[src] = tcs;
    // g.sbase (phase H) is visible after the scan's barriers
    if (src == m && sub == 0)
        for (int r = tid; r < R; r += NT) o.send_count[r] = g.sbase[r + 1] - g.sbase[r];

    // J. (piece starts are read from g.pst in place)
    const int shift = bucket_table(g, NP, totU, f.bkt);
    return PhaseScalars{NP, ef_m, nat_m, g.fp[m], nim, shift};
}

// Phases A-J of the plan, run by one work-group with every table in LDS.
// FUSED = false: the single plan_global work-group, which writes the whole
// plan's tables to the workspace for plan_routes. FUSED = true: every
// plan_fused work-group runs them for itself (phases F-J in fused_tail);
// work-group 0 writes the per-expert and per-rank outputs, the first
// work-group of each source rank its receive count (and, for this rank, the
// send counts), and only this rank's own source chunks need the send bases
// of phase H. The receive bases of phase I are then those of the
// work-group's source alone, which only needs the routes of each expert
// below that source and below the next (f.pre0, f.pre1). c, pm, pm1: expert e's route total and the routes of e
// from source ranks below m and below m+1 (-1 when m is the last rank),
// held by thread e; pm and pm1 are read only by phase H (fused: only where
// src == m). One element per thread in the per-expert and per-rank phases
// (E, R <= NT).
template <bool FUSED>
__device__ __forceinline__ PhaseScalars global_phases(const PlanDims& d, const PlanWs& w,
                                                      const PlanOut& o, const GlobalLds& g,
                                                      const FusedLds& f, int c, int pm, int pm1,
                                                      int src, int sub) {
    const int E = d.E, R = d.R, C = d.C, m = d.m;
    const int tid = threadIdx.x, NT = blockDim.x;
    const bool out_block = !FUSED || blockIdx.x == 0;
    // two scan buffers, alternated between the block scans so that a scan
    // needs no closing barrier
    int* scr0 = g.scratch;
    int* scr1 = g.scratch + 2 * (kGlobalThreads / kWave + 1);

    // A. expert totals and this rank's per-expert offsets
    int total;
    const int ex = block_exclusive_sum<false>(c, scr0, &total);
    if (tid < E) {
        g.cnt[tid] = c;
        g.eex[tid] = ex;
        g.prem[tid] = pm;
        g.prem1[tid] = pm1 < 0 ? c : pm1;
        if constexpr (!FUSED) w.eex[tid] = ex;
        if (out_block) o.expert_count[tid] = c;
    }
    if (tid == 0) {
        g.eex[E] = total;
        if constexpr (!FUSED) w.eex[E] = total;
    }
    lds_barrier();

    // B. rank blocks, native loads, surplus and deficit prefixes
    for (int r = tid; r <= R; r += NT) {  // R may equal the block size
        const int ef = efirst_of(r, R, E);
        const int rb = g.eex[ef];
        g.ef[r] = ef;
        g.rb[r] = rb;
        if constexpr (!FUSED) w.rb[r] = rb;
    }
    int U = 0, D = 0;
    if (tid < R) {
        const int Lr = g.eex[efirst_of(tid + 1, R, E)] - g.eex[efirst_of(tid, R, E)];
        U = max(Lr - C, 0);
        D = max(C - Lr, 0);
        g.L[tid] = Lr;
        if constexpr (!FUSED) w.load[tid] = Lr;
        if (out_block) o.rank_load[tid] = Lr;
    }
    int uex = 0, dex = 0, totU, totD;
    if (R <= kWave) {
        if (tid < kWave) {
            uex = wave0_exclusive_sum(U, &totU);
            dex = wave0_exclusive_sum(D, &totD);
        }
    } else {
        block_exclusive_sum2<false>(U, D, scr1, &uex, &dex, &totU, &totD);
    }
    if (tid < R) {
        g.uex[tid] = uex;
        g.dex[tid] = dex;
        if constexpr (!FUSED) {
            w.uex[tid] = uex;
            w.dex[tid] = dex;
        }
    }
    if (tid == 0) {
        g.uex[R] = totU;
        g.dex[R] = totD;
        if constexpr (!FUSED) {
            w.uex[R] = totU;
            w.dex[R] = totD;
        }
    }
    lds_barrier();
    totU = g.uex[R];
    totD = g.dex[R];

    // C. rows of each expert kept at home, start of its excess; compacted
    //    lists of spilling experts and under-loaded ranks
    int spill = 0, under = 0, js = 0;
    if (tid < E) {
        const int h = home_of(tid, R, E);
        const long long rb = g.rb[h];
        const int kept = (int)std::min<long long>(std::max<long long>(rb + C - g.eex[tid], 0), c);
        js = g.uex[h] + (int)std::max<long long>(0, g.eex[tid] + kept - rb - C);
        g.kept[tid] = kept;
        g.js[tid] = js;
        spill = kept < c;
    }
    if (tid < R) under = g.L[tid] < C;
    int si, ui, NS, NU;
    block_exclusive_sum2<false>(spill, under, scr0, &si, &ui, &NS, &NU);
    if (spill) {
        g.cjs[si] = js;
        g.cje[si] = tid;
    }
    if (under) {
        g.cdl[ui] = g.dex[tid];
        g.cdu[ui] = tid;
    }
    if (tid < R) g.np[tid] = 0;
    lds_barrier();

    // D. deficit starts that coincide with an expert's excess start
    int coin = 0, lb_d = 0;  // lb_d: first excess start >= this deficit start
    if (tid < NU) {
        const int s = g.cdl[tid];
        lb_d = lower_bound(g.cjs, NS, s);
        coin = lb_d < NS && g.cjs[lb_d] == s;
    }
    int NC, ci = 0;  // NU <= R
    if (R <= kWave) {
        if (tid < kWave) ci = wave0_exclusive_sum(coin, &NC);
    } else {
        ci = block_exclusive_sum<false>(coin, scr1, &NC);
    }
    if (tid < NU) g.coin[tid] = ci;
    if (tid == 0) g.coin[NU] = NC;
    lds_barrier();
    NC = g.coin[NU];
    const int NP = NS + NU - NC;

    // E. pieces (redundant instances): the excess list [0, totU) cut at every
    //    expert boundary and every under-loaded rank boundary, in order; a
    //    piece's index is its start's rank in the merged list of starts.
    if (tid < NS) {
        const int s = g.cjs[tid];
        const int e = g.cje[tid];
        const int lb = lower_bound(g.cdl, NU, s);
        const int pi = tid + lb - g.coin[lb];
        // deficit starts are strictly increasing: upper_bound = lb + (equal)
        const int u = g.cdu[lb + (lb < NU && g.cdl[lb] == s) - 1];
        const int kp = g.kept[e];
        const int end = min(s + g.cnt[e] - kp, g.dex[u] + (C - g.L[u]));
        g.pst[pi] = s;
        g.phost[pi] = u;
        g.pexp[pi] = e;
        g.pn[pi] = end - s;
        g.ppos[pi] = g.eex[e] + kp;
    }
    if (tid < NU && !coin) {
        const int s = g.cdl[tid];
        const int u = g.cdu[tid];
        const int lb = lb_d;
        const int pi = tid + lb - g.coin[tid];
        const int e = g.cje[lb - 1];
        const int jse = g.js[e];
        const int kp = g.kept[e];
        const int end = min(jse + g.cnt[e] - kp, s + (C - g.L[u]));
        g.pst[pi] = s;
        g.phost[pi] = u;
        g.pexp[pi] = e;
        g.pn[pi] = end - s;
        g.ppos[pi] = g.eex[e] + kp + (s - jse);
    }
    if (tid < NU) g.fp[g.cdu[tid]] = tid + lb_d - g.coin[tid];
    if (tid == 0) g.pst[NP] = totU;
    lds_barrier();
    if (tid < NU) {
        const int u = g.cdu[tid];
        const int nxt = tid + 1 < NU ? g.fp[g.cdu[tid + 1]] : NP;
        g.np[u] = nxt - g.fp[u];
    }
    lds_barrier();

    if constexpr (FUSED) return fused_tail(d, o, g, f, NP, totU, src, sub);

    const int NI = instance_bases(g, o, R, true, scr0);  // F

    // G. per-rank instance layout for the table fill done by plan_routes
    for (int u = tid; u < R; u += NT)
        w.rinfo[u] = make_int4(g.ef[u], g.ef[u + 1] - g.ef[u], g.np[u], g.fp[u]);

    send_bases(g, R, NI, w.nsend, w.prec, scr1);  // H

    // I. receive bases of this rank: items (source, local instance i) in
    //    arrival order; recvbase = sources' rows before the item minus the
    //    item's start rank within its expert. The first kItemCache items of
    //    a thread keep their counts (two global loads each) for the second
    //    pass.
    const int ef_m = g.ef[m];
    const int nat_m = g.ef[m + 1] - ef_m;
    const int nim = nat_m + g.np[m];
    {
        const int items = R * nim;
        const int ipt = (items + NT - 1) / NT;
        const int q0i = min(tid * ipt, items), q1i = min(q0i + ipt, items);
        int rq0[kItemCache], rcs[kItemCache];
        auto counts = [&](int q, int* q0, int* cs) {
            const int src = q / nim, i = q - src * nim;
            int e, P, n, pi;
            inst_of(g, m, i, &e, &P, &n, &pi);
            const int pre = pre_of(d, w.chunk, g.cnt, src, e);
            const int Hs = pre_of(d, w.chunk, g.cnt, src + 1, e) - pre;
            *q0 = clampi(P - g.eex[e] - pre, 0, Hs);
            *cs = clampi(P + n - g.eex[e] - pre, 0, Hs) - *q0;
        };
        int sum = 0;
#pragma unroll
        for (int k = 0; k < kItemCache; ++k) {
            rcs[k] = 0;
            if (q0i + k < q1i) counts(q0i + k, &rq0[k], &rcs[k]);
            sum += rcs[k];
        }
        for (int q = q0i + kItemCache; q < q1i; ++q) {
            int q0, cs;
            counts(q, &q0, &cs);
            sum += cs;
        }
        int tot;
        int run = block_exclusive_sum<false>(sum, scr0, &tot);
        auto place = [&](int q, int q0, int cs) {
            const int src = q / nim, i = q - src * nim;
            w.recvbase[src * E + i] = run - q0;
            if (i == 0) g.roff[src] = run;
            run += cs;
        };
#pragma unroll
        for (int k = 0; k < kItemCache; ++k)
            if (q0i + k < q1i) place(q0i + k, rq0[k], rcs[k]);
        for (int q = q0i + kItemCache; q < q1i; ++q) {
            int q0, cs;
            counts(q, &q0, &cs);
            place(q, q0, cs);
        }
        if (tid == 0) g.roff[R] = tot;
    }
    lds_barrier();
    for (int r = tid; r < R; r += NT) {
        o.send_count[r] = g.sbase[r + 1] - g.sbase[r];
        o.recv_count[r] = g.roff[r + 1] - g.roff[r];
    }

    // J. tables the per-route kernel stages: piece starts and the bucket table
    for (int i = tid; i <= NP; i += NT) w.pstart[i] = g.pst[i];
    const int shift = bucket_table(g, NP, totU, w.bucket);
    if (tid == 0) {
        w.scal[SC_NP] = NP;
        w.scal[SC_EFIRST_M] = ef_m;
        w.scal[SC_NAT_M] = nat_m;
        w.scal[SC_FP_M] = g.fp[m];
        w.scal[SC_NIM] = nim;
        w.scal[SC_SHIFT] = shift;
    }
    return PhaseScalars{NP, ef_m, nat_m, g.fp[m], nim, shift};
}

// One element per thread in the per-expert and per-rank phases (E, R <= NT).
__global__ __launch_bounds__(kGlobalThreads) void plan_global(PlanDims d, PlanWs w, PlanOut o) {
    // the first loads' arguments as one batch of scalar loads (as in plan_hist)
    asm volatile("" ::"s"(w.cnt), "s"(w.chunk), "s"(d.E), "s"(d.R), "s"(d.m), "s"(d.cps));
    extern __shared__ int lds[];
    const int E = d.E, R = d.R, m = d.m;
    const int tid = threadIdx.x;
    const GlobalLds g = carve_global(lds, E, R);
    // one round trip: expert totals and this rank's per-expert offsets
    int c = 0, pm = 0, pm1 = 0;
    if (tid < E) {
        c = w.cnt[tid];
        pm = w.chunk[(m * d.cps) * E + tid];
        pm1 = m + 1 < R ? w.chunk[((m + 1) * d.cps) * E + tid] : -1;
    }
    (void)global_phases<false>(d, w, o, g, FusedLds{}, c, pm, pm1, 0, 0);
}

// -------------------------------------------------------------- plan_routes
// Element i of a route-sized array through a 32-bit byte offset: route
// indices stay below 2^30, so 4*i fits, and the store can take its base
// from scalar registers with no 64-bit address arithmetic per lane.
__device__ __forceinline__ int& at32(int* base, int i) {
    return *(int*)((char*)base + (uint32_t)i * 4u);
}

// plan_routes stages its tables through registers: every load is issued
// first, at clamped indices and with no branches, and the LDS writes follow
// once all of them are in flight. Staged table by table, each table's
// writes waited for its loads before the next table's loads went out: five
// global round trips in the prologue where one suffices.
constexpr int kPmRegs = (kMaxE + kMaxR + 1 + kRouteThreads - 1) / kRouteThreads;
constexpr int kBktRegs = (kBuckets + kRouteThreads - 1) / kRouteThreads;
constexpr int kIdRegs = (kStageIds + kRouteThreads - 1) / kRouteThreads;

// v[u] = src[min(u * NT + tid, n - 1)]; needs 1 <= n.
template <int NT, int U, typename T>
__device__ __forceinline__ void regs_load(T (&v)[U], const T* __restrict__ src, int n) {
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[min(u * NT + (int)threadIdx.x, n - 1)];
}

// dst[i] = v[u] for i = u * NT + tid < n.
template <int NT, int U, typename T>
__device__ __forceinline__ void regs_store(T* dst, const T (&v)[U], int n) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = u * NT + (int)threadIdx.x;
        if (i < n) dst[i] = v[u];
    }
}

// LDS per work-group: per-wave counters, two packed per-expert tables, the
// receive bases of this source, piece starts and records, the bucket table
// and (for chunks up to kStageIds routes) the chunk's ids.
__host__ __device__ inline size_t routes_lds_ints(int E, int R, int T) {
    const size_t PM = (size_t)E + R + 1;
    return (size_t)kRouteWaves * E + (size_t)4 * E + (size_t)4 * E + PM + 4 * PM + kBuckets +
           (T <= kStageIds ? T : 0);
}

// Passes 1 and 2 of a chunk (shared by plan_routes and plan_fused), on the
// staged tables: s_ex0/s_ex1 per expert, piece starts s_ps and records
// s_prec, the bucket table s_bkt, zeroed per-wave counters s_cnt and, when
// STAGED, the chunk's ids in s_ids. The chunk is routes [f0, f0 + len) of
// source rank src.
template <bool STAGED, int KEY_BITS, int NT>
__device__ __forceinline__ void route_passes(const PlanDims& d, const int* __restrict__ ids,
                                             const PlanOut& o, int src, int f0, int len,
                                             const int4* s_ex0, const int4* s_ex1,
                                             const int4* s_prec, const int* s_ps,
                                             const int* s_bkt, int* s_cnt, const int* s_ids,
                                             int NP, int nat_m, int fp_m, int shift) {
    const int E = d.E, R = d.R, C = d.C, m = d.m;
    const int tid = threadIdx.x;
    const int PM = E + R + 1;
    const int wave = tid / kWave;
    const int lane = tid & (kWave - 1);
    const int seg = (((len + (NT / kWave) - 1) / (NT / kWave)) + kWave - 1) & ~(kWave - 1);
    const int a = min(wave * seg, len);
    const int b = min(a + seg, len);
    int* my_cnt = s_cnt + wave * E;

    // pass 1: per-wave expert counts
    if (STAGED) {
        for (int j = a + lane; j < b; j += kWave) {
            const int e = s_ids[j];
            if ((unsigned)e < (unsigned)E) atomicAdd(&my_cnt[e], 1);
        }
    } else {
        constexpr int U = 4;  // global id loads in flight per lane
        for (int j0 = a + lane; j0 < b; j0 += U * kWave) {
            int ev[U];
#pragma unroll
            for (int u = 0; u < U; ++u) ev[u] = j0 + u * kWave < b ? ids[f0 + j0 + u * kWave] : -1;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if ((unsigned)ev[u] < (unsigned)E) atomicAdd(&my_cnt[ev[u]], 1);
        }
    }
    lds_barrier();
    for (int e = tid; e < E; e += NT) {
        int run = 0;
#pragma unroll 4
        for (int v = 0; v < (NT / kWave); ++v) {
            const int t = s_cnt[v * E + e];
            s_cnt[v * E + e] = run;
            run += t;
        }
    }
    lds_barrier();

    // pass 2: stable rank within the chunk, then placement
    int e_next = 0;
    if (!STAGED && a + lane < b) e_next = ids[f0 + a + lane];
    for (int base = a; base < b; base += kWave) {
        const int j = base + lane;
        const int f = f0 + j;
        bool valid = j < b;
        int e;
        if (STAGED) {
            e = valid ? s_ids[j] : 0;
        } else {
            e = valid ? e_next : 0;
            if (j + kWave < b) e_next = ids[f + kWave];  // before this step's stores
        }
        valid = valid && (unsigned)e < (unsigned)E;
        if (!valid) e = 0;
        // the expert's records are read with its count, in one LDS round
        // trip (read after the count's update they would wait for it)
        const int4 x0 = s_ex0[e];
        const int4 x1 = s_ex1[e];
        const uint64_t peers = match_peers<KEY_BITS>(e, valid);
        const int below = count_below(peers);
        const int cnt = my_cnt[e];
        int rin = cnt + below;
        // rin is formed before the branch below: formed after it, the merge
        // of the two paths made the compiler wait for the count's update to
        // complete as well
        asm volatile("" : "+v"(rin));
        // the group's lowest lane moves the count past the whole group
        if (valid && below == 0) my_cnt[e] = cnt + __popcll(peers);
        int dest = -1, slot = -1;
        if (valid) {
            const int q = x0.x + rin;
            const int qs = x0.y + rin;
            if (q < C) {
                dest = x0.w;
                slot = q;
                if (src == m) at32(o.send_pos, f - m * C) = x0.z + qs;
                if (dest == m && (unsigned)slot < (unsigned)C) at32(o.recv_pos, slot) = x1.y + qs;
            } else {
                const int jx = x1.x + rin;
                const int bi = jx >> shift;
                int pi = s_bkt[bi < 0 ? 0 : min(bi, kBuckets - 1)];
                // the bucket's first piece and the next piece's start come
                // in one round trip; a later piece needs further steps
                int4 pr = s_prec[pi];
                const int next_start = s_ps[min(pi + 1, PM - 1)];
                if (pi + 1 < NP && next_start <= jx) {
                    do ++pi;
                    while (pi + 1 < NP && s_ps[pi + 1] <= jx);
                    pr = s_prec[pi];
                }
                if ((unsigned)pr.x < (unsigned)R && pi < NP) {
                    dest = pr.x;
                    slot = pr.y + jx;
                    if (src == m) at32(o.send_pos, f - m * C) = pr.z + qs;
                    const int i = nat_m + pi - fp_m;
                    if (dest == m && (unsigned)slot < (unsigned)C && (unsigned)i < (unsigned)E)
                        at32(o.recv_pos, slot) = s_ex1[i].w + qs;
                }
            }
        }
        if (j < b && o.route_dest) {
            at32(o.route_dest, f) = dest;
            at32(o.route_slot, f) = slot;
        }
    }
}

// STAGED: the chunk's ids are copied to LDS (chunks of at most kStageIds
// routes), else both passes read them from global memory (the second time
// from L2): pass 1 with several loads in flight per lane, pass 2 loading the
// next step's ids before this step's work. Larger chunks only occur at
// N > 2M routes, where leaving the ids out of LDS shortened the table-staging
// prologue and measured 2 us faster on a 4M-route plan. KEY_BITS: width of
// the expert ids in the wave multi-split (8 ballots when E <= 256).
template <bool STAGED, int KEY_BITS>
__global__ __launch_bounds__(kRouteThreads) void plan_routes(PlanDims d, PlanWs w,
                                                             const int* __restrict__ ids,
                                                             PlanOut o) {
    extern __shared__ int4 lds4[];  // 16-byte aligned base
    const int E = d.E, R = d.R, C = d.C, m = d.m;
    const int tid = threadIdx.x;
    const int PM = E + R + 1;  // room for every piece start
    int4* s_ex0 = lds4;                                   // [E] {qbase, q0, nsend, home}
    int4* s_prec = s_ex0 + E;                             // [PM] piece records
    int4* s_ex1 = s_prec + PM;  // [E] {jbase, native recv base, native cu, recv base of local instance e}
    int* s_cnt = (int*)(s_ex1 + E);                       // [waves][E]
    int* s_ps = s_cnt + kRouteWaves * E;                  // [PM] piece starts
    int* s_bkt = s_ps + PM;                               // [kBuckets]
    int* s_ids = s_bkt + kBuckets;                        // [T] when T <= kStageIds

    const int c = blockIdx.x;
    const int src = c / d.cps, sub = c - src * d.cps;
    const int f0 = src * C + sub * d.T;
    const int f1 = min(f0 + d.T, (src + 1) * C);
    const int len = f1 - f0;  // >= 1: a source's last chunk holds the rest of its C routes

    // the staged tables' loads go out first (their LDS writes follow below)
    int ps_r[kPmRegs], bk_r[kBktRegs], id_r[STAGED ? kIdRegs : 1];
    i32x4 pr_r[kPmRegs];
    regs_load<kRouteThreads>(ps_r, w.pstart, PM);
    regs_load<kRouteThreads>(pr_r, (const i32x4*)w.prec, PM);
    regs_load<kRouteThreads>(bk_r, w.bucket, kBuckets);
    if constexpr (STAGED) regs_load<kRouteThreads>(id_r, ids + f0, len);
    // this block's share of the instance tables (filled after the barrier):
    // its first rank record joins this round trip
    const int E1 = E + 1;
    const int per = (R * E1 + gridDim.x - 1) / gridDim.x;
    const int lo = min(blockIdx.x * per, R * E1), hi = min(lo + per, R * E1);
    const int step_u = kRouteThreads / E1, step_i = kRouteThreads - step_u * E1;
    const int u0 = (lo + tid) / E1, i0 = (lo + tid) - u0 * E1;
    const int4 ri0 = lo + tid < hi ? w.rinfo[u0] : make_int4(0, 0, 0, 0);

    // one round trip: every table this block reads, and its routes.
    // For a route of expert e at rank rin among the chunk's routes of e:
    //   q  = qbase[e] + rin   slot on the home rank if q < C
    //   qs = q0[e] + rin      rank among this source's routes of e
    //   j  = jbase[e] + rin   index in the global excess list otherwise
    const int NP = w.scal[SC_NP];
    const int ef_m = w.scal[SC_EFIRST_M];
    const int nat_m = w.scal[SC_NAT_M];
    const int fp_m = w.scal[SC_FP_M];
    const int shift = w.scal[SC_SHIFT];
    for (int e = tid; e < E; e += kRouteThreads) {
        const int h = home_of(e, R, E);
        const int off = w.chunk[c * E + e];
        const int pre = w.chunk[(src * d.cps) * E + e];
        const int eex = w.eex[e], rbh = w.rb[h];
        const int qbase = eex + off - rbh;
        const int rcv = w.recvbase[src * E + e];
        const int nrcv = h == m ? w.recvbase[src * E + (e - ef_m)] : 0;
        s_ex0[e] = make_int4(qbase, off - pre, w.nsend[e], h);
        s_ex1[e] = make_int4(w.uex[h] + qbase - C, nrcv, min(eex - rbh, C), rcv);
    }
    for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) s_cnt[i] = 0;
    regs_store<kRouteThreads>(s_ps, ps_r, PM);
    regs_store<kRouteThreads>((i32x4*)s_prec, pr_r, PM);
    regs_store<kRouteThreads>(s_bkt, bk_r, kBuckets);
    if constexpr (STAGED) regs_store<kRouteThreads>(s_ids, id_r, len);
    lds_barrier();

    // this block's slice of the instance tables inst_cu [R][E+1] and
    // inst_expert [R][E]: idx = u*(E+1) + i, walked without divisions; the
    // first step's rank record was loaded with the tables above
    {
        int u = u0, i = i0;
        for (int idx = lo + tid; idx < hi; idx += kRouteThreads) {
            const int4 ri = idx == lo + tid ? ri0 : w.rinfo[u];
            int cu = C, ie = -1;
            if (i < ri.y) {
                ie = ri.x + i;
                cu = s_ex1[ie].z;
            } else if (i < ri.y + ri.z) {
                const int pi = ri.w + i - ri.y;
                const int4 pr = s_prec[pi];
                cu = pr.y + s_ps[pi];
                ie = pr.w;
            }
            o.inst_cu[idx] = cu;
            if (i < E) o.inst_expert[u * E + i] = ie;
            u += step_u;
            i += step_i;
            if (i >= E1) {
                i -= E1;
                ++u;
            }
        }
    }

    route_passes<STAGED, KEY_BITS, kRouteThreads>(d, ids, o, src, f0, len, s_ex0, s_ex1, s_prec,
                                                  s_ps, s_bkt, s_cnt, s_ids, NP, nat_m, fp_m,
                                                  shift);
}

// -------------------------------------------------------------- plan_fused
// plan_global and plan_routes in one launch: every work-group runs the
// global phases for itself in LDS, then its chunk's routes. It saves the
// launch boundary between the two and the prologue in which plan_routes
// stages the global tables from the workspace; the loads the work-group
// needs (expert totals, chunk offsets, its ids) go out together at the
// start. Used when its LDS fits (the global and the per-route tables side
// by side).
__host__ __device__ inline size_t fused_lds_ints(int E, int R, int T, int NT) {
    const size_t PM = (size_t)E + R + 1;
    return (size_t)4 * E + 4 * PM + (size_t)4 * E + (size_t)(NT / kWave) * E + kBuckets +
           (T <= kStageIds ? T : 0) + (size_t)4 * E + global_lds_ints(E, R);
}

static_assert(kRouteThreads <= kGlobalThreads, "the global phases' scan scratch covers the block");

// Two work-groups per CU (8 waves per SIMD) when there are more chunks than
// CUs: without the waves-per-EU bound the fused body took 106 scalar
// registers, which leaves room for 7 waves per SIMD, i.e. one work-group.
template <bool STAGED, int KEY_BITS, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8)))
void plan_fused(PlanDims d, PlanWs w, const int* __restrict__ ids, PlanOut o) {
    // the prologue loads' arguments as one batch of scalar loads (as in
    // plan_hist): the workspace pointers had come one round trip later
    asm volatile("" ::"s"(w.cnt), "s"(w.chunk), "s"(ids), "s"(d.E), "s"(d.R), "s"(d.C),
                 "s"(d.m), "s"(d.T), "s"(d.cps));
    extern __shared__ int4 lds4[];  // 16-byte aligned base
    const int E = d.E, R = d.R, C = d.C, m = d.m;
    const int tid = threadIdx.x;
    const int PM = E + R + 1;
    int4* s_ex0 = lds4;          // [E] {qbase, q0, nsend, home}
    int4* s_prec = s_ex0 + E;    // [PM] piece records
    int4* s_ex1 = s_prec + PM;   // [E] {jbase, native recv base, native cu, recv base of local instance e}
    int* s_cnt = (int*)(s_ex1 + E);        // [waves][E]
    int* s_bkt = s_cnt + (NT / kWave) * E;  // [kBuckets]
    int* s_ids = s_bkt + kBuckets;         // [T] when STAGED
    int* s_pre0 = s_ids + (STAGED ? d.T : 0);
    int* s_pre1 = s_pre0 + E;
    int* s_nsend = s_pre1 + E;
    int* s_rcv = s_nsend + E;
    const GlobalLds g = carve_global(s_rcv + E, E, R);
    const FusedLds f{s_pre0, s_pre1, s_prec, s_nsend, s_rcv, s_bkt};

    const int c = blockIdx.x;
    const int src = c / d.cps, sub = c - src * d.cps;
    const int f0 = src * C + sub * d.T;
    const int f1 = min(f0 + d.T, (src + 1) * C);
    const int len = f1 - f0;  // >= 1: a source's last chunk holds the rest of its C routes

    // one round trip: expert e's total and its routes from source ranks
    // below this chunk, below this source and below the next. The global
    // phases need the routes below m and m + 1 only in this rank's own
    // chunks (src == m), where they are the last two. The ids' loads go out
    // after the LDS writes that wait for these, so that the wait does not
    // include them; they are needed only after the global phases.
    const int sn = min(src + 1, R - 1);
    int cnt = 0, off = 0, pre0 = 0, pre1 = -1;
    if (tid < E) {
        cnt = w.cnt[tid];
        off = w.chunk[c * E + tid];
        pre0 = w.chunk[(src * d.cps) * E + tid];
        const int nxt = w.chunk[(sn * d.cps) * E + tid];
        if (src + 1 < R) pre1 = nxt;
        s_pre0[tid] = pre0;
        s_pre1[tid] = pre1 < 0 ? cnt : pre1;
    }
    int id_r[STAGED ? ((kStageIds + NT - 1) / NT) : 1];
    if constexpr (STAGED) regs_load<NT>(id_r, ids + f0, len);

    const PhaseScalars ps = global_phases<true>(d, w, o, g, f, cnt, pre0, pre1, src, sub);

    for (int i = tid; i < (NT / kWave) * E; i += NT) s_cnt[i] = 0;
    if constexpr (STAGED) regs_store<NT>(s_ids, id_r, len);
    lds_barrier();

    // per-expert records of this chunk (see plan_routes)
    if (tid < E) {
        const int e = tid;
        const int h = home_of(e, R, E);
        const int eex = g.eex[e], rbh = g.rb[h];
        const int qbase = eex + off - rbh;
        const int nrcv = h == m ? s_rcv[e - ps.ef_m] : 0;
        s_ex0[e] = make_int4(qbase, off - pre0, s_nsend[e], h);
        s_ex1[e] = make_int4(g.uex[h] + qbase - C, nrcv, min(eex - rbh, C), s_rcv[e]);
    }

    // this block's slice of the instance tables inst_cu [R][E+1] and
    // inst_expert [R][E], idx = u*(E+1) + i
    {
        const int E1 = E + 1;
        const int per = (R * E1 + gridDim.x - 1) / gridDim.x;
        const int lo = min(blockIdx.x * per, R * E1), hi = min(lo + per, R * E1);
        for (int idx = lo + tid; idx < hi; idx += NT) {
            const int u = idx / E1, i = idx - u * E1;
            const int ef = g.ef[u], nat = g.ef[u + 1] - ef;
            int cu = C, ie = -1;
            if (i < nat) {
                ie = ef + i;
                cu = min(g.eex[ie] - g.rb[u], C);
            } else if (i < nat + g.np[u]) {
                const int pi = g.fp[u] + i - nat;
                const int4 pr = s_prec[pi];
                cu = pr.y + g.pst[pi];
                ie = pr.w;
            }
            o.inst_cu[idx] = cu;
            if (i < E) o.inst_expert[u * E + i] = ie;
        }
    }

    // the records above are read after the first pass's barriers
    route_passes<STAGED, KEY_BITS, NT>(d, ids, o, src, f0, len, s_ex0, s_ex1, s_prec,
                                                  g.pst, s_bkt, s_cnt, s_ids, ps.NP, ps.nat_m,
                                                  ps.fp_m, ps.shift);
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
    long long T = kMinChunk;
    while (T < C && T < kStageIds && (long long)R * ((C + T - 1) / T) > kTargetChunks) T *= 2;
    while (T < C && (long long)R * ((C + T - 1) / T) > kTargetChunksLong) T *= 2;
    d->T = (int)std::min<long long>(T, C);
    d->cps = (int)((C + d->T - 1) / d->T);
    d->nchunks = R * d->cps;
    return true;
}

struct WsOffsets {
    size_t chunk, cnt, eex, rb, load, uex, dex, pstart, prec, bucket, nsend, recvbase, rinfo, scal, total;
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
    o.pstart = take(E + R + 1);
    o.prec = take(4 * (E + R + 1));
    o.bucket = take(kBuckets);
    o.nsend = take(E);
    o.recvbase = take(R * E);
    o.rinfo = take(4 * R);
    o.scal = take(SC_COUNT);
    o.total = at;
    return o;
}

size_t global_lds_bytes(const PlanDims& d) { return global_lds_ints(d.E, d.R) * sizeof(int); }

size_t routes_lds_bytes(const PlanDims& d) { return routes_lds_ints(d.E, d.R, d.T) * sizeof(int); }

// plan_fused's block size: 512 threads when the chunks outnumber the CUs
// (two or more work-groups per CU) and are short enough to stage, else
// 1024. Measured: a 524288-route plan with E=384 in 512 chunks of 1024
// routes took 25.3 us with 512 threads against 27.1 us with 1024; the
// 262144-route plan in 256 chunks 23.5 against 23.2 us, and the 4M-route
// plan in 512 chunks of 8192 routes 46.0 against 43.4 us.
int fused_threads(const PlanDims& d) {
    const bool small = d.nchunks > 256 && d.T <= kStageIds && d.E <= kFusedThreadsSmall &&
                       d.R <= kFusedThreadsSmall;
    return small ? kFusedThreadsSmall : kRouteThreads;
}

size_t fused_lds_bytes(const PlanDims& d) {
    return fused_lds_ints(d.E, d.R, d.T, fused_threads(d)) * sizeof(int);
}

bool lds_ready() {
    // Allow the single-pass kernels to use more than 64 KiB of LDS when
    // the sizes call for it (gfx950 has 160 KiB per CU).
    static const bool ok = [] {
        const int lim = (int)kMaxLds;
        bool good = hipFuncSetAttribute((const void*)plan_global,
                                        hipFuncAttributeMaxDynamicSharedMemorySize,
                                        lim) == hipSuccess;
        for (const void* k : {(const void*)plan_routes<true, kKeyBits>,
                              (const void*)plan_routes<false, kKeyBits>,
                              (const void*)plan_fused<true, 8, kRouteThreads>,
                              (const void*)plan_fused<true, kKeyBits, kRouteThreads>,
                              (const void*)plan_fused<false, 8, kRouteThreads>,
                              (const void*)plan_fused<false, kKeyBits, kRouteThreads>,
                              (const void*)plan_fused<true, 8, kFusedThreadsSmall>,
                              (const void*)plan_fused<true, kKeyBits, kFusedThreadsSmall>})
            good = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, lim) ==
                       hipSuccess &&
                   good;
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

namespace mep {
namespace {

// Validation shared by both plan entry points (everything but the
// workspace). On success *d holds the sizes and *o the outputs.
int plan_check(int R, int E, int S, int K, int my_rank, const int32_t* topk_ids,
               int32_t* expert_count, int32_t* rank_load, int32_t* route_dest,
               int32_t* route_slot, int32_t* inst_count, int32_t* inst_expert, int32_t* inst_cu,
               int32_t* inst_gid_base, int32_t* send_pos, int32_t* send_count, int32_t* recv_pos,
               int32_t* recv_count, PlanDims* d, PlanOut* o) {
    if (!topk_ids || !expert_count || !rank_load || !inst_count || !inst_expert || !inst_cu ||
        !inst_gid_base || !send_pos || !send_count || !recv_pos || !recv_count)
        return MEP_ERR_NULLPTR;
    if (!plan_dims(R, E, S, K, my_rank, d)) return MEP_ERR_SHAPE;
    if (K > E || my_rank < 0 || my_rank >= R) return MEP_ERR_PARAM;
    if ((route_dest == nullptr) != (route_slot == nullptr)) return MEP_ERR_PARAM;
    const size_t glds = global_lds_bytes(*d), rlds = routes_lds_bytes(*d);
    if (glds > kMaxLds || rlds > kMaxLds) return MEP_ERR_SHAPE;  // not reachable within the limits
    *o = PlanOut{expert_count, rank_load, route_dest, route_slot, inst_count, inst_expert,
                 inst_cu, inst_gid_base, send_pos, send_count, recv_pos, recv_count};
    return MEP_OK;
}

// The four launches on a workspace already checked against ws_offsets(d).
int plan_launch(const PlanDims& d, char* ws, const int32_t* topk_ids, const PlanOut& o,
                hipStream_t s) {
    const WsOffsets off = ws_offsets(d);
    PlanWs w;
    w.chunk = (int*)(ws + off.chunk);
    w.cnt = (int*)(ws + off.cnt);
    w.eex = (int*)(ws + off.eex);
    w.rb = (int*)(ws + off.rb);
    w.load = (int*)(ws + off.load);
    w.uex = (int*)(ws + off.uex);
    w.dex = (int*)(ws + off.dex);
    w.pstart = (int*)(ws + off.pstart);
    w.prec = (int4*)(ws + off.prec);
    w.bucket = (int*)(ws + off.bucket);
    w.nsend = (int*)(ws + off.nsend);
    w.recvbase = (int*)(ws + off.recvbase);
    w.rinfo = (int4*)(ws + off.rinfo);
    w.scal = (int*)(ws + off.scal);
    const size_t glds = global_lds_bytes(d), rlds = routes_lds_bytes(d), flds = fused_lds_bytes(d);
    // the fused work-group runs the global phases with one element per
    // thread
    const int fnt = fused_threads(d);
    const bool fused = flds <= kMaxLds && d.E <= fnt && d.R <= fnt;
    const size_t big = fused ? flds : std::max(glds, rlds);
    if (big > 64 * 1024 && !lds_ready()) return MEP_ERR_HIP;

    hipLaunchKernelGGL(plan_hist, dim3(d.nchunks), dim3(kHistThreads), d.E * sizeof(int), s, d,
                       (const int*)topk_ids, w.chunk);
    MEP_LAUNCH_CHECK();
    {
        const int per = (d.nchunks + kScanRanges - 1) / kScanRanges;
        const dim3 sg((d.E + kScanExperts - 1) / kScanExperts), sb(kScanThreads);
        if (per <= 1) hipLaunchKernelGGL(plan_scan<1>, sg, sb, 0, s, d, w.chunk, w.cnt);
        else if (per <= 2) hipLaunchKernelGGL(plan_scan<2>, sg, sb, 0, s, d, w.chunk, w.cnt);
        else if (per <= 4) hipLaunchKernelGGL(plan_scan<4>, sg, sb, 0, s, d, w.chunk, w.cnt);
        else hipLaunchKernelGGL(plan_scan<kScanItems>, sg, sb, 0, s, d, w.chunk, w.cnt);
    }
    MEP_LAUNCH_CHECK();
    // expert ids below 256 need 8 ballots in the multi-split, not 10
    const dim3 rg(d.nchunks), rb(kRouteThreads), fb(fnt);
    const int* ids = (const int*)topk_ids;
    if (fused) {
        constexpr int NS = kFusedThreadsSmall, NL = kRouteThreads;
        if (fnt == NS) {  // staged ids only
            if (d.E <= 256) hipLaunchKernelGGL((plan_fused<true, 8, NS>), rg, fb, flds, s, d, w, ids, o);
            else hipLaunchKernelGGL((plan_fused<true, kKeyBits, NS>), rg, fb, flds, s, d, w, ids, o);
        } else if (d.T <= kStageIds) {
            if (d.E <= 256) hipLaunchKernelGGL((plan_fused<true, 8, NL>), rg, fb, flds, s, d, w, ids, o);
            else hipLaunchKernelGGL((plan_fused<true, kKeyBits, NL>), rg, fb, flds, s, d, w, ids, o);
        } else {
            if (d.E <= 256) hipLaunchKernelGGL((plan_fused<false, 8, NL>), rg, fb, flds, s, d, w, ids, o);
            else hipLaunchKernelGGL((plan_fused<false, kKeyBits, NL>), rg, fb, flds, s, d, w, ids, o);
        }
        MEP_LAUNCH_CHECK();
        return MEP_OK;
    }
    hipLaunchKernelGGL(plan_global, dim3(1), dim3(kGlobalThreads), glds, s, d, w, o);
    MEP_LAUNCH_CHECK();
    // only E above 256 reaches the two-launch form (with E <= 256 the fused
    // tables fit for every R up to the limit), so its keys are 10-bit
    if (d.T <= kStageIds)
        hipLaunchKernelGGL((plan_routes<true, kKeyBits>), rg, rb, rlds, s, d, w, ids, o);
    else
        hipLaunchKernelGGL((plan_routes<false, kKeyBits>), rg, rb, rlds, s, d, w, ids, o);
    MEP_LAUNCH_CHECK();
    return MEP_OK;
}

}  // namespace
}  // namespace mep

extern "C" int mep_plan(int R, int E, int S, int K, int my_rank, const int32_t* topk_ids,
                        void* workspace, size_t workspace_bytes, int32_t* expert_count,
                        int32_t* rank_load, int32_t* route_dest, int32_t* route_slot,
                        int32_t* inst_count, int32_t* inst_expert, int32_t* inst_cu,
                        int32_t* inst_gid_base, int32_t* send_pos, int32_t* send_count,
                        int32_t* recv_pos, int32_t* recv_count, void* stream) {
    if (!workspace) return MEP_ERR_NULLPTR;
    PlanDims d;
    PlanOut o;
    const int st = plan_check(R, E, S, K, my_rank, topk_ids, expert_count, rank_load, route_dest,
                              route_slot, inst_count, inst_expert, inst_cu, inst_gid_base,
                              send_pos, send_count, recv_pos, recv_count, &d, &o);
    if (st != MEP_OK) return st;
    if (workspace_bytes < ws_offsets(d).total || ((uintptr_t)workspace & 255u) != 0)
        return MEP_ERR_PARAM;
    return plan_launch(d, (char*)workspace, topk_ids, o, (hipStream_t)stream);
}

// ------------------------------------------------------ allocation-free plan
// mep_plan_noalloc keeps its workspace in this file-scope device array: each
// GPU holds its own copy, at its own address, for the life of the process.
// In host code the name `scratch` stands for a host-side shadow, not a device
// address, so the kernels only ever see the address hipGetSymbolAddress
// returns for the current device.
static __device__ __align__(256) unsigned char scratch[MEP_PLAN_NOALLOC_SCRATCH_BYTES];

namespace mep {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up once per
// device (the first call on that device) and kept.
int scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return MEP_ERR_HIP;
    }
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
                (void)hipGetLastError();
                return MEP_ERR_HIP;
            }
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MEP_OK;
}

}  // namespace
}  // namespace mep

extern "C" int mep_plan_noalloc(int R, int E, int S, int K, int my_rank, const int32_t* topk_ids,
                                int32_t* expert_count, int32_t* rank_load, int32_t* route_dest,
                                int32_t* route_slot, int32_t* inst_count, int32_t* inst_expert,
                                int32_t* inst_cu, int32_t* inst_gid_base, int32_t* send_pos,
                                int32_t* send_count, int32_t* recv_pos, int32_t* recv_count,
                                void* stream) {
    PlanDims d;
    PlanOut o;
    const int st = plan_check(R, E, S, K, my_rank, topk_ids, expert_count, rank_load, route_dest,
                              route_slot, inst_count, inst_expert, inst_cu, inst_gid_base,
                              send_pos, send_count, recv_pos, recv_count, &d, &o);
    if (st != MEP_OK) return st;
    // sizes whose workspace exceeds the static array are refused
    if (ws_offsets(d).total > (size_t)MEP_PLAN_NOALLOC_SCRATCH_BYTES) return MEP_ERR_SHAPE;
    void* ws = nullptr;
    const int sst = scratch_on_current_device(&ws);
    if (sst != MEP_OK) return sst;
    // the plan's outputs do not depend on what its workspace holds on entry
    // (every value it uses is written earlier in the same call), so the
    // array needs no clearing between calls
    return plan_launch(d, (char*)ws, topk_ids, o, (hipStream_t)stream);
}
