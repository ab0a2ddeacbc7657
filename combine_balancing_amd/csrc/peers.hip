// Zero-copy dispatch and combine, and the expert-side return.
//
// Method ("MoonEP" technical overview, architecture section): tokens are
// written straight to their final position on the receiving rank, already
// grouped by expert instance, and the application works on views of that
// buffer; the combine side reads expert outputs where they are. With the
// plan's global (destination, slot) of every route, a rank can therefore
// write each of its rows into the destination's grouped buffer directly
// (no send buffer, no receive-side grouping) and later read each returned
// expert output from the destination's grouped output buffer.
//
// The destination buffers are named by a device array of R row pointers
// (peer memory mapped into this process on a multi-GPU system; on one GPU,
// slices of one allocation). mep_ungroup is the return step of the
// non-zero-copy path: grouped expert outputs back to arrival order.
//
// Kernel shapes follow the pack, combine and grouping kernels (flat, one
// thread per (token, vector), for the push and the pull; one work-group per
// row for the ungroup); all three are HBM-bound row movers.
#include <algorithm>

#include "rows.h"

namespace mep {
namespace {

using namespace rows;

// R <= 1024, mep_plan's rank limit. The pull copies the R-entry table of
// source buffers to LDS in every work-group: a route's row address is then
// one LDS read after its index loads instead of a dependent global load
// (101 -> 90 us at the dsv3 shape). The push keeps the global table: its
// stores do not wait on the address, and the copy's barrier cost more.
constexpr int kStagePeers = 1024;

// LDS reserved, and not used, by every push launch: of gfx950's 160 KiB per
// CU, 40 KiB leaves room for four work-groups. Fewer rows are then being
// written at once: the dsv3 push went from 105.9-106.9 to 101.6-101.8 us.
// Five work-groups per CU measured 102.6-104.5 us, three 113 us, and two
// (the pack's cap) 40 us slower. As for the pack, launches of fewer than
// kPushCapVectors vectors (8192 work-groups) are not capped: on small grids
// the cap leaves the GPU partly idle.
constexpr size_t kPushReserveLds = 40 * 1024;
constexpr uint32_t kPushCapVectors = 2u << 20;

// peers[route_dest[t*K+k]][route_slot[t*K+k]] = x[t] for every valid route.
// One thread per (token, vector), as the pack: the row is read once and
// stored to each of the K destinations.
template <int KT>
__global__ __launch_bounds__(kFlatThreads) void push_flat(const u32x4* __restrict__ x,
                                                          const int* __restrict__ rdest,
                                                          const int* __restrict__ rslot,
                                                          u32x4* const* __restrict__ peers,
                                                          uint32_t total, int K, int R, int C,
                                                          FastDiv rowdiv) {
    const uint32_t i = blockIdx.x * kFlatThreads + threadIdx.x;
    if (i >= total) return;
    const uint32_t t = fast_div(i, rowdiv);
    const uint32_t v = i - t * rowdiv.d;
    const int kk = KT > 0 ? KT : K;
    const u32x4 w = __builtin_nontemporal_load(x + i);
#pragma unroll
    for (int k = 0; k < kk; ++k) {
        const int d = rdest[(size_t)t * kk + k];
        const int sl = rslot[(size_t)t * kk + k];
        if ((unsigned)d < (unsigned)R && (unsigned)sl < (unsigned)C)
            __builtin_nontemporal_store(w, peers[d] + (size_t)sl * rowdiv.d + v);
    }
}

// out[t] = sum over k in order of score * peers[dest][slot], fp32, from +0.
// One thread per (token, vector) with its K loads in flight together;
// skipped routes read row 0 of rank 0's buffer and are left out exactly.
template <int KT>
__global__ __launch_bounds__(kFlatThreads) void pull_flat(
    const u32x4* const* __restrict__ peers, const int* __restrict__ rdest,
    const int* __restrict__ rslot, const float* __restrict__ scores, u32x4* __restrict__ out_bf16,
    f32x4* __restrict__ out_f32, uint32_t total, int R, int C, FastDiv rowdiv) {
    __shared__ const u32x4* s_peer[kStagePeers];
    for (int r = threadIdx.x; r < R; r += kFlatThreads) s_peer[r] = peers[r];
    __syncthreads();
    const uint32_t i = blockIdx.x * kFlatThreads + threadIdx.x;
    if (i >= total) return;
    const uint32_t t = fast_div(i, rowdiv);
    const uint32_t v = i - t * rowdiv.d;
    u32x4 yk[KT];
    float sc[KT];
    uint32_t use = 0;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
        const int d = rdest[(size_t)t * KT + k];
        const int sl = rslot[(size_t)t * KT + k];
        const bool ok = (unsigned)d < (unsigned)R && (unsigned)sl < (unsigned)C;
        use |= (uint32_t)ok << k;
        const u32x4* src = ok ? s_peer[d] + (size_t)sl * rowdiv.d : s_peer[0];
        yk[k] = __builtin_nontemporal_load(src + v);
        sc[k] = scores[(size_t)t * KT + k];
    }
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int k = 0; k < KT; ++k)
        if ((use >> k) & 1u) accumulate(acc, yk[k], sc[k]);
    store_out(acc, out_bf16, out_f32, i);
}

// Any K up to 64: one route at a time, in k order, loading valid routes only.
__global__ __launch_bounds__(kFlatThreads) void pull_flat_any(
    const u32x4* const* __restrict__ peers, const int* __restrict__ rdest,
    const int* __restrict__ rslot, const float* __restrict__ scores, u32x4* __restrict__ out_bf16,
    f32x4* __restrict__ out_f32, uint32_t total, int K, int R, int C, FastDiv rowdiv) {
    const uint32_t i = blockIdx.x * kFlatThreads + threadIdx.x;
    if (i >= total) return;
    const uint32_t t = fast_div(i, rowdiv);
    const uint32_t v = i - t * rowdiv.d;
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
    for (int k = 0; k < K; ++k) {
        const int d = rdest[(size_t)t * K + k];
        const int sl = rslot[(size_t)t * K + k];
        if ((unsigned)d >= (unsigned)R || (unsigned)sl >= (unsigned)C) continue;
        accumulate(acc, __builtin_nontemporal_load(peers[d] + (size_t)sl * rowdiv.d + v),
                   scores[(size_t)t * K + k]);
    }
    store_out(acc, out_bf16, out_f32, i);
}

// y_arrival[recv_pos[t]] = y_grouped[t]: the inverse of the grouping.
template <int VPT>
__global__ __launch_bounds__(kMaxTpr) void ungroup_rows(const u32x4* __restrict__ in,
                                                        const int* __restrict__ pos,
                                                        u32x4* __restrict__ out, int n, int nvec,
                                                        int tpr, int rpb) {
    const int r = row_in_group(tpr, rpb);
    const int tid = threadIdx.x - r * tpr;
    const int t = blockIdx.x * rpb + r;
    if (t >= n) return;
    const int to = pos[t];
    if ((unsigned)to >= (unsigned)n) return;
    const u32x4* src = in + (size_t)t * nvec;
    u32x4* dst = out + (size_t)to * nvec;
    if constexpr (VPT == 1) {
        // one vector per thread covers the row (as in group_rows)
        if (tid < nvec) __builtin_nontemporal_store(__builtin_nontemporal_load(src + tid), dst + tid);
    } else {
        rows::copy_row<VPT>(src, dst, nvec, tid, tpr);
    }
}

template <int KT>
void launch_pull(hipStream_t s, const u32x4* const* peers, const int* rd, const int* rs,
                 const float* sc, u32x4* ob, f32x4* of, uint32_t total, int R, int C,
                 FastDiv dv) {
    hipLaunchKernelGGL(pull_flat<KT>, dim3((total + kFlatThreads - 1) / kFlatThreads),
                       dim3(kFlatThreads), 0, s, peers, rd, rs, sc, ob, of, total, R, C, dv);
}

}  // namespace
}  // namespace mep

using namespace mep;
using namespace mep::rows;

extern "C" int mep_dispatch_to_peers(int T, int K, int H, int R, int C, const uint16_t* x,
                                     const int32_t* route_dest, const int32_t* route_slot,
                                     uint16_t* const* peer_bufs, void* stream) {
    if (T < 0 || K < 1 || K > 64 || H < 8 || H > 65536 || (H % 8) != 0 || R < 1 ||
        R > kStagePeers || C < 1 ||
        (long long)T * K >= (1ll << 31) || !flat_fits(T, H / 8))
        return MEP_ERR_SHAPE;
    if (T == 0) return MEP_OK;
    if (!x || !route_dest || !route_slot || !peer_bufs) return MEP_ERR_NULLPTR;
    if (!aligned16(x)) return MEP_ERR_SHAPE;
    const uint32_t total = (uint32_t)T * (uint32_t)(H / 8);
    const dim3 g((total + kFlatThreads - 1) / kFlatThreads), b(kFlatThreads);
    const FastDiv dv = make_fastdiv((uint32_t)(H / 8));
    hipStream_t s = (hipStream_t)stream;
    const u32x4* xv = (const u32x4*)x;
    const int* rd = (const int*)route_dest;
    const int* rs = (const int*)route_slot;
    u32x4* const* p = (u32x4* const*)peer_bufs;
    const size_t plds = total < kPushCapVectors ? 0 : kPushReserveLds;
    switch (K) {
        case 1: hipLaunchKernelGGL(push_flat<1>, g, b, plds, s, xv, rd, rs, p, total, K, R, C, dv); break;
        case 2: hipLaunchKernelGGL(push_flat<2>, g, b, plds, s, xv, rd, rs, p, total, K, R, C, dv); break;
        case 4: hipLaunchKernelGGL(push_flat<4>, g, b, plds, s, xv, rd, rs, p, total, K, R, C, dv); break;
        case 6: hipLaunchKernelGGL(push_flat<6>, g, b, plds, s, xv, rd, rs, p, total, K, R, C, dv); break;
        case 8: hipLaunchKernelGGL(push_flat<8>, g, b, plds, s, xv, rd, rs, p, total, K, R, C, dv); break;
        case 16: hipLaunchKernelGGL(push_flat<16>, g, b, plds, s, xv, rd, rs, p, total, K, R, C, dv); break;
        default: hipLaunchKernelGGL(push_flat<0>, g, b, plds, s, xv, rd, rs, p, total, K, R, C, dv); break;
    }
    MEP_LAUNCH_CHECK();
    return MEP_OK;
}

extern "C" int mep_combine_from_peers(int T, int K, int H, int R, int C,
                                      const uint16_t* const* peer_bufs,
                                      const int32_t* route_dest, const int32_t* route_slot,
                                      const float* scores, uint16_t* out_bf16, float* out_f32,
                                      void* stream) {
    if (T < 0 || K < 1 || K > 64 || H < 8 || H > 65536 || (H % 8) != 0 || R < 1 ||
        R > kStagePeers || C < 1 ||
        (long long)T * K >= (1ll << 31) || !flat_fits(T, H / 8))
        return MEP_ERR_SHAPE;
    if (T == 0) return MEP_OK;
    if (!peer_bufs || !route_dest || !route_slot || !scores) return MEP_ERR_NULLPTR;
    if (!out_bf16 && !out_f32) return MEP_ERR_NULLPTR;
    if ((out_bf16 && !aligned16(out_bf16)) || (out_f32 && !aligned16(out_f32))) return MEP_ERR_SHAPE;
    hipStream_t s = (hipStream_t)stream;
    const u32x4* const* p = (const u32x4* const*)peer_bufs;
    const int* rd = (const int*)route_dest;
    const int* rs = (const int*)route_slot;
    u32x4* ob = (u32x4*)out_bf16;
    f32x4* of = (f32x4*)out_f32;
    const uint32_t total = (uint32_t)T * (uint32_t)(H / 8);
    const FastDiv dv = make_fastdiv((uint32_t)(H / 8));
    switch (K) {
        case 1: launch_pull<1>(s, p, rd, rs, scores, ob, of, total, R, C, dv); break;
        case 2: launch_pull<2>(s, p, rd, rs, scores, ob, of, total, R, C, dv); break;
        case 4: launch_pull<4>(s, p, rd, rs, scores, ob, of, total, R, C, dv); break;
        case 6: launch_pull<6>(s, p, rd, rs, scores, ob, of, total, R, C, dv); break;
        case 8: launch_pull<8>(s, p, rd, rs, scores, ob, of, total, R, C, dv); break;
        case 16: launch_pull<16>(s, p, rd, rs, scores, ob, of, total, R, C, dv); break;
        default:
            hipLaunchKernelGGL(pull_flat_any, dim3((total + kFlatThreads - 1) / kFlatThreads),
                               dim3(kFlatThreads), 0, s, p, rd, rs, scores, ob, of, total, K, R,
                               C, dv);
            break;
    }
    MEP_LAUNCH_CHECK();
    return MEP_OK;
}

extern "C" int mep_ungroup(int n, int H, const int32_t* recv_pos, const uint16_t* y_grouped,
                           uint16_t* y_arrival, void* stream) {
    if (n < 0 || H < 8 || H > 65536 || (H % 8) != 0) return MEP_ERR_SHAPE;
    if (n == 0) return MEP_OK;
    if (!recv_pos || !y_grouped || !y_arrival) return MEP_ERR_NULLPTR;
    if (!aligned16(y_grouped) || !aligned16(y_arrival)) return MEP_ERR_SHAPE;
    const int nvec = H / 8;
    int vpt = 1;
    while (vpt < 8 && nvec > kMaxTpr * vpt) vpt *= 2;
    const RowShape rsh = row_shape(nvec, vpt, kMaxTpr);
    const dim3 g((n + rsh.rpb - 1) / rsh.rpb), b(rsh.tpr * rsh.rpb);
    hipStream_t s = (hipStream_t)stream;
    const u32x4* in = (const u32x4*)y_grouped;
    const int* pos = (const int*)recv_pos;
    u32x4* out = (u32x4*)y_arrival;
    switch (vpt) {
        case 1: hipLaunchKernelGGL(ungroup_rows<1>, g, b, 0, s, in, pos, out, n, nvec, rsh.tpr, rsh.rpb); break;
        case 2: hipLaunchKernelGGL(ungroup_rows<2>, g, b, 0, s, in, pos, out, n, nvec, rsh.tpr, rsh.rpb); break;
        case 4: hipLaunchKernelGGL(ungroup_rows<4>, g, b, 0, s, in, pos, out, n, nvec, rsh.tpr, rsh.rpb); break;
        default: hipLaunchKernelGGL(ungroup_rows<8>, g, b, 0, s, in, pos, out, n, nvec, rsh.tpr, rsh.rpb); break;
    }
    MEP_LAUNCH_CHECK();
    return MEP_OK;
}
