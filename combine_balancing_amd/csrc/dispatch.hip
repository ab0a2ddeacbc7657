// mep_dispatch (pack + receive grouping) and mep_combine.
//
// Method ("MoonEP API完全参考", section 3.1 dispatch/combine; "MoonEP"
// technical overview, architecture section: rows land grouped by expert on
// the receiving rank): dispatch copies each token row into the send
// segment of every destination its routes go to, and turns the
// source-major arrival buffer into rows grouped by expert instance; combine
// sums the K returned expert outputs of each token, weighted by its scores,
// in fixed k order in fp32.
//
// All three kernels move whole bf16 rows and are HBM-bound (no
// contraction, no MFMA). Every access is a 16-byte vector and consecutive
// threads touch consecutive vectors of a row, so each wave-wide access is a
// contiguous 1 KiB segment. Outputs are written once and not re-read by
// these kernels, and inputs are read once, so loads and stores are
// non-temporal. There is no reuse between work-groups, so the
// work-group -> XCD assignment does not matter here.
//
// Launch shapes (measured on MI355X at H=7168): pack and combine are flat,
// one thread per (token, vector), pack in 256-thread work-groups and combine
// in 128-thread ones; the grouping copy runs one work-group per row, which
// reaches the read+write copy ceiling.
#include <algorithm>

#include "rows.h"

namespace mep {
namespace {

using namespace rows;

// ------------------------------------------------------------------- pack
// LDS reserved, and not used, by a pack launch, which caps the work-groups
// sharing a CU (gfx950 has 160 KiB of LDS per CU). A map that writes every
// position: 56 KiB, two work-groups. A map that skips positions (dedup,
// pruning): 40 KiB, four work-groups, which took the dsv3 dedup pack from
// 70.4-72.1 to 67.6-68.3 us (five per CU: 68.8-69.8 us, three 70.9-71.7,
// two 10 us slower than none).
// Only a launch of at least kPackCapVectors vectors (8192 work-groups) is
// capped: on smaller ones the cap leaves the GPU partly idle (random maps:
// T=512, H=7168 took 16.9 us capped against 14.5 uncapped; T=1024, H=2048
// 8.7 against 7.4; T=2048, H=7168 even; T=4096 and 8192 1.5-2.5 us faster).
constexpr size_t kPackReserveLds = 56 * 1024;
constexpr size_t kPackSkipReserveLds = 40 * 1024;
constexpr uint32_t kPackCapVectors = 2u << 20;

// send_buf[send_pos[t*K+k]] = x[t] for each k with 0 <= send_pos < nrows (the
// send buffer's row count).
// One thread per (token, vector): the token's row is read once and stored to
// each of its K send rows, one store in flight at a time (each waits for the
// previous one): fewer outstanding stores measured faster on MI355X (dsv3
// shape: 8 back-to-back stores 113 us, one at a time 104 us). Neither
// scalar position loads nor prefetching a next item per thread gained
// anything. Residency is capped through the launch's LDS reservation
// (kPackReserveLds, kPackSkipReserveLds).
template <int KT>
__global__ __launch_bounds__(kFlatThreads) void pack_flat(const u32x4* __restrict__ x,
                                                          const int* __restrict__ send_pos,
                                                          u32x4* __restrict__ send_buf,
                                                          uint32_t total, int K, int nrows,
                                                          FastDiv rowdiv) {
    const uint32_t i = blockIdx.x * kFlatThreads + threadIdx.x;
    if (i >= total) return;
    const uint32_t t = fast_div(i, rowdiv);
    const uint32_t v = i - t * rowdiv.d;
    if constexpr (KT > 0) {
        int p[KT];  // all positions first, so each store waits only for the last
#pragma unroll
        for (int k = 0; k < KT; ++k) p[k] = send_pos[(size_t)t * KT + k];
        const u32x4 w = __builtin_nontemporal_load(x + i);
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            if ((unsigned)p[k] < (unsigned)nrows)
                __builtin_nontemporal_store(w, send_buf + (size_t)p[k] * rowdiv.d + v);
            if (k + 1 < KT) __builtin_amdgcn_s_waitcnt(kWaitVmem);
        }
    } else {
        const int* sp = send_pos + (size_t)t * K;
        const u32x4 w = __builtin_nontemporal_load(x + i);
        for (int k = 0; k < K; ++k) {
            const int p = sp[k];
            if ((unsigned)p < (unsigned)nrows)
                __builtin_nontemporal_store(w, send_buf + (size_t)p * rowdiv.d + v);
            __builtin_amdgcn_s_waitcnt(kWaitVmem);
        }
    }
}

// ------------------------------------------------------------------ group
// recv_grouped[t] = recv_raw[recv_pos[t]] for t < n and 0 <= recv_pos[t] < n_raw.
// blockDim = tpr * rpb; row t = blockIdx * rpb + threadIdx / tpr.
template <int VPT>
__global__ __launch_bounds__(kMaxTpr) void group_rows(const u32x4* __restrict__ raw,
                                                      const int* __restrict__ recv_pos,
                                                      u32x4* __restrict__ out, int n, int n_raw,
                                                      int nvec, int tpr, int rpb) {
    const int r = row_in_group(tpr, rpb);
    const int tid = threadIdx.x - r * tpr;
    const int t = blockIdx.x * rpb + r;
    if (t >= n) return;
    const int from = recv_pos[t];
    if ((unsigned)from >= (unsigned)n_raw) return;
    const u32x4* src = raw + (size_t)from * nvec;
    u32x4* dst = out + (size_t)t * nvec;
    if constexpr (VPT == 1) {
        // tpr >= nvec here (one vector per thread covers the row): no loop.
        // The single-pass loop it replaces cost 2 us of 147 on the dsv3
        // grouping (probe on the real map).
        if (tid < nvec) __builtin_nontemporal_store(__builtin_nontemporal_load(src + tid), dst + tid);
    } else {
        rows::copy_row<VPT>(src, dst, nvec, tid, tpr);
    }
}

// ---------------------------------------------------------------- combine
// acc = +0; for k in order: acc = acc + score_k * y[pos_k] (each op rounded
// to fp32: built without FMA contraction). One thread per (token, vector)
// with its K loads in flight together; skipped routes load row 0 and are
// left out exactly.
template <int KT>
__global__ __launch_bounds__(kCombineThreads) void combine_flat(const u32x4* __restrict__ y, int n_y,
                                                             const int* __restrict__ send_pos,
                                                             const float* __restrict__ scores,
                                                             u32x4* __restrict__ out_bf16,
                                                             f32x4* __restrict__ out_f32,
                                                             uint32_t total, FastDiv rowdiv) {
    const uint32_t i = blockIdx.x * kCombineThreads + threadIdx.x;
    if (i >= total) return;
    const uint32_t t = fast_div(i, rowdiv);
    const uint32_t v = i - t * rowdiv.d;
    u32x4 yk[KT];
    float sc[KT];
    uint32_t use = 0;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
        const int p = send_pos[(size_t)t * KT + k];
        const bool ok = (unsigned)p < (unsigned)n_y;
        use |= (uint32_t)ok << k;
        yk[k] = __builtin_nontemporal_load(y + (size_t)(ok ? p : 0) * rowdiv.d + v);
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

// Any K up to 64 (and the case with no rows to read): one route at a time,
// in k order, loading only valid routes.
__global__ __launch_bounds__(kCombineThreads) void combine_flat_any(
    const u32x4* __restrict__ y, int n_y, const int* __restrict__ send_pos,
    const float* __restrict__ scores, u32x4* __restrict__ out_bf16, f32x4* __restrict__ out_f32,
    uint32_t total, int K, FastDiv rowdiv) {
    const uint32_t i = blockIdx.x * kCombineThreads + threadIdx.x;
    if (i >= total) return;
    const uint32_t t = fast_div(i, rowdiv);
    const uint32_t v = i - t * rowdiv.d;
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
    for (int k = 0; k < K; ++k) {
        const int p = send_pos[(size_t)t * K + k];
        if ((unsigned)p >= (unsigned)n_y) continue;
        accumulate(acc, __builtin_nontemporal_load(y + (size_t)p * rowdiv.d + v),
                   scores[(size_t)t * K + k]);
    }
    store_out(acc, out_bf16, out_f32, i);
}

// ------------------------------------------------------------------- host
void launch_group(hipStream_t s, const u32x4* raw, const int* rp, u32x4* out, int n, int n_raw,
                  int nvec) {
    // one vector per thread up to 1024 vectors (16 KiB rows), then 2, 4, 8
    int vpt = 1;
    while (vpt < 8 && nvec > kMaxTpr * vpt) vpt *= 2;
    const RowShape rs = row_shape(nvec, vpt, kMaxTpr);
    const dim3 g((n + rs.rpb - 1) / rs.rpb), b(rs.tpr * rs.rpb);
    switch (vpt) {
        case 1: hipLaunchKernelGGL(group_rows<1>, g, b, 0, s, raw, rp, out, n, n_raw, nvec, rs.tpr, rs.rpb); break;
        case 2: hipLaunchKernelGGL(group_rows<2>, g, b, 0, s, raw, rp, out, n, n_raw, nvec, rs.tpr, rs.rpb); break;
        case 4: hipLaunchKernelGGL(group_rows<4>, g, b, 0, s, raw, rp, out, n, n_raw, nvec, rs.tpr, rs.rpb); break;
        default: hipLaunchKernelGGL(group_rows<8>, g, b, 0, s, raw, rp, out, n, n_raw, nvec, rs.tpr, rs.rpb); break;
    }
}

template <int KT>
void launch_combine(hipStream_t s, const u32x4* y, int n_y, const int* sp, const float* sc,
                    u32x4* ob, f32x4* of, uint32_t total, FastDiv dv) {
    hipLaunchKernelGGL(combine_flat<KT>, dim3((total + kCombineThreads - 1) / kCombineThreads),
                       dim3(kCombineThreads), 0, s, y, n_y, sp, sc, ob, of, total, dv);
}

}  // namespace
}  // namespace mep

using namespace mep;

extern "C" int mep_dispatch(int T, int K, int H, const uint16_t* x, const int32_t* send_pos,
                            uint16_t* send_buf, int n_send, int n_recv, const int32_t* recv_pos,
                            const uint16_t* recv_raw, int n_raw, uint16_t* recv_grouped,
                            void* stream) {
    const bool do_pack = x != nullptr;
    const bool do_group = recv_raw != nullptr;
    if (!do_pack && !do_group) return (T == 0 && n_recv == 0) ? MEP_OK : MEP_ERR_PARAM;
    if (do_pack && (!send_pos || !send_buf)) return MEP_ERR_NULLPTR;
    if (do_group && (!recv_pos || !recv_grouped)) return MEP_ERR_NULLPTR;
    if (H < 8 || H > 65536 || (H % 8) != 0) return MEP_ERR_SHAPE;
    if (do_pack && (T < 0 || K < 1 || K > 64 || (long long)T * K >= (1ll << 31) ||
                    !flat_fits(T, H / 8)))
        return MEP_ERR_SHAPE;
    if (do_pack && n_send < 0) return MEP_ERR_SHAPE;
    if (do_group && (n_recv < 0 || n_raw < 0)) return MEP_ERR_SHAPE;
    if (do_pack && (!aligned16(x) || !aligned16(send_buf))) return MEP_ERR_SHAPE;
    if (do_group && (!aligned16(recv_raw) || !aligned16(recv_grouped))) return MEP_ERR_SHAPE;
    hipStream_t s = (hipStream_t)stream;
    const int nvec = H / 8;
    if (do_pack && T > 0 && n_send > 0) {
        const uint32_t total = (uint32_t)T * (uint32_t)nvec;
        const dim3 g((total + kFlatThreads - 1) / kFlatThreads), b(kFlatThreads);
        const FastDiv dv = make_fastdiv((uint32_t)nvec);
        const u32x4* xv = (const u32x4*)x;
        const int* sp = (const int*)send_pos;
        u32x4* buf = (u32x4*)send_buf;
        // The launch reserves LDS the kernel does not use, so that fewer
        // work-groups share a CU and fewer rows are being written at once.
        // When every position is written (n_send = T*K: the plain send
        // map), two per CU: on the dsv3 map pack went from 104 to 100 us,
        // and three or four per CU measured 107-109 us. Maps that skip
        // positions (dedup, pruning) leave each thread fewer stores in
        // flight and do best with four.
        const size_t plds =
            total < kPackCapVectors ? 0
            : (long long)n_send == (long long)T * K ? kPackReserveLds : kPackSkipReserveLds;
        switch (K) {
            case 1: hipLaunchKernelGGL(pack_flat<1>, g, b, plds, s, xv, sp, buf, total, K, n_send, dv); break;
            case 2: hipLaunchKernelGGL(pack_flat<2>, g, b, plds, s, xv, sp, buf, total, K, n_send, dv); break;
            case 4: hipLaunchKernelGGL(pack_flat<4>, g, b, plds, s, xv, sp, buf, total, K, n_send, dv); break;
            case 6: hipLaunchKernelGGL(pack_flat<6>, g, b, plds, s, xv, sp, buf, total, K, n_send, dv); break;
            case 8: hipLaunchKernelGGL(pack_flat<8>, g, b, plds, s, xv, sp, buf, total, K, n_send, dv); break;
            case 16: hipLaunchKernelGGL(pack_flat<16>, g, b, plds, s, xv, sp, buf, total, K, n_send, dv); break;
            default: hipLaunchKernelGGL(pack_flat<0>, g, b, plds, s, xv, sp, buf, total, K, n_send, dv); break;
        }
        MEP_LAUNCH_CHECK();
    }
    if (do_group && n_recv > 0 && n_raw > 0) {
        launch_group(s, (const u32x4*)recv_raw, (const int*)recv_pos, (u32x4*)recv_grouped,
                     n_recv, n_raw, nvec);
        MEP_LAUNCH_CHECK();
    }
    return MEP_OK;
}

extern "C" int mep_combine(int T, int K, int H, const uint16_t* y_ret, int n_y,
                           const int32_t* send_pos, const float* scores, uint16_t* out_bf16,
                           float* out_f32, void* stream) {
    if (T < 0 || K < 1 || K > 64 || n_y < 0 || H < 8 || H > 65536 || (H % 8) != 0)
        return MEP_ERR_SHAPE;
    if (T == 0) return MEP_OK;  // nothing to do; empty buffers may be NULL
    if (!y_ret || !send_pos || !scores) return MEP_ERR_NULLPTR;
    if (!out_bf16 && !out_f32) return MEP_ERR_NULLPTR;
    if ((long long)T * K >= (1ll << 31) || !flat_fits(T, H / 8)) return MEP_ERR_SHAPE;
    if (!aligned16(y_ret) || (out_bf16 && !aligned16(out_bf16)) || (out_f32 && !aligned16(out_f32)))
        return MEP_ERR_SHAPE;
    hipStream_t s = (hipStream_t)stream;
    const int nvec = H / 8;
    const u32x4* y = (const u32x4*)y_ret;
    const int* sp = (const int*)send_pos;
    u32x4* ob = (u32x4*)out_bf16;
    f32x4* of = (f32x4*)out_f32;
    const uint32_t total = (uint32_t)T * (uint32_t)nvec;
    const FastDiv dv = make_fastdiv((uint32_t)nvec);
    // with no rows to read, the generic kernel (which loads valid routes only)
    switch (n_y > 0 ? K : 0) {
        case 1: launch_combine<1>(s, y, n_y, sp, scores, ob, of, total, dv); break;
        case 2: launch_combine<2>(s, y, n_y, sp, scores, ob, of, total, dv); break;
        case 3: launch_combine<3>(s, y, n_y, sp, scores, ob, of, total, dv); break;
        case 4: launch_combine<4>(s, y, n_y, sp, scores, ob, of, total, dv); break;
        case 5: launch_combine<5>(s, y, n_y, sp, scores, ob, of, total, dv); break;
        case 6: launch_combine<6>(s, y, n_y, sp, scores, ob, of, total, dv); break;
        case 7: launch_combine<7>(s, y, n_y, sp, scores, ob, of, total, dv); break;
        case 8: launch_combine<8>(s, y, n_y, sp, scores, ob, of, total, dv); break;
        case 9: launch_combine<9>(s, y, n_y, sp, scores, ob, of, total, dv); break;
        case 10: launch_combine<10>(s, y, n_y, sp, scores, ob, of, total, dv); break;
        case 11: launch_combine<11>(s, y, n_y, sp, scores, ob, of, total, dv); break;
        case 12: launch_combine<12>(s, y, n_y, sp, scores, ob, of, total, dv); break;
        case 13: launch_combine<13>(s, y, n_y, sp, scores, ob, of, total, dv); break;
        case 14: launch_combine<14>(s, y, n_y, sp, scores, ob, of, total, dv); break;
        case 15: launch_combine<15>(s, y, n_y, sp, scores, ob, of, total, dv); break;
        case 16: launch_combine<16>(s, y, n_y, sp, scores, ob, of, total, dv); break;
        default:
            hipLaunchKernelGGL(combine_flat_any, dim3((total + kCombineThreads - 1) / kCombineThreads),
                               dim3(kCombineThreads), 0, s, y, n_y, sp, scores, ob, of, total, K, dv);
            break;
    }
    MEP_LAUNCH_CHECK();
    return MEP_OK;
}
