// int8 dispatch: the pack with dynamic quantization of every routed row.
//
// Method ("aclnnMoeDistributeDispatchSetup" op doc, interface description
// and parameter notes): token rows may be quantized before they are sent;
// dynamic quantization can take optional per-expert smoothing scales; each
// token message is Align512(Align32(H) + 4) bytes: H int8 values, padding to
// a multiple of 32, one 4-byte scale. The pages give no formula; this
// library computes symmetric per-route int8 quantization in fp32:
//   v[h] = float(x[t,h])  or  fl(float(x[t,h]) * smooth[e,h])
//   s    = fl(amax_h |v[h]| / 127)
//   q[h] = rint(fl(v[h] / s)) clamped to [-127, 127], ties to even
//          (q = 0 everywhere when s == 0)
// Message row send_pos[t*K+k] gets q in bytes [0, H) and s at byte
// Align32(H); other bytes of the row are not written.
//
// One work-group per token (several per group for short rows), as the fused
// norm: each thread holds up to 2 units of 1 or 2 adjacent 16-byte vectors
// (8 or 16 values) of the row, the row's amax is reduced by a wave shuffle
// tree and across waves through LDS, and each thread writes its units'
// codes (8 or 16 bytes each, so a wave writes 512 B or 1 KiB contiguous) to
// each of the token's K message rows. Without smoothing one
// reduction serves all K routes; with it, each route has its own.
// HBM-bound: S*H*2 bytes read, C*(H+4) written.
//
// mep_group_quant is the receive side: message rows in arrival order become
// the expert-side layout, int8 rows [n, H] grouped by instance plus one fp32
// scale per row.
#include <algorithm>

#include "rows.h"

namespace mep {
namespace {

using namespace rows;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQuantThreads = 1024;
constexpr int kQuantMaxNv = 2;  // units per thread: H <= 2 * 1024 * 8 = 16384 (W = 1)

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
    return v;
}

// max of `a` over the row's waves; s_red holds one slot per wave of the group
__device__ __forceinline__ float row_max(float a, float* s_red, int r, int wpr) {
    a = wave_max(a);
    if (lane_id() == 0) s_red[threadIdx.x / kWave] = a;
    lds_barrier();
    float m = 0.0f;
    for (int q = 0; q < wpr; ++q) m = fmaxf(m, s_red[r * wpr + q]);
    return m;
}

// 8 fp32 values -> 8 int8 codes packed little-endian into two words
__device__ __forceinline__ void quantize8(const float* v, float s, uint32_t* o) {
    o[0] = o[1] = 0u;
    if (s > 0.0f) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float q = __builtin_rintf(v[j] / s);
            q = fminf(fmaxf(q, -127.0f), 127.0f);
            o[j >> 2] |= ((uint32_t)(int32_t)q & 0xffu) << (8 * (j & 3));
        }
    }
}

template <int W>
struct Codes;  // the store type of W vectors' codes (8 bytes per vector)
template <>
struct Codes<1> {
    typedef u32x2 type;
};
template <>
struct Codes<2> {
    typedef u32x4 type;
};

// A thread owns NU units of W adjacent 16-byte vectors (W = 2 when the row
// has an even number of vectors: 16 values -> one 16-byte code store).
template <int W, int NU, bool SMOOTH>
__global__ __launch_bounds__(kQuantThreads) void quant_pack_rows(
    const u32x4* __restrict__ x, const float* __restrict__ smooth, int E,
    const int* __restrict__ route_expert, const int* __restrict__ send_pos, int n_rows,
    uint8_t* __restrict__ msgs, int msg_bytes, int hq, int T, int K, int nvec, int tpr, int rpb) {
    typedef typename Codes<W>::type CT;
    constexpr int NV = W * NU;
    __shared__ float s_red[2][kQuantThreads / kWave];
    const int r = row_in_group(tpr, rpb);
    const int tid = threadIdx.x - r * tpr;
    const int t_raw = blockIdx.x * rpb + r;
    const bool live = t_raw < T;
    const int t = live ? t_raw : T - 1;  // rows past T load a real row, store nothing
    const int wpr = tpr / kWave;
    const int nunits = nvec / W;

    // vector index of slot (unit i, part w); units past the row are clamped
    // for loads and skipped for stores
    auto vec_of = [&](int i, int w) { return min(i * tpr + tid, nunits - 1) * W + w; };
    auto unit_ok = [&](int i) { return i * tpr + tid < nunits; };

    float v[NV][8];
#pragma unroll
    for (int i = 0; i < NU; ++i)
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const u32x4 q = __builtin_nontemporal_load(x + (size_t)t * nvec + vec_of(i, w));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[i * W + w][2 * j] = __uint_as_float(q[j] << 16);
                v[i * W + w][2 * j + 1] = __uint_as_float(q[j] & 0xffff0000u);
            }
        }

    if constexpr (!SMOOTH) {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < NU; ++i)
            if (unit_ok(i))
#pragma unroll
                for (int w = 0; w < W; ++w)
#pragma unroll
                    for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(v[i * W + w][j]));
        const float s = row_max(a, s_red[0], r, wpr) / 127.0f;
        CT q[NU];
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            uint32_t o[2 * W];
#pragma unroll
            for (int w = 0; w < W; ++w) quantize8(v[i * W + w], s, o + 2 * w);
#pragma unroll
            for (int j = 0; j < 2 * W; ++j) q[i][j] = o[j];
        }
        if (!live) return;
        for (int k = 0; k < K; ++k) {
            const int p = send_pos[(size_t)t * K + k];
            if ((unsigned)p >= (unsigned)n_rows) continue;
            CT* row = (CT*)(msgs + (size_t)p * msg_bytes);
#pragma unroll
            for (int i = 0; i < NU; ++i)
                if (unit_ok(i)) __builtin_nontemporal_store(q[i], row + i * tpr + tid);
            if (tid == 0) __builtin_nontemporal_store(s, (float*)((uint8_t*)row + hq));
        }
    } else {
        for (int k = 0; k < K; ++k) {
            const int p = send_pos[(size_t)t * K + k];
            const int e = route_expert[(size_t)t * K + k];
            const bool use = (unsigned)p < (unsigned)n_rows && (unsigned)e < (unsigned)E;
            const float* sm = smooth + (size_t)(use ? e : 0) * (nvec * 8);
            float wv[NV][8];
            float a = 0.0f;
#pragma unroll
            for (int i = 0; i < NU; ++i)
#pragma unroll
                for (int w = 0; w < W; ++w) {
                    const int vi = vec_of(i, w);
                    const f32x4 s0 = *(const f32x4*)(sm + (size_t)vi * 8);
                    const f32x4 s1 = *(const f32x4*)(sm + (size_t)vi * 8 + 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        wv[i * W + w][j] = v[i * W + w][j] * s0[j];
                        wv[i * W + w][4 + j] = v[i * W + w][4 + j] * s1[j];
                    }
                    if (unit_ok(i))
#pragma unroll
                        for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(wv[i * W + w][j]));
                }
            // one reduction per route; alternating LDS slots make one
            // barrier per route enough
            const float s = row_max(a, s_red[k & 1], r, wpr) / 127.0f;
            if (!live || !use) continue;
            CT* row = (CT*)(msgs + (size_t)p * msg_bytes);
#pragma unroll
            for (int i = 0; i < NU; ++i) {
                if (!unit_ok(i)) continue;
                uint32_t o[2 * W];
#pragma unroll
                for (int w = 0; w < W; ++w) quantize8(wv[i * W + w], s, o + 2 * w);
                CT c;
#pragma unroll
                for (int j = 0; j < 2 * W; ++j) c[j] = o[j];
                __builtin_nontemporal_store(c, row + i * tpr + tid);
            }
            if (tid == 0) __builtin_nontemporal_store(s, (float*)((uint8_t*)row + hq));
        }
    }
}

// x_q[t] = codes of message recv_pos[t], scales[t] = its scale. One
// work-group per row, as the bf16 grouping copy; the unit U is 16 bytes when
// rows of H bytes stay 16-byte aligned (H % 16 == 0) and 8 bytes otherwise,
// and thread 0 copies the scale. (A flat launch, one thread per (row, unit),
// measured 1 us slower at H = 7168.)
template <typename U, int VPT>
__global__ __launch_bounds__(kMaxTpr) void quant_group_rows(
    const uint8_t* __restrict__ msgs, int msg_bytes, int hq, int n_msgs,
    const int* __restrict__ recv_pos, U* __restrict__ x_q, float* __restrict__ scales, int n,
    int nunits, int tpr, int rpb) {
    const int r = row_in_group(tpr, rpb);
    const int tid = threadIdx.x - r * tpr;
    const int t = blockIdx.x * rpb + r;
    if (t >= n) return;
    const int from = recv_pos[t];
    if ((unsigned)from >= (unsigned)n_msgs) return;
    const uint8_t* m = msgs + (size_t)from * msg_bytes;
    const U* src = (const U*)m;
    U* dst = x_q + (size_t)t * nunits;
    if constexpr (VPT == 1) {
        // one unit per thread covers the row: no loop (as in group_rows)
        if (tid < nunits) __builtin_nontemporal_store(__builtin_nontemporal_load(src + tid), dst + tid);
    } else {
        rows::copy_row<VPT>(src, dst, nunits, tid, tpr);
    }
    if (tid == 0) scales[t] = *(const float*)(m + hq);
}

template <typename U>
void launch_group_quant_rows(hipStream_t s, const uint8_t* msgs, int msg_bytes, int hq,
                             int n_msgs, const int* rp, U* xq, float* sc, int n, int nunits) {
    int vpt = 1;
    while (vpt < 8 && nunits > kMaxTpr * vpt) vpt *= 2;
    const RowShape rs = row_shape(nunits, vpt, kMaxTpr);
    const dim3 g((n + rs.rpb - 1) / rs.rpb), b(rs.tpr * rs.rpb);
#define MEP_QG_LAUNCH(V)                                                                        \
    hipLaunchKernelGGL((quant_group_rows<U, V>), g, b, 0, s, msgs, msg_bytes, hq, n_msgs, rp, xq, \
                       sc, n, nunits, rs.tpr, rs.rpb)
    switch (vpt) {
        case 1: MEP_QG_LAUNCH(1); break;
        case 2: MEP_QG_LAUNCH(2); break;
        case 4: MEP_QG_LAUNCH(4); break;
        default: MEP_QG_LAUNCH(8); break;
    }
#undef MEP_QG_LAUNCH
}

}  // namespace
}  // namespace mep

using namespace mep;
using namespace mep::rows;

extern "C" size_t mep_quant_msg_bytes(int H) {
    if (H < 1) return 0;
    const size_t hq = ((size_t)H + 31) / 32 * 32;
    return (hq + 4 + 511) / 512 * 512;
}

extern "C" int mep_dispatch_quant(int T, int K, int H, const uint16_t* x, const float* smooth,
                                  int E, const int32_t* route_expert, const int32_t* send_pos,
                                  int n_rows, int msg_bytes, uint8_t* send_msgs, void* stream) {
    const int hq = (H + 31) / 32 * 32;
    if (T < 0 || K < 1 || K > 64 || H < 8 || H > kQuantMaxNv * kQuantThreads * 8 || (H % 8) != 0 ||
        n_rows < 0 || msg_bytes < hq + 4 || (msg_bytes % 16) != 0 ||
        (long long)T * K >= (1ll << 31))
        return MEP_ERR_SHAPE;
    if (smooth && (!route_expert || E < 1)) return MEP_ERR_PARAM;
    if (T == 0 || n_rows == 0) return MEP_OK;
    if (!x || !send_pos || !send_msgs) return MEP_ERR_NULLPTR;
    if (!aligned16(x) || !aligned16(send_msgs) || (smooth && !aligned16(smooth)))
        return MEP_ERR_SHAPE;
    const int nvec = H / 8;
    const int W = (nvec % 2) == 0 ? 2 : 1;  // 16 values per thread unit when possible
    const int nunits = nvec / W;
    const int nu = std::min(kQuantMaxNv, std::max(1, (nunits + kQuantThreads - 1) / kQuantThreads));
    const RowShape rsh = row_shape(nunits, nu, kQuantThreads);
    const dim3 g((T + rsh.rpb - 1) / rsh.rpb), b(rsh.tpr * rsh.rpb);
    hipStream_t s = (hipStream_t)stream;
    const u32x4* xv = (const u32x4*)x;
    const int* re = (const int*)route_expert;
    const int* sp = (const int*)send_pos;
#define MEP_QUANT_LAUNCH(WW, N, SM)                                                               \
    hipLaunchKernelGGL((quant_pack_rows<WW, N, SM>), g, b, 0, s, xv, smooth, E, re, sp, n_rows,  \
                       send_msgs, msg_bytes, hq, T, K, nvec, rsh.tpr, rsh.rpb)
    if (W == 2) {
        if (smooth) {
            if (nu == 1) MEP_QUANT_LAUNCH(2, 1, true); else MEP_QUANT_LAUNCH(2, 2, true);
        } else {
            if (nu == 1) MEP_QUANT_LAUNCH(2, 1, false); else MEP_QUANT_LAUNCH(2, 2, false);
        }
    } else {
        if (smooth) {
            if (nu == 1) MEP_QUANT_LAUNCH(1, 1, true); else MEP_QUANT_LAUNCH(1, 2, true);
        } else {
            if (nu == 1) MEP_QUANT_LAUNCH(1, 1, false); else MEP_QUANT_LAUNCH(1, 2, false);
        }
    }
#undef MEP_QUANT_LAUNCH
    MEP_LAUNCH_CHECK();
    return MEP_OK;
}

extern "C" int mep_group_quant(int n, int H, int msg_bytes, const int32_t* recv_pos, int n_msgs,
                               const uint8_t* recv_msgs, uint8_t* x_q, float* scales,
                               void* stream) {
    const int hq = (H + 31) / 32 * 32;
    if (n < 0 || H < 8 || H > 65536 || (H % 8) != 0 || n_msgs < 0 || msg_bytes < hq + 4 ||
        (msg_bytes % 16) != 0 || (long long)n * (H / 8) >= (1ll << 31))
        return MEP_ERR_SHAPE;
    if (n == 0) return MEP_OK;
    if (!recv_pos || !x_q || !scales || (n_msgs > 0 && !recv_msgs)) return MEP_ERR_NULLPTR;
    if ((recv_msgs && !aligned16(recv_msgs)) || ((uintptr_t)x_q & 7u) || ((uintptr_t)scales & 3u))
        return MEP_ERR_SHAPE;
    const bool wide = (H % 16) == 0 && aligned16(x_q);
    const int unit = wide ? 16 : 8;
    hipStream_t s = (hipStream_t)stream;
    if (wide)
        launch_group_quant_rows(s, recv_msgs, msg_bytes, hq, n_msgs, (const int*)recv_pos,
                                (u32x4*)x_q, scales, n, H / unit);
    else
        launch_group_quant_rows(s, recv_msgs, msg_bytes, hq, n_msgs, (const int*)recv_pos,
                                (u32x2*)x_q, scales, n, H / unit);
    MEP_LAUNCH_CHECK();
    return MEP_OK;
}
