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
// norm: each thread holds NV <= 2 vectors (8 values) of the row, the row's
// amax is reduced by a wave shuffle tree and across waves through LDS, and
// each thread writes 8 code bytes per vector (a 512-byte contiguous segment
// per wave) to each of the token's K message rows. Without smoothing one
// reduction serves all K routes; with it, each route has its own.
// HBM-bound: S*H*2 bytes read, C*(H+4) written.
#include <algorithm>

#include "rows.h"

namespace mep {
namespace {

using namespace rows;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQuantThreads = 1024;
constexpr int kQuantMaxNv = 2;  // H <= 2 * 1024 * 8 = 16384

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

__device__ __forceinline__ u32x2 quantize8(const float* v, float s) {
    u32x2 o = {0u, 0u};
    if (s > 0.0f) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float q = __builtin_rintf(v[j] / s);
            q = fminf(fmaxf(q, -127.0f), 127.0f);
            o[j >> 2] |= ((uint32_t)(int32_t)q & 0xffu) << (8 * (j & 3));
        }
    }
    return o;
}

template <int NV, bool SMOOTH>
__global__ __launch_bounds__(kQuantThreads) void quant_pack_rows(
    const u32x4* __restrict__ x, const float* __restrict__ smooth, int E,
    const int* __restrict__ route_expert, const int* __restrict__ send_pos, int n_rows,
    uint8_t* __restrict__ msgs, int msg_bytes, int hq, int T, int K, int nvec, int tpr, int rpb) {
    __shared__ float s_red[2][kQuantThreads / kWave];
    const int r = row_in_group(tpr);
    const int tid = threadIdx.x - r * tpr;
    const int t_raw = blockIdx.x * rpb + r;
    const bool live = t_raw < T;
    const int t = live ? t_raw : T - 1;  // rows past T load a real row, store nothing
    const int wpr = tpr / kWave;

    float v[NV][8];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const u32x4 w = __builtin_nontemporal_load(x + (size_t)t * nvec + min(i * tpr + tid, nvec - 1));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[i][2 * j] = __uint_as_float(w[j] << 16);
            v[i][2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
    }

    if constexpr (!SMOOTH) {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (i * tpr + tid < nvec)
#pragma unroll
                for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(v[i][j]));
        const float s = row_max(a, s_red[0], r, wpr) / 127.0f;
        u32x2 q[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) q[i] = quantize8(v[i], s);
        if (!live) return;
        for (int k = 0; k < K; ++k) {
            const int p = send_pos[(size_t)t * K + k];
            if ((unsigned)p >= (unsigned)n_rows) continue;
            uint8_t* row = msgs + (size_t)p * msg_bytes;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int vi = i * tpr + tid;
                if (vi < nvec) __builtin_nontemporal_store(q[i], (u32x2*)(row + (size_t)vi * 8));
            }
            if (tid == 0) __builtin_nontemporal_store(s, (float*)(row + hq));
        }
    } else {
        for (int k = 0; k < K; ++k) {
            const int p = send_pos[(size_t)t * K + k];
            const int e = route_expert[(size_t)t * K + k];
            const bool use = (unsigned)p < (unsigned)n_rows && (unsigned)e < (unsigned)E;
            const float* sm = smooth + (size_t)(use ? e : 0) * (nvec * 8);
            float w[NV][8];
            float a = 0.0f;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int vi = min(i * tpr + tid, nvec - 1);
                const f32x4 s0 = *(const f32x4*)(sm + (size_t)vi * 8);
                const f32x4 s1 = *(const f32x4*)(sm + (size_t)vi * 8 + 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    w[i][j] = v[i][j] * s0[j];
                    w[i][4 + j] = v[i][4 + j] * s1[j];
                }
                if (i * tpr + tid < nvec)
#pragma unroll
                    for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(w[i][j]));
            }
            // one reduction per route; alternating LDS slots make one
            // barrier per route enough
            const float s = row_max(a, s_red[k & 1], r, wpr) / 127.0f;
            if (!live || !use) continue;
            uint8_t* row = msgs + (size_t)p * msg_bytes;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int vi = i * tpr + tid;
                if (vi < nvec)
                    __builtin_nontemporal_store(quantize8(w[i], s), (u32x2*)(row + (size_t)vi * 8));
            }
            if (tid == 0) __builtin_nontemporal_store(s, (float*)(row + hq));
        }
    }
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
    const int nv = std::min(kQuantMaxNv, std::max(1, (nvec + kQuantThreads - 1) / kQuantThreads));
    const RowShape rsh = row_shape(nvec, nv, kQuantThreads);
    const dim3 g((T + rsh.rpb - 1) / rsh.rpb), b(rsh.tpr * rsh.rpb);
    hipStream_t s = (hipStream_t)stream;
    const u32x4* xv = (const u32x4*)x;
    const int* re = (const int*)route_expert;
    const int* sp = (const int*)send_pos;
#define MEP_QUANT_LAUNCH(N, SM)                                                                   \
    hipLaunchKernelGGL((quant_pack_rows<N, SM>), g, b, 0, s, xv, smooth, E, re, sp, n_rows,      \
                       send_msgs, msg_bytes, hq, T, K, nvec, rsh.tpr, rsh.rpb)
    if (smooth) {
        if (nv == 1) MEP_QUANT_LAUNCH(1, true); else MEP_QUANT_LAUNCH(2, true);
    } else {
        if (nv == 1) MEP_QUANT_LAUNCH(1, false); else MEP_QUANT_LAUNCH(2, false);
    }
#undef MEP_QUANT_LAUNCH
    MEP_LAUNCH_CHECK();
    return MEP_OK;
}
