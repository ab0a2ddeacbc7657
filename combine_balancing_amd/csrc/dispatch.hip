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
// contraction, no MFMA). One wave owns one row: each lane moves 16-byte
// vectors at stride 64, so every wave-wide access is a contiguous 1 KiB
// segment; a lane keeps up to 16 vectors (a 16 KiB row per wave) in flight
// before its stores. Per-row indices and scores are wave-uniform and come
// through scalar loads. Outputs are written once and not re-read by these
// kernels, so stores are non-temporal. There is no reuse between blocks,
// so the block -> XCD assignment does not matter for these kernels.
#include "mep_device.h"

namespace mep {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowThreads = 256;
constexpr int kRowsPerBlock = kRowThreads / kWave;
constexpr int kMaxVpl = 16;

__device__ __forceinline__ int wave_row() {
    return __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kRowsPerBlock + threadIdx.x / kWave));
}

// ------------------------------------------------------------------- pack
// send_buf[send_pos[t*K+k]] = x[t] for each k with 0 <= send_pos < nrows.
template <int VPL>
__global__ __launch_bounds__(kRowThreads) void pack_rows(const u32x4* __restrict__ x,
                                                         const int* __restrict__ send_pos,
                                                         u32x4* __restrict__ send_buf, int T, int K,
                                                         int nvec, int nrows) {
    const int t = wave_row();
    if (t >= T) return;
    const int lane = lane_id();
    const int my_pos = lane < K ? send_pos[(size_t)t * K + lane] : -1;
    const u32x4* src = x + (size_t)t * nvec;
    for (int v0 = 0; v0 < nvec; v0 += kWave * VPL) {
        u32x4 r[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int v = v0 + i * kWave + lane;
            if (v < nvec) r[i] = __builtin_nontemporal_load(src + v);
        }
        for (int k = 0; k < K; ++k) {
            const int pos = __builtin_amdgcn_readlane(my_pos, k);
            if ((unsigned)pos >= (unsigned)nrows) continue;
            u32x4* dst = send_buf + (size_t)pos * nvec;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int v = v0 + i * kWave + lane;
                if (v < nvec) __builtin_nontemporal_store(r[i], dst + v);
            }
        }
    }
}

// ------------------------------------------------------------------ group
// recv_grouped[t] = recv_raw[recv_pos[t]] for 0 <= recv_pos[t] < n.
template <int VPL>
__global__ __launch_bounds__(kRowThreads) void group_rows(const u32x4* __restrict__ raw,
                                                          const int* __restrict__ recv_pos,
                                                          u32x4* __restrict__ out, int n,
                                                          int nvec) {
    const int t = wave_row();
    if (t >= n) return;
    const int from = recv_pos[t];
    if ((unsigned)from >= (unsigned)n) return;
    const int lane = lane_id();
    const u32x4* src = raw + (size_t)from * nvec;
    u32x4* dst = out + (size_t)t * nvec;
    for (int v0 = 0; v0 < nvec; v0 += kWave * VPL) {
        u32x4 r[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int v = v0 + i * kWave + lane;
            if (v < nvec) r[i] = __builtin_nontemporal_load(src + v);
        }
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int v = v0 + i * kWave + lane;
            if (v < nvec) __builtin_nontemporal_store(r[i], dst + v);
        }
    }
}

// ---------------------------------------------------------------- combine
// acc = +0; for k in order: acc = acc + score_k * y[pos_k] (each op rounded
// to fp32: built without FMA contraction).
template <int KT>
__device__ __forceinline__ void combine_vec(const u32x4* __restrict__ y, const int* pos,
                                            const float* sc, int nvec, int v,
                                            u32x4* __restrict__ out_bf16,
                                            f32x4* __restrict__ out_f32, size_t t) {
    u32x4 yk[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k)
        if (pos[k] >= 0) yk[k] = __builtin_nontemporal_load(y + (size_t)pos[k] * nvec + v);
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
        if (pos[k] < 0) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t w = yk[k][j];
            acc[2 * j] = acc[2 * j] + sc[k] * __uint_as_float(w << 16);
            acc[2 * j + 1] = acc[2 * j + 1] + sc[k] * __uint_as_float(w & 0xffff0000u);
        }
    }
    if (out_bf16) {
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = float_to_bf16_bits(acc[2 * j]) | (float_to_bf16_bits(acc[2 * j + 1]) << 16);
        __builtin_nontemporal_store(o, out_bf16 + t * nvec + v);
    }
    if (out_f32) {
        const f32x4 a = {acc[0], acc[1], acc[2], acc[3]};
        const f32x4 b = {acc[4], acc[5], acc[6], acc[7]};
        __builtin_nontemporal_store(a, out_f32 + (t * nvec + v) * 2);
        __builtin_nontemporal_store(b, out_f32 + (t * nvec + v) * 2 + 1);
    }
}

template <int KT>
__global__ __launch_bounds__(kRowThreads) void combine_rows(const u32x4* __restrict__ y, int n_y,
                                                            const int* __restrict__ send_pos,
                                                            const float* __restrict__ scores,
                                                            u32x4* __restrict__ out_bf16,
                                                            f32x4* __restrict__ out_f32, int T,
                                                            int nvec) {
    const int t = wave_row();
    if (t >= T) return;
    int pos[KT];
    float sc[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
        const int p = send_pos[(size_t)t * KT + k];
        pos[k] = (unsigned)p < (unsigned)n_y ? p : -1;
        sc[k] = scores[(size_t)t * KT + k];
    }
    const int lane = lane_id();
#pragma unroll 2
    for (int v = lane; v < nvec; v += kWave)
        combine_vec<KT>(y, pos, sc, nvec, v, out_bf16, out_f32, (size_t)t);
}

// Any K up to 64: one route at a time, in k order.
__global__ __launch_bounds__(kRowThreads) void combine_rows_any(
    const u32x4* __restrict__ y, int n_y, const int* __restrict__ send_pos,
    const float* __restrict__ scores, u32x4* __restrict__ out_bf16, f32x4* __restrict__ out_f32,
    int T, int K, int nvec) {
    const int t = wave_row();
    if (t >= T) return;
    const int lane = lane_id();
    for (int v = lane; v < nvec; v += kWave) {
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
        for (int k = 0; k < K; ++k) {
            const int p = send_pos[(size_t)t * K + k];
            if ((unsigned)p >= (unsigned)n_y) continue;
            const float s = scores[(size_t)t * K + k];
            const u32x4 w4 = y[(size_t)p * nvec + v];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[2 * j] = acc[2 * j] + s * __uint_as_float(w4[j] << 16);
                acc[2 * j + 1] = acc[2 * j + 1] + s * __uint_as_float(w4[j] & 0xffff0000u);
            }
        }
        if (out_bf16) {
            u32x4 o;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[j] = float_to_bf16_bits(acc[2 * j]) | (float_to_bf16_bits(acc[2 * j + 1]) << 16);
            out_bf16[(size_t)t * nvec + v] = o;
        }
        if (out_f32) {
            const f32x4 a = {acc[0], acc[1], acc[2], acc[3]};
            const f32x4 b = {acc[4], acc[5], acc[6], acc[7]};
            out_f32[((size_t)t * nvec + v) * 2] = a;
            out_f32[((size_t)t * nvec + v) * 2 + 1] = b;
        }
    }
}

// ------------------------------------------------------------------- host
int vpl_for(int nvec) {
    const int v = (nvec + kWave - 1) / kWave;
    return v < 1 ? 1 : (v > kMaxVpl ? kMaxVpl : v);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

template <int VPL>
void launch_pack(dim3 g, hipStream_t s, const u32x4* x, const int* sp, u32x4* buf, int T, int K,
                 int nvec, int nrows) {
    hipLaunchKernelGGL(pack_rows<VPL>, g, dim3(kRowThreads), 0, s, x, sp, buf, T, K, nvec, nrows);
}

template <int VPL>
void launch_group(dim3 g, hipStream_t s, const u32x4* raw, const int* rp, u32x4* out, int n,
                  int nvec) {
    hipLaunchKernelGGL(group_rows<VPL>, g, dim3(kRowThreads), 0, s, raw, rp, out, n, nvec);
}

#define MEP_VPL_SWITCH(vpl, FN, ...)         \
    switch (vpl) {                           \
        case 1: FN<1>(__VA_ARGS__); break;   \
        case 2: FN<2>(__VA_ARGS__); break;   \
        case 3: FN<3>(__VA_ARGS__); break;   \
        case 4: FN<4>(__VA_ARGS__); break;   \
        case 5: FN<5>(__VA_ARGS__); break;   \
        case 6: FN<6>(__VA_ARGS__); break;   \
        case 7: FN<7>(__VA_ARGS__); break;   \
        case 8: FN<8>(__VA_ARGS__); break;   \
        case 9: FN<9>(__VA_ARGS__); break;   \
        case 10: FN<10>(__VA_ARGS__); break; \
        case 11: FN<11>(__VA_ARGS__); break; \
        case 12: FN<12>(__VA_ARGS__); break; \
        case 13: FN<13>(__VA_ARGS__); break; \
        case 14: FN<14>(__VA_ARGS__); break; \
        case 15: FN<15>(__VA_ARGS__); break; \
        default: FN<16>(__VA_ARGS__); break; \
    }

template <int KT>
void launch_combine(dim3 g, hipStream_t s, const u32x4* y, int n_y, const int* sp,
                    const float* sc, u32x4* ob, f32x4* of, int T, int nvec) {
    hipLaunchKernelGGL(combine_rows<KT>, g, dim3(kRowThreads), 0, s, y, n_y, sp, sc, ob, of, T,
                       nvec);
}

}  // namespace
}  // namespace mep

using namespace mep;

extern "C" int mep_dispatch(int T, int K, int H, const uint16_t* x, const int32_t* send_pos,
                            uint16_t* send_buf, int n_recv, const int32_t* recv_pos,
                            const uint16_t* recv_raw, uint16_t* recv_grouped, void* stream) {
    const bool do_pack = x != nullptr;
    const bool do_group = recv_raw != nullptr;
    if (!do_pack && !do_group) return (T == 0 && n_recv == 0) ? MEP_OK : MEP_ERR_PARAM;
    if (do_pack && (!send_pos || !send_buf)) return MEP_ERR_NULLPTR;
    if (do_group && (!recv_pos || !recv_grouped)) return MEP_ERR_NULLPTR;
    if (H < 8 || H > 65536 || (H % 8) != 0) return MEP_ERR_SHAPE;
    if (do_pack && (T < 0 || K < 1 || K > 64 || (long long)T * K >= (1ll << 31)))
        return MEP_ERR_SHAPE;
    if (do_group && n_recv < 0) return MEP_ERR_SHAPE;
    if (do_pack && (!aligned16(x) || !aligned16(send_buf))) return MEP_ERR_SHAPE;
    if (do_group && (!aligned16(recv_raw) || !aligned16(recv_grouped))) return MEP_ERR_SHAPE;
    hipStream_t s = (hipStream_t)stream;
    const int nvec = H / 8;
    const int vpl = vpl_for(nvec);
    if (do_pack && T > 0) {
        const dim3 g((T + kRowsPerBlock - 1) / kRowsPerBlock);
        MEP_VPL_SWITCH(vpl, launch_pack, g, s, (const u32x4*)x, (const int*)send_pos,
                       (u32x4*)send_buf, T, K, nvec, T * K);
        MEP_LAUNCH_CHECK();
    }
    if (do_group && n_recv > 0) {
        const dim3 g((n_recv + kRowsPerBlock - 1) / kRowsPerBlock);
        MEP_VPL_SWITCH(vpl, launch_group, g, s, (const u32x4*)recv_raw, (const int*)recv_pos,
                       (u32x4*)recv_grouped, n_recv, nvec);
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
    if ((long long)T * K >= (1ll << 31)) return MEP_ERR_SHAPE;
    if (!aligned16(y_ret) || (out_bf16 && !aligned16(out_bf16)) || (out_f32 && !aligned16(out_f32)))
        return MEP_ERR_SHAPE;
    hipStream_t s = (hipStream_t)stream;
    const int nvec = H / 8;
    const dim3 g((T + kRowsPerBlock - 1) / kRowsPerBlock);
    const u32x4* y = (const u32x4*)y_ret;
    const int* sp = (const int*)send_pos;
    u32x4* ob = (u32x4*)out_bf16;
    f32x4* of = (f32x4*)out_f32;
    switch (K) {
        case 1: launch_combine<1>(g, s, y, n_y, sp, scores, ob, of, T, nvec); break;
        case 2: launch_combine<2>(g, s, y, n_y, sp, scores, ob, of, T, nvec); break;
        case 3: launch_combine<3>(g, s, y, n_y, sp, scores, ob, of, T, nvec); break;
        case 4: launch_combine<4>(g, s, y, n_y, sp, scores, ob, of, T, nvec); break;
        case 5: launch_combine<5>(g, s, y, n_y, sp, scores, ob, of, T, nvec); break;
        case 6: launch_combine<6>(g, s, y, n_y, sp, scores, ob, of, T, nvec); break;
        case 7: launch_combine<7>(g, s, y, n_y, sp, scores, ob, of, T, nvec); break;
        case 8: launch_combine<8>(g, s, y, n_y, sp, scores, ob, of, T, nvec); break;
        case 9: launch_combine<9>(g, s, y, n_y, sp, scores, ob, of, T, nvec); break;
        case 10: launch_combine<10>(g, s, y, n_y, sp, scores, ob, of, T, nvec); break;
        case 11: launch_combine<11>(g, s, y, n_y, sp, scores, ob, of, T, nvec); break;
        case 12: launch_combine<12>(g, s, y, n_y, sp, scores, ob, of, T, nvec); break;
        case 13: launch_combine<13>(g, s, y, n_y, sp, scores, ob, of, T, nvec); break;
        case 14: launch_combine<14>(g, s, y, n_y, sp, scores, ob, of, T, nvec); break;
        case 15: launch_combine<15>(g, s, y, n_y, sp, scores, ob, of, T, nvec); break;
        case 16: launch_combine<16>(g, s, y, n_y, sp, scores, ob, of, T, nvec); break;
        default:
            hipLaunchKernelGGL(combine_rows_any, g, dim3(kRowThreads), 0, s, y, n_y, sp, scores,
                               ob, of, T, K, nvec);
            break;
    }
    MEP_LAUNCH_CHECK();
    return MEP_OK;
}
