// Combine fused with the residual add and RMS normalisation that follow it.
//
// Method ("aclnnMoeUpdateExpert" op doc, call example): the combine step has
// a variant that also takes the layer's residual x and the norm's gamma and
// returns the normalised y, the per-token rstd and the summed x. The pages
// give the tensors, not the formula; this library computes the usual
// add + RMSNorm of the unrounded fp32 sum:
//   a       = combine accumulator: +0, then a = a + score_k * y_k in k order
//   x       = a + residual                                (fp32)
//   rstd    = 1 / sqrt(sum(x^2) / H + eps)   squares and sum in fp64, then
//             rounded to fp32 (the square of an fp32 value is exact in fp64
//             and never leaves its range, so the sum keeps full precision
//             for rows of any magnitude)
//   y       = (x * rstd) * gamma, rounded to bf16; x_out = bf16(x)
//
// One work-group per token (several tokens per group for short rows), up to
// 1024 threads, each keeping NV <= 2 vectors (8 values each) of its token's
// row in registers from the K-way sum through the normalisation, so the row
// is read once and written once; the sum of squares is reduced across the
// work-group through LDS. HBM-bound like the plain combine: K rows plus the
// residual read, two rows written. (Measured on MI355X at H = 7168: 896
// threads x 1 vector and 256 x 4 move the same bytes in about the same time;
// what matters is that the row index is wave-uniform, so a token's
// positions and scores come through scalar loads.)
#include <algorithm>

#include "rows.h"

namespace mep {
namespace {

using namespace rows;

constexpr int kNormThreads = 1024;
constexpr int kNormMaxNv = 2;  // H <= 2 * 1024 * 8 = 16384

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ void load_add(float* x, u32x4 w) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[2 * j] = x[2 * j] + __uint_as_float(w[j] << 16);
        x[2 * j + 1] = x[2 * j + 1] + __uint_as_float(w[j] & 0xffff0000u);
    }
}

__device__ __forceinline__ u32x4 pack_bf16(const float* a) {
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = bf16x2_bits(a[2 * j], a[2 * j + 1]);
    return o;
}

// KT = K known at compile time (its loads batched), or 0 for any K <= 64.
template <int KT, int NV>
__global__ __launch_bounds__(kNormThreads) void combine_norm_rows(
    const u32x4* __restrict__ y, int n_y, const int* __restrict__ send_pos,
    const float* __restrict__ scores, const u32x4* __restrict__ residual,
    const u32x4* __restrict__ gamma, float eps, u32x4* __restrict__ x_out,
    u32x4* __restrict__ y_out, float* __restrict__ rstd_out, int T, int K, int nvec, int tpr,
    int rpb) {
    __shared__ double s_red[kNormThreads / kWave];
    const int r = row_in_group(tpr, rpb);
    const int tid = threadIdx.x - r * tpr;
    const int t_raw = blockIdx.x * rpb + r;
    const bool live = t_raw < T;
    const int t = live ? t_raw : T - 1;  // rows past T load a real row, store nothing

    float x[NV][8];
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) x[i][j] = 0.0f;

    // The residual and gamma vectors are loaded first, with the expert rows:
    // loaded where they are used, each cost one more round trip after the
    // rows (the loads wait in issue order).
    u32x4 rv[NV], gv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int v = min(i * tpr + tid, nvec - 1);
        rv[i] = __builtin_nontemporal_load(residual + (size_t)t * nvec + v);
        gv[i] = gamma[v];
    }

    if constexpr (KT > 0) {
        int pos[KT];
        float sc[KT];
        uint32_t use = 0;
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            const int p = send_pos[(size_t)t * KT + k];
            const bool ok = (unsigned)p < (unsigned)n_y;
            use |= (uint32_t)ok << k;
            pos[k] = ok ? p : 0;
            sc[k] = scores[(size_t)t * KT + k];
        }
        constexpr int kBatch = std::max(1, std::min(NV, 32 / KT));
#pragma unroll
        for (int i0 = 0; i0 < NV; i0 += kBatch) {
            u32x4 yk[kBatch][KT];
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                if (i0 + b >= NV) break;
                const int v = min((i0 + b) * tpr + tid, nvec - 1);
#pragma unroll
                for (int k = 0; k < KT; ++k)
                    yk[b][k] = __builtin_nontemporal_load(y + (size_t)pos[k] * nvec + v);
            }
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                if (i0 + b >= NV) break;
#pragma unroll
                for (int k = 0; k < KT; ++k)
                    if ((use >> k) & 1u) accumulate(x[i0 + b], yk[b][k], sc[k]);
            }
        }
    } else {
        for (int k = 0; k < K; ++k) {
            const int p = send_pos[(size_t)t * K + k];
            if ((unsigned)p >= (unsigned)n_y) continue;
            const float s = scores[(size_t)t * K + k];
            u32x4 w[NV];
#pragma unroll
            for (int i = 0; i < NV; ++i)
                w[i] = __builtin_nontemporal_load(y + (size_t)p * nvec + min(i * tpr + tid, nvec - 1));
#pragma unroll
            for (int i = 0; i < NV; ++i) accumulate(x[i], w[i], s);
        }
    }

    // x = a + residual; sum of squares over this thread's real vectors
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        load_add(x[i], rv[i]);
        if (i * tpr + tid < nvec) {
#pragma unroll
            for (int j = 0; j < 8; ++j) ss = ss + (double)x[i][j] * (double)x[i][j];
        }
    }

    ss = wave_sum(ss);
    const int wpr = tpr / kWave;  // waves per row: each wave lies in one row
    const int w = threadIdx.x / kWave;
    if (lane_id() == 0) s_red[w] = ss;
    lds_barrier();
    double tot = 0.0;
    for (int q = 0; q < wpr; ++q) tot = tot + s_red[r * wpr + q];
    const float rstd = (float)(1.0 / sqrt(tot / (double)(nvec * 8) + (double)eps));

    if (!live) return;
    if (tid == 0 && rstd_out) rstd_out[t] = rstd;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int v = i * tpr + tid;
        if (v >= nvec) continue;
        const size_t at = (size_t)t * nvec + v;
        if (x_out) __builtin_nontemporal_store(pack_bf16(x[i]), x_out + at);
        float o[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            o[2 * j] = (x[i][2 * j] * rstd) * __uint_as_float(gv[i][j] << 16);
            o[2 * j + 1] = (x[i][2 * j + 1] * rstd) * __uint_as_float(gv[i][j] & 0xffff0000u);
        }
        __builtin_nontemporal_store(pack_bf16(o), y_out + at);
    }
}

template <int KT>
void launch_norm(hipStream_t s, int nv, dim3 g, dim3 b, const u32x4* y, int n_y, const int* sp,
                 const float* sc, const u32x4* res, const u32x4* gam, float eps, u32x4* xo,
                 u32x4* yo, float* rs, int T, int K, int nvec, int tpr, int rpb) {
#define MEP_NORM_CASE(N)                                                                       \
    case N:                                                                                    \
        hipLaunchKernelGGL((combine_norm_rows<KT, N>), g, b, 0, s, y, n_y, sp, sc, res, gam, eps, \
                           xo, yo, rs, T, K, nvec, tpr, rpb);                                  \
        break;
    switch (nv) {
        MEP_NORM_CASE(1)
        default: MEP_NORM_CASE(2)
    }
#undef MEP_NORM_CASE
}

}  // namespace
}  // namespace mep

using namespace mep;
using namespace mep::rows;

extern "C" int mep_combine_add_rmsnorm(int T, int K, int H, const uint16_t* y_ret, int n_y,
                                       const int32_t* send_pos, const float* scores,
                                       const uint16_t* residual, const uint16_t* gamma, float eps,
                                       uint16_t* x_out, uint16_t* y_out, float* rstd_out,
                                       void* stream) {
    if (T < 0 || K < 1 || K > 64 || H < 8 || H > kNormMaxNv * kNormThreads * 8 || (H % 8) != 0 ||
        n_y < 0 || (long long)T * K >= (1ll << 31))
        return MEP_ERR_SHAPE;
    if (!(eps >= 0.0f) || eps > 3.0e38f) return MEP_ERR_PARAM;
    if (T == 0) return MEP_OK;
    if (!send_pos || !scores || !residual || !gamma || !y_out) return MEP_ERR_NULLPTR;
    if (n_y > 0 && !y_ret) return MEP_ERR_NULLPTR;
    if ((y_ret && !aligned16(y_ret)) || !aligned16(residual) || !aligned16(gamma) ||
        !aligned16(y_out) || (x_out && !aligned16(x_out)))
        return MEP_ERR_SHAPE;
    const int nvec = H / 8;
    const int nv = std::min(kNormMaxNv, std::max(1, (nvec + kNormThreads - 1) / kNormThreads));
    const RowShape rsh = row_shape(nvec, nv, kNormThreads);
    const dim3 g((T + rsh.rpb - 1) / rsh.rpb), b(rsh.tpr * rsh.rpb);
    hipStream_t s = (hipStream_t)stream;
    const u32x4* y = (const u32x4*)y_ret;
    const int* sp = (const int*)send_pos;
    const u32x4* res = (const u32x4*)residual;
    const u32x4* gam = (const u32x4*)gamma;
    u32x4* xo = (u32x4*)x_out;
    u32x4* yo = (u32x4*)y_out;
    // With no rows to read (n_y == 0) the generic path, which loads only
    // valid routes, runs: the batched one reads row 0 for skipped routes.
    switch (n_y > 0 ? K : 0) {
        case 1: launch_norm<1>(s, nv, g, b, y, n_y, sp, scores, res, gam, eps, xo, yo, rstd_out, T, K, nvec, rsh.tpr, rsh.rpb); break;
        case 2: launch_norm<2>(s, nv, g, b, y, n_y, sp, scores, res, gam, eps, xo, yo, rstd_out, T, K, nvec, rsh.tpr, rsh.rpb); break;
        case 4: launch_norm<4>(s, nv, g, b, y, n_y, sp, scores, res, gam, eps, xo, yo, rstd_out, T, K, nvec, rsh.tpr, rsh.rpb); break;
        case 8: launch_norm<8>(s, nv, g, b, y, n_y, sp, scores, res, gam, eps, xo, yo, rstd_out, T, K, nvec, rsh.tpr, rsh.rpb); break;
        default: launch_norm<0>(s, nv, g, b, y, n_y, sp, scores, res, gam, eps, xo, yo, rstd_out, T, K, nvec, rsh.tpr, rsh.rpb); break;
    }
    MEP_LAUNCH_CHECK();
    return MEP_OK;
}
