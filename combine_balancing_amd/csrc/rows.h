// Row-moving helpers shared by the dispatch, combine and peer kernels
// (gfx950, wave64). A row is H bf16 values = H/8 16-byte vectors.
#pragma once

#include "mep_device.h"

namespace mep {
namespace rows {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Launch shapes (chosen by measurement on MI355X at H=7168):
//  - pack: one wave per token; the row (up to 16 vectors per lane) is loaded
//    once and each vector is stored to the K destinations back to back.
//  - group and combine: one work-group per row (per token for combine),
//    each thread owning VPT vectors of it, so a whole 14 KiB row is in flight
//    at once; small rows share a work-group (RPB rows per group).
constexpr int kPackThreads = 256;
constexpr int kPackRows = kPackThreads / kWave;
constexpr int kMaxVpl = 16;
constexpr int kMaxTpr = 1024;
constexpr int kCombineThreads = 256;  // K*VPT row loads in flight need the VGPRs

__device__ __forceinline__ int wave_row() {
    return __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kPackRows + threadIdx.x / kWave));
}

__device__ __forceinline__ void accumulate(float* acc, u32x4 w, float s) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        acc[2 * j] = acc[2 * j] + s * __uint_as_float(w[j] << 16);
        acc[2 * j + 1] = acc[2 * j + 1] + s * __uint_as_float(w[j] & 0xffff0000u);
    }
}

__device__ __forceinline__ void store_out(const float* acc, u32x4* __restrict__ out_bf16,
                                          f32x4* __restrict__ out_f32, size_t at) {
    if (out_bf16) {
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = float_to_bf16_bits(acc[2 * j]) | (float_to_bf16_bits(acc[2 * j + 1]) << 16);
        __builtin_nontemporal_store(o, out_bf16 + at);
    }
    if (out_f32) {
        const f32x4 a = {acc[0], acc[1], acc[2], acc[3]};
        const f32x4 b = {acc[4], acc[5], acc[6], acc[7]};
        __builtin_nontemporal_store(a, out_f32 + at * 2);
        __builtin_nontemporal_store(b, out_f32 + at * 2 + 1);
    }
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Threads per row for `vpt` vectors per thread: a multiple of the wave size,
// at most 1024; rows per work-group so that small rows still fill 256 threads.
struct RowShape {
    int tpr, rpb;
};

inline RowShape row_shape(int nvec, int vpt, int max_tpr) {
    int tpr = (nvec + vpt - 1) / vpt;
    tpr = (tpr + kWave - 1) / kWave * kWave;
    if (tpr > max_tpr) tpr = max_tpr;
    int rpb = 256 / tpr;
    if (rpb < 1) rpb = 1;
    return {tpr, rpb};
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

}  // namespace rows
}  // namespace mep
