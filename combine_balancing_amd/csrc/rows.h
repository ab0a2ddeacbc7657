// Row-moving helpers shared by the dispatch, combine and peer kernels
// (gfx950, wave64). A row is H bf16 values = H/8 16-byte vectors.
#pragma once

#include "mep_device.h"

namespace mep {
namespace rows {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Row-per-work-group launches (grouping copies, the fused norm): up to
// 1024 threads per row, each owning VPT vectors of it, so a whole row is in
// flight at once; short rows share a work-group (RPB rows per group).
constexpr int kMaxTpr = 1024;

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
            o[j] = bf16x2_bits(acc[2 * j], acc[2 * j + 1]);
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

// Flat launches: one thread per 16-byte vector of a [rows, nvec] block, 256
// threads per work-group, rows found by a division of the flat index. Many
// light work-groups keep more stores in flight than a few heavy ones (on
// MI355X a 256-thread, one-vector-per-thread write reaches ~6.4 TB/s where
// 896-thread row groups stay near 4.7 TB/s).
constexpr int kFlatThreads = 256;

// The flat combine (K row loads, one store per thread) runs 128-thread
// work-groups: 90.3 us against 92.6 us at 256 on the dsv3 shape (64: 90.4-91,
// 512 and 1024: 91-92.5). Pack measured no better below 256 and slower above.
constexpr int kCombineThreads = 128;

// s_waitcnt operand that waits for every outstanding vector memory operation
// (vmcnt(0)) and leaves the export and LDS/scalar counters alone (gfx9
// encoding: vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
constexpr unsigned kWaitVmem = 0x0F70;

// q = n / d for 0 <= n < 2^31 by one 64-bit multiply and a shift, with
// s = ceil(log2 d) and m = ceil(2^(32+s) / d) < 2^33: the rounding error of m
// times n stays below 2^(32+s) / d, so the quotient is exact.
struct FastDiv {
    uint64_t m;
    uint32_t s;
    uint32_t d;
};

inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    const unsigned __int128 num = (unsigned __int128)1 << (32 + s);
    return {(uint64_t)((num + d - 1) / d), s, d};
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f) {
    return (uint32_t)(((uint64_t)n * f.m) >> (32 + f.s));
}

inline bool flat_fits(long long rows, int nvec) { return rows * (long long)nvec < (1ll << 31); }

// Threads per row for `vpt` vectors per thread: a multiple of the wave size,
// at most 1024; rows per work-group so that small rows still fill 256 threads.
struct RowShape {
    int tpr, rpb;
};

// Row of this thread within its work-group. tpr is a multiple of the wave
// size, so a wave lies inside one row and the row is wave-uniform: reading
// it from the first lane makes the row's index, position and score loads
// scalar (and the row base an SGPR pair). A work-group holds several rows
// only when tpr <= 128 (row_shape), and then tpr is 64 or 128, so the row is
// a shift of the thread index; with one row per group it is 0. No integer
// division: these work-groups are short-lived, and a division in the
// prologue (about 25 dependent scalar instructions) measured 2 us slower on
// a 32768-row grouping copy.
__device__ __forceinline__ int row_in_group(int tpr, int rpb) {
    if (rpb == 1) return 0;
    return __builtin_amdgcn_readfirstlane((int)threadIdx.x) >> __builtin_ctz((unsigned)tpr);
}

// dst[v] = src[v] for v in [0, n) (n >= 1), the row's nthr threads taking
// VPT vectors each per pass, all of a pass's loads issued before its
// stores. The loads are unconditional, at indices clamped into the row (a
// lane past its end reloads the last vector and stores nothing): with each
// load under its lane condition the compiler waited for the previous load
// before issuing the next, one round trip per vector.
template <int VPT, typename T>
__device__ __forceinline__ void copy_row(const T* __restrict__ src, T* __restrict__ dst, int n,
                                         int tid, int nthr) {
    for (int v0 = 0; v0 < n; v0 += nthr * VPT) {
        T q[VPT];
#pragma unroll
        for (int i = 0; i < VPT; ++i)
            q[i] = __builtin_nontemporal_load(src + min(v0 + i * nthr + tid, n - 1));
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int v = v0 + i * nthr + tid;
            if (v < n) __builtin_nontemporal_store(q[i], dst + v);
        }
    }
}

inline RowShape row_shape(int nvec, int vpt, int max_tpr) {
    int tpr = (nvec + vpt - 1) / vpt;
    tpr = (tpr + kWave - 1) / kWave * kWave;
    if (tpr > max_tpr) tpr = max_tpr;
    int rpb = 256 / tpr;  // >= 2 only for tpr = 64 or 128 (row_in_group shifts)
    if (rpb < 1) rpb = 1;
    return {tpr, rpb};
}

}  // namespace rows
}  // namespace mep
