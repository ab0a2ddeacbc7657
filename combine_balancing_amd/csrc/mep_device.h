// Device helpers shared by the mep kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mep.h"

namespace mep {

constexpr int kWave = 64;

// Lane index within the wave.
__device__ __forceinline__ int lane_id() {
    return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Number of set bits of `mask` at lanes below this one.
__device__ __forceinline__ int count_below(uint64_t mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Lanes (among `valid` ones) whose key equals this lane's key, found with one
// ballot per key bit: a wave-wide multi-split, so equal keys are ranked by
// lane order without atomics (deterministic). Keys must lie in
// [0, 2^NBITS); the loop is fully unrolled (bits above a key's width are 0
// on every lane and leave the groups unchanged). Call with the whole wave.
constexpr int kKeyBits = 10;  // keys below 1024: experts and instances

// gfx950's three-input bitwise op, truth table indexed by
// (bit of a) * 4 + (bit of b) * 2 + (bit of c): 0x90 is a & ~(b ^ c).
constexpr int kAndXnor = 0x90;

template <int NBITS = kKeyBits>
__device__ __forceinline__ uint64_t match_peers(int key, bool valid) {
    // Invalid lanes are dropped by the first ballot; the per-bit ballots need
    // not exclude them again.
    // Per bit: lb = 0 or ~0 (the lane's bit, sign-extended), m = ballot of
    // the bit; lanes agreeing with this lane on the bit are ~(m ^ lb). Each
    // half of the mask takes that in one v_bitop3, so a bit costs four
    // vector instructions (extract, compare, two bitop3) where the plain
    // expression compiled to about six.
    const uint64_t v = __ballot(valid);
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
#pragma unroll
    for (int b = 0; b < NBITS; ++b) {
        uint32_t lb = (uint32_t)__builtin_amdgcn_sbfe((int)key, b, 1);
        // opaque, so the ballot compares lb itself (seen through, it is
        // rebuilt from a shift of the key: one more instruction per bit)
        asm("" : "+v"(lb));
        const uint64_t m = __ballot(lb != 0u);
        lo = __builtin_amdgcn_bitop3_b32(lo, (uint32_t)m, lb, kAndXnor);
        hi = __builtin_amdgcn_bitop3_b32(hi, (uint32_t)(m >> 32), lb, kAndXnor);
    }
    return ((uint64_t)hi << 32) | lo;
}

// Work-group barrier for LDS data: waits for this wave's LDS (and scalar)
// operations, then meets the other waves. Unlike __syncthreads() it does not
// wait for outstanding global stores, so a phase that writes outputs does
// not stall the next one; use it only where no thread reads global memory
// that another thread of the work-group wrote in the same launch. The memory
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Inclusive sum over the wave (lanes 0..lane). Within each row of 16 lanes a
// Kogge-Stone scan uses DPP row shifts (ALU-speed cross-lane moves; lanes
// whose source falls outside the row read 0); the three row totals are then
// read as scalars and added to the later rows. Call with the whole wave
// active.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    const int row = lane_id() >> 4;
    const int r0 = __builtin_amdgcn_readlane(x, 15);
    const int r1 = __builtin_amdgcn_readlane(x, 31);
    const int r2 = __builtin_amdgcn_readlane(x, 47);
    return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Exclusive block-wide sum. `scratch` holds at least blockDim/64 + 1 ints of
// LDS. Every thread of the block must call it (it uses lds_barrier). Returns
// the exclusive prefix; *total receives the block sum. CLOSE = false leaves
// out the closing barrier that lets the next call reuse `scratch`: the
// caller then alternates two scratch buffers between consecutive calls (a
// call's two barriers keep the buffer of the call before it from being
// rewritten while it is still read).
template <bool CLOSE = true>
__device__ __forceinline__ int block_exclusive_sum(int v, int* scratch, int* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nw = (blockDim.x + kWave - 1) / kWave;
    const int inc = wave_inclusive_sum(v);
    if (lane == kWave - 1 || (int)threadIdx.x == (int)blockDim.x - 1) scratch[wave] = inc;
    lds_barrier();
    if (wave == 0) {
        const int w = lane < nw ? scratch[lane] : 0;
        const int s = wave_inclusive_sum(w);
        if (lane < nw) scratch[lane] = s - w;
        if (lane == nw - 1) scratch[nw] = s;
    }
    lds_barrier();
    const int res = inc - v + scratch[wave];
    *total = scratch[nw];
    if (CLOSE) lds_barrier();
    return res;
}

// Two exclusive block-wide sums with one pair of barriers. `scratch` holds
// at least 2*(blockDim/64 + 1) ints of LDS. CLOSE as for block_exclusive_sum.
template <bool CLOSE = true>
__device__ __forceinline__ void block_exclusive_sum2(int a, int b, int* scratch, int* ea, int* eb,
                                                     int* ta, int* tb) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nw = (blockDim.x + kWave - 1) / kWave;
    int* sa = scratch;
    int* sb = scratch + nw + 1;
    const int ia = wave_inclusive_sum(a);
    const int ib = wave_inclusive_sum(b);
    if (lane == kWave - 1 || (int)threadIdx.x == (int)blockDim.x - 1) {
        sa[wave] = ia;
        sb[wave] = ib;
    }
    lds_barrier();
    if (wave == 0) {
        const int wa = lane < nw ? sa[lane] : 0;
        const int wb = lane < nw ? sb[lane] : 0;
        const int xa = wave_inclusive_sum(wa);
        const int xb = wave_inclusive_sum(wb);
        if (lane < nw) {
            sa[lane] = xa - wa;
            sb[lane] = xb - wb;
        }
        if (lane == nw - 1) {
            sa[nw] = xa;
            sb[nw] = xb;
        }
    }
    lds_barrier();
    *ea = ia - a + sa[wave];
    *eb = ib - b + sb[wave];
    *ta = sa[nw];
    *tb = sb[nw];
    if (CLOSE) lds_barrier();
}

// Smallest index i in [0, n) with a[i] >= x (n if none).
__device__ __forceinline__ int lower_bound(const int* a, int n, int x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// Smallest index i in [0, n) with a[i] > x (n if none).
__device__ __forceinline__ int upper_bound(const int* a, int n, int x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] <= x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// Native 4 x int vector: arrays of it stay in registers, where arrays of
// HIP's int4 struct can be left on the stack (scratch memory).
typedef int i32x4 __attribute__((ext_vector_type(4)));

// dst[i] = src[i] for i in [0, n), the block's threads striding by NT. The
// loads of up to U strides are issued together before any store, so the
// copy costs one memory round trip per U strides instead of one per stride.
// T must be a scalar or a native vector type (i32x4, not int4).
template <int NT, int U, typename T>
__device__ __forceinline__ void stage(T* __restrict__ dst, const T* __restrict__ src, int n) {
    for (int base = 0; base < n; base += NT * U) {
        T v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * NT + (int)threadIdx.x;
            if (i < n) v[u] = src[i];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * NT + (int)threadIdx.x;
            if (i < n) dst[i] = v[u];
        }
    }
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) {
    return v < lo ? lo : (v > hi ? hi : v);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> one word of two bf16 (lo in the low half) with gfx950's
// v_cvt_pk_bf16_f32: round to nearest, ties to even. Checked on the MI355X
// over all 2^32 inputs against the integer rounding (u + 0x7fff + lsb) >> 16,
// with a NaN kept quiet with its sign and top payload bits
// ((u >> 16) | 0x40): bit-identical.
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

}  // namespace mep

// Host-side launch check shared by the entry points.
#define MEP_LAUNCH_CHECK()                                   \
    do {                                                     \
        if (hipGetLastError() != hipSuccess) return MEP_ERR_HIP; \
    } while (0)
