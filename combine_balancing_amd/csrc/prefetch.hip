// Weight rows of the planned instances under a cap of B prefetch slots.
//
// Method ("MoonEP" technical overview, memory contract): the group GEMM
// reads its weights from one [E+B, H, H'] tensor whose rows 0..E-1 are the
// experts of all ranks and rows E..E+B-1 a rank's prefetch slots; training
// uses B = E/R, inference a smaller B (3-4), and redundant experts beyond
// the slots are served from their home rank. With the plan's local layout
// (rank u's natives first, in ascending expert order, zero-row natives
// included; then its redundant instances in ascending expert order), local
// index i of rank u reads
//   row e              if i < n_nat(u)            (native)
//   row E + (i - n_nat) if i - n_nat(u) < B       (prefetched copy)
//   row e              otherwise                  (home rank's weights)
// where n_nat(u) = first(u+1) - first(u), first(u) = ceil(u*E/R) being the
// first expert with home rank u (home(e) = floor(e*R/E)).
//
// Latency only: R work-groups of up to 1024 threads, one per local index.
#include "mep_device.h"

namespace mep {
namespace {

__device__ __forceinline__ int first_native(int u, int R, int E) {
    return (int)(((long long)u * E + R - 1) / R);
}

__global__ __launch_bounds__(1024) void weight_rows_kernel(int R, int E, int B,
                                                           const int* __restrict__ inst_count,
                                                           const int* __restrict__ inst_expert,
                                                           int* __restrict__ wrow) {
    const int u = blockIdx.x;
    const int n = inst_count[u];
    const int nat = first_native(u + 1, R, E) - first_native(u, R, E);
    for (int i = threadIdx.x; i < E; i += blockDim.x) {
        int w = -1;
        if (i < n) {
            const int e = inst_expert[(size_t)u * E + i];
            const int j = i - nat;
            w = (j < 0 || j >= B) ? e : E + j;
        }
        wrow[(size_t)u * E + i] = w;
    }
}

}  // namespace
}  // namespace mep

using namespace mep;

extern "C" int mep_plan_weight_rows(int R, int E, int B, const int32_t* inst_count,
                                    const int32_t* inst_expert, int32_t* inst_wrow,
                                    void* stream) {
    if (R < 1 || R > 1024 || E < 1 || E > 1024) return MEP_ERR_SHAPE;
    if (B < 0) return MEP_ERR_PARAM;
    if (!inst_count || !inst_expert || !inst_wrow) return MEP_ERR_NULLPTR;
    const int threads = E < 64 ? 64 : (E > 1024 ? 1024 : (E + 63) / 64 * 64);
    hipLaunchKernelGGL(weight_rows_kernel, dim3(R), dim3(threads), 0, (hipStream_t)stream, R, E,
                       B, (const int*)inst_count, (const int*)inst_expert, (int*)inst_wrow);
    MEP_LAUNCH_CHECK();
    return MEP_OK;
}
