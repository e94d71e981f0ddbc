// Post-routing steps on a routing result, in place (gfx950).  One thread per
// token row; both are a single pass over the [M, K] outputs.
//
// Shared-expert slot ("[SGLang] MoE routing: token-to-expert assignment
// algorithms", section 6): the last slot of every row gets the caller's
// shared-expert id (the page draws it at random; the caller supplies the
// draw), and with a routed scaling factor its weight becomes the sum of the
// row's other weights divided by that factor.
//
// Ascending ids: each row's (id, weight) pairs reordered by expert id, equal
// ids in slot order.  A pair's new slot is its rank: the number of pairs in
// the row with a smaller id, or the same id and an earlier slot.  Every pair
// of the row is loaded before any is stored, and each pair is stored straight
// to its slot (no register indexed at run time): one thread per row for
// K <= 16, one lane per pair for longer rows.
#include <hip/hip_runtime.h>

#include "route_common.cuh"
#include "route_internal.h"

namespace moe_route {
namespace {

constexpr int kPostThreads = 256;

__global__ __launch_bounds__(kPostThreads) void fuse_shared_kernel(
    float* __restrict__ w, int32_t* __restrict__ ids, int64_t M, int K,
    const int32_t* __restrict__ shared_ids, float rsf) {
    const int64_t m = (int64_t)blockIdx.x * kPostThreads + threadIdx.x;
    if (m >= M) return;
    float* wr = w + m * K;
    ids[m * K + (K - 1)] = shared_ids[m];
    if (rsf != 0.0f) {
        float s = 0.0f;
        for (int k = 0; k < K - 1; ++k) s += wr[k];
        wr[K - 1] = s / rsf;  // IEEE division (no fast-math)
    }
}

// K <= KMAX <= 16: one thread per row, the pairs in registers.
template <int KMAX>
__global__ __launch_bounds__(kPostThreads) void sort_ids_kernel(float* __restrict__ w,
                                                                int32_t* __restrict__ ids,
                                                                int64_t M, int K) {
    const int64_t m = (int64_t)blockIdx.x * kPostThreads + threadIdx.x;
    if (m >= M) return;
    float* wr = w + m * K;
    int32_t* dr = ids + m * K;
    int32_t d[KMAX];
    float v[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
        d[i] = i < K ? dr[i] : 0;
        v[i] = i < K ? wr[i] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
        if (i < K) {
            int rank = 0;
#pragma unroll
            for (int j = 0; j < KMAX; ++j)
                if (j < K && (d[j] < d[i] || (d[j] == d[i] && j < i))) ++rank;
            dr[rank] = d[i];
            wr[rank] = v[i];
        }
    }
}

// 16 < K <= 64: one wave per row, lane i holds pair i.
__global__ __launch_bounds__(kPostThreads) void sort_ids_wave_kernel(float* __restrict__ w,
                                                                     int32_t* __restrict__ ids,
                                                                     int64_t M, int K) {
    const int lane = threadIdx.x % kWave;
    const int64_t m = (int64_t)blockIdx.x * (kPostThreads / kWave) + threadIdx.x / kWave;
    if (m >= M) return;  // wave-uniform
    const bool own = lane < K;
    const int32_t d = own ? ids[m * K + lane] : 0x7fffffff;
    const float v = own ? w[m * K + lane] : 0.0f;
    int rank = 0;
#pragma unroll 1
    for (int j = 0; j < K; ++j) {
        const int32_t dj = __shfl(d, j, kWave);
        rank += (dj < d || (dj == d && j < lane)) ? 1 : 0;
    }
    if (own) {
        ids[m * K + rank] = d;
        w[m * K + rank] = v;
    }
}

}  // namespace

route_status_t launch_fuse_shared(float* w, int32_t* ids, int64_t M, int K,
                                  const int32_t* shared_ids, float rsf, hipStream_t stream) {
    const int64_t blocks = (M + kPostThreads - 1) / kPostThreads;
    hipLaunchKernelGGL(fuse_shared_kernel, dim3((unsigned)blocks), dim3(kPostThreads), 0, stream,
                       w, ids, M, K, shared_ids, rsf);
    return hipGetLastError() == hipSuccess ? ROUTE_OK : ROUTE_ELAUNCH;
}

route_status_t launch_sort_ids(float* w, int32_t* ids, int64_t M, int K, hipStream_t stream) {
    const dim3 grid((unsigned)((M + kPostThreads - 1) / kPostThreads));
    static_assert(kMaxTopK <= kWave, "one lane per pair");
    if (K <= 8) {
        hipLaunchKernelGGL(sort_ids_kernel<8>, grid, dim3(kPostThreads), 0, stream, w, ids, M, K);
    } else if (K <= 16) {
        hipLaunchKernelGGL(sort_ids_kernel<16>, grid, dim3(kPostThreads), 0, stream, w, ids, M, K);
    } else {
        const int64_t rows_per_block = kPostThreads / kWave;
        const dim3 wgrid((unsigned)((M + rows_per_block - 1) / rows_per_block));
        hipLaunchKernelGGL(sort_ids_wave_kernel, wgrid, dim3(kPostThreads), 0, stream, w, ids, M,
                           K);
    }
    return hipGetLastError() == hipSuccess ? ROUTE_OK : ROUTE_ELAUNCH;
}

}  // namespace moe_route
