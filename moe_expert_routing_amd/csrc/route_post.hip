// Post-routing steps on a routing result, in place (gfx950).  Both are a
// single pass over the [M, K] outputs.  KP lanes serve one row (KP = the
// power of two >= K, at most 64), lane j holding slot j, so that a row's loads
// and stores are contiguous across lanes.
//
// Shared-expert slot ("[SGLang] MoE routing: token-to-expert assignment
// algorithms", section 6): the last slot of every row gets the caller's
// shared-expert id (the page draws it at random; the caller supplies the
// draw), and with a routed scaling factor its weight becomes the sum of the
// row's other weights divided by that factor.  The sum is a butterfly over
// the row's lanes: a fixed order, so results do not depend on timing.
//
// Ascending ids: each row's (id, weight) pairs reordered by expert id, equal
// ids in slot order.  A pair's new slot is its rank: the number of pairs in
// the row with a smaller id, or the same id and an earlier slot, counted by
// reading every pair of the row through lane shuffles.  Every pair is loaded
// before any is stored.
#include <hip/hip_runtime.h>

#include "route_common.hpp"
#include "route_internal.h"

namespace moe_route {
namespace {

constexpr int kPostThreads = 256;

template <int KP>
__global__ __launch_bounds__(kPostThreads) void fuse_shared_kernel(
    float* __restrict__ w, int32_t* __restrict__ ids, int64_t M, int K,
    const int32_t* __restrict__ shared_ids, float rsf) {
    const int j = threadIdx.x % KP;
    const int64_t m = (int64_t)blockIdx.x * (kPostThreads / KP) + threadIdx.x / KP;
    const bool row = m < M;
    float v = row && j < K - 1 ? w[m * K + j] : 0.0f;
#pragma unroll
    for (int o = KP / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, KP);
    if (row && j == K - 1) {
        ids[m * K + j] = shared_ids[m];
        if (rsf != 0.0f) w[m * K + j] = v / rsf;  // IEEE division (no fast-math)
    }
}

template <int KP>
__global__ __launch_bounds__(kPostThreads) void sort_ids_kernel(float* __restrict__ w,
                                                                int32_t* __restrict__ ids,
                                                                int64_t M, int K) {
    const int j = threadIdx.x % KP;
    const int64_t m = (int64_t)blockIdx.x * (kPostThreads / KP) + threadIdx.x / KP;
    const bool own = m < M && j < K;
    const int32_t d = own ? ids[m * K + j] : 0x7fffffff;
    const float v = own ? w[m * K + j] : 0.0f;
    int rank = 0;
    for (int i = 0; i < K; ++i) {
        const int32_t di = __shfl(d, i, KP);
        rank += (di < d || (di == d && i < j)) ? 1 : 0;
    }
    if (own) {
        ids[m * K + rank] = d;
        w[m * K + rank] = v;
    }
}

template <template <int> class Kern, typename... Args>
route_status_t launch_kp(int K, int64_t M, hipStream_t stream, Args... args) {
    auto go = [&](auto kernel, int kp) {
        const int64_t rows = kPostThreads / kp;
        hipLaunchKernelGGL(kernel, dim3((unsigned)((M + rows - 1) / rows)), dim3(kPostThreads), 0,
                           stream, args...);
    };
    static_assert(kMaxTopK <= kWave, "one lane per slot");
    if (K <= 2) go(Kern<2>::fn, 2);
    else if (K <= 4) go(Kern<4>::fn, 4);
    else if (K <= 8) go(Kern<8>::fn, 8);
    else if (K <= 16) go(Kern<16>::fn, 16);
    else if (K <= 32) go(Kern<32>::fn, 32);
    else go(Kern<64>::fn, 64);
    return hipGetLastError() == hipSuccess ? ROUTE_OK : ROUTE_ELAUNCH;
}

template <int KP> struct SharedK { static constexpr auto fn = fuse_shared_kernel<KP>; };
template <int KP> struct SortK { static constexpr auto fn = sort_ids_kernel<KP>; };

}  // namespace

route_status_t launch_fuse_shared(float* w, int32_t* ids, int64_t M, int K,
                                  const int32_t* shared_ids, float rsf, hipStream_t stream) {
    return launch_kp<SharedK>(K, M, stream, w, ids, M, K, shared_ids, rsf);
}

route_status_t launch_sort_ids(float* w, int32_t* ids, int64_t M, int K, hipStream_t stream) {
    return launch_kp<SortK>(K, M, stream, w, ids, M, K);
}

}  // namespace moe_route
