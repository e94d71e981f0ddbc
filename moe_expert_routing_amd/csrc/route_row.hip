// Routing of few tokens for gfx950: one wavefront per token row, 256 experts,
// sigmoid scoring (with or without a correction bias), no groups or 8 groups.
//
// The shape-specialised kernel (route_fast.hip) routes 8 rows per wave with
// 32 experts per lane; at a few tokens every wave routes one such tile alone
// on its SIMD, and the tile's serial chain sets the call's latency.  Here a
// wave routes one row with 4 experts per lane, so each lane scores 4 logits
// instead of 32 and sorts 4 keys instead of merging lists of 16 candidates.
// Nothing is staged in LDS: every exchange between lanes is a DPP move, a
// readlane or a permute.
//
// The per-row steps ("[SGLang] MoE routing: token-to-expert assignment
// algorithms", sections 3 and 4) are in route_row.hpp; this file holds the
// kernel that walks the rows and its launchers.
#include <hip/hip_runtime.h>

#include "route_common.hpp"
#include "route_internal.h"
#include "route_row.hpp"
#include "route_tile.hpp"

namespace moe_route {
namespace {

// Waves (rows) per block: one up to kRowOneWaveTokens tokens, where blocks of
// a single wave spread over more compute units and a call finishes sooner
// (64 tokens: 3.06 against 3.25 µs a call, graph replay); four above.
constexpr int kRowWaves = 4;
constexpr int64_t kRowOneWaveTokens = 1024;

template <typename T>
__device__ __forceinline__ void load_row4(const T* __restrict__ p, int lane, float (&x)[4]);
template <>
__device__ __forceinline__ void load_row4<uint16_t>(const uint16_t* __restrict__ p, int lane,
                                                    float (&x)[4]) {
    const uint2 u = reinterpret_cast<const uint2*>(p)[lane];
    x[0] = __uint_as_float(u.x << 16);
    x[1] = __uint_as_float(u.x & 0xffff0000u);
    x[2] = __uint_as_float(u.y << 16);
    x[3] = __uint_as_float(u.y & 0xffff0000u);
}
template <>
__device__ __forceinline__ void load_row4<float>(const float* __restrict__ p, int lane,
                                                 float (&x)[4]) {
    const float4 v = reinterpret_cast<const float4*>(p)[lane];
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}

template <typename T, bool BIAS, int GRP /*0 none, 1 max, 2 top-2 sum*/>
__global__ __launch_bounds__(kRowWaves* kWave) void route_row_kernel(
    const T* __restrict__ logits, BiasRef bias, int64_t M, int TG, int K, int renorm,
    float* __restrict__ w_out, int32_t* __restrict__ id_out) {
    const int lane = threadIdx.x % kWave;
    const int waves = blockDim.x / kWave;  // 1 or kRowWaves
    const int64_t stride = (int64_t)gridDim.x * waves;
    int64_t row = (int64_t)blockIdx.x * waves + threadIdx.x / kWave;

    // The row's logits are requested first (a wave past the last row loads
    // that row and leaves), then the bias (4 entries a lane).
    float x[4];
    load_row4<T>(logits + min(row, M - 1) * kRowE, lane, x);
    float off[4];
    const KeyParams kp = row_wave_key_window<BIAS>(bias, lane, off);
    if (row >= M) return;  // a whole wave; the kernel has no block barrier
    while (true) {
        const T* xr = logits + row * kRowE;
        route_row_wave<BIAS, GRP>(x, lane, bias, off, kp, TG, K, renorm, w_out + row * K,
                                  id_out + row * K, [&](int e) { return load_one<T>(xr, e); });
        row += stride;
        if (row >= M) break;
        load_row4<T>(logits + row * kRowE, lane, x);
    }
}

template <typename T, bool BIAS, int GRP>
route_status_t launch_row(const RouteProblem& p) {
    auto kernel = route_row_kernel<T, BIAS, GRP>;
    static const int resident = resident_blocks(kernel, kRowWaves * kWave);
    const int waves = p.M <= kRowOneWaveTokens ? 1 : kRowWaves;
    int64_t blocks = (p.M + waves - 1) / waves;
    const int64_t cap = (int64_t)device_cu_count() * resident * (kRowWaves / waves);
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(waves * kWave), 0, p.stream,
                       static_cast<const T*>(p.logits), p.bias, p.M, p.TG, p.K,
                       p.renorm ? 1 : 0, p.weights, p.ids);
    return hipGetLastError() == hipSuccess ? ROUTE_OK : ROUTE_ELAUNCH;
}

template <typename T, bool BIAS>
route_status_t launch_row_grp(const RouteProblem& p) {
    if (p.G == 1) return launch_row<T, BIAS, 0>(p);
    if (p.rule == ROUTE_GROUP_TOP2_SUM) return launch_row<T, BIAS, 2>(p);
    return launch_row<T, BIAS, 1>(p);
}

template <typename T>
route_status_t launch_row_bias(const RouteProblem& p) {
    return p.bias.p ? launch_row_grp<T, true>(p) : launch_row_grp<T, false>(p);
}

}  // namespace

bool route_row_supported(const RouteProblem& p) {
    return p.E == kRowE && p.scoring == ROUTE_SIGMOID && p.K <= kRowKMax &&
           (p.G == 1 || p.G == 8) && p.M <= kRowMaxTokens;
}

route_status_t launch_route_row(const RouteProblem& p) {
    return p.dtype == ROUTE_F32 ? launch_row_bias<float>(p) : launch_row_bias<uint16_t>(p);
}

}  // namespace moe_route
