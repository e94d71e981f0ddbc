// Generic routing kernel: any shape inside the compiled range (E <= 1024,
// K <= 64, G <= 64), any alignment.  One wavefront routes one token row at a
// time; scores go through LDS so that group scores and the top-K can be read
// by any lane.  This is the fallback behind the shape-specialised kernels in
// route_fast.hip, and the path for odd shapes.
//
// Steps follow "[SGLang] MoE routing: token-to-expert assignment algorithms":
// scoring (sections 2 and 4), group scores and group selection (sections 3
// and 4), top-K among the kept groups (section 3), unbiased weights with
// optional renormalisation (sections 2 and 4).
#include <hip/hip_runtime.h>

#include "route_common.hpp"
#include "route_internal.h"

namespace moe_route {
namespace {

constexpr int kGenericWaves = 4;  // wavefronts per workgroup
__host__ __device__ constexpr int generic_wave_floats(int E) { return 2 * E + kMaxGroups; }

template <typename T>
__device__ __forceinline__ float load_logit(const T* p, int i);
template <>
__device__ __forceinline__ float load_logit<float>(const float* p, int i) { return p[i]; }
template <>
__device__ __forceinline__ float load_logit<uint16_t>(const uint16_t* p, int i) {
    return bf16_bits_to_float(p[i]);
}

template <typename T, bool SOFTMAX, bool TOP2>
__global__ __launch_bounds__(kGenericWaves* kWave) void route_generic_kernel(
    const T* __restrict__ logits, BiasRef bias, int64_t M, int E, int G,
    int TG, int K, int renorm, float* __restrict__ w_out, int32_t* __restrict__ id_out) {
    // per wave: unbiased scores s [E], selection scores c [E], group scores
    // [kMaxGroups], sized by E so that small expert counts fit more blocks
    extern __shared__ float s_wave[];
    const int lane = threadIdx.x % kWave;
    const int wv = threadIdx.x / kWave;
    float* sc = s_wave + (size_t)wv * generic_wave_floats(E);
    float* ch = sc + E;
    float* gh = ch + E;
    const int gs = E / G;

    for (int64_t row = (int64_t)blockIdx.x * kGenericWaves + wv; row < M;
         row += (int64_t)gridDim.x * kGenericWaves) {
        const T* xr = logits + row * E;

        // ---- scores s and selection scores c = s + bias
        if (SOFTMAX) {
            float mx = -INFINITY;
            for (int e = lane; e < E; e += kWave) mx = fmaxf(mx, load_logit(xr, e));
            mx = wave_max_all(mx);
            float sum = 0.f;
            for (int e = lane; e < E; e += kWave) {
                float u = fast_exp2((load_logit(xr, e) - mx) * kLog2e);
                sc[e] = u;
                sum += u;
            }
            sum = wave_sum_all(sum);
            for (int e = lane; e < E; e += kWave) {
                float s = sc[e] / sum;
                sc[e] = s;
                ch[e] = s + (bias.p ? bias_at(bias, e) : 0.f);
            }
        } else {
            for (int e = lane; e < E; e += kWave) {
                float s = sigmoid_f32(load_logit(xr, e));
                sc[e] = s;
                ch[e] = s + (bias.p ? bias_at(bias, e) : 0.f);
            }
        }
        wave_lds_sync();

        // ---- group scores (max or top-2 sum), then keep the best TG groups
        uint64_t kept = 1;
        if (G > 1) {
            for (int g = lane; g < G; g += kWave) {
                float m1 = -INFINITY, m2 = -INFINITY;
                for (int j = 0; j < gs; ++j) {
                    float v = ch[g * gs + j];
                    if (v > m1) { m2 = m1; m1 = v; }
                    else if (v > m2) { m2 = v; }
                }
                gh[g] = TOP2 ? m1 + m2 : m1;
            }
            wave_lds_sync();
            bool keep = false;
            if (lane < G) {
                const float h = gh[lane];
                int rank = 0;
                for (int g = 0; g < G; ++g) rank += beats(gh[g], g, h, lane) ? 1 : 0;
                keep = rank < TG;
            }
            kept = __ballot(keep);
        }

        // ---- top-K among the kept groups, K rounds of a wave-wide argmax
        float my_w = 0.f;
        int my_id = 0;
        for (int k = 0; k < K; ++k) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
            for (int e = lane; e < E; e += kWave) {
                if (!((kept >> (e / gs)) & 1ull)) continue;
                float v = ch[e];
                if (beats(v, e, bv, bi)) { bv = v; bi = e; }
            }
            wave_argmax_all(bv, bi);
            // bi keeps its sentinel only when no candidate beats -inf (NaN
            // scores): the output is then unspecified, but stays inside the row
            bi = min(max(bi, 0), E - 1);
            if (lane == k) { my_id = bi; my_w = sc[bi]; }
            if (lane == (bi % kWave)) ch[bi] = -INFINITY;  // taken
            wave_lds_sync();
        }

        // ---- weights: unbiased scores, optionally renormalised
        float tot = wave_sum_all(lane < K ? my_w : 0.f);
        if (lane < K) {
            w_out[row * K + lane] = renorm ? my_w / tot : my_w;
            id_out[row * K + lane] = my_id;
        }
        wave_lds_sync();
    }
}

template <typename T, bool SOFTMAX, bool TOP2>
route_status_t launch_generic_t(const RouteProblem& p) {
    int64_t blocks = (p.M + kGenericWaves - 1) / kGenericWaves;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL((route_generic_kernel<T, SOFTMAX, TOP2>), dim3((unsigned)blocks),
                       dim3(kGenericWaves * kWave),
                       sizeof(float) * kGenericWaves * generic_wave_floats(p.E), p.stream,
                       static_cast<const T*>(p.logits), p.bias, p.M, p.E, p.G, p.TG, p.K,
                       p.renorm ? 1 : 0, p.weights, p.ids);
    return hipGetLastError() == hipSuccess ? ROUTE_OK : ROUTE_ELAUNCH;
}

template <typename T>
route_status_t launch_generic_dtype(const RouteProblem& p) {
    const bool soft = p.scoring == ROUTE_SOFTMAX;
    const bool top2 = p.rule == ROUTE_GROUP_TOP2_SUM;
    if (soft) return top2 ? launch_generic_t<T, true, true>(p) : launch_generic_t<T, true, false>(p);
    return top2 ? launch_generic_t<T, false, true>(p) : launch_generic_t<T, false, false>(p);
}

}  // namespace

route_status_t launch_route_generic(const RouteProblem& p) {
    if (p.dtype == ROUTE_F32) return launch_generic_dtype<float>(p);
    return launch_generic_dtype<uint16_t>(p);
}

}  // namespace moe_route
