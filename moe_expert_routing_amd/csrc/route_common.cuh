// Device helpers shared by the routing kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe_route {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// v_exp_f32 computes 2^x; v_rcp_f32 is the hardware reciprocal (1 ulp).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// sigmoid(x) = 1 / (1 + e^-x), with e^-x = 2^(-x log2 e).
__device__ __forceinline__ float sigmoid_f32(float x) {
    return fast_rcp(1.0f + fast_exp2(x * -kLog2e));
}

// tanh(y) = sign(y) * (1 - 2 / (exp(2|y|) + 1)); absolute error ~1e-7, and
// exactly +-1 once exp overflows.
__device__ __forceinline__ float tanh_f32(float y) {
    const float t = fast_exp2(2.0f * kLog2e * fabsf(y));
    return copysignf(1.0f - 2.0f * fast_rcp(t + 1.0f), y);
}

// Make the LDS writes of this wave visible to its other lanes before they read.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// (value, index) order used for every selection: larger value first, equal
// values by the lower index.
__device__ __forceinline__ bool beats(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, shfl_xor(v, o));
    return v;
}

// Sum over the wave; every lane receives lane 0's total so that all lanes use
// the very same value.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += shfl_xor(v, o);
    return __shfl(v, 0, kWave);
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        float ov = shfl_xor(v, o);
        int oi = shfl_xor(i, o);
        if (beats(ov, oi, v, i)) { v = ov; i = oi; }
    }
}

}  // namespace moe_route
