// Device helpers shared by the routing kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "route_internal.h"

namespace moe_route {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Entry i of a correction bias, widened to fp32 (exactly, for bf16).
__device__ __forceinline__ float bias_at(const BiasRef& b, int i) {
    return b.bf16 ? bf16_bits_to_float(static_cast<const uint16_t*>(b.p)[i])
                  : static_cast<const float*>(b.p)[i];
}
// Entries 4i .. 4i+3 of a correction bias: one 16-byte load (fp32) or one
// 8-byte load (bf16, widened exactly).
__device__ __forceinline__ float4 bias4_at(const BiasRef& b, int i) {
    if (b.bf16) {
        const uint2 u = static_cast<const uint2*>(b.p)[i];
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
    }
    return static_cast<const float4*>(b.p)[i];
}

// v_exp_f32 computes 2^x; v_rcp_f32 is the hardware reciprocal (1 ulp).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// sigmoid(x) = 1 / (1 + e^-x), with e^-x = 2^(-x log2 e).
__device__ __forceinline__ float sigmoid_f32(float x) {
    return fast_rcp(1.0f + fast_exp2(x * -kLog2e));
}

// e^v in double precision, for the rare re-ranking of near-tied picks (a
// relative error near 1e-14 is far more than that needs): Cody and Waite's
// reduction v = n ln2 + r (ln2 split into its nearest float, so that n * hi
// is exact, and the float nearest the remainder), then e^r = (e^(r/64))^64
// with the Taylor series of e^(r/64) to degree 6.  With |r/64| below 0.017
// every coefficient can be a float value (its rounding, times (r/64)^3 or
// smaller, stays below 1e-13), so all constants are 32-bit literals and no
// register holds a 64-bit constant.  Arguments are clamped to the range
// where e^v is finite and normal.
__device__ __forceinline__ double exp_f64(double v) {
    v = fmin(fmax(v, -708.0), 709.0);
    const double n = rint(v * (double)1.44269502f);  // ~1/ln2; n may be off by one
    const double r = fma(-n, (double)-1.90465421e-09f,  // ~ln2 - hi
                         fma(-n, (double)0.693147182f, v));  // hi: float nearest ln2
    const double q = r * 0.015625;  // r / 64, exact
    double p = (double)(1.0f / 720.0f);
    p = fma(p, q, (double)(1.0f / 120.0f));
    p = fma(p, q, (double)(1.0f / 24.0f));
    p = fma(p, q, (double)(1.0f / 6.0f));
    p = fma(p, q, 0.5);
    p = fma(p, q, 1.0);
    p = fma(p, q, 1.0);
#pragma unroll
    for (int k = 0; k < 6; ++k) p *= p;
    return ldexp(p, static_cast<int>(n));
}

// sigmoid in double precision: 1 / (1 + e^-x), correctly rounded division.
__device__ __forceinline__ double sigmoid_f64(double x) { return 1.0 / (1.0 + exp_f64(-x)); }

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
