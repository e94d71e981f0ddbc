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

// DPP lane permutations (wave64 rows of 16 lanes) and the row reductions
// built on them.
constexpr int kDppXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppXor3 = 0x1B;     // quad_perm [3,2,1,0]
constexpr int kDppMirror8 = 0x141; // row_half_mirror: lane i <-> 7 - i within 8
constexpr int kDppRowMirror = 0x140;  // row_mirror: lane i <-> 15 - i within 16
constexpr int kDppRowShl1 = 0x101;    // row_shl:1: lane i reads lane i + 1 within 16

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
// A plain DPP move for values that are compared rather than combined (the
// form above folds into the combining instruction; this one needs no zeroed
// old value).  Every control used here (quad_perm, row_half_mirror) reads a
// lane of the same row for every lane, so no lane keeps an old value.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov_u32(uint32_t v) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

// Reductions over the LPR lanes of a row (LPR <= 16, rows aligned to 16
// lanes); every lane of the row gets the same bits (xor/mirror butterflies
// combine the same operands in each lane).
template <int LPR>
constexpr bool row_width_ok = LPR == 1 || LPR == 2 || LPR == 4 || LPR == 8 || LPR == 16;
template <int LPR>
__device__ __forceinline__ float row_max(float v) {
    static_assert(row_width_ok<LPR>, "row width");
    if (LPR >= 2) v = fmaxf(v, dpp_f32<kDppXor1>(v));
    if (LPR >= 4) v = fmaxf(v, dpp_f32<kDppXor2>(v));
    if (LPR >= 8) v = fmaxf(v, dpp_f32<kDppMirror8>(v));
    if (LPR >= 16) v = fmaxf(v, dpp_f32<kDppRowMirror>(v));
    return v;
}
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
    static_assert(row_width_ok<LPR>, "row width");
    if (LPR >= 2) v = v + dpp_f32<kDppXor1>(v);
    if (LPR >= 4) v = v + dpp_f32<kDppXor2>(v);
    if (LPR >= 8) v = v + dpp_f32<kDppMirror8>(v);
    if (LPR >= 16) v = v + dpp_f32<kDppRowMirror>(v);
    return v;
}
template <int LPR>
__device__ __forceinline__ float row_min(float v) {
    static_assert(row_width_ok<LPR>, "row width");
    if (LPR >= 2) v = fminf(v, dpp_f32<kDppXor1>(v));
    if (LPR >= 4) v = fminf(v, dpp_f32<kDppXor2>(v));
    if (LPR >= 8) v = fminf(v, dpp_f32<kDppMirror8>(v));
    if (LPR >= 16) v = fminf(v, dpp_f32<kDppRowMirror>(v));
    return v;
}
template <int LPR>
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
    static_assert(row_width_ok<LPR>, "row width");
    if (LPR >= 2) v = max(v, dpp_u32<kDppXor1>(v));
    if (LPR >= 4) v = max(v, dpp_u32<kDppXor2>(v));
    if (LPR >= 8) v = max(v, dpp_u32<kDppMirror8>(v));
    if (LPR >= 16) v = max(v, dpp_u32<kDppRowMirror>(v));
    return v;
}
// Row argmax over (value desc, index asc) pairs.
template <int LPR>
__device__ __forceinline__ void row_argmax(float& v, int& i) {
    static_assert(row_width_ok<LPR>, "row width");
#define MOE_ROUTE_ARGMAX_STEP(CTRL)                                   \
    {                                                                 \
        float ov = dpp_f32<CTRL>(v);                                  \
        int oi = static_cast<int>(dpp_u32<CTRL>(static_cast<uint32_t>(i))); \
        if (beats(ov, oi, v, i)) { v = ov; i = oi; }                  \
    }
    if (LPR >= 2) MOE_ROUTE_ARGMAX_STEP(kDppXor1)
    if (LPR >= 4) MOE_ROUTE_ARGMAX_STEP(kDppXor2)
    if (LPR >= 8) MOE_ROUTE_ARGMAX_STEP(kDppMirror8)
    if (LPR >= 16) MOE_ROUTE_ARGMAX_STEP(kDppRowMirror)
#undef MOE_ROUTE_ARGMAX_STEP
}

// Inclusive prefix sum over the 64 lanes of a wave, on DPP: shifts by 1, 2,
// 4 and 8 lanes within each row of 16 (lanes without a source add the zero
// old value), then each row's total carried into the next rows by the
// row_bcast:15 and row_bcast:31 broadcasts (GFX9 DPP).
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr1, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr2, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr4, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr8, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast15, 0xA, 0xF, false);  // rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast31, 0xC, 0xF, false);  // rows 2, 3
    return x;
}

// Whole-wave reductions (every lane holds the same result), on the VALU: DPP
// within each row of 16 lanes, then the four row results through SGPRs, added
// or compared in a fixed order.
__device__ __forceinline__ float lane_f32(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_min_all(float v) {
    v = row_min<16>(v);
    return fminf(fminf(lane_f32(v, 0), lane_f32(v, 16)), fminf(lane_f32(v, 32), lane_f32(v, 48)));
}
__device__ __forceinline__ float wave_max_all(float v) {
    v = row_max<16>(v);
    return fmaxf(fmaxf(lane_f32(v, 0), lane_f32(v, 16)), fmaxf(lane_f32(v, 32), lane_f32(v, 48)));
}

__device__ __forceinline__ float wave_sum_all(float v) {
    v = row_sum<16>(v);
    return (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
}
// Arg-max over the wave by (value desc, index asc).
__device__ __forceinline__ void wave_argmax_all(float& v, int& i) {
    row_argmax<16>(v, i);
    float bv = lane_f32(v, 0);
    int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        const float ov = lane_f32(v, 16 * r);
        const int oi = __builtin_amdgcn_readlane(i, 16 * r);
        if (beats(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    v = bv;
    i = bi;
}

}  // namespace moe_route
