// One wavefront routes one token row of 256 experts, 4 per lane: sigmoid
// scoring with or without a correction bias, no groups or 8 groups, K <= 8
// ("[SGLang] MoE routing: token-to-expert assignment algorithms", sections 3
// and 4).  The routing kernel for few tokens (route_row.hip) walks the rows.
//
//   1. s = sigmoid(x) and the selection score c = s + bias, held as its
//      fixed-point value t (the same key window and arithmetic as the
//      8-row core in route_tile.hpp, so both take the same decisions);
//   2. group g (experts 32g .. 32g+31) is lanes 8g .. 8g+7: the top two of
//      each lane, merged over the 8 lanes by three DPP butterflies, give the
//      group score (max, or sum of the top two); the 8 scores are read into
//      scalar registers and each lane counts the groups that beat its own;
//   3. every lane of a kept group sorts its 4 keys
//          key = fixed_point(c) << 9 | (511 - expert)
//      (unsigned order = c desc, expert asc) and K rounds take the wave
//      maximum of the lanes' first keys; the lane holding it moves on;
//   4. lane r takes pick r: its unbiased score comes from the lane that
//      scored it (a permute), then the optional renormalisation and stores,
//      with the 8-row core's arithmetic: both give the same bits for a row.
// A wide bias spread (key step too coarse) takes an exact (value, index)
// selection instead; adjacent picks closer than a few key steps are ranked
// again in double precision, as in the 8-row core.  Nothing is staged in
// LDS: every exchange between lanes is a DPP move, a readlane or a permute.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "route_common.hpp"
#include "route_tile.hpp"

namespace moe_route {

constexpr int kRowE = 256;    // experts: 4 per lane
constexpr int kRowKMax = 8;

// Top two of {m1 >= m2} and {o1 >= o2}: the larger first value, and as the
// second the median of (m1, o1, max(m2, o2)).
__device__ __forceinline__ void top2_merge(float& m1, float& m2, float o1, float o2) {
    const float lo = fmaxf(m2, o2);
    m2 = __builtin_amdgcn_fmed3f(m1, o1, lo);
    m1 = fmaxf(m1, o1);
}

// Largest value over the wave, in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = row_max_u32<16>(v);
    const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                           (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
    const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                           (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
    return max(a, b);
}

// Smallest and largest value over the wave, in every lane: both reductions
// at once, on integers whose signed order is the order of the floats (the
// bits, with the magnitude bits flipped for negative values).
__device__ __forceinline__ int float_order_key(float f) {
    const int b = __float_as_int(f);
    return b ^ ((b >> 31) & 0x7fffffff);
}
__device__ __forceinline__ void wave_min_max(float& mn, float& mx) {
    int a = float_order_key(mn), b = float_order_key(mx);
#define MOE_ROUTE_MINMAX_STEP(CTRL)                                            \
    a = min(a, __builtin_amdgcn_update_dpp(0, a, CTRL, 0xF, 0xF, false));      \
    b = max(b, __builtin_amdgcn_update_dpp(0, b, CTRL, 0xF, 0xF, false));
    MOE_ROUTE_MINMAX_STEP(kDppXor1)
    MOE_ROUTE_MINMAX_STEP(kDppXor2)
    MOE_ROUTE_MINMAX_STEP(kDppMirror8)
    MOE_ROUTE_MINMAX_STEP(kDppRowMirror)
#undef MOE_ROUTE_MINMAX_STEP
    a = min(min(__builtin_amdgcn_readlane(a, 0), __builtin_amdgcn_readlane(a, 16)),
            min(__builtin_amdgcn_readlane(a, 32), __builtin_amdgcn_readlane(a, 48)));
    b = max(max(__builtin_amdgcn_readlane(b, 0), __builtin_amdgcn_readlane(b, 16)),
            max(__builtin_amdgcn_readlane(b, 32), __builtin_amdgcn_readlane(b, 48)));
    mn = __int_as_float(a ^ ((a >> 31) & 0x7fffffff));
    mx = __int_as_float(b ^ ((b >> 31) & 0x7fffffff));
}

// Value of lane `src` (a lane index per lane), through the permute network.
__device__ __forceinline__ float lane_gather(float v, int src) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

// Key window of a biased call (or the fixed window without a bias) and the
// staged offsets of the lane's 4 bias entries (experts 4 lane .. 4 lane + 3).
template <bool BIAS>
__device__ __forceinline__ KeyParams row_wave_key_window(const BiasRef& bias, int lane,
                                                         float (&off)[4]) {
    KeyParams kp;
    float b[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (BIAS) {
        const float4 bq = bias4_at(bias, lane);
        b[0] = bq.x; b[1] = bq.y; b[2] = bq.z; b[3] = bq.w;
        float bmin = fminf(fminf(b[0], b[1]), fminf(b[2], b[3]));
        float bmax = fmaxf(fmaxf(b[0], b[1]), fmaxf(b[2], b[3]));
        wave_min_max(bmin, bmax);
        kp = key_params(bmin, 1.0f + bmax);
    } else {
        kp = key_params(0.0f, 1.0f);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) off[i] = BIAS ? sel_offset(b[i], kp) : 0.0f;
    return kp;
}

// Route one row: lane `lane` brings the fp32 logits x of experts 4 lane ..
// 4 lane + 3; the K weights and ids go to w_row[0..K) and id_row[0..K).
// logit_of(e) returns the row's logit of expert e (the rare near-tie path).
template <bool BIAS, int GRP /*0 none, 1 max, 2 top-2 sum*/, typename LogitFn>
__device__ __forceinline__ void route_row_wave(const float (&x)[4], const int lane,
                                               const BiasRef& bias, const float (&off)[4],
                                               const KeyParams& kp, const int TG, const int K,
                                               const int renorm, float* __restrict__ w_row,
                                               int32_t* __restrict__ id_row, LogitFn logit_of) {
    // group scores as fixed point for the max rule without a bias
    const float h_offs = (GRP == 2 ? 2.0f : 1.0f) * (kp.offs - 8388608.0f);
    const int grp = lane / 8;  // this lane's group (G = 8)
    // ---- 1. scores s and selection values t (c, or its fixed-point value)
    float s[4], t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s[i] = sigmoid_f32(x[i]);
        t[i] = BIAS ? __builtin_fmaf(s[i], kp.sel_mul, off[i]) : s[i];
    }

    // ---- 2. group scores, rank of this lane's group, kept or not
    bool kept = true;
    if constexpr (GRP != 0) {
        float m1 = fmaxf(t[0], t[1]), m2 = fminf(t[0], t[1]);
        top2_merge(m1, m2, fmaxf(t[2], t[3]), fminf(t[2], t[3]));
        if constexpr (GRP == 2) {
            top2_merge(m1, m2, dpp_f32<kDppXor1>(m1), dpp_f32<kDppXor1>(m2));
            top2_merge(m1, m2, dpp_f32<kDppXor2>(m1), dpp_f32<kDppXor2>(m2));
            top2_merge(m1, m2, dpp_f32<kDppMirror8>(m1), dpp_f32<kDppMirror8>(m2));
        } else {
            m1 = row_max<8>(m1);
        }
        int rank = 0;
        if (!kp.exact_only) {
            uint32_t hq;
            if constexpr (BIAS) {
                // t values are integers below 2^24: their bits less the
                // exponent field are the fixed-point values, added exactly
                hq = GRP == 2 ? __float_as_uint(m1) + __float_as_uint(m2) - 2u * 0x4B000000u
                              : __float_as_uint(m1) - 0x4B000000u;
            } else {
                const float h = GRP == 2 ? m1 + m2 : m1;
                hq = static_cast<uint32_t>(__builtin_fmaf(h, kp.scale, h_offs));
            }
            const uint32_t hk = (hq << 3) | static_cast<uint32_t>(7 - grp);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                rank += (uint32_t)__builtin_amdgcn_readlane((int)hk, 8 * j) > hk ? 1 : 0;
        } else {
            const float h = GRP == 2 ? m1 + m2 : m1;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                rank += beats(lane_f32(h, 8 * j), j, h, grp) ? 1 : 0;
        }
        kept = rank < TG;
    }

    // ---- 3. top-K: lane r ends with pick r (its expert in pick_e)
    int pick_e = 0;
    uint32_t pick_key = 0u;
    if (!kp.exact_only) {
        uint32_t L[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t low9 = 511u - (uint32_t)(4 * lane + i);
            const uint32_t key = BIAS ? (__float_as_uint(t[i]) << 9) | low9
                                      : make_key(t[i], kp.scale, kp.offs, low9);
            L[i] = kept ? key : 0u;  // real keys are above 4096
        }
        auto cx = [](uint32_t& a, uint32_t& c) {
            const uint32_t hi = max(a, c);
            c = min(a, c);
            a = hi;
        };
        cx(L[0], L[1]); cx(L[2], L[3]); cx(L[0], L[2]); cx(L[1], L[3]); cx(L[1], L[2]);
#pragma unroll
        for (int r = 0; r < kRowKMax; ++r) {
            if (r >= K) break;
            const uint32_t w = wave_max_u32(L[0]);
            const bool mine = L[0] == w;  // keys are unique
            L[0] = mine ? L[1] : L[0];
            L[1] = mine ? L[2] : L[1];
            L[2] = mine ? L[3] : L[2];
            L[3] = mine ? 0u : L[3];
            if (lane == r) pick_key = w;
        }
        pick_e = 511 - (int)(pick_key & 511u);
    } else {
        // exact path: K rounds of a wave argmax on (c, expert), each
        // taking the best candidate after the previous pick
        float pv = INFINITY;
        int pi = -1;
#pragma unroll 1
        for (int r = 0; r < K; ++r) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
            if (kept) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int e = 4 * lane + i;
                    if (beats(pv, pi, t[i], e) && beats(t[i], e, bv, bi)) {
                        bv = t[i];
                        bi = e;
                    }
                }
            }
            wave_argmax_all(bv, bi);
            pv = bv;
            pi = bi;
            if (lane == r) pick_e = bi;
        }
    }
    pick_e = min(max(pick_e, 0), kRowE - 1);  // never read outside the row

    // ---- exact order of near-tied adjacent picks (as in the 8-row
    // kernel: keys within kNearKeySteps key steps are re-ranked on
    // selection scores recomputed in double precision)
    int slot = lane;
    {
        constexpr uint32_t kNearKeySteps = 4;
        const uint32_t nxt = dpp_mov_u32<kDppRowShl1>(pick_key);
        const bool near = !kp.exact_only && lane + 1 < K &&
                          pick_key - nxt < ((kNearKeySteps + 1) << 9);
        if (__builtin_expect(__ballot(near) != 0ull, 0)) {
            double c64 = 0.0;
            if (lane < K)
                c64 = sigmoid_f64((double)logit_of(pick_e)) +
                      (BIAS ? (double)bias_at(bias, pick_e) : 0.0);
            int rank = 0;
#pragma unroll 1
            for (int j = 0; j < K; ++j) {
                const int lo = __builtin_amdgcn_readlane(__double2loint(c64), j);
                const int hi = __builtin_amdgcn_readlane(__double2hiint(c64), j);
                const double co = __hiloint2double(hi, lo);
                const int eo = __builtin_amdgcn_readlane(pick_e, j);
                if (co > c64 || (co == c64 && eo < pick_e)) ++rank;
            }
            slot = rank;
        }
    }

    // ---- 4. weights: the unbiased score of the pick, from its lane.  With a
    // bias it is (t - offset) / sel_mul, as the 8-row kernel computes it
    // (an exact subtraction and a power-of-two scale; c - bias on the
    // exact path), so that both kernels give the same bits.
    float u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = BIAS ? (t[i] - off[i]) * kp.sel_inv : s[i];
    const int i3 = pick_e & 3, src = pick_e >> 2;
    const float g0 = lane_gather(u[0], src), g1 = lane_gather(u[1], src);
    const float g2 = lane_gather(u[2], src), g3 = lane_gather(u[3], src);
    float wv = i3 == 0 ? g0 : i3 == 1 ? g1 : i3 == 2 ? g2 : g3;
    wv = lane < K ? wv : 0.f;
    const float inv_tot = fast_rcp(row_sum<8>(wv));  // picks are in lanes 0 .. K-1
    if (lane < K) {
        w_row[slot] = renorm ? wv * inv_tot : wv;
        id_row[slot] = pick_e;
    }

}

}  // namespace moe_route
