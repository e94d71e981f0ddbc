// Device-side routing core shared by the standalone routing kernel and the
// fused router's epilogue (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "route_common.hpp"

namespace moe_route {

template <typename T>
__device__ __forceinline__ float load_one(const T* p, int i);
template <>
__device__ __forceinline__ float load_one<float>(const float* p, int i) { return p[i]; }
template <>
__device__ __forceinline__ float load_one<uint16_t>(const uint16_t* p, int i) {
    return bf16_bits_to_float(p[i]);
}

// Median of three (one v_med3_u32).
__device__ __forceinline__ uint32_t umed3(uint32_t a, uint32_t b, uint32_t c) {
    return max(min(a, b), min(max(a, b), c));
}

// Insert key k into the descending list L[0..T-1] (keys are unique): the new
// t-th largest of {L, k} is the median of (L[t-1], L[t], k).  The key that
// drops out is min(L[T-1], k); ev keeps the largest key dropped so far.
// Every dropped key is below every key still held, so ev <= L[T-1] and
// max(ev, min(L[T-1], k)) is the median of (ev, L[T-1], k).
template <int T, bool TRACK>
__device__ __forceinline__ void list_insert(uint32_t (&L)[T], uint32_t k, uint32_t& ev) {
    if constexpr (TRACK) ev = umed3(ev, L[T - 1], k);
#pragma unroll
    for (int t = T - 1; t >= 1; --t) L[t] = umed3(L[t - 1], L[t], k);
    L[0] = max(L[0], k);
}

template <int N>
struct ListLen {
    static constexpr int value = N;
};

// Fixed-point key of a selection score: t = (c - lo) * 2^23 / R + 2^23 lies in
// [2^23, 2^24), so its fp32 mantissa is the fixed-point value; shifting the
// float bits left by 9 drops the exponent and leaves room for the index.
__device__ __forceinline__ uint32_t make_key(float c, float scale, float offs, uint32_t low9) {
    float t = __builtin_fmaf(c, scale, offs);
    return (__float_as_uint(t) << 9) | low9;
}

// LDS tile of a wave: RPW rows x E fp32 selection scores, stored in 16-byte
// chunks.  Logical chunk q of a row lives at physical chunk
// q ^ ((q >> 3) & 7), a permutation inside each aligned block of 8 chunks.
// With 8 chunks per lane (E = 256) the 8 lanes of a row, which write the same
// chunk number in one instruction, land in 8 different bank groups.
__device__ __forceinline__ int swz_chunk(int q) { return q ^ ((q >> 3) & 7); }
__device__ __forceinline__ int swz_elem(int e) { return swz_chunk(e >> 2) * 4 + (e & 3); }

struct KeyParams {
    float scale, offs;
    bool exact_only;  // the fixed-point step would be too coarse
    // With a correction bias the routing core holds y = fma(s, sel_mul,
    // off[e]) per expert, where off[e] is the staged offset of the expert's
    // bias (sel_offset): the fixed-point value t of c = s + bias on the key
    // path, c itself on the exact path.  sel_inv = 1 / sel_mul (a power of 2).
    float sel_mul, sel_inv;
};

// Choose the fixed-point window [lo, lo + R) that holds every selection score.
__device__ __forceinline__ KeyParams key_params(float cmin, float cmax) {
    const float span = (cmax - cmin) * 1.001f + 1e-6f;
    // R = 2^e, the smallest power of two >= span and at least 2: e is the
    // exponent of span, plus one when its mantissa is not zero (a NaN span
    // keeps R = 2; a span above 2^127 gives R = inf and scale 0)
    int e = 1;
    if (span > 2.0f) {
        const uint32_t u = __float_as_uint(span);
        e = static_cast<int>(u >> 23) - 127 + ((u & 0x7fffffu) != 0u ? 1 : 0);
    }
    const float R = e >= 128 ? INFINITY : __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
    float lo = cmin - R * (1.0f / 1048576.0f);  // keeps t >= 2^23 + 8
    KeyParams kp;
    // 2^23 / R, exactly
    kp.scale = e >= 128 ? 0.0f : __uint_as_float(static_cast<uint32_t>(150 - e) << 23);
    kp.offs = 8388608.0f - lo * kp.scale;
    kp.exact_only = R > 4.0f;
    kp.sel_mul = kp.exact_only ? 1.0f : kp.scale;
    kp.sel_inv = kp.exact_only ? 1.0f : R * (1.0f / 8388608.0f);
    return kp;
}

// The staged offset of a bias value: its fixed-point image b * scale + offs
// (an integer in [2^23, 2^24)), so that one fma of the score gives the
// fixed-point value of c = s + b within one step; on the exact path, b.
__device__ __forceinline__ float sel_offset(float b, const KeyParams& kp) {
    return kp.exact_only ? b : __builtin_fmaf(b, kp.scale, kp.offs);
}

// The bias entries lane l of a full wave holds for the key window: l, l + 64,
// l + 128, l + 192 (0 past E), as fp32 bit patterns.  The branch on the bias
// type holds only the loads, so that they stay in flight past it; the bf16
// entries are widened (exactly) where the bits are first used.
template <int E>
__device__ __forceinline__ void bias_lane_load(const BiasRef& bias, uint32_t (&raw)[4]) {
    static_assert(E <= 4 * kWave, "four bias entries per lane");
    const int lane = threadIdx.x % kWave;
    if (bias.bf16) {
        const uint16_t* p = static_cast<const uint16_t*>(bias.p);
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[i] = lane + kWave * i < E ? p[lane + kWave * i] : 0u;
    } else {
        const uint32_t* p = static_cast<const uint32_t*>(bias.p);
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[i] = lane + kWave * i < E ? p[lane + kWave * i] : 0u;
    }
}
__device__ __forceinline__ void bias_lane_widen(const BiasRef& bias, const uint32_t (&raw)[4],
                                                float (&b)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = __uint_as_float(bias.bf16 ? raw[i] << 16 : raw[i]);
}
// Key window of a biased routing call from the entries bias_lane_load gave
// every lane of a full wave; the range is reduced over the wave.
template <int E>
__device__ __forceinline__ KeyParams bias_lane_key_params(const float (&b)[4]) {
    const int lane = threadIdx.x % kWave;
    float bmin = INFINITY, bmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (lane + kWave * i < E) { bmin = fminf(bmin, b[i]); bmax = fmaxf(bmax, b[i]); }
    return key_params(wave_min_all(bmin), 1.0f + wave_max_all(bmax));
}
// Both of the above.
template <int E>
__device__ __forceinline__ KeyParams bias_key_params(const BiasRef& bias, float (&b)[4]) {
    uint32_t raw[4];
    bias_lane_load<E>(bias, raw);
    bias_lane_widen(bias, raw, b);
    return bias_lane_key_params<E>(b);
}

// Offsets inside a row of the per-wave LDS tile (ROW fp32 values); 16-byte
// chunks are permuted within aligned blocks of 8 (see swz_chunk) when the row
// spans whole blocks, and rows of odd index (rw, the row within the wave)
// also swap neighbouring blocks when the row spans whole pairs of blocks.
// With 8 lanes per row writing the same chunk number of 8 rows, the 64 lanes
// of a store then cover all 16 bank groups, 4 lanes each.
template <int ROW>
__device__ __forceinline__ int tile_chunk(int q, int rw) {
    if constexpr ((ROW / 4) % 16 == 0) return swz_chunk(q) ^ (8 * (rw & 1));
    else if constexpr ((ROW / 4) % 8 == 0) return swz_chunk(q);
    return q;
}
template <int ROW>
__device__ __forceinline__ int tile_elem(int i, int rw) {
    return tile_chunk<ROW>(i >> 2, rw) * 4 + (i & 3);
}
// Layout of the bias staged in LDS (E values): chunks permuted like a tile
// row, so that the 8 lanes of a row, reading the same chunk number of their
// own 32 (or 20) experts, hit different bank groups.
template <int E>
__device__ __forceinline__ int bias_chunk(int q) { return tile_chunk<E>(q, 0); }
template <int E>
__device__ __forceinline__ int bias_elem(int e) { return tile_elem<E>(e, 0); }

// Unbiased score of a logit: sigmoid, or the softmax numerator exp(x - max).
template <bool SOFTMAX>
__device__ __forceinline__ float lane_score(float x, float mx) {
    if constexpr (SOFTMAX) return fast_exp2((x - mx) * kLog2e);
    return sigmoid_f32(x);
}

// Route the rows of one wave tile.  Lane `sub` of row-in-wave `rw` brings the
// fp32 logits x[0..VPL) of experts [sub*VPL, sub*VPL + VPL) of its token,
// whose K weights and ids go to w_row[0..K) and id_row[0..K) (valid ==
// false past the last token: computed, never stored).  my_row is
// this row's E-float LDS scratch (LPR > 1); s_bias the staged bias offsets
// (sel_offset of each expert's bias) in LDS, in the bias_elem layout (BIAS);
// logit_of(e) returns the fp32 logit of expert e of this row and bias_of(e)
// its correction bias (0 without one) (rare paths).
// Steps follow "[SGLang] MoE routing: token-to-expert assignment algorithms",
// sections 2-4; see the file header of route_fast.hip for the design.
template <int LPR, int VPL, bool SOFTMAX, bool BIAS, int GRP /*0 none, 1 max, 2 top2*/, int SPLIT,
          int TL, int KMAX, typename LogitFn, typename BiasFn>
__device__ __forceinline__ void route_rows(float (&x)[VPL], const int sub, const int rw,
                                           const bool valid, float* my_row,
                                           const float* s_bias, const KeyParams& kp, const int TG,
                                           const int K, const int renorm, float* __restrict__ w_row,
                                           int32_t* __restrict__ id_row, LogitFn logit_of,
                                           BiasFn bias_of) {
    constexpr int E = LPR * VPL;
    constexpr int NC = GRP ? VPL / SPLIT : VPL;    // candidates per lane in the list step
    constexpr int SLOTS = (KMAX + LPR - 1) / LPR;  // output slots per lane
    constexpr int CPL = VPL / 4;                   // 16-byte chunks per lane
    constexpr int ROW = LPR > 1 ? E : 4;           // fp32 values per row in LDS
    static_assert(GRP == 0 || VPL % SPLIT == 0, "a group splits evenly");
    static_assert(E <= 512, "9 index bits");
    static_assert(LPR == 1 || LPR == 2 || LPR == 4 || LPR == 8 || (LPR == 16 && GRP == 0),
                  "lanes per row");
    static_assert(GRP == 0 || LPR == 8, "grouped kernels hold one of 8 groups per lane");
    static_assert(LPR > 1 || TL >= KMAX, "one lane per row reads its picks off its list");
    // A lane keeps only its TL best keys.  When that can be fewer than a
    // row needs from one lane, the keys it dropped are tracked, and a wave in
    // which a dropped key beats the K-th pick selects again with longer lists.
    constexpr bool TRACK = TL < KMAX && TL < NC;
    static_assert(VPL % 4 == 0 && SLOTS <= 2, "");
    // Group scores as fixed point with the key step: (h - lo) * scale for the
    // max rule, (h - 2 lo) * scale for the top-2 sum; both lie in [0, 2^24).
    const float h_offs = (GRP == 2 ? 2.0f : 1.0f) * (kp.offs - 8388608.0f);

    // ---- 1. scores s and selection scores c = s + bias (c stored to LDS)
    float mx = 0.f, row_total = 1.f;
    if constexpr (SOFTMAX) {
        float m = x[0];
#pragma unroll
        for (int j = 1; j < VPL; ++j) m = fmaxf(m, x[j]);
        mx = row_max<LPR>(m);
    }
    {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            x[j] = lane_score<SOFTMAX>(x[j], mx);
            if constexpr (SOFTMAX) acc += x[j];
        }
        if constexpr (SOFTMAX) row_total = row_sum<LPR>(acc);
    }
    if constexpr (BIAS) {
        // y = fma(s, sel_mul, offset): the fixed-point value t of c = s + bias
        // (or c itself on the exact path)
        const float a = kp.sel_mul;
#pragma unroll
        for (int v = 0; v < CPL; ++v) {
            const float4 d = reinterpret_cast<const float4*>(s_bias)[bias_chunk<E>(sub * CPL + v)];
            x[4 * v] = __builtin_fmaf(x[4 * v], a, d.x);
            x[4 * v + 1] = __builtin_fmaf(x[4 * v + 1], a, d.y);
            x[4 * v + 2] = __builtin_fmaf(x[4 * v + 2], a, d.z);
            x[4 * v + 3] = __builtin_fmaf(x[4 * v + 3], a, d.w);
        }
    }
    if constexpr (LPR > 1) {
#pragma unroll
        for (int v = 0; v < CPL; ++v)
            reinterpret_cast<float4*>(my_row)[tile_chunk<ROW>(sub * CPL + v, rw)] =
                make_float4(x[4 * v], x[4 * v + 1], x[4 * v + 2], x[4 * v + 3]);
    }
    // x now holds the selection scores c of the lane's experts, or with a
    // bias (key path) their fixed-point values t in [2^23, 2^24)

    // ---- 2. group score, rank among the row's 8 groups, keep the best TG
    uint32_t kept_row = 1u;
    if constexpr (GRP != 0) {
        // top two of the lane's values, two values a step: the new second is
        // the larger of the old second and the median of (m1, a, b)
        float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll
        for (int j = 0; j < VPL; j += 2) {
            if (GRP == 2) m2 = fmaxf(__builtin_amdgcn_fmed3f(m1, x[j], x[j + 1]), m2);
            m1 = fmaxf(fmaxf(m1, x[j]), x[j + 1]);
        }
        uint32_t hq;
        if constexpr (BIAS) {
            // t values are integers below 2^24 in fp32: their bits less the
            // exponent field are the fixed-point values, summed exactly
            hq = GRP == 2 ? __float_as_uint(m1) + __float_as_uint(m2) - 2u * 0x4B000000u
                          : __float_as_uint(m1) - 0x4B000000u;
        } else {
            const float h = GRP == 2 ? m1 + m2 : m1;
            hq = static_cast<uint32_t>(__builtin_fmaf(h, kp.scale, h_offs));
        }
        const uint32_t hk = (hq << 3) | static_cast<uint32_t>(7 - sub);
        uint32_t rank = 0;
        const uint32_t m7 = dpp_mov_u32<kDppMirror8>(hk);
        rank += dpp_mov_u32<kDppXor1>(hk) > hk;
        rank += dpp_mov_u32<kDppXor2>(hk) > hk;
        rank += dpp_mov_u32<kDppXor3>(hk) > hk;
        rank += m7 > hk;
        rank += dpp_mov_u32<kDppXor1>(m7) > hk;
        rank += dpp_mov_u32<kDppXor2>(m7) > hk;
        rank += dpp_mov_u32<kDppXor3>(m7) > hk;
        const uint64_t kept_wave = __ballot(rank < static_cast<uint32_t>(TG));
        kept_row = static_cast<uint32_t>(kept_wave >> (rw * LPR)) & 0xffu;
    }

    // ---- 3. candidates -> keys -> sorted list of the lane's TL best keys
    int cand_base = sub * VPL;  // expert index of this lane's first candidate
    bool has_cand = true;
    float cc[NC];
    if constexpr (GRP != 0) {
        wave_lds_sync();
        const int k = sub / SPLIT, part = sub % SPLIT;
        uint32_t m = kept_row;
#pragma unroll
        for (int i = 0; i < LPR / SPLIT - 1; ++i)
            if (i < k) m &= m - 1u;
        const int g = m ? __builtin_ctz(m) : 0;
        has_cand = k < TG && m != 0u;
        cand_base = g * VPL + part * NC;
        if constexpr (NC % 4 == 0) {
#pragma unroll
            for (int v = 0; v < NC / 4; ++v) {
                const float4 d = reinterpret_cast<const float4*>(
                    my_row)[tile_chunk<ROW>((cand_base >> 2) + v, rw)];
                cc[4 * v] = d.x; cc[4 * v + 1] = d.y; cc[4 * v + 2] = d.z; cc[4 * v + 3] = d.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < NC; ++j) cc[j] = my_row[tile_elem<ROW>(cand_base + j, rw)];
        }
    } else {
#pragma unroll
        for (int j = 0; j < NC; ++j) cc[j] = x[j];
    }
    // low 9 bits := 511 - expert index; empty slots stay below 512
    const uint32_t base9 = 511u - (uint32_t)(cand_base + NC - 1);

    // ---- 4. per-lane lists of the T best keys, then K merge rounds: the
    // row-wide maximum of the list heads is the next pick and its lane pops
    // its head.  wk receives this lane's picks, w_last the K-th pick, ev the
    // largest key a list dropped (when T can be short of what a row needs).
    uint32_t wk[SLOTS];
    uint32_t w_last = 0u;
    auto select = [&](auto t_c, uint32_t& ev) {
        constexpr int T = decltype(t_c)::value;
        constexpr bool TR = T < KMAX && T < NC;
        uint32_t L[T];
#pragma unroll
        for (int t = 0; t < T; ++t) L[t] = 0u;
        if (has_cand) {
#pragma unroll
            for (int j = 0; j < NC; ++j)
                list_insert<T, TR>(
                    L,
                    BIAS ? (__float_as_uint(cc[j]) << 9) | (uint32_t)(NC - 1 - j)
                         : make_key(cc[j], kp.scale, kp.offs, (uint32_t)(NC - 1 - j)),
                    ev);
        }
#pragma unroll
        for (int t = 0; t < T; ++t) L[t] += base9;
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) wk[s] = 0u;
        if constexpr (LPR == 1) {
#pragma unroll
            for (int s = 0; s < SLOTS; ++s) wk[s] = L[s];
        } else {
            auto round = [&](int r) {
                const uint32_t w = row_max_u32<LPR>(L[0]);
                w_last = w;
                const bool mine = (L[0] == w);
#pragma unroll
                for (int t = 0; t < T - 1; ++t) L[t] = mine ? L[t + 1] : L[t];
                L[T - 1] = mine ? base9 : L[T - 1];
                if (sub == r % LPR) {
                    if (SLOTS == 1 || r < LPR) wk[0] = w;
                    else wk[SLOTS - 1] = w;
                }
            };
            if constexpr (BIAS) {
                // unrolled to KMAX rounds, leaving at the first round past K:
                // ~2% faster for the biased kernels, whose register count it
                // leaves alone (the others grow by ~13 VGPRs)
#pragma unroll
                for (int r = 0; r < KMAX; ++r) {
                    if (r >= K) break;
                    round(r);
                }
            } else {
#pragma unroll 1
                for (int r = 0; r < K; ++r) round(r);
            }
        }
    };
    uint32_t ev = 0u;
    select(ListLen<TL>{}, ev);
    if constexpr (TRACK) {
        // A dropped key beats the K-th pick somewhere in the wave: redo the
        // wave's selection with lists as long as K, which cannot run dry.
        if (__ballot(ev != 0u && ev + base9 > w_last) != 0) {
            uint32_t unused = 0u;
            select(ListLen<KMAX>{}, unused);
        }
    }
    int pick[SLOTS];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) pick[s] = 511 - (int)(wk[s] & 511u);

    // ---- exact path, for a bias spread too wide for the key window: K
    // rounds of a (value, index) argmax on the fp32 selection scores.  With
    // several lanes per row the scores are read from the row's LDS tile, 16
    // bytes at a time, in rolled loops that keep this rare path off the
    // register budget of the main path.
    if (kp.exact_only) {
        // c of this lane's experts sub*VPL + 4q .. +3
        auto chunk = [&](int q) -> float4 {
            if constexpr (LPR > 1) {
                return reinterpret_cast<const float4*>(my_row)[tile_chunk<ROW>(sub * CPL + q, rw)];
            } else {
                float c4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    c4[i] = lane_score<SOFTMAX>(logit_of(4 * q + i), mx);
                    if constexpr (BIAS) c4[i] += s_bias[bias_elem<E>(4 * q + i)];
                }
                return make_float4(c4[0], c4[1], c4[2], c4[3]);
            }
        };
        bool kept = true;
        if constexpr (GRP != 0) {
            float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll 1
            for (int q = 0; q < CPL; ++q) {
                const float4 d = chunk(q);
                const float c4[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (GRP == 2) m2 = __builtin_amdgcn_fmed3f(m1, m2, c4[i]);
                    m1 = fmaxf(m1, c4[i]);
                }
            }
            const float h = GRP == 2 ? m1 + m2 : m1;
            int rank = 0;
#pragma unroll 1
            for (int d = 1; d < LPR; ++d) {
                const float o = __shfl(h, rw * LPR + (sub ^ d), kWave);
                rank += beats(o, sub ^ d, h, sub) ? 1 : 0;
            }
            kept = rank < TG;
        }
        float bv_prev = INFINITY;
        int bi_prev = -1;
#pragma unroll 1
        for (int r = 0; r < K; ++r) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
            if (kept) {
#pragma unroll 1
                for (int q = 0; q < CPL; ++q) {
                    const float4 d = chunk(q);
                    const float c4[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int e = sub * VPL + 4 * q + i;
                        if (beats(bv_prev, bi_prev, c4[i], e) && beats(c4[i], e, bv, bi)) {
                            bv = c4[i];
                            bi = e;
                        }
                    }
                }
            }
            row_argmax<LPR>(bv, bi);
            bv_prev = bv;
            bi_prev = bi;
#pragma unroll
            for (int s = 0; s < SLOTS; ++s)
                if (r == s * LPR + sub) pick[s] = bi;
        }
    }

    // ---- exact order of near-tied picks (sigmoid scoring, eight lanes per
    // row, one pick per lane).  A key is within 1.5 key steps of the exact
    // fixed-point value of c (half a step each for the staged bias offset,
    // the final rounding and the fp32 sigmoid), so two adjacent picks whose
    // keys differ by more than kNearKeySteps are in the exact order.  When a
    // row of the wave has a closer pair, the selection scores of every
    // row's picks are recomputed in double precision and each pick takes
    // its rank among its row's picks (c desc, expert asc) as its output
    // slot.  The branch is taken in about one tile in a thousand.  (Near
    // ties at the K-th pick itself, or between kept and dropped groups, are
    // left to the keys.)
    int slot0 = sub;  // output slot of this lane's first pick
    // (With 16 lanes a row the K <= 8 picks sit in the first 8 lanes, and the
    // DPP patterns below stay inside each half of the row.)
    if constexpr (!SOFTMAX && (LPR == 8 || LPR == 16) && SLOTS == 1) {
        // keys are (value << 9 | index bits), sorted descending along the
        // row's lanes: a value gap of at most kNearKeySteps makes the key
        // difference less than (kNearKeySteps + 1) << 9 (a gap one step
        // larger may also pass: a harmless extra re-ranking)
        constexpr uint32_t kNearKeySteps = 4;
        const uint32_t nxt = dpp_mov_u32<kDppRowShl1>(wk[0]);
        const bool near = !kp.exact_only && sub + 1 < K &&
                          wk[0] - nxt < ((kNearKeySteps + 1) << 9);
        if (__builtin_expect(__ballot(near) != 0ull, 0)) {
            const int p0 = min(max(pick[0], 0), E - 1);
            const double c64 = sigmoid_f64((double)logit_of(p0)) + (double)bias_of(p0);
            // rank among the row's K picks: the other 7 lanes of the row by
            // the all-to-all DPP pattern of the group rank (lane i ^ 1, i ^ 2,
            // i ^ 3, 7 - i and 7 - (i ^ 1..3)); lanes sub >= K hold no pick
            const uint32_t lo = __double2loint(c64), hi = __double2hiint(c64);
            const uint32_t me = static_cast<uint32_t>(p0) | (static_cast<uint32_t>(sub) << 16);
            int rank = 0;
            auto count = [&](uint32_t olo, uint32_t ohi, uint32_t ome) {
                const double co = __hiloint2double((int)ohi, (int)olo);
                const int po = (int)(ome & 0xffffu), so = (int)(ome >> 16);
                if (so < K && (co > c64 || (co == c64 && po < p0))) ++rank;
            };
            count(dpp_mov_u32<kDppXor1>(lo), dpp_mov_u32<kDppXor1>(hi), dpp_mov_u32<kDppXor1>(me));
            count(dpp_mov_u32<kDppXor2>(lo), dpp_mov_u32<kDppXor2>(hi), dpp_mov_u32<kDppXor2>(me));
            count(dpp_mov_u32<kDppXor3>(lo), dpp_mov_u32<kDppXor3>(hi), dpp_mov_u32<kDppXor3>(me));
            const uint32_t mlo = dpp_mov_u32<kDppMirror8>(lo), mhi = dpp_mov_u32<kDppMirror8>(hi),
                           mme = dpp_mov_u32<kDppMirror8>(me);
            count(mlo, mhi, mme);
            count(dpp_mov_u32<kDppXor1>(mlo), dpp_mov_u32<kDppXor1>(mhi), dpp_mov_u32<kDppXor1>(mme));
            count(dpp_mov_u32<kDppXor2>(mlo), dpp_mov_u32<kDppXor2>(mhi), dpp_mov_u32<kDppXor2>(mme));
            count(dpp_mov_u32<kDppXor3>(mlo), dpp_mov_u32<kDppXor3>(mhi), dpp_mov_u32<kDppXor3>(mme));
            if (sub < K) slot0 = rank;
        }
    }

    // ---- 5. weights from the unbiased scores, renormalisation, stores
    if constexpr (LPR > 1 && GRP == 0) wave_lds_sync();
    float wsl[SLOTS];
    float part_sum = 0.f;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
        const int r = s * LPR + sub;
        pick[s] = min(max(pick[s], 0), E - 1);  // never read outside the row
        float sv;
        if constexpr (LPR > 1) {
            // the row holds c, or with a bias fma(s, sel_mul, offset): the
            // weight is the unbiased score, (y - offset) / sel_mul (exact
            // subtraction; s to within half a key step, or c - bias on the
            // exact path)
            sv = my_row[tile_elem<ROW>(pick[s], rw)];
            if constexpr (BIAS) sv = (sv - s_bias[bias_elem<E>(pick[s])]) * kp.sel_inv;
        } else if constexpr (SOFTMAX) {
            sv = x[0];  // one lane per row: x holds the numerators
#pragma unroll
            for (int j = 1; j < VPL; ++j) sv = (pick[s] == j) ? x[j] : sv;
        } else {
            // one lane per row: x holds c; recompute s of the pick from its logit
            sv = valid ? sigmoid_f32(logit_of(pick[s])) : 0.f;
        }
        if constexpr (SOFTMAX) sv = sv / row_total;
        wsl[s] = (r < K) ? sv : 0.f;
        part_sum += wsl[s];
    }
    const float inv_tot = fast_rcp(row_sum<LPR>(part_sum));
    if (valid) {
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int r = s * LPR + sub;
            const int o = s == 0 ? slot0 : r;
            if (r < K) {
                w_row[o] = renorm ? wsl[s] * inv_tot : wsl[s];
                id_row[o] = pick[s];
            }
        }
    }
    if constexpr (LPR > 1) wave_lds_sync();  // the next tile rewrites the LDS rows
}

}  // namespace moe_route
