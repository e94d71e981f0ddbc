// Fused router for few experts (E = 8 or 16), gfx950.
//
// "[SGLang] MoE routing: token-to-expert assignment algorithms", section 5:
// besides the tensor-core router, the page has a plain elementwise router
// (each logit a product summed along the hidden dimension) followed by
// optional soft-capping and a softmax top-1/top-2, and sends small batches
// and routers with at most 8 experts to it.  Here two kernels serve these
// expert counts at every batch size; all read the hidden states once, which
// bounds them (2H bytes per token against 2EH multiply-adds):
//
//  - MFMA kernels (hidden_dim <= 8192): 16-token tiles on
//    v_mfma_f32_16x16x32_bf16, W held in registers (described below).  With
//    hidden_dim a multiple of 1024 the hidden states come through a ring of
//    LDS stages in whole 1 KiB row runs; otherwise each lane loads its MFMA
//    operand straight from global memory;
//  - a vector-ALU kernel: bf16 pairs on v_dot2_f32_bf16, used for more than
//    8192 hidden units, and for 8 experts with few tokens, where its 8-token
//    blocks spread over more compute units than 16-token tiles do.
//
// Vector-ALU layout.  A block of 4 waves routes groups of T = 8 tokens
// (persistent blocks stride over the groups); the waves take turns over
// chunks of the hidden dimension.  Each lane owns a slice of 8 experts
// (E / 8 slices over the wave) and 8 consecutive hidden units: one 16-byte
// load per token and the lane's 16-byte slice of the 8 matching W rows.
// Pairs of hidden units meet v_dot2_f32_bf16 (two bf16 products added to an
// fp32 accumulator); v_perm_b32 pairs the two W rows' entries of one expert
// to match.  Each lane keeps T x 8 fp32 partial sums, and W is read once per
// 8 tokens; the next chunk's loads are issued before the current chunk's
// products.  The block then sums the partials of its lanes in LDS in a fixed
// order, soft-caps the logits and one lane per token routes (softmax or
// sigmoid, optional bias, top-K by (score desc, index asc), optional
// renormalisation).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "route_common.hpp"
#include "lds_copy.hpp"
#include "route_internal.h"

namespace moe_route {
namespace {

constexpr int kSrWaves = 4;
constexpr int kSrThreads = kSrWaves * kWave;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// One token's routing over its E logits (cap already applied): scores,
// selection scores c = s + bias, K picks by (c desc, index asc), weights s
// of the picks, optionally divided by their sum (added in pick order).
template <int E, bool SOFTMAX, bool BIAS>
__device__ __forceinline__ void route_token(const float (&x)[E], BiasRef bias,
                                            int K, int renorm, float* __restrict__ w_row,
                                            int32_t* __restrict__ id_row) {
    float s[E], c[E];
    if constexpr (SOFTMAX) {
        float mx = x[0];
#pragma unroll
        for (int e = 1; e < E; ++e) mx = fmaxf(mx, x[e]);
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            s[e] = fast_exp2((x[e] - mx) * kLog2e);
            sum += s[e];
        }
#pragma unroll
        for (int e = 0; e < E; ++e) s[e] = s[e] / sum;
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) s[e] = sigmoid_f32(x[e]);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) c[e] = BIAS ? s[e] + bias_at(bias, e) : s[e];

    int slot[E];  // pick rank of each expert, -1 if not picked
#pragma unroll
    for (int e = 0; e < E; ++e) slot[e] = -1;
    float tot = 0.f;
    for (int k = 0; k < K; ++k) {
        float bv = -INFINITY, bs = 0.f;
        int bi = E;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            // scanning e upwards with a strict > keeps the lower index on ties
            if (slot[e] < 0 && (c[e] > bv || bi == E)) { bv = c[e]; bi = e; bs = s[e]; }
        }
#pragma unroll
        for (int e = 0; e < E; ++e) slot[e] = e == bi ? k : slot[e];
        tot += bs;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (slot[e] >= 0) {
            w_row[slot[e]] = renorm ? s[e] / tot : s[e];
            id_row[slot[e]] = e;
        }
    }
}

constexpr int kSrTokens = 8;  // tokens per group

template <int E, bool SOFTMAX, bool BIAS>
__global__ __launch_bounds__(kSrThreads) void small_router_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ w,
    BiasRef bias, int64_t M, int H, int K, int renorm, float cap,
    float* __restrict__ w_out, int32_t* __restrict__ id_out) {
    constexpr int T = kSrTokens;
    constexpr int NS = E / 8;          // expert slices per wave
    constexpr int LPS = kWave / NS;    // lanes per slice
    constexpr int UPC = 8 * LPS;       // hidden units per wave and chunk
    constexpr int NV = T * 8;          // partial sums per lane
    static_assert(NV % 32 == 0, "partials are reduced 32 at a time");
    __shared__ __align__(16) float red[32][kSrThreads + 4];
    __shared__ float logit[T * E];

    const int t = threadIdx.x, lane = t % kWave, wv = t / kWave;
    const int es = lane / LPS, lp = lane % LPS;
    const int64_t groups = (M + T - 1) / T;
    const int chunks = (H + UPC - 1) / UPC;

    struct Chunk {
        uint4 hv[T];
        uint4 wr[8];
    };
    float acc[T][8];
#pragma unroll
    for (int tk = 0; tk < T; ++tk)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[tk][e] = 0.f;

    // Loads of chunk c (c < chunks) of group g.  Lanes past H load unit 0
    // and zero it; rows past M read row M-1 (never stored).
    auto load = [&](int64_t g, int c, Chunk& b) __attribute__((always_inline)) {
        const int h = c * UPC + 8 * lp;
        const int hc = h < H ? h : 0;
#pragma unroll
        for (int tk = 0; tk < T; ++tk)
            b.hv[tk] = *reinterpret_cast<const uint4*>(hidden + min(g * T + tk, M - 1) * H + hc);
#pragma unroll
        for (int r = 0; r < 8; ++r)
            b.wr[r] = *reinterpret_cast<const uint4*>(w + (int64_t)(hc + r) * E + 8 * es);
        if (c * UPC + UPC > H && h >= H) {
#pragma unroll
            for (int tk = 0; tk < T; ++tk) b.hv[tk] = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto compute = [&](const Chunk& b) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {  // hidden units 8 lp + 2p, 8 lp + 2p + 1
            const uint32_t* lo = reinterpret_cast<const uint32_t*>(&b.wr[2 * p]);
            const uint32_t* hi = reinterpret_cast<const uint32_t*>(&b.wr[2 * p + 1]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {  // slice experts 2j, 2j + 1
                const uint32_t we = __builtin_amdgcn_perm(hi[j], lo[j], 0x05040100u);
                const uint32_t wo = __builtin_amdgcn_perm(hi[j], lo[j], 0x07060302u);
#pragma unroll
                for (int tk = 0; tk < T; ++tk) {
                    const uint32_t a = reinterpret_cast<const uint32_t*>(&b.hv[tk])[p];
                    acc[tk][2 * j] = dot2(a, we, acc[tk][2 * j]);
                    acc[tk][2 * j + 1] = dot2(a, wo, acc[tk][2 * j + 1]);
                }
            }
        }
    };

    // Sum the block's partials of group g, soft-cap them and route its
    // tokens; acc is cleared for the next group.
    auto finish = [&](int64_t g) __attribute__((always_inline)) {
        const int64_t m0 = g * T;
        // Sum the partials, 32 values per round.  Thread t writes its values
        // to column t.  Columns come in blocks of 32 lanes (one slice of a
        // wave, or half a slice when E = 8); the threads of output
        // (value j, slice s) add one such block each, blocks in a fixed
        // order, then combine by butterfly.  The order never changes, so
        // results do not depend on timing.
#pragma unroll
        for (int r = 0; r < NV / 32; ++r) {
#pragma unroll
            for (int j = 0; j < 32; ++j) red[j][t] = acc[(32 * r + j) / 8][(32 * r + j) % 8];
            __syncthreads();
            constexpr int TPO = kSrThreads / 32 / NS;  // threads per output
            const int o = t / TPO, q = t % TPO;
            const int j = o % 32, s = o / 32;
            const int cb = q * NS + s;   // column block: lanes 32 (cb % 2) .. of wave cb / 2
            float v = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 d = *reinterpret_cast<const float4*>(&red[j][32 * cb + 4 * i]);
                v += (d.x + d.y) + (d.z + d.w);
            }
            v = row_sum<TPO>(v);  // the output's TPO lanes, on DPP
            if (q == 0) {
                const int vi = 32 * r + j;  // token vi / 8, expert 8 s + vi % 8
                logit[(vi / 8) * E + 8 * s + vi % 8] = cap != 0.0f ? cap * tanh_f32(v / cap) : v;
            }
            __syncthreads();
        }

        if (t < T && m0 + t < M) {
            float x[E];
#pragma unroll
            for (int e = 0; e < E; ++e) x[e] = logit[t * E + e];
            route_token<E, SOFTMAX, BIAS>(x, bias, K, renorm, w_out + (m0 + t) * K,
                                          id_out + (m0 + t) * K);
        }
#pragma unroll
        for (int tk = 0; tk < T; ++tk)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[tk][e] = 0.f;
    };

    // Each wave streams its (group, chunk) items -- chunks wv, wv + 4, ...
    // of groups blockIdx.x, blockIdx.x + gridDim.x, ... -- through two
    // buffers: the loads of the next item, possibly of the next group, are in
    // flight while the current one is computed and while a finished group is
    // reduced.  Every wave finishes each group once, so all pass the same
    // barriers.  The last item's successor repeats it (one load, no branch).
    const int n = wv < chunks ? (chunks - 1 - wv) / kSrWaves + 1 : 0;  // items per group
    int64_t g = blockIdx.x;
    if (n == 0) {
        for (; g < groups; g += gridDim.x) finish(g);
        return;
    }
    int k = 0;  // item of group g held in the current buffer
    auto step = [&](Chunk& cur, Chunk& nxt) __attribute__((always_inline)) {
        int64_t g2 = g;
        int k2 = k + 1;
        if (k2 == n) { g2 = g + gridDim.x; k2 = 0; }
        const bool more = g2 < groups;
        load(more ? g2 : g, wv + kSrWaves * (more ? k2 : k), nxt);
        compute(cur);
        if (k + 1 == n) finish(g);
        g = g2;
        k = k2;
        return g < groups;
    };
    Chunk A, B;
    load(g, wv, A);
    while (step(A, B) && step(B, A)) {
    }
}

template <int E, bool SOFTMAX, bool BIAS>
route_status_t launch_sr(const FusedProblem& f) {
    const RouteProblem& p = f.route;
    auto kernel = small_router_kernel<E, SOFTMAX, BIAS>;
    // blocks per CU for this instantiation (a thread-safe one-time query)
    static const int resident = resident_blocks(kernel, kSrThreads);
    const int64_t groups = (f.M + kSrTokens - 1) / kSrTokens;
    const int64_t blocks = std::min<int64_t>(groups, (int64_t)device_cu_count() * resident);
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kSrThreads), 0, p.stream,
                       static_cast<const uint16_t*>(f.hidden), static_cast<const uint16_t*>(f.w),
                       p.bias, f.M, f.H, p.K, p.renorm ? 1 : 0, f.softcap, p.weights, p.ids);
    return hipGetLastError() == hipSuccess ? ROUTE_OK : ROUTE_ELAUNCH;
}

// One token's routing over 16 consecutive lanes (one DPP row): lane j holds
// expert j's logit x (cap applied); lanes j >= E hold none.  Same rule as
// route_token: K rounds of an argmax by (c desc, index asc); the weights s
// of the picks are then added across the row, and the pick of rank k is
// stored by its lane.  Every reduction is a DPP butterfly within the row
// (no LDS permutes), so every lane of the row holds the same bits.
template <int E, bool SOFTMAX, bool BIAS>
__device__ __forceinline__ void route_lanes16_b(float x, int j, bool store, float bj, int K,
                                                int renorm, float* __restrict__ w_row,
                                                int32_t* __restrict__ id_row) {
    const bool live = j < E;
    float s;
    if constexpr (SOFTMAX) {
        const float mx = row_max<16>(live ? x : -INFINITY);
        const float u = live ? fast_exp2((x - mx) * kLog2e) : 0.f;
        s = u / row_sum<16>(u);
    } else {
        s = sigmoid_f32(x);
    }
    const float c = BIAS && live ? s + bj : s;
    // K rounds of a 16-lane arg-max (value desc, index asc) on DPP; the
    // picked lanes' unbiased scores are summed once at the end
    bool open = live;  // not picked yet
    int rank = -1;
    for (int k = 0; k < K; ++k) {
        float bv = open ? c : -INFINITY;
        int bi = open ? j : 0x7fffffff;
        row_argmax<16>(bv, bi);
        if (bi == j) { rank = k; open = false; }
    }
    const float tot = row_sum<16>(rank >= 0 ? s : 0.f);
    if (store && rank >= 0) {
        w_row[rank] = renorm ? s / tot : s;
        id_row[rank] = j;
    }
}
// The same with the bias entry of lane j read here.
template <int E, bool SOFTMAX, bool BIAS>
__device__ __forceinline__ void route_lanes16(float x, int j, bool store,
                                              BiasRef bias, int K, int renorm,
                                              float* __restrict__ w_row,
                                              int32_t* __restrict__ id_row) {
    const float bj = BIAS && j < E ? bias_at(bias, j) : 0.0f;
    route_lanes16_b<E, SOFTMAX, BIAS>(x, j, store, bj, K, renorm, w_row, id_row);
}

// ---- MFMA variant (hidden_dim <= 8192)
//
// The projection is a [M, H] x [H, E] product with E <= 16, which fits
// v_mfma_f32_16x16x32_bf16 (16 tokens x 32 hidden units x 16 experts; with
// E = 8 half of the tile's columns are zero).  A block of 8 waves fills a
// compute unit (256 registers per lane) and strides over tiles of 16 tokens.
// The 32-unit fragments of H are dealt to the waves round-robin (fragment f
// to wave f mod 8), and each wave keeps its fragments of W in registers as MFMA B operands for the
// whole launch.  A operands come straight from global memory: in the MFMA
// layout, lane (token i, quarter q) of fragment f holds hidden units
// 32 f + 8 q .. +7 of token i, one 16-byte load.  A wave loads its
// fragments 4 at a time into two register buffers, both in flight: the next
// two batches (or the next tile's first two) load while the current one is
// multiplied and while a finished tile is reduced.  Partial tiles of the 8 waves are added in LDS
// in wave order, then soft-capped and routed by 16 lanes per token.
constexpr int kSmWaves = 8;
constexpr int kSmThreads = kSmWaves * kWave;
constexpr int kSmTile = 16;      // tokens per tile
constexpr int kSmFragMax = 32;   // fragments per wave: hidden_dim <= 8 * 32 * 32
constexpr int kSmBatch = 4;      // fragments per load batch
constexpr int kSmHMax = kSmWaves * kSmFragMax * 32;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int E, int NB, bool SOFTMAX, bool BIAS>
__global__ __launch_bounds__(kSmThreads) void small_router_mfma_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ w,
    BiasRef bias, int64_t M, int H, int K, int renorm, float cap,
    float* __restrict__ w_out, int32_t* __restrict__ id_out) {
    __shared__ float part[kSmWaves][kSmTile * 16];
    __shared__ __align__(16) unsigned char wstage[kSmWaves][kSmBatch * 1024];

    const int t = threadIdx.x, lane = t % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(t / kWave);
    const int i16 = lane % 16, q = lane / 16;
    const int nf = (H + 31) / 32;
    const int fw = wv < nf ? (nf - 1 - wv) / kSmWaves + 1 : 0;  // fragments of this wave
    // Every wave runs NB batches of 4 fragments (NB = ceil(ceil(nf / 8) / 4));
    // fragments a wave does not have are loaded from a clamped address,
    // zeroed and multiplied as zeros, so no load sits under a branch.
    const int64_t tiles = (M + kSmTile - 1) / kSmTile;

    // B operands: lane (expert i16, quarter q) of fragment i holds
    // W[32 f + 8 q + j][i16], j = 0..7, f = wv + 8 i; zeros past H or E.
    // Each fragment's 32 W rows are one contiguous piece of W: the wave loads
    // it with 16-byte loads into an LDS image of 32 rows x 16 experts (E = 8
    // rows padded with zeros), four fragments at a time, and the transposing
    // read ds_read_b64_tr_b16 turns the image into B operands: in a 16-lane
    // group, lane j receives element j % 4 of the 8-byte rows addressed by
    // lanes j / 4 + 4 m, m = 0..3, so lane a points at row 8 q + 4 h + a / 4,
    // experts 4 (a % 4) .. +3, and lane j gets k = 8 q + 4 h + m of expert j.
    constexpr int FM = NB * kSmBatch;  // fragment slots per wave
    static_assert(FM <= kSmFragMax, "fragments per wave");
    bf16x8 wf[FM];
    struct Batch {
        uint4 a[kSmBatch];
    };
    // Batch b of tile g: fragments 4b .. 4b+3 of this wave.  Rows past M read
    // row M-1 (never stored); units past H are zero.
    auto load = [&](int64_t g, int b, Batch& x) __attribute__((always_inline)) {
        const int64_t row = min(g * kSmTile + i16, M - 1);
        const uint16_t* hr = hidden + row * H;
#pragma unroll
        for (int i = 0; i < kSmBatch; ++i) {
            const int fi = kSmBatch * b + i;
            const int k = 32 * (wv + kSmWaves * fi) + 8 * q;
            const bool ok = fi < fw && k < H;
            x.a[i] = *reinterpret_cast<const uint4*>(hr + (ok ? k : 0));
            if (!ok) x.a[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    f32x4 c0, c1;
    auto compute = [&](const Batch& x, int b) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kSmBatch; ++i) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, x.a[i]);
            if (i % 2 == 0)
                c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, wf[kSmBatch * b + i], c0, 0, 0, 0);
            else
                c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, wf[kSmBatch * b + i], c1, 0, 0, 0);
        }
    };

    // Two batch buffers, both in flight: batch b sits in P[b % 2]; once it
    // is multiplied its buffer takes batch b + 2, so batches b + 1 and b + 2
    // load during the MFMAs of batch b, and the next tile's first two
    // batches load while this tile is reduced.
    Batch P[2];
    int64_t g = blockIdx.x;
    // the first tile's hidden states load while W is turned into B operands
    load(g, 0, P[0]);
    if (NB > 1) load(g, 1, P[1]);
    {
        uint4 raw[FM];
        const int row = lane / 2, half = lane % 2;  // this lane's 16 bytes of an image
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int k = 32 * (wv + kSmWaves * i) + row;
            const bool ok = i < fw && k < H && (E == 16 || half == 0);
            raw[i] = *reinterpret_cast<const uint4*>(w + (ok ? (int64_t)k * E + 8 * half : 0));
            if (!ok) raw[i] = make_uint4(0u, 0u, 0u, 0u);
        }
        unsigned char* img = wstage[wv];
#pragma unroll
        for (int rr = 0; rr < NB; ++rr) {
#pragma unroll
            for (int i = 0; i < kSmBatch; ++i)
                *reinterpret_cast<uint4*>(img + 1024 * i + 16 * lane) = raw[kSmBatch * rr + i];
            wave_lds_sync();
#pragma unroll
            for (int i = 0; i < kSmBatch; ++i) {
                i16x4 h2[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int off = 1024 * i + 32 * (8 * q + 4 * h + i16 / 4) + 8 * (i16 % 4);
                    h2[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(img + off));
                }
                wf[kSmBatch * rr + i] = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(h2[0], h2[1], 0, 1, 2, 3, 4, 5, 6, 7));
            }
            wave_lds_sync();
        }
    }

    for (; g < tiles; g += gridDim.x) {
        const int64_t gn = g + gridDim.x < tiles ? g + gridDim.x : g;
#pragma unroll
        for (int r = 0; r < 4; ++r) { c0[r] = 0.f; c1[r] = 0.f; }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            compute(P[b % 2], b);
            if (b + 2 < NB) load(g, b + 2, P[b % 2]);
        }
        load(gn, 0, P[0]);
        if (NB > 1) load(gn, 1, P[1]);

        // D layout: lane (expert i16, quarter q) holds tokens 4q .. 4q+3
#pragma unroll
        for (int r = 0; r < 4; ++r) part[wv][(4 * q + r) * 16 + i16] = c0[r] + c1[r];
        __syncthreads();
        // thread t < 256: token t / 16, expert t % 16 (the 16 lanes of a token
        // are consecutive); partials added in wave order
        float v = 0.f;
        if (t < kSmTile * 16) {
#pragma unroll
            for (int x = 0; x < kSmWaves; ++x) v += part[x][t];
            if (cap != 0.0f) v = cap * tanh_f32(v / cap);
        }
        __syncthreads();  // part is free for the next tile
        const int64_t row = g * kSmTile + t / 16;
        if (t < kSmTile * 16)
            route_lanes16<E, SOFTMAX, BIAS>(v, t % 16, row < M, bias, K, renorm, w_out + row * K,
                                            id_out + row * K);
    }
}

template <int E, int NB, bool SOFTMAX, bool BIAS>
route_status_t launch_sm_nb(const FusedProblem& f) {
    const RouteProblem& p = f.route;
    const int64_t tiles = (f.M + kSmTile - 1) / kSmTile;
    const int64_t blocks = std::min<int64_t>(tiles, (int64_t)device_cu_count());
    hipLaunchKernelGGL((small_router_mfma_kernel<E, NB, SOFTMAX, BIAS>), dim3((unsigned)blocks),
                       dim3(kSmThreads), 0, p.stream, static_cast<const uint16_t*>(f.hidden),
                       static_cast<const uint16_t*>(f.w), p.bias, f.M, f.H, p.K,
                       p.renorm ? 1 : 0, f.softcap, p.weights, p.ids);
    return hipGetLastError() == hipSuccess ? ROUTE_OK : ROUTE_ELAUNCH;
}

// ---- MFMA variant with a hidden-state ring in LDS (hidden_dim a multiple of
// 1024, at most 8192)
//
// The kernel above loads its A operands straight from global memory in the
// MFMA layout: a (token, quarter) lane per 16 bytes, so every wave load
// touches 16 rows, 64 bytes of each.  Here the hidden states of a 16-token
// tile come through LDS, 1024 hidden units (a chunk) at a time: every wave
// copy (global_load_lds_dwordx4) is 1 KiB of one row, and the fragments are
// read from LDS in the MFMA layout.  A ring of 4 chunk stages keeps 3 chunks
// in flight ahead of the MFMAs, running on across the block's tiles.  Inside
// a copy, lane l fetches 16-byte piece l ^ (row mod 16) of the copy's run, so
// that the 16 rows of a fragment read land in different LDS banks.  W sits in
// registers as in the kernel above (fragment f of H with wave f mod 8); the
// 8 waves' partial tiles are added in LDS in wave order and routed by 16
// lanes per token.
constexpr int kRgChunk = 1024;                                       // hidden units
constexpr int kRgStages = 4;
constexpr int kRgAhead = kRgStages - 1;                              // chunks in flight
constexpr int kRgStageBytes = kSmTile * kRgChunk * 2;                // 32 KiB
constexpr int kRgCopies = kRgStageBytes / 1024 / kSmWaves;           // 4 a wave a chunk
constexpr int kRgFrags = kRgChunk / 32 / kSmWaves;                   // 4 a wave a chunk
static_assert(kRgCopies == 4 && kSmTile == 2 * kSmWaves, "wave w copies rows 2w, 2w + 1");
static_assert(kRgCopies * (kRgAhead - 1) <= 63, "a wait counts at most 63 loads");
static_assert(kSmWaves * kSmBatch * 1024 <= kRgStageBytes, "the W images fit one stage");

// LDS barrier that leaves the copies in flight alone (waits for this wave's
// LDS accesses only).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int E, int NCH, bool SOFTMAX, bool BIAS>
__global__ __launch_bounds__(kSmThreads) void small_router_ring_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ w,
    BiasRef bias, int64_t M, int K, int renorm, float cap,
    float* __restrict__ w_out, int32_t* __restrict__ id_out) {
    constexpr int H = NCH * kRgChunk;
    constexpr int FM = NCH * kRgFrags;  // fragments of W per wave
    __shared__ __align__(1024) unsigned char ring[kRgStages][kRgStageBytes];
    __shared__ float part[kSmWaves][kSmTile * 16];

    const int t = threadIdx.x, lane = t % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(t / kWave);
    const int i16 = lane % 16, q = lane / 16;
    const int64_t tiles = (M + kSmTile - 1) / kSmTile;
    const int64_t steps = ((tiles - 1 - blockIdx.x) / gridDim.x + 1) * NCH;  // blockIdx.x < tiles

    // The copies of step s (chunk s mod NCH of the block's tile s / NCH):
    // copy u is half u % 2 of row 2 wv + u / 2's run (rows past M read row
    // M-1, never stored).
    auto issue = [&](int64_t s, int stage) {
        const int64_t g = blockIdx.x + (s / NCH) * gridDim.x;
        const int c = (int)(s % NCH);
#pragma unroll
        for (int u = 0; u < kRgCopies; ++u) {
            const int r = 2 * wv + u / 2, j = u % 2;
            const int64_t row = min(g * kSmTile + r, M - 1);
            const int piece = 64 * j + (lane ^ (r & 15));
            lds_copy16(hidden + row * H + c * kRgChunk + 8 * piece,
                       lds_addr(ring[stage] + r * (2 * kRgChunk) + 1024 * j));
        }
    };
    // The bias entry of expert i16 (the lanes that route take expert t % 16),
    // loaded first: the waits of the W loads below then cover it, and no
    // wait for it is left inside the loop (one there would drain the ring).
    const float bj = BIAS && i16 < E ? bias_at(bias, i16) : 0.0f;
    // W into registers: wf[i] holds fragment wv + 8 i (units 32 (wv + 8 i)
    // ..), built through a per-wave LDS image of 32 rows x 16 experts in the
    // last ring stage, which the first copies do not use.  The first copy
    // goes out first; then every W load of the wave is in flight at once,
    // so that only the first image round waits (for that copy, as loads
    // complete in issue order) and W streams at the cache's rate.
    issue(0, 0);
    uint4 raw[FM];
    {
        const int row = lane / 2, half = lane % 2;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int k = 32 * (wv + kSmWaves * i) + row;
            raw[i] = *reinterpret_cast<const uint4*>(w + (int64_t)k * E + (E == 16 ? 8 * half : 0));
        }
    }
    bf16x8 wf[FM];  // from the image rounds
    {
        unsigned char* img = ring[kRgAhead] + wv * (kSmBatch * 1024);
        const int half = lane % 2;
        // with 8 experts the second 16 bytes of an image row are zeros (both
        // halves load the row's 16 bytes; the second is masked)
        const uint32_t keep = E == 16 || half == 0 ? ~0u : 0u;
#pragma unroll
        for (int rr = 0; rr < FM / kSmBatch; ++rr) {
#pragma unroll
            for (int i = 0; i < kSmBatch; ++i) {
                const uint4 v = raw[kSmBatch * rr + i];
                *reinterpret_cast<uint4*>(img + 1024 * i + 16 * lane) =
                    make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
            }
            wave_lds_sync();
#pragma unroll
            for (int i = 0; i < kSmBatch; ++i) {
                i16x4 h2[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int off = 1024 * i + 32 * (8 * q + 4 * h + i16 / 4) + 8 * (i16 % 4);
                    h2[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(img + off));
                }
                wf[kSmBatch * rr + i] = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(h2[0], h2[1], 0, 1, 2, 3, 4, 5, 6, 7));
            }
            wave_lds_sync();
        }
    }
    for (int s = 1; s < kRgAhead; ++s) issue(min<int64_t>(s, steps - 1), s);

    // Step s: wait for this wave's copies of step s (those of the next
    // kRgAhead - 1 steps may stay in flight), then a barrier makes every
    // wave's copies visible and frees the stage of step s - 1 for step
    // s + kRgAhead.  Copies past the last step repeat it into a stage that
    // is never read again.
    f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
    int stage = 0;
    for (int64_t tt = 0; tt * NCH < steps; ++tt) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {  // unrolled: wf is indexed with constants
            const int64_t s = tt * NCH + c;
            wait_vmcnt<kRgCopies * (kRgAhead - 1)>();
            barrier_no_fence();
            issue(min(s + kRgAhead, steps - 1), (stage + kRgAhead) % kRgStages);
            const unsigned char* st = ring[stage];
#pragma unroll
            for (int i = 0; i < kRgFrags; ++i) {
                const int gc = 4 * (wv + kSmWaves * i) + q;  // 16-byte piece of the row's run
                const int off = i16 * (2 * kRgChunk) + 1024 * (gc >> 6) + 16 * ((gc & 63) ^ i16);
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(st + off);
                if (i % 2 == 0)
                    c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, wf[kRgFrags * c + i], c0, 0, 0, 0);
                else
                    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, wf[kRgFrags * c + i], c1, 0, 0, 0);
            }
            stage = stage + 1 == kRgStages ? 0 : stage + 1;
        }
        // D layout: lane (expert i16, quarter q) holds tokens 4q .. 4q+3
#pragma unroll
        for (int r = 0; r < 4; ++r) part[wv][(4 * q + r) * 16 + i16] = c0[r] + c1[r];
        lds_barrier();
        // thread t < 256: token t / 16, expert t % 16; waves added in order
        float v = 0.f;
        if (t < kSmTile * 16) {
#pragma unroll
            for (int x = 0; x < kSmWaves; ++x) v += part[x][t];
            if (cap != 0.0f) v = cap * tanh_f32(v / cap);
        }
        lds_barrier();  // part is free for the next tile
        const int64_t row = (blockIdx.x + tt * gridDim.x) * kSmTile + t / 16;
        if (t < kSmTile * 16)
            route_lanes16_b<E, SOFTMAX, BIAS>(v, t % 16, row < M, bj, K, renorm,
                                              w_out + row * K, id_out + row * K);
#pragma unroll
        for (int r = 0; r < 4; ++r) { c0[r] = 0.f; c1[r] = 0.f; }
    }
    wait_vmcnt<0>();  // no copy is left in flight when the workgroup ends
}

template <int E, int NCH, bool SOFTMAX, bool BIAS>
route_status_t launch_rg_nch(const FusedProblem& f) {
    const RouteProblem& p = f.route;
    const int64_t tiles = (f.M + kSmTile - 1) / kSmTile;
    const int64_t blocks = std::min<int64_t>(tiles, (int64_t)device_cu_count());
    hipLaunchKernelGGL((small_router_ring_kernel<E, NCH, SOFTMAX, BIAS>), dim3((unsigned)blocks),
                       dim3(kSmThreads), 0, p.stream, static_cast<const uint16_t*>(f.hidden),
                       static_cast<const uint16_t*>(f.w), p.bias, f.M, p.K, p.renorm ? 1 : 0,
                       f.softcap, p.weights, p.ids);
    return hipGetLastError() == hipSuccess ? ROUTE_OK : ROUTE_ELAUNCH;
}

bool ring_shape(const FusedProblem& f) {
    return f.H % kRgChunk == 0 && f.H <= kSmHMax;
}

template <int E, bool SOFTMAX, bool BIAS>
route_status_t launch_rg(const FusedProblem& f) {
    switch (f.H / kRgChunk) {
        case 1: return launch_rg_nch<E, 1, SOFTMAX, BIAS>(f);
        case 2: return launch_rg_nch<E, 2, SOFTMAX, BIAS>(f);
        case 3: return launch_rg_nch<E, 3, SOFTMAX, BIAS>(f);
        case 4: return launch_rg_nch<E, 4, SOFTMAX, BIAS>(f);
        case 5: return launch_rg_nch<E, 5, SOFTMAX, BIAS>(f);
        case 6: return launch_rg_nch<E, 6, SOFTMAX, BIAS>(f);
        case 7: return launch_rg_nch<E, 7, SOFTMAX, BIAS>(f);
        default: return launch_rg_nch<E, 8, SOFTMAX, BIAS>(f);
    }
}

template <int E, bool SOFTMAX, bool BIAS>
route_status_t launch_sm(const FusedProblem& f) {
    const int nf = (f.H + 31) / 32;
    const int nb = ((nf + kSmWaves - 1) / kSmWaves + kSmBatch - 1) / kSmBatch;
    switch (nb) {
        case 1: return launch_sm_nb<E, 1, SOFTMAX, BIAS>(f);
        case 2: return launch_sm_nb<E, 2, SOFTMAX, BIAS>(f);
        case 3: return launch_sm_nb<E, 3, SOFTMAX, BIAS>(f);
        case 4: return launch_sm_nb<E, 4, SOFTMAX, BIAS>(f);
        case 5: return launch_sm_nb<E, 5, SOFTMAX, BIAS>(f);
        case 6: return launch_sm_nb<E, 6, SOFTMAX, BIAS>(f);
        case 7: return launch_sm_nb<E, 7, SOFTMAX, BIAS>(f);
        default: return launch_sm_nb<E, 8, SOFTMAX, BIAS>(f);
    }
}

template <int E>
route_status_t launch_sr_e(const FusedProblem& f) {
    const RouteProblem& p = f.route;
    // One MFMA block per 16-token tile leaves compute units idle with few
    // tiles; with 8 experts the vector-ALU kernel (8 tokens per block, half
    // the work per token of 16 experts) measured faster below 64 tiles with
    // the LDS ring (at 1024 tokens 6.6 against 7.8 us, at 512 even) and below
    // 256 tiles with the direct loads.
    if (ring_shape(f) && (E == 16 || f.M >= 64 * kSmTile)) {
        if (p.scoring == ROUTE_SOFTMAX) return launch_rg<E, true, false>(f);
        return p.bias.p ? launch_rg<E, false, true>(f) : launch_rg<E, false, false>(f);
    }
    const bool mfma = f.H <= kSmHMax && (E == 16 || f.M >= 256 * kSmTile);
    if (mfma) {
        if (p.scoring == ROUTE_SOFTMAX) return launch_sm<E, true, false>(f);
        return p.bias.p ? launch_sm<E, false, true>(f) : launch_sm<E, false, false>(f);
    }
    if (p.scoring == ROUTE_SOFTMAX) return launch_sr<E, true, false>(f);
    return p.bias.p ? launch_sr<E, false, true>(f) : launch_sr<E, false, false>(f);
}

}  // namespace

bool small_router_supported(const FusedProblem& f) {
    const RouteProblem& p = f.route;
    const uintptr_t a = reinterpret_cast<uintptr_t>(f.hidden) | reinterpret_cast<uintptr_t>(f.w);
    if ((p.E != 8 && p.E != 16) || f.H % 8 != 0 || (a % 16) != 0) return false;
    if (p.G != 1) return false;
    return !(p.scoring == ROUTE_SOFTMAX && p.bias.p != nullptr);
}

route_status_t launch_small_router(const FusedProblem& f) {
    return f.route.E == 8 ? launch_sr_e<8>(f) : launch_sr_e<16>(f);
}

}  // namespace moe_route
