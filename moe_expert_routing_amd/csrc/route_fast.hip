// Shape-specialised routing kernels for gfx950, and the dispatch between them
// and the generic kernel.
//
// Layout.  LPR consecutive lanes route one token row; lane `sub` of the row
// holds the VPL consecutive logits [sub*VPL, sub*VPL + VPL), so a wave routes
// 64/LPR rows and its loads are fully coalesced.  With expert groups, the
// kernel requires one group per lane (G == LPR), which turns the group score
// into a lane-local reduction.
//
// Steps ("[SGLang] MoE routing: token-to-expert assignment algorithms"):
//   1. scores: sigmoid, or softmax over the row (sections 2 and 4);
//      selection score c = s + correction_bias (section 4), kept in a
//      per-wave LDS tile.
//   2. group score per lane: max or top-2 sum of c (sections 3 and 4), then
//      the rank of every group among the row's groups by a DPP all-to-all;
//      the best topk_group groups survive (ties: lower group index).
//   3. candidates of the surviving groups are spread over the row's lanes
//      through LDS; each lane turns its candidates into 32-bit keys
//          key = fixed_point(c) << 9 | (511 - expert)
//      whose unsigned order is (c desc, expert asc), and keeps a sorted list
//      of its 4 or 5 best keys (v_max / v_med3 insertion).
//   4. K merge rounds: the row maximum of the list heads (DPP) is the next
//      pick; its lane pops its head.
//   5. weights: the unbiased score of each pick (c - bias, read back from
//      LDS), optionally renormalised; stores.
// The fixed-point step is 2^-23 * R, with R the smallest power of two above
// the range of c (2 for softmax or unbiased sigmoid).  Keys therefore order
// the selection scores exactly up to about 2.4e-7 for R = 2.  When the bias
// spread would make that step coarser than 4.8e-7 (R > 4), or when a lane
// dropped a key that beats the K-th pick, the wave redoes the selection with
// exact (value, index) comparisons on the fp32 scores.
#include <hip/hip_runtime.h>

#include <atomic>

#include "route_common.hpp"
#include "route_tile.hpp"
#include "route_internal.h"

namespace moe_route {

route_status_t launch_route_generic(const RouteProblem& p);

namespace {

constexpr int kWavesPerBlock = 4;
#ifndef MOE_ROUTE_MID_MAX_TOKENS
#define MOE_ROUTE_MID_MAX_TOKENS 4096
#endif
// Ungrouped rows of 256 experts up to this many tokens use 16 lanes a row.
constexpr int64_t kMidMaxTokens = MOE_ROUTE_MID_MAX_TOKENS;
// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left unbounded
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVmcnt0 = 0x0F70;

// Raw logits of one lane (kept packed until scoring so that the next tile's
// loads can be in flight while this tile is scored).
template <typename T, int VPL>
struct RawLane;
template <int VPL>
struct RawLane<uint16_t, VPL> {
    static_assert(VPL % 8 == 0, "bf16 lanes load 16-byte vectors");
    uint4 q[VPL / 8];
    __device__ __forceinline__ void load(const uint16_t* __restrict__ p) {
#pragma unroll
        for (int v = 0; v < VPL / 8; ++v) q[v] = reinterpret_cast<const uint4*>(p)[v];
    }
    __device__ __forceinline__ void unpack(float (&x)[VPL]) const {
#pragma unroll
        for (int v = 0; v < VPL / 8; ++v) {
            const uint32_t w[4] = {q[v].x, q[v].y, q[v].z, q[v].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x[v * 8 + 2 * k] = __uint_as_float(w[k] << 16);
                x[v * 8 + 2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
            }
        }
    }
};
template <int VPL>
struct RawLane<float, VPL> {
    static_assert(VPL % 4 == 0, "f32 lanes load 16-byte vectors");
    float4 q[VPL / 4];
    __device__ __forceinline__ void load(const float* __restrict__ p) {
#pragma unroll
        for (int v = 0; v < VPL / 4; ++v) q[v] = reinterpret_cast<const float4*>(p)[v];
    }
    __device__ __forceinline__ void unpack(float (&x)[VPL]) const {
#pragma unroll
        for (int v = 0; v < VPL / 4; ++v) {
            x[4 * v] = q[v].x; x[4 * v + 1] = q[v].y; x[4 * v + 2] = q[v].z; x[4 * v + 3] = q[v].w;
        }
    }
};

template <typename T, int LPR, int VPL, bool SOFTMAX, bool BIAS, int GRP /*0 none, 1 max, 2 top2*/,
          int SPLIT, int TL, int KMAX>
__global__ __launch_bounds__(kWavesPerBlock* kWave, 3) void route_fast_kernel(
    const T* __restrict__ logits, BiasRef bias, int64_t M, int TG, int K, int renorm,
    float* __restrict__ w_out, int32_t* __restrict__ id_out) {
    constexpr int E = LPR * VPL;
    constexpr int RPW = kWave / LPR;               // rows per wave
    static_assert(GRP == 0 || VPL % SPLIT == 0, "a group splits evenly");
    static_assert(E <= 512, "9 index bits");
    static_assert(LPR == 1 || LPR == 2 || LPR == 4 || LPR == 8 || (LPR == 16 && GRP == 0),
                  "lanes per row");
    static_assert(GRP == 0 || LPR == 8, "grouped kernels hold one of 8 groups per lane");

    // Selection scores of the wave's rows (the candidate exchange and the
    // weights read them); the block's staged bias offsets.
    constexpr int ROW = LPR > 1 ? E : 4;  // fp32 values per row in LDS
    __shared__ __align__(16) float s_s[kWavesPerBlock][RPW * ROW];
    __shared__ __align__(16) float s_bias[BIAS ? E : 4];

    const int lane = threadIdx.x % kWave;
    const int wv = threadIdx.x / kWave;
    const int sub = lane % LPR;
    const int rw = lane / LPR;  // row within the wave
    float* my_row = s_s[wv] + (LPR > 1 ? rw * ROW : 0);

    const int64_t tiles = (M + RPW - 1) / RPW;
    const int64_t tstride = (int64_t)gridDim.x * kWavesPerBlock;
    int64_t tile = (int64_t)blockIdx.x * kWavesPerBlock + wv;
    // Rows of a tile past M read row M-1 (computed, never stored).
    auto load_tile = [&](RawLane<T, VPL>& r, int64_t t) {
        const int64_t row = min(t * RPW + rw, M - 1);
        r.load(logits + row * E + sub * VPL);
    };
    // The bias (four entries per lane, fp32 or bf16) is requested before the
    // first tile, so that the prologue below needs only the bias to have
    // arrived.
    static_assert(!BIAS || E <= 4 * kWave, "four bias entries per lane");
    const bool has_b = BIAS && 4 * lane < E;
    float4 bq = make_float4(0.f, 0.f, 0.f, 0.f);
    if (has_b) bq = bias4_at(bias, lane);
    RawLane<T, VPL> ra, rb;  // ping-pong: one tile routed while the next loads
    // In flight during the prologue below.  A wave without a tile loads the
    // last one anyway: with the load unconditional, the prologue's wait
    // counts the bias alone.
    load_tile(ra, tile < tiles ? tile : tiles - 1);

    // ---- key window.  Keys are compared only within a row; the window holds
    // every selection score c = s + bias of any row, so it comes from the
    // range of the bias, reduced over the wave.
    KeyParams kp;
    if constexpr (BIAS) {
        const float bmin = has_b ? fminf(fminf(bq.x, bq.y), fminf(bq.z, bq.w)) : INFINITY;
        const float bmax = has_b ? fmaxf(fmaxf(bq.x, bq.y), fmaxf(bq.z, bq.w)) : -INFINITY;
        kp = key_params(wave_min_all(bmin), 1.0f + wave_max_all(bmax));
        if (wv == 0 && has_b)
            *reinterpret_cast<float4*>(s_bias + bias_chunk<E>(lane) * 4) =
                make_float4(sel_offset(bq.x, kp), sel_offset(bq.y, kp), sel_offset(bq.z, kp),
                            sel_offset(bq.w, kp));
        __syncthreads();
    } else {
        kp = key_params(0.0f, 1.0f);
    }

    // The row's outputs move by a fixed stride from one tile of the wave to
    // the next (no multiply by the runtime K in the loop).
    const int64_t out_step = tstride * RPW * K;
    int64_t out_off = (tile * RPW + rw) * K;
    auto route_tile = [&](const RawLane<T, VPL>& r, int64_t t) {
        const int64_t row = t * RPW + rw;
        const bool valid = row < M;
        float x[VPL];
        r.unpack(x);
        const T* xr = logits + (valid ? row : 0) * E;
        route_rows<LPR, VPL, SOFTMAX, BIAS, GRP, SPLIT, TL, KMAX>(
            x, sub, rw, valid, my_row, s_bias, kp, TG, K, renorm, w_out + out_off,
            id_out + out_off, [&](int e) { return load_one<T>(xr, e); },
            [&](int e) { return BIAS ? bias_at(bias, e) : 0.0f; });
        out_off += out_step;
    };
    // The second tile is requested only once the first has arrived: at the
    // start every wave of the grid requests at once, and second tiles
    // requested alongside the first ones delay them.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    while (tile < tiles) {
        if (tile + tstride < tiles) load_tile(rb, tile + tstride);
        route_tile(ra, tile);
        tile += tstride;
        if (tile >= tiles) break;
        if (tile + tstride < tiles) load_tile(ra, tile + tstride);
        route_tile(rb, tile);
        tile += tstride;
    }
}


template <typename T, int LPR, int VPL, bool SOFTMAX, bool BIAS, int GRP, int SPLIT, int TL,
          int KMAX>
route_status_t launch_fast(const RouteProblem& p) {
    constexpr int RPW = kWave / LPR;
    auto kernel = route_fast_kernel<T, LPR, VPL, SOFTMAX, BIAS, GRP, SPLIT, TL, KMAX>;
    // Persistent grid: every block resident at once, tiles strided over them.
    // Blocks per CU for this instantiation (a thread-safe one-time query).
    static const int resident = resident_blocks(kernel, kWavesPerBlock * kWave);
    const int64_t tiles = (p.M + RPW - 1) / RPW;
    int64_t blocks = (tiles + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t cap = (int64_t)device_cu_count() * resident;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kWavesPerBlock * kWave), 0, p.stream,
                       static_cast<const T*>(p.logits), p.bias, p.M, p.TG, p.K,
                       p.renorm ? 1 : 0, p.weights, p.ids);
    return hipGetLastError() == hipSuccess ? ROUTE_OK : ROUTE_ELAUNCH;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// E = 256 (or 160) with one group per lane (G == 8) or no groups.  With
// groups, each surviving group is split over two lanes.  A lane keeps its 4
// (grouped) or 5 (ungrouped, more candidates per lane) best keys; on the
// synthetic workloads a row needs more than that from one lane in well under
// 1% of waves, which then take the exact path.
template <typename T, int VPL, int KMAX>
route_status_t dispatch_lpr8_k(const RouteProblem& p, bool& handled) {
    constexpr int TLU = KMAX < 5 ? KMAX : 5;  // list length, ungrouped
    constexpr int TLG = KMAX < 4 ? KMAX : 4;  // list length, grouped
    handled = true;
    const bool soft = p.scoring == ROUTE_SOFTMAX;
    const bool bias = p.bias.p != nullptr;
    if (p.G == 1) {
        if constexpr (VPL == 32) {
            // up to kMidMaxTokens, 16 lanes a row: twice the waves, each
            // with half the experts per lane
            if (p.M <= kMidMaxTokens) {
                if (soft) return launch_fast<T, 16, 16, true, false, 0, 1, TLU, KMAX>(p);
                if (bias) return launch_fast<T, 16, 16, false, true, 0, 1, TLU, KMAX>(p);
                return launch_fast<T, 16, 16, false, false, 0, 1, TLU, KMAX>(p);
            }
        }
        if (soft) return launch_fast<T, 8, VPL, true, false, 0, 1, TLU, KMAX>(p);
        if (bias) return launch_fast<T, 8, VPL, false, true, 0, 1, TLU, KMAX>(p);
        return launch_fast<T, 8, VPL, false, false, 0, 1, TLU, KMAX>(p);
    }
    if (p.G == 8 && p.TG <= 4) {
        if (p.rule == ROUTE_GROUP_TOP2_SUM) {
            if (soft) { handled = false; return ROUTE_OK; }
            if (bias) return launch_fast<T, 8, VPL, false, true, 2, 2, TLG, KMAX>(p);
            return launch_fast<T, 8, VPL, false, false, 2, 2, TLG, KMAX>(p);
        }
        if (soft) return launch_fast<T, 8, VPL, true, false, 1, 2, TLG, KMAX>(p);
        if (bias) return launch_fast<T, 8, VPL, false, true, 1, 2, TLG, KMAX>(p);
        return launch_fast<T, 8, VPL, false, false, 1, 2, TLG, KMAX>(p);
    }
    handled = false;
    return ROUTE_OK;
}

template <typename T, int VPL>
route_status_t dispatch_lpr8(const RouteProblem& p, bool& handled) {
    if (p.K <= 8) return dispatch_lpr8_k<T, VPL, 8>(p, handled);
    handled = false;
    return ROUTE_OK;
}

}  // namespace

int device_cu_count() {
    // Per-device cache; concurrent first calls may both query, and store the
    // same value.
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

route_status_t launch_route(const RouteProblem& p) {
    const size_t esz = p.dtype == ROUTE_F32 ? 4 : 2;
    const bool vec_ok = aligned16(p.logits) && ((size_t)p.E * esz) % 16 == 0 &&
                        (p.bias.p == nullptr ||
                         (reinterpret_cast<uintptr_t>(p.bias.p) % (p.bias.bf16 ? 8 : 16)) == 0);
    if (vec_ok && route_row_supported(p)) return launch_route_row(p);
    bool handled = false;
    route_status_t st = ROUTE_OK;
    if (vec_ok) {
        if (p.E == 256) {
            st = p.dtype == ROUTE_F32 ? dispatch_lpr8<float, 32>(p, handled)
                                      : dispatch_lpr8<uint16_t, 32>(p, handled);
        } else if (p.E == 160 && p.dtype == ROUTE_F32) {
            st = dispatch_lpr8<float, 20>(p, handled);
        } else if (p.E == 8 && p.G == 1 && p.dtype == ROUTE_F32 && p.K <= 2) {
            handled = true;
            if (p.scoring == ROUTE_SOFTMAX)
                st = launch_fast<float, 1, 8, true, false, 0, 1, 2, 2>(p);
            else if (p.bias.p)
                st = launch_fast<float, 1, 8, false, true, 0, 1, 2, 2>(p);
            else
                st = launch_fast<float, 1, 8, false, false, 0, 1, 2, 2>(p);
        }
    }
    if (handled) return st;
    return launch_route_generic(p);
}

}  // namespace moe_route
