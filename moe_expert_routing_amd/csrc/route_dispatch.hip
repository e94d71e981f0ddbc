// Expert-sorted dispatch metadata of a routing result (gfx950).
//
// The routing page ("[SGLang] MoE routing: token-to-expert assignment
// algorithms", section "output format") names a kernel-oriented output made of
// routing data, a gather index and a scatter index.  Here that is the stable
// order of the M*K (token, slot) assignments a = m*K + k by expert id:
// per-expert counts and offsets, the assignment at each sorted position
// (gather), the sorted position of each assignment (scatter), and the
// weights in sorted order.  Ids outside [0, E) are dropped.
//
// Three kernels, all on the caller's stream, with a caller-provided
// workspace cnt[E][W] + totals[E] (W = chunks of kChunk assignments):
//   1. hist:  each wave counts its chunk's assignments per expert (LDS
//             atomics in a wave-private histogram) into cnt[e][w];
//   2. scan:  one wave per expert turns cnt[e][*] into exclusive offsets
//             across chunks and writes the expert's total;
//   3. place: every block scans the totals into expert offsets; each wave
//             walks its chunk 64 assignments at a time.  Lanes with the same
//             expert find each other with one ballot per bit of the expert
//             id; a lane's rank among them (mbcnt) plus the expert's running
//             cursor (wave-private LDS) is its sorted position, so equal ids
//             keep their order without ordered atomics.
#include <hip/hip_runtime.h>

#include "route_common.cuh"
#include "route_internal.h"

namespace moe_route {
namespace {

constexpr int kChunk = 512;  // assignments per wave chunk
constexpr int kDispWaves = 4;
constexpr int kDispThreads = kDispWaves * kWave;

__device__ __forceinline__ bool valid_id(int32_t id, int E) { return id >= 0 && id < E; }

__global__ __launch_bounds__(kDispThreads) void dispatch_hist_kernel(
    const int32_t* __restrict__ ids, int64_t n, int E, int W, int32_t* __restrict__ cnt) {
    extern __shared__ int32_t s_hist[];  // [kDispWaves][E]
    const int lane = threadIdx.x % kWave;
    const int wv = threadIdx.x / kWave;
    const int w = blockIdx.x * kDispWaves + wv;
    if (w >= W) return;  // no block-wide barrier in this kernel
    int32_t* h = s_hist + wv * E;
    for (int e = lane; e < E; e += kWave) h[e] = 0;
    // A wave's LDS operations complete in order: the zeros land before the
    // increments, the increments before the reads below.
    const int64_t a0 = (int64_t)w * kChunk;
    const int64_t a1 = min(a0 + kChunk, n);
    for (int64_t a = a0 + lane; a < a1; a += kWave) {
        const int32_t id = ids[a];
        if (valid_id(id, E)) atomicAdd(&h[id], 1);
    }
    for (int e = lane; e < E; e += kWave) cnt[(int64_t)e * W + w] = h[e];
}

__global__ __launch_bounds__(kWave) void dispatch_scan_kernel(int W, int32_t* __restrict__ cnt,
                                                              int32_t* __restrict__ totals) {
    const int e = blockIdx.x;
    const int lane = threadIdx.x;
    int32_t* row = cnt + (int64_t)e * W;
    const int per = (W + kWave - 1) / kWave;
    const int b0 = min(lane * per, W), b1 = min(b0 + per, W);
    int sum = 0;
    for (int i = b0; i < b1; ++i) sum += row[i];
    int incl = sum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += v;
    }
    int run = incl - sum;
    for (int i = b0; i < b1; ++i) {
        const int c = row[i];
        row[i] = run;
        run += c;
    }
    if (lane == kWave - 1) totals[e] = incl;
}

__global__ __launch_bounds__(kDispThreads) void dispatch_place_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ wts, int64_t n, int E, int W,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ totals,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ gather,
    int32_t* __restrict__ scatter, float* __restrict__ sorted_w) {
    extern __shared__ int32_t smem[];
    int32_t* s_off = smem;               // [E + 1] expert offsets
    int32_t* s_wsum = smem + E + 1;      // [kDispWaves] scan carries
    int32_t* s_run = s_wsum + kDispWaves;  // [kDispWaves][E] running cursors
    const int t = threadIdx.x;
    const int lane = t % kWave;
    const int wv = t / kWave;

    // expert offsets: exclusive scan of the totals over the block
    const int per = (E + kDispThreads - 1) / kDispThreads;
    const int e0 = min(t * per, E), e1 = min(e0 + per, E);
    int sum = 0;
    for (int e = e0; e < e1; ++e) sum += totals[e];
    int incl = sum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += v;
    }
    if (lane == kWave - 1) s_wsum[wv] = incl;
    __syncthreads();
    int carry = 0;
    for (int q = 0; q < wv; ++q) carry += s_wsum[q];
    int run = carry + incl - sum;
    for (int e = e0; e < e1; ++e) {
        s_off[e] = run;
        run += totals[e];
    }
    if (t == kDispThreads - 1) s_off[E] = carry + incl;
    __syncthreads();
    if (blockIdx.x == 0) {
        for (int e = t; e < E; e += kDispThreads) {
            counts[e] = totals[e];
            offsets[e] = s_off[e];
        }
        if (t == 0) offsets[E] = s_off[E];
    }
    const int64_t nvalid = s_off[E];
    // sorted positions past the valid assignments
    for (int64_t p = nvalid + (int64_t)blockIdx.x * kDispThreads + t; p < n;
         p += (int64_t)gridDim.x * kDispThreads) {
        gather[p] = -1;
        if (sorted_w) sorted_w[p] = 0.0f;
    }

    const int w = blockIdx.x * kDispWaves + wv;
    if (w >= W) return;  // no block-wide barrier below
    int32_t* cur = s_run + wv * E;
    for (int e = lane; e < E; e += kWave) cur[e] = s_off[e] + cnt[(int64_t)e * W + w];
    // expert ids need nb bits; the all-ones pattern of nb bits is >= E and
    // tags dropped or absent assignments
    const int nb = 32 - __clz(E);
    const uint32_t none = (1u << nb) - 1u;
    const int64_t a0 = (int64_t)w * kChunk;
    const int64_t a1 = min(a0 + kChunk, n);
    for (int64_t base = a0; base < a1; base += kWave) {
        const int64_t a = base + lane;
        const bool in = a < a1;
        const int32_t id = in ? ids[a] : -1;
        const bool ok = valid_id(id, E);
        const uint32_t key = ok ? static_cast<uint32_t>(id) : none;
        uint64_t same = ~0ull;  // lanes whose key equals this lane's
        for (int b = 0; b < nb; ++b) {
            const bool bit = (key >> b) & 1u;
            const uint64_t m = __ballot(bit);
            same &= bit ? m : ~m;
        }
        const int rank = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(same >> 32),
                                                   __builtin_amdgcn_mbcnt_lo(
                                                       static_cast<uint32_t>(same), 0u));
        const int size = __popcll(same);
        if (ok) {
            const int32_t start = cur[id];
            const int32_t p = start + rank;
            gather[p] = static_cast<int32_t>(a);
            scatter[a] = p;
            if (sorted_w) sorted_w[p] = wts[a];
            if (rank == size - 1) cur[id] = start + size;  // one writer per expert
        } else if (in) {
            scatter[a] = -1;
        }
    }
}

}  // namespace

size_t dispatch_workspace_bytes(int64_t n, int E) {
    const int64_t W = (n + kChunk - 1) / kChunk;
    return sizeof(int32_t) * static_cast<size_t>(E) * static_cast<size_t>(W + 1);
}

route_status_t launch_dispatch(const DispatchProblem& d) {
    const int64_t W64 = (d.n + kChunk - 1) / kChunk;
    const int W = static_cast<int>(W64);
    int32_t* cnt = static_cast<int32_t*>(d.workspace);
    int32_t* totals = cnt + static_cast<int64_t>(d.E) * W;
    const int blocks = W > 0 ? (W + kDispWaves - 1) / kDispWaves : 1;
    if (W > 0) {
        hipLaunchKernelGGL(dispatch_hist_kernel, dim3(blocks), dim3(kDispThreads),
                           sizeof(int32_t) * kDispWaves * d.E, d.stream, d.ids, d.n, d.E, W, cnt);
    }
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(d.E), dim3(kWave), 0, d.stream, W, cnt, totals);
    hipLaunchKernelGGL(dispatch_place_kernel, dim3(blocks), dim3(kDispThreads),
                       sizeof(int32_t) * (d.E + 1 + kDispWaves + kDispWaves * d.E), d.stream,
                       d.ids, d.weights, d.n, d.E, W, cnt, totals, d.counts, d.offsets, d.gather,
                       d.scatter, d.sorted_weights);
    return hipGetLastError() == hipSuccess ? ROUTE_OK : ROUTE_ELAUNCH;
}

}  // namespace moe_route
