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
// workspace cnt[B][E] + totals[E] (B = blocks of kBlockChunk assignments):
//   1. hist:  each block counts its chunk per expert (LDS atomics) into its
//             row cnt[b][*];
//   2. scan:  64 experts per block, each column cnt[*][e] split over 16
//             segments (held in registers between its two passes), turns
//             each column into exclusive offsets across blocks and writes
//             the expert's total;
//   3. place: each block scans the totals into expert offsets (block 0 also
//             writes counts and offsets), recounts its chunk per wave, so that every wave
//             starts from its own cursor per expert (the expert offset plus
//             the counts of earlier blocks and earlier waves), then walks its
//             part 64 assignments at a time.  Lanes with the same expert find
//             each other with one ballot per bit of the expert id; a lane's
//             rank among them (mbcnt) plus its wave's cursor is its sorted
//             position, so equal ids keep their order without ordered
//             atomics.
#include <hip/hip_runtime.h>

#include <atomic>

#include "route_common.hpp"
#include "route_internal.h"

namespace moe_route {
namespace {

// Scratch of route_dispatch_metadata_noalloc (cnt[B][E] + totals[E]), for
// callers that cannot allocate.  Each device holds its own copy until the
// process ends.  On the host, `scratch` names a stand-in, not a device
// address: host code uses only the address hipGetSymbolAddress returns for
// the current device (dispatch_noalloc_scratch below).
constexpr size_t kNoAllocScratchInts = size_t(1) << 20;  // 4 MiB
static __device__ __align__(256) int32_t scratch[kNoAllocScratchInts];

constexpr int kDispWaves = 8;                            // 2 per SIMD: shorter place loops
constexpr int kDispThreads = kDispWaves * kWave;
constexpr int kPerLane = 4;                              // assignments per lane
constexpr int kWaveChunk = kPerLane * kWave;             // 256 per wave
constexpr int kBlockChunk = kDispWaves * kWaveChunk;     // 2048 per block
constexpr int kScanThreads = 1024;                       // >= max experts
constexpr int kScanBatch = 16;                           // loads in flight per thread

__device__ __forceinline__ bool valid_id(int32_t id, int E) { return id >= 0 && id < E; }

__global__ __launch_bounds__(kDispThreads) void dispatch_hist_kernel(
    const int32_t* __restrict__ ids, int64_t n, int E, int32_t* __restrict__ cnt) {
    extern __shared__ int32_t s_hist[];  // [E]
    const int t = threadIdx.x;
    const int64_t a0 = (int64_t)blockIdx.x * kBlockChunk + t;
    int32_t idv[kPerLane];  // all loads in flight at once
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        const int64_t a = a0 + (int64_t)j * kDispThreads;
        idv[j] = a < n ? ids[a] : -1;
    }
    for (int e = t; e < E; e += kDispThreads) s_hist[e] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPerLane; ++j)
        if (valid_id(idv[j], E)) atomicAdd(&s_hist[idv[j]], 1);
    __syncthreads();
    for (int e = t; e < E; e += kDispThreads) cnt[(int64_t)blockIdx.x * E + e] = s_hist[e];
}

// Block x, thread t: expert e = 64 x + t % 64 over segment t / 64 of the
// block rows.  Segments combine in LDS; each column is rewritten as exclusive
// offsets across blocks and the expert's total is written.
__global__ __launch_bounds__(kScanThreads) void dispatch_scan_kernel(
    int E, int B, int32_t* __restrict__ cnt, int32_t* __restrict__ totals) {
    constexpr int S = kScanThreads / kWave;  // 16 segments
    __shared__ int32_t s_part[S][kWave];
    const int t = threadIdx.x;
    const int lane = t % kWave, seg = t / kWave;
    const int e = blockIdx.x * kWave + lane;
    const bool active = e < E;
    const int per = (B + S - 1) / S;
    const int b0 = min(seg * per, B), b1 = min(b0 + per, B);
    // up to S * kScanBatch blocks a segment stays in registers between the
    // two passes; beyond, the second pass reads it again
    const bool held = per <= kScanBatch;
    int v[kScanBatch];
    int part = 0;
    if (held) {
#pragma unroll
        for (int i = 0; i < kScanBatch; ++i)
            v[i] = (active && b0 + i < b1) ? cnt[(int64_t)(b0 + i) * E + e] : 0;
#pragma unroll
        for (int i = 0; i < kScanBatch; ++i) part += v[i];
    } else {
        for (int b = b0; b < b1; b += kScanBatch) {
#pragma unroll
            for (int i = 0; i < kScanBatch; ++i)
                v[i] = (active && b + i < b1) ? cnt[(int64_t)(b + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < kScanBatch; ++i) part += v[i];
        }
    }
    s_part[seg][lane] = part;
    __syncthreads();
    int start = 0, total = 0;
    for (int q = 0; q < S; ++q) {
        const int v = s_part[q][lane];
        if (q < seg) start += v;
        total += v;
    }
    if (active) {
        if (held) {
#pragma unroll
            for (int i = 0; i < kScanBatch; ++i) {
                if (b0 + i < b1) cnt[(int64_t)(b0 + i) * E + e] = start;
                start += v[i];
            }
        } else {
            for (int b = b0; b < b1; b += kScanBatch) {
#pragma unroll
                for (int i = 0; i < kScanBatch; ++i)
                    v[i] = (b + i < b1) ? cnt[(int64_t)(b + i) * E + e] : 0;
#pragma unroll
                for (int i = 0; i < kScanBatch; ++i) {
                    if (b + i < b1) cnt[(int64_t)(b + i) * E + e] = start;
                    start += v[i];
                }
            }
        }
        if (seg == 0) totals[e] = total;
    }
}

__global__ __launch_bounds__(kDispThreads) void dispatch_place_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ wts, int64_t n, int E,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ totals,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ gather,
    int32_t* __restrict__ scatter, float* __restrict__ sorted_w) {
    extern __shared__ int32_t smem[];
    int32_t* s_off = smem;                     // [E + 1] expert offsets
    int32_t* s_wsum = s_off + E + 1;           // [kDispWaves] scan carries
    int32_t* s_cur = s_wsum + kDispWaves;      // [kDispWaves][E] counts, then cursors
    constexpr int kEPT = kMaxExperts / kDispThreads;  // experts per thread (<= 4)
    const int t = threadIdx.x;
    const int lane = t % kWave;
    const int wv = t / kWave;
    // every global load of the block goes out first: this lane's assignments
    // a0 + 64 j, the expert totals (experts kEPT t ..), the block's row of
    // offsets across blocks
    const int64_t a0 = (int64_t)blockIdx.x * kBlockChunk + (int64_t)wv * kWaveChunk + lane;
    int32_t idv[kPerLane];
    float wv8[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        const int64_t a = a0 + (int64_t)j * kWave;
        idv[j] = a < n ? ids[a] : -1;
        wv8[j] = (sorted_w && a < n) ? wts[a] : 0.0f;
    }
    const int32_t* row = cnt + (int64_t)blockIdx.x * E;
    int tot[kEPT], rowv[kEPT];
#pragma unroll
    for (int i = 0; i < kEPT; ++i) {
        const int e = kEPT * t + i;
        tot[i] = e < E ? totals[e] : 0;
        rowv[i] = e < E ? row[e] : 0;
    }
    // expert offsets: exclusive scan of the totals over the block
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kEPT; ++i) sum += tot[i];
    int incl = sum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += v;
    }
    if (lane == kWave - 1) s_wsum[wv] = incl;
    for (int i = t; i < kDispWaves * E; i += kDispThreads) s_cur[i] = 0;
    __syncthreads();
    int run = incl - sum;
    for (int q = 0; q < wv; ++q) run += s_wsum[q];
#pragma unroll
    for (int i = 0; i < kEPT; ++i) {
        const int e = kEPT * t + i;
        if (e < E) s_off[e] = run;
        run += tot[i];
    }
    if (t == kDispThreads - 1) s_off[E] = run;
    int32_t* cur = s_cur + wv * E;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j)
        if (valid_id(idv[j], E)) atomicAdd(&cur[idv[j]], 1);
    __syncthreads();
    if (blockIdx.x == 0) {
#pragma unroll
        for (int i = 0; i < kEPT; ++i) {
            const int e = kEPT * t + i;
            if (e < E) {
                counts[e] = tot[i];
                offsets[e] = s_off[e];
            }
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
    // cursor of wave q for expert e: expert offset + earlier blocks + earlier waves
#pragma unroll
    for (int i = 0; i < kEPT; ++i) {
        const int e = kEPT * t + i;
        if (e < E) {
            int c = s_off[e] + rowv[i];
#pragma unroll
            for (int q = 0; q < kDispWaves; ++q) {
                const int v = s_cur[q * E + e];
                s_cur[q * E + e] = c;
                c += v;
            }
        }
    }
    __syncthreads();
    // expert ids need nb bits; the all-ones pattern of nb bits is >= E and
    // tags dropped or absent assignments
    const int nb = 32 - __clz(E);
    const uint32_t none = (1u << nb) - 1u;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        const int64_t a = a0 + (int64_t)j * kWave;
        const int32_t id = idv[j];
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
            if (sorted_w) sorted_w[p] = wv8[j];
            if (rank == size - 1) cur[id] = start + size;  // one writer per expert
        } else if (a < n) {
            scatter[a] = -1;
        }
    }
}

}  // namespace

size_t dispatch_noalloc_scratch_bytes() { return sizeof(int32_t) * kNoAllocScratchInts; }

void* dispatch_noalloc_scratch() {
    // Device address of `scratch` on the current device, looked up on the
    // first call on each device (with that device current) and kept.
    static std::atomic<void*> addr[64];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return nullptr;
        addr[dev].store(p, std::memory_order_release);
    }
    return p;
}

size_t dispatch_workspace_bytes(int64_t n, int E) {
    const int64_t B = (n + kBlockChunk - 1) / kBlockChunk;
    return sizeof(int32_t) * static_cast<size_t>(E) * static_cast<size_t>(B + 1);
}

route_status_t launch_dispatch(const DispatchProblem& d) {
    const int B = static_cast<int>((d.n + kBlockChunk - 1) / kBlockChunk);
    int32_t* cnt = static_cast<int32_t*>(d.workspace);
    int32_t* totals = cnt + static_cast<int64_t>(d.E) * B;
    static_assert(kMaxExperts % kDispThreads == 0, "experts per place thread");
    if (B > 0) {
        hipLaunchKernelGGL(dispatch_hist_kernel, dim3(B), dim3(kDispThreads),
                           sizeof(int32_t) * d.E, d.stream, d.ids, d.n, d.E, cnt);
    }
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3((d.E + kWave - 1) / kWave), dim3(kScanThreads),
                       0, d.stream, d.E, B, cnt, totals);
    hipLaunchKernelGGL(dispatch_place_kernel, dim3(B > 0 ? B : 1), dim3(kDispThreads),
                       sizeof(int32_t) * (d.E + 1 + kDispWaves + kDispWaves * d.E), d.stream,
                       d.ids, d.weights, d.n, d.E, cnt, totals, d.counts, d.offsets, d.gather,
                       d.scatter, d.sorted_weights);
    return hipGetLastError() == hipSuccess ? ROUTE_OK : ROUTE_ELAUNCH;
}

}  // namespace moe_route
