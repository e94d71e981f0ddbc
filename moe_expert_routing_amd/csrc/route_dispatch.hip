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
// Up to 16384 counts in a coarse matrix (the usual case: 65536 tokens x 8
// slots over 256 experts), two kernels on the caller's stream:
//   1. hist:  one count row per 8192 assignments, cnt[C][E];
//   2. place: as in 3. below, except that each block first reduces the whole
//             coarse matrix itself (its rows before the block's own row give
//             the counts of earlier blocks, all rows the expert totals) and
//             recounts the at most three 2048-assignment chunks of its own
//             row that precede it.
// Otherwise three kernels, with a caller-provided workspace cnt[B][E] +
// totals[E] (B = blocks of kBlockChunk assignments):
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

#include <algorithm>
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

// Coarse counts: one row per kCoarseChunk assignments, read whole by every
// place block when the matrix holds at most kCoarseMaxInts counts.
constexpr int kCoarseThreads = 1024;
constexpr int kCoarsePer = 8;                                    // assignments per thread
constexpr int kCoarseChunk = kCoarseThreads * kCoarsePer;        // 8192 per row
constexpr int kSubPerRow = kCoarseChunk / kBlockChunk;           // 4 place blocks per row
constexpr int kCoarseMaxInts = 16384;                            // 64 KiB
constexpr int kCoarseRowsPerLane = kCoarseMaxInts / 4 / kDispThreads;  // int4 loads, <= 8
static_assert(kCoarseChunk % kBlockChunk == 0, "place blocks tile a coarse row");

__device__ __forceinline__ bool valid_id(int32_t id, int E) { return id >= 0 && id < E; }

// Block b counts assignments [b * THREADS * PER, +THREADS * PER) per expert
// (LDS atomics) into row cnt[b][*].
template <int THREADS, int PER>
__global__ __launch_bounds__(THREADS) void dispatch_hist_kernel(
    const int32_t* __restrict__ ids, int64_t n, int E, int32_t* __restrict__ cnt) {
    extern __shared__ int32_t s_hist[];  // [E]
    const int t = threadIdx.x;
    const int64_t a0 = (int64_t)blockIdx.x * (THREADS * PER) + t;
    int32_t idv[PER];  // all loads in flight at once
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int64_t a = a0 + (int64_t)j * THREADS;
        idv[j] = a < n ? ids[a] : -1;
    }
    for (int e = t; e < E; e += THREADS) s_hist[e] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j)
        if (valid_id(idv[j], E)) atomicAdd(&s_hist[idv[j]], 1);
    __syncthreads();
    for (int e = t; e < E; e += THREADS) cnt[(int64_t)blockIdx.x * E + e] = s_hist[e];
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

// LDS layout of the place kernel: offsets [E + 1], carries [kDispWaves], then
// (16-byte aligned) the per-wave counts and cursors, or first the coarse
// partials.
__host__ __device__ constexpr int place_cur_offset(int E) { return (E + 1 + kDispWaves + 3) & ~3; }

// COARSE: cnt is the coarse matrix [C][E] (E a multiple of 4, 16-byte
// aligned rows, C * E <= kCoarseMaxInts) and totals is unused; otherwise cnt
// holds the scanned rows [B][E] and totals the expert totals.
template <bool COARSE>
__global__ __launch_bounds__(kDispThreads) void dispatch_place_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ wts, int64_t n, int E,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ totals, int C,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ gather,
    int32_t* __restrict__ scatter, float* __restrict__ sorted_w) {
    extern __shared__ int32_t smem[];
    int32_t* s_off = smem;                     // [E + 1] expert offsets
    int32_t* s_wsum = s_off + E + 1;           // [kDispWaves] scan carries
    int32_t* s_cur = smem + place_cur_offset(E);  // [kDispWaves][E] counts, then cursors
    constexpr int kEPT = kMaxExperts / kDispThreads;  // experts per thread (<= 4)
    const int t = threadIdx.x;
    const int lane = t % kWave;
    const int wv = t / kWave;
    // every global load of the block goes out first: this lane's assignments
    // a0 + 64 j, the expert totals (experts kEPT t ..), the block's row of
    // offsets across blocks (COARSE: the coarse matrix and the assignments
    // to recount)
    const int64_t a0 = (int64_t)blockIdx.x * kBlockChunk + (int64_t)wv * kWaveChunk + lane;
    int32_t idv[kPerLane];
    float wv8[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        const int64_t a = a0 + (int64_t)j * kWave;
        idv[j] = a < n ? ids[a] : -1;
        wv8[j] = (sorted_w && a < n) ? wts[a] : 0.0f;
    }
    int tot[kEPT], rowv[kEPT];
    if constexpr (COARSE) {
        // Thread t < Q * G reduces 16-byte quad q = t % Q of rows
        // r = g, g + G, ... (g = t / Q) into a before-my-row and an all-rows
        // partial; the G partials of an expert are added in LDS.  The
        // assignments of the preceding chunks of this block's coarse row are
        // recounted into s_cur row 0.
        const int Q = E / 4, G = kDispThreads / Q;
        const int c = blockIdx.x / kSubPerRow;
        const int q = t % Q, g = t / Q;
        int4 m[kCoarseRowsPerLane];
#pragma unroll
        for (int i = 0; i < kCoarseRowsPerLane; ++i) {
            const int r = g + G * i;
            m[i] = (g < G && r < C)
                       ? reinterpret_cast<const int4*>(cnt + (int64_t)r * E)[q]
                       : make_int4(0, 0, 0, 0);
        }
        const int64_t rc0 = (int64_t)c * kCoarseChunk;
        const int nrc = (blockIdx.x % kSubPerRow) * kBlockChunk;  // assignments to recount
        int32_t rid[kSubPerRow - 1][kPerLane];
#pragma unroll
        for (int u = 0; u < kSubPerRow - 1; ++u)
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) {
                const int o = (u * kPerLane + j) * kDispThreads + t;
                rid[u][j] = o < nrc ? ids[rc0 + o] : -1;  // rc0 + o < n: earlier chunks are full
            }
        int32_t* s_pre = s_cur;                    // [G][E] partials (rows before c)
        int32_t* s_all = s_cur + G * E;            // [G][E] partials (all rows)
        int32_t* s_rc = s_all + G * E;             // [E] recount
        for (int e = t; e < E; e += kDispThreads) s_rc[e] = 0;
        if (g < G) {
            int4 pre = make_int4(0, 0, 0, 0), all = make_int4(0, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < kCoarseRowsPerLane; ++i) {
                all.x += m[i].x; all.y += m[i].y; all.z += m[i].z; all.w += m[i].w;
                if (g + G * i < c) { pre.x += m[i].x; pre.y += m[i].y; pre.z += m[i].z; pre.w += m[i].w; }
            }
            reinterpret_cast<int4*>(s_pre + g * E)[q] = pre;
            reinterpret_cast<int4*>(s_all + g * E)[q] = all;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kSubPerRow - 1; ++u)
#pragma unroll
            for (int j = 0; j < kPerLane; ++j)
                if (valid_id(rid[u][j], E)) atomicAdd(&s_rc[rid[u][j]], 1);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kEPT; ++i) {
            const int e = kEPT * t + i;
            int p = 0, a = 0;
            if (e < E) {
                for (int gg = 0; gg < G; ++gg) {
                    p += s_pre[gg * E + e];
                    a += s_all[gg * E + e];
                }
                p += s_rc[e];
            }
            tot[i] = a;
            rowv[i] = p;
        }
        __syncthreads();  // s_cur is reused below
    } else {
        const int32_t* row = cnt + (int64_t)blockIdx.x * E;
#pragma unroll
        for (int i = 0; i < kEPT; ++i) {
            const int e = kEPT * t + i;
            tot[i] = e < E ? totals[e] : 0;
            rowv[i] = e < E ? row[e] : 0;
        }
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
    static_assert(kMaxExperts % kDispThreads == 0, "experts per place thread");
    const int C = static_cast<int>((d.n + kCoarseChunk - 1) / kCoarseChunk);
    // coarse partial groups of the place kernel: G threads per 16-byte quad,
    // each reducing up to kCoarseRowsPerLane rows
    const int G = d.E >= 4 ? kDispThreads / (d.E / 4) : 0;
    const bool coarse = B > 0 && d.E % 4 == 0 && (int64_t)C * d.E <= kCoarseMaxInts &&
                        C <= kCoarseRowsPerLane * G &&
                        (reinterpret_cast<uintptr_t>(cnt) & 15u) == 0;
    if (coarse) {
        // place LDS: offsets, carries, and the larger of the per-wave counts
        // and the coarse partials (2 G E + E)
        const size_t cur_ints = std::max<size_t>((size_t)kDispWaves * d.E, (size_t)(2 * G + 1) * d.E);
        hipLaunchKernelGGL((dispatch_hist_kernel<kCoarseThreads, kCoarsePer>), dim3(C),
                           dim3(kCoarseThreads), sizeof(int32_t) * d.E, d.stream, d.ids, d.n,
                           d.E, cnt);
        hipLaunchKernelGGL(dispatch_place_kernel<true>, dim3(B), dim3(kDispThreads),
                           sizeof(int32_t) * (place_cur_offset(d.E) + cur_ints), d.stream, d.ids,
                           d.weights, d.n, d.E, cnt, nullptr, C, d.counts, d.offsets, d.gather,
                           d.scatter, d.sorted_weights);
        return hipGetLastError() == hipSuccess ? ROUTE_OK : ROUTE_ELAUNCH;
    }
    int32_t* totals = cnt + static_cast<int64_t>(d.E) * B;
    if (B > 0) {
        hipLaunchKernelGGL((dispatch_hist_kernel<kDispThreads, kPerLane>), dim3(B),
                           dim3(kDispThreads), sizeof(int32_t) * d.E, d.stream, d.ids, d.n, d.E,
                           cnt);
    }
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3((d.E + kWave - 1) / kWave), dim3(kScanThreads),
                       0, d.stream, d.E, B, cnt, totals);
    hipLaunchKernelGGL(dispatch_place_kernel<false>, dim3(B > 0 ? B : 1), dim3(kDispThreads),
                       sizeof(int32_t) * (place_cur_offset(d.E) + kDispWaves * d.E), d.stream,
                       d.ids, d.weights, d.n, d.E, cnt, totals, B, d.counts, d.offsets,
                       d.gather, d.scatter, d.sorted_weights);
    return hipGetLastError() == hipSuccess ? ROUTE_OK : ROUTE_ELAUNCH;
}

}  // namespace moe_route
