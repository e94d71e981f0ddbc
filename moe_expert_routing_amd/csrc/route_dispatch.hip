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
//   1. hist:  one count row per 8192 assignments, cnt[C][E], and for each
//             place block after the first of a row, the counts of the row's
//             2048-assignment chunks before it (a prefix row);
//   2. place: as in 3. below, except that each block first reduces the whole
//             coarse matrix itself (its rows before the block's own row give
//             the counts of earlier blocks, all rows the expert totals) and
//             adds its prefix row.
// Otherwise three kernels, with a caller-provided workspace cnt[B][E] +
// totals[E] (B = blocks of kBlockChunk assignments):
//   1. hist:  each block counts its chunk per expert (LDS atomics) into its
//             row cnt[b][*];
//   2. scan:  64 experts per block, each column cnt[*][e] split over 16
//             segments (held in registers between its two passes), turns
//             each column into exclusive offsets across blocks and writes
//             the expert's total;
//   3. place: each block scans the totals into expert offsets (block 0 also
//             writes counts and offsets) and its own per-expert counts into
//             block slots (its assignments in expert order, each wave
//             starting from its own cursor per expert), then walks its part
//             64 assignments at a time.  Lanes with the same expert find each
//             other with one ballot per bit of the expert id; a lane's rank
//             among them (mbcnt) plus its wave's cursor is its block slot, so
//             equal ids keep their order without ordered atomics.  The
//             scatter index is stored at once; the slots go through LDS and
//             are stored in slot order, so that each expert's run of the
//             block lands in consecutive gather and weight entries instead of
//             one scattered 4-byte store per assignment.
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

// Row of the coarse workspace that holds, for place block kSubPerRow c + s
// (s >= 1), the counts of coarse row c's chunks before it.  The C coarse
// rows come first; rows exist only for place blocks that exist, so the B
// place blocks need B rows in all.
__host__ __device__ constexpr int64_t coarse_prefix_row(int C, int c, int s) {
    return (int64_t)C + (int64_t)(kSubPerRow - 1) * c + s - 1;
}

// Coarse row c = block x: its kCoarseChunk assignments counted per expert
// (LDS atomics, one histogram per place-block chunk) into cnt[c][*], and for
// each later place block of the row the counts of the chunks before it into
// its prefix row.  B = place blocks.
__global__ __launch_bounds__(kCoarseThreads) void dispatch_hist_coarse_kernel(
    const int32_t* __restrict__ ids, int64_t n, int E, int C, int B, int32_t* __restrict__ cnt) {
    extern __shared__ int32_t s_hist[];  // [kSubPerRow][E]
    constexpr int kPerChunk = kBlockChunk / kCoarseThreads;  // loads of a thread per chunk
    static_assert(kBlockChunk % kCoarseThreads == 0 && kCoarsePer == kSubPerRow * kPerChunk,
                  "a thread's loads j fall in chunk j / kPerChunk");
    const int t = threadIdx.x;
    const int c = blockIdx.x;
    const int64_t a0 = (int64_t)c * kCoarseChunk + t;
    int32_t idv[kCoarsePer];  // all loads in flight at once
#pragma unroll
    for (int j = 0; j < kCoarsePer; ++j) {
        const int64_t a = a0 + (int64_t)j * kCoarseThreads;
        idv[j] = a < n ? ids[a] : -1;
    }
    for (int i = t; i < kSubPerRow * E; i += kCoarseThreads) s_hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kCoarsePer; ++j)
        if (valid_id(idv[j], E)) atomicAdd(&s_hist[(j / kPerChunk) * E + idv[j]], 1);
    __syncthreads();
    for (int e = t; e < E; e += kCoarseThreads) {
        int run = 0;
#pragma unroll
        for (int sb = 0; sb < kSubPerRow; ++sb) {
            if (sb > 0 && kSubPerRow * c + sb < B) cnt[coarse_prefix_row(C, c, sb) * E + e] = run;
            run += s_hist[sb * E + e];
        }
        cnt[(int64_t)c * E + e] = run;
    }
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

// LDS layout of the place kernel, in ints: expert offsets [E + 1], scan
// carries [2 kDispWaves], per-expert global bases [E]; then, 16-byte
// aligned, the per-wave counts and cursors [kDispWaves][E], and a region
// that first holds the coarse partials [2 G][E] (COARSE) and afterwards the
// block's assignments in sorted order [kBlockChunk] and their weights
// [kBlockChunk].  At most 56 KiB (E = 1024).
struct PlaceLds {
    int off, wsum, gb, cnt, slot, slot_w, pre, all, ints;
};
__host__ __device__ constexpr PlaceLds place_lds(int E, int G) {
    PlaceLds l{};
    l.off = 0;
    l.wsum = E + 1;
    l.gb = l.wsum + 2 * kDispWaves;
    l.cnt = (l.gb + E + 3) & ~3;
    l.slot = l.cnt + kDispWaves * E;
    l.slot_w = l.slot + kBlockChunk;
    l.pre = l.slot;
    l.all = l.pre + G * E;
    const int tail = 2 * G * E;
    l.ints = l.slot + (tail > 2 * kBlockChunk ? tail : 2 * kBlockChunk);
    return l;
}
static_assert(place_lds(kMaxExperts, kDispThreads / (kMaxExperts / 4)).ints * 4 <= 64 * 1024,
              "place kernel LDS within 64 KiB");
constexpr int kLocalBits = 11;  // assignment index within a block
static_assert(kBlockChunk == 1 << kLocalBits, "block-local index width");
static_assert(kMaxExperts << kLocalBits <= 0x7fffffff, "expert and local index in one int");

// COARSE: cnt is the coarse matrix [C][E] (E a multiple of 4, 16-byte
// aligned rows, C * E <= kCoarseMaxInts) followed by the prefix rows of
// dispatch_hist_coarse_kernel, and totals is unused; otherwise cnt holds the
// scanned rows [B][E] and totals the expert totals.
template <bool COARSE>
__global__ __launch_bounds__(kDispThreads) void dispatch_place_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ wts, int64_t n, int E,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ totals, int C,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ gather,
    int32_t* __restrict__ scatter, float* __restrict__ sorted_w) {
    extern __shared__ int32_t smem[];
    const int G = COARSE ? kDispThreads / (E / 4) : 0;
    const PlaceLds L = place_lds(E, G);
    int32_t* s_off = smem + L.off;    // [E + 1] expert offsets
    int32_t* s_wsum = smem + L.wsum;  // [2][kDispWaves] scan carries
    int32_t* s_gb = smem + L.gb;      // [E] sorted position = s_gb[e] + block slot
    int32_t* s_cnt = smem + L.cnt;    // [kDispWaves][E] counts, then block-slot cursors
    int32_t* s_slot = smem + L.slot;  // [kBlockChunk] expert << kLocalBits | local index
    float* s_slot_w = reinterpret_cast<float*>(smem + L.slot_w);  // [kBlockChunk]
    constexpr int kEPT = kMaxExperts / kDispThreads;  // experts per thread (<= 4)
    const int t = threadIdx.x;
    const int lane = t % kWave;
    const int wv = t / kWave;
    // every global load of the block goes out first: this lane's assignments
    // a0 + 64 j, the expert totals (experts kEPT t ..), the block's row of
    // offsets across blocks (COARSE: the coarse matrix and the assignments
    // to recount)
    const int64_t blk0 = (int64_t)blockIdx.x * kBlockChunk;
    const int l0 = wv * kWaveChunk + lane;  // block-local index of assignment j = 0
    int32_t idv[kPerLane];
    float wv8[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        const int64_t a = blk0 + l0 + j * kWave;
        idv[j] = a < n ? ids[a] : -1;
        wv8[j] = (sorted_w && a < n) ? wts[a] : 0.0f;
    }
    int tot[kEPT], rowv[kEPT];
    for (int i = t; i < kDispWaves * E; i += kDispThreads) s_cnt[i] = 0;
    if constexpr (COARSE) {
        // Thread t < Q * G reduces 16-byte quad q = t % Q of rows
        // r = g, g + G, ... (g = t / Q) into a before-my-row and an all-rows
        // partial; the G partials of an expert are added in LDS.  The counts
        // of the chunks of this block's coarse row before it come from the
        // row's prefix rows, written by the histogram kernel.
        const int Q = E / 4;
        const int c = blockIdx.x / kSubPerRow, sb = blockIdx.x % kSubPerRow;
        const int q = t % Q, g = t / Q;
        int4 m[kCoarseRowsPerLane];
#pragma unroll
        for (int i = 0; i < kCoarseRowsPerLane; ++i) {
            const int r = g + G * i;
            m[i] = (g < G && r < C)
                       ? reinterpret_cast<const int4*>(cnt + (int64_t)r * E)[q]
                       : make_int4(0, 0, 0, 0);
        }
        int sub[kEPT];
        const int32_t* srow = cnt + (int64_t)coarse_prefix_row(C, c, sb) * E;
#pragma unroll
        for (int i = 0; i < kEPT; ++i) {
            const int e = kEPT * t + i;
            sub[i] = sb > 0 && e < E ? srow[e] : 0;
        }
        int32_t* s_pre = smem + L.pre;  // [G][E] partials (rows before c)
        int32_t* s_all = smem + L.all;  // [G][E] partials (all rows)
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
        for (int j = 0; j < kPerLane; ++j)
            if (valid_id(idv[j], E)) atomicAdd(&s_cnt[wv * E + idv[j]], 1);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kEPT; ++i) {
            const int e = kEPT * t + i;
            int p = sub[i], a = 0;
            if (e < E) {
                for (int gg = 0; gg < G; ++gg) {
                    p += s_pre[gg * E + e];
                    a += s_all[gg * E + e];
                }
            }
            tot[i] = a;
            rowv[i] = p;
        }
    } else {
        const int32_t* row = cnt + (int64_t)blockIdx.x * E;
#pragma unroll
        for (int i = 0; i < kEPT; ++i) {
            const int e = kEPT * t + i;
            tot[i] = e < E ? totals[e] : 0;
            rowv[i] = e < E ? row[e] : 0;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kPerLane; ++j)
            if (valid_id(idv[j], E)) atomicAdd(&s_cnt[wv * E + idv[j]], 1);
        __syncthreads();
    }
    // per expert: the block's count and each wave's exclusive prefix in it
    int wpre[kEPT][kDispWaves], bc[kEPT];
#pragma unroll
    for (int i = 0; i < kEPT; ++i) {
        const int e = kEPT * t + i;
        int c = 0;
#pragma unroll
        for (int q = 0; q < kDispWaves; ++q) {
            wpre[i][q] = c;
            c += e < E ? s_cnt[q * E + e] : 0;
        }
        bc[i] = c;
    }
    // exclusive scans over the experts of the totals (expert offsets) and of
    // the block's counts (the block's own slots, in expert order)
    int sum_t = 0, sum_b = 0;
#pragma unroll
    for (int i = 0; i < kEPT; ++i) {
        sum_t += tot[i];
        sum_b += bc[i];
    }
    const int inc_t = wave_incl_scan(sum_t), inc_b = wave_incl_scan(sum_b);
    if (lane == kWave - 1) {
        s_wsum[wv] = inc_t;
        s_wsum[kDispWaves + wv] = inc_b;
    }
    __syncthreads();
    int run_t = inc_t - sum_t, run_b = inc_b - sum_b, nblk = 0;
#pragma unroll
    for (int q = 0; q < kDispWaves; ++q) {
        const int vb = s_wsum[kDispWaves + q];
        if (q < wv) {
            run_t += s_wsum[q];
            run_b += vb;
        }
        nblk += vb;  // the block's valid assignments
    }
#pragma unroll
    for (int i = 0; i < kEPT; ++i) {
        const int e = kEPT * t + i;
        if (e < E) {
            s_off[e] = run_t;
            // sorted position of block slot s (expert e) = expert offset +
            // earlier blocks' count + (s - first slot of e in the block)
            s_gb[e] = run_t + rowv[i] - run_b;
#pragma unroll
            for (int q = 0; q < kDispWaves; ++q) s_cnt[q * E + e] = run_b + wpre[i][q];
            if (blockIdx.x == 0) {
                counts[e] = tot[i];
                offsets[e] = run_t;
            }
        }
        run_t += tot[i];
        run_b += bc[i];
    }
    if (t == kDispThreads - 1) {
        s_off[E] = run_t;
        if (blockIdx.x == 0) offsets[E] = run_t;
    }
    __syncthreads();
    const int64_t nvalid = s_off[E];
    // sorted positions past the valid assignments
    for (int64_t p = nvalid + (int64_t)blockIdx.x * kDispThreads + t; p < n;
         p += (int64_t)gridDim.x * kDispThreads) {
        gather[p] = -1;
        if (sorted_w) sorted_w[p] = 0.0f;
    }
    // expert ids need nb bits; the all-ones pattern of nb bits is >= E and
    // tags dropped or absent assignments
    int32_t* cur = s_cnt + wv * E;
    const int nb = 32 - __clz(E);
    const uint32_t none = (1u << nb) - 1u;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        const int l = l0 + j * kWave;
        const int64_t a = blk0 + l;
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
            const int32_t s = start + rank;  // block slot
            scatter[a] = s_gb[id] + s;
            s_slot[s] = (id << kLocalBits) | l;
            s_slot_w[s] = wv8[j];
            if (rank == size - 1) cur[id] = start + size;  // one writer per expert
        } else if (a < n) {
            scatter[a] = -1;
        }
    }
    __syncthreads();
    // the block's slots in order: each expert's run lands contiguously
    for (int s = t; s < nblk; s += kDispThreads) {
        const int32_t v = s_slot[s];
        const int32_t p = s_gb[v >> kLocalBits] + s;
        gather[p] = static_cast<int32_t>(blk0 + (v & (kBlockChunk - 1)));
        if (sorted_w) sorted_w[p] = s_slot_w[s];
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
        hipLaunchKernelGGL(dispatch_hist_coarse_kernel, dim3(C), dim3(kCoarseThreads),
                           sizeof(int32_t) * kSubPerRow * d.E, d.stream, d.ids, d.n, d.E, C, B,
                           cnt);
        hipLaunchKernelGGL(dispatch_place_kernel<true>, dim3(B), dim3(kDispThreads),
                           sizeof(int32_t) * place_lds(d.E, G).ints, d.stream, d.ids,
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
                       sizeof(int32_t) * place_lds(d.E, 0).ints, d.stream,
                       d.ids, d.weights, d.n, d.E, cnt, totals, B, d.counts, d.offsets,
                       d.gather, d.scatter, d.sorted_weights);
    return hipGetLastError() == hipSuccess ? ROUTE_OK : ROUTE_ELAUNCH;
}

}  // namespace moe_route
