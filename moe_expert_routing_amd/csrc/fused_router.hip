// Fused router for gfx950: router projection on MFMA with the routing step as
// the epilogue, in one kernel ("[SGLang] MoE routing: token-to-expert
// assignment algorithms", section 5: the router matmul and the top-k share a
// kernel; here the routing is the biased grouped top-k of section 4).
//
// One workgroup owns 32 tokens and all 256 experts:
//   logits[32][256] = hidden[32][H] x W[H][256],  bf16 x bf16 -> fp32,
// computed with v_mfma_f32_32x32x16_bf16.  Wave w owns experts [64w, 64w+64)
// (two 32x32 accumulator tiles).  The hidden dimension is walked in steps of
// 64 through two rings of LDS stages ahead of the MFMAs:
//   - every tile goes from global memory straight into LDS; a fifth wave
//     copies the hidden states, the MFMA waves copy W;
//     (global_load_lds_dwordx4: each lane moves 16 bytes, a wave 1 KiB);
//     the W tile of a step is one contiguous 32 KiB block of W; hidden
//     states (read once, from HBM) run 11 steps ahead, W (re-read by every
//     workgroup, from L2) 2 steps ahead;
//   - W stays in its natural [k][expert] layout in LDS and the MFMA B
//     operand (8 consecutive k of one expert per lane) is read with the
//     transposing LDS read ds_read_b64_tr_b16: within each 16-lane group,
//     lane j receives element j%4 of the 8-byte rows addressed by lanes
//     j/4, j/4+4, j/4+8 and j/4+12 -- so lane i points at 4 experts of
//     k row i/4 and every lane gets 4 consecutive k of its expert;
//   - 16-byte chunks are XOR-swizzled inside LDS rows (by the source address
//     each lane picks, since a wave's direct-to-LDS write is contiguous) so
//     that both fragment reads are free of bank conflicts.
// After the last step the fp32 logits (soft-capped when asked) go to LDS and
// the same routing core as
// the standalone kernel (route_tile.hpp) routes the 32 rows, 8 lanes per row.
// The logits never leave the compute unit.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "route_common.hpp"
#include "route_internal.h"
#include "lds_copy.hpp"
#include "route_row.hpp"
#include "route_tile.hpp"

namespace moe_route {
namespace {

#ifndef FR_WAVE_ROUTE
#define FR_WAVE_ROUTE 1
#endif
constexpr int kFrRows = 32;                   // tokens per workgroup
constexpr int kFrE = 256;                     // experts
constexpr int kFrBK = 64;                     // hidden units per step
constexpr int kFrMathWaves = 4;               // MFMA waves; each also copies W
constexpr int kFrThreads = 64 * (kFrMathWaves + 1);  // + one wave that copies hidden states
constexpr int kFrAStages = 12;                // hidden-state ring (HBM)
constexpr int kFrWStages = 3;                 // W ring (L2-resident)
constexpr int kFrAAhead = kFrAStages - 1;     // steps each ring runs ahead
constexpr int kFrWAhead = kFrWStages - 1;
static_assert(kFrAAhead >= kFrWAhead, "hidden states run at least as far ahead as W");
constexpr int kFrABytes = kFrRows * kFrBK * 2;  // 4 KiB: [32 rows][64 k] bf16, 128 B rows
constexpr int kFrWBytes = kFrBK * kFrE * 2;     // 32 KiB: [64 k][256 experts] bf16, 512 B rows
constexpr int kFrWCopies = kFrWBytes / 1024 / kFrMathWaves;   // 8 per MFMA wave per step
static_assert(2 * kFrRows * kFrE * 4 <= 2 * kFrWBytes, "epilogue reuses two W stages");
static_assert(kFrAStages * kFrABytes + kFrWStages * kFrWBytes + kFrE * 4 <= 160 * 1024,
              "LDS of one workgroup");
// A ring of a ROWS-row tile: 32 rows (the fused kernel, which also keeps
// the bias in LDS) take 12 stages of 4 KiB; 64 and 128 rows (the partial
// kernel, no bias) take 8 stages of 8 KiB and 4 of 16 KiB, the rest of the
// 160 KiB beside the W ring.
template <int ROWS> struct ARing {
    static constexpr int kBytes = ROWS * kFrBK * 2;
    static constexpr int kStages = ROWS == 32 ? 12 : ROWS == 64 ? 8 : 4;
    static constexpr int kAhead = kStages - 1;
    static constexpr int kCopies = kBytes / 1024;        // 4, 8 or 16 wave loads per step
    static_assert(kAhead >= kFrWAhead, "hidden states run at least as far ahead as W");
    static_assert(kCopies * (kAhead - 1) <= 63, "a wait counts at most 63 loads");
    static_assert(kStages * kBytes + kFrWStages * kFrWBytes + (ROWS == 32 ? kFrE * 4 : 0) <=
                      160 * 1024,
                  "LDS of one workgroup");
};
static_assert(ARing<kFrRows>::kStages == kFrAStages && ARing<kFrRows>::kBytes == kFrABytes,
              "the fused kernel's ring is the 32-row ring");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef short i16x8 __attribute__((ext_vector_type(8)));

// Swizzles of the 16-byte chunk index inside an LDS row.
// A rows (8 chunks): chunk c of row m lives at c ^ ((m >> 1) & 7).
// W rows (32 chunks): chunk c of k row k lives at c ^ (4 * (k & 3)).
__device__ __forceinline__ int a_swz(int m, int c) { return c ^ ((m >> 1) & 7); }
__device__ __forceinline__ int w_swz(int k, int c) { return c ^ (4 * (k & 3)); }

// The projection of one workgroup: acc = hidden rows m0 .. m0+31 (rows past M
// read row M-1) times W over the hidden steps s_lo .. s_lo+steps-1 (kFrBK
// hidden units each), in the MFMA layout the epilogues below unpack.  The
// copy wave (its return value true) leaves acc alone.  Returns after every
// copy has landed and a workgroup barrier, so the caller may reuse sA and sW.
template <int ROWS>
__device__ __forceinline__ bool fr_project(const uint16_t* __restrict__ hidden,
                                           const uint16_t* __restrict__ w, int64_t M, int H,
                                           int64_t m0, int s_lo, int steps,
                                           unsigned char (*sA)[ARing<ROWS>::kBytes],
                                           unsigned char (*sW)[kFrWBytes],
                                           f32x16 (&acc)[ROWS / 32][2]) {
    using AR = ARing<ROWS>;
    constexpr int MH = ROWS / 32;  // 32-row halves of the tile
    const int t = threadIdx.x;
    const int lane = t % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(t / kWave);
    hidden += (int64_t)s_lo * kFrBK;
    w += (int64_t)s_lo * kFrBK * kFrE;

    // Direct-to-LDS copy assignment: every copy writes a 1 KiB block, lane l
    // its chunk l, and reads the global chunk that the swizzle puts there.
    //   hidden-state wave: A block j (rows 8j .. 8j+7), j < ROWS / 8; rows
    //     past M read row M-1 (never stored);
    //   MFMA wave w: W blocks 8w .. 8w+7 (k rows 2b, 2b+1 of block b).
    // Hidden states come from HBM and W from L2.  Waits count a wave's own
    // loads in issue order, so a wave that copied both would wait on the slow
    // hidden-state loads whenever it needs a W tile; giving them to a wave of
    // their own lets each ring keep its own distance.
    const bool copier = wv == kFrMathWaves;
    const uint16_t* a_src[AR::kCopies];
#pragma unroll
    for (int j = 0; j < AR::kCopies; ++j) {
        const int m = 8 * j + lane / 8;
        a_src[j] = hidden + min(m0 + m, M - 1) * H + 8 * a_swz(m, lane % 8);
    }
    uint32_t w_off[kFrWCopies];  // byte offset inside a step's W block
#pragma unroll
    for (int j = 0; j < kFrWCopies; ++j) {
        const int k = 2 * (kFrWCopies * wv + j) + lane / 32;
        w_off[j] = 2u * (k * kFrE + 8 * w_swz(k, lane % 32));
    }
    auto issue_a = [&](int step, int stage) {
#pragma unroll
        for (int j = 0; j < AR::kCopies; ++j)
            lds_copy16(a_src[j] + step * kFrBK, lds_addr(sA[stage] + 1024 * j));
    };
    // W copies j0 .. j0+n-1 of a step.
    auto issue_w = [&](int step, int stage, int j0, int n) {
        const uint16_t* wk = w + (int64_t)step * kFrBK * kFrE;
#pragma unroll
        for (int j = j0; j < j0 + n; ++j)
            lds_copy16(wk, w_off[j], lds_addr(sW[stage] + 1024 * (kFrWCopies * wv + j)));
    };

    // Fragment addresses.  A (half mh): lane l reads row 32 mh + l%32, k chunk
    // 2kk + l/32.
    // B (tile nt, k half h): lane l of 16-lane group g points at k row
    // 16kk + 8(g/2) + 4h + (l%16)/4 and experts n0 + 16(g%2) + 4(l%4) .. +3.
    const int fa_m = lane % 32;
    const int g = lane / 16, gi = lane % 16;
#pragma unroll
    for (int mh = 0; mh < MH; ++mh)
#pragma unroll
        for (int q = 0; q < 16; ++q) { acc[mh][0][q] = 0.f; acc[mh][1][q] = 0.f; }

    // The MFMAs of one step.  All fragments of the step are read first (so
    // the LDS latency is paid once, not per k slice); before the MFMAs of k
    // slice kk it calls copies(kk), which issues a share of the next copies,
    // so that issuing them (the address unit takes a 1 KiB wave load every
    // 16 cycles) overlaps the math.
    auto compute = [&](const unsigned char* a_base, const unsigned char* w_base, auto copies) {
        bf16x8 af[MH][kFrBK / 16], bfr[kFrBK / 16][2];
#pragma unroll
        for (int kk = 0; kk < kFrBK / 16; ++kk) {
            const int ac = 2 * kk + lane / 32;
#pragma unroll
            for (int mh = 0; mh < MH; ++mh) {
                const int m = 32 * mh + fa_m;
                af[mh][kk] = *reinterpret_cast<const bf16x8*>(a_base + m * 128 +
                                                              16 * a_swz(m, ac));
            }
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int e = wv * 64 + nt * 32 + 16 * (g % 2) + 4 * (gi % 4);
                i16x4 part[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int k = 16 * kk + 8 * (g / 2) + 4 * h + gi / 4;
                    const int off = k * 512 + 16 * w_swz(k, e / 8) + 2 * (e % 8);
                    part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4*)(w_base + off));
                }
                bfr[kk][nt] = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
            }
        }
#pragma unroll
        for (int kk = 0; kk < kFrBK / 16; ++kk) {
            copies(kk);
#pragma unroll
            for (int mh = 0; mh < MH; ++mh)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    acc[mh][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        af[mh][kk], bfr[kk][nt], acc[mh][nt], 0, 0, 0);
        }
    };

    // Rings.  At step s the hidden-state wave issues the copies of step
    // s + AR::kAhead and each MFMA wave those of W for step s + kFrWAhead (spread
    // over its MFMAs); the prologues issue what the steps before step 0 would
    // have.  At the top of step s a wave's loads issued after those of step s
    // belong to the AR::kAhead - 1 (kFrWAhead - 1) later steps, so waiting until
    // at most that many remain completes step s.  The barrier then makes every
    // wave's copies visible and retires the reads of step s-1, whose stages the
    // copies of step s reuse.  Copies past the last step repeat it into a stage
    // that is never read again, so the count in flight is the same at every
    // step.  Both kinds of wave pass the same number of barriers.
    if (copier) {
        for (int q = 0; q < AR::kAhead; ++q) issue_a(min(q, steps - 1), q);
        int ia = 0;
        for (int s = 0; s < steps; ++s) {
            wait_vmcnt<AR::kCopies * (AR::kAhead - 1)>();
            barrier_no_fence();
            issue_a(min(s + AR::kAhead, steps - 1), ia == 0 ? AR::kStages - 1 : ia - 1);
            ia = ia == AR::kStages - 1 ? 0 : ia + 1;
        }
    } else {
        for (int q = 0; q < kFrWAhead; ++q) issue_w(min(q, steps - 1), q, 0, kFrWCopies);
        int ia = 0, iw = 0;  // stages of step s
        for (int s = 0; s < steps; ++s) {
            wait_vmcnt<kFrWCopies * (kFrWAhead - 1)>();
            barrier_no_fence();
            const int w_step = min(s + kFrWAhead, steps - 1);
            const int w_stage = iw == 0 ? kFrWStages - 1 : iw - 1;
            compute(sA[ia], sW[iw], [&](int kk) {
                issue_w(w_step, w_stage, kk * kFrWCopies / 4, kFrWCopies / 4);
            });
            ia = ia == AR::kStages - 1 ? 0 : ia + 1;
            iw = iw == kFrWStages - 1 ? 0 : iw + 1;
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    return copier;
}

template <bool SOFTMAX, bool BIAS, int GRP>
__global__ __launch_bounds__(kFrThreads) void fused_router_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ w,
    BiasRef bias, int64_t M, int H, int TG, int K, int renorm, float cap,
    float* __restrict__ w_out, int32_t* __restrict__ id_out) {
    __shared__ __align__(1024) unsigned char sA[kFrAStages][kFrABytes];
    __shared__ __align__(1024) unsigned char sW[kFrWStages][kFrWBytes];
    __shared__ __align__(16) float s_bias[BIAS ? kFrE : 4];

    const int t = threadIdx.x;
    const int lane = t % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(t / kWave);
    const int64_t m0 = (int64_t)blockIdx.x * kFrRows;
    f32x16 acc[1][2];
    // The bias entries of the key window are requested before the main loop
    // (they arrive before its first wait, which counts loads in issue order).
    uint32_t braw[4];
    if constexpr (BIAS)
        if (wv < kFrMathWaves) bias_lane_load<kFrE>(bias, braw);
    const bool copier = fr_project<kFrRows>(hidden, w, M, H, m0, 0, H / kFrBK, sA, sW, acc);

    // ---- epilogue: logits to LDS, then route the 32 rows (8 lanes per row)
    float* L = reinterpret_cast<float*>(sW[0]);  // [32][256] fp32 logits
    float* S = reinterpret_cast<float*>(sW[1]);  // [32][256] routing scratch
#pragma unroll
    for (int nt = 0; nt < 2 && !copier; ++nt) {
        const int n = wv * 64 + nt * 32 + (lane % 32);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int m = 8 * (j / 4) + 4 * (lane / 32) + (j % 4);
            // soft-capping (cap != 0): every consumer below sees capped logits
            L[m * kFrE + n] = cap != 0.0f ? cap * tanh_f32(acc[0][nt][j] / cap) : acc[0][nt][j];
        }
    }
    // key window (every routing wave), and the staged bias offsets: wave i
    // writes entries [64 i, 64 i + 64)
    KeyParams kp = key_params(0.0f, 1.0f);
    if constexpr (BIAS) {
        if (!copier) {
            float b[4];
            bias_lane_widen(bias, braw, b);
            kp = bias_lane_key_params<kFrE>(b);
            if (t < kFrE) s_bias[bias_elem<kFrE>(t)] = sel_offset(b[t / kWave], kp);
        }
    }
    __syncthreads();
    if (copier) return;

    const int r = t / 8, sub = t % 8, rw_in_wave = (t % kWave) / 8;
    float x[32];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const float4 d = reinterpret_cast<const float4*>(L + r * kFrE + sub * 32)[v];
        x[4 * v] = d.x; x[4 * v + 1] = d.y; x[4 * v + 2] = d.z; x[4 * v + 3] = d.w;
    }
    const int64_t row = m0 + r;
    const float* lrow = L + r * kFrE;
    route_rows<8, 32, SOFTMAX, BIAS, GRP, (GRP ? 2 : 1), (GRP ? 4 : 5), 8>(
        x, sub, rw_in_wave, row < M, S + r * kFrE, s_bias, kp, TG, K, renorm,
        w_out + min(row, M - 1) * K, id_out + min(row, M - 1) * K, [&](int e) { return lrow[e]; },
        [&](int e) { return BIAS ? bias_at(bias, e) : 0.0f; });
}

// ---- up to 8192 tokens: the hidden dimension split over workgroups
//
// With fewer than 256 row tiles the single kernel leaves compute units idle
// and each workgroup walks all of H one W tile after the other; and every
// workgroup streams all of W for its 32 tokens.  The split path gives
// workgroup (tile, s) the hidden steps of split s only, on tiles of 32, 64 or
// 128 tokens (W is streamed once per tile); it writes its fp32 partial
// logits to part[s][M][256].  A second kernel sums the splits of each logit
// in a fixed order (so results do not depend on timing), soft-caps the sum
// and routes the row; the summed logits never reach memory.
template <int ROWS>
__global__ __launch_bounds__(kFrThreads) void fused_router_partial_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ w, int64_t M, int H,
    int nsplit, float* __restrict__ part) {
    using AR = ARing<ROWS>;
    __shared__ __align__(1024) unsigned char sA[AR::kStages][AR::kBytes];
    __shared__ __align__(1024) unsigned char sW[kFrWStages][kFrWBytes];

    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t m0 = (int64_t)blockIdx.x * ROWS;
    const int split = blockIdx.y, steps_all = H / kFrBK;
    const int s_lo = split * steps_all / nsplit, s_hi = (split + 1) * steps_all / nsplit;
    f32x16 acc[ROWS / 32][2];
    if (fr_project<ROWS>(hidden, w, M, H, m0, s_lo, s_hi - s_lo, sA, sW, acc)) return;

    float* out = part + (int64_t)split * M * kFrE;
#pragma unroll
    for (int mh = 0; mh < ROWS / 32; ++mh)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int n = wv * 64 + nt * 32 + (lane % 32);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int64_t row = m0 + 32 * mh + 8 * (j / 4) + 4 * (lane / 32) + (j % 4);
                if (row < M) out[row * kFrE + n] = acc[mh][nt][j];
            }
        }
}

// Splits of at most kFrNoRingSteps hidden steps on 32-row tiles (few
// tokens): no ring, so no copies run past the split.  The four MFMA waves
// each copy one 8-row block of the hidden-state tile and their eight W blocks
// of every step of the split into the same LDS layout as a ring stage, wait
// for all of them, and do the MFMAs step by step.
constexpr int kFrNoRingSteps = 4;
constexpr int kFrStepThreads = 64 * kFrMathWaves;
static_assert(kFrNoRingSteps * (kFrABytes + kFrWBytes) <= 160 * 1024, "LDS of one workgroup");
__global__ __launch_bounds__(kFrStepThreads) void fused_router_step_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ w, int64_t M, int H,
    int nsplit, float* __restrict__ part) {
    __shared__ __align__(1024) unsigned char sA[kFrNoRingSteps][kFrABytes];
    __shared__ __align__(1024) unsigned char sW[kFrNoRingSteps][kFrWBytes];
    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t m0 = (int64_t)blockIdx.x * kFrRows;
    const int split = blockIdx.y, steps_all = H / kFrBK;
    const int s_lo = split * steps_all / nsplit;
    const int steps = (split + 1) * steps_all / nsplit - s_lo;  // 1 .. kFrNoRingSteps
    static_assert(kFrABytes / 1024 == kFrMathWaves, "one hidden-state block per MFMA wave");
    const int m = 8 * wv + lane / 8;
    const uint16_t* a_src = hidden + min(m0 + m, M - 1) * H + (int64_t)s_lo * kFrBK +
                            8 * a_swz(m, lane % 8);
    for (int q = 0; q < steps; ++q) {
        lds_copy16(a_src + q * kFrBK, lds_addr(sA[q] + 1024 * wv));
        const uint16_t* wk = w + (int64_t)(s_lo + q) * kFrBK * kFrE;
#pragma unroll
        for (int j = 0; j < kFrWCopies; ++j) {
            const int k = 2 * (kFrWCopies * wv + j) + lane / 32;
            lds_copy16(wk, 2u * (k * kFrE + 8 * w_swz(k, lane % 32)),
                       lds_addr(sW[q] + 1024 * (kFrWCopies * wv + j)));
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // fragments and MFMAs of each step, as in fr_project
    const int fa_m = lane % 32;
    const int g = lane / 16, gi = lane % 16;
    f32x16 acc[2];
#pragma unroll
    for (int q = 0; q < 16; ++q) { acc[0][q] = 0.f; acc[1][q] = 0.f; }
    for (int q = 0; q < steps; ++q) {
        bf16x8 af[kFrBK / 16], bfr[kFrBK / 16][2];
#pragma unroll
        for (int kk = 0; kk < kFrBK / 16; ++kk) {
            af[kk] = *reinterpret_cast<const bf16x8*>(sA[q] + fa_m * 128 +
                                                      16 * a_swz(fa_m, 2 * kk + lane / 32));
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int e = wv * 64 + nt * 32 + 16 * (g % 2) + 4 * (gi % 4);
                i16x4 p[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int k = 16 * kk + 8 * (g / 2) + 4 * h + gi / 4;
                    p[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4*)(sW[q] + k * 512 + 16 * w_swz(k, e / 8) + 2 * (e % 8)));
                }
                bfr[kk][nt] = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(p[0], p[1], 0, 1, 2, 3, 4, 5, 6, 7));
            }
        }
#pragma unroll
        for (int kk = 0; kk < kFrBK / 16; ++kk)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                acc[nt] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk], bfr[kk][nt], acc[nt], 0, 0, 0);
    }

    float* out = part + (int64_t)split * M * kFrE;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int n = wv * 64 + nt * 32 + (lane % 32);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int64_t row = m0 + 8 * (j / 4) + 4 * (lane / 32) + (j % 4);
            if (row < M) out[row * kFrE + n] = acc[nt][j];
        }
    }
}

// Many splits (8 or more): one row per block of 1024 threads, 64 float4
// columns x 16 split slices.  Slice q adds splits q, q + 16, ... in that
// order and the slice sums are added in slice order; the sum is soft-capped
// and the first wave routes the row: with sigmoid scoring (WAVE) by the
// one-row-per-wave core (route_row.hpp, 4 experts a lane), otherwise with
// the fused kernel's epilogue (its other 7 row slots computed, never
// stored).
template <bool SOFTMAX, bool BIAS, int GRP, bool WAVE>
__global__ __launch_bounds__(1024) void fr_reduce_route_kernel(
    const float* __restrict__ part, int64_t M, int nsplit, float cap,
    BiasRef bias, int TG, int K, int renorm, float* __restrict__ w_out,
    int32_t* __restrict__ id_out) {
    __shared__ float4 red[16][64];
    __shared__ __align__(16) float L[kFrE];         // the row's logits
    __shared__ __align__(16) float S[8][kFrE];      // routing scratch of the wave's 8 row slots
    __shared__ __align__(16) float s_bias[BIAS ? kFrE : 4];

    const int t = threadIdx.x, c4 = t % 64, q = t / 64;
    const int64_t row = blockIdx.x;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    const float4* src = reinterpret_cast<const float4*>(part) + row * 64 + c4;
    const int64_t split_stride = M * 64;
#pragma unroll 4
    for (int sp = q; sp < nsplit; sp += 16) {
        const float4 v = src[sp * split_stride];
        a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
    }
    red[q][c4] = a;
    // key window (waves 0-3, which stage the bias offsets: wave i entries
    // [64 i, 64 i + 64); wave 0 routes the row)
    KeyParams kp = key_params(0.0f, 1.0f);
    float off[4];  // WAVE: the bias offsets of wave 0's lanes (4 experts each)
    if constexpr (WAVE) {
        static_assert(!SOFTMAX, "the one-row-per-wave core scores with sigmoid");
        if (t < kWave) kp = row_wave_key_window<BIAS>(bias, t, off);
    } else if constexpr (BIAS) {
        if (t < kFrE) {
            float b[4];
            kp = bias_key_params<kFrE>(bias, b);
            s_bias[bias_elem<kFrE>(t)] = sel_offset(b[t / kWave], kp);
        }
    }
    __syncthreads();
    if (q == 0) {
#pragma unroll
        for (int j = 1; j < 16; ++j) {
            const float4 v = red[j][c4];
            a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
        }
        if (cap != 0.0f) {
            a.x = cap * tanh_f32(a.x / cap);
            a.y = cap * tanh_f32(a.y / cap);
            a.z = cap * tanh_f32(a.z / cap);
            a.w = cap * tanh_f32(a.w / cap);
        }
        reinterpret_cast<float4*>(L)[c4] = a;
    }
    __syncthreads();
    if (t >= kWave) return;

    if constexpr (WAVE) {
        const float4 d = reinterpret_cast<const float4*>(L)[t];
        const float x4[4] = {d.x, d.y, d.z, d.w};
        route_row_wave<BIAS, GRP>(x4, t, bias, off, kp, TG, K, renorm, w_out + row * K,
                                  id_out + row * K, [&](int e) { return L[e]; });
        return;
    }
    const int sub = t % 8, rw = t / 8;
    float x[32];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const float4 d = reinterpret_cast<const float4*>(L + sub * 32)[v];
        x[4 * v] = d.x; x[4 * v + 1] = d.y; x[4 * v + 2] = d.z; x[4 * v + 3] = d.w;
    }
    route_rows<8, 32, SOFTMAX, BIAS, GRP, (GRP ? 2 : 1), (GRP ? 4 : 5), 8>(
        x, sub, rw, rw == 0, S[rw], s_bias, kp, TG, K, renorm, w_out + row * K, id_out + row * K,
        [&](int e) { return L[e]; },
        [&](int e) { return BIAS ? bias_at(bias, e) : 0.0f; });
}

// Otherwise a wave per 8 rows, in the routing kernel's layout: lane sub of
// row rw adds its 32 logits over the splits in split order, soft-caps them
// and the wave routes its rows with the fused kernel's epilogue.  Rows past
// M read row M-1 and are never stored.
template <bool SOFTMAX, bool BIAS, int GRP>
__global__ __launch_bounds__(kWave) void fr_reduce_route_rows_kernel(
    const float* __restrict__ part, int64_t M, int nsplit, float cap,
    BiasRef bias, int TG, int K, int renorm, float* __restrict__ w_out,
    int32_t* __restrict__ id_out) {
    __shared__ __align__(16) float S[8][kFrE];      // routing scratch of the 8 rows
    __shared__ __align__(16) float s_bias[BIAS ? kFrE : 4];

    const int t = threadIdx.x, sub = t % 8, rw = t / 8;
    const int64_t row = (int64_t)blockIdx.x * 8 + rw;
    const int64_t rrow = row < M ? row : M - 1;
    // Every load is issued before the first wait: the bias entries (lane l:
    // l + 64 i), then the logits of the first 4 splits; the key window needs
    // only the bias.  Splits are added in split order, 4 in flight at a time.
    uint32_t braw[4];
    if constexpr (BIAS) bias_lane_load<kFrE>(bias, braw);
    const int64_t split_stride = M * kFrE;
    const float4* src = reinterpret_cast<const float4*>(part + rrow * kFrE + sub * 32);
    float4 d[4][8];
    auto load4 = [&](int s0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int sp = min(s0 + j, nsplit - 1);  // past the last split: not added
#pragma unroll
            for (int v = 0; v < 8; ++v) d[j][v] = src[sp * split_stride / 4 + v];
        }
    };
    load4(0);
    // key window, and the staged bias offsets
    KeyParams kp = key_params(0.0f, 1.0f);
    if constexpr (BIAS) {
        float b[4];
        bias_lane_widen(bias, braw, b);
        kp = bias_lane_key_params<kFrE>(b);
#pragma unroll
        for (int i = 0; i < 4; ++i) s_bias[bias_elem<kFrE>(t + kWave * i)] = sel_offset(b[i], kp);
    }
    float x[32];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        x[4 * v] = d[0][v].x; x[4 * v + 1] = d[0][v].y;
        x[4 * v + 2] = d[0][v].z; x[4 * v + 3] = d[0][v].w;
    }
    for (int s0 = 0; s0 < nsplit; s0 += 4) {
        if (s0 > 0) load4(s0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if ((s0 == 0 && j == 0) || s0 + j >= nsplit) continue;
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                x[4 * v] += d[j][v].x; x[4 * v + 1] += d[j][v].y;
                x[4 * v + 2] += d[j][v].z; x[4 * v + 3] += d[j][v].w;
            }
        }
    }
    if (cap != 0.0f) {
#pragma unroll
        for (int j = 0; j < 32; ++j) x[j] = cap * tanh_f32(x[j] / cap);
    }
    __syncthreads();

    // the logit of expert e, summed in the same order (route_rows reads it only
    // with one lane per row, so not here; it stays exact for any later use)
    const float* rsrc = part + rrow * kFrE;
    route_rows<8, 32, SOFTMAX, BIAS, GRP, (GRP ? 2 : 1), (GRP ? 4 : 5), 8>(
        x, sub, rw, row < M, S[rw], s_bias, kp, TG, K, renorm, w_out + rrow * K, id_out + rrow * K,
        [&](int e) {
            float v = rsrc[e];
            for (int sp = 1; sp < nsplit; ++sp) v += rsrc[sp * split_stride + e];
            return cap != 0.0f ? cap * tanh_f32(v / cap) : v;
        },
        [&](int e) { return BIAS ? bias_at(bias, e) : 0.0f; });
}

template <bool SOFTMAX, bool BIAS, int GRP>
route_status_t launch_rr(const FusedProblem& f, const float* part, int nsplit) {
    const RouteProblem& p = f.route;
    // 8+ splits (up to 1024 tokens of a 7168-wide router): a block per row
    // sums them 16 wide; fewer splits: a wave per 8 rows, each lane adding
    // its logits over the splits
    // The one-row-per-wave routing loads the bias 4 entries at a time.
    const bool bias_4x = p.bias.p == nullptr ||
                         reinterpret_cast<uintptr_t>(p.bias.p) % (p.bias.bf16 ? 8 : 16) == 0;
    if (nsplit >= 8 && !SOFTMAX && bias_4x && p.K <= kRowKMax && FR_WAVE_ROUTE)
        hipLaunchKernelGGL((fr_reduce_route_kernel<false, BIAS, GRP, true>), dim3((unsigned)f.M),
                           dim3(1024), 0, p.stream, part, f.M, nsplit, f.softcap, p.bias, p.TG,
                           p.K, p.renorm ? 1 : 0, p.weights, p.ids);
    else if (nsplit >= 8)
        hipLaunchKernelGGL((fr_reduce_route_kernel<SOFTMAX, BIAS, GRP, false>), dim3((unsigned)f.M),
                           dim3(1024), 0, p.stream, part, f.M, nsplit, f.softcap, p.bias, p.TG,
                           p.K, p.renorm ? 1 : 0, p.weights, p.ids);
    else
        hipLaunchKernelGGL((fr_reduce_route_rows_kernel<SOFTMAX, BIAS, GRP>),
                           dim3((unsigned)((f.M + 7) / 8)), dim3(kWave), 0, p.stream, part, f.M,
                           nsplit, f.softcap, p.bias, p.TG, p.K, p.renorm ? 1 : 0, p.weights,
                           p.ids);
    return hipGetLastError() == hipSuccess ? ROUTE_OK : ROUTE_ELAUNCH;
}

route_status_t launch_reduce_route(const FusedProblem& f, const float* part, int nsplit) {
    const RouteProblem& p = f.route;
    const bool soft = p.scoring == ROUTE_SOFTMAX;
    const bool bias = p.bias.p != nullptr;
    if (p.G == 1) {
        if (soft) return launch_rr<true, false, 0>(f, part, nsplit);
        return bias ? launch_rr<false, true, 0>(f, part, nsplit)
                    : launch_rr<false, false, 0>(f, part, nsplit);
    }
    if (p.rule == ROUTE_GROUP_TOP2_SUM)
        return bias ? launch_rr<false, true, 2>(f, part, nsplit)
                    : launch_rr<false, false, 2>(f, part, nsplit);
    if (soft) return launch_rr<true, false, 1>(f, part, nsplit);
    return bias ? launch_rr<false, true, 1>(f, part, nsplit)
                : launch_rr<false, false, 1>(f, part, nsplit);
}

route_status_t launch_split(const FusedProblem& f, SplitPlan plan) {
    const RouteProblem& p = f.route;
    const int nsplit = plan.splits;
    const int64_t tiles = (f.M + plan.rows - 1) / plan.rows;
    float* part = f.workspace;  // [nsplit][M][256] fp32
    if (plan.rows == 128)
        hipLaunchKernelGGL(fused_router_partial_kernel<128>, dim3((unsigned)tiles, (unsigned)nsplit),
                           dim3(kFrThreads), 0, p.stream, static_cast<const uint16_t*>(f.hidden),
                           static_cast<const uint16_t*>(f.w), f.M, f.H, nsplit, part);
    else if (plan.rows == 64)
        hipLaunchKernelGGL(fused_router_partial_kernel<64>, dim3((unsigned)tiles, (unsigned)nsplit),
                           dim3(kFrThreads), 0, p.stream, static_cast<const uint16_t*>(f.hidden),
                           static_cast<const uint16_t*>(f.w), f.M, f.H, nsplit, part);
    else if ((f.H / kFrBK + nsplit - 1) / nsplit <= kFrNoRingSteps)  // a few steps per split
        hipLaunchKernelGGL(fused_router_step_kernel, dim3((unsigned)tiles, (unsigned)nsplit),
                           dim3(kFrStepThreads), 0, p.stream, static_cast<const uint16_t*>(f.hidden),
                           static_cast<const uint16_t*>(f.w), f.M, f.H, nsplit, part);
    else
        hipLaunchKernelGGL(fused_router_partial_kernel<32>, dim3((unsigned)tiles, (unsigned)nsplit),
                           dim3(kFrThreads), 0, p.stream, static_cast<const uint16_t*>(f.hidden),
                           static_cast<const uint16_t*>(f.w), f.M, f.H, nsplit, part);
    if (hipGetLastError() != hipSuccess) return ROUTE_ELAUNCH;
    return launch_reduce_route(f, part, nsplit);
}

template <bool SOFTMAX, bool BIAS, int GRP>
route_status_t launch_fr(const FusedProblem& f) {
    const RouteProblem& p = f.route;
    const int64_t blocks = (f.M + kFrRows - 1) / kFrRows;
    hipLaunchKernelGGL((fused_router_kernel<SOFTMAX, BIAS, GRP>), dim3((unsigned)blocks),
                       dim3(kFrThreads), 0, p.stream, static_cast<const uint16_t*>(f.hidden),
                       static_cast<const uint16_t*>(f.w), p.bias, f.M, f.H, p.TG, p.K,
                       p.renorm ? 1 : 0, f.softcap, p.weights, p.ids);
    return hipGetLastError() == hipSuccess ? ROUTE_OK : ROUTE_ELAUNCH;
}

}  // namespace

bool fused_router_supported(const FusedProblem& f) {
    const RouteProblem& p = f.route;
    if (p.E != kFrE) return small_router_supported(f);
    // the bias is read one entry at a time: its own alignment is enough
    const uintptr_t a = reinterpret_cast<uintptr_t>(f.hidden) | reinterpret_cast<uintptr_t>(f.w);
    if (p.E != kFrE || f.H % kFrBK != 0 || (a % 16) != 0 || p.K > 8) return false;
    if (p.scoring == ROUTE_SOFTMAX && p.bias.p != nullptr) return false;
    if (p.G == 1) return true;
    if (p.G != 8 || p.TG > 4) return false;
    // softmax with a top-2-sum group score has no specialised routing core
    return !(p.scoring == ROUTE_SOFTMAX && p.rule == ROUTE_GROUP_TOP2_SUM);
}

SplitPlan fused_router_split_plan(int64_t M, int H) {
    // One workgroup fills a compute unit (its LDS), so up to 256 workgroups
    // run in one round.  Larger tiles stream W once for more tokens: 64 rows
    // above 2048 tokens, 128 rows above 6144 (at 8192 tokens 4 splits of 128
    // rows take 45.5 us a call against 51.7 for 2 splits of 64; up to 6144
    // tokens the 64-row tiles are as fast or faster).  Split as far as one
    // round allows, then back off to the fewest splits that keep the same
    // steps per workgroup (every split costs partial-logit traffic).  Above
    // 8192 tokens the single fused kernel runs.
    if (M > 8192) return {kFrRows, 1};
    const int rows = M > 6144 ? 128 : M > 2048 ? 64 : 32;
    const int64_t tiles = (M + rows - 1) / rows;
    const int steps = H / kFrBK;
    if (M <= 0 || steps < 2) return {kFrRows, 1};
    const int64_t most = std::min<int64_t>(steps, 256 / tiles);
    if (most < 2) return {kFrRows, 1};
    int per_split = (steps + (int)most - 1) / (int)most;
    // Each split also writes and re-reads 1 KiB of partial logits per token.
    // Above 8 tokens a 32-row split takes at least 4 steps (measured: 64
    // tokens of a 7168-wide router, 9.6 us a call against 11.9 with one step
    // per split; at one token one step is best).
    if (rows == 32 && M > 8) per_split = std::max(per_split, std::min(kFrNoRingSteps, steps));
    return {rows, (steps + per_split - 1) / per_split};
}

size_t fused_router_workspace_bytes(int64_t M, int H) {
    const int n = fused_router_split_plan(M, H).splits;
    return n == 1 ? 0 : sizeof(float) * kFrE * (size_t)M * (size_t)n;
}

route_status_t launch_fused_router(const FusedProblem& f) {
    const RouteProblem& p = f.route;
    if (p.E != kFrE) return launch_small_router(f);
    if (f.workspace != nullptr) {
        const SplitPlan plan = fused_router_split_plan(f.M, f.H);
        if (plan.splits > 1) return launch_split(f, plan);
    }
    const bool soft = p.scoring == ROUTE_SOFTMAX;
    const bool bias = p.bias.p != nullptr;
    if (p.G == 1) {
        if (soft) return launch_fr<true, false, 0>(f);
        return bias ? launch_fr<false, true, 0>(f) : launch_fr<false, false, 0>(f);
    }
    if (p.rule == ROUTE_GROUP_TOP2_SUM)
        return bias ? launch_fr<false, true, 2>(f) : launch_fr<false, false, 2>(f);
    if (soft) return launch_fr<true, false, 1>(f);
    return bias ? launch_fr<false, true, 1>(f) : launch_fr<false, false, 1>(f);
}

}  // namespace moe_route
