// Fused router for gfx950: router projection on MFMA with the routing step as
// the epilogue, in one kernel ("[SGLang] MoE routing: token-to-expert
// assignment algorithms", section 5: the router matmul and the top-k share a
// kernel; here the routing is the biased grouped top-k of section 4).
//
// One workgroup owns 32 tokens and all 256 experts:
//   logits[32][256] = hidden[32][H] x W[H][256],  bf16 x bf16 -> fp32,
// computed with v_mfma_f32_32x32x16_bf16.  Wave w owns experts [64w, 64w+64)
// (two 32x32 accumulator tiles).  The hidden dimension is walked in steps of
// 64; each step stages a 32x64 tile of hidden states and a 64x256 tile of W
// in LDS (double-buffered); register rings keep the loads of the next six
// hidden-state tiles and the next three W tiles in flight.
// W is stored expert-contiguous ([H][E]) but an MFMA B operand wants 8
// consecutive k per lane, so each thread transposes an 8x8 bf16 block in
// registers (v_perm_b32) on its way to an [expert][k] LDS layout; rows are
// padded to 144 bytes so that fragment reads are bank-conflict free.
// After the last step the fp32 logits go to LDS and the same routing core as
// the standalone kernel (route_tile.cuh) routes the 32 rows, 8 lanes per row.
// The logits never leave the compute unit.
#include <hip/hip_runtime.h>

#include "route_common.cuh"
#include "route_internal.h"
#include "route_tile.cuh"

namespace moe_route {
namespace {

constexpr int kFrRows = 32;                      // tokens per workgroup
constexpr int kFrE = 256;                        // experts
constexpr int kFrBK = 64;                        // hidden units per step
constexpr int kFrThreads = 256;                  // 4 waves
constexpr int kFrRowBytes = kFrBK * 2 + 16;      // padded LDS row (A row or W column)
constexpr int kFrBufA = kFrRows * kFrRowBytes;   // 4608 B
constexpr int kFrBufB = kFrE * kFrRowBytes;      // 36864 B
constexpr int kFrStage = kFrBufA + kFrBufB;      // 41472 B per stage
constexpr int kFrLds = 2 * kFrStage;             // 82944 B
static_assert(kFrLds >= 2 * kFrRows * kFrE * 4, "epilogue reuses the staging buffers");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// 8x8 bf16 transpose: in[i] holds row i (8 values in 4 dwords); out[j]
// receives column j.  Output dword d of column j packs element j of rows 2d
// (low half) and 2d+1 (high half).
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t o[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint4& lo4 = in[2 * d];
            const uint4& hi4 = in[2 * d + 1];
            const uint32_t lo = (j / 2 == 0) ? lo4.x : (j / 2 == 1) ? lo4.y : (j / 2 == 2) ? lo4.z : lo4.w;
            const uint32_t hi = (j / 2 == 0) ? hi4.x : (j / 2 == 1) ? hi4.y : (j / 2 == 2) ? hi4.z : hi4.w;
            o[d] = __builtin_amdgcn_perm(hi, lo, (j % 2) ? 0x07060302u : 0x05040100u);
        }
        out[j] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

template <bool SOFTMAX, bool BIAS, int GRP>
__global__ __launch_bounds__(kFrThreads) void fused_router_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ w,
    const float* __restrict__ bias, int64_t M, int H, int TG, int K, int renorm,
    float* __restrict__ w_out, int32_t* __restrict__ id_out) {
    __shared__ __align__(16) unsigned char smem[kFrLds];
    __shared__ __align__(16) float s_bias[BIAS ? kFrE : 4];

    const int t = threadIdx.x;
    const int lane = t % kWave;
    const int wv = t / kWave;
    const int64_t m0 = (int64_t)blockIdx.x * kFrRows;

    // Load assignment.  A: thread t copies 16 bytes of row t/8 at k-chunk t%8.
    // W: thread t copies the 8x8 block (k rows 8*(t%8).., experts 8*(t/8)..).
    const int a_row = t / 8, a_kc = t % 8;
    const bool a_ok = m0 + a_row < M;
    const uint16_t* a_src = hidden + (a_ok ? (m0 + a_row) * H : 0) + a_kc * 8;
    const int w_kb = t % 8, w_nb = t / 8;
    const uint16_t* w_src = w + (int64_t)(w_kb * 8) * kFrE + w_nb * 8;

    // Register rings: the hidden-state tile of step t is loaded DA steps
    // ahead (it comes from HBM), the W tile DW steps ahead (L2-resident).
    constexpr int DA = 6, DW = 3, UNROLL = 6;
    static_assert(UNROLL % DA == 0 && UNROLL % DW == 0, "ring slots must be compile-time");
    uint4 ra[DA], rw[DW][8];
    // Hidden states are read once: non-temporal loads keep them from evicting
    // W, which every workgroup re-reads, from L2.
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    // Rows past M read row 0 (always valid) and are zeroed when staged, so the
    // load itself is unconditional.
    auto load_a = [&](int slot_a, int k0) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a_src + k0));
        ra[slot_a] = make_uint4(v[0], v[1], v[2], v[3]);
    };
    auto load_w = [&](int slot_w, int k0) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            rw[slot_w][i] = *reinterpret_cast<const uint4*>(w_src + (int64_t)(k0 + i) * kFrE);
    };
    auto store_step = [&](int buf, int slot_a, int slot_w) {
        unsigned char* st = smem + buf * kFrStage;
        *reinterpret_cast<uint4*>(st + a_row * kFrRowBytes + a_kc * 16) =
            a_ok ? ra[slot_a] : make_uint4(0, 0, 0, 0);
        uint4 tw[8];
        transpose8x8(rw[slot_w], tw);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            *reinterpret_cast<uint4*>(st + kFrBufA + (w_nb * 8 + j) * kFrRowBytes + w_kb * 16) =
                tw[j];
    };

    f32x16 acc[2];
#pragma unroll
    for (int q = 0; q < 16; ++q) { acc[0][q] = 0.f; acc[1][q] = 0.f; }

    const int steps = H / kFrBK;
    const int frag_m = lane % 32;          // A row / B column within a 32-tile
    const int frag_k = 8 * (lane / 32);    // first of the lane's 8 k values
    // One step: refill the ring slots freed by step s (staged during step s-1)
    // with the tiles DA / DW steps ahead, run the MFMAs on the staged tile, stage
    // step s+1, barrier.  Loads past the last step re-read the last tile rather
    // than branch: without branches the compiler tracks the outstanding loads
    // exactly and waits only for the ones a step needs.
    auto step = [&](const int s, const int u) {
        load_a(u % DA, min(s + DA, steps - 1) * kFrBK);
        load_w(u % DW, min(s + DW, steps - 1) * kFrBK);
        const unsigned char* st = smem + (s & 1) * kFrStage;
#pragma unroll
        for (int kk = 0; kk < kFrBK / 16; ++kk) {
            const int koff = (kk * 16 + frag_k) * 2;
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(st + frag_m * kFrRowBytes + koff);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int n = wv * 64 + nt * 32 + frag_m;
                const bf16x8 b =
                    *reinterpret_cast<const bf16x8*>(st + kFrBufA + n * kFrRowBytes + koff);
                acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[nt], 0, 0, 0);
            }
        }
        store_step((s + 1) & 1, (u + 1) % DA, (u + 1) % DW);  // step s+1 (or a spare copy)
        __syncthreads();
    };
    // prologue: steps 0..DA-1 of A and 0..DW-1 of W in flight; step 0 staged
#pragma unroll
    for (int q = 0; q < DA; ++q) load_a(q, min(q, steps - 1) * kFrBK);
#pragma unroll
    for (int q = 0; q < DW; ++q) load_w(q, min(q, steps - 1) * kFrBK);
    store_step(0, 0, 0);
    __syncthreads();
    int s0 = 0;
    for (; s0 + UNROLL <= steps; s0 += UNROLL) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) step(s0 + u, u);
    }
#pragma unroll
    for (int u = 0; u < UNROLL - 1; ++u)
        if (s0 + u < steps) step(s0 + u, u);

    // ---- epilogue: logits to LDS, then route the 32 rows (8 lanes per row)
    float* L = reinterpret_cast<float*>(smem);     // [32][256] fp32 logits
    float* S = L + kFrRows * kFrE;                 // [32][256] routing scratch
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int n = wv * 64 + nt * 32 + (lane % 32);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int m = 8 * (j / 4) + 4 * (lane / 32) + (j % 4);
            L[m * kFrE + n] = acc[nt][j];
        }
    }
    if constexpr (BIAS) s_bias[t] = bias[t];
    __syncthreads();

    const int r = t / 8, sub = t % 8, rw_in_wave = (t % kWave) / 8;
    KeyParams kp;
    if constexpr (BIAS) {
        float bmin = INFINITY, bmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            bmin = fminf(bmin, s_bias[sub * 32 + j]);
            bmax = fmaxf(bmax, s_bias[sub * 32 + j]);
        }
        kp = key_params(row_min<8>(bmin), 1.0f + row_max<8>(bmax));
    } else {
        kp = key_params(0.0f, 1.0f);
    }
    float x[32];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const float4 d = reinterpret_cast<const float4*>(L + r * kFrE + sub * 32)[v];
        x[4 * v] = d.x; x[4 * v + 1] = d.y; x[4 * v + 2] = d.z; x[4 * v + 3] = d.w;
    }
    const int64_t row = m0 + r;
    const float* lrow = L + r * kFrE;
    route_rows<8, 32, SOFTMAX, BIAS, GRP, (GRP ? 2 : 1), 8, 8>(
        x, sub, rw_in_wave, row < M, row, S + r * kFrE, s_bias, kp, TG, K, renorm, w_out,
        id_out, [&](int e) { return lrow[e]; });
}

template <bool SOFTMAX, bool BIAS, int GRP>
route_status_t launch_fr(const FusedProblem& f) {
    const RouteProblem& p = f.route;
    const int64_t blocks = (f.M + kFrRows - 1) / kFrRows;
    hipLaunchKernelGGL((fused_router_kernel<SOFTMAX, BIAS, GRP>), dim3((unsigned)blocks),
                       dim3(kFrThreads), 0, p.stream, static_cast<const uint16_t*>(f.hidden),
                       static_cast<const uint16_t*>(f.w), p.bias, f.M, f.H, p.TG, p.K,
                       p.renorm ? 1 : 0, p.weights, p.ids);
    return hipGetLastError() == hipSuccess ? ROUTE_OK : ROUTE_ELAUNCH;
}

}  // namespace

bool fused_router_supported(const FusedProblem& f) {
    const RouteProblem& p = f.route;
    const uintptr_t a = reinterpret_cast<uintptr_t>(f.hidden) | reinterpret_cast<uintptr_t>(f.w) |
                        reinterpret_cast<uintptr_t>(p.bias);
    if (p.E != kFrE || f.H % kFrBK != 0 || (a % 16) != 0 || p.K > 8) return false;
    if (p.scoring == ROUTE_SOFTMAX && p.bias != nullptr) return false;
    if (p.G == 1) return true;
    if (p.G != 8 || p.TG > 4) return false;
    // softmax with a top-2-sum group score has no specialised routing core
    return !(p.scoring == ROUTE_SOFTMAX && p.rule == ROUTE_GROUP_TOP2_SUM);
}

route_status_t launch_fused_router(const FusedProblem& f) {
    const RouteProblem& p = f.route;
    const bool soft = p.scoring == ROUTE_SOFTMAX;
    const bool bias = p.bias != nullptr;
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
