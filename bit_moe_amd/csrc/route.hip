// Routing: router logits (bf16 router weights, fp32 accumulation), top-k with
// ties to the lower expert index, and the softmax renormalised over the k
// selected experts.  The router is one of the unquantised parts of the
// layer (page "ds4 : analyse pratique pour un usage documente", section
// "Support de modeles et choix de quantification"); it chooses a few experts
// per token (page "Un modele de 284 milliards de parametres tourne desormais
// sur un Mac de 128 Go. Qui y perd ?", section "Comment un modele de 284
// milliards de parametres tient sur une seule machine").
#include "device_util.h"

namespace {

using namespace bm;

using bm_cfg::kRouterNT;       // tokens per launch of the small-T router

// ---------------------------------------------------------------------------
// Small-T router: one wave per expert row, lanes across K (16-byte pieces,
// each wave reads its row once in 1 KiB coalesced steps), a wave reduction
// per token.  Each logit is produced by exactly one wave, in a fixed order,
// so results are reproducible run to run.
// ---------------------------------------------------------------------------
template <int XBF16>
__global__ void __launch_bounds__(256)
k_router_gemv(const uint16_t *__restrict__ wr, const void *__restrict__ x, int T, int H, int E,
              float *__restrict__ logits) {
    const int e = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (e >= E) return;
    const uint4 *wrow = reinterpret_cast<const uint4 *>(wr + (int64_t)e * H);
    if (T == 1)
        router_row<XBF16, 1>(wrow, x, H, T, E, e, logits);
    else if (T <= 4)
        router_row<XBF16, 4>(wrow, x, H, T, E, e, logits);
    else
        router_row<XBF16, kRouterNT>(wrow, x, H, T, E, e, logits);
}

// ---------------------------------------------------------------------------
// Large-T router (bf16 activations): logits = X[T][H] . W[E][H]^T on bf16
// MFMA (v_mfma_f32_16x16x32_bf16) with fp32 accumulation.  64x64 output tile
// per workgroup, 4 waves of 32x32, K staged through LDS 64 columns at a time.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Split-K: workgroup (token tile of 64, expert tile of 256, K slice s)
// writes its partial sums to part[s][t][e]; k_topk_sum adds the slices in a
// fixed order (deterministic).  Four waves, each 64 tokens x 64 experts.
using bm_cfg::kRouterSplit;
__global__ void __launch_bounds__(256)
k_router_splitk(const uint16_t *__restrict__ X, const uint16_t *__restrict__ W, int T, int H, int E, int kslice,
                float *__restrict__ part) {
    constexpr int BK = 64, LD = BK + 8;   // padded row stride (bf16 elements)
    __shared__ __attribute__((aligned(16))) uint16_t sa[64 * LD];
    __shared__ __attribute__((aligned(16))) uint16_t sb[256 * LD];
    const int m0 = blockIdx.x * 64, n0 = blockIdx.y * 256, sl = blockIdx.z;
    const int kbeg = sl * kslice, kend = min(H, kbeg + kslice);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // A: 64 rows x 64 = 512 pieces of 8 bf16 (2 per thread); B: 256 rows (8
    // per thread).  Two register sets take the pieces of the next two stages
    // while the current stage's MFMAs run (at 2048 tokens the grid is one
    // workgroup per CU, one wave per SIMD, so the loads' latency, not the
    // MFMAs, sets the pace); loads past the slice re-read its last stage,
    // unused.
    const int pr = tid >> 3, pc = (tid & 7) * 8;          // piece p: row pr + 32 p, column pc
    const uint16_t *xa0 = X + (int64_t)min(m0 + pr, T - 1) * H + pc;
    const uint16_t *xa1 = X + (int64_t)min(m0 + pr + 32, T - 1) * H + pc;
    const uint16_t *wrow[8];
#pragma unroll
    for (int p = 0; p < 8; p++) wrow[p] = W + (int64_t)min(n0 + pr + 32 * p, E - 1) * H + pc;
    auto ld = [](const uint16_t *q, int k) { return *reinterpret_cast<const uint4 *>(q + k); };
    auto st = [&](int r, uint4 v) { *reinterpret_cast<uint4 *>((r < 64 ? sa + r * LD : sb + (r - 64) * LD) + pc) = v; };
#define BM_RT_LOAD(S, k)                                                                                     \
    do {                                                                                                     \
        const int kk_ = min(k, kend - BK);                                                                   \
        a0##S = ld(xa0, kk_); a1##S = ld(xa1, kk_);                                                          \
        b0##S = ld(wrow[0], kk_); b1##S = ld(wrow[1], kk_); b2##S = ld(wrow[2], kk_); b3##S = ld(wrow[3], kk_); \
        b4##S = ld(wrow[4], kk_); b5##S = ld(wrow[5], kk_); b6##S = ld(wrow[6], kk_); b7##S = ld(wrow[7], kk_); \
    } while (0)
#define BM_RT_STORE(S)                                                                                       \
    do {                                                                                                     \
        st(pr, a0##S); st(pr + 32, a1##S);                                                                   \
        st(64 + pr, b0##S); st(96 + pr, b1##S); st(128 + pr, b2##S); st(160 + pr, b3##S);                   \
        st(192 + pr, b4##S); st(224 + pr, b5##S); st(256 + pr, b6##S); st(288 + pr, b7##S);                 \
    } while (0)
    auto compute = [&]() {
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            const int kof = kk + 8 * (lane >> 4);
            bf16x8 fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; i++) fa[i] = *reinterpret_cast<const bf16x8 *>(sa + (16 * i + (lane & 15)) * LD + kof);
#pragma unroll
            for (int j = 0; j < 4; j++)
                fb[j] = *reinterpret_cast<const bf16x8 *>(sb + (64 * wave + 16 * j + (lane & 15)) * LD + kof);
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    };
    uint4 a00, a10, b00, b10, b20, b30, b40, b50, b60, b70;
    uint4 a01, a11, b01, b11, b21, b31, b41, b51, b61, b71;
    if (kbeg < kend) {
        BM_RT_LOAD(0, kbeg);
        BM_RT_LOAD(1, kbeg + BK);
    }
    for (int k0 = kbeg; k0 < kend; k0 += 2 * BK) {
        BM_RT_STORE(0);
        __syncthreads();
        BM_RT_LOAD(0, k0 + 2 * BK);
        compute();
        __syncthreads();
        if (k0 + BK >= kend) break;
        BM_RT_STORE(1);
        __syncthreads();
        BM_RT_LOAD(1, k0 + 3 * BK);
        compute();
        __syncthreads();
    }
#undef BM_RT_LOAD
#undef BM_RT_STORE
    float *P = part + (int64_t)sl * T * E;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int n = n0 + 64 * wave + 16 * j + (lane & 15);
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int m = m0 + 16 * i + 4 * (lane >> 4) + q;
                if (m < T && n < E) P[(int64_t)m * E + n] = acc[i][j][q];
            }
        }
}

// Logits of one token = sum over the K slices (fixed order), kept in LDS for
// the top-k and written to `logits` when given; one wave per token.
__global__ void __launch_bounds__(256)
k_topk_sum(const float *__restrict__ part, int S, int T, int E, int k, float *__restrict__ logits,
           int32_t *__restrict__ ids, float *__restrict__ wout) {
    __shared__ float srow[4][1024];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wv;
    if (E <= 256) {         // four logits per lane, the keyed one-wave top-k
        if (t >= T) return;
        // every slice's partial loaded first (at most kRouterSplit), then
        // summed in slice order: one round trip instead of one per slice
        float pv[4][kRouterSplit];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int e = min(lane + 64 * i, E - 1);
#pragma unroll
            for (int sl = 0; sl < kRouterSplit; sl++)
                pv[i][sl] = sl < S ? part[((int64_t)sl * T + t) * E + e] : 0.f;
        }
        float lv[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int e = min(lane + 64 * i, E - 1);
            float v = 0.f;
#pragma unroll
            for (int sl = 0; sl < kRouterSplit; sl++)
                if (sl < S) v += pv[i][sl];
            lv[i] = v;
            if (logits && lane + 64 * i < E) logits[(int64_t)t * E + e] = v;
        }
        topk_wave4(lv, E, k, ids + (int64_t)t * k, wout + (int64_t)t * k, nullptr);
        return;
    }
    if (t < T)
        for (int e = lane; e < E; e += 64) {
            float v = 0.f;
            for (int sl = 0; sl < S; sl++) v += part[((int64_t)sl * T + t) * E + e];
            srow[wv][e] = v;
            if (logits) logits[(int64_t)t * E + e] = v;
        }
    __syncthreads();
    if (t < T) topk_wave(srow[wv], E, k, ids + (int64_t)t * k, wout + (int64_t)t * k);
}

// ---------------------------------------------------------------------------
// Top-k: one wave per token over the final logits.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
k_topk(const float *__restrict__ logits, int T, int E, int k, int32_t *__restrict__ ids,
       float *__restrict__ wout) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    if (E <= 256) {         // four logits per lane, one key round per pick
        float lv[4];
#pragma unroll
        for (int i = 0; i < 4; i++) lv[i] = logits[(int64_t)t * E + min(lane_id() + 64 * i, E - 1)];
        topk_wave4(lv, E, k, ids + (int64_t)t * k, wout + (int64_t)t * k, nullptr);
        return;
    }
    topk_wave(logits + (int64_t)t * E, E, k, ids + (int64_t)t * k, wout + (int64_t)t * k);
}

}  // namespace

namespace bm_host {

int launch_router_gemv(const bitmoe_layer *L, const void *x, int x_dtype, int T, float *logits,
                       hipStream_t s) {
    dim3 g((L->E + 3) / 4);
    if (x_dtype == BITMOE_BF16)
        k_router_gemv<1><<<g, 256, 0, s>>>((const uint16_t *)L->router_w, x, T, L->H, L->E, logits);
    else
        k_router_gemv<0><<<g, 256, 0, s>>>((const uint16_t *)L->router_w, x, T, L->H, L->E, logits);
    BM_LAUNCH_CHECK();
    return BITMOE_OK;
}

int launch_router_mfma(const bitmoe_layer *L, const void *x, int T, float *logits, int32_t *ids, float *w,
                       float *part, hipStream_t s) {
    const int kslice = (L->H / 64 + kRouterSplit - 1) / kRouterSplit * 64;
    const int S = (L->H + kslice - 1) / kslice;
    dim3 g((T + 63) / 64, (L->E + 255) / 256, S);
    k_router_splitk<<<g, 256, 0, s>>>((const uint16_t *)x, (const uint16_t *)L->router_w, T, L->H, L->E, kslice,
                                      part);
    BM_LAUNCH_CHECK();
    k_topk_sum<<<(T + 3) / 4, 256, 0, s>>>(part, S, T, L->E, L->k, logits, ids, w);
    BM_LAUNCH_CHECK();
    return BITMOE_OK;
}

int launch_topk(const float *logits, int T, int E, int k, int32_t *ids, float *w, hipStream_t s) {
    k_topk<<<(T + 3) / 4, 256, 0, s>>>(logits, T, E, k, ids, w);
    BM_LAUNCH_CHECK();
    return BITMOE_OK;
}

}  // namespace bm_host
