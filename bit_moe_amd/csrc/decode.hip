// Decode FFN: fused dequant-GEMVs over the active experts' packed blocks.
//
// y[t] = sum_j w[t][j] * D_e(silu(G_e x_t) * U_e x_t)  (+ shared expert)
// with up/gate in the IQ2_XXS-style codebook format and down in Q2_K, the
// shared expert in bf16 (page "ds4 : analyse pratique pour un usage
// documente", section "Support de modeles et choix de quantification").
// Decoding is bandwidth-bound (page "Faire tenir un MoE de 284B dans un
// portable de 128 Go", section "Un pre-remplissage a 790 t/s revele le
// veritable goulot d'etranglement"): each active expert's blocks are read
// from HBM once per call and decoded in registers.
//
// Launches (T <= 128/k: three; larger batches add a routing/bucketing
// launch, experts chosen by several tokens a second gate/up and down):
//   front  : router rows; clears the combine counters
//            || shared-expert gate/up partial sums per (panel, K chunk)
//   gateup : routing of the batch (top-k and bucketing, in every
//            workgroup), then routed gate/up + SwiGLU per (active expert,
//            64-row panel) through run lookup tables built in LDS
//   down   : routed down per (active expert, 64-row panel) || shared down
//            per (panel, K chunk), its h built from the gate/up partials;
//            the last workgroup to finish a panel combines it,
//            y = sum of the k weighted slots + shared partials, in a fixed
//            order, so results are reproducible run to run.
//
// Mapping: lane r of every wave owns row P*64 + r of a panel (tiled layout),
// so one 16-byte load by 64 lanes is one contiguous 1 KiB access; the waves
// of a workgroup split K and meet once in LDS.  Activations are identical
// for all lanes and arrive through wave-uniform (scalar) loads.
#include <hip/hip_ext.h>

#include <algorithm>
#include <mutex>

#include "device_util.h"

namespace {

using namespace bm;

constexpr int kW = bm_cfg::kFrontWaves;   // waves per front workgroup
using bm_cfg::kRouterRowWaves;       // several tokens: waves per router row in the front launch
constexpr int kWG = 16;            // waves per routed gate/up workgroup
constexpr int kWD = 4;             // waves per down workgroup (at one token the plan sizes the
                                   // shared-down chunks so that all of them are resident at once)
constexpr int kNT = 4;             // tokens per pass over the weights
using bm_cfg::kMaxChunks;           // K chunks of the shared expert, at most
// per token, the LDS staging of a routed down wave's two superblocks of h:
// 64 pieces of 8 fp16, 16 pieces of two {hs, hb}, two pieces of 4 scales
constexpr int kHst = 64 + 16 + 2;
// 16-byte pieces per load batch of a gate/up wave (fewer when several
// tokens share the pass, to bound register use)
template <int NT>
constexpr int pieces_per_batch() { return NT == 1 ? 2 : 1; }

// ---- per-token dot products --------------------------------------------------

// sum_i w_i * x_i over 8 weights (4 bf16 pairs), bf16 or fp32 activations.
template <int XBF16>
BM_DEV float dot8(uint2 lo, uint2 hi, const void *xp, float acc) {
    if (XBF16) {
        const uint4 xv = *reinterpret_cast<const uint4 *>(xp);
        acc = dot2_bf16(lo.x, xv.x, acc);
        acc = dot2_bf16(lo.y, xv.y, acc);
        acc = dot2_bf16(hi.x, xv.z, acc);
        acc = dot2_bf16(hi.y, xv.w, acc);
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(xp);
        const float4 a = p[0], b = p[1];
        acc = fmaf(bf16_lo(lo.x), a.x, acc); acc = fmaf(bf16_hi(lo.x), a.y, acc);
        acc = fmaf(bf16_lo(lo.y), a.z, acc); acc = fmaf(bf16_hi(lo.y), a.w, acc);
        acc = fmaf(bf16_lo(hi.x), b.x, acc); acc = fmaf(bf16_hi(hi.x), b.y, acc);
        acc = fmaf(bf16_lo(hi.y), b.z, acc); acc = fmaf(bf16_hi(hi.y), b.w, acc);
    }
    return acc;
}

template <int XBF16>
BM_DEV const void *xrow(const void *x, int t, int H, int k) {
    return XBF16 ? (const void *)(static_cast<const uint16_t *>(x) + (int64_t)t * H + k)
                 : (const void *)(static_cast<const float *>(x) + (int64_t)t * H + k);
}

// One group's activations (32 values per token), held in scalar registers
// when the activations are bf16.
template <int XBF16, int NT>
struct XGroup {
    uint4 v[XBF16 ? NT : 1][4];
};

template <int XBF16, int NT>
BM_DEV void load_xgroup(XGroup<XBF16, NT> &g, const void *__restrict__ x, const int (&tok)[NT], int H, int gg) {
#pragma unroll
    for (int t = 0; t < NT; t++) {
        if (XBF16) {
            const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + (int64_t)tok[t] * H + 32 * gg);
#pragma unroll
            for (int q = 0; q < 4; q++) g.v[t][q] = p[q];
        }
    }
}

// One IQ2X group (32 weights, words W0, W1) of this lane's row dotted with
// NT activation rows.  Each run of 8 weights is two 16-byte lookups (the
// codebook row's magnitudes as bf16 pairs, the sign masks of its sign
// byte), four XORs giving the signed bf16 pairs, and four bf16 dot
// products per token; the group scale d/8 (2s+1) is applied to the group's
// fp32 sum.  SGN: bytes of the sign table (the half table drops the scale
// bit from the offset).
template <int XBF16, int NT, int SGN>
BM_DEV void iq2x_group(uint32_t W0, uint32_t W1, float dq8, uint32_t lc,
                       const XGroup<XBF16, NT> &xg, const void *x, const int (&tok)[NT], int H, int gg,
                       float (&acc)[NT]) {
    const float scale = dq8 * (float)iq2x_scale_odd(W0, W1);
    uint4 m[4], g[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const uint32_t W = r < 2 ? W0 : W1;
        const uint32_t so = lut_sgn_off(W, lc, r & 1);
        m[r] = lds_ld16(lut_mag_off(W, lc, r & 1));
        g[r] = lds_ld16(SGN == kLutSgnFull ? so : so & ~0x8000u);
    }
    float part[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) part[t] = 0.f;
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const uint2 lo = make_uint2(m[r].x ^ g[r].x, m[r].y ^ g[r].y);
        const uint2 hi = make_uint2(m[r].z ^ g[r].z, m[r].w ^ g[r].w);
#pragma unroll
        for (int t = 0; t < NT; t++) {
            if (XBF16) {
                const uint4 xv = xg.v[t][r];
                part[t] = dot2_bf16(lo.x, xv.x, part[t]);
                part[t] = dot2_bf16(lo.y, xv.y, part[t]);
                part[t] = dot2_bf16(hi.x, xv.z, part[t]);
                part[t] = dot2_bf16(hi.y, xv.w, part[t]);
            } else {
                part[t] = dot8<0>(lo, hi, xrow<0>(x, tok[t], H, 32 * gg + 8 * r), part[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = fmaf(scale, part[t], acc[t]);
}

// Even split of [0, n) over `parts`; returns [lo, hi) of part `i`.
BM_DEV void split_range(int n, int parts, int i, int &lo, int &hi) {
    lo = (int)((int64_t)n * i / parts);
    hi = (int)((int64_t)n * (i + 1) / parts);
}

// Shared-expert gate/up partial sums of panel P over K pieces [c0, c1) for
// tokens t0..t0+NT-1, by NW waves; sgp layout [kc_sg][2][T][I].
template <int XBF16, int NT, int NW>
BM_DEV void shared_gateup_pass(int H, int I, int T, int t0, int P, int c0, int c1,
                               const uint4 *__restrict__ sg, const uint4 *__restrict__ su,
                               const void *__restrict__ x, float *__restrict__ gp,
                               float *__restrict__ up_, float *red) {
    const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int K8 = H / 8;
    int tok[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) tok[t] = min(t0 + t, T - 1);
    float ag[NT], au[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) ag[t] = au[t] = 0.f;
    int w0, w1;
    split_range(c1 - c0, NW, wv, w0, w1);
    // the loads of up to kB pieces of both matrices at once (past the
    // wave's range: its last piece again, unused)
    constexpr int kB = NT == 1 ? 8 : 4;
    for (int cb = c0 + w0; cb < c0 + w1; cb += kB) {
        uint4 gw[kB], uw[kB];
#pragma unroll
        for (int i = 0; i < kB; i++) {
            const int64_t pc = ((int64_t)P * K8 + min(cb + i, c0 + w1 - 1)) * 64 + lane;
            gw[i] = sg[pc];
            uw[i] = su[pc];
        }
        __builtin_amdgcn_sched_barrier(0);      // keep the batch's loads together, ahead of their use
        // every loaded piece is used (a branch around the extra ones would
        // let the compiler sink their loads next to the use); the extra
        // ones' sums are dropped
#pragma unroll
        for (int i = 0; i < kB; i++) {
            const int c = min(cb + i, c0 + w1 - 1);
            const bool keep = cb + i < c0 + w1;
#pragma unroll
            for (int t = 0; t < NT; t++) {
                const void *xp = xrow<XBF16>(x, tok[t], H, 8 * c);
                const float g = dot8<XBF16>(make_uint2(gw[i].x, gw[i].y), make_uint2(gw[i].z, gw[i].w), xp, ag[t]);
                const float u = dot8<XBF16>(make_uint2(uw[i].x, uw[i].y), make_uint2(uw[i].z, uw[i].w), xp, au[t]);
                ag[t] = keep ? g : ag[t];
                au[t] = keep ? u : au[t];
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; t++) {
        red[((wv * kNT + t) * 2 + 0) * 64 + lane] = ag[t];
        red[((wv * kNT + t) * 2 + 1) * 64 + lane] = au[t];
    }
    __syncthreads();
    if (wv < NT && t0 + wv < T) {
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int v = 0; v < NW; v++) {
            g += red[((v * kNT + wv) * 2 + 0) * 64 + lane];
            u += red[((v * kNT + wv) * 2 + 1) * 64 + lane];
        }
        gp[(int64_t)(t0 + wv) * I + P * 64 + lane] = g;
        up_[(int64_t)(t0 + wv) * I + P * 64 + lane] = u;
    }
    __syncthreads();
}

// Shared-expert gate/up partial sums of panel P over K pieces [c0, c1) for
// the tokens t0 .. t0+15 on the matrix cores (bf16 activations; a dense
// contraction once there are several tokens), so that the bf16 weights
// stream once for 16 tokens.  v_mfma_f32_16x16x32_bf16 takes the weights as
// they are stored as operand B: lane l's 8 values (panel row l) are column
// l % 16 of K block l / 16 of the instruction's 32.  Operand A carries the
// activations of 4 tokens per instruction, block-diagonally: A row m = 4 j +
// t (token t of the four) is nonzero only on K block j, so D row m, column n
// is token t against panel row 16 j + n, and lane l's four results are panel
// row l for the four tokens.  Lanes off the diagonal read a zero row.  The chunk's
// activations are staged in LDS (xs), rows padded by 16 bytes so that the
// four token rows fall on different banks; the 16 waves' sums meet in red,
// one group of four tokens at a time.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kSgMfmaPieces = 160;          // K pieces of a chunk the LDS staging holds
constexpr int kSgXsBytes = 16 * (kSgMfmaPieces * 16 + 16) + 16;
BM_DEV void shared_gateup_mfma(int H, int I, int T, int t0, int P, int c0, int c1,
                               const uint4 *__restrict__ sg, const uint4 *__restrict__ su,
                               const uint16_t *__restrict__ x, float *__restrict__ gp, float *__restrict__ up_,
                               float *red, uint8_t *xs) {
    const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int K8 = H / 8, nc = c1 - c0, nt = min(16, T - t0);
    const int stride = nc * 16 + 16, zero = 16 * stride;
    __syncthreads();                     // the previous group's readers of xs and red are done
    for (int i = threadIdx.x; i < 16 * nc; i += blockDim.x) {
        const int tt = i / nc, cl = i - tt * nc;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (tt < nt) v = *reinterpret_cast<const uint4 *>(x + (int64_t)(t0 + tt) * H + 8 * (c0 + cl));
        *reinterpret_cast<uint4 *>(xs + tt * stride + cl * 16) = v;
    }
    if (threadIdx.x == 0) *reinterpret_cast<uint4 *>(xs + zero) = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    const int j = lane >> 4, m = lane & 15;
    const bool act = (m >> 2) == j;
    f32x4_t ag[4], au[4];
#pragma unroll
    for (int g = 0; g < 4; g++) ag[g] = au[g] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    int w0, w1;
    split_range(nc, kW, wv, w0, w1);
    constexpr int kB = 4;
    const uint4 *gbase = sg + (int64_t)P * K8 * 64 + lane, *ubase = su + (int64_t)P * K8 * 64 + lane;
    for (int cb = w0; cb < w1; cb += kB) {
        uint4 gw[kB], uw[kB];
#pragma unroll
        for (int i = 0; i < kB; i++) {
            const int pc = c0 + min(cb + i, w1 - 1);
            gw[i] = gbase[(int64_t)pc * 64];
            uw[i] = ubase[(int64_t)pc * 64];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kB; i++) {
            // past the wave's share: the zero row (the piece is its last one again)
            const int cl = min(cb + i, w1 - 1);
            const bool use = act && cb + i < w1;
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int addr = use ? (4 * g + (m & 3)) * stride + cl * 16 : zero;
                const uint4 a = *reinterpret_cast<const uint4 *>(xs + addr);
                ag[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                                __builtin_bit_cast(bf16x8_t, gw[i]), ag[g], 0, 0, 0);
                au[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                                __builtin_bit_cast(bf16x8_t, uw[i]), au[g], 0, 0, 0);
            }
        }
    }
    // lane l, result i of group g: panel row l, token 4 g + i
#pragma unroll
    for (int g = 0; g < 4; g++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            red[((wv * 4 + i) * 2 + 0) * 64 + lane] = ag[g][i];
            red[((wv * 4 + i) * 2 + 1) * 64 + lane] = au[g][i];
        }
        __syncthreads();
        if (wv < 4 && 4 * g + wv < nt) {
            float gs = 0.f, us = 0.f;
#pragma unroll
            for (int v = 0; v < kW; v++) {
                gs += red[((v * 4 + wv) * 2 + 0) * 64 + lane];
                us += red[((v * 4 + wv) * 2 + 1) * 64 + lane];
            }
            gp[(int64_t)(t0 + 4 * g + wv) * I + P * 64 + lane] = gs;
            up_[(int64_t)(t0 + 4 * g + wv) * I + P * 64 + lane] = us;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Bucketing of a decode batch's n <= kWaveBucketMax pairs on wave 0 of the
// calling workgroup (every thread calls it: it holds block barriers; sk is
// kWaveBucketMax ints of LDS): counts, offsets, perm, the active list, with
// tiles the row tiles of the experts chosen by several tokens, with single
// the experts chosen by one token, compacted as {expert, pair row, 1, token}
// (their gate/up items are claimed one at a time).
// ---------------------------------------------------------------------------
BM_DEV void bucket_decode_wave(const int32_t *__restrict__ ids, int n, int k, int E, int32_t *__restrict__ counts,
                               int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
                               int32_t *__restrict__ active, int32_t *__restrict__ n_active,
                               int32_t *__restrict__ tiles, int32_t *__restrict__ n_tiles,
                               int4 *__restrict__ single, int32_t *__restrict__ n_single, int *sk) {
    const int wv = threadIdx.x >> 6;
    if (wv == 0) bucket_wave_rank(ids, n, E, perm, sk);
    __syncthreads();
    if (wv == 0) bucket_wave_lists(n, sk, counts, offsets, active, n_active);
    if (wv == 0 && tiles) bucket_wave_multi_tiles(n, sk, tiles, n_tiles);
    if (!single) return;
    __syncthreads();
    if (wv == 0) {
        const int lane = lane_id(), na = *n_active;
        const uint64_t below = (1ull << lane) - 1ull;
        int4 v[2];
        bool one[2];
#pragma unroll
        for (int m = 0; m < 2; m++) {
            const int sl = lane + 64 * m;
            one[m] = false;
            if (sl < na) {
                const int e = active[sl], off = offsets[e];
                one[m] = counts[e] == 1;
                v[m] = make_int4(e, off, 1, perm[off] / k);
            }
        }
        const uint64_t B0 = __ballot(one[0]), B1 = __ballot(one[1]);
        if (one[0]) single[__popcll(B0 & below)] = v[0];
        if (one[1]) single[__popcll(B0) + __popcll(B1 & below)] = v[1];
        if (lane == 0) *n_single = __popcll(B0) + __popcll(B1);
    }
}

// Router partial logits of T <= NT tokens over the row's 512-wide K steps
// [s0, s1), all of a lane's pieces loaded at once (at most 4 steps); wave
// sums to out[0..NT) (LDS).  Tokens past T repeat token 0 and are not used.
template <int XBF16, int NT>
BM_DEV void router_row_part(const uint4 *__restrict__ wrow, const void *__restrict__ x, int H, int T, int s0,
                            int s1, float *out) {
    constexpr int CH = 4;
    const int lane = lane_id();
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = 0.f;
    const int spare = lane < H / 8 ? lane : 0;
    for (int sb = s0; sb < s1; sb += CH) {
        uint4 wv[CH];
#pragma unroll
        for (int i = 0; i < CH; i++) {
            // steps past the part, and the idle half-wave of a half-width
            // last step, re-read a piece of the row's first step, unused
            const int s = sb + i, k = 512 * s + 8 * lane;
            wv[i] = wrow[(s < s1 && k < H) ? 64 * s + lane : spare];
        }
#pragma unroll
        for (int i = 0; i < CH; i++) {
            const int s = sb + i, k = 512 * s + 8 * lane;
            if (!(s < s1 && k < H)) continue;
#pragma unroll
            for (int t = 0; t < NT; t++) acc[t] = router_dot8<XBF16, NT>(wv[i], x, H, t < T ? t : 0, k, acc[t]);
        }
    }
#pragma unroll
    for (int t = 0; t < NT; t++) {
        const float v = wave_sum(acc[t]);
        if (lane == 0) out[t] = v;
    }
}

// Decode batches: work that the front launch's first n_wg workgroups take
// before its other roles.  With ids (given by the caller) the first one
// buckets them on its wave 0 (no mid launch); with x16 workgroup t < T
// prepares token t's fp16 activations for the prefill kernels.
struct FrontPrep {
    int n_wg, k;
    const int32_t *ids;
    bm_host::Buckets bk;        // tiles null unless the prefill kernels run
    int4 *single;               // null unless the prefill kernels run
    int32_t *n_single;
    uint16_t *x16;
    float *xsc;
};
template <int XBF16>
BM_DEV void front_prep(int H, int T, int E, const void *x, const FrontPrep &pr, int b, float *lds) {
    if (b == 0 && pr.ids)
        bucket_decode_wave(pr.ids, T * pr.k, pr.k, E, pr.bk.counts, pr.bk.offsets, pr.bk.perm, pr.bk.active,
                           pr.bk.n_active, pr.bk.tiles, pr.bk.n_tiles, pr.single, pr.n_single,
                           reinterpret_cast<int *>(lds));
    if (pr.x16 && b < T) xprep_token_block<XBF16>(H, x, b, pr.x16, pr.xsc, lds + kWaveBucketMax);
}

// Workgroup roles, in blockIdx order: preparation (pr.n_wg, above) | router
// rows (n_rwg: one per wave for one token, one per kRouterRowWaves waves for
// several) | shared-expert gate/up partial sums per
// (panel, K chunk).  Workgroup 0 also clears the down launch's per-panel
// combine counters.  Launched with
// kW waves, or (no shared chunks) fewer, so that the router rows spread
// over more compute units.
template <int XBF16>
__global__ void __launch_bounds__(kW * 64) __attribute__((amdgpu_waves_per_eu(4)))
k_dec_front(int H, int I, int E, int T, int n_rwg, int kc_sg, const uint16_t *__restrict__ wr,
            const void *__restrict__ x, float *__restrict__ logits, int32_t *__restrict__ ycount,
            int32_t *__restrict__ gctr, const uint4 *__restrict__ sg, const uint4 *__restrict__ su,
            float *__restrict__ sgp, FrontPrep pr) {
    __shared__ float red[kW * kNT * 2 * 64];
    static_assert(kW * kNT * 2 * 64 >= kWaveBucketMax + kW, "front prep LDS");
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), nw = blockDim.x >> 6;
    int b = blockIdx.x;
    if (b == 0) {
        for (int p = threadIdx.x; p < H / 64; p += blockDim.x) ycount[p] = 0;
        if (gctr && threadIdx.x == 0) *gctr = 0;
    }
    if (b < pr.n_wg) {
        front_prep<XBF16>(H, T, E, x, pr, b, red);
        return;
    }
    b -= pr.n_wg;
    if (b < n_rwg && T > 1) {
        // several tokens: kRouterRowWaves waves per row, each over a quarter
        // of the row's 512-wide K steps, the parts summed in a fixed order
        static_assert(kW % kRouterRowWaves == 0 && kW * 16 <= kW * kNT * 2 * 64, "router row parts");
        const int e = b * (nw / kRouterRowWaves) + wv / kRouterRowWaves, part = wv % kRouterRowWaves;
        const bool live = e < E;
        const uint4 *wrow = reinterpret_cast<const uint4 *>(wr + (int64_t)min(e, E - 1) * H);
        int s0, s1;
        split_range((H + 511) / 512, kRouterRowWaves, part, s0, s1);
        if (T <= 4)
            router_row_part<XBF16, 4>(wrow, x, H, T, s0, s1, red + wv * 16);
        else if (T <= 8)
            router_row_part<XBF16, 8>(wrow, x, H, T, s0, s1, red + wv * 16);
        else
            router_row_part<XBF16, 16>(wrow, x, H, T, s0, s1, red + wv * 16);
        __syncthreads();
        if (live && part == 0 && lane_id() < T) {
            float v = 0.f;
#pragma unroll
            for (int j = 0; j < kRouterRowWaves; j++) v += red[(wv + j) * 16 + lane_id()];
            logits[(int64_t)lane_id() * E + e] = v;
        }
        return;
    }
    if (b < n_rwg) {
        const int e = b * nw + wv;
        if (e >= E) return;
        const uint4 *wrow = reinterpret_cast<const uint4 *>(wr + (int64_t)e * H);
        if (T == 1)
            router_row<XBF16, 1>(wrow, x, H, T, E, e, logits);
        else if (T <= 4)
            router_row<XBF16, 4>(wrow, x, H, T, E, e, logits);
        else
            router_row<XBF16, 16>(wrow, x, H, T, E, e, logits);
        return;
    }
    b -= n_rwg;
    // shared gate/up: panel P of the I rows, K chunk c (none without a
    // shared expert: the grid then holds one workgroup for the counters)
    if (kc_sg == 0 || b >= (I / 64) * kc_sg) return;
    const int P = b / kc_sg, c = b % kc_sg;
    int c0, c1;
    split_range(H / 8, kc_sg, c, c0, c1);
    float *gp = sgp + (int64_t)(c * 2 + 0) * T * I;
    float *up_ = sgp + (int64_t)(c * 2 + 1) * T * I;
    // several bf16 tokens: the matrix cores, 16 tokens per pass over the weights
    if (XBF16 && T > 1 && c1 - c0 <= kSgMfmaPieces) {
        __shared__ __attribute__((aligned(16))) uint8_t xs[kSgXsBytes];
        for (int t0 = 0; t0 < T; t0 += 16)
            shared_gateup_mfma(H, I, T, t0, P, c0, c1, sg, su, static_cast<const uint16_t *>(x), gp, up_, red, xs);
        return;
    }
    for (int t0 = 0; t0 < T; t0 += kNT) {
        if (T - t0 == 1)
            shared_gateup_pass<XBF16, 1, kW>(H, I, T, t0, P, c0, c1, sg, su, x, gp, up_, red);
        else
            shared_gateup_pass<XBF16, kNT, kW>(H, I, T, t0, P, c0, c1, sg, su, x, gp, up_, red);
    }
}

// ---------------------------------------------------------------------------
// mid: one workgroup of kBT threads.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kBT)
k_dec_mid(int E, int k, int T, const float *__restrict__ logits, int32_t *__restrict__ ids,
          float *__restrict__ w, int do_bucket, int32_t *__restrict__ counts,
          int32_t *__restrict__ offsets, int32_t *__restrict__ perm, int32_t *__restrict__ active,
          int32_t *__restrict__ n_active, int32_t *__restrict__ tiles, int32_t *__restrict__ n_tiles,
          int4 *__restrict__ single, int32_t *__restrict__ n_single) {
    extern __shared__ int smem[];
    __shared__ int swave[kBW + 1];
    const int tid = threadIdx.x, wv = tid >> 6;
    if (logits) {
        for (int t = wv; t < T; t += kBW) {
            if (E <= 256) {
                float lv[4];
#pragma unroll
                for (int i = 0; i < 4; i++) lv[i] = logits[(int64_t)t * E + min(lane_id() + 64 * i, E - 1)];
                topk_wave4(lv, E, k, ids + (int64_t)t * k, w + (int64_t)t * k, nullptr);
            } else {
                topk_wave(logits + (int64_t)t * E, E, k, ids + (int64_t)t * k, w + (int64_t)t * k);
            }
        }
        __threadfence_block();
        __syncthreads();
    }
    if (!do_bucket) return;
    const int n = T * k;
    if (n <= kWaveBucketMax) {        // decode batches: one wave, no block scans
        bucket_decode_wave(ids, n, k, E, counts, offsets, perm, active, n_active, tiles, n_tiles, single, n_single,
                           smem);
        return;
    }
    bucket_block(ids, n, E, counts, offsets, perm, active, n_active, nullptr, nullptr, 1, smem, swave);
}

// ---------------------------------------------------------------------------
// gateup: routed gate/up + SwiGLU || shared down partial sums over K.
// grid = slots*(I/64) routed workgroups, then (H/64)*kc_sd shared ones.
// ---------------------------------------------------------------------------
struct Tok {
    int cnt, off, e;
};

// Cross-wave sums of the gate/up partials of NT tokens, then for token
// t0 + t (wave t): h = silu(g) u as fp16 scaled by 2^-e so that the panel's
// largest |h| lies in [2^14, 2^15) (no overflow, full fp16 precision; 2^e is
// kept), with per-16-column sums for the down launch.
template <int NT, int SUMS = 1>
BM_DEV void gateup_epilogue(int I, const Tok &tk, int t0, int P, const float (&ag)[NT], const float (&au)[NT],
                            uint16_t *__restrict__ h, float2 *__restrict__ hsum2, float *__restrict__ hscale,
                            float *red) {
    const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int t = 0; t < NT; t++) {
        red[((wv * NT + t) * 2 + 0) * 64 + lane] = ag[t];
        red[((wv * NT + t) * 2 + 1) * 64 + lane] = au[t];
    }
    __syncthreads();
    if (wv < NT && t0 + wv < tk.cnt) {
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int v = 0; v < kWG; v++) {
            g += red[((v * NT + wv) * 2 + 0) * 64 + lane];
            u += red[((v * NT + wv) * 2 + 1) * 64 + lane];
        }
        const float hv = silu(g) * u;
        const int n = P * 64 + lane;
        const int64_t row = tk.off + t0 + wv;
        const float amax = wave_max_f32(fabsf(hv));
        int e = amax > 0.f ? (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 127 - 14 : 0;
        e = max(-100, min(100, e));
        const float inv = __uint_as_float((uint32_t)(127 - e) << 23), scl = __uint_as_float((uint32_t)(127 + e) << 23);
        const _Float16 hf = (_Float16)(hv * inv);
        h[row * I + n] = __builtin_bit_cast(uint16_t, hf);
        if (SUMS) {
            // per 16 columns: the sum of h (the Q2K down's min term)
            const float hs = row16_sum((float)hf);
            if ((lane & 15) == 15) hsum2[row * (I / 16) + (n >> 4)] = make_float2(hs, 0.f);
        }
        if (lane == 0) hscale[row * (I / 64) + P] = scl;
    }
    __syncthreads();
}

template <int XBF16, int NT, int SGN>
BM_DEV void routed_gateup_pass(int H, int I, int k, const Tok &tk, int t0, int P,
                               const uint8_t *__restrict__ gate, const uint8_t *__restrict__ up,
                               const void *__restrict__ x, const int32_t *perm,
                               uint16_t *__restrict__ h, float2 *__restrict__ hsum2,
                               float *__restrict__ hscale, float *red) {
    const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int tok[NT];
#pragma unroll
    for (int t = 0; t < NT; t++)
        tok[t] = __builtin_amdgcn_readfirstlane(perm[tk.off + min(t0 + t, tk.cnt - 1)] / k);
    float ag[NT], au[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) ag[t] = au[t] = 0.f;
    const int nb = H / kQK;
    const int64_t slab = (int64_t)I * nb * 66;
    const uint8_t *G = gate + tk.e * slab, *U = up + tk.e * slab;
    const uint4 *gq = reinterpret_cast<const uint4 *>(G) + (int64_t)P * nb * 4 * 64 + lane;
    const uint4 *uq = reinterpret_cast<const uint4 *>(U) + (int64_t)P * nb * 4 * 64 + lane;
    const uint16_t *gd = reinterpret_cast<const uint16_t *>(G + (int64_t)I * nb * 64) + (int64_t)P * nb * 64 + lane;
    const uint16_t *ud = reinterpret_cast<const uint16_t *>(U + (int64_t)I * nb * 64) + (int64_t)P * nb * 64 + lane;
    // this wave's share of the panel's 16-byte pieces (two groups each), in
    // batches of kPB; the next batch is in flight while one is decoded
    int p0, p1;
    split_range(4 * nb, kWG, wv, p0, p1);
    constexpr int kPB = pieces_per_batch<NT>();
    uint4 g4[kPB], u4[kPB], ng[kPB], nu[kPB];
    uint32_t gdw[kPB], udw[kPB], ngd[kPB], nud[kPB];
    auto load = [&](int pb, uint4 (&a4)[kPB], uint4 (&b4)[kPB], uint32_t (&da)[kPB], uint32_t (&db)[kPB]) {
#pragma unroll
        for (int i = 0; i < kPB; i++) {
            const int pc = min(pb + i, p1 - 1);      // a short last batch re-reads its last piece
            a4[i] = gq[(int64_t)pc * 64];
            b4[i] = uq[(int64_t)pc * 64];
            da[i] = gd[(int64_t)(pc >> 2) * 64];
            db[i] = ud[(int64_t)(pc >> 2) * 64];
        }
    };
    if (p0 < p1) load(p0, g4, u4, gdw, udw);
    const uint32_t lc = lut_lane_const(lane);
    // activations of the current group, the next one in flight
    XGroup<XBF16, NT> xa, xb;
    if (p0 < p1) load_xgroup<XBF16, NT>(xa, x, tok, H, 2 * p0);
    for (int pb = p0; pb < p1; pb += kPB) {
        if (pb + kPB < p1) load(pb + kPB, ng, nu, ngd, nud);
        const int n = min(kPB, p1 - pb);
#pragma unroll
        for (int i = 0; i < kPB; i++) {
            if (i < n) {
                const int gg = 2 * (pb + i);
                const float dg = 0.125f * fp16_to_f32(gdw[i]), du = 0.125f * fp16_to_f32(udw[i]);
                load_xgroup<XBF16, NT>(xb, x, tok, H, gg + 1);
                iq2x_group<XBF16, NT, SGN>(g4[i].x, g4[i].y, dg, lc, xa, x, tok, H, gg, ag);
                iq2x_group<XBF16, NT, SGN>(u4[i].x, u4[i].y, du, lc, xa, x, tok, H, gg, au);
                load_xgroup<XBF16, NT>(xa, x, tok, H, pb + i + 1 < p1 ? gg + 2 : gg);
                iq2x_group<XBF16, NT, SGN>(g4[i].z, g4[i].w, dg, lc, xb, x, tok, H, gg + 1, ag);
                iq2x_group<XBF16, NT, SGN>(u4[i].z, u4[i].w, du, lc, xb, x, tok, H, gg + 1, au);
            }
        }
#pragma unroll
        for (int i = 0; i < kPB; i++) {
            g4[i] = ng[i];
            u4[i] = nu[i];
            gdw[i] = ngd[i];
            udw[i] = nud[i];
        }
    }
    gateup_epilogue<NT>(I, tk, t0, P, ag, au, h, hsum2, hscale, red);
}

// The same for an expert chosen by one token: the wave's pieces stream
// through a ring of kRing register slots, each refilled with the piece
// kRing places ahead as soon as it is decoded (no copies between slots, so
// the loads stay in flight while earlier pieces are decoded).
template <int XBF16, int SGN>
BM_DEV void routed_gateup_1(int H, int I, int k, const Tok &tk, int P, const uint8_t *__restrict__ gate,
                            const uint8_t *__restrict__ up, const void *__restrict__ x, const int32_t *perm,
                            uint16_t *__restrict__ h, float2 *__restrict__ hsum2, float *__restrict__ hscale,
                            float *red, int tok0 = -1, int nrw = kWG) {
    constexpr int kRing = 4;
    const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tok[1] = {__builtin_amdgcn_readfirstlane(tok0 >= 0 ? tok0 : perm ? perm[tk.off] / k : 0)};
    const int nb = H / kQK;
    const int64_t slab = (int64_t)I * nb * 66;
    const uint8_t *G = gate + tk.e * slab, *U = up + tk.e * slab;
    const uint4 *gq = reinterpret_cast<const uint4 *>(G) + (int64_t)P * nb * 4 * 64 + lane;
    const uint4 *uq = reinterpret_cast<const uint4 *>(U) + (int64_t)P * nb * 4 * 64 + lane;
    const uint16_t *gd = reinterpret_cast<const uint16_t *>(G + (int64_t)I * nb * 64) + (int64_t)P * nb * 64 + lane;
    const uint16_t *ud = reinterpret_cast<const uint16_t *>(U + (int64_t)I * nb * 64) + (int64_t)P * nb * 64 + lane;
    int p0 = 0, p1 = 0;                                // waves from nrw on take none
    if (wv < nrw) split_range(4 * nb, nrw, wv, p0, p1);
    struct Piece { uint4 g, u; uint32_t dg, du; };
    // pieces past the wave's last re-read it (cached) and are not decoded
    auto load = [&](int pc, Piece &q) {
        pc = min(pc, p1 - 1);
        q.g = gq[(int64_t)pc * 64];
        q.u = uq[(int64_t)pc * 64];
        q.dg = gd[(int64_t)(pc >> 2) * 64];
        q.du = ud[(int64_t)(pc >> 2) * 64];
    };
    float ag[1] = {0.f}, au[1] = {0.f};
    const uint32_t lc = lut_lane_const(lane);
    auto decode = [&](int pc, const Piece &q) {
        XGroup<XBF16, 1> x0, x1;
        load_xgroup<XBF16, 1>(x0, x, tok, H, 2 * pc);
        load_xgroup<XBF16, 1>(x1, x, tok, H, 2 * pc + 1);
        const float dg = 0.125f * fp16_to_f32(q.dg), du = 0.125f * fp16_to_f32(q.du);
        iq2x_group<XBF16, 1, SGN>(q.g.x, q.g.y, dg, lc, x0, x, tok, H, 2 * pc, ag);
        iq2x_group<XBF16, 1, SGN>(q.u.x, q.u.y, du, lc, x0, x, tok, H, 2 * pc, au);
        iq2x_group<XBF16, 1, SGN>(q.g.z, q.g.w, dg, lc, x1, x, tok, H, 2 * pc + 1, ag);
        iq2x_group<XBF16, 1, SGN>(q.u.z, q.u.w, du, lc, x1, x, tok, H, 2 * pc + 1, au);
    };
    // decode a slot, then refill it (the refill stays after the decode of
    // the registers it overwrites)
    auto step = [&](int pc, Piece &q) {
        decode(pc, q);
        __builtin_amdgcn_sched_barrier(0);
        load(pc + kRing, q);
        __builtin_amdgcn_sched_barrier(0);
    };
    static_assert(kRing == 4, "four slots below");
    if (p0 < p1) {
        Piece q0, q1, q2, q3;
        load(p0, q0);
        load(p0 + 1, q1);
        load(p0 + 2, q2);
        load(p0 + 3, q3);
        int pc = p0;
        for (; pc + kRing <= p1; pc += kRing) {
            step(pc, q0);
            step(pc + 1, q1);
            step(pc + 2, q2);
            step(pc + 3, q3);
        }
        if (pc < p1) decode(pc, q0);
        if (pc + 1 < p1) decode(pc + 1, q1);
        if (pc + 2 < p1) decode(pc + 2, q2);
    }
    gateup_epilogue<1>(I, tk, 0, P, ag, au, h, hsum2, hscale, red);
}

// ---- MXFP4 routed experts ---------------------------------------------------
// A piece is one 32-weight block of a row (16 bytes, byte i holding weights
// 2i and 2i+1) with its scale byte X.  The hardware conversion turns each
// byte into two exact bf16 (gate/up: dotted with the bf16 activations) or
// fp16 (down: dotted with the fp16 h) values; the block's fp32 sum is then
// multiplied by 2^(X-127).  Piece pc of row P*64 + r (pc = 8 kb + c) sits at
// ((P nb 8 + pc) 64 + r) * 16, its scale at N K/2 + (P nb 64 + (pc >> 3) 64
// + r) 8 + (pc & 7), nb = K/256.
template <int XBF16, int NT>
BM_DEV void mx_piece(uint4 q, float scale, const XGroup<XBF16, NT> &xg, const void *x, const int (&tok)[NT],
                     int H, int pc, float (&acc)[NT]) {
    float part[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) part[t] = 0.f;
    const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const uint32_t W = qw[r];
        const uint2 lo = make_uint2(fp4x2_bf16<0>(W), fp4x2_bf16<1>(W));
        const uint2 hi = make_uint2(fp4x2_bf16<2>(W), fp4x2_bf16<3>(W));
#pragma unroll
        for (int t = 0; t < NT; t++) {
            if (XBF16) {
                const uint4 xv = xg.v[t][r];
                part[t] = dot2_bf16(lo.x, xv.x, part[t]);
                part[t] = dot2_bf16(lo.y, xv.y, part[t]);
                part[t] = dot2_bf16(hi.x, xv.z, part[t]);
                part[t] = dot2_bf16(hi.y, xv.w, part[t]);
            } else {
                part[t] = dot8<0>(lo, hi, xrow<0>(x, tok[t], H, 32 * pc + 8 * r), part[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = fmaf(scale, part[t], acc[t]);
}

struct MxRows {
    const uint4 *q;          // piece 0 of this lane's row
    const uint8_t *sc;       // scale byte of piece 0
    BM_DEV uint4 piece(int pc) const { return q[(int64_t)pc * 64]; }
    BM_DEV uint32_t scale(int pc) const { return sc[(int64_t)(pc >> 3) * 512 + (pc & 7)]; }
};
// rows of 64-row panel P of an expert's [N][K] slab at `slab`, this lane's row
BM_DEV MxRows mx_rows(const uint8_t *slab, int N, int K, int P) {
    const int nb = K / kQK, lane = lane_id();
    MxRows m;
    m.q = reinterpret_cast<const uint4 *>(slab) + (int64_t)P * nb * 8 * 64 + lane;
    m.sc = slab + (int64_t)N * K / 2 + ((int64_t)P * nb * 64 + lane) * 8;
    return m;
}

// Gate/up of panel P for tokens t0..t0+NT-1 of expert tk (MXFP4); the
// wave's pieces in batches of two, the next batch in flight.
template <int XBF16, int NT>
BM_DEV void mx_gateup_pass(int H, int I, int k, const Tok &tk, int t0, int P, const uint8_t *__restrict__ gate,
                           const uint8_t *__restrict__ up, const void *__restrict__ x, const int32_t *perm,
                           uint16_t *__restrict__ h, float *__restrict__ hscale, float *red) {
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int tok[NT];
#pragma unroll
    for (int t = 0; t < NT; t++)
        tok[t] = __builtin_amdgcn_readfirstlane(perm[tk.off + min(t0 + t, tk.cnt - 1)] / k);
    float ag[NT], au[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) ag[t] = au[t] = 0.f;
    const int64_t slab = (int64_t)I * H / 32 * 17;
    const MxRows G = mx_rows(gate + tk.e * slab, I, H, P), U = mx_rows(up + tk.e * slab, I, H, P);
    int p0, p1;
    split_range(8 * (H / kQK), kWG, wv, p0, p1);
    constexpr int kPB = 2;
    struct Batch { uint4 g[kPB], u[kPB]; uint32_t sg[kPB], su[kPB]; };
    auto load = [&](int pb, Batch &b) {
#pragma unroll
        for (int i = 0; i < kPB; i++) {
            const int pc = min(pb + i, p1 - 1);      // a short last batch re-reads its last piece
            b.g[i] = G.piece(pc);
            b.u[i] = U.piece(pc);
            b.sg[i] = G.scale(pc);
            b.su[i] = U.scale(pc);
        }
    };
    Batch cur{}, nxt{};
    if (p0 < p1) load(p0, cur);
    for (int pb = p0; pb < p1; pb += kPB) {
        if (pb + kPB < p1) load(pb + kPB, nxt);
#pragma unroll
        for (int i = 0; i < kPB; i++) {
            if (pb + i < p1) {
                XGroup<XBF16, NT> xg;
                load_xgroup<XBF16, NT>(xg, x, tok, H, pb + i);
                mx_piece<XBF16, NT>(cur.g[i], mx_scale(cur.sg[i]), xg, x, tok, H, pb + i, ag);
                mx_piece<XBF16, NT>(cur.u[i], mx_scale(cur.su[i]), xg, x, tok, H, pb + i, au);
            }
        }
        cur = nxt;
    }
    gateup_epilogue<NT, 0>(I, tk, t0, P, ag, au, h, nullptr, hscale, red);
}

// The same for an expert chosen by one token: the pieces stream through a
// ring of four register slots, each refilled as soon as it is decoded.
template <int XBF16>
BM_DEV void mx_gateup_1(int H, int I, int k, const Tok &tk, int P, const uint8_t *__restrict__ gate,
                        const uint8_t *__restrict__ up, const void *__restrict__ x, const int32_t *perm,
                        uint16_t *__restrict__ h, float *__restrict__ hscale, float *red, int tok0 = -1,
                        int nrw = kWG) {
    constexpr int kRing = 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tok[1] = {__builtin_amdgcn_readfirstlane(tok0 >= 0 ? tok0 : perm ? perm[tk.off] / k : 0)};
    const int64_t slab = (int64_t)I * H / 32 * 17;
    const MxRows G = mx_rows(gate + tk.e * slab, I, H, P), U = mx_rows(up + tk.e * slab, I, H, P);
    int p0 = 0, p1 = 0;                                // waves from nrw on take none
    if (wv < nrw) split_range(8 * (H / kQK), nrw, wv, p0, p1);
    struct Piece { uint4 g, u; uint32_t sg, su; };
    auto load = [&](int pc, Piece &q) {
        pc = min(pc, p1 - 1);                          // past the wave's last: re-read, not decoded
        q.g = G.piece(pc);
        q.u = U.piece(pc);
        q.sg = G.scale(pc);
        q.su = U.scale(pc);
    };
    float ag[1] = {0.f}, au[1] = {0.f};
    auto decode = [&](int pc, const Piece &q) {
        XGroup<XBF16, 1> xg;
        load_xgroup<XBF16, 1>(xg, x, tok, H, pc);
        mx_piece<XBF16, 1>(q.g, mx_scale(q.sg), xg, x, tok, H, pc, ag);
        mx_piece<XBF16, 1>(q.u, mx_scale(q.su), xg, x, tok, H, pc, au);
    };
    auto step = [&](int pc, Piece &q) {
        decode(pc, q);
        __builtin_amdgcn_sched_barrier(0);
        load(pc + kRing, q);
        __builtin_amdgcn_sched_barrier(0);
    };
    static_assert(kRing == 4, "four slots below");
    if (p0 < p1) {
        Piece q0, q1, q2, q3;
        load(p0, q0);
        load(p0 + 1, q1);
        load(p0 + 2, q2);
        load(p0 + 3, q3);
        int pc = p0;
        for (; pc + kRing <= p1; pc += kRing) {
            step(pc, q0);
            step(pc + 1, q1);
            step(pc + 2, q2);
            step(pc + 3, q3);
        }
        if (pc < p1) decode(pc, q0);
        if (pc + 1 < p1) decode(pc + 1, q1);
        if (pc + 2 < p1) decode(pc + 2, q2);
    }
    gateup_epilogue<1, 0>(I, tk, 0, P, ag, au, h, nullptr, hscale, red);
}

// Format dispatch of the routed gate/up passes.
template <int FMT, int XBF16, int SGN>
BM_DEV void gateup_1(int H, int I, int k, const Tok &tk, int P, const uint8_t *__restrict__ gate,
                     const uint8_t *__restrict__ up, const void *__restrict__ x, const int32_t *perm,
                     uint16_t *__restrict__ h, float2 *__restrict__ hsum2, float *__restrict__ hscale, float *red,
                     int tok0 = -1, int nrw = kWG) {
    if constexpr (FMT == BITMOE_FORMAT_MXFP4)
        mx_gateup_1<XBF16>(H, I, k, tk, P, gate, up, x, perm, h, hscale, red, tok0, nrw);
    else
        routed_gateup_1<XBF16, SGN>(H, I, k, tk, P, gate, up, x, perm, h, hsum2, hscale, red, tok0, nrw);
}
template <int FMT, int XBF16, int NT, int SGN>
BM_DEV void gateup_pass(int H, int I, int k, const Tok &tk, int t0, int P, const uint8_t *__restrict__ gate,
                        const uint8_t *__restrict__ up, const void *__restrict__ x, const int32_t *perm,
                        uint16_t *__restrict__ h, float2 *__restrict__ hsum2, float *__restrict__ hscale,
                        float *red) {
    if constexpr (FMT == BITMOE_FORMAT_MXFP4)
        mx_gateup_pass<XBF16, NT>(H, I, k, tk, t0, P, gate, up, x, perm, h, hscale, red);
    else
        routed_gateup_pass<XBF16, NT, SGN>(H, I, k, tk, t0, P, gate, up, x, perm, h, hsum2, hscale, red);
}

// sum of 8 products of bf16 weight pairs with h given as bf16 hi + lo
BM_DEV float dot8_hilo(uint4 wq, uint4 hh, uint4 hl, float acc) {
    acc = dot2_bf16(wq.x, hh.x, acc); acc = dot2_bf16(wq.x, hl.x, acc);
    acc = dot2_bf16(wq.y, hh.y, acc); acc = dot2_bf16(wq.y, hl.y, acc);
    acc = dot2_bf16(wq.z, hh.z, acc); acc = dot2_bf16(wq.z, hl.z, acc);
    acc = dot2_bf16(wq.w, hh.w, acc); acc = dot2_bf16(wq.w, hl.w, acc);
    return acc;
}

// One token's routing inside a gate/up workgroup (LDS): the experts by slot
// (slot = rank of the expert index), the picks of the general top-k.
constexpr int kMaxK = 16;
constexpr int kMaxWgItems = 32;     // (expert, panel) items of one gate/up workgroup, routing held in LDS
struct SmallRoute {
    int active[kMaxK], ids[kMaxK];
    int n_active, claim;
    int4 items[kMaxWgItems];        // batches: {expert (-1: none), first pair row, pairs, first token}
};

// Lane l of the wave: the logits of experts l, l+64, l+128, l+192 of token t
// (E <= 256; indices past E re-read the last one and are ignored).
BM_DEV void route_logits_load(const float *__restrict__ logits, int E, int t, float (&lv)[4]) {
    const int lane = lane_id();
#pragma unroll
    for (int i = 0; i < 4; i++) lv[i] = logits[(int64_t)t * E + min(lane + 64 * i, E - 1)];
}

// One token (k distinct experts, as a top-k gives), by wave 0: the top-k of
// the logits (mode 1) or the given ids (mode 2), the k experts ranked by
// index with k lane reads; slot = rank, each expert one pair, in LDS
// (r.active) and, by the workgroup that writes out, in bk.  The other waves
// read r after the next workgroup barrier.
BM_DEV void route_token_wave0(int mode, int E, int k, const float *__restrict__ logits, int32_t *ids, float *w,
                              const bm_host::Buckets &bk, SmallRoute &r, float (&lv)[4], bool lv_loaded, bool out) {
    const int lane = lane_id();
    int id;
    if (mode == 1) {
        if (E <= 256) {
            if (!lv_loaded) route_logits_load(logits, E, 0, lv);
            id = topk_wave4(lv, E, k, out ? ids : nullptr, out ? w : nullptr, nullptr);
        } else {
            topk_wave(logits, E, k, out ? ids : nullptr, out ? w : nullptr, r.ids);
            id = lane < k ? r.ids[lane] : 0;
        }
    } else {
        id = lane < k ? user_id(ids[lane], E) : 0;
    }
    // rank by (expert, position): a permutation of 0..k-1 even if a row
    // repeats an expert (which a top-k never does), so every slot is set
    int rank = 0;
    for (int i = 0; i < k; i++) {
        const int o = __builtin_amdgcn_readlane(id, i);
        rank += (o < id || (o == id && i < lane)) ? 1 : 0;
    }
    if (lane < k) {
        r.active[rank] = id;
        if (out) {
            bk.perm[rank] = lane;
            bk.active[rank] = id;
            bk.counts[id] = 1;
            bk.offsets[id] = rank;
        }
    }
    if (lane == 0) {
        r.n_active = k;
        if (out) *bk.n_active = k;
    }
}

// Shared-expert h of elements [f0, f1) by this workgroup: h = silu(sum of
// the gate partials) * (sum of the up partials), in a fixed order, as bf16
// hi + lo for the down launch.  The first element's partials may have been
// loaded already (fg, fu).
BM_DEV void shared_h_store(int64_t n, int kc_sg, const float *__restrict__ sgp, uint16_t *__restrict__ hs, int64_t i,
                           const float (&fg)[kMaxChunks], const float (&fu)[kMaxChunks]) {
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int c = 0; c < kMaxChunks; c++)
        if (c < kc_sg) { g += fg[c]; u += fu[c]; }
    (void)sgp;
    const float hv = silu(g) * u;
    const uint32_t hi = f32_to_bf16_rne(hv);
    hs[i] = (uint16_t)hi;
    hs[n + i] = (uint16_t)f32_to_bf16_rne(hv - bf16_to_f32(hi));
}
BM_DEV void shared_h_load(int64_t n, int kc_sg, const float *__restrict__ sgp, int64_t i, float (&fg)[kMaxChunks],
                          float (&fu)[kMaxChunks]) {
#pragma unroll
    for (int c = 0; c < kMaxChunks; c++) {
        const int cc = min(c, kc_sg - 1);
        fg[c] = sgp[(int64_t)(2 * cc) * n + i];
        fu[c] = sgp[(int64_t)(2 * cc + 1) * n + i];
    }
}

// The shared expert's gate/up for the one token of a single-token batch,
// inside the routed gate/up launch, on kSgWaves waves of each workgroup
// beside the routed ones: workgroup (slot s, panel P) takes rows r0 = s R ..
// r0 + R - 1 of panel P (R = 64/k: the k workgroups of a panel share its 64
// rows) over all of K, so that no sum crosses workgroups.  Lane l of
// shared wave sw takes row r0 + l % R and the pieces c = q + j Q, q = sw
// (64/R) + l / R, Q = kSgWaves (64/R), rounds j: one load of the wave
// covers 64/R pieces of R consecutive rows (R adjacent 16-byte pieces each
// in the tiled layout).  The routed waves decode (VALU-bound) while these
// stream (memory-bound), and none of it depends on the routing, so the
// first rounds run while the token is routed.  The rounds stream through a
// ring of kRing register slots, each refilled as soon as it is summed.
constexpr int kSgWaves = 4;
constexpr int kSgPreRounds = 8;      // rounds before the routing barrier
constexpr int kSredFloats = kSgWaves * 2 * 64;
BM_DEV float dot8x(uint4 w, uint4 xv, float acc) {
    acc = dot2_bf16(w.x, xv.x, acc);
    acc = dot2_bf16(w.y, xv.y, acc);
    acc = dot2_bf16(w.z, xv.z, acc);
    return dot2_bf16(w.w, xv.w, acc);
}
BM_DEV int shared_rows_rounds(int H, int R) { return (H / 8 + kSgWaves * (64 / R) - 1) / (kSgWaves * (64 / R)); }
template <int XBF16>
BM_DEV void shared_rows_range(int H, int R, int r0, int P, int sw, int j0, int j1, const uint4 *__restrict__ sg,
                              const uint4 *__restrict__ su, const void *__restrict__ x, float &ag, float &au) {
    constexpr int kRing = 8;
    if (j0 >= j1) return;
    const int lane = lane_id();
    const int K8 = H / 8, G = 64 / R, Q = kSgWaves * G, sh = __builtin_ctz(R);
    const int q = sw * G + (lane >> sh);
    const int64_t base = (int64_t)P * K8 * 64 + r0 + (lane & (R - 1));
    struct Slot { uint4 g, u, xv; };
    // rounds past j1 re-read the last one (cached) and are not summed;
    // pieces past K8 (a ragged last round) likewise
    auto load = [&](int j, Slot &sl) {
        const int c = min(q + min(j, j1 - 1) * Q, K8 - 1);
        sl.g = sg[base + (int64_t)c * 64];
        sl.u = su[base + (int64_t)c * 64];
        if (XBF16) sl.xv = reinterpret_cast<const uint4 *>(x)[c];
    };
    auto sum = [&](int j, const Slot &sl) {
        const int c = q + j * Q;
        float g, u;
        if (XBF16) {
            g = dot8x(sl.g, sl.xv, ag);
            u = dot8x(sl.u, sl.xv, au);
        } else {
            const void *xp = static_cast<const float *>(x) + 8 * min(c, K8 - 1);
            g = dot8<0>(make_uint2(sl.g.x, sl.g.y), make_uint2(sl.g.z, sl.g.w), xp, ag);
            u = dot8<0>(make_uint2(sl.u.x, sl.u.y), make_uint2(sl.u.z, sl.u.w), xp, au);
        }
        ag = c < K8 ? g : ag;
        au = c < K8 ? u : au;
    };
    Slot ring[kRing];
#pragma unroll
    for (int i = 0; i < kRing; i++) load(j0 + i, ring[i]);
    int j = j0;
    for (; j + kRing <= j1; j += kRing) {
#pragma unroll
        for (int i = 0; i < kRing; i++) {
            sum(j + i, ring[i]);
            __builtin_amdgcn_sched_barrier(0);
            load(j + i + kRing, ring[i]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int i = 0; i < kRing; i++)
        if (j + i < j1) sum(j + i, ring[i]);
}
// the lanes of a row meet by lane exchanges (xor over l / R), the shared
// waves in sred ([kSgWaves][2][64])
BM_DEV void shared_rows_reduce(int R, int sw, float ag, float au, float *sred) {
    const int lane = lane_id();
    for (int m = R; m < 64; m <<= 1) {
        ag += __shfl_xor(ag, m, 64);
        au += __shfl_xor(au, m, 64);
    }
    if (lane < R) {
        sred[(sw * 2 + 0) * 64 + lane] = ag;
        sred[(sw * 2 + 1) * 64 + lane] = au;
    }
}
// h of the R rows (after a workgroup barrier, by one wave): the shared
// waves' sums in wave order, h = silu(g) u as bf16 hi + lo for the down
// launch.
BM_DEV void shared_rows_finish(int I, int R, int r0, int P, const float *sred, uint16_t *__restrict__ hs) {
    const int lane = lane_id();
    if (lane >= R) return;
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int v = 0; v < kSgWaves; v++) {
        g += sred[(v * 2 + 0) * 64 + lane];
        u += sred[(v * 2 + 1) * 64 + lane];
    }
    const float hv = silu(g) * u;
    const int n = P * 64 + r0 + lane;
    const uint32_t hi = f32_to_bf16_rne(hv);
    hs[n] = (uint16_t)hi;
    hs[I + n] = (uint16_t)f32_to_bf16_rne(hv - bf16_to_f32(hi));
}

// MULTI = 0 takes the experts chosen by exactly one token, MULTI = 1 the
// experts with several tokens (passes of kNT tokens); keeping the two apart
// keeps each kernel's register use low.  MULTI = 2 takes both in one launch
// (batches of 2 to 8 tokens, whose few experts with several tokens would
// otherwise leave most of the GPU idle in a launch of their own).  route_mode: 0 the bucketing is in
// bk already; one token (MULTI = 0 only): route_one_token from the logits
// (1) or the given ids (2).  The run lookup tables
// (dynamic LDS, dec_lut_bytes) are built from the codebook while the batch
// is routed.
template <int MULTI>
constexpr int dec_sgn_bytes() { return MULTI ? kLutSgnHalf : kLutSgnFull; }
template <int FMT, int MULTI>
constexpr int dec_lut_bytes() { return FMT == BITMOE_FORMAT_MXFP4 ? 0 : kLutMagBytes + dec_sgn_bytes<MULTI>(); }
// all LDS of a gate/up workgroup, dynamic so that the tables start at
// address 0 (their lookup offsets are then the permutes' results as they
// are): tables | cross-wave sums | routing | (MULTI = 0) shared-row sums
template <int MULTI>
constexpr int dec_red_floats() { return kWG * (MULTI ? kNT : 1) * 2 * 64; }
template <int FMT, int MULTI>
constexpr int dec_gateup_lds() {
    return dec_lut_bytes<FMT, MULTI>() + dec_red_floats<MULTI>() * 4 + (int)sizeof(SmallRoute) +
           (MULTI ? 0 : kSredFloats * 4);
}

template <int FMT, int XBF16, int MULTI>
__global__ void __launch_bounds__(kWG * 64)
k_dec_gateup(int H, int I, int E, int k, int T, int n_gwg, int route_mode, const uint8_t *__restrict__ gate,
             const uint8_t *__restrict__ up, const uint8_t *__restrict__ grid,
             const void *__restrict__ x, const float *__restrict__ logits,
             int32_t *ids, float *w, bm_host::Buckets bk, uint16_t *__restrict__ h, float2 *__restrict__ hsum2,
             float *__restrict__ hscale, int kc_sg, const float *__restrict__ sgp, uint16_t *__restrict__ hs,
             int sg_rows, const uint4 *__restrict__ sg, const uint4 *__restrict__ su,
             const int4 *__restrict__ single, const int32_t *__restrict__ n_single, int32_t *__restrict__ gctr) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lut[];
    float *red = reinterpret_cast<float *>(lut + dec_lut_bytes<FMT, MULTI>());
    SmallRoute &sr = *reinterpret_cast<SmallRoute *>(red + dec_red_floats<MULTI>());
    float *sred = reinterpret_cast<float *>(&sr + 1);
    constexpr int SGN = dec_sgn_bytes<MULTI>();
    const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = blockIdx.x, panels = I / 64, slot = b / panels, P = b % panels;
    const int32_t *counts = bk.counts, *offsets = bk.offsets, *perm = bk.perm, *active = bk.active;
    // shared-expert h, spread over all workgroups of the MULTI = 0 launch
    const int64_t nfin = (MULTI != 1 && kc_sg) ? (int64_t)T * I : 0;
    const int64_t fchunk = (nfin + gridDim.x - 1) / gridDim.x, f0 = b * fchunk, f1 = min(nfin, f0 + fchunk);
    float fg[kMaxChunks], fu[kMaxChunks];
    if (!MULTI && route_mode) {
        // one token, routed in every workgroup, one (slot, panel) item each.
        // Loads that do not depend on each other go out first: the codebook
        // rows, the logits, this workgroup's shared-h partials (on wave 1:
        // wave 0 routes); the tables are written while they arrive.
        constexpr bool kTab = FMT != BITMOE_FORMAT_MXFP4;
        uint2 grow = make_uint2(0u, 0u);
        if (kTab && tid < 256) grow = *reinterpret_cast<const uint2 *>(grid + 8 * tid);
        float lv[4];
        const bool pre = route_mode == 1 && E <= 256 && wv == 0;
        if (pre) route_logits_load(logits, E, 0, lv);
        const int64_t fi = f0 + tid - 64;
        if (tid >= 64 && fi < f1) shared_h_load(nfin, kc_sg, sgp, fi, fg, fu);
        if constexpr (kTab) {
            if (tid < 256) lut_write_line(lut, 0, tid, lut_mag_from_row<1>(grow));
            else if (tid < 256 + SGN / 256) lut_write_line(lut, kLutMagBytes, tid - 256, lut_sign_entry(tid - 256));
        }
        if (tid >= 64 && fi < f1) shared_h_store(nfin, kc_sg, sgp, hs, fi, fg, fu);
        for (int64_t i = fi + blockDim.x - 64; tid >= 64 && i < f1; i += blockDim.x - 64) {
            shared_h_load(nfin, kc_sg, sgp, i, fg, fu);
            shared_h_store(nfin, kc_sg, sgp, hs, i, fg, fu);
        }
        if (wv == 0) route_token_wave0(route_mode, E, k, logits, ids, w, bk, sr, lv, pre, b == 0);
        // sg_rows: the last kSgWaves waves take this workgroup's shared rows
        // (the grid holds the k slots' workgroups, so slot < k), their
        // first rounds while wave 0 routes
        const int nrw = sg_rows ? kWG - kSgWaves : kWG, sw = wv - nrw;
        float sa = 0.f, sb = 0.f;
        const int sj = sg_rows ? shared_rows_rounds(H, sg_rows) : 0;
        if (sw >= 0)
            shared_rows_range<XBF16>(H, sg_rows, slot * sg_rows, P, sw, 0, min(sj, kSgPreRounds), sg, su, x, sa, sb);
        __syncthreads();
        // slot = rank: one pair each, pair row = slot, token 0
        if (slot >= k) return;
        if (sw >= 0) {
            shared_rows_range<XBF16>(H, sg_rows, slot * sg_rows, P, sw, kSgPreRounds, sj, sg, su, x, sa, sb);
            shared_rows_reduce(sg_rows, sw, sa, sb, sred);
        }
        Tok tk;
        tk.e = sr.active[slot];
        tk.off = slot;
        tk.cnt = 1;
        // (the shared waves take no routed pieces; the pass's barriers make
        // sred whole before it returns)
        gateup_1<FMT, XBF16, SGN>(H, I, k, tk, P, gate, up, x, nullptr, h, hsum2, hscale, red, -1, nrw);
        if (sw == 0) shared_rows_finish(I, sg_rows, slot * sg_rows, P, sred, hs);
        return;
    }
    int na = 0;
    if constexpr (MULTI != 1) {
        for (int64_t i = f0 + tid; i < f1; i += blockDim.x) {
            shared_h_load(nfin, kc_sg, sgp, i, fg, fu);
            shared_h_store(nfin, kc_sg, sgp, hs, i, fg, fu);
        }
    }
    if (!MULTI && gctr) {
        // a batch whose experts with several tokens run at the same time on
        // the prefill kernels (another stream): the single-token experts'
        // (expert, panel) items are claimed one at a time from a counter the
        // front launch cleared, each next claim in flight while an item is
        // decoded, so that workgroups that start late take fewer items
        if constexpr (FMT != BITMOE_FORMAT_MXFP4) lut_build<1, SGN>(grid, lut);
        if (tid == 0) sr.claim = __hip_atomic_fetch_add(gctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int n_items = *n_single * panels;
        __syncthreads();
        int it = sr.claim;
        while (it < n_items) {
            const int4 in = single[it / panels];
            int nxt = 0;
            if (tid == 0) nxt = __hip_atomic_fetch_add(gctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            Tok tk;
            tk.e = in.x;
            tk.off = in.y;
            tk.cnt = 1;
            gateup_1<FMT, XBF16, SGN>(H, I, k, tk, it % panels, gate, up, x, nullptr, h, hsum2, hscale, red, in.w);
            if (tid == 0) sr.claim = nxt;      // every thread read the last claim before the item's barriers
            __syncthreads();
            it = sr.claim;
        }
        return;
    }
    // one (expert, panel) item: an expert chosen by one token through the
    // one-token ring, one with several in passes of up to kNT tokens
    auto run_item = [&](const Tok &tk, int Pi, int tok0) {
        if (MULTI != 1 && tk.cnt == 1) {
            gateup_1<FMT, XBF16, SGN>(H, I, k, tk, Pi, gate, up, x, perm, h, hsum2, hscale, red, tok0);
            return;
        }
        if constexpr (MULTI != 0) {
            for (int t0 = 0; t0 < tk.cnt; t0 += kNT) {
                const int n = tk.cnt - t0;
                if (n == 1)
                    gateup_pass<FMT, XBF16, 1, SGN>(H, I, k, tk, t0, Pi, gate, up, x, perm, h, hsum2, hscale, red);
                else if (n == 2)
                    gateup_pass<FMT, XBF16, 2, SGN>(H, I, k, tk, t0, Pi, gate, up, x, perm, h, hsum2, hscale, red);
                else
                    gateup_pass<FMT, XBF16, kNT, SGN>(H, I, k, tk, t0, Pi, gate, up, x, perm, h, hsum2, hscale,
                                                        red);
            }
        }
    };
    // routing done by an earlier launch.  The routing of this workgroup's
    // items (it = b + j G) is loaded at once, one thread per item, instead of
    // one chain of dependent loads per item (the active slot, its expert's
    // row and count, its first token); indices past the active slots are
    // clamped into range and their items marked empty.
    const int G = gridDim.x, n_it = b < n_gwg ? (n_gwg - b + G - 1) / G : 0;
    if (n_it <= kMaxWgItems) {
        if (tid < n_it) {
            const int si = (b + tid * G) / panels, nact = *bk.n_active;
            const int e = min(max(active[si], 0), E - 1);
            const int off = offsets[e], cnt = counts[e];
            const int tok = perm[min(max(off, 0), T * k - 1)] / k;
            sr.items[tid] = si < nact ? make_int4(e, off, cnt, tok) : make_int4(-1, 0, 0, 0);
        }
        if constexpr (FMT != BITMOE_FORMAT_MXFP4) lut_build<1, SGN>(grid, lut);
        __syncthreads();
        for (int j = 0; j < n_it; j++) {
            const int4 in = sr.items[j];
            if (in.x < 0) break;
            Tok tk;
            tk.e = in.x;
            tk.off = in.y;
            tk.cnt = in.z;
            if (MULTI != 2 && (tk.cnt > 1) != (MULTI != 0)) continue;
            run_item(tk, (b + j * G) % panels, in.w);
        }
        return;
    }
    na = *bk.n_active;
    // (more items than the table holds) the workgroups loop over the
    // (slot, panel) items, the tables built once by each
    bool built = false;
    for (int it = b; it < n_gwg; it += gridDim.x) {
        const int si = it / panels, Pi = it - si * panels;
        if (si >= na) break;
        Tok tk;
        tk.e = active[si];
        tk.off = offsets[tk.e];
        tk.cnt = counts[tk.e];
        if (MULTI != 2 && (tk.cnt > 1) != (MULTI != 0)) continue;
        if (!built) {
            if constexpr (FMT != BITMOE_FORMAT_MXFP4) lut_build<1, SGN>(grid, lut);
            __syncthreads();
            built = true;
        }
        run_item(tk, Pi, -1);
    }
}

// ---------------------------------------------------------------------------
// down: routed Q2K down per (slot, panel) || shared down split over K.
// grid = slots*(H/64) + (H/64)*kc_sd.  o[pair][H] unweighted.
// ---------------------------------------------------------------------------
// Routed Q2K down of panel P for the pair rows of tokens t0..t0+NT-1 of
// expert tk.  h arrives as fp16 scaled per 64 columns (hscale), with per-16
// sums hs (hsum2 = {hs, 0}); each sub-block is 8 fp16 dot products of exact
// quant pairs (the hardware E2M1 conversion of the masked word), then
// d sc S - dmin m hs.
template <int NT>
BM_DEV void routed_down_pass(int H, int I, const Tok &tk, int t0, int P,
                             const uint8_t *__restrict__ down, const int32_t *__restrict__ perm,
                             const uint16_t *__restrict__ h, const float2 *__restrict__ hsum2,
                             const float *__restrict__ hscale, float *__restrict__ o, float *red,
                             uint4 *hst) {
    const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int rows[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) rows[t] = tk.off + min(t0 + t, tk.cnt - 1);
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = 0.f;
    const int nb = I / kQK;
    const int64_t S = (int64_t)H * nb;
    const uint8_t *D = down + tk.e * S * 84;
    const uint4 *dq = reinterpret_cast<const uint4 *>(D);
    const uint4 *ds = reinterpret_cast<const uint4 *>(D + S * 64);
    const uint32_t *dd = reinterpret_cast<const uint32_t *>(D + S * 80);
    int kb0, kb1;
    split_range(nb, kWD, wv, kb0, kb1);
    // superblocks two at a time, both loaded before either is decoded (the
    // second of an odd tail is the first again, decoded and dropped: a
    // branch around it would let the compiler sink its loads to the use)
    struct Sb { uint4 q[4], sc; uint32_t dm; };
    auto load = [&](int kb, Sb &v) {
        const int64_t pk = (int64_t)P * nb + kb;
#pragma unroll
        for (int c = 0; c < 4; c++) v.q[c] = dq[(pk * 4 + c) * 64 + lane];
        v.sc = ds[pk * 64 + lane];
        v.dm = dd[pk * 64 + lane];
    };
    // The h the two superblocks need (per token: 512 fp16, their 32 sums
    // {hs, hb}, their 8 scales) is staged in this wave's slice of LDS by
    // three vector loads per token, issued before the weights: as scalar
    // loads, the first touch of each line came back one round trip at a time.
    auto stage = [&](int kb, int kb2) {
        uint4 hv[NT], sv[NT], cv[NT];
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const int sb = lane < 32 ? kb : kb2;
            hv[t] = *reinterpret_cast<const uint4 *>(h + (int64_t)rows[t] * I + sb * kQK + 8 * (lane & 31));
            const int sb2 = (lane & 15) < 8 ? kb : kb2;
            sv[t] = *reinterpret_cast<const uint4 *>(hsum2 + (int64_t)rows[t] * (I / 16) + sb2 * 16 + 2 * (lane & 7));
            const int sb3 = (lane & 1) ? kb2 : kb;
            cv[t] = *reinterpret_cast<const uint4 *>(hscale + (int64_t)rows[t] * (I / 64) + sb3 * 4);
        }
        return [=](void) {
#pragma unroll
            for (int t = 0; t < NT; t++) {
                hst[t * kHst + lane] = hv[t];
                if (lane < 16) hst[t * kHst + 64 + lane] = sv[t];
                if (lane < 2) hst[t * kHst + 80 + lane] = cv[t];
            }
        };
    };
    // superblock s (0, 1) of the staged pair
    auto decode = [&](int s, const Sb &v, bool keep) {
        const float d = fp16_to_f32(v.dm & 0xFFFFu), dmin = fp16_to_f32(v.dm >> 16);
#pragma unroll
        for (int c = 0; c < 4; c++) {                 // 64 columns: sub-blocks 4c..4c+3
            const uint32_t qw[4] = {v.q[c].x, v.q[c].y, v.q[c].z, v.q[c].w};
            const uint32_t scw = c == 0 ? v.sc.x : c == 1 ? v.sc.y : c == 2 ? v.sc.z : v.sc.w;
            const uint32_t scl = scw & 0x0F0F0F0Fu, mnb = (scw >> 4) & 0x0F0F0F0Fu;
            float a1[NT], a2[NT];
#pragma unroll
            for (int t = 0; t < NT; t++) a1[t] = a2[t] = 0.f;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t lo = q2k_lo(qw[i]), hi = q2k_hi(qw[i]);
                const uint32_t pr[8] = {q2k_pair_f16<0>(lo), q2k_pair_f16<1>(lo), q2k_pair_f16<2>(lo),
                                        q2k_pair_f16<3>(lo), q2k_pair_f16<0>(hi), q2k_pair_f16<1>(hi),
                                        q2k_pair_f16<2>(hi), q2k_pair_f16<3>(hi)};
                const float scf = (float)((scl >> (8 * i)) & 0xFFu), mf = (float)((mnb >> (8 * i)) & 0xFFu);
#pragma unroll
                for (int t = 0; t < NT; t++) {
                    const uint4 *hp = hst + t * kHst + s * 32 + 8 * c + 2 * i;
                    const uint4 x0 = hp[0], x1 = hp[1];
                    float sacc = dot2_f16(pr[0], x0.x, 0.f);
                    sacc = dot2_f16(pr[1], x0.y, sacc);
                    sacc = dot2_f16(pr[2], x0.z, sacc);
                    sacc = dot2_f16(pr[3], x0.w, sacc);
                    sacc = dot2_f16(pr[4], x1.x, sacc);
                    sacc = dot2_f16(pr[5], x1.y, sacc);
                    sacc = dot2_f16(pr[6], x1.z, sacc);
                    sacc = dot2_f16(pr[7], x1.w, sacc);
                    const float2 sb = reinterpret_cast<const float2 *>(hst + t * kHst + 64)[s * 16 + 4 * c + i];   // {hs, 0}
                    a1[t] = fmaf(scf, sacc, a1[t]);
                    a2[t] = fmaf(mf, sb.x, a2[t]);
                }
            }
#pragma unroll
            for (int t = 0; t < NT; t++) {
                const float hsc = reinterpret_cast<const float *>(hst + t * kHst + 80)[s * 4 + c];
                const float v2 = fmaf(hsc, fmaf(d, a1[t], -dmin * a2[t]), acc[t]);
                acc[t] = keep ? v2 : acc[t];
            }
        }
    };
    for (int kb = kb0; kb < kb1; kb += 2) {
        const int kb2 = kb + 1 < kb1 ? kb + 1 : kb;
        auto put = stage(kb, kb2);
        Sb va, vb;
        load(kb, va);
        load(kb2, vb);
        __builtin_amdgcn_sched_barrier(0);
        put();
        decode(0, va, true);
        decode(1, vb, kb + 1 < kb1);
    }
#pragma unroll
    for (int t = 0; t < NT; t++) red[(wv * NT + t) * 64 + lane] = acc[t];
    __syncthreads();
    if (wv < NT && t0 + wv < tk.cnt) {
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < kWD; v++) s += red[(v * NT + wv) * 64 + lane];
        st_dev(&o[(int64_t)perm[tk.off + t0 + wv] * H + P * 64 + lane], s);
    }
    __syncthreads();
}

// Routed MXFP4 down of panel P for the pair rows of tokens t0..t0+NT-1 of
// expert tk.  h arrives as fp16 scaled per 64 columns (hscale); each piece
// (32 columns of h) is 16 fp16 dot products, times its block scale and the
// h scale.  The wave's share of h (16 pieces at a time, with their scales)
// is staged in its slice of LDS by one vector load per token.
template <int NT>
BM_DEV void mx_down_pass(int H, int I, const Tok &tk, int t0, int P, const uint8_t *__restrict__ down,
                         const int32_t *__restrict__ perm, const uint16_t *__restrict__ h,
                         const float *__restrict__ hscale, float *__restrict__ o, float *red, uint4 *hst) {
    constexpr int kChunk = 16;                       // pieces per staging (64 uint4 of h per token)
    static_assert(4 * kChunk + 4 <= kHst, "staging slice");
    const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int rows[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) rows[t] = tk.off + min(t0 + t, tk.cnt - 1);
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = 0.f;
    const int64_t slab = (int64_t)H * I / 32 * 17;
    const MxRows D = mx_rows(down + tk.e * slab, H, I, P);
    const int nsc = I / 64;
    int p0, p1;
    split_range(8 * (I / kQK), kWD, wv, p0, p1);
    struct B4 { uint4 q[4]; uint32_t s[4]; };
    auto load = [&](int pb, B4 &b) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int pc = min(pb + i, p1 - 1);
            b.q[i] = D.piece(pc);
            b.s[i] = D.scale(pc);
        }
    };
    for (int c0 = p0; c0 < p1; c0 += kChunk) {
        const int c1 = min(c0 + kChunk, p1), g0 = c0 >> 1;
        uint4 hv[NT];
        float sv[NT];
#pragma unroll
        for (int t = 0; t < NT; t++) {
            hv[t] = make_uint4(0u, 0u, 0u, 0u);
            if (lane < 4 * (c1 - c0))
                hv[t] = *reinterpret_cast<const uint4 *>(h + (int64_t)rows[t] * I + 32 * c0 + 8 * lane);
            sv[t] = hscale[(int64_t)rows[t] * nsc + min(g0 + (lane & 15), nsc - 1)];
        }
        B4 cur{}, nxt{};
        load(c0, cur);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < NT; t++) {
            hst[t * kHst + lane] = hv[t];
            if (lane < 16) reinterpret_cast<float *>(hst + t * kHst + 4 * kChunk)[lane] = sv[t];
        }
        for (int pb = c0; pb < c1; pb += 4) {
            if (pb + 4 < c1) load(pb + 4, nxt);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int pc = pb + i;
                if (pc < c1) {
                    const uint32_t qw[4] = {cur.q[i].x, cur.q[i].y, cur.q[i].z, cur.q[i].w};
                    const float bs = mx_scale(cur.s[i]);
#pragma unroll
                    for (int t = 0; t < NT; t++) {
                        float part = 0.f;
#pragma unroll
                        for (int r = 0; r < 4; r++) {
                            const uint4 hp = hst[t * kHst + 4 * (pc - c0) + r];
                            part = dot2_f16(fp4x2_f16<0>(qw[r]), hp.x, part);
                            part = dot2_f16(fp4x2_f16<1>(qw[r]), hp.y, part);
                            part = dot2_f16(fp4x2_f16<2>(qw[r]), hp.z, part);
                            part = dot2_f16(fp4x2_f16<3>(qw[r]), hp.w, part);
                        }
                        const float hsc = reinterpret_cast<const float *>(hst + t * kHst + 4 * kChunk)[(pc >> 1) - g0];
                        acc[t] = fmaf(bs, part * hsc, acc[t]);
                    }
                }
            }
            cur = nxt;
        }
    }
#pragma unroll
    for (int t = 0; t < NT; t++) red[(wv * NT + t) * 64 + lane] = acc[t];
    __syncthreads();
    if (wv < NT && t0 + wv < tk.cnt) {
        float sum = 0.f;
#pragma unroll
        for (int v = 0; v < kWD; v++) sum += red[(v * NT + wv) * 64 + lane];
        st_dev(&o[(int64_t)perm[tk.off + t0 + wv] * H + P * 64 + lane], sum);
    }
    __syncthreads();
}

template <int FMT, int NT>
BM_DEV void down_pass(int H, int I, const Tok &tk, int t0, int P, const uint8_t *__restrict__ down,
                      const int32_t *__restrict__ perm, const uint16_t *__restrict__ h,
                      const float2 *__restrict__ hsum2, const float *__restrict__ hscale, float *__restrict__ o,
                      float *red, uint4 *hst) {
    if constexpr (FMT == BITMOE_FORMAT_MXFP4)
        mx_down_pass<NT>(H, I, tk, t0, P, down, perm, h, hscale, o, red, hst);
    else
        routed_down_pass<NT>(H, I, tk, t0, P, down, perm, h, hsum2, hscale, o, red, hst);
}

// Shared down of panel P over the K pieces [c0, c1); h as bf16 hi + lo
// (hs[2][T][I]) through scalar loads.
template <int NT>
BM_DEV void shared_down_pass(int H, int I, int T, int t0, int P, int c0, int c1,
                             const uint4 *__restrict__ sd, const uint16_t *__restrict__ hs,
                             float *__restrict__ osp, float *red, uint4 *hst) {
    const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int K8 = I / 8;
    const int64_t lo_off = (int64_t)T * I;
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = 0.f;
    int w0, w1;
    split_range(c1 - c0, kWD, wv, w0, w1);
    // batches of B pieces loaded at once (past the wave's range: its last
    // piece again, used and dropped, so that the loads stay together)
    constexpr int B = 8;
    const uint4 *base = sd + (int64_t)P * K8 * 64 + lane;
    static_assert(NT * 2 * B <= kHst, "staging slice");
    for (int cb = c0 + w0; cb < c0 + w1; cb += B) {
        // the batch's h (hi pieces in lanes 0-7, lo pieces in lanes 8-15, per
        // token) is staged in this wave's LDS slice by one vector load per
        // token, issued before the weights
        uint4 hv[NT];
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const int c = min(cb + (lane & 7), c0 + w1 - 1);
            hv[t] = *reinterpret_cast<const uint4 *>(hs + ((lane & 8) ? lo_off : 0) +
                                                     (int64_t)min(t0 + t, T - 1) * I + 8 * c);
        }
        uint4 cur[B];
#pragma unroll
        for (int i = 0; i < B; i++) cur[i] = base[(int64_t)min(cb + i, c0 + w1 - 1) * 64];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < NT; t++)
            if (lane < 2 * B) hst[t * 2 * B + lane] = hv[t];
#pragma unroll
        for (int i = 0; i < B; i++) {
            const bool keep = cb + i < c0 + w1;
#pragma unroll
            for (int t = 0; t < NT; t++) {
                const float v = dot8_hilo(cur[i], hst[t * 2 * B + i], hst[t * 2 * B + B + i], acc[t]);
                acc[t] = keep ? v : acc[t];
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; t++) red[(wv * NT + t) * 64 + lane] = acc[t];
    __syncthreads();
    if (wv < NT && t0 + wv < T) {
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < kWD; v++) s += red[(v * NT + wv) * 64 + lane];
        st_dev(&osp[(int64_t)(t0 + wv) * H + P * 64 + lane], s);
    }
    __syncthreads();
}

// y for the 64 outputs of panel P: sum over the k slots of w * o, plus the
// shared partials, in a fixed order (device-scope loads of this launch's
// results).
BM_DEV void combine_panel(int H, int k, int T, int kc_sd, int P, const float *o, const float *w,
                          const float *osp, float *y) {
    const int wv = threadIdx.x >> 6, n = P * 64 + lane_id();
    for (int t = wv; t < T; t += kWD) {
        // every load issued before the first is used (k <= 16, kc_sd <= 4)
        float ov[16], sv[kMaxChunks];
#pragma unroll
        for (int j = 0; j < 16; j++) ov[j] = ld_dev(&o[((uint32_t)t * k + min(j, k - 1)) * (uint32_t)H + n]);
#pragma unroll
        for (int c = 0; c < kMaxChunks; c++)
            sv[c] = kc_sd ? ld_dev(&osp[((uint32_t)min(c, kc_sd - 1) * T + t) * (uint32_t)H + n]) : 0.f;
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 16; j++)
            if (j < k) s = fmaf(w[t * k + j], ov[j], s);
#pragma unroll
        for (int c = 0; c < kMaxChunks; c++)
            if (c < kc_sd) s += sv[c];
        y[(int64_t)t * H + n] = s;
    }
}

// After a workgroup's outputs for panel P are stored (device scope): count
// it in the panel's counter (cleared by the front launch); the workgroup
// that brings the count to all contributors (the active experts and the
// shared chunks) combines the panel.
BM_DEV void count_and_combine(int H, int k, int T, int kc_sd, int P, int n_contrib, int32_t *ycount,
                              const float *o, const float *w, const float *osp, float *y, int *sdo) {
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0)
        *sdo = __hip_atomic_fetch_add(&ycount[P], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_contrib - 1;
    __syncthreads();
    if (*sdo) combine_panel(H, k, T, kc_sd, P, o, w, osp, y);
}

// Shared down of a decode batch on the matrix cores (batches that run the
// prefill kernels): panel P of the H output rows, K chunk c of the I columns
// (kc chunks), 16 tokens per pass over the bf16 weights, with the operand
// scheme of shared_gateup_mfma.  h arrives as bf16 hi + lo; the two parts
// are two instructions into the same accumulators.  Four waves split the
// chunk's pieces and meet in LDS; outputs go to osp[c][T][H] as in the
// other shared down.
constexpr int kSdmW = 4;
constexpr int kSdmPieces = 64;              // K pieces of a chunk the staging holds
constexpr int kSdmXsBytes = 2 * 16 * (kSdmPieces * 16 + 16) + 16;
__global__ void __launch_bounds__(kSdmW * 64)
k_shared_down_mfma(int H, int I, int T, int kc, const uint4 *__restrict__ sd, const uint16_t *__restrict__ hs,
                   float *__restrict__ osp) {
    __shared__ float red[kSdmW * 4 * 64];
    __shared__ __attribute__((aligned(16))) uint8_t xs[kSdmXsBytes];
    const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int P = blockIdx.x / kc, c = blockIdx.x % kc, K8 = I / 8;
    int c0, c1;
    split_range(K8, kc, c, c0, c1);
    const int nc = c1 - c0, stride = nc * 16 + 16, half = 16 * stride, zero = 2 * half;
    const int j = lane >> 4, m = lane & 15;
    const bool act = (m >> 2) == j;
    const int64_t lo_off = (int64_t)T * I;
    const uint4 *wbase = sd + (int64_t)P * K8 * 64 + lane;
    int w0, w1;
    split_range(nc, kSdmW, wv, w0, w1);
    for (int t0 = 0; t0 < T; t0 += 16) {
        const int nt = min(16, T - t0);
        __syncthreads();                 // the previous pass's readers of xs and red are done
        for (int i = threadIdx.x; i < 2 * 16 * nc; i += blockDim.x) {
            const int part = i / (16 * nc), r = i - part * 16 * nc, tt = r / nc, cl = r - tt * nc;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (tt < nt)
                v = *reinterpret_cast<const uint4 *>(hs + (part ? lo_off : 0) + (int64_t)(t0 + tt) * I + 8 * (c0 + cl));
            *reinterpret_cast<uint4 *>(xs + part * half + tt * stride + cl * 16) = v;
        }
        if (threadIdx.x == 0) *reinterpret_cast<uint4 *>(xs + zero) = make_uint4(0u, 0u, 0u, 0u);
        __syncthreads();
        f32x4_t acc[4];
#pragma unroll
        for (int g = 0; g < 4; g++) acc[g] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        constexpr int kB = 4;
        for (int cb = w0; cb < w1; cb += kB) {
            uint4 wq[kB];
#pragma unroll
            for (int i = 0; i < kB; i++) wq[i] = wbase[(int64_t)(c0 + min(cb + i, w1 - 1)) * 64];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < kB; i++) {
                const int cl = min(cb + i, w1 - 1);
                const bool use = act && cb + i < w1;
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    const int a = use ? (4 * g + (m & 3)) * stride + cl * 16 : zero;
                    const uint4 ah = *reinterpret_cast<const uint4 *>(xs + (use ? a : zero));
                    const uint4 al = *reinterpret_cast<const uint4 *>(xs + (use ? half + a : zero));
                    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ah),
                                                                     __builtin_bit_cast(bf16x8_t, wq[i]), acc[g], 0, 0, 0);
                    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, al),
                                                                     __builtin_bit_cast(bf16x8_t, wq[i]), acc[g], 0, 0, 0);
                }
            }
        }
        // lane l, result i of group g: panel row l, token 4 g + i
#pragma unroll
        for (int g = 0; g < 4; g++) {
#pragma unroll
            for (int i = 0; i < 4; i++) red[(wv * 4 + i) * 64 + lane] = acc[g][i];
            __syncthreads();
            if (wv < 4 && 4 * g + wv < nt) {
                float sum = 0.f;
#pragma unroll
                for (int v = 0; v < kSdmW; v++) sum += red[(v * 4 + wv) * 64 + lane];
                osp[((int64_t)c * T + t0 + 4 * g + wv) * H + P * 64 + lane] = sum;
            }
            __syncthreads();
        }
    }
}

// The panel combine as a launch of its own, one thread per output, in the
// same fixed order (batches whose down launch runs beside the prefill
// kernels' down: the combine waits for both).
__global__ void __launch_bounds__(256)
k_dec_combine(int H, int k, int T, int kc_sd, const float *__restrict__ o, const float *__restrict__ w,
              const float *__restrict__ osp, float *__restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * H) return;
    const int t = (int)(i / H), n = (int)(i - (int64_t)t * H);
    float ov[16], sv[kMaxChunks];
#pragma unroll
    for (int j = 0; j < 16; j++) ov[j] = o[((int64_t)t * k + min(j, k - 1)) * H + n];
#pragma unroll
    for (int c = 0; c < kMaxChunks; c++) sv[c] = kc_sd ? osp[((int64_t)min(c, kc_sd - 1) * T + t) * H + n] : 0.f;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 16; j++)
        if (j < k) s = fmaf(w[t * k + j], ov[j], s);
#pragma unroll
    for (int c = 0; c < kMaxChunks; c++)
        if (c < kc_sd) s += sv[c];
    y[i] = s;
}

// MULTI = 0: experts chosen by one token, and the shared down; MULTI = 1:
// experts chosen by several tokens (launched only when T > 1); MULTI = 2:
// all of them and the shared down, in one launch (batches of 2 to 8 tokens).
// combine = 0: the outputs are only stored (k_dec_combine sums them).
template <int FMT, int MULTI>
__global__ void __launch_bounds__(kWD * 64) __attribute__((amdgpu_waves_per_eu(MULTI ? 1 : bm_cfg::kDownWavesPerSimd)))
k_dec_down(int H, int I, int k, int T, int n_dwg, int kc_sd, const int32_t *__restrict__ n_multi, int combine,
           const uint8_t *__restrict__ down,
           const uint4 *__restrict__ sd, const int32_t *__restrict__ counts,
           const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm,
           const int32_t *__restrict__ active, const int32_t *__restrict__ n_active,
           const uint16_t *__restrict__ h, const float2 *__restrict__ hsum2, const float *__restrict__ hscale,
           const uint16_t *__restrict__ hs, const float *__restrict__ w, int32_t *__restrict__ ycount,
           float *__restrict__ osp, float *__restrict__ o, float *__restrict__ y) {
    __shared__ float red[kWD * kNT * 64];
    __shared__ uint4 hstage[kWD][MULTI ? kNT : 1][kHst];
    __shared__ int sdo;
    uint4 *hst = &hstage[threadIdx.x >> 6][0][0];
    const int panels = H / 64;
    const int na = *n_active;
    // n_multi (batches): the experts chosen by several tokens wrote their
    // outputs in an earlier launch (as many as there are row tiles) and are
    // not counted, unless no other contributor would combine the panel
    const int nm = n_multi ? *n_multi : 0;
    const bool count_multi = na - nm + kc_sd == 0;
    const int n_contrib = count_multi ? na + kc_sd : na - nm + kc_sd;
    if ((int)blockIdx.x < n_dwg) {
        const int slot = blockIdx.x / panels, P = blockIdx.x % panels;
        if (slot >= na) return;
        Tok tk;
        tk.e = active[slot];
        tk.off = offsets[tk.e];
        tk.cnt = counts[tk.e];
        if (!MULTI && tk.cnt > 1 && n_multi) {
            if (combine && count_multi) count_and_combine(H, k, T, kc_sd, P, n_contrib, ycount, o, w, osp, y, &sdo);
            return;
        }
        if (MULTI != 2 && (tk.cnt > 1) != (MULTI != 0)) return;
        if (MULTI == 0 || tk.cnt == 1) {
            down_pass<FMT, 1>(H, I, tk, 0, P, down, perm, h, hsum2, hscale, o, red, hst);
        } else if constexpr (MULTI != 0) {
            for (int t0 = 0; t0 < tk.cnt; t0 += kNT) {
                const int n = tk.cnt - t0;
                if (n == 1)
                    down_pass<FMT, 1>(H, I, tk, t0, P, down, perm, h, hsum2, hscale, o, red, hst);
                else if (n == 2)
                    down_pass<FMT, 2>(H, I, tk, t0, P, down, perm, h, hsum2, hscale, o, red, hst);
                else
                    down_pass<FMT, kNT>(H, I, tk, t0, P, down, perm, h, hsum2, hscale, o, red, hst);
            }
        }
        if (combine) count_and_combine(H, k, T, kc_sd, P, n_contrib, ycount, o, w, osp, y, &sdo);
    } else if (MULTI != 1) {
        const int bs = blockIdx.x - n_dwg, c = bs % kc_sd, P = bs / kc_sd;
        int c0, c1;
        split_range(I / 8, kc_sd, c, c0, c1);
        float *op = osp + (int64_t)c * T * H;
        for (int t0 = 0; t0 < T; t0 += kNT) {
            if (T - t0 == 1)
                shared_down_pass<1>(H, I, T, t0, P, c0, c1, sd, hs, op, red, hst);
            else
                shared_down_pass<kNT>(H, I, T, t0, P, c0, c1, sd, hs, op, red, hst);
        }
        if (combine) count_and_combine(H, k, T, kc_sd, P, n_contrib, ycount, o, w, osp, y, &sdo);
    }
}

}  // namespace

namespace bm_host {

// The library's own stream on the current device (default priority) and the
// events of a fork/join onto it, created on first use.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    std::mutex mu;
};
static SideStream *side_stream() {
    static SideStream ss[64];
    static std::mutex create;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lk(create);
    SideStream &d = ss[dev];
    if (!d.s) {
        hipStream_t st = nullptr;
        hipEvent_t f = nullptr, j = nullptr;
        // the fork and join order two streams of this device only: no
        // system-scope fence (about 2 us less per event on the device)
        const unsigned ef = hipEventDisableTiming | hipEventDisableSystemFence;
        if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess ||
            hipEventCreateWithFlags(&f, ef) != hipSuccess || hipEventCreateWithFlags(&j, ef) != hipSuccess)
            return nullptr;
        d.fork = f;
        d.join = j;
        d.s = st;
    }
    return &d;
}

size_t decode_mid_lds(int E) {
    return (size_t)std::max<int64_t>((int64_t)(2 + kBW) * E, kWaveBucketMax) * sizeof(int);
}

template <int FMT>
static int launch_decode_fmt(const bitmoe_layer *L, const void *x, int x_dtype, int T, const DecodePlan &p,
                             const DecodeBufs &b, hipStream_t s) {
    const int H = L->H, I = L->I, E = L->E, k = L->k;
    const bool shared = L->shared_gate != nullptr;
    const bool bf = x_dtype == BITMOE_BF16;
    if (p.kc_sd > kMaxChunks || p.kc_sg > kMaxChunks) return BITMOE_EUNSUPPORTED;
    // front: preparation, router rows, shared gate/up (at least one
    // workgroup: it clears the combine counters)
    const int n_front = std::max(1, p.prep_wg + p.n_rwg + (shared ? (I / 64) * p.kc_sg : 0));
    if (p.front_waves < 1 || p.front_waves > kW || (p.kc_sg && p.front_waves != kW)) return BITMOE_EINVAL;
    if (p.sg_rows && (T != 1 || p.sg_rows * k != 64 || p.slots != k || !shared)) return BITMOE_EINVAL;
    if ((p.bucket_in_front && (T * k > kWaveBucketMax || p.n_rwg)) ||
        (p.xprep_in_front && (!p.pf_tiles || FMT != BITMOE_FORMAT_2BIT || p.prep_wg != T)) ||
        p.prep_wg < (p.bucket_in_front ? 1 : 0))
        return BITMOE_EINVAL;
    {
        Buckets bk = b.bk;
        if (!p.pf_tiles) bk.tiles = nullptr;
        const FrontPrep pr{p.prep_wg, k, p.bucket_in_front ? b.ids : nullptr, bk, p.pf_tiles ? b.single : nullptr,
                           b.n_single, p.xprep_in_front ? b.pf.x16 : nullptr, b.pf.xsc};
        auto kf = bf ? k_dec_front<1> : k_dec_front<0>;
        kf<<<n_front, p.front_waves * 64, 0, s>>>(H, I, E, T, p.n_rwg, p.kc_sg, (const uint16_t *)L->router_w, x, b.logits,
                                       b.ycount, p.pf_tiles ? b.gctr : nullptr, (const uint4 *)L->shared_gate,
                                       (const uint4 *)L->shared_up, b.sgp, pr);
        BM_LAUNCH_CHECK();
    }
    // mid: top-k and bucketing of batches of more than one token
    if (p.need_mid) {
        const int64_t n = (int64_t)T * k;
        const bool in_mid = n <= 4096;
        const size_t sh = decode_mid_lds(E);
        if (sh > 64 * 1024)
            (void)hipFuncSetAttribute(reinterpret_cast<const void *>(k_dec_mid),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh);
        k_dec_mid<<<1, kBT, sh, s>>>(E, k, T, p.n_rwg ? b.logits : nullptr, b.ids, b.w, in_mid ? 1 : 0,
                                     b.bk.counts, b.bk.offsets, b.bk.perm, b.bk.active, b.bk.n_active,
                                     p.pf_tiles ? b.bk.tiles : nullptr, b.bk.n_tiles,
                                     p.pf_tiles ? b.single : nullptr, b.n_single);
        BM_LAUNCH_CHECK();
        if (!in_mid) {
            int rc = launch_bucket(b.ids, T, k, E, b.bk, s);
            if (rc) return rc;
        }
    }
    // routed gate/up; experts chosen by several tokens in a second launch
    const int n_gwg = p.slots * (I / 64);
    const int route_mode = T == 1 ? (p.n_rwg ? 1 : 2) : 0;
    static const bool lds_set = [] {
        bool ok = true;
        for (auto f : {k_dec_gateup<FMT, 1, 0>, k_dec_gateup<FMT, 0, 0>, k_dec_gateup<FMT, 1, 1>,
                       k_dec_gateup<FMT, 0, 1>}) {
            hipFuncAttributes fa;      // the tables must start at LDS address 0
            ok &= hipFuncGetAttributes(&fa, reinterpret_cast<const void *>(f)) == hipSuccess && fa.sharedSizeBytes == 0;
        }
        for (auto f : {k_dec_gateup<FMT, 1, 0>, k_dec_gateup<FMT, 0, 0>})
            ok &= hipFuncSetAttribute(reinterpret_cast<const void *>(f), hipFuncAttributeMaxDynamicSharedMemorySize,
                                      dec_gateup_lds<FMT, 0>()) == hipSuccess;
        for (auto f : {k_dec_gateup<FMT, 1, 1>, k_dec_gateup<FMT, 0, 1>})
            ok &= hipFuncSetAttribute(reinterpret_cast<const void *>(f), hipFuncAttributeMaxDynamicSharedMemorySize,
                                      dec_gateup_lds<FMT, 1>()) == hipSuccess;
        for (auto f : {k_dec_gateup<FMT, 1, 2>, k_dec_gateup<FMT, 0, 2>}) {
            hipFuncAttributes fa;
            ok &= hipFuncGetAttributes(&fa, reinterpret_cast<const void *>(f)) == hipSuccess && fa.sharedSizeBytes == 0;
            ok &= hipFuncSetAttribute(reinterpret_cast<const void *>(f), hipFuncAttributeMaxDynamicSharedMemorySize,
                                      dec_gateup_lds<FMT, 2>()) == hipSuccess;
        }
        return ok;
    }();
    if (!lds_set) return BITMOE_EHIP;
    // experts chosen by several tokens: the prefill kernels on the caller's
    // stream, and the single-token experts' gate/up and down beside them on
    // a stream of the library's own that forks after the routing and joins
    // before the combine launch.  The prefill kernels' activation preparation
    // needs no routing and goes before the fork (in the front launch up to
    // kFrontPrepMaxT tokens of 2-bit experts), and the prefill kernels are
    // enqueued before the other stream's, so that the device does not wait
    // for the host's fork.  They take their compute units first; the gate/up
    // workgroups claim their items one at a time, so those that start late
    // take fewer.  The lock keeps the fork/join sequence of one call whole
    // when several host threads share the stream.  Without the fork (p.fork
    // false) the same launches run one after the other on the caller's stream.
    const bool split = p.pf_tiles > 0;
    if (split && !p.xprep_in_front) {
        const int rc = launch_prefill_routed(L, x, x_dtype, T, b.bk, p.pf_tiles, b.pf, s, kPfPrep);
        if (rc) return rc;
    }
    SideStream *ss = nullptr;
    std::unique_lock<std::mutex> side_lock;
    hipStream_t sg_stream = s;
    if (split && p.fork) {
        ss = side_stream();
        if (!ss) return BITMOE_EHIP;
        side_lock = std::unique_lock<std::mutex>(ss->mu);
        if (hipEventRecord(ss->fork, s) != hipSuccess) return BITMOE_EHIP;
        if (hipStreamWaitEvent(ss->s, ss->fork, 0) != hipSuccess) return BITMOE_EHIP;
        sg_stream = ss->s;
    }
    // After the fork every return joins the side stream back into the
    // caller's first, so that no kernel of this call that writes the
    // workspace can still be running once the caller's stream moves on.
    auto fail = [&](int rc) {
        if (ss) {
            (void)hipEventRecord(ss->join, ss->s);
            (void)hipStreamWaitEvent(s, ss->join, 0);
        }
        return rc;
    };
#define BM_CHECK_JOIN()                                                   \
    do {                                                                  \
        if (hipGetLastError() != hipSuccess) return fail(BITMOE_EHIP);   \
    } while (0)
    if (split) {
        const int rc = launch_prefill_routed(L, x, x_dtype, T, b.bk, p.pf_tiles, b.pf, s, kPfRouted);
        if (rc) return fail(rc);
    }
    // gate/up launches: experts chosen by one token (all experts of a batch
    // of one), then, for larger batches without the prefill kernels, those
    // chosen by several tokens; batches of 2 to 8 tokens take both kinds in
    // one launch (MULTI = 2)
    const bool mixed = T > 1 && !split && T < bm_cfg::kSplitMinT;
    const int n_gu = T > 1 && !split && !mixed ? 2 : 1;
    for (int li = 0; li < n_gu; li++) {
        const int multi = li ? 1 : mixed ? 2 : 0;
        auto kg = multi == 2 ? (bf ? k_dec_gateup<FMT, 1, 2> : k_dec_gateup<FMT, 0, 2>)
                  : multi    ? (bf ? k_dec_gateup<FMT, 1, 1> : k_dec_gateup<FMT, 0, 1>)
                             : (bf ? k_dec_gateup<FMT, 1, 0> : k_dec_gateup<FMT, 0, 0>);
        const int lds = multi == 2 ? dec_gateup_lds<FMT, 2>() : multi ? dec_gateup_lds<FMT, 1>()
                                                                       : dec_gateup_lds<FMT, 0>();
        // the timing events, when set, are taken by the dispatch itself
        // around the first gate/up launch
        const TimingEvents ev = li ? TimingEvents{} : timing_for(BITMOE_TIME_GATEUP);
        const int grid = route_mode ? n_gwg : std::min(n_gwg, cu_count());
        hipExtLaunchKernelGGL(kg, dim3(grid), dim3(kWG * 64), lds, sg_stream, ev.start, ev.stop, 0, H, I,
                              E, k,
                              T, n_gwg, multi ? 0 : route_mode, (const uint8_t *)L->gate_q,
                              (const uint8_t *)L->up_q, (const uint8_t *)L->grid, x, (const float *)b.logits, b.ids,
                              b.w, b.bk, b.h, b.hsum2, b.hscale, p.kc_sg, (const float *)b.sgp, b.hs,
                              multi ? 0 : p.sg_rows, (const uint4 *)L->shared_gate, (const uint4 *)L->shared_up,
                              (const int4 *)b.single, (const int32_t *)b.n_single,
                              (!multi && split) ? b.gctr : nullptr);
        BM_CHECK_JOIN();
    }
    // down || shared down; the last workgroup to finish a panel combines it
    // (with the prefill kernels: the down runs on the library stream too,
    // beside the prefill down, and a combine launch follows the join)
    const int n_dwg = p.slots * (H / 64);
    // (beside the prefill kernels the shared down runs on the matrix cores,
    // in a launch of its own on the library stream)
    const bool sd_mfma = split && shared && (I / 8 + p.kc_sd - 1) / p.kc_sd <= kSdmPieces;
    if (sd_mfma) {
        k_shared_down_mfma<<<(H / 64) * p.kc_sd, kSdmW * 64, 0, sg_stream>>>(H, I, T, p.kc_sd,
                                                                           (const uint4 *)L->shared_down, b.hs, b.osp);
        BM_CHECK_JOIN();
    }
    const int n_sd = shared && !sd_mfma ? (H / 64) * p.kc_sd : 0;
    {
        const TimingEvents ev = timing_for(BITMOE_TIME_DOWN);
        hipExtLaunchKernelGGL(mixed ? k_dec_down<FMT, 2> : k_dec_down<FMT, 0>, dim3(n_dwg + n_sd), dim3(kWD * 64), 0,
                              sg_stream, ev.start, ev.stop, 0,
                              H, I, k, T, n_dwg, p.kc_sd, (const int32_t *)(split ? b.bk.n_tiles : nullptr),
                              split ? 0 : 1, (const uint8_t *)L->down_q, (const uint4 *)L->shared_down,
                              (const int32_t *)b.bk.counts, (const int32_t *)b.bk.offsets, (const int32_t *)b.bk.perm,
                              (const int32_t *)b.bk.active, (const int32_t *)b.bk.n_active, (const uint16_t *)b.h,
                              (const float2 *)b.hsum2, (const float *)b.hscale, (const uint16_t *)b.hs,
                              (const float *)b.w, b.ycount, shared ? b.osp : nullptr, b.o, b.y);
        BM_CHECK_JOIN();
    }
    if (split) {
        if (ss && hipEventRecord(ss->join, ss->s) != hipSuccess) return fail(BITMOE_EHIP);
        if (ss && hipStreamWaitEvent(s, ss->join, 0) != hipSuccess) return fail(BITMOE_EHIP);
        ss = nullptr;                                    // joined
        const int64_t n = (int64_t)T * H;
        k_dec_combine<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(H, k, T, shared ? p.kc_sd : 0, b.o, b.w,
                                                                  shared ? b.osp : nullptr, b.y);
        BM_LAUNCH_CHECK();
    }
#undef BM_CHECK_JOIN
    if (T > 1 && !split && !mixed) {
        k_dec_down<FMT, 1><<<n_dwg, kWD * 64, 0, s>>>(H, I, k, T, n_dwg, p.kc_sd, nullptr, 1, (const uint8_t *)L->down_q,
                                                (const uint4 *)L->shared_down, b.bk.counts, b.bk.offsets,
                                                b.bk.perm, b.bk.active, b.bk.n_active, b.h, b.hsum2, b.hscale, b.hs,
                                                b.w, b.ycount, shared ? b.osp : nullptr, b.o, b.y);
        BM_LAUNCH_CHECK();
    }
    return BITMOE_OK;
}

int launch_decode(const bitmoe_layer *L, const void *x, int x_dtype, int T, const DecodePlan &p,
                  const DecodeBufs &b, hipStream_t s) {
    return L->format == BITMOE_FORMAT_MXFP4 ? launch_decode_fmt<BITMOE_FORMAT_MXFP4>(L, x, x_dtype, T, p, b, s)
                                            : launch_decode_fmt<BITMOE_FORMAT_2BIT>(L, x, x_dtype, T, p, b, s);
}

}  // namespace bm_host
