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
// Launches, each balanced so that every wave streams a similar number of
// bytes:
//   front  : codebook table, router rows (optional) || shared-expert
//            gate/up, split over K
//   mid    : top-k (optional) and bucketing (one workgroup)
//   gateup : routed gate/up + SwiGLU per (active expert, 64-row panel)
//            || shared h = silu(sum of gate partials) * (sum of up partials)
//            (experts chosen by several tokens: a second launch)
//   down   : routed down per (active expert, 64-row panel) || shared down,
//            split over K
//   combine: y = sum of the k weighted slots + shared partials, in a fixed
//            order, so results are reproducible run to run.
//
// Mapping: lane r of every wave owns row P*64 + r of a panel (tiled layout),
// so one 16-byte load by 64 lanes is one contiguous 1 KiB access; the waves
// of a workgroup split K and meet once in LDS.  Activations are identical
// for all lanes and arrive through wave-uniform (scalar) loads.
#include <algorithm>

#include "device_util.h"

namespace {

using namespace bm;

constexpr int kW = 8;              // waves per workgroup
constexpr int kWG = 16;            // waves per routed gate/up workgroup
constexpr int kNT = 4;             // tokens per pass over the weights
constexpr int kTabU4 = kIq2xMainEntries + kIq2xMaskBytes / 16;   // decode tables, uint4 units
constexpr int kTabWG = (kTabU4 + kW * 64 - 1) / (kW * 64);      // front workgroups that build them

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

// One IQ2X superblock of this lane's row: four 16-byte pieces (8 groups of
// four 16-bit fields) and the fp16 d; dotted with NT activation rows.
// Per run of 8 weights: one 16-byte main-table read (weights 0..7, signs of
// 0..3 and the parity sign of 7 applied) and one read of the 64-byte mask
// table (all lanes hit 8 addresses: broadcast, no bank conflicts).
template <int XBF16, int NT>
BM_DEV void iq2x_superblock(const uint4 (&q)[4], float d, const char *tab, const void *x,
                            const int (&tok)[NT], int H, int k0, float (&acc)[NT]) {
#pragma unroll
    for (int g = 0; g < 8; g++) {
        const uint32_t W0 = (g & 1) ? q[g >> 1].z : q[g >> 1].x;
        const uint32_t W1 = (g & 1) ? q[g >> 1].w : q[g >> 1].y;
        const float scale = d * fmaf((float)iq2x_scale(W0, W1), 0.25f, 0.125f);   // d*(0.5+s)/4
        uint4 v[4];
        uint2 m[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t F = ((j < 2 ? W0 : W1) >> (16 * (j & 1))) & 0xFFFFu;
            v[j] = *reinterpret_cast<const uint4 *>(tab + iq2x_main_off(F));
            m[j] = *reinterpret_cast<const uint2 *>(tab + 16 * kIq2xMainEntries + iq2x_mask_off(F));
        }
        float part[NT];
#pragma unroll
        for (int t = 0; t < NT; t++) part[t] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint2 lo = make_uint2(v[j].x, v[j].y);
            const uint2 hi = make_uint2(v[j].z ^ m[j].x, v[j].w ^ m[j].y);
#pragma unroll
            for (int t = 0; t < NT; t++)
                part[t] = dot8<XBF16>(lo, hi, xrow<XBF16>(x, tok[t], H, k0 + 32 * g + 8 * j), part[t]);
        }
#pragma unroll
        for (int t = 0; t < NT; t++) acc[t] = fmaf(scale, part[t], acc[t]);
    }
}

// Even split of [0, n) over `parts`; returns [lo, hi) of part `i`.
BM_DEV void split_range(int n, int parts, int i, int &lo, int &hi) {
    lo = (int)((int64_t)n * i / parts);
    hi = (int)((int64_t)n * (i + 1) / parts);
}

// ---------------------------------------------------------------------------
// front: router rows || shared gate/up partial sums over K chunk c.
// grid = n_rwg + (I/64)*kc_sg workgroups of kW waves.
// sgp layout [kc_sg][2][T][I] (gate, up).
// ---------------------------------------------------------------------------
template <int XBF16, int NT>
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
    split_range(c1 - c0, kW, wv, w0, w1);
#pragma unroll 4
    for (int c = c0 + w0; c < c0 + w1; c++) {
        const int64_t pc = ((int64_t)P * K8 + c) * 64 + lane;
        const uint4 gw = sg[pc], uw = su[pc];
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const void *xp = xrow<XBF16>(x, tok[t], H, 8 * c);
            ag[t] = dot8<XBF16>(make_uint2(gw.x, gw.y), make_uint2(gw.z, gw.w), xp, ag[t]);
            au[t] = dot8<XBF16>(make_uint2(uw.x, uw.y), make_uint2(uw.z, uw.w), xp, au[t]);
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
        for (int v = 0; v < kW; v++) {
            g += red[((v * kNT + wv) * 2 + 0) * 64 + lane];
            u += red[((v * kNT + wv) * 2 + 1) * 64 + lane];
        }
        gp[(int64_t)(t0 + wv) * I + P * 64 + lane] = g;
        up_[(int64_t)(t0 + wv) * I + P * 64 + lane] = u;
    }
    __syncthreads();
}

template <int XBF16>
__global__ void __launch_bounds__(kW * 64)
k_dec_front(int H, int I, int E, int T, int n_rwg, int kc_sg, const uint16_t *__restrict__ wr,
            const void *__restrict__ x, const uint4 *__restrict__ sg, const uint4 *__restrict__ su,
            const uint8_t *__restrict__ grid, uint4 *__restrict__ gtab, float *__restrict__ logits,
            float *__restrict__ sgp) {
    __shared__ float red[kW * kNT * 2 * 64];
    int b = blockIdx.x;
    if (b < kTabWG) {          // the decode tables, once per call
        const int i = b * kW * 64 + threadIdx.x;
        if (i < kIq2xMainEntries) {
            gtab[i] = iq2x_main_entry(grid, i);
        } else if (i < kTabU4) {
            const int m = 2 * (i - kIq2xMainEntries);
            const uint2 a = iq2x_mask_entry(m), c = iq2x_mask_entry(m + 1);
            gtab[i] = make_uint4(a.x, a.y, c.x, c.y);
        }
        return;
    }
    b -= kTabWG;
    if (b < n_rwg) {
        const int e = b * kW + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
    const int bs = b - n_rwg, P = bs / kc_sg, c = bs % kc_sg;
    int c0, c1;
    split_range(H / 8, kc_sg, c, c0, c1);
    float *gp = sgp + (int64_t)(c * 2 + 0) * T * I;
    float *up_ = sgp + (int64_t)(c * 2 + 1) * T * I;
    for (int t0 = 0; t0 < T; t0 += kNT) {
        if (T - t0 == 1)
            shared_gateup_pass<XBF16, 1>(H, I, T, t0, P, c0, c1, sg, su, x, gp, up_, red);
        else
            shared_gateup_pass<XBF16, kNT>(H, I, T, t0, P, c0, c1, sg, su, x, gp, up_, red);
    }
}

// ---------------------------------------------------------------------------
// mid: one workgroup of kBT threads.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kBT)
k_dec_mid(int E, int k, int T, const float *__restrict__ logits, int32_t *__restrict__ ids,
          float *__restrict__ w, int do_bucket, int32_t *__restrict__ counts,
          int32_t *__restrict__ offsets, int32_t *__restrict__ perm, int32_t *__restrict__ active,
          int32_t *__restrict__ n_active) {
    extern __shared__ int smem[];
    __shared__ int swave[kBW + 1];
    const int tid = threadIdx.x, wv = tid >> 6;
    if (logits) {
        for (int t = wv; t < T; t += kBW)
            topk_wave(logits + (int64_t)t * E, E, k, ids + (int64_t)t * k, w + (int64_t)t * k);
        __threadfence_block();
        __syncthreads();
    }
    if (do_bucket)
        bucket_block(ids, T * k, E, counts, offsets, perm, active, n_active, nullptr, nullptr, 1, smem,
                     swave);
}

// ---------------------------------------------------------------------------
// gateup: routed gate/up + SwiGLU || shared down partial sums over K.
// grid = slots*(I/64) routed workgroups, then (H/64)*kc_sd shared ones.
// ---------------------------------------------------------------------------
struct Tok {
    int cnt, off, e;
};

template <int XBF16, int NT>
BM_DEV void routed_gateup_pass(int H, int I, int k, const Tok &tk, int t0, int P, const char *tab,
                               const uint8_t *__restrict__ gate, const uint8_t *__restrict__ up,
                               const void *__restrict__ x, const int32_t *__restrict__ perm,
                               uint16_t *__restrict__ h, int64_t hrows, float *__restrict__ hsum,
                               float *red) {
    const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int tok[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) tok[t] = perm[tk.off + min(t0 + t, tk.cnt - 1)] / k;
    float ag[NT], au[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) ag[t] = au[t] = 0.f;
    const int nb = H / kQK;
    const int64_t slab = (int64_t)I * nb * 66;
    const uint8_t *G = gate + tk.e * slab, *U = up + tk.e * slab;
    const uint4 *gq = reinterpret_cast<const uint4 *>(G);
    const uint4 *uq = reinterpret_cast<const uint4 *>(U);
    const uint16_t *gd = reinterpret_cast<const uint16_t *>(G + (int64_t)I * nb * 64);
    const uint16_t *ud = reinterpret_cast<const uint16_t *>(U + (int64_t)I * nb * 64);
    int kb0, kb1;
    split_range(nb, kWG, wv, kb0, kb1);
    // software pipeline: the next superblock's 8 pieces are in flight while
    // the current one is decoded
    uint4 g4[4], u4[4], ng[4], nu[4];
    uint32_t gdw = 0, udw = 0, ngd = 0, nud = 0;
    auto load = [&](int kb, uint4 (&a)[4], uint4 (&bq)[4], uint32_t &da, uint32_t &db) {
        const int64_t pk = (int64_t)P * nb + kb;
#pragma unroll
        for (int c = 0; c < 4; c++) {
            a[c] = gq[(pk * 4 + c) * 64 + lane];
            bq[c] = uq[(pk * 4 + c) * 64 + lane];
        }
        da = gd[pk * 64 + lane];
        db = ud[pk * 64 + lane];
    };
    if (kb0 < kb1) load(kb0, g4, u4, gdw, udw);
    for (int kb = kb0; kb < kb1; kb++) {
        if (kb + 1 < kb1) load(kb + 1, ng, nu, ngd, nud);
        iq2x_superblock<XBF16, NT>(g4, fp16_to_f32(gdw), tab, x, tok, H, kb * kQK, ag);
        iq2x_superblock<XBF16, NT>(u4, fp16_to_f32(udw), tab, x, tok, H, kb * kQK, au);
#pragma unroll
        for (int c = 0; c < 4; c++) {
            g4[c] = ng[c];
            u4[c] = nu[c];
        }
        gdw = ngd;
        udw = nud;
    }
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
        // h as bf16 hi + lo (about 16 significant bits); within every aligned
        // quad the order is [0, 2, 1, 3] so that the down kernel's bf16 pairs
        // line up with pairs of 2-bit quants taken from bytes (0, 2), (1, 3)
        const uint32_t hi = f32_to_bf16_rne(hv);
        const uint32_t lo = f32_to_bf16_rne(hv - bf16_to_f32(hi));
        const int pn = (n & ~3) | ((n & 1) << 1) | ((n >> 1) & 1);
        h[row * I + pn] = (uint16_t)hi;
        h[((int64_t)row + hrows) * I + pn] = (uint16_t)lo;
        float s = bf16_to_f32(hi) + bf16_to_f32(lo);
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        s += __shfl_xor(s, 4, 64);
        s += __shfl_xor(s, 8, 64);
        if ((lane & 15) == 0) hsum[row * (I / 16) + (n >> 4)] = s;
    }
    __syncthreads();
}

// sum of 8 products of bf16 weight pairs with h given as bf16 hi + lo
BM_DEV float dot8_hilo(uint4 wq, uint4 hh, uint4 hl, float acc) {
    acc = dot2_bf16(wq.x, hh.x, acc); acc = dot2_bf16(wq.x, hl.x, acc);
    acc = dot2_bf16(wq.y, hh.y, acc); acc = dot2_bf16(wq.y, hl.y, acc);
    acc = dot2_bf16(wq.z, hh.z, acc); acc = dot2_bf16(wq.z, hl.z, acc);
    acc = dot2_bf16(wq.w, hh.w, acc); acc = dot2_bf16(wq.w, hl.w, acc);
    return acc;
}

template <int NT>
BM_DEV void shared_down_pass(int H, int I, int T, int t0, int P, int c0, int c1,
                             const uint4 *__restrict__ sd, const uint16_t *__restrict__ hs,
                             float *__restrict__ osp, float *red) {
    const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int K8 = I / 8;
    const int64_t lo_off = (int64_t)T * I;
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = 0.f;
    int w0, w1;
    split_range(c1 - c0, kW, wv, w0, w1);
#pragma unroll 4
    for (int c = c0 + w0; c < c0 + w1; c++) {
        const uint4 wq = sd[((int64_t)P * K8 + c) * 64 + lane];
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const uint16_t *hp = hs + (int64_t)min(t0 + t, T - 1) * I + 8 * c;
            acc[t] = dot8_hilo(wq, *reinterpret_cast<const uint4 *>(hp),
                               *reinterpret_cast<const uint4 *>(hp + lo_off), acc[t]);
        }
    }
#pragma unroll
    for (int t = 0; t < NT; t++) red[(wv * kNT + t) * 64 + lane] = acc[t];
    __syncthreads();
    if (wv < NT && t0 + wv < T) {
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < kW; v++) s += red[(v * kNT + wv) * 64 + lane];
        osp[(int64_t)(t0 + wv) * H + P * 64 + lane] = s;
    }
    __syncthreads();
}

// MULTI = 0 takes the experts chosen by exactly one token (and the shared
// h); MULTI = 1 the experts with several tokens (passes of kNT tokens).
// Keeping the two apart keeps each kernel's register use low.
template <int XBF16, int MULTI>
__global__ void __launch_bounds__(kWG * 64)
k_dec_gateup(int H, int I, int k, int T, int n_gwg, int kc_sg, const uint8_t *__restrict__ gate,
             const uint8_t *__restrict__ up, const uint4 *__restrict__ gtab,
             const void *__restrict__ x, const int32_t *__restrict__ counts,
             const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm,
             const int32_t *__restrict__ active, const int32_t *__restrict__ n_active,
             const float *__restrict__ sgp, uint16_t *__restrict__ hs, uint16_t *__restrict__ h,
             float *__restrict__ hsum) {
    const int64_t hrows = (int64_t)T * k;
    __shared__ uint4 tab[kTabU4];
    __shared__ float red[kWG * (MULTI ? kNT : 1) * 2 * 64];
    const int b = blockIdx.x;
    if (b < n_gwg) {
        const int panels = I / 64, slot = b / panels, P = b % panels;
        if (slot >= *n_active) return;
        Tok tk;
        tk.e = active[slot];
        tk.off = offsets[tk.e];
        tk.cnt = counts[tk.e];
        if ((tk.cnt > 1) != (MULTI != 0)) return;
        for (int i = threadIdx.x; i < kTabU4; i += blockDim.x) tab[i] = gtab[i];
        __syncthreads();
        const char *tb = reinterpret_cast<const char *>(tab);
        if (!MULTI) {
            routed_gateup_pass<XBF16, 1>(H, I, k, tk, 0, P, tb, gate, up, x, perm, h, hrows, hsum, red);
            return;
        }
        for (int t0 = 0; t0 < tk.cnt; t0 += kNT) {
            if (tk.cnt - t0 == 1)
                routed_gateup_pass<XBF16, 1>(H, I, k, tk, t0, P, tb, gate, up, x, perm, h, hrows, hsum, red);
            else
                routed_gateup_pass<XBF16, kNT>(H, I, k, tk, t0, P, tb, gate, up, x, perm, h, hrows, hsum, red);
        }
        return;
    }
    if (MULTI) return;
    // shared h = silu(sum of gate partials) * (sum of up partials), fixed order
    const int64_t n = (int64_t)T * I;
    const int64_t i = (int64_t)(b - n_gwg) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float g = 0.f, u = 0.f;
    for (int c = 0; c < kc_sg; c++) {
        g += sgp[(int64_t)(2 * c) * n + i];
        u += sgp[(int64_t)(2 * c + 1) * n + i];
    }
    const float hv = silu(g) * u;
    const uint32_t hi = f32_to_bf16_rne(hv);
    hs[i] = (uint16_t)hi;
    hs[n + i] = (uint16_t)f32_to_bf16_rne(hv - bf16_to_f32(hi));
}

// ---------------------------------------------------------------------------
// down: routed Q2K down per (slot, panel) || shared down split over K.
// grid = slots*(H/64) + (H/64)*kc_sd.  o[pair][H] unweighted.
// ---------------------------------------------------------------------------
template <int NT>
BM_DEV void routed_down_pass(int H, int I, const Tok &tk, int t0, int P,
                             const uint8_t *__restrict__ down, const int32_t *__restrict__ perm,
                             const uint16_t *__restrict__ h, int64_t hrows,
                             const float *__restrict__ hsum, float *__restrict__ o, float *red) {
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
    split_range(nb, kW, wv, kb0, kb1);
    for (int kb = kb0; kb < kb1; kb++) {
        const int64_t pk = (int64_t)P * nb + kb;
        uint4 q4[4];
#pragma unroll
        for (int c = 0; c < 4; c++) q4[c] = dq[(pk * 4 + c) * 64 + lane];
        const uint4 sc4 = ds[pk * 64 + lane];
        const uint32_t dm = dd[pk * 64 + lane];
        const float d = fp16_to_f32(dm & 0xFFFFu), dmin = fp16_to_f32(dm >> 16);
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const int hh = c >> 1, l0 = 16 * (c & 1);
            const uint32_t qw[4] = {q4[c].x, q4[c].y, q4[c].z, q4[c].w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int b = 8 * hh + 2 * j + (c & 1);
                const uint32_t scw = (b < 4) ? sc4.x : (b < 8) ? sc4.y : (b < 12) ? sc4.z : sc4.w;
                const uint32_t sb = (scw >> (8 * (b & 3))) & 0xFFu;
                const float dsc = d * (float)(sb & 15u), dmm = dmin * (float)(sb >> 4);
                const int kcol = kb * kQK + 128 * hh + 32 * j + l0;
                // (128 + q) as bf16 pairs from quant bytes (0,2) and (1,3)
                uint32_t qp[8];
#pragma unroll
                for (int w4 = 0; w4 < 4; w4++) {
                    const uint32_t t4 = qw[w4] >> (2 * j);
                    qp[2 * w4] = (t4 & 0x00030003u) | 0x43004300u;
                    qp[2 * w4 + 1] = ((t4 >> 8) & 0x00030003u) | 0x43004300u;
                }
#pragma unroll
                for (int t = 0; t < NT; t++) {
                    const uint4 *hp = reinterpret_cast<const uint4 *>(h + (int64_t)rows[t] * I + kcol);
                    const uint4 *lp = reinterpret_cast<const uint4 *>(h + ((int64_t)rows[t] + hrows) * I + kcol);
                    const uint4 a0 = hp[0], a1 = hp[1], b0 = lp[0], b1 = lp[1];
                    float sacc = dot2_bf16(qp[0], a0.x, 0.f);
                    sacc = dot2_bf16(qp[0], b0.x, sacc);
                    sacc = dot2_bf16(qp[1], a0.y, sacc); sacc = dot2_bf16(qp[1], b0.y, sacc);
                    sacc = dot2_bf16(qp[2], a0.z, sacc); sacc = dot2_bf16(qp[2], b0.z, sacc);
                    sacc = dot2_bf16(qp[3], a0.w, sacc); sacc = dot2_bf16(qp[3], b0.w, sacc);
                    sacc = dot2_bf16(qp[4], a1.x, sacc); sacc = dot2_bf16(qp[4], b1.x, sacc);
                    sacc = dot2_bf16(qp[5], a1.y, sacc); sacc = dot2_bf16(qp[5], b1.y, sacc);
                    sacc = dot2_bf16(qp[6], a1.z, sacc); sacc = dot2_bf16(qp[6], b1.z, sacc);
                    sacc = dot2_bf16(qp[7], a1.w, sacc); sacc = dot2_bf16(qp[7], b1.w, sacc);
                    // sum (128+q) h = 128 hsum + sum q h
                    const float hsb = hsum[(int64_t)rows[t] * (I / 16) + (kcol >> 4)];
                    acc[t] = fmaf(dsc, sacc, fmaf(-fmaf(128.f, dsc, dmm), hsb, acc[t]));
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; t++) red[(wv * kNT + t) * 64 + lane] = acc[t];
    __syncthreads();
    if (wv < NT && t0 + wv < tk.cnt) {
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < kW; v++) s += red[(v * kNT + wv) * 64 + lane];
        o[(int64_t)perm[tk.off + t0 + wv] * H + P * 64 + lane] = s;
    }
    __syncthreads();
}

__global__ void __launch_bounds__(kW * 64)
k_dec_down(int H, int I, int k, int T, int n_dwg, int kc_sd, const uint8_t *__restrict__ down,
           const uint4 *__restrict__ sd, const int32_t *__restrict__ counts,
           const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm,
           const int32_t *__restrict__ active, const int32_t *__restrict__ n_active,
           const uint16_t *__restrict__ h, const float *__restrict__ hsum,
           const uint16_t *__restrict__ hs, float *__restrict__ osp, float *__restrict__ o) {
    const int64_t hrows = (int64_t)T * k;
    __shared__ float red[kW * kNT * 64];
    const int panels = H / 64;
    const int na = *n_active;
    int P;
    if ((int)blockIdx.x < n_dwg) {
        const int slot = blockIdx.x / panels;
        P = blockIdx.x % panels;
        if (slot >= na) return;
        Tok tk;
        tk.e = active[slot];
        tk.off = offsets[tk.e];
        tk.cnt = counts[tk.e];
        for (int t0 = 0; t0 < tk.cnt; t0 += kNT) {
            if (tk.cnt - t0 == 1)
                routed_down_pass<1>(H, I, tk, t0, P, down, perm, h, hrows, hsum, o, red);
            else
                routed_down_pass<kNT>(H, I, tk, t0, P, down, perm, h, hrows, hsum, o, red);
        }
    } else {
        const int bs = blockIdx.x - n_dwg, c = bs % kc_sd;
        P = bs / kc_sd;
        int c0, c1;
        split_range(I / 8, kc_sd, c, c0, c1);
        float *op = osp + (int64_t)c * T * H;
        for (int t0 = 0; t0 < T; t0 += kNT) {
            if (T - t0 == 1)
                shared_down_pass<1>(H, I, T, t0, P, c0, c1, sd, hs, op, red);
            else
                shared_down_pass<kNT>(H, I, T, t0, P, c0, c1, sd, hs, op, red);
        }
    }
}

// y[t][n] = sum_j w[t][j] * o[t*k+j][n] (+ shared partials), fixed order.
__global__ void __launch_bounds__(256)
k_dec_combine(int H, int k, int T, int kc_sd, const float *__restrict__ o,
              const float *__restrict__ w, const float *__restrict__ osp, float *__restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * H) return;
    const int t = (int)(i / H);
    const int n = (int)(i - (int64_t)t * H);
    float s = 0.f;
    for (int j = 0; j < k; j++) s = fmaf(w[t * k + j], o[((int64_t)t * k + j) * H + n], s);
    if (osp)
        for (int c = 0; c < kc_sd; c++) s += osp[((int64_t)c * T + t) * H + n];
    y[i] = s;
}

}  // namespace

namespace bm_host {

DecodePlan decode_plan(const bitmoe_layer *L, int T, bool with_router) {
    DecodePlan p;
    const bool shared = L->shared_gate != nullptr;
    p.slots = (int)std::min<int64_t>(L->E, (int64_t)T * L->k);
    p.n_rwg = with_router ? (L->E + kW - 1) / kW : 0;
    p.kc_sg = shared ? 8 : 0;
    p.kc_sd = shared ? 4 : 0;
    p.bucket_in_mid = (int64_t)T * L->k <= 4096;
    return p;
}

size_t decode_mid_lds(int E) { return (size_t)(2 + kBW) * E * sizeof(int); }

int launch_decode(const bitmoe_layer *L, const void *x, int x_dtype, int T, const DecodePlan &p,
                  const DecodeBufs &b, hipStream_t s) {
    const int H = L->H, I = L->I, E = L->E, k = L->k;
    const bool shared = L->shared_gate != nullptr;
    // front
    const int n_front = kTabWG + p.n_rwg + (shared ? (I / 64) * p.kc_sg : 0);
    {
        if (x_dtype == BITMOE_BF16)
            k_dec_front<1><<<n_front, kW * 64, 0, s>>>(H, I, E, T, p.n_rwg, p.kc_sg,
                                                       (const uint16_t *)L->router_w, x,
                                                       (const uint4 *)L->shared_gate,
                                                       (const uint4 *)L->shared_up, (const uint8_t *)L->grid,
                                                       b.tab, b.logits, b.sgp);
        else
            k_dec_front<0><<<n_front, kW * 64, 0, s>>>(H, I, E, T, p.n_rwg, p.kc_sg,
                                                       (const uint16_t *)L->router_w, x,
                                                       (const uint4 *)L->shared_gate,
                                                       (const uint4 *)L->shared_up, (const uint8_t *)L->grid,
                                                       b.tab, b.logits, b.sgp);
        BM_LAUNCH_CHECK();
    }
    // mid
    const size_t sh = decode_mid_lds(E);
    if (sh > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(k_dec_mid),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh);
    k_dec_mid<<<1, kBT, sh, s>>>(E, k, T, p.n_rwg ? b.logits : nullptr, b.ids, b.w,
                                 p.bucket_in_mid ? 1 : 0, b.bk.counts, b.bk.offsets, b.bk.perm,
                                 b.bk.active, b.bk.n_active);
    BM_LAUNCH_CHECK();
    if (!p.bucket_in_mid) {
        int rc = launch_bucket(b.ids, T, k, E, b.bk, s);
        if (rc) return rc;
    }
    // gateup (+ shared h)
    const int n_gwg = p.slots * (I / 64);
    const int n_fin = shared ? (int)(((int64_t)T * I + kWG * 64 - 1) / (kWG * 64)) : 0;
    timing_begin(s);
    if (x_dtype == BITMOE_BF16)
        k_dec_gateup<1, 0><<<n_gwg + n_fin, kWG * 64, 0, s>>>(H, I, k, T, n_gwg, p.kc_sg,
                                                              (const uint8_t *)L->gate_q, (const uint8_t *)L->up_q,
                                                              (const uint4 *)b.tab, x, b.bk.counts, b.bk.offsets,
                                                              b.bk.perm, b.bk.active, b.bk.n_active, b.sgp, b.hs,
                                                              b.h, b.hsum);
    else
        k_dec_gateup<0, 0><<<n_gwg + n_fin, kWG * 64, 0, s>>>(H, I, k, T, n_gwg, p.kc_sg,
                                                              (const uint8_t *)L->gate_q, (const uint8_t *)L->up_q,
                                                              (const uint4 *)b.tab, x, b.bk.counts, b.bk.offsets,
                                                              b.bk.perm, b.bk.active, b.bk.n_active, b.sgp, b.hs,
                                                              b.h, b.hsum);
    BM_LAUNCH_CHECK();
    if (T > 1) {   // experts chosen by several tokens
        if (x_dtype == BITMOE_BF16)
            k_dec_gateup<1, 1><<<n_gwg, kWG * 64, 0, s>>>(H, I, k, T, n_gwg, p.kc_sg,
                                                          (const uint8_t *)L->gate_q, (const uint8_t *)L->up_q,
                                                          (const uint4 *)b.tab, x, b.bk.counts, b.bk.offsets,
                                                          b.bk.perm, b.bk.active, b.bk.n_active, b.sgp, b.hs,
                                                          b.h, b.hsum);
        else
            k_dec_gateup<0, 1><<<n_gwg, kWG * 64, 0, s>>>(H, I, k, T, n_gwg, p.kc_sg,
                                                          (const uint8_t *)L->gate_q, (const uint8_t *)L->up_q,
                                                          (const uint4 *)b.tab, x, b.bk.counts, b.bk.offsets,
                                                          b.bk.perm, b.bk.active, b.bk.n_active, b.sgp, b.hs,
                                                          b.h, b.hsum);
    }
    BM_LAUNCH_CHECK();
    timing_end(s);
    // down (+ shared down), then the combine
    const int n_dwg = p.slots * (H / 64);
    const int n_sd = shared ? (H / 64) * p.kc_sd : 0;
    k_dec_down<<<n_dwg + n_sd, kW * 64, 0, s>>>(H, I, k, T, n_dwg, p.kc_sd, (const uint8_t *)L->down_q,
                                                (const uint4 *)L->shared_down, b.bk.counts, b.bk.offsets,
                                                b.bk.perm, b.bk.active, b.bk.n_active, b.h, b.hsum, b.hs,
                                                shared ? b.osp : nullptr, b.o);
    BM_LAUNCH_CHECK();
    const int64_t ny = (int64_t)T * H;
    k_dec_combine<<<(unsigned)((ny + 255) / 256), 256, 0, s>>>(H, k, T, p.kc_sd, b.o, b.w,
                                                               shared ? b.osp : nullptr, b.y);
    BM_LAUNCH_CHECK();
    return BITMOE_OK;
}

}  // namespace bm_host
