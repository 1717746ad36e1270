// Decode FFN: fused dequant-GEMV over the active experts' packed blocks.
//
// y[t] = sum_j w[t][j] * D_e(silu(G_e x_t) * U_e x_t)  (+ shared expert)
// with up/gate in the IQ2_XXS-style codebook format and down in Q2_K, the
// shared expert in bf16 (page "ds4 : analyse pratique pour un usage
// documente", section "Support de modeles et choix de quantification").
// Decoding is bandwidth-bound (page "Faire tenir un MoE de 284B dans un
// portable de 128 Go", section "Un pre-remplissage a 790 t/s revele le
// veritable goulot d'etranglement"), so each active expert's blocks are read
// from HBM exactly once per call and decoded in registers.
//
// Mapping (tiled layout, see bitmoe.h): a workgroup owns one 64-row panel of
// one active expert; its KS waves split K; lane r of every wave owns row
// P*64 + r, so a wave's load of one 16-byte piece of 64 rows is one
// contiguous 1 KiB access.  Lanes never exchange partial dot products until
// the end (one LDS reduction over the KS waves).  The activations are the
// same for all 64 lanes: they are read with wave-uniform (scalar) loads.
//
// IQ2X decode: an LDS table holds, for every (codebook index, half of the 8,
// 4 sign bits), the four signed magnitudes as bf16 (64 KiB); one 8-byte read
// gives four signed weights, which a v_dot2 pairs with bf16 activations.
// The group scale d*(0.5+s)/4 multiplies the per-group fp32 sum.
#include "common.h"

namespace {

using namespace bm;

constexpr int kKS = 8;                 // waves per workgroup (K split)
constexpr int kNT = 4;                 // tokens per pass over the weights
constexpr int kTabEntries = 256 * 2 * 16;

struct DecodeArgs {
    int H, I, k, T;
    int slots;                 // grid.y slots reserved for routed experts
    const uint8_t *gate, *up, *down;       // tiled routed weights
    const uint8_t *grid;
    const uint8_t *sgate, *sup, *sdown;    // tiled bf16 shared weights or null
    const void *x;
    const int32_t *counts, *offsets, *perm, *active, *n_active;
    const float *w;
    float *h;        // [T*k][I]   routed h, bucket order
    float *hsum;     // [T*k][I/16] sums of h over 16-row sub-blocks
    float *o;        // [T*k][H]   routed down outputs, pair order
    float *hs;       // [T][I]     shared h
    float *os;       // [T][H]     shared down outputs
    float *y;        // [T][H]
};

// Token list of a workgroup: routed slot -> bucket entries, shared -> all T.
struct Tokens {
    int cnt, off, e;
    bool shared;
};

BM_DEV bool get_tokens(const DecodeArgs &a, Tokens &tk) {
    int slot = blockIdx.y;
    if (slot >= a.slots) {
        tk.shared = true;
        tk.cnt = a.T;
        tk.off = 0;
        tk.e = -1;
        return true;
    }
    tk.shared = false;
    if (slot >= *a.n_active) return false;
    tk.e = a.active[slot];
    tk.off = a.offsets[tk.e];
    tk.cnt = a.counts[tk.e];
    return true;
}

BM_DEV int token_of(const DecodeArgs &a, const Tokens &tk, int i) {
    return tk.shared ? i : a.perm[tk.off + i] / a.k;
}

BM_DEV void build_sign_table(const uint8_t *__restrict__ grid, uint2 *tab) {
    for (int i = threadIdx.x; i < kTabEntries; i += blockDim.x) {
        int idx = i >> 5, half = (i >> 4) & 1, nib = i & 15;
        uint32_t m4 = *reinterpret_cast<const uint32_t *>(grid + 8 * idx + 4 * half);
        uint32_t v[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            uint32_t b = __float_as_uint((float)((m4 >> (8 * q)) & 0xFFu)) >> 16;
            v[q] = b | (((uint32_t)nib >> q & 1u) << 15);
        }
        tab[i] = make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
    }
}

// sum_i w_i * x_i over 8 weights given as 4 bf16 pairs, for bf16 or fp32 x.
template <int XBF16>
BM_DEV float dot8(uint2 lo, uint2 hi, const void *xp, float acc) {
    if (XBF16) {
        uint4 xv = *reinterpret_cast<const uint4 *>(xp);
        acc = dot2_bf16(lo.x, xv.x, acc);
        acc = dot2_bf16(lo.y, xv.y, acc);
        acc = dot2_bf16(hi.x, xv.z, acc);
        acc = dot2_bf16(hi.y, xv.w, acc);
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(xp);
        float4 a = p[0], b = p[1];
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

// One IQ2X superblock of one row (this lane's), four 16-byte pieces + d,
// dotted with NT token rows starting at column k0.
template <int XBF16, int NT>
BM_DEV void iq2x_superblock(const uint4 (&q)[4], float d, const uint2 *tab, const void *x,
                            const int (&tok)[NT], int H, int k0, float (&acc)[NT]) {
#pragma unroll
    for (int g = 0; g < 8; g++) {
        uint32_t idxw = (g & 1) ? q[g >> 1].z : q[g >> 1].x;
        uint32_t aw = (g & 1) ? q[g >> 1].w : q[g >> 1].y;
        float scale = d * fmaf((float)(aw >> 28), 0.25f, 0.125f);
        float part[NT];
#pragma unroll
        for (int t = 0; t < NT; t++) part[t] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            uint32_t idx = (idxw >> (8 * j)) & 0xFFu;
            uint32_t s7 = (aw >> (7 * j)) & 0x7Fu;
            uint32_t par = __popc(s7) & 1u;
            uint2 lo = tab[idx * 32 + (s7 & 15u)];
            uint2 hi = tab[idx * 32 + 16 + ((s7 >> 4) | (par << 3))];
#pragma unroll
            for (int t = 0; t < NT; t++)
                part[t] = dot8<XBF16>(lo, hi, xrow<XBF16>(x, tok[t], H, k0 + 32 * g + 8 * j), part[t]);
        }
#pragma unroll
        for (int t = 0; t < NT; t++) acc[t] = fmaf(scale, part[t], acc[t]);
    }
}

// 8 bf16 weights (one 16-byte piece) dotted with NT token rows at column k.
template <int XBF16, int NT>
BM_DEV void bf16_piece(uint4 wv, const void *x, const int (&tok)[NT], int H, int k, float (&acc)[NT]) {
    uint2 lo = make_uint2(wv.x, wv.y), hi = make_uint2(wv.z, wv.w);
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = dot8<XBF16>(lo, hi, xrow<XBF16>(x, tok[t], H, k), acc[t]);
}

// ---------------------------------------------------------------------------
// gate/up + SwiGLU.  grid = (I/64 panels, slots [+1 shared]), block = KS waves.
// ---------------------------------------------------------------------------
template <int XBF16, int NT>
BM_DEV void gateup_pass(const DecodeArgs &a, const Tokens &tk, int t0, int P, const uint2 *tab,
                        float *red) {
    const int H = a.H, I = a.I, lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int tok[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) tok[t] = token_of(a, tk, min(t0 + t, tk.cnt - 1));
    float ag[NT], au[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) ag[t] = au[t] = 0.f;
    if (!tk.shared) {
        const int nb = H / kQK;
        const int64_t slab = (int64_t)I * nb * 66;
        const uint8_t *G = a.gate + tk.e * slab, *U = a.up + tk.e * slab;
        const uint4 *gq = reinterpret_cast<const uint4 *>(G);
        const uint4 *uq = reinterpret_cast<const uint4 *>(U);
        const uint16_t *gd = reinterpret_cast<const uint16_t *>(G + (int64_t)I * nb * 64);
        const uint16_t *ud = reinterpret_cast<const uint16_t *>(U + (int64_t)I * nb * 64);
        int per = (nb + kKS - 1) / kKS, kb0 = wv * per, kb1 = min(nb, kb0 + per);
        for (int kb = kb0; kb < kb1; kb++) {
            int64_t pk = (int64_t)P * nb + kb;
            uint4 g4[4], u4[4];
#pragma unroll
            for (int c = 0; c < 4; c++) {
                g4[c] = gq[(pk * 4 + c) * 64 + lane];
                u4[c] = uq[(pk * 4 + c) * 64 + lane];
            }
            float dg = fp16_to_f32(gd[pk * 64 + lane]);
            float du = fp16_to_f32(ud[pk * 64 + lane]);
            iq2x_superblock<XBF16, NT>(g4, dg, tab, a.x, tok, H, kb * kQK, ag);
            iq2x_superblock<XBF16, NT>(u4, du, tab, a.x, tok, H, kb * kQK, au);
        }
    } else {
        const int K8 = H / 8;
        const uint4 *gq = reinterpret_cast<const uint4 *>(a.sgate);
        const uint4 *uq = reinterpret_cast<const uint4 *>(a.sup);
        int per = (K8 + kKS - 1) / kKS, c0 = wv * per, c1 = min(K8, c0 + per);
#pragma unroll 4
        for (int c = c0; c < c1; c++) {
            int64_t pc = (int64_t)P * K8 + c;
            uint4 gw = gq[pc * 64 + lane], uw = uq[pc * 64 + lane];
            bf16_piece<XBF16, NT>(gw, a.x, tok, H, 8 * c, ag);
            bf16_piece<XBF16, NT>(uw, a.x, tok, H, 8 * c, au);
        }
    }
    // reduce over the KS waves: red[wave][t][0/1][lane]
#pragma unroll
    for (int t = 0; t < NT; t++) {
        red[((wv * NT + t) * 2 + 0) * 64 + lane] = ag[t];
        red[((wv * NT + t) * 2 + 1) * 64 + lane] = au[t];
    }
    __syncthreads();
    if (wv < NT && t0 + wv < tk.cnt) {
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int v = 0; v < kKS; v++) {
            g += red[((v * NT + wv) * 2 + 0) * 64 + lane];
            u += red[((v * NT + wv) * 2 + 1) * 64 + lane];
        }
        float hv = silu(g) * u;
        int n = P * 64 + lane;
        if (tk.shared) {
            a.hs[(int64_t)(t0 + wv) * I + n] = hv;
        } else {
            int64_t row = tk.off + t0 + wv;
            a.h[row * I + n] = hv;
            float s = hv;
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            s += __shfl_xor(s, 4, 64);
            s += __shfl_xor(s, 8, 64);
            if ((lane & 15) == 0) a.hsum[row * (I / 16) + (n >> 4)] = s;
        }
    }
    __syncthreads();
}

#define BM_DECODE_PARAMS                                                                    \
    int H, int I, int k, int T, int slots, const uint8_t *__restrict__ gate,                \
        const uint8_t *__restrict__ up, const uint8_t *__restrict__ down,                   \
        const uint8_t *__restrict__ grid, const uint8_t *__restrict__ sgate,                \
        const uint8_t *__restrict__ sup, const uint8_t *__restrict__ sdown,                 \
        const void *__restrict__ x, const int32_t *__restrict__ counts,                     \
        const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm,              \
        const int32_t *__restrict__ active, const int32_t *__restrict__ n_active,           \
        const float *__restrict__ w, float *__restrict__ h, float *__restrict__ hsum,       \
        float *__restrict__ o, float *__restrict__ hs, float *__restrict__ os,              \
        float *__restrict__ y
#define BM_DECODE_ARGS(a)                                                                   \
    a.H, a.I, a.k, a.T, a.slots, a.gate, a.up, a.down, a.grid, a.sgate, a.sup, a.sdown, a.x, \
        a.counts, a.offsets, a.perm, a.active, a.n_active, a.w, a.h, a.hsum, a.o, a.hs, a.os, a.y
#define BM_DECODE_UNPACK(a)                                                                 \
    DecodeArgs a{H,      I,      k,      T,     slots,  gate,    up,   down, grid,          \
                 sgate,  sup,    sdown,  x,     counts, offsets, perm, active, n_active,   \
                 w,      h,      hsum,   o,     hs,     os,      y}

template <int XBF16>
__global__ void __launch_bounds__(kKS * 64)
k_decode_gateup(BM_DECODE_PARAMS) {
    BM_DECODE_UNPACK(a);
    __shared__ uint2 tab[kTabEntries];           // 64 KiB signed-codebook table
    __shared__ float red[kKS * kNT * 2 * 64];    // 16 KiB cross-wave reduction
    Tokens tk;
    if (!get_tokens(a, tk)) return;
    if (!tk.shared) build_sign_table(a.grid, tab);
    __syncthreads();
    const int P = blockIdx.x;
    for (int t0 = 0; t0 < tk.cnt; t0 += kNT) {
        if (tk.cnt - t0 == 1)
            gateup_pass<XBF16, 1>(a, tk, t0, P, tab, red);
        else
            gateup_pass<XBF16, kNT>(a, tk, t0, P, tab, red);
    }
}

// ---------------------------------------------------------------------------
// down (+ weighted combine happens in k_combine).
// grid = (H/64 panels, slots [+1 shared]), block = KS waves splitting K = I.
// ---------------------------------------------------------------------------
template <int NT>
BM_DEV void down_pass(const DecodeArgs &a, const Tokens &tk, int t0, int P, float *red) {
    const int H = a.H, I = a.I, lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int rows[NT];   // h row of each token of the pass
#pragma unroll
    for (int t = 0; t < NT; t++) {
        int i = min(t0 + t, tk.cnt - 1);
        rows[t] = tk.shared ? i : tk.off + i;
    }
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = 0.f;
    if (!tk.shared) {
        const int nb = I / kQK;
        const int64_t slabsz = (int64_t)H * nb;
        const uint8_t *D = a.down + tk.e * slabsz * 84;
        const uint4 *dq = reinterpret_cast<const uint4 *>(D);
        const uint4 *ds = reinterpret_cast<const uint4 *>(D + slabsz * 64);
        const uint32_t *dd = reinterpret_cast<const uint32_t *>(D + slabsz * 80);
        int per = (nb + kKS - 1) / kKS, kb0 = wv * per, kb1 = min(nb, kb0 + per);
        for (int kb = kb0; kb < kb1; kb++) {
            int64_t pk = (int64_t)P * nb + kb;
            uint4 q4[4];
#pragma unroll
            for (int c = 0; c < 4; c++) q4[c] = dq[(pk * 4 + c) * 64 + lane];
            uint4 sc4 = ds[pk * 64 + lane];
            uint32_t dm = dd[pk * 64 + lane];
            float d = fp16_to_f32(dm & 0xFFFFu), dmin = fp16_to_f32(dm >> 16);
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const int hh = c >> 1, l0 = 16 * (c & 1);
                uint32_t qw[4] = {q4[c].x, q4[c].y, q4[c].z, q4[c].w};
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int b = 8 * hh + 2 * j + (c & 1);
                    uint32_t scw = (b < 4) ? sc4.x : (b < 8) ? sc4.y : (b < 12) ? sc4.z : sc4.w;
                    uint32_t sb = (scw >> (8 * (b & 3))) & 0xFFu;
                    float dsc = d * (float)(sb & 15u), dmm = dmin * (float)(sb >> 4);
                    const int kcol = kb * kQK + 128 * hh + 32 * j + l0;
#pragma unroll
                    for (int t = 0; t < NT; t++) {
                        const float4 *hp = reinterpret_cast<const float4 *>(
                            (tk.shared ? a.hs : a.h) + (int64_t)rows[t] * I + kcol);
                        float s = 0.f;
#pragma unroll
                        for (int w4 = 0; w4 < 4; w4++) {
                            uint32_t qv = (qw[w4] >> (2 * j)) & 0x03030303u;
                            float4 hv = hp[w4];
                            s = fmaf((float)(qv & 0xFFu), hv.x, s);
                            s = fmaf((float)((qv >> 8) & 0xFFu), hv.y, s);
                            s = fmaf((float)((qv >> 16) & 0xFFu), hv.z, s);
                            s = fmaf((float)(qv >> 24), hv.w, s);
                        }
                        float hsb = a.hsum[(int64_t)rows[t] * (I / 16) + (kcol >> 4)];
                        acc[t] = fmaf(dsc, s, fmaf(-dmm, hsb, acc[t]));
                    }
                }
            }
        }
    } else {
        const int K8 = I / 8;
        const uint4 *dq = reinterpret_cast<const uint4 *>(a.sdown);
        int per = (K8 + kKS - 1) / kKS, c0 = wv * per, c1 = min(K8, c0 + per);
#pragma unroll 4
        for (int c = c0; c < c1; c++) {
            uint4 wv4 = dq[((int64_t)P * K8 + c) * 64 + lane];
#pragma unroll
            for (int t = 0; t < NT; t++)
                acc[t] = dot8<0>(make_uint2(wv4.x, wv4.y), make_uint2(wv4.z, wv4.w),
                                 a.hs + (int64_t)rows[t] * I + 8 * c, acc[t]);
        }
    }
#pragma unroll
    for (int t = 0; t < NT; t++) red[(wv * NT + t) * 64 + lane] = acc[t];
    __syncthreads();
    if (wv < NT && t0 + wv < tk.cnt) {
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < kKS; v++) s += red[(v * NT + wv) * 64 + lane];
        int n = P * 64 + lane;
        if (tk.shared)
            a.os[(int64_t)(t0 + wv) * H + n] = s;
        else
            a.o[(int64_t)a.perm[tk.off + t0 + wv] * H + n] = s;
    }
    __syncthreads();
}

__global__ void __launch_bounds__(kKS * 64)
k_decode_down(BM_DECODE_PARAMS) {
    BM_DECODE_UNPACK(a);
    __shared__ float red[kKS * kNT * 64];
    Tokens tk;
    if (!get_tokens(a, tk)) return;
    const int P = blockIdx.x;
    for (int t0 = 0; t0 < tk.cnt; t0 += kNT) {
        if (tk.cnt - t0 == 1)
            down_pass<1>(a, tk, t0, P, red);
        else
            down_pass<kNT>(a, tk, t0, P, red);
    }
}

// y[t][n] = sum_j w[t][j] * o[t*k+j][n] (+ os[t][n]), slots in order.
__global__ void __launch_bounds__(256)
k_combine(const float *__restrict__ o, const float *__restrict__ w, const float *__restrict__ os,
          float *__restrict__ y, int T, int H, int k) {
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * H) return;
    int t = (int)(i / H), n = (int)(i % H);
    float s = 0.f;
    for (int j = 0; j < k; j++) s = fmaf(w[t * k + j], o[((int64_t)t * k + j) * H + n], s);
    if (os) s += os[i];
    y[i] = s;
}

}  // namespace

namespace bm_host {

int launch_decode_ffn(const bitmoe_layer *L, const void *x, int x_dtype, int T, const int32_t *ids,
                      const float *w, float *y, const Buckets &b, float *h, float *hsum, float *o,
                      float *hs, float *os, hipStream_t s) {
    (void)ids;
    DecodeArgs a;
    a.H = L->H; a.I = L->I; a.k = L->k; a.T = T;
    a.slots = (int)std::min<int64_t>(L->E, (int64_t)T * L->k);
    a.gate = (const uint8_t *)L->gate_q; a.up = (const uint8_t *)L->up_q;
    a.down = (const uint8_t *)L->down_q; a.grid = (const uint8_t *)L->grid;
    a.sgate = (const uint8_t *)L->shared_gate; a.sup = (const uint8_t *)L->shared_up;
    a.sdown = (const uint8_t *)L->shared_down;
    a.x = x;
    a.counts = b.counts; a.offsets = b.offsets; a.perm = b.perm;
    a.active = b.active; a.n_active = b.n_active;
    a.w = w; a.h = h; a.hsum = hsum; a.o = o; a.hs = hs; a.os = os; a.y = y;
    const bool shared = L->shared_gate != nullptr;
    dim3 g1(L->I / 64, a.slots + (shared ? 1 : 0));
    timing_begin(s);
    if (x_dtype == BITMOE_BF16)
        k_decode_gateup<1><<<g1, kKS * 64, 0, s>>>(BM_DECODE_ARGS(a));
    else
        k_decode_gateup<0><<<g1, kKS * 64, 0, s>>>(BM_DECODE_ARGS(a));
    BM_LAUNCH_CHECK();
    timing_end(s);
    dim3 g2(L->H / 64, a.slots + (shared ? 1 : 0));
    k_decode_down<<<g2, kKS * 64, 0, s>>>(BM_DECODE_ARGS(a));
    BM_LAUNCH_CHECK();
    int64_t n = (int64_t)T * L->H;
    k_combine<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(o, w, shared ? os : nullptr, y, T, L->H, L->k);
    BM_LAUNCH_CHECK();
    return BITMOE_OK;
}

}  // namespace bm_host
