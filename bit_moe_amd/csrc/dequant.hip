// Standalone dequantisation of canonical IQ2X / Q2K / MXFP4 blocks, and the
// load-time canonical -> tiled layout transforms.
//
// Formats: the routed experts' IQ2_XXS-style up/gate blocks and Q2_K down
// blocks (page "ds4 : analyse pratique pour un usage documente", section
// "Support de modeles et choix de quantification"), in GGML's byte order
// (page "antirez/ds4 - Moteur local d'inference DeepSeek V4 Flash pour
// Metal", section "Remerciements a llama.cpp et GGML").
//
// Exactness: an IQ2X value d*(0.5+s)/4*g has at most 11+5+3 significant bits,
// so every product below is exact in fp32 whatever the evaluation order.  A
// Q2K value is one fp32 rounding of (d*scale)*q - dmin*min, both products
// exact; fmaf gives that single rounding.
#include "common.h"

namespace {

using namespace bm;

// One thread per (block, group of 32 weights).
template <int OUT_BF16>
__global__ void __launch_bounds__(256)
k_dequant_iq2x(const uint8_t *__restrict__ blocks, const uint8_t *__restrict__ grid,
               int64_t nblocks, void *__restrict__ out) {
    __shared__ uint32_t sgrid32[256 * 2];
    const uint8_t *sgrid = reinterpret_cast<const uint8_t *>(sgrid32);
    for (int i = threadIdx.x; i < 256 * 2; i += blockDim.x)
        sgrid32[i] = reinterpret_cast<const uint32_t *>(grid)[i];
    __syncthreads();
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= nblocks * 8) return;
    int64_t b = gid >> 3;
    int g = (int)(gid & 7);
    const uint16_t *blk = reinterpret_cast<const uint16_t *>(blocks + 66 * b);
    float d = fp16_to_f32(blk[0]);
    const uint16_t *grp = blk + 1 + 4 * g;               // 8 bytes, 2-byte aligned
    uint32_t idxw = (uint32_t)grp[0] | ((uint32_t)grp[1] << 16);
    uint32_t a = (uint32_t)grp[2] | ((uint32_t)grp[3] << 16);
    float db = d * fmaf((float)(a >> 28), 0.25f, 0.125f);  // d*(0.5+s)/4, exact
    float v[32];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        uint32_t s7 = (a >> (7 * j)) & 0x7Fu;
        uint32_t sig = s7 | ((uint32_t)(__popc(s7) & 1) << 7);
        const uint8_t *row = sgrid + 8 * ((idxw >> (8 * j)) & 0xFFu);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            float m = db * (float)row[i];
            v[8 * j + i] = ((sig >> i) & 1u) ? -m : m;
        }
    }
    if (OUT_BF16) {
        uint4 *o = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + 256 * b + 32 * g);
#pragma unroll
        for (int q = 0; q < 4; q++) {
            uint32_t w[4];
#pragma unroll
            for (int p = 0; p < 4; p++)
                w[p] = f32_to_bf16_rne(v[8 * q + 2 * p]) | (f32_to_bf16_rne(v[8 * q + 2 * p + 1]) << 16);
            o[q] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    } else {
        float4 *o = reinterpret_cast<float4 *>(static_cast<float *>(out) + 256 * b + 32 * g);
#pragma unroll
        for (int q = 0; q < 8; q++) o[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
}

// One thread per (block, sub-block of 16 weights).
template <int OUT_BF16>
__global__ void __launch_bounds__(256)
k_dequant_q2k(const uint8_t *__restrict__ blocks, int64_t nblocks, void *__restrict__ out) {
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= nblocks * 16) return;
    int64_t b = gid >> 4;
    int sb = (int)(gid & 15);
    const uint8_t *blk = blocks + 84 * b;
    const uint32_t *w32 = reinterpret_cast<const uint32_t *>(blk);
    uint32_t dd = w32[20];                                  // bytes 80..83
    float d = fp16_to_f32(dd & 0xFFFFu), dmin = fp16_to_f32(dd >> 16);
    uint32_t scb = blk[sb];
    float dsc = d * (float)(scb & 15u);                     // exact
    float dm = dmin * (float)(scb >> 4);                    // exact
    int h = sb >> 3, j = (sb & 7) >> 1, l0 = 16 * (sb & 1);
    const uint32_t *q32 = reinterpret_cast<const uint32_t *>(blk + 16 + 32 * h + l0);
    float v[16];
#pragma unroll
    for (int w = 0; w < 4; w++) {
        uint32_t q = (q32[w] >> (2 * j)) & 0x03030303u;
#pragma unroll
        for (int i = 0; i < 4; i++) v[4 * w + i] = fmaf(dsc, (float)((q >> (8 * i)) & 3u), -dm);
    }
    if (OUT_BF16) {
        uint4 *o = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + 256 * b + 16 * sb);
#pragma unroll
        for (int q = 0; q < 2; q++) {
            uint32_t w[4];
#pragma unroll
            for (int p = 0; p < 4; p++)
                w[p] = f32_to_bf16_rne(v[8 * q + 2 * p]) | (f32_to_bf16_rne(v[8 * q + 2 * p + 1]) << 16);
            o[q] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    } else {
        float4 *o = reinterpret_cast<float4 *>(static_cast<float *>(out) + 256 * b + 16 * sb);
#pragma unroll
        for (int q = 0; q < 4; q++) o[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
}

// One canonical IQ2X group (4 index bytes, u32 of 4 x 7 sign bits and the
// 4-bit scale) -> the two words of the tiled layout: per run its index
// byte, then its 7 sign bits with one scale bit on top (see common.h).
BM_DEV uint2 iq2x_group_fields(uint32_t idxw, uint32_t a) {
    uint32_t r[4];
#pragma unroll
    for (int j = 0; j < 4; j++)
        r[j] = ((idxw >> (8 * j)) & 0xFFu) | (((a >> (7 * j)) & 0x7Fu) << 8) | (((a >> (28 + j)) & 1u) << 15);
    return make_uint2(r[0] | (r[1] << 16), r[2] | (r[3] << 16));
}

// canonical IQ2X -> tiled; one thread per block
__global__ void __launch_bounds__(256)
k_pack_iq2x(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int E, int N, int nb) {
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t per_e = (int64_t)N * nb;
    if (gid >= per_e * E) return;
    int64_t e = gid / per_e, rem = gid % per_e;
    int n = (int)(rem / nb), kb = (int)(rem % nb);
    int P = n >> 6, r = n & 63;
    const uint16_t *s = reinterpret_cast<const uint16_t *>(src + 66 * gid);
    uint8_t *slab = dst + e * per_e * 66;
    int64_t pk = (int64_t)P * nb + kb;
#pragma unroll
    for (int c = 0; c < 4; c++) {
        uint2 f[2];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int g = 2 * c + h;                         // group; its 8 bytes at 2 + 8g
            uint32_t idxw = (uint32_t)s[1 + 4 * g] | ((uint32_t)s[2 + 4 * g] << 16);
            uint32_t a = (uint32_t)s[3 + 4 * g] | ((uint32_t)s[4 + 4 * g] << 16);
            f[h] = iq2x_group_fields(idxw, a);
        }
        reinterpret_cast<uint4 *>(slab)[(pk * 4 + c) * 64 + r] = make_uint4(f[0].x, f[0].y, f[1].x, f[1].y);
    }
    reinterpret_cast<uint16_t *>(slab + 64 * per_e)[pk * 64 + r] = s[0];
}

// canonical Q2K -> tiled; one thread per block
__global__ void __launch_bounds__(256)
k_pack_q2k(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int E, int N, int nb) {
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t per_e = (int64_t)N * nb;
    if (gid >= per_e * E) return;
    int64_t e = gid / per_e, rem = gid % per_e;
    int n = (int)(rem / nb), kb = (int)(rem % nb);
    int P = n >> 6, r = n & 63;
    const uint32_t *s = reinterpret_cast<const uint32_t *>(src + 84 * gid);
    const uint8_t *qs = src + 84 * gid + 16;
    uint8_t *slab = dst + e * per_e * 84;
    int64_t pk = (int64_t)P * nb + kb;
    // sub-block b = 8h + 2j + lh holds weights l = 16 lh .. 16 lh + 15 of
    // plane j of half h: q = (qs[32h + l] >> 2j) & 3; weight t of the
    // sub-block goes to bits 8 ((t & 7) >> 1) + 4 (t & 1) + 2 (t >> 3)
    uint32_t W[16];
#pragma unroll
    for (int b = 0; b < 16; b++) {
        const int h = b >> 3, j = (b >> 1) & 3, lh = b & 1;
        uint32_t w = 0;
#pragma unroll
        for (int t = 0; t < 16; t++) {
            const uint32_t q = (qs[32 * h + 16 * lh + t] >> (2 * j)) & 3u;
            w |= q << q2k_word_shift(t);
        }
        W[b] = w;
    }
#pragma unroll
    for (int c = 0; c < 4; c++)
        reinterpret_cast<uint4 *>(slab)[(pk * 4 + c) * 64 + r] =
            make_uint4(W[4 * c], W[4 * c + 1], W[4 * c + 2], W[4 * c + 3]);
    reinterpret_cast<uint4 *>(slab + 64 * per_e)[pk * 64 + r] = make_uint4(s[0], s[1], s[2], s[3]);
    reinterpret_cast<uint32_t *>(slab + 80 * per_e)[pk * 64 + r] = s[20];
}

// One thread per canonical MXFP4 block (17 bytes, no alignment).  The
// gfx950 scaled conversion turns each byte's two elements (weights j and
// j+16 of the block) into element * 2^(X-127), exactly (fp32), or rounded
// to nearest-even (bf16), from the E8M0 scale in the exponent field of its
// scale operand; the FFN kernels use the same conversion.
template <int OUT_BF16>
__global__ void __launch_bounds__(256)
k_dequant_mxfp4(const uint8_t *__restrict__ blocks, int64_t nblocks, void *__restrict__ out) {
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblocks) return;
    const uint8_t *blk = blocks + 17 * b;
    const float sc = mx_cvt_scale(blk[0]);
    uint32_t q[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
        q[i] = (uint32_t)blk[1 + 4 * i] | ((uint32_t)blk[2 + 4 * i] << 8) | ((uint32_t)blk[3 + 4 * i] << 16) |
               ((uint32_t)blk[4 + 4 * i] << 24);
    if (OUT_BF16) {
        uint32_t lo[8], hi[8];          // bf16 bits of weights 0..15 and 16..31
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t p[4] = {fp4x2_bf16s<0>(q[i], sc), fp4x2_bf16s<1>(q[i], sc), fp4x2_bf16s<2>(q[i], sc),
                                   fp4x2_bf16s<3>(q[i], sc)};
            lo[2 * i] = (p[0] & 0xFFFFu) | (p[1] << 16);
            lo[2 * i + 1] = (p[2] & 0xFFFFu) | (p[3] << 16);
            hi[2 * i] = (p[0] >> 16) | (p[1] & 0xFFFF0000u);
            hi[2 * i + 1] = (p[2] >> 16) | (p[3] & 0xFFFF0000u);
        }
        uint4 *o = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + 32 * b);
        o[0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        o[1] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
        o[2] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        o[3] = make_uint4(hi[4], hi[5], hi[6], hi[7]);
    } else {
        float v[32];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float2 p[4] = {fp4x2_f32s<0>(q[i], sc), fp4x2_f32s<1>(q[i], sc), fp4x2_f32s<2>(q[i], sc),
                                 fp4x2_f32s<3>(q[i], sc)};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                v[4 * i + j] = p[j].x;
                v[16 + 4 * i + j] = p[j].y;
            }
        }
        float4 *o = reinterpret_cast<float4 *>(static_cast<float *>(out) + 32 * b);
#pragma unroll
        for (int q4 = 0; q4 < 8; q4++) o[q4] = make_float4(v[4 * q4], v[4 * q4 + 1], v[4 * q4 + 2], v[4 * q4 + 3]);
    }
}

// canonical MXFP4 -> tiled; one thread per block (n, 32-weight block kc):
// its 16 element bytes re-paired so that byte i holds weights 2i, 2i+1,
// its scale byte into the row's 8 scales of the 256-weight chunk
__global__ void __launch_bounds__(256)
k_pack_mxfp4(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int E, int N, int nb) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_e = (int64_t)N * nb * 8;
    if (gid >= per_e * E) return;
    const int64_t e = gid / per_e, rem = gid % per_e;
    const int n = (int)(rem / (8 * nb)), kc = (int)(rem % (8 * nb)), kb = kc >> 3, c = kc & 7;
    const int P = n >> 6, r = n & 63;
    const uint8_t *s = src + 17 * gid;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; i++) {
        // weights 2i and 2i+1: element j sits in qs[j % 16], high nibble if j >= 16
        const int j0 = 2 * i, j1 = 2 * i + 1;
        const uint32_t e0 = j0 < 16 ? (s[1 + j0] & 15u) : (s[1 + j0 - 16] >> 4);
        const uint32_t e1 = j1 < 16 ? (s[1 + j1] & 15u) : (s[1 + j1 - 16] >> 4);
        w[i >> 2] |= (e0 | (e1 << 4)) << (8 * (i & 3));
    }
    uint8_t *slab = dst + e * per_e * 17;
    const int64_t pk = (int64_t)P * nb + kb;
    reinterpret_cast<uint4 *>(slab)[(pk * 8 + c) * 64 + r] = make_uint4(w[0], w[1], w[2], w[3]);
    slab[per_e * 16 + (pk * 64 + r) * 8 + c] = s[0];
}

// row-major bf16 [N][K] -> tiled; one thread per 8-value piece
__global__ void __launch_bounds__(256)
k_pack_bf16(const uint4 *__restrict__ src, uint4 *__restrict__ dst, int N, int K8) {
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (int64_t)N * K8) return;
    int n = (int)(gid / K8), c = (int)(gid % K8);
    dst[((int64_t)(n >> 6) * K8 + c) * 64 + (n & 63)] = src[gid];
}

inline unsigned grid_for(int64_t n, int bs) { return (unsigned)((n + bs - 1) / bs); }

}  // namespace

namespace bm_host {

int launch_dequant_iq2x(const void *blocks, const void *grid, int64_t nblocks, void *out,
                        int out_dtype, hipStream_t s) {
    unsigned g = grid_for(nblocks * 8, 256);
    if (out_dtype == BITMOE_BF16)
        k_dequant_iq2x<1><<<g, 256, 0, s>>>((const uint8_t *)blocks, (const uint8_t *)grid, nblocks, out);
    else
        k_dequant_iq2x<0><<<g, 256, 0, s>>>((const uint8_t *)blocks, (const uint8_t *)grid, nblocks, out);
    BM_LAUNCH_CHECK();
    return BITMOE_OK;
}

int launch_dequant_q2k(const void *blocks, int64_t nblocks, void *out, int out_dtype, hipStream_t s) {
    unsigned g = grid_for(nblocks * 16, 256);
    if (out_dtype == BITMOE_BF16)
        k_dequant_q2k<1><<<g, 256, 0, s>>>((const uint8_t *)blocks, nblocks, out);
    else
        k_dequant_q2k<0><<<g, 256, 0, s>>>((const uint8_t *)blocks, nblocks, out);
    BM_LAUNCH_CHECK();
    return BITMOE_OK;
}

int launch_pack_iq2x(const void *src, void *dst, int E, int N, int K, hipStream_t s) {
    int64_t n = (int64_t)E * N * (K / 256);
    k_pack_iq2x<<<grid_for(n, 256), 256, 0, s>>>((const uint8_t *)src, (uint8_t *)dst, E, N, K / 256);
    BM_LAUNCH_CHECK();
    return BITMOE_OK;
}

int launch_pack_q2k(const void *src, void *dst, int E, int N, int K, hipStream_t s) {
    int64_t n = (int64_t)E * N * (K / 256);
    k_pack_q2k<<<grid_for(n, 256), 256, 0, s>>>((const uint8_t *)src, (uint8_t *)dst, E, N, K / 256);
    BM_LAUNCH_CHECK();
    return BITMOE_OK;
}

int launch_dequant_mxfp4(const void *blocks, int64_t nblocks, void *out, int out_dtype, hipStream_t s) {
    unsigned g = grid_for(nblocks, 256);
    if (out_dtype == BITMOE_BF16)
        k_dequant_mxfp4<1><<<g, 256, 0, s>>>((const uint8_t *)blocks, nblocks, out);
    else
        k_dequant_mxfp4<0><<<g, 256, 0, s>>>((const uint8_t *)blocks, nblocks, out);
    BM_LAUNCH_CHECK();
    return BITMOE_OK;
}

int launch_pack_mxfp4(const void *src, void *dst, int E, int N, int K, hipStream_t s) {
    int64_t n = (int64_t)E * N * (K / 32);
    k_pack_mxfp4<<<grid_for(n, 256), 256, 0, s>>>((const uint8_t *)src, (uint8_t *)dst, E, N, K / 256);
    BM_LAUNCH_CHECK();
    return BITMOE_OK;
}

int launch_pack_bf16(const void *src, void *dst, int N, int K, hipStream_t s) {
    int64_t n = (int64_t)N * (K / 8);
    k_pack_bf16<<<grid_for(n, 256), 256, 0, s>>>((const uint4 *)src, (uint4 *)dst, N, K / 8);
    BM_LAUNCH_CHECK();
    return BITMOE_OK;
}

}  // namespace bm_host
