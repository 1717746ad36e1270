// Quantizer: fp32 weights -> canonical IQ2X, Q2K and MXFP4 blocks by an
// error-minimising search over each format's own choices.
//
// The pages say the routed experts are quantised asymmetrically to 2 bits,
// up/gate in IQ2_XXS and down in Q2_K ("antirez/ds4 - Moteur local
// d'inference DeepSeek V4 Flash pour Metal", section "Poids du modele"),
// with an importance matrix ("ds4 : un MoE de 284 milliards sur un Mac de
// 128 Go", section "Comment un 284B tient en memoire"); they give no
// algorithm.  The search here minimises the plain squared error (no
// calibration data exists to weight it):
//  IQ2X (per superblock): d = fp16(max|w| / 27.125); per group of 32, the
//   group scale s in 0..15 and, per run of 8, the codebook row whose
//   magnitudes d (0.5 + s) / 4 * g are closest to |w| (squared error), the
//   signs those of w except that a run with an odd number of negative
//   weights flips the element where that costs least (the eighth sign is
//   the parity of the stored seven); ties to the lower row, scale, element.
//  Q2K (per superblock): per sub-block of 16 the min m = max(0, -min w) and
//   range a = (max w + m) / 3; d = fp16(max a / 15), dmin = fp16(max m / 15);
//   per sub-block the best of the 3 x 3 (scale, min) codes around
//   rint(a / d), rint(m / dmin), with quants clamp(rint((w + M) / A), 0, 3).
// Every decision is taken in double precision with no fused operations (the
// pragma below), sums in element order, so that the bytes are a function of
// the input alone: a reference implementation that keeps that order gets
// the same bytes.
#pragma clang fp contract(off)

#include "common.h"

namespace {

using namespace bm;

// binary16 value nearest to x >= 0 (ties to even), at most 65504
BM_DEV double fp16_round(double x) {
    if (!(x > 0.0)) return 0.0;
    const int e = ilogb(x);
    const double r = e < -14 ? ldexp(rint(ldexp(x, 24)), -24) : ldexp(rint(ldexp(x, 10 - e)), e - 10);
    return r > 65504.0 ? 65504.0 : r;
}
// bit pattern of a value fp16_round returned
BM_DEV uint32_t fp16_pattern(double v) {
    if (v == 0.0) return 0u;
    if (v < 0x1p-14) return (uint32_t)ldexp(v, 24);
    const int e = ilogb(v);
    return (uint32_t)((e + 15) << 10) | (uint32_t)(ldexp(v, 10 - e) - 1024.0);
}

// (error, row) of the wave's lanes -> the least error, ties to the lower row
BM_DEV void wave_argmin(double &e, int &r) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const double e2 = __shfl_xor(e, o, kWave);
        const int r2 = __shfl_xor(r, o, kWave);
        if (e2 < e || (e2 == e && r2 < r)) {
            e = e2;
            r = r2;
        }
    }
}

// One IQ2X superblock per wave; lane l evaluates codebook rows l, l+64,
// l+128, l+192 (in that order, so its first minimum is its lowest row).
__global__ void __launch_bounds__(256)
k_quant_iq2x(const float *__restrict__ w, const uint8_t *__restrict__ grid, int64_t nblocks,
             uint8_t *__restrict__ out) {
    const int lane = lane_id();
    const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= nblocks) return;
    const float *wb = w + blk * 256;
    // this lane's four codebook rows (8 magnitudes each, as bytes)
    uint2 g[4];
#pragma unroll
    for (int q = 0; q < 4; q++) g[q] = *reinterpret_cast<const uint2 *>(grid + 8 * (lane + 64 * q));
    auto mag = [&](int q, int i) {
        return (double)(((i < 4 ? g[q].x : g[q].y) >> (8 * (i & 3))) & 0xFFu);
    };
    const float4 v4 = reinterpret_cast<const float4 *>(wb)[lane];
    float am = fmaxf(fmaxf(fabsf(v4.x), fabsf(v4.y)), fmaxf(fabsf(v4.z), fabsf(v4.w)));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, kWave));
    const double d = fp16_round((double)am / 27.125);
    uint8_t *ob = out + blk * 66;
    const uint32_t dbits = fp16_pattern(d);
    if (d == 0.0) {                      // an all-zero superblock: zero bytes
        ob[lane] = 0;
        if (lane < 2) ob[64 + lane] = 0;
        return;
    }
    if (lane < 2) ob[lane] = (uint8_t)(dbits >> (8 * lane));
    for (int grp = 0; grp < 8; grp++) {
        // the group's 32 |weights| (identical in every lane), widened to
        // double where used (exact)
        float aw[32];
        unsigned neg[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 32; i++) {
            const float x = wb[32 * grp + i];
            aw[i] = fabsf(x);
            if (x < 0.0f) neg[i >> 3] |= 1u << (i & 7);
        }
        double best_total = 0.0;
        int best_s = -1, best_row[4] = {0, 0, 0, 0};
        unsigned best_sign[4] = {0u, 0u, 0u, 0u};
        for (int s = 0; s < 16; s++) {
            const double db = d * (0.5 + s) * 0.25;
            double total = 0.0;
            int row[4];
            unsigned sign[4];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const bool odd = __popc(neg[j]) & 1;
                double be = 0.0;
                int br = -1, bflip = 0;
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    double e = 0.0;
#pragma unroll
                    for (int i = 0; i < 8; i++) {
                        const double diff = (double)aw[8 * j + i] - db * mag(q, i);
                        e = e + diff * diff;
                    }
                    int flip = 0;
                    if (odd) {
                        double pmin = 0.0;
#pragma unroll
                        for (int i = 0; i < 8; i++) {
                            const double pen = 4.0 * (double)aw[8 * j + i] * db * mag(q, i);
                            if (i == 0 || pen < pmin) {
                                pmin = pen;
                                flip = i;
                            }
                        }
                        e = e + pmin;
                    }
                    if (br < 0 || e < be) {
                        be = e;
                        br = lane + 64 * q;
                        bflip = flip;
                    }
                }
                int r = br;
                double e = be;
                wave_argmin(e, r);
                // the signs: the winning lane's flip
                const int owner = r & 63;
                const int flip = __shfl(bflip, owner, kWave);
                total = total + e;
                row[j] = r;
                sign[j] = odd ? neg[j] ^ (1u << flip) : neg[j];
            }
            if (best_s < 0 || total < best_total) {
                best_total = total;
                best_s = s;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    best_row[j] = row[j];
                    best_sign[j] = sign[j];
                }
            }
        }
        uint32_t a = (uint32_t)best_s << 28;
#pragma unroll
        for (int j = 0; j < 4; j++) a |= (best_sign[j] & 0x7Fu) << (7 * j);
        uint8_t *gp = ob + 2 + 8 * grp;
        if (lane < 4) gp[lane] = (uint8_t)(lane == 0 ? best_row[0] : lane == 1 ? best_row[1] : lane == 2 ? best_row[2]
                                                                                             : best_row[3]);
        else if (lane < 8) gp[lane] = (uint8_t)(a >> (8 * (lane - 4)));
    }
}

// Q2K: one lane per sub-block, four superblocks per wave (16 lanes each).
__global__ void __launch_bounds__(256)
k_quant_q2k(const float *__restrict__ w, int64_t nblocks, uint8_t *__restrict__ out) {
    __shared__ uint32_t qsw[16][16];                  // per superblock of the workgroup: 64 quant bytes
    const int lane = lane_id(), sbl = threadIdx.x >> 4, b = threadIdx.x & 15;
    const int64_t blk = (int64_t)blockIdx.x * 16 + sbl;
    const bool live = blk < nblocks;
    qsw[sbl][b] = 0u;
    double a = 0.0, m = 0.0;
    float x[16];
    if (live) {
        const float4 *p = reinterpret_cast<const float4 *>(w + blk * 256 + 16 * b);
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const float4 v = p[q];
            x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
        }
        double lo = (double)x[0], hi = lo;
#pragma unroll
        for (int j = 1; j < 16; j++) {
            const double v = (double)x[j];
            if (v < lo) lo = v;
            if (v > hi) hi = v;
        }
        m = lo < 0.0 ? -lo : 0.0;
        a = hi + m > 0.0 ? (hi + m) / 3.0 : 0.0;
    }
    // maxima over the superblock's 16 lanes (a, m >= 0)
    double amax = a, mmax = m;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
        amax = fmax(amax, __shfl_xor(amax, o, kWave));
        mmax = fmax(mmax, __shfl_xor(mmax, o, kWave));
    }
    (void)lane;
    const double d = fp16_round(amax / 15.0), dmin = fp16_round(mmax / 15.0);
    __syncthreads();
    int bs = 0, bm = 0;
    if (live) {
        const int cs = d > 0.0 ? min(max((int)rint(a / d), 0), 15) : 0;
        const int cm = dmin > 0.0 ? min(max((int)rint(m / dmin), 0), 15) : 0;
        double best = 0.0;
        bool found = false;
        uint32_t bq = 0u;                               // quants j at bits 2j
        for (int s2 = cs - 1; s2 <= cs + 1; s2++) {
            if (s2 < 0 || s2 > 15) continue;
            for (int m2 = cm - 1; m2 <= cm + 1; m2++) {
                if (m2 < 0 || m2 > 15) continue;
                const double A = d * s2, M = dmin * m2;
                double e = 0.0;
                uint32_t qw = 0u;
#pragma unroll
                for (int j = 0; j < 16; j++) {
                    const double wj = (double)x[j];
                    const int q = A > 0.0 ? min(max((int)rint((wj + M) / A), 0), 3) : 0;
                    const double diff = wj - (A * q - M);
                    e = e + diff * diff;
                    qw |= (uint32_t)q << (2 * j);
                }
                if (!found || e < best) {
                    found = true;
                    best = e;
                    bs = s2;
                    bm = m2;
                    bq = qw;
                }
            }
        }
        // weight i = 16 b + j of the superblock sits in quant byte
        // 32 (i / 128) + i % 32 at bit 2 ((i % 128) / 32)
#pragma unroll
        for (int j = 0; j < 16; j++) {
            const int i = 16 * b + j, h = i >> 7, r = i & 127, sh = r >> 5, l = r & 31;
            const int byte = 32 * h + l;
            atomicOr(&qsw[sbl][byte >> 2], ((bq >> (2 * j)) & 3u) << (8 * (byte & 3) + 2 * sh));
        }
    }
    __syncthreads();
    if (!live) return;
    uint8_t *ob = out + blk * 84;
    ob[b] = (uint8_t)(bs | (bm << 4));
#pragma unroll
    for (int q = 0; q < 4; q++) ob[16 + 4 * b + q] = (uint8_t)(qsw[sbl][b] >> (8 * q));
    if (b == 0) {
        const uint32_t dd = fp16_pattern(d) | (fp16_pattern(dmin) << 16);
#pragma unroll
        for (int q = 0; q < 4; q++) ob[80 + q] = (uint8_t)(dd >> (8 * q));
    }
}

// MXFP4: one thread per 32-weight block.  The OCP Microscaling conversion's
// shared exponent e0 = floor(log2 max|w|) - 2 and the next one up are both
// tried (each clamped to -127..127); elements go to the nearest E2M1
// magnitude (ties to the even mantissa bit, saturating at 6), and the scale
// with the smaller squared error is kept (ties to e0).  All-zero blocks are
// zero bytes.
BM_DEV int e2m1_code(double t) {
    return t <= 0.25 ? 0 : t < 0.75 ? 1 : t <= 1.25 ? 2 : t < 1.75 ? 3 : t <= 2.5 ? 4 : t < 3.5 ? 5 : t <= 5.0 ? 6 : 7;
}
BM_DEV double e2m1_mag(int c) {
    return c == 0 ? 0.0 : c == 1 ? 0.5 : c == 2 ? 1.0 : c == 3 ? 1.5 : c == 4 ? 2.0 : c == 5 ? 3.0 : c == 6 ? 4.0 : 6.0;
}

__global__ void __launch_bounds__(256)
k_quant_mxfp4(const float *__restrict__ w, int64_t nblocks, uint8_t *__restrict__ out) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblocks) return;
    float x[32];
    const float4 *p = reinterpret_cast<const float4 *>(w + 32 * b);
#pragma unroll
    for (int q = 0; q < 8; q++) {
        const float4 v = p[q];
        x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
    }
    double amax = 0.0;
#pragma unroll
    for (int j = 0; j < 32; j++) amax = fmax(amax, fabs((double)x[j]));
    uint8_t *ob = out + 17 * b;
    if (amax == 0.0) {
#pragma unroll
        for (int j = 0; j < 17; j++) ob[j] = 0;
        return;
    }
    const int e0 = ilogb(amax) - 2;
    int best_e = 0;
    double best = 0.0;
    for (int e = e0; e <= e0 + 1; e++) {
        const int ec = min(max(e, -127), 127);
        const double s = ldexp(1.0, ec);
        double err = 0.0;
#pragma unroll
        for (int j = 0; j < 32; j++) {
            const double a = fabs((double)x[j]);
            const double diff = a - e2m1_mag(e2m1_code(a / s)) * s;
            err = err + diff * diff;
        }
        if (e == e0 || err < best) {
            best = err;
            best_e = ec;
        }
    }
    const double s = ldexp(1.0, best_e);
    uint32_t q[4] = {0u, 0u, 0u, 0u};                   // qs bytes 0..15: weight j low, j + 16 high
#pragma unroll
    for (int j = 0; j < 32; j++) {
        int c = e2m1_code(fabs((double)x[j]) / s);
        if (c && x[j] < 0.f) c |= 8;
        const int byte = j & 15;
        q[byte >> 2] |= (uint32_t)c << (8 * (byte & 3) + (j < 16 ? 0 : 4));
    }
    ob[0] = (uint8_t)(best_e + 127);
#pragma unroll
    for (int j = 0; j < 16; j++) ob[1 + j] = (uint8_t)(q[j >> 2] >> (8 * (j & 3)));
}

}  // namespace

namespace bm_host {

int launch_quant_mxfp4(const float *w, int64_t nblocks, void *out, hipStream_t s) {
    k_quant_mxfp4<<<(unsigned)((nblocks + 255) / 256), 256, 0, s>>>(w, nblocks, (uint8_t *)out);
    BM_LAUNCH_CHECK();
    return BITMOE_OK;
}

int launch_quant_iq2x(const float *w, const void *grid, int64_t nblocks, void *out, hipStream_t s) {
    const int64_t grid_n = (nblocks + 3) / 4;
    k_quant_iq2x<<<(unsigned)grid_n, 256, 0, s>>>(w, (const uint8_t *)grid, nblocks, (uint8_t *)out);
    BM_LAUNCH_CHECK();
    return BITMOE_OK;
}

int launch_quant_q2k(const float *w, int64_t nblocks, void *out, hipStream_t s) {
    const int64_t grid_n = (nblocks + 15) / 16;
    k_quant_q2k<<<(unsigned)grid_n, 256, 0, s>>>(w, nblocks, (uint8_t *)out);
    BM_LAUNCH_CHECK();
    return BITMOE_OK;
}

}  // namespace bm_host
