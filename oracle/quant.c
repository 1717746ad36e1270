/*
 * CPU oracle of the quantizer round trip: fp32 weights -> canonical IQ2X,
 * Q2K and MXFP4 blocks by an error-minimising search.
 *
 * TEST INFRASTRUCTURE ONLY, like oracle.c: only the tests, the smoke check
 * and the CPU-baseline leg of the benchmark use it.  It shares no code with
 * the HIP encoder.
 *
 * What the pages say: the routed experts are quantised asymmetrically to
 * 2 bits, up/gate in IQ2_XXS and down in Q2_K ("antirez/ds4 - Moteur local
 * d'inference DeepSeek V4 Flash pour Metal", section "Poids du modele"),
 * with an importance matrix ("ds4 : un MoE de 284 milliards sur un Mac de
 * 128 Go", section "Comment un 284B tient en memoire").  They give no
 * algorithm and no calibration data is available here, so the encoder below
 * is this build's reading: an unweighted squared-error search over the
 * format's own choices, in the format definitions of oracle.c.
 *
 * Arithmetic.  Every decision is taken in double precision with each
 * operation written out (this file is built with -ffp-contract=off), in the
 * order given in the comments; "rint" is round half to even, "fp16(x)" the
 * binary16 value nearest to x >= 0 (ties to even), never above 65504.  The
 * HIP encoder takes the same decisions in the same order, which is what
 * makes the bytes comparable bit for bit.
 *
 * IQ2X superblock (256 weights w, 8 groups of 32, 4 runs of 8 per group):
 *   d = fp16(max|w| / 27.125)              (27.125 = (0.5 + 15) / 4 * 7: the
 *                                           largest scale times the largest
 *                                           codebook magnitude)
 *   for each group, each scale s = 0..15: db = d * (0.5 + s) * 0.25 and, for
 *   each run, the codebook row r minimising
 *       E(r) = sum_i (|w_i| - db * g[r][i])^2             (i = 0..7 in order)
 *              + (odd number of w_i < 0 ? min_i 4 |w_i| db g[r][i] : 0)
 *   (the eighth sign is the parity of the other seven, so a run with an odd
 *   number of negative weights flips the sign of the element where that
 *   costs least; 4|w| db g is the squared-error increase of that flip);
 *   ties go to the lower row.  The group keeps the scale whose summed run
 *   errors (runs 0..3 in order) are least, ties to the lower scale; each run
 *   stores its row and its signs (negative weights, plus the flip: the
 *   element with the least penalty, ties to the lower index).
 *   d = 0 (an all-zero superblock) stores zero bytes and d = 0.
 *
 * Q2K superblock (256 weights, 16 sub-blocks of 16):
 *   per sub-block: lo, hi = min, max of w; m = lo < 0 ? -lo : 0;
 *                  a = hi + m > 0 ? (hi + m) / 3 : 0
 *   d = fp16(max a / 15), dmin = fp16(max m / 15)
 *   per sub-block: cs = clamp(rint(a / d), 0, 15) (0 if d = 0),
 *                  cm = clamp(rint(m / dmin), 0, 15) (0 if dmin = 0);
 *                  over cs' = cs-1..cs+1 and cm' = cm-1..cm+1 within 0..15
 *                  (cs' outer, ascending): A = d cs', M = dmin cm',
 *                  q_j = A > 0 ? clamp(rint((w_j + M) / A), 0, 3) : 0,
 *                  E = sum_j (w_j - (A q_j - M))^2 (j in order);
 *                  the least E wins, ties to the earlier candidate.
 *
 * MXFP4 block (32 weights, OCP Microscaling conversion with a two-way scale
 * search):
 *   amax = max |w|; amax = 0 stores zero bytes (scale byte 0, codes 0).
 *   e0 = floor(log2 amax) - 2 (2 = the largest E2M1 exponent, as the OCP
 *   conversion sets the shared exponent); for e = e0, e0 + 1 (each clamped to
 *   -127..127): t_j = |w_j| / 2^e, the E2M1 magnitude nearest t_j among 0,
 *   0.5, 1, 1.5, 2, 3, 4, 6 (t_j > 6 saturates to 6; a tie goes to the one
 *   with an even mantissa bit: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2,
 *   2.5 -> 2, 3.5 -> 4, 5 -> 4), E = sum_j (w_j - sign(w_j) m_j 2^e)^2 (j in
 *   order); the least E wins, ties to e0.  Code = magnitude code, plus 8 for a
 *   negative weight with a nonzero magnitude; byte 0 = e + 127.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* binary16 value nearest to x (x >= 0, finite), ties to even, at most 65504 */
static double fp16_round(double x)
{
    if (!(x > 0.0))
        return 0.0;
    double r;
    int e = ilogb(x);
    if (e < -14)
        r = ldexp(rint(ldexp(x, 24)), -24);           /* subnormal grid 2^-24 */
    else
        r = ldexp(rint(ldexp(x, 10 - e)), e - 10);    /* 11 significant bits */
    return r > 65504.0 ? 65504.0 : r;
}

/* binary16 bit pattern of a value fp16_round returned */
static uint16_t fp16_bits(double v)
{
    if (v == 0.0)
        return 0;
    if (v < ldexp(1.0, -14))
        return (uint16_t)ldexp(v, 24);
    int e = ilogb(v);
    int mant = (int)(ldexp(v, 10 - e) - 1024.0);
    return (uint16_t)(((e + 15) << 10) | mant);
}

static void put16(uint8_t *p, uint16_t v)
{
    p[0] = (uint8_t)v;
    p[1] = (uint8_t)(v >> 8);
}

static void iq2x_encode_block(const float *w, const uint8_t *grid, uint8_t *blk)
{
    memset(blk, 0, 66);
    double amax = 0.0;
    for (int i = 0; i < 256; i++) {
        double a = fabs((double)w[i]);
        if (a > amax)
            amax = a;
    }
    double d = fp16_round(amax / 27.125);
    put16(blk, fp16_bits(d));
    if (d == 0.0)
        return;
    for (int g = 0; g < 8; g++) {
        const float *wg = w + 32 * g;
        double best_total = 0.0;
        int best_s = -1, best_row[4] = {0, 0, 0, 0};
        unsigned best_sign[4] = {0, 0, 0, 0};
        for (int s = 0; s < 16; s++) {
            double db = d * (0.5 + s) * 0.25;
            double total = 0.0;
            int row[4];
            unsigned sign[4];
            for (int j = 0; j < 4; j++) {
                const float *wr = wg + 8 * j;
                unsigned neg = 0;
                for (int i = 0; i < 8; i++)
                    if (wr[i] < 0.0f)
                        neg |= 1u << i;
                int odd = 0;
                for (int i = 0; i < 8; i++)
                    odd ^= (neg >> i) & 1;
                double best_e = 0.0;
                int best_r = -1;
                unsigned best_sg = 0;
                for (int r = 0; r < 256; r++) {
                    const uint8_t *gr = grid + 8 * r;
                    double e = 0.0;
                    for (int i = 0; i < 8; i++) {
                        double diff = fabs((double)wr[i]) - db * (double)gr[i];
                        e = e + diff * diff;
                    }
                    unsigned sg = neg;
                    if (odd) {
                        double pmin = 0.0;
                        int imin = -1;
                        for (int i = 0; i < 8; i++) {
                            double pen = 4.0 * fabs((double)wr[i]) * db * (double)gr[i];
                            if (imin < 0 || pen < pmin) {
                                pmin = pen;
                                imin = i;
                            }
                        }
                        e = e + pmin;
                        sg = neg ^ (1u << imin);
                    }
                    if (best_r < 0 || e < best_e) {
                        best_e = e;
                        best_r = r;
                        best_sg = sg;
                    }
                }
                total = total + best_e;
                row[j] = best_r;
                sign[j] = best_sg;
            }
            if (best_s < 0 || total < best_total) {
                best_total = total;
                best_s = s;
                for (int j = 0; j < 4; j++) {
                    best_row[j] = row[j];
                    best_sign[j] = sign[j];
                }
            }
        }
        uint8_t *grp = blk + 2 + 8 * g;
        uint32_t a = (uint32_t)best_s << 28;
        for (int j = 0; j < 4; j++) {
            grp[j] = (uint8_t)best_row[j];
            a |= (best_sign[j] & 0x7Fu) << (7 * j);   /* bit 7 is the parity */
        }
        grp[4] = (uint8_t)a;
        grp[5] = (uint8_t)(a >> 8);
        grp[6] = (uint8_t)(a >> 16);
        grp[7] = (uint8_t)(a >> 24);
    }
}

static int clampi(int v, int lo, int hi)
{
    return v < lo ? lo : v > hi ? hi : v;
}

static void q2k_encode_block(const float *w, uint8_t *blk)
{
    memset(blk, 0, 84);
    double a[16], m[16], amax = 0.0, mmax = 0.0;
    for (int b = 0; b < 16; b++) {
        double lo = (double)w[16 * b], hi = lo;
        for (int j = 1; j < 16; j++) {
            double v = (double)w[16 * b + j];
            if (v < lo) lo = v;
            if (v > hi) hi = v;
        }
        m[b] = lo < 0.0 ? -lo : 0.0;
        a[b] = hi + m[b] > 0.0 ? (hi + m[b]) / 3.0 : 0.0;
        if (a[b] > amax) amax = a[b];
        if (m[b] > mmax) mmax = m[b];
    }
    double d = fp16_round(amax / 15.0), dmin = fp16_round(mmax / 15.0);
    put16(blk + 80, fp16_bits(d));
    put16(blk + 82, fp16_bits(dmin));
    for (int b = 0; b < 16; b++) {
        int cs = d > 0.0 ? clampi((int)rint(a[b] / d), 0, 15) : 0;
        int cm = dmin > 0.0 ? clampi((int)rint(m[b] / dmin), 0, 15) : 0;
        double best_e = 0.0;
        int found = 0, bs = 0, bm = 0, bq[16];
        for (int s2 = cs - 1; s2 <= cs + 1; s2++) {
            if (s2 < 0 || s2 > 15) continue;
            for (int m2 = cm - 1; m2 <= cm + 1; m2++) {
                if (m2 < 0 || m2 > 15) continue;
                double A = d * s2, M = dmin * m2, e = 0.0;
                int q[16];
                for (int j = 0; j < 16; j++) {
                    double wj = (double)w[16 * b + j];
                    q[j] = A > 0.0 ? clampi((int)rint((wj + M) / A), 0, 3) : 0;
                    double diff = wj - (A * q[j] - M);
                    e = e + diff * diff;
                }
                if (!found || e < best_e) {
                    found = 1;
                    best_e = e;
                    bs = s2;
                    bm = m2;
                    memcpy(bq, q, sizeof q);
                }
            }
        }
        blk[b] = (uint8_t)(bs | (bm << 4));
        for (int j = 0; j < 16; j++) {
            int i = 16 * b + j;                        /* weight index in the superblock */
            int h = i / 128, r = i % 128, sh = r / 32, l = r % 32;
            blk[16 + 32 * h + l] |= (uint8_t)(bq[j] << (2 * sh));
        }
    }
}

/* E2M1 magnitude code nearest t >= 0 (ties to the even mantissa bit) */
static int e2m1_code(double t)
{
    if (t <= 0.25) return 0;
    if (t < 0.75) return 1;
    if (t <= 1.25) return 2;
    if (t < 1.75) return 3;
    if (t <= 2.5) return 4;
    if (t < 3.5) return 5;
    if (t <= 5.0) return 6;
    return 7;
}

static const double e2m1_mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

static void mxfp4_encode_block(const float *w, uint8_t *blk)
{
    memset(blk, 0, 17);
    double amax = 0.0;
    for (int j = 0; j < 32; j++) {
        double a = fabs((double)w[j]);
        if (a > amax)
            amax = a;
    }
    if (amax == 0.0)
        return;
    int fe;
    frexp(amax, &fe);                              /* amax = f 2^fe, f in [0.5, 1) */
    int e0 = fe - 1 - 2;
    int best_e = 0, found = 0;
    double best_err = 0.0;
    for (int e = e0; e <= e0 + 1; e++) {
        int ec = e < -127 ? -127 : e > 127 ? 127 : e;
        double s = ldexp(1.0, ec), err = 0.0;
        for (int j = 0; j < 32; j++) {
            double m = e2m1_mag[e2m1_code(fabs((double)w[j]) / s)] * s;
            double diff = fabs((double)w[j]) - m;
            err = err + diff * diff;
        }
        if (!found || err < best_err) {
            found = 1;
            best_err = err;
            best_e = ec;
        }
    }
    double s = ldexp(1.0, best_e);
    blk[0] = (uint8_t)(best_e + 127);
    for (int j = 0; j < 32; j++) {
        int c = e2m1_code(fabs((double)w[j]) / s);
        if (c && w[j] < 0.0f)
            c |= 8;
        if (j < 16)
            blk[1 + j] |= (uint8_t)c;
        else
            blk[1 + j - 16] |= (uint8_t)(c << 4);
    }
}

void oracle_quantize_mxfp4(const float *w, int64_t nblocks, uint8_t *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblocks; b++)
        mxfp4_encode_block(w + 32 * b, out + 17 * b);
}

/* nblocks superblocks of 256 fp32 weights -> canonical blocks (66 or 84
 * bytes each); OpenMP over superblocks (independent). */
void oracle_quantize_iq2x(const float *w, const uint8_t *grid, int64_t nblocks, uint8_t *out)
{
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t b = 0; b < nblocks; b++)
        iq2x_encode_block(w + 256 * b, grid, out + 66 * b);
}

void oracle_quantize_q2k(const float *w, int64_t nblocks, uint8_t *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblocks; b++)
        q2k_encode_block(w + 256 * b, out + 84 * b);
}
