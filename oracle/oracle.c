/*
 * CPU oracle for the 2-bit routed-expert MoE feed-forward layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library path links, loads or calls
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header, table or constant with the HIP
 * library: it is the plain definition of what the layer computes, evaluated
 * slowly in double precision so that a reader can check it against the pages.
 *
 * What the layer is (sources, by page title and section):
 *  - "Un modele de 284 milliards de parametres tourne desormais sur un Mac de
 *    128 Go. Qui y perd ?", section "Comment un modele de 284 milliards de
 *    parametres tient sur une seule machine": a router chooses a few experts
 *    per token; most of the weights live in these routed experts.
 *  - "ds4 : analyse pratique pour un usage documente", section "Support de
 *    modeles et choix de quantification", and "antirez/ds4 - Moteur local
 *    d'inference DeepSeek V4 Flash pour Metal", section "Poids du modele":
 *    only the routed experts are quantised, up/gate as IQ2_XXS and down as
 *    Q2_K; shared experts, projections and the router stay unquantised.
 *  - same page 5, section "Remerciements a llama.cpp et GGML": the GGUF
 *    quantisation layouts and tables are GGML's, which fixes the readings of
 *    the byte order below (the synthetic codebook replaces GGML's table).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - IQ2X superblock, 66 bytes per 256 weights: fp16 d, then 8 groups of 8
 *    bytes: 4 codebook indices, then a little-endian u32 holding four 7-bit
 *    sign fields at bits 7j..7j+6 and the 4-bit group scale in bits 28..31.
 *    The eighth sign of each run of 8 is the even-parity bit of the seven
 *    stored ones; a set bit means negative.  Group scale db = d*(0.5+s)/4.
 *  - Q2K superblock, 84 bytes: 16 bytes of (scale | min<<4) for 16 sub-blocks
 *    of 16 weights, 64 bytes of 2-bit quants, fp16 d, fp16 dmin; weight i has
 *    quant (qs[32*(i/128) + i%32] >> 2*((i%128)/32)) & 3 and value
 *    d*scale*q - dmin*min of sub-block i/16.
 *  - FFN: y_t = sum_j w_tj * D_e (silu(G_e x_t) * (U_e x_t)) over the k routed
 *    slots (+ the shared expert with weight 1 when present), silu(z) =
 *    z/(1+exp(-z)); no biases, no extra routed scaling.
 *  - Routing: k largest logits (ties: lower expert index first), slots in
 *    descending-logit order, weights = softmax over the selected k.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* IEEE-754 binary16 -> double, straight from the encoding. */
double oracle_fp16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1F;
    int mant = h & 0x3FF;
    double v;
    if (expo == 0)
        v = ldexp((double)mant, -24);                 /* subnormal: m * 2^-24 */
    else if (expo == 31)
        v = mant ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + mant), expo - 25);  /* (1.m) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 bits -> double: the high half of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static int popcount7(unsigned v)
{
    int c = 0;
    for (int i = 0; i < 7; i++)
        c += (v >> i) & 1;
    return c;
}

/* Decode one IQ2X superblock into 256 values. */
static void iq2x_block(const uint8_t *blk, const uint8_t *grid, double *out)
{
    double d = oracle_fp16_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
    for (int g = 0; g < 8; g++) {
        const uint8_t *grp = blk + 2 + 8 * g;
        uint32_t a = (uint32_t)grp[4] | ((uint32_t)grp[5] << 8) |
                     ((uint32_t)grp[6] << 16) | ((uint32_t)grp[7] << 24);
        unsigned s = a >> 28;
        double db = d * (0.5 + s) * 0.25;
        for (int j = 0; j < 4; j++) {
            unsigned s7 = (a >> (7 * j)) & 0x7F;
            unsigned sigma = s7 | ((unsigned)(popcount7(s7) & 1) << 7);
            const uint8_t *row = grid + 8 * grp[j];
            for (int i = 0; i < 8; i++) {
                double sgn = ((sigma >> i) & 1) ? -1.0 : 1.0;
                out[32 * g + 8 * j + i] = db * (double)row[i] * sgn;
            }
        }
    }
}

/* Decode one Q2K superblock into 256 values. */
static void q2k_block(const uint8_t *blk, double *out)
{
    const uint8_t *scales = blk;
    const uint8_t *qs = blk + 16;
    double d = oracle_fp16_to_double((uint16_t)(blk[80] | (blk[81] << 8)));
    double dmin = oracle_fp16_to_double((uint16_t)(blk[82] | (blk[83] << 8)));
    for (int i = 0; i < 256; i++) {
        int h = i / 128, r = i % 128, j = r / 32, l = r % 32;
        int q = (qs[32 * h + l] >> (2 * j)) & 3;
        int b = i / 16;
        int sc = scales[b] & 0xF, m = scales[b] >> 4;
        out[i] = d * sc * q - dmin * m;
    }
}

/*
 * MXFP4 (OCP Microscaling format, FP4 E2M1 elements with one E8M0 scale per
 * 32): the format of the pages' MXFP4 variant, which keeps DeepSeek's
 * released FP4 expert weights ("ds4 : analyse pratique pour un usage
 * documente", section "Support de modeles et choix de quantification").
 * Block of 17 bytes per 32 consecutive weights of one row, GGML's order:
 * byte 0 the scale X (value 2^(X-127); X = 255 is NaN), bytes 1-16 qs:
 * weight j (0..15) in the low nibble of qs[j], weight j+16 in its high
 * nibble.  Element code c: sign c >> 3, exponent field (c >> 1) & 3,
 * mantissa bit c & 1; exponent field 0 gives m * 0.5, otherwise
 * 2^(e-1) * (1 + m/2): 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 */
static double e2m1(unsigned c)
{
    unsigned e = (c >> 1) & 3, m = c & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, (int)e - 1);
    return (c >> 3) ? -v : v;
}

static void mxfp4_block(const uint8_t *blk, double *out)
{
    double scale = blk[0] == 255 ? NAN : ldexp(1.0, (int)blk[0] - 127);
    for (int j = 0; j < 16; j++) {
        out[j] = e2m1(blk[1 + j] & 0xF) * scale;
        out[j + 16] = e2m1(blk[1 + j] >> 4) * scale;
    }
}

void oracle_dequant_mxfp4(const uint8_t *blocks, int64_t nblocks, double *out)
{
    for (int64_t b = 0; b < nblocks; b++)
        mxfp4_block(blocks + 17 * b, out + 32 * b);
}

void oracle_dequant_iq2x(const uint8_t *blocks, const uint8_t *grid,
                         int64_t nblocks, double *out)
{
    for (int64_t b = 0; b < nblocks; b++)
        iq2x_block(blocks + 66 * b, grid, out + 256 * b);
}

void oracle_dequant_q2k(const uint8_t *blocks, int64_t nblocks, double *out)
{
    for (int64_t b = 0; b < nblocks; b++)
        q2k_block(blocks + 84 * b, out + 256 * b);
}

/* x element as double; dtype 0 = fp32, 1 = bf16 bits. */
static double x_at(const void *x, int dtype, int64_t i)
{
    if (dtype == 0)
        return (double)((const float *)x)[i];
    return oracle_bf16_to_double(((const uint16_t *)x)[i]);
}

/* logits[t][e] = sum_h x[t][h] * Wr[e][h], Wr bf16 [E][H]. */
void oracle_router_logits(const void *x, int x_dtype, int T, int H,
                          const uint16_t *wr, int E, double *logits)
{
    #pragma omp parallel for schedule(static)
    for (int64_t te = 0; te < (int64_t)T * E; te++) {
        int64_t t = te / E, e = te % E;
        double acc = 0.0;
        for (int h = 0; h < H; h++)
            acc += x_at(x, x_dtype, t * H + h) *
                   oracle_bf16_to_double(wr[e * (int64_t)H + h]);
        logits[te] = acc;
    }
}

/* Top-k by (logit descending, index ascending); w = softmax over the k. */
void oracle_topk(const double *logits, int T, int E, int k,
                 int32_t *ids, double *w)
{
    char *taken = (char *)malloc(E > 0 ? (size_t)E : 1);
    for (int t = 0; t < T; t++) {
        const double *l = logits + (int64_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int e = 0; e < E; e++)
                if (!taken[e] && (best < 0 || l[e] > l[best]))
                    best = e;
            taken[best] = 1;
            ids[t * k + j] = best;
        }
        double lmax = l[ids[t * k]], z = 0.0;
        for (int j = 0; j < k; j++)
            z += exp(l[ids[t * k + j]] - lmax);
        for (int j = 0; j < k; j++)
            w[t * k + j] = exp(l[ids[t * k + j]] - lmax) / z;
    }
    free(taken);
}

/* counts[e] = number of (token, slot) pairs on expert e; offsets = exclusive
 * prefix sum (E+1 entries); perm lists pair indices p = t*k + j grouped by
 * expert, ascending p inside each expert. */
void oracle_bucket(const int32_t *ids, int T, int k, int E,
                   int32_t *counts, int32_t *offsets, int32_t *perm)
{
    for (int e = 0; e < E; e++)
        counts[e] = 0;
    for (int p = 0; p < T * k; p++)
        counts[ids[p]]++;
    offsets[0] = 0;
    for (int e = 0; e < E; e++)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = (int32_t *)calloc(E > 0 ? (size_t)E : 1, sizeof(int32_t));
    for (int p = 0; p < T * k; p++) {
        int e = ids[p];
        perm[offsets[e] + fill[e]++] = p;
    }
    free(fill);
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* out[n] = sum_k W[n][k] * v[k] for an IQ2X [N][K] matrix. */
static void matvec_iq2x(const uint8_t *m, const uint8_t *grid, int N, int K,
                        const double *v, double *out)
{
    int nb = K / 256;
    #pragma omp parallel for schedule(static)
    for (int n = 0; n < N; n++) {
        double row[256], acc = 0.0;
        for (int kb = 0; kb < nb; kb++) {
            iq2x_block(m + 66 * ((int64_t)n * nb + kb), grid, row);
            for (int i = 0; i < 256; i++)
                acc += row[i] * v[256 * kb + i];
        }
        out[n] = acc;
    }
}

static void matvec_q2k(const uint8_t *m, int N, int K, const double *v,
                       double *out)
{
    int nb = K / 256;
    #pragma omp parallel for schedule(static)
    for (int n = 0; n < N; n++) {
        double row[256], acc = 0.0;
        for (int kb = 0; kb < nb; kb++) {
            q2k_block(m + 84 * ((int64_t)n * nb + kb), row);
            for (int i = 0; i < 256; i++)
                acc += row[i] * v[256 * kb + i];
        }
        out[n] = acc;
    }
}

static void matvec_mxfp4(const uint8_t *m, int N, int K, const double *v,
                         double *out)
{
    int nb = K / 32;
    #pragma omp parallel for schedule(static)
    for (int n = 0; n < N; n++) {
        double row[32], acc = 0.0;
        for (int kb = 0; kb < nb; kb++) {
            mxfp4_block(m + 17 * ((int64_t)n * nb + kb), row);
            for (int i = 0; i < 32; i++)
                acc += row[i] * v[32 * kb + i];
        }
        out[n] = acc;
    }
}

static void matvec_bf16(const uint16_t *m, int N, int K, const double *v,
                        double *out)
{
    #pragma omp parallel for schedule(static)
    for (int n = 0; n < N; n++) {
        double acc = 0.0;
        for (int k = 0; k < K; k++)
            acc += oracle_bf16_to_double(m[(int64_t)n * K + k]) * v[k];
        out[n] = acc;
    }
}

/*
 * y[t][:] = sum_j w[t][j] * D_e(silu(G_e x_t) * U_e x_t)  (+ shared expert).
 *
 * gate/up/down: arrays of E pointers to each expert's canonical blocks
 * (gate/up: I rows of H/256 IQ2X blocks; down: H rows of I/256 Q2K blocks);
 * an expert no token uses may be NULL.  shared_*: bf16 bits [I][H], [I][H],
 * [H][I], or NULL for none.  y: double [T][H], overwritten.
 */
static void moe_ffn(int mx, int H, int I, int E, int k, const uint8_t *grid,
                    const uint8_t *const *gate, const uint8_t *const *up,
                    const uint8_t *const *down,
                    const uint16_t *shared_gate, const uint16_t *shared_up,
                    const uint16_t *shared_down,
                    const void *x, int x_dtype, int T,
                    const int32_t *ids, const double *w, double *y)
{
    double *xv = (double *)malloc(sizeof(double) * H);
    double *g = (double *)malloc(sizeof(double) * I);
    double *u = (double *)malloc(sizeof(double) * I);
    double *o = (double *)malloc(sizeof(double) * H);
    (void)E;
    for (int t = 0; t < T; t++) {
        double *yt = y + (int64_t)t * H;
        for (int h = 0; h < H; h++) {
            xv[h] = x_at(x, x_dtype, (int64_t)t * H + h);
            yt[h] = 0.0;
        }
        for (int j = 0; j < k; j++) {
            int e = ids[t * k + j];
            if (mx) {
                matvec_mxfp4(gate[e], I, H, xv, g);
                matvec_mxfp4(up[e], I, H, xv, u);
            } else {
                matvec_iq2x(gate[e], grid, I, H, xv, g);
                matvec_iq2x(up[e], grid, I, H, xv, u);
            }
            for (int n = 0; n < I; n++)
                g[n] = silu(g[n]) * u[n];
            if (mx)
                matvec_mxfp4(down[e], H, I, g, o);
            else
                matvec_q2k(down[e], H, I, g, o);
            for (int n = 0; n < H; n++)
                yt[n] += w[t * k + j] * o[n];
        }
        if (shared_gate) {
            matvec_bf16(shared_gate, I, H, xv, g);
            matvec_bf16(shared_up, I, H, xv, u);
            for (int n = 0; n < I; n++)
                g[n] = silu(g[n]) * u[n];
            matvec_bf16(shared_down, H, I, g, o);
            for (int n = 0; n < H; n++)
                yt[n] += o[n];
        }
    }
    free(xv); free(g); free(u); free(o);
}

/* Routed experts in IQ2X (gate, up) and Q2K (down). */
void oracle_moe_ffn(int H, int I, int E, int k, const uint8_t *grid,
                    const uint8_t *const *gate, const uint8_t *const *up,
                    const uint8_t *const *down,
                    const uint16_t *shared_gate, const uint16_t *shared_up,
                    const uint16_t *shared_down,
                    const void *x, int x_dtype, int T,
                    const int32_t *ids, const double *w, double *y)
{
    moe_ffn(0, H, I, E, k, grid, gate, up, down, shared_gate, shared_up,
            shared_down, x, x_dtype, T, ids, w, y);
}

/* Routed experts in MXFP4 (gate, up and down; grid unused). */
void oracle_moe_ffn_mxfp4(int H, int I, int E, int k,
                          const uint8_t *const *gate, const uint8_t *const *up,
                          const uint8_t *const *down,
                          const uint16_t *shared_gate, const uint16_t *shared_up,
                          const uint16_t *shared_down,
                          const void *x, int x_dtype, int T,
                          const int32_t *ids, const double *w, double *y)
{
    moe_ffn(1, H, I, E, k, NULL, gate, up, down, shared_gate, shared_up,
            shared_down, x, x_dtype, T, ids, w, y);
}

#ifdef _OPENMP
#include <omp.h>
int oracle_max_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }
#else
int oracle_max_threads(void) { return 1; }
void oracle_set_threads(int n) { (void)n; }
#endif
