/*
 * Host sanitizer driver for the CPU oracle (test infrastructure): runs every
 * oracle entry point on small seeded inputs under AddressSanitizer and
 * UndefinedBehaviorSanitizer, with a few sanity checks.  Exit status 0 when
 * everything ran clean.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_fp16_to_double(uint16_t h);
double oracle_bf16_to_double(uint16_t b);
void oracle_dequant_iq2x(const uint8_t *blocks, const uint8_t *grid, int64_t nblocks, double *out);
void oracle_dequant_q2k(const uint8_t *blocks, int64_t nblocks, double *out);
void oracle_router_logits(const void *x, int x_dtype, int T, int H, const uint16_t *wr, int E, double *logits);
void oracle_topk(const double *logits, int T, int E, int k, int32_t *ids, double *w);
void oracle_bucket(const int32_t *ids, int T, int k, int E, int32_t *counts, int32_t *offsets, int32_t *perm);
void oracle_moe_ffn(int H, int I, int E, int k, const uint8_t *grid, const uint8_t *const *gate,
                    const uint8_t *const *up, const uint8_t *const *down, const uint16_t *shared_gate,
                    const uint16_t *shared_up, const uint16_t *shared_down, const void *x, int x_dtype, int T,
                    const int32_t *ids, const double *w, double *y);

static uint64_t rs = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    rs ^= rs << 13; rs ^= rs >> 7; rs ^= rs << 17;
    return (uint32_t)(rs >> 16);
}

/* bf16 bits of a small value: sign, exponent 2^-8 .. 2^-5, random mantissa */
static uint16_t small_bf16(void)
{
    uint32_t e = 119 + rnd() % 4, m = rnd() & 0x7F, s = rnd() & 1;
    return (uint16_t)((s << 15) | (e << 7) | m);
}

static void blocks(uint8_t *b, int64_t n, int bytes, int d_at, int nd)
{
    for (int64_t i = 0; i < n * bytes; i++)
        b[i] = (uint8_t)rnd();
    for (int64_t i = 0; i < n; i++)
        for (int j = 0; j < nd; j++) {      /* finite positive fp16 scale around 2^-6 */
            uint16_t h = (uint16_t)((9u << 10) | (rnd() & 0x3FF));
            b[i * bytes + d_at + 2 * j] = (uint8_t)h;
            b[i * bytes + d_at + 2 * j + 1] = (uint8_t)(h >> 8);
        }
}

int main(void)
{
    enum { H = 256, I = 512, E = 8, K = 2, T = 5, NB = 64 };
    int bad = 0;
    uint8_t grid[256 * 8];
    for (int i = 0; i < 256 * 8; i++)
        grid[i] = (uint8_t)(2 * (rnd() % 4) + 1);

    /* standalone dequantisation, random bytes everywhere (any fp16 scale) */
    uint8_t *qb = malloc((size_t)NB * 84);
    double *dq = malloc(sizeof(double) * NB * 256);
    for (int i = 0; i < NB * 84; i++) qb[i] = (uint8_t)rnd();
    oracle_dequant_iq2x(qb, grid, NB, dq);
    oracle_dequant_q2k(qb, NB, dq);
    for (uint32_t h = 0; h < 65536; h++) {
        (void)oracle_fp16_to_double((uint16_t)h);
        (void)oracle_bf16_to_double((uint16_t)h);
    }

    /* one layer: routing, bucketing, FFN with and without a shared expert */
    size_t gsz = (size_t)I * (H / 256) * 66, dsz = (size_t)H * (I / 256) * 84;
    uint8_t *gate[E], *up[E], *down[E];
    for (int e = 0; e < E; e++) {
        gate[e] = malloc(gsz); up[e] = malloc(gsz); down[e] = malloc(dsz);
        blocks(gate[e], (int64_t)I * (H / 256), 66, 0, 1);
        blocks(up[e], (int64_t)I * (H / 256), 66, 0, 1);
        blocks(down[e], (int64_t)H * (I / 256), 84, 80, 2);
    }
    uint16_t *wr = malloc(sizeof(uint16_t) * E * H);
    for (int i = 0; i < E * H; i++) wr[i] = small_bf16();
    uint16_t *sg = malloc(sizeof(uint16_t) * I * H), *su = malloc(sizeof(uint16_t) * I * H);
    uint16_t *sd = malloc(sizeof(uint16_t) * H * I);
    for (int i = 0; i < I * H; i++) { sg[i] = small_bf16(); su[i] = small_bf16(); sd[i] = small_bf16(); }
    float x[T * H];
    uint16_t xb[T * H];
    for (int i = 0; i < T * H; i++) {
        x[i] = (float)((int)(rnd() % 2001) - 1000) / 500.0f;
        xb[i] = small_bf16();
    }
    double logits[T * E], w[T * K], y[T * H];
    int32_t ids[T * K], counts[E], offsets[E + 1], perm[T * K];
    for (int dt = 0; dt < 2; dt++) {
        const void *xp = dt ? (const void *)xb : (const void *)x;
        oracle_router_logits(xp, dt, T, H, wr, E, logits);
        oracle_topk(logits, T, E, K, ids, w);
        oracle_bucket(ids, T, K, E, counts, offsets, perm);
        for (int t = 0; t < T; t++) {
            double s = 0.0;
            for (int j = 0; j < K; j++) {
                s += w[t * K + j];
                if (ids[t * K + j] < 0 || ids[t * K + j] >= E) bad = 1;
            }
            if (fabs(s - 1.0) > 1e-12) bad = 1;
        }
        if (offsets[E] != T * K) bad = 1;
        for (int sh = 0; sh < 2; sh++) {
            oracle_moe_ffn(H, I, E, K, grid, (const uint8_t *const *)gate, (const uint8_t *const *)up,
                           (const uint8_t *const *)down, sh ? sg : NULL, sh ? su : NULL, sh ? sd : NULL,
                           xp, dt, T, ids, w, y);
            for (int i = 0; i < T * H; i++)
                if (!isfinite(y[i])) bad = 1;
        }
    }
    for (int e = 0; e < E; e++) { free(gate[e]); free(up[e]); free(down[e]); }
    free(wr); free(sg); free(su); free(sd); free(qb); free(dq);
    printf(bad ? "oracle sanitizer driver: check failed\n" : "oracle sanitizer driver: ok\n");
    return bad;
}
