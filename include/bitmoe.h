/*
 * bitmoe.h -- C ABI of the 2-bit routed-expert MoE feed-forward layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (DeepSeek-V4-Flash-class routed MoE FFN) and its weight scheme
 * come from the pages:
 *  - "Un modele de 284 milliards de parametres tourne desormais sur un Mac de
 *    128 Go. Qui y perd ?", section "Comment un modele de 284 milliards de
 *    parametres tient sur une seule machine": a router selects a few experts
 *    for every token; the routed experts hold most of the weights.
 *  - "ds4 : analyse pratique pour un usage documente", section "Support de
 *    modeles et choix de quantification" (and "antirez/ds4 - Moteur local
 *    d'inference DeepSeek V4 Flash pour Metal", section "Poids du modele"):
 *    the asymmetric 2-bit scheme quantises only the routed experts, up and
 *    gate as IQ2_XXS, down as Q2_K; the shared expert, projections and the
 *    router stay unquantised (bf16 here).
 *  - "antirez/ds4 ...", section "Remerciements a llama.cpp et GGML": the
 *    GGUF block layouts are GGML's, which fixes the canonical byte order.
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller; they must
 *    stay valid until the work queued on `stream` has finished.  Nothing is
 *    retained after the call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).  All
 *    compute entry points are asynchronous: they validate on the host, queue
 *    kernels and return; they never synchronise and never allocate device
 *    memory (scratch lives in the caller's workspace).
 *  - Every call returns BITMOE_OK (0) or a negative error code; on error no
 *    kernel has been queued (BITMOE_EHIP: a launch failed; work queued before
 *    the failing launch may have run).  moe_strerror() names the code.
 *  - Shapes: H (hidden) and I (expert intermediate) must be multiples of
 *    256; 1 <= k <= 16; k <= E <= 1024; T >= 0 (T = 0 is a no-op).
 *  - Calls are thread-safe; calls on different streams may overlap.
 *  - moe_ffn_decode / moe_forward_decode on a batch in which some expert is
 *    chosen by several tokens (2 <= T, T*k <= 128, T <= 96) fork part of the
 *    work onto a stream the library keeps per device (created on the first
 *    such call, default priority) and join it back into `stream` before the
 *    call's last kernel: the call is still ordered on `stream` as a whole.
 *
 * Weight formats
 *  CANONICAL blocks (the interchange format, GGML order):
 *   IQ2X, 66 bytes per 256 consecutive weights of one row:
 *     bytes 0-1   fp16 d (little-endian)
 *     bytes 2-65  8 groups g of 8 bytes: 4 codebook indices idx[j], then a
 *                 little-endian u32 a; sign field j = (a >> 7j) & 0x7F, group
 *                 scale s = a >> 28.  The eighth sign of each run of 8 is the
 *                 even-parity bit of the seven stored ones; set = negative.
 *     weight 32g+8j+i = d * (0.5 + s) / 4 * grid[idx[j]][i] * (+-1)
 *   Q2K, 84 bytes per 256 weights:
 *     bytes 0-15  scales: sub-block b (weights 16b..16b+15) has
 *                 scale = byte & 15 and min = byte >> 4
 *     bytes 16-79 qs: weight i has q = (qs[32*(i/128) + i%32] >> 2*((i%128)/32)) & 3
 *     bytes 80-83 fp16 d, fp16 dmin
 *     weight i = d * scale * q - dmin * min
 *   A projection with N outputs and K inputs stores block (n, kb) at index
 *   n*(K/256) + kb; experts are stacked on a leading axis [E].
 *
 *  TILED layout (what the FFN entry points read; moe_pack_* produces it).
 *   The same information in the same number of bytes, regrouped into 64-row
 *   panels so that 64 lanes reading one 16-byte piece of 64 consecutive rows
 *   issue one contiguous 1 KiB access.
 *   Per expert the slab has exactly the canonical size, with nb = K/256,
 *   P = n/64, r = n%64:
 *   IQ2X slab (N*nb*66 bytes):
 *     [0, 64*N*nb):           piece c (groups 2c, 2c+1 of block (n,kb)) at
 *                             ((P*nb + kb)*4 + c)*64 + r, 16 bytes each; each
 *                             group regrouped (bijectively, same 8 bytes) as
 *                             two little-endian words, W0 for runs 0,1 and W1
 *                             for runs 2,3 (a run is 8 weights); the first
 *                             run of a word in bytes 0-1, the second in
 *                             bytes 2-3: the run's codebook index idx[j],
 *                             then its sign field (bits 0-6) with bit j of
 *                             the group scale s in bit 7
 *     [64*N*nb, 66*N*nb):     d of block (n,kb) at (P*nb + kb)*64 + r, 2 bytes
 *   Q2K slab (N*nb*84 bytes):
 *     [0, 64*N*nb):           piece c at ((P*nb + kb)*4 + c)*64 + r, 16 bytes:
 *                             the quants of sub-blocks 4c..4c+3 (weights
 *                             64c..64c+63), one little-endian word each: the
 *                             quant of weight 2p of the sub-block at bits 2p,
 *                             that of weight 2p+1 at bits 16+2p
 *     [64*N*nb, 80*N*nb):     scales (bytes 0-15) at (P*nb + kb)*64 + r, 16 B
 *     [80*N*nb, 84*N*nb):     d, dmin (bytes 80-83) at (P*nb + kb)*64 + r, 4 B
 *   BF16 (shared expert) matrix [N][K] row-major -> tiled: the 8 values
 *   K = 8c..8c+7 of row n at ((P*(K/8) + c)*64 + r)*16 bytes.
 */
#ifndef BITMOE_H
#define BITMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITMOE_OK            0
#define BITMOE_EINVAL       (-1)  /* null pointer, bad dtype/mode, negative size */
#define BITMOE_EUNSUPPORTED (-2)  /* H or I not a multiple of 256, k > 16, k > E, E > 1024, T too large */
#define BITMOE_EWORKSPACE   (-3)  /* workspace missing, too small or misaligned */
#define BITMOE_EHIP         (-4)  /* a HIP launch failed */

#define BITMOE_F32  0   /* float32 activations / outputs */
#define BITMOE_BF16 1   /* bfloat16 activations / outputs */

#define BITMOE_DECODE  0
#define BITMOE_PREFILL 1

/* One routed-MoE layer.  All pointers are device pointers. */
typedef struct bitmoe_layer {
    int32_t H;                 /* hidden size (multiple of 256) */
    int32_t I;                 /* expert intermediate size (multiple of 256) */
    int32_t E;                 /* routed experts, k <= E <= 1024 */
    int32_t k;                 /* experts per token, 1..16 */
    const void *router_w;      /* bf16 [E][H] row-major */
    const void *gate_q;        /* TILED IQ2X, E slabs of I*(H/256)*66 bytes */
    const void *up_q;          /* TILED IQ2X, same shape as gate_q */
    const void *down_q;        /* TILED Q2K, E slabs of H*(I/256)*84 bytes */
    const void *grid;          /* uint8 [256][8] codebook magnitudes (the
                                  format's codebook holds 1, 3, 5, 7; any
                                  byte is accepted) */
    const void *shared_gate;   /* TILED bf16 [I][H], or NULL: no shared expert */
    const void *shared_up;     /* TILED bf16 [I][H] (NULL iff shared_gate is) */
    const void *shared_down;   /* TILED bf16 [H][I] (NULL iff shared_gate is) */
} bitmoe_layer;

/*
 * Routing (router logits, top-k, renormalised softmax).
 * x: [T][H] of x_dtype (BITMOE_F32 or BITMOE_BF16).
 * logits (may be NULL): float32 [T][E], logits[t][e] = sum_h x[t][h]*W[e][h]
 *   accumulated in fp32.
 * ids: int32 [T][k], the k largest logits in descending order, ties to the
 *   lower expert index.  w: float32 [T][k], softmax over the k selected
 *   logits (sums to 1).
 * ws: device scratch of at least moe_route_workspace_bytes(L, T, x_dtype)
 *   bytes, 256-byte aligned (partial sums of the split-K router; results do
 *   not depend on scheduling: the splits are added in a fixed order).
 */
size_t moe_route_workspace_bytes(const bitmoe_layer *L, int T, int x_dtype);
int moe_route(const bitmoe_layer *L, const void *x, int x_dtype, int T,
              float *logits, int32_t *ids, float *w, void *ws, size_t ws_bytes,
              void *stream);

/* Top-k + renormalised softmax of given float32 logits [T][E]. */
int moe_topk(const float *logits, int T, int E, int k, int32_t *ids,
             float *w, void *stream);

/*
 * Token->expert bucketing.  ids int32 [T][k] with values in [0,E) (trusted).
 * counts int32 [E]; offsets int32 [E+1] exclusive prefix sum of counts;
 * perm int32 [T*k]: pair indices p = t*k + j grouped by expert, ascending p
 * within each expert; active int32 [E]: experts with counts > 0 ascending,
 * padded with -1; n_active int32 [1].  Scratch comes from ws, which must be
 * at least moe_bucket_workspace_bytes(T, k, E) bytes, 256-byte aligned.
 */
size_t moe_bucket_workspace_bytes(int T, int k, int E);
int moe_bucket(const int32_t *ids, int T, int k, int E, int32_t *counts,
               int32_t *offsets, int32_t *perm, int32_t *active,
               int32_t *n_active, void *ws, size_t ws_bytes, void *stream);

/* Bytes of workspace moe_ffn_decode / moe_ffn_prefill need for T tokens. */
size_t moe_workspace_bytes(const bitmoe_layer *L, int T, int mode);

/*
 * The MoE FFN: y[t] = sum_j w[t][j] * D_e(silu(G_e x_t) * U_e x_t)
 *                     (+ D_s(silu(G_s x_t) * U_s x_t) when the layer has a
 *                     shared expert), e = ids[t][j], silu(z) = z/(1+e^-z).
 * x [T][H] (x_dtype), ids int32 [T][k] (values in [0,E), trusted; each row
 * k distinct experts, as a top-k gives: moe_ffn_decode does not support a
 * row that repeats an expert), w float32 [T][k], y float32 [T][H]
 * (overwritten).  ws: device workspace of at least
 * moe_workspace_bytes(L, T, mode) bytes, 256-byte aligned.
 * moe_ffn_decode streams each active expert's packed blocks once and decodes
 * them in registers (fp32 accumulation); it is tuned for T <= 16 and correct
 * for any T.  moe_ffn_prefill runs grouped fp16 MFMA GEMMs (fp32
 * accumulation) over weights dequantised into matrix-core operands on chip;
 * it is tuned for large T and correct for any T.  Its operands are fp16:
 * each token's x and each row of h scaled by powers of two, and weights
 * rounded to fp16 after folding the scales (d/8 (2s+1) for IQ2X, d sc and
 * dmin m for Q2K) with a fixed factor 2^8, so full fp16 precision holds for
 * superblock scales d, dmin in [2^-19, 8] (codebook magnitudes up to 7);
 * larger scales can overflow.
 */
int moe_ffn_decode(const bitmoe_layer *L, const void *x, int x_dtype, int T,
                   const int32_t *ids, const float *w, float *y, void *ws,
                   size_t ws_bytes, void *stream);
int moe_ffn_prefill(const bitmoe_layer *L, const void *x, int x_dtype, int T,
                    const int32_t *ids, const float *w, float *y, void *ws,
                    size_t ws_bytes, void *stream);

/*
 * The whole layer for a decode batch: moe_route followed by moe_ffn_decode
 * in one call.  For T <= 16 and T*k <= 128 the router rows, the shared expert
 * and the bookkeeping share launches with the expert GEMVs (three launches
 * in all; more for larger batches).
 * ids int32 [T][k] and w float32 [T][k] receive the routing (same values as
 * moe_route); y float32 [T][H] as moe_ffn_decode.  Needs L->router_w.
 * ws: at least moe_workspace_bytes(L, T, BITMOE_DECODE) bytes.
 */
int moe_forward_decode(const bitmoe_layer *L, const void *x, int x_dtype, int T,
                       int32_t *ids, float *w, float *y, void *ws,
                       size_t ws_bytes, void *stream);

/*
 * Standalone dequantisation of CANONICAL blocks: nblocks blocks ->
 * out [nblocks*256] of out_dtype.  BITMOE_F32 output is the exact value
 * (IQ2X) or the single fp32 rounding of d*scale*q - dmin*min (Q2K);
 * BITMOE_BF16 output is that fp32 value rounded to nearest-even.
 */
int moe_dequant_iq2x(const void *blocks, const void *grid, int64_t nblocks,
                     void *out, int out_dtype, void *stream);
int moe_dequant_q2k(const void *blocks, int64_t nblocks, void *out,
                    int out_dtype, void *stream);

/*
 * Load-time layout transforms (canonical -> TILED, see above), E experts of
 * an [N][K] projection; N multiple of 64, K multiple of 256 (bf16: of 8).
 * src and dst must not overlap.
 */
int moe_pack_iq2x(const void *src, void *dst, int E, int N, int K, void *stream);
int moe_pack_q2k(const void *src, void *dst, int E, int N, int K, void *stream);
int moe_pack_bf16(const void *src, void *dst, int N, int K, void *stream);

/*
 * Measurement hook.  When start and stop are both hipEvent_t handles (passed
 * as void*), every later decode or prefill FFN call made from the calling
 * thread launches its routed gate/up projection kernel with hipExtLaunchKernel
 * and these events, which the dispatch itself takes when the kernel starts
 * and when it ends, so hipEventElapsedTime gives that kernel's duration
 * (for a decode batch with experts chosen by several tokens, the first of
 * its two gate/up launches).  Pass NULL, NULL to turn it off.  The setting
 * is per host thread.
 */
int moe_set_timing_events(void *start, void *stop);

const char *moe_strerror(int code);
const char *moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BITMOE_H */
