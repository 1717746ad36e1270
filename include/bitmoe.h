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
 *  - The one piece of library state: moe_ffn_decode / moe_forward_decode on
 *    a batch of 9 <= T <= 96 tokens with T*k <= 128 (whose experts chosen
 *    by several tokens take the prefill kernels) fork part of the work onto
 *    a stream the library keeps per device (created on the first such call,
 *    default priority, with two events) and join it back into `stream`
 *    before the call's last kernel, also when a launch fails after the
 *    fork: the call is ordered on `stream` as a whole.  Such calls from
 *    several host threads take turns at that stream (a lock held while the
 *    call queues its work), so their side-stream halves run one after
 *    another.
 *  - Routing ids given by the caller (moe_bucket, moe_ffn_decode,
 *    moe_ffn_prefill) must lie in [0, E); this library trusts them.  The
 *    same sources built with BITMOE_CHECK_IDS=1 (libbitmoe_checked.so,
 *    built beside libbitmoe.so; its moe_version() says so) check them on
 *    the device: those calls first write the count of ids outside [0, E)
 *    into the int32 at the start of their workspace (0: all valid), and read
 *    every id clamped into range, so that a bad id gives a wrong result but
 *    no access out of bounds.  The first 256 bytes of those workspaces are
 *    reserved for that count in both builds.
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
 *   MXFP4 (OCP Microscaling: FP4 E2M1 elements, one E8M0 scale per 32; the
 *   pages' MXFP4 variant keeps the released FP4 expert weights, "ds4 :
 *   analyse pratique ...", section "Support de modeles et choix de
 *   quantification"), 17 bytes per 32 consecutive weights of one row:
 *     byte 0      scale exponent X: the block's scale is 2^(X-127) (X = 255: NaN)
 *     bytes 1-16  qs: weight j (0..15) in the low nibble of qs[j], weight
 *                 j+16 in its high nibble
 *     element code c: sign c >> 3, then 0, 0.5, 1, 1.5, 2, 3, 4, 6 for c & 7
 *     weight = element * 2^(X-127)
 *   Block (n, kb) of an [N][K] projection at index n*(K/32) + kb.
 *
 *  TILED layout (what the FFN entry points read; moe_pack_* produces it;
 *  bitmoe_layer.layout says which of the two a descriptor's blocks are in).
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
 *                             quant of weight t (0..15) of the sub-block at
 *                             bits 8*((t & 7) >> 1) + 4*(t & 1) + 2*(t >> 3)
 *                             (byte s: weights 2s, 2s+1 in bits 0-1, 4-5 and
 *                             weights 8+2s, 9+2s in bits 2-3, 6-7)
 *     [64*N*nb, 80*N*nb):     scales (bytes 0-15) at (P*nb + kb)*64 + r, 16 B
 *     [80*N*nb, 84*N*nb):     d, dmin (bytes 80-83) at (P*nb + kb)*64 + r, 4 B
 *   MXFP4 slab (N*(K/32)*17 bytes), nb = K/256 again:
 *     [0, N*K/2):             piece c (the block of weights 32c..32c+31 of
 *                             the 256 at kb) at ((P*nb + kb)*8 + c)*64 + r,
 *                             16 bytes: byte i holds weight 2i in its low
 *                             nibble and weight 2i+1 in its high nibble
 *     [N*K/2, N*K*17/32):     the 8 scale bytes X of (n, kb) at
 *                             ((P*nb + kb)*64 + r)*8, piece c's at + c
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
#define BITMOE_ESCRATCH     (-5)  /* more scratch than BITMOE_STATIC_SCRATCH_BYTES (noalloc call) */

#define BITMOE_F32  0   /* float32 activations / outputs */
#define BITMOE_BF16 1   /* bfloat16 activations / outputs */

#define BITMOE_DECODE  0
#define BITMOE_PREFILL 1

#define BITMOE_LAYOUT_CANONICAL 0   /* GGML block order (the interchange format) */
#define BITMOE_LAYOUT_TILED     1   /* 64-row panels (moe_pack_*), read by the FFN calls */

#define BITMOE_FORMAT_2BIT  0   /* routed gate/up IQ2X, down Q2K (grid required) */
#define BITMOE_FORMAT_MXFP4 1   /* routed gate, up and down MXFP4 (grid unused) */

#define BITMOE_TIME_GATEUP 0        /* moe_set_timing_events: the routed gate/up kernel */
#define BITMOE_TIME_DOWN   1        /* moe_set_timing_events: the routed down kernel */

/*
 * One routed-MoE layer.  All pointers are device pointers.  The FFN entry
 * points read TILED blocks and return BITMOE_EUNSUPPORTED for a descriptor
 * whose layout is BITMOE_LAYOUT_CANONICAL (convert with moe_pack_* first);
 * moe_route and moe_topk read only the router, in either case.
 */
typedef struct bitmoe_layer {
    int32_t H;                 /* hidden size (multiple of 256) */
    int32_t I;                 /* expert intermediate size (multiple of 256) */
    int32_t E;                 /* routed experts, k <= E <= 1024 */
    int32_t k;                 /* experts per token, 1..16 */
    const void *router_w;      /* bf16 [E][H] row-major */
    const void *gate_q;        /* TILED IQ2X, E slabs of I*(H/256)*66 bytes
                                  (MXFP4: I*(H/32)*17 bytes) */
    const void *up_q;          /* same shape as gate_q */
    const void *down_q;        /* TILED Q2K, E slabs of H*(I/256)*84 bytes
                                  (MXFP4: H*(I/32)*17 bytes) */
    const void *grid;          /* uint8 [256][8] codebook magnitudes (the
                                  format's codebook holds 1, 3, 5, 7; any
                                  byte is accepted); unused for MXFP4 */
    const void *shared_gate;   /* TILED bf16 [I][H], or NULL: no shared expert */
    const void *shared_up;     /* TILED bf16 [I][H] (NULL iff shared_gate is) */
    const void *shared_down;   /* TILED bf16 [H][I] (NULL iff shared_gate is) */
    int32_t layout;            /* BITMOE_LAYOUT_TILED or BITMOE_LAYOUT_CANONICAL:
                                  the layout of gate_q, up_q, down_q and the
                                  shared matrices */
    int32_t format;            /* BITMOE_FORMAT_2BIT (0) or BITMOE_FORMAT_MXFP4:
                                  the routed experts' block format */
} bitmoe_layer;

/*
 * Routing (router logits, top-k, renormalised softmax).  The router picks a
 * few experts for every token ("Un modele de 284 milliards de parametres
 * tourne desormais sur un Mac de 128 Go. Qui y perd ?", section "Comment un
 * modele de 284 milliards de parametres tient sur une seule machine"); it
 * stays unquantised ("antirez/ds4 - Moteur local d'inference DeepSeek V4
 * Flash pour Metal", section "Poids du modele").
 * x: [T][H] of x_dtype (BITMOE_F32 or BITMOE_BF16).
 * logits (may be NULL): float32 [T][E], logits[t][e] = sum_h x[t][h]*W[e][h]
 *   accumulated in fp32.
 * ids: int32 [T][k], the k largest logits in descending order, ties to the
 *   lower expert index.  w: float32 [T][k], softmax over the k selected
 *   logits (sums to 1).
 * ws: device scratch of at least moe_route_workspace_bytes(L, T, x_dtype)
 *   bytes, 256-byte aligned (partial sums of the split-K router; results do
 *   not depend on scheduling: the splits are added in a fixed order).
 * Errors: EINVAL (null x/ids/w or router, bad dtype, T < 0, x not 16-byte
 * aligned), EUNSUPPORTED (shape), EWORKSPACE, EHIP.
 */
size_t moe_route_workspace_bytes(const bitmoe_layer *L, int T, int x_dtype);
int moe_route(const bitmoe_layer *L, const void *x, int x_dtype, int T,
              float *logits, int32_t *ids, float *w, void *ws, size_t ws_bytes,
              void *stream);

/*
 * Top-k + renormalised softmax of given float32 logits [T][E] (the second
 * half of moe_route, same passage): ids int32 [T][k], w float32 [T][k] as
 * in moe_route.  Errors: EINVAL (null pointer, T < 0, E or k < 1),
 * EUNSUPPORTED (k > 16, k > E, E > 1024), EHIP.
 */
int moe_topk(const float *logits, int T, int E, int k, int32_t *ids,
             float *w, void *stream);

/*
 * Token->expert bucketing, so that each chosen expert's weights are streamed
 * once per call: decode is bound by memory bandwidth ("Faire tenir un MoE de
 * 284B dans un portable de 128 Go", section "Un pre-remplissage a 790 t/s
 * revele le veritable goulot d'etranglement").
 * ids int32 [T][k] with values in [0,E) (trusted; checked builds: above).
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

/*
 * Bytes of workspace moe_ffn_decode / moe_forward_decode (mode
 * BITMOE_DECODE) or moe_ffn_prefill (BITMOE_PREFILL) need for T tokens; 0
 * for an invalid layer, T or mode.
 */
size_t moe_workspace_bytes(const bitmoe_layer *L, int T, int mode);

/*
 * The MoE FFN, with the routed experts' up/gate in IQ2_XXS and down in Q2_K
 * and the shared expert unquantised ("ds4 : analyse pratique pour un usage
 * documente", section "Support de modeles et choix de quantification";
 * "antirez/ds4 ...", section "Poids du modele"); decode is bound by memory
 * bandwidth, prefill by compute ("Faire tenir un MoE de 284B ...", section
 * "Un pre-remplissage a 790 t/s revele le veritable goulot
 * d'etranglement"):
 *         y[t] = sum_j w[t][j] * D_e(silu(G_e x_t) * U_e x_t)
 *                     (+ D_s(silu(G_s x_t) * U_s x_t) when the layer has a
 *                     shared expert), e = ids[t][j], silu(z) = z/(1+e^-z).
 * x [T][H] (x_dtype), ids int32 [T][k] (values in [0,E), trusted or
 * checked as above; each row
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
 * Errors: EINVAL (null x/ids/w/y or quantised weights, a shared matrix
 * without the other two, bad dtype, T < 0, x or y not 16-byte aligned),
 * EUNSUPPORTED (shape, or a CANONICAL layout), EWORKSPACE, EHIP.
 */
int moe_ffn_decode(const bitmoe_layer *L, const void *x, int x_dtype, int T,
                   const int32_t *ids, const float *w, float *y, void *ws,
                   size_t ws_bytes, void *stream);
int moe_ffn_prefill(const bitmoe_layer *L, const void *x, int x_dtype, int T,
                    const int32_t *ids, const float *w, float *y, void *ws,
                    size_t ws_bytes, void *stream);

/*
 * The whole layer for a decode batch (the passages of moe_route and
 * moe_ffn_decode): moe_route followed by moe_ffn_decode in one call.  For T <= 16 and T*k <= 128 the router rows, the shared expert
 * and the bookkeeping share launches with the expert GEMVs (three launches
 * in all; more for larger batches).
 * ids int32 [T][k] and w float32 [T][k] receive the routing (same values as
 * moe_route); y float32 [T][H] as moe_ffn_decode.  Needs L->router_w.
 * ws: at least moe_workspace_bytes(L, T, BITMOE_DECODE) bytes (which
 * includes the router's scratch for batches routed in a launch of their
 * own).  Errors: those of moe_ffn_decode, and EINVAL without a router.
 */
int moe_forward_decode(const bitmoe_layer *L, const void *x, int x_dtype, int T,
                       int32_t *ids, float *w, float *y, void *ws,
                       size_t ws_bytes, void *stream);

/*
 * moe_forward_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same routing and decode FFN, with the same outputs, but
 * its scratch lives in a device array of the library
 * (BITMOE_STATIC_SCRATCH_BYTES per device, held from load until the process
 * ends) instead of a caller workspace, and every launch stays on `stream`
 * (no side stream).  The call allocates nothing.  Calls whose scratch would
 * exceed the array return BITMOE_ESCRATCH before any launch (at H 7168,
 * I 2048, E 256, k 8 with a shared expert: up to 16 tokens fit).  Every
 * call on one device shares that device's array: calls that overlap on one
 * device race and must be serialised by the caller.
 * Errors: those of moe_forward_decode (no EWORKSPACE), ESCRATCH, and EHIP if
 * the array's device address cannot be looked up.
 */
#define BITMOE_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
int moe_forward_decode_noalloc(const bitmoe_layer *L, const void *x, int x_dtype, int T,
                               int32_t *ids, float *w, float *y, void *stream);

/*
 * Standalone dequantisation of CANONICAL blocks (GGML's GGUF block layouts:
 * "antirez/ds4 ...", section "Remerciements a llama.cpp et GGML"; the two
 * formats: "ds4 : analyse pratique ...", section "Support de modeles et
 * choix de quantification"): nblocks blocks ->
 * out [nblocks*256] of out_dtype.  BITMOE_F32 output is the exact value
 * (IQ2X) or the single fp32 rounding of d*scale*q - dmin*min (Q2K);
 * BITMOE_BF16 output is that fp32 value rounded to nearest-even.
 * Errors: EINVAL (null or misaligned pointer: blocks 2-byte (IQ2X) or
 * 4-byte (Q2K), grid 8-byte, out 16-byte aligned; nblocks < 0; bad dtype),
 * EHIP.
 */
int moe_dequant_iq2x(const void *blocks, const void *grid, int64_t nblocks,
                     void *out, int out_dtype, void *stream);
int moe_dequant_q2k(const void *blocks, int64_t nblocks, void *out,
                    int out_dtype, void *stream);
/*
 * The same for CANONICAL MXFP4 blocks (17 bytes, see above): nblocks blocks
 * -> out [nblocks*32].  BITMOE_F32 output is the fp32 rounding of
 * element * 2^(X-127) (exact unless it overflows to +-inf; X = 255 gives
 * NaN); BITMOE_BF16 output rounds that to nearest-even.  Errors: EINVAL
 * (null pointer, out not 16-byte aligned, nblocks < 0, bad dtype), EHIP.
 */
int moe_dequant_mxfp4(const void *blocks, int64_t nblocks, void *out,
                      int out_dtype, void *stream);

/*
 * Routed-expert residency cache, for layers whose routed experts do not all
 * fit in HBM: the experts' TILED slabs stay in host memory (pinned, for
 * asynchronous copies) and a pool of `slots` HBM slots holds the ones in
 * use.  This is the pages' streaming of routed experts from SSD through an
 * in-memory expert cache, non-routed weights staying resident ("Faire tenir
 * un MoE de 284B dans un portable de 128 Go", section "Streaming depuis le
 * SSD quand la memoire fait defaut"), with host memory in the SSD's place.
 *  moe_cache_pool_bytes: device bytes of the pool for `slots` slots
 *   (k <= slots <= E; 0 if invalid).
 *  moe_cache_create: L gives H, I, E, k and the DEVICE router, grid and
 *   shared expert (its gate_q/up_q/down_q are ignored); host_gate, host_up,
 *   host_down are the E experts' TILED slabs in host memory (owned by the
 *   caller, valid until destroy); pool is caller-owned device memory of at
 *   least moe_cache_pool_bytes(L, slots).  *cache receives a handle owned by
 *   the caller (moe_cache_destroy frees it); the library keeps no other
 *   state.
 *  moe_cache_layer: a descriptor over the pool (E = slots, routed slabs in
 *   the pool, the rest as given) for moe_ffn_decode / moe_ffn_prefill.
 *  moe_cache_map: routing ids (HOST int32 [n], values in [0, E)) -> slot ids
 *   (HOST int32 [n]) for the pool descriptor; experts not resident are copied
 *   into slots with hipMemcpyAsync on `stream` (so FFN calls queued after it
 *   on that stream see them, and earlier calls on it finish reading a slot
 *   before it is overwritten).  Policy: the call's distinct experts, in
 *   order of first appearance, keep their slots; a missing one takes the
 *   lowest-numbered empty slot, else the least recently used slot not used
 *   by this call (ties to the lower slot).  *loaded (may be NULL) receives
 *   the number of experts copied.  Errors: EINVAL (null pointer, an id out
 *   of range), EUNSUPPORTED (more distinct experts than slots), EHIP.
 *  moe_cache_stats: cumulative hits and misses (experts), and the expert
 *   in each slot (-1: empty) into expert_in_slot [slots] (any may be NULL).
 * A handle is not thread-safe: calls on one handle must be serialised.
 */
size_t moe_cache_pool_bytes(const bitmoe_layer *L, int slots);
int moe_cache_create(const bitmoe_layer *L, const void *host_gate, const void *host_up,
                     const void *host_down, int slots, void *pool, size_t pool_bytes,
                     void **cache);
int moe_cache_layer(const void *cache, bitmoe_layer *out);
int moe_cache_map(void *cache, const int32_t *ids, int n, int32_t *slot_ids, int *loaded,
                  void *stream);
int moe_cache_stats(const void *cache, int64_t *hits, int64_t *misses, int32_t *expert_in_slot);
int moe_cache_destroy(void *cache);

/*
 * Quantizer (the step before the layer): fp32 weights -> CANONICAL blocks,
 * nblocks superblocks of 256 consecutive weights of one row each.  The
 * routed experts are quantised asymmetrically to 2 bits, up/gate in IQ2_XXS
 * and down in Q2_K ("antirez/ds4 ...", section "Poids du modele"), with an
 * importance matrix ("ds4 : un MoE de 284 milliards sur un Mac de 128 Go",
 * section "Comment un 284B tient en memoire"); with no calibration data the
 * search minimises the plain squared error:
 *  IQ2X: d = fp16(max|w| / 27.125); per group of 32 the group scale 0..15
 *   and per run of 8 the codebook row (of grid, uint8 [256][8]) and signs
 *   (those of w, with the cheapest single flip when the parity rule needs
 *   one) of least squared error; ties to the lower row, scale, element.
 *  Q2K: per sub-block of 16, m = max(0, -min w), a = (max w + m) / 3;
 *   d = fp16(max a / 15), dmin = fp16(max m / 15); per sub-block the best
 *   (scale, min) codes within +-1 of rint(a / d), rint(m / dmin), quants
 *   clamp(rint((w + M) / A), 0, 3).
 * Every decision is taken in double precision with unfused operations in a
 * fixed order, so the bytes depend on the input alone.  fp16(x) is the
 * nearest binary16 (ties to even), at most 65504.
 * w: float32 [nblocks * 256], 16-byte aligned; blocks: uint8 [nblocks][66]
 * or [nblocks][84].  Errors: EINVAL (null or misaligned pointer, nblocks <
 * 0), EHIP.
 */
int moe_quantize_iq2x(const float *w, const void *grid, int64_t nblocks, void *blocks, void *stream);
int moe_quantize_q2k(const float *w, int64_t nblocks, void *blocks, void *stream);
/*
 * The same for MXFP4 (OCP Microscaling conversion; the pages' MXFP4 variant,
 * "ds4 : analyse pratique ...", section "Support de modeles et choix de
 * quantification"): nblocks blocks of 32 consecutive weights -> canonical
 * 17-byte blocks.  The shared exponent e0 = floor(log2 max|w|) - 2 of the
 * OCP conversion and e0 + 1 are both tried (clamped to -127..127); each
 * weight goes to the nearest E2M1 magnitude (ties to the even mantissa bit,
 * saturating at 6), and the exponent with the smaller squared error is kept
 * (ties to e0); a negative weight with a nonzero magnitude takes the sign
 * bit.  All-zero blocks are zero bytes.  Decisions in double precision as
 * above; inputs must be finite.  w: float32 [nblocks * 32], 16-byte
 * aligned; blocks: uint8 [nblocks][17].  Errors: EINVAL, EHIP.
 */
int moe_quantize_mxfp4(const float *w, int64_t nblocks, void *blocks, void *stream);

/*
 * Load-time layout transforms (canonical -> TILED, see above), E experts of
 * an [N][K] projection; N multiple of 64, K multiple of 256 (bf16: of 8).
 * The canonical order is GGML's ("antirez/ds4 ...", section "Remerciements
 * a llama.cpp et GGML"); the tiled one is this library's, with the same
 * bytes.  src and dst must not overlap.  Errors: EINVAL (null or misaligned
 * pointer, negative size), EUNSUPPORTED (N or K not a multiple), EHIP.
 */
int moe_pack_iq2x(const void *src, void *dst, int E, int N, int K, void *stream);
int moe_pack_q2k(const void *src, void *dst, int E, int N, int K, void *stream);
int moe_pack_bf16(const void *src, void *dst, int N, int K, void *stream);
int moe_pack_mxfp4(const void *src, void *dst, int E, int N, int K, void *stream);

/*
 * Measurement hook.  When start and stop are both hipEvent_t handles (passed
 * as void*), every later decode or prefill FFN call made from the calling
 * thread launches one kernel with hipExtLaunchKernel and these events, which
 * the dispatch itself takes when the kernel starts and when it ends, so
 * hipEventElapsedTime gives that kernel's duration.  which: BITMOE_TIME_GATEUP
 * (the routed gate/up kernel; for a decode batch with experts chosen by
 * several tokens, the single-token experts' one) or BITMOE_TIME_DOWN (the
 * routed down kernel; for decode, the one that also runs the shared down).
 * Pass NULL, NULL to turn it off.  The setting is per host thread.
 * Errors: EINVAL (one event without the other, unknown which).
 */
int moe_set_timing_events(void *start, void *stop, int which);

const char *moe_strerror(int code);
const char *moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BITMOE_H */
