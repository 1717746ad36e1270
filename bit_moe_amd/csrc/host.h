// Host-side interface between the C ABI (api.cpp), the launch planning
// (plan.cpp) and the launchers in the .hip files.  Host code only: this
// header needs nothing but the HIP runtime API, so the validation and
// workspace logic that includes it builds with a plain C++ compiler (and
// under the host sanitizers).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/bitmoe.h"

namespace bm_cfg {

// bucketing
constexpr int kBT = 1024;                 // threads per bucketing block = pairs per chunk
constexpr int kBW = kBT / 64;             // waves per bucketing block
constexpr int kSmallPairs = 4096;         // pairs bucketed by a single block
constexpr int kWaveBucketMax = 128;       // pairs bucketed by a single wave (decode batches)
// routing
constexpr int kRouterNT = 16;             // tokens per launch of the small-batch router
constexpr int kRouterSplit = 8;           // K slices of the matrix-core router
constexpr int kMfmaRouterMinT = 64;       // bf16 tokens from which the matrix-core router runs
constexpr int kFusedRouterMaxT = 16;      // decode: router rows fused into the first launch
// decode
constexpr int kFrontWaves = 16;           // waves per front workgroup
constexpr int kFrontRouterWaves = 4;      // the same when it only computes router rows
constexpr int kRouterRowWaves = 4;        // several tokens: waves per router row in the front launch
                                          // (each a quarter of K)
constexpr int kFrontPrepMaxT = 32;        // decode batches up to this size prepare the prefill
                                          // kernels' activations in the front launch
constexpr int kMaxChunks = 8;             // K chunks of the shared expert, at most
constexpr int kSharedChunkCols = 512;     // I columns of one shared-down K chunk, at most
constexpr int kDownWavesPerSimd = 5;      // waves per SIMD of the one-token decode down kernel: its
                                          // 4-wave workgroups, 5 to a compute unit
// prefill
constexpr int kPfRows = 96;               // rows per prefill row tile (three blocks of 32)
constexpr int kSplitMinT = 9;             // decode batches from this many tokens run the prefill kernels
                                          // for their experts chosen by several tokens
constexpr int kPfDnCols = 512;            // output columns per prefill down workgroup (one exponent each per pair)

}  // namespace bm_cfg

namespace bm_host {

int launch_dequant_iq2x(const void *blocks, const void *grid, int64_t nblocks,
                        void *out, int out_dtype, hipStream_t s);
int launch_dequant_q2k(const void *blocks, int64_t nblocks, void *out,
                       int out_dtype, hipStream_t s);
int launch_pack_iq2x(const void *src, void *dst, int E, int N, int K, hipStream_t s);
int launch_pack_q2k(const void *src, void *dst, int E, int N, int K, hipStream_t s);
int launch_pack_bf16(const void *src, void *dst, int N, int K, hipStream_t s);
int launch_dequant_mxfp4(const void *blocks, int64_t nblocks, void *out, int out_dtype, hipStream_t s);
int launch_pack_mxfp4(const void *src, void *dst, int E, int N, int K, hipStream_t s);

int launch_quant_iq2x(const float *w, const void *grid, int64_t nblocks, void *out, hipStream_t s);
int launch_quant_q2k(const float *w, int64_t nblocks, void *out, hipStream_t s);
int launch_quant_mxfp4(const float *w, int64_t nblocks, void *out, hipStream_t s);

// router logits [T][E] fp32 for at most bm_cfg::kRouterNT tokens
int launch_router_gemv(const bitmoe_layer *L, const void *x, int x_dtype, int T,
                       float *logits, hipStream_t s);
// split-K partial sums of the matrix-core router (floats)
size_t router_mfma_part_floats(int T, int E);
int launch_router_mfma(const bitmoe_layer *L, const void *x, int T, float *logits, int32_t *ids, float *w,
                       float *part, hipStream_t s);
int launch_topk(const float *logits, int T, int E, int k, int32_t *ids, float *w, hipStream_t s);
// bytes of scratch moe_route needs (0: none)
size_t route_ws_bytes(const bitmoe_layer *L, int T, int x_dtype);
bool route_uses_mfma(int T, int x_dtype);

// bucketing
struct Buckets {
    int32_t *counts;    // [E]
    int32_t *offsets;   // [E+1]
    int32_t *perm;      // [T*k]
    int32_t *active;    // [E]
    int32_t *n_active;  // [1]
    int32_t *tiles;     // [max_tiles][2] (expert, row0) or nullptr
    int32_t *n_tiles;   // [1] or nullptr
    int32_t *scratch;   // block histograms
    int tile_rows;      // rows per tile when tiles != nullptr
};
size_t bucket_scratch_bytes(int T, int k, int E);
int launch_bucket(const int32_t *ids, int T, int k, int E, const Buckets &b, hipStream_t s);
// the checked build (BITMOE_CHECK_IDS): *flag = the count of ids outside
// [0, E); a no-op otherwise
int launch_check_ids(const int32_t *ids, int64_t n, int E, int32_t *flag, hipStream_t s);
constexpr size_t kIdsFlagBytes = 256;        // at the start of the workspaces that take caller ids
#ifndef BITMOE_CHECK_IDS
#define BITMOE_CHECK_IDS 0
#endif

// decode FFN (three launches for decode batches, see decode.hip)
struct DecodePlan {
    int slots = 0;          // workgroup rows reserved for active experts
    int n_rwg = 0;          // router workgroups in the front launch (0: ids given)
    int kc_sg = 0;          // K chunks of the shared gate/up in the front launch (0: none there)
    int sg_rows = 0;        // > 0: one token, the shared gate/up inside the routed gate/up
                            // launch, sg_rows = 64/k rows of a panel per workgroup
    int front_waves = bm_cfg::kFrontWaves;   // waves per front workgroup (router rows: one per wave)
    int kc_sd = 0;          // K chunks of the shared down
    bool small = false;     // T*k <= kWaveBucketMax: one-wave bucketing
    bool need_mid = true;   // top-k and/or bucketing in a launch of their own
    int prep_wg = 0;        // preparation workgroups at the head of the front launch:
    bool bucket_in_front = false;   // the caller's ids bucketed there (no mid launch)
    bool xprep_in_front = false;    // the prefill kernels' fp16 activations, one workgroup per token
    int pf_tiles = 0;       // > 0: experts chosen by several tokens take the prefill
                            // kernels, one row tile each (at most pf_tiles tiles)
    bool fork = true;       // with pf_tiles: may fork onto the library's side stream
};
// Prefill working buffers (all device memory, carved from the workspace).
struct PrefillBufs {
    uint16_t *x16;      // [T][H] fp16 activations, scaled per token by 1/xsc
    float *xsc;         // [T] power-of-two token scales
    uint16_t *h;        // [T*k][I] fp16 h rows in bucket order, scaled per 256 columns
    int32_t *hexp;      // [T*k][I/256] exponents of those scales
    float *o;           // [T*k][H] per-pair expert outputs in fp32 (decode batches), or
    uint16_t *o16;      // [T*k][H] in fp16 (prefill) with
    int32_t *oexp;      // [T*k][ceil(H/512)] their power-of-two exponents
    float *hs, *os;     // shared expert h [T][I] and output [T][H] (or null)
};

struct DecodeBufs {
    float *logits;          // [T][E] (router in the front launch)
    int32_t *ids;           // [T][k]
    float *w;               // [T][k]
    Buckets bk;
    float *sgp;             // [kc_sg][2][T][I] shared gate/up partial sums
    uint16_t *hs;           // [2][T][I] shared h as bf16 hi, lo
    uint16_t *h;            // [T*k][I] routed h as fp16, scaled per 64 columns (bucket order)
    float2 *hsum2;          // [T*k][I/16] per 16 columns: {sum h, sum B_p h} of the scaled fp16 h
    float *hscale;          // [T*k][I/64] the power of two that undoes the scaling
    float *o;               // [T*k][H] routed down outputs, pair order
    float *osp;             // [kc_sd][T][H] shared down partial sums
    int32_t *ycount;        // [H/64] finished down workgroups per panel
    int4 *single;           // [slots] batches with the prefill kernels: the single-token experts, compacted
    int32_t *n_single;      // [1] their number
    int32_t *gctr;          // [1] their gate/up items claimed so far
    PrefillBufs pf;         // batches: experts chosen by several tokens take the prefill kernels
                            // (x16, xsc, h, hexp; their o is this o)
    float *y;               // [T][H]
};
// compute units of the current device (256 when the query fails)
int cu_count();
DecodePlan decode_plan(const bitmoe_layer *L, int T, bool with_router);
int launch_decode(const bitmoe_layer *L, const void *x, int x_dtype, int T, const DecodePlan &p,
                  const DecodeBufs &b, hipStream_t s);

// moe_forward_decode on a given workspace; fork = false keeps every launch
// on the caller's stream (no library stream is created or used).
// forward_decode_check validates every argument but the workspace and
// gives the workspace bytes the call needs.
int forward_decode_check(const bitmoe_layer *L, const void *x, int x_dtype, int T, const int32_t *ids,
                         const float *w, const float *y, size_t *ws_need);
int forward_decode(const bitmoe_layer *L, const void *x, int x_dtype, int T, int32_t *ids, float *w, float *y,
                   void *ws, size_t ws_bytes, void *stream, bool fork);

// prefill FFN
// xprep + routed gate/up + routed down over b's row tiles; o written per pair.
// parts: kPfPrep the activations' preparation only (it needs no routing),
// kPfRouted the rest, kPfAll both
enum { kPfPrep = 1, kPfRouted = 2, kPfAll = 3 };
int launch_prefill_routed(const bitmoe_layer *L, const void *x, int x_dtype, int T, const Buckets &b,
                          int max_tiles, const PrefillBufs &pb, hipStream_t s, int parts = kPfAll);
int launch_prefill_ffn(const bitmoe_layer *L, const void *x, int x_dtype, int T, const float *w, float *y,
                       const Buckets &b, int max_tiles, const PrefillBufs &pb, hipStream_t s);

// Events taken by the dispatch of one kernel at its start and end
// (moe_set_timing_events): `which` names the kernel (BITMOE_TIME_*).
struct TimingEvents {
    hipEvent_t start = nullptr, stop = nullptr;
    int which = 0;
};
TimingEvents &timing_events();
// the events for kernel `which`, or none
TimingEvents timing_for(int which);

}  // namespace bm_host

#define BM_LAUNCH_CHECK()                                      \
    do {                                                       \
        if (hipGetLastError() != hipSuccess) return BITMOE_EHIP; \
    } while (0)
