// C ABI of libbitmoe: host-side validation, workspace layout and launch
// orchestration.  Every check runs before the first launch, so a call that
// returns an error has queued nothing; the checks never touch the GPU and
// can be exercised without one.
#include <algorithm>
#include <cstdint>

#include "host.h"

namespace {

using bm_cfg::kFusedRouterMaxT;
// the decode front launch's router rows take at most 16 tokens per pass
static_assert(kFusedRouterMaxT <= 16, "router rows fused into the decode front launch: at most 16 tokens");

constexpr size_t kAlign = 256;
constexpr int kMaxT = 1 << 20;           // tokens per call

inline size_t up256(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

int check_layer_shape(const bitmoe_layer *L) {
    if (!L) return BITMOE_EINVAL;
    if (L->H <= 0 || L->I <= 0 || L->E <= 0 || L->k <= 0) return BITMOE_EINVAL;
    if (L->H % 256 || L->I % 256) return BITMOE_EUNSUPPORTED;
    if (L->k > 16 || L->k > L->E || L->E > 1024) return BITMOE_EUNSUPPORTED;
    return BITMOE_OK;
}

int check_ffn_layer(const bitmoe_layer *L) {
    int rc = check_layer_shape(L);
    if (rc) return rc;
    // the FFN kernels read the tiled layout only
    if (L->layout == BITMOE_LAYOUT_CANONICAL) return BITMOE_EUNSUPPORTED;
    if (L->layout != BITMOE_LAYOUT_TILED) return BITMOE_EINVAL;
    if (L->format != BITMOE_FORMAT_2BIT && L->format != BITMOE_FORMAT_MXFP4) return BITMOE_EINVAL;
    if (!L->gate_q || !L->up_q || !L->down_q) return BITMOE_EINVAL;
    if (L->format == BITMOE_FORMAT_2BIT && !L->grid) return BITMOE_EINVAL;
    const bool a = L->shared_gate, b = L->shared_up, c = L->shared_down;
    if (a != b || b != c) return BITMOE_EINVAL;
    return BITMOE_OK;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ---- workspace layouts -------------------------------------------------------

struct Carve {
    char *base;
    size_t off = 0;
    explicit Carve(void *b) : base(static_cast<char *>(b)) {}
    template <class T>
    T *take(size_t count) {
        T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
        off += up256(count * sizeof(T));
        return p;
    }
};

struct FfnWs {
    bm_host::Buckets b{};
    int max_tiles = 0;
    // prefill
    bm_host::PrefillBufs p{};
    // decode
    bm_host::DecodeBufs d{};
    void *route_ws = nullptr;      // moe_forward_decode, batches routed by moe_route
    size_t route_ws_bytes = 0;
    int32_t *ids_flag = nullptr;   // the checked build's count of caller ids outside [0, E)
    size_t bytes = 0;
};

FfnWs carve_ffn(const bitmoe_layer *L, int T, int mode, void *ws) {
    FfnWs f;
    Carve c(ws);
    const int64_t n = (int64_t)T * L->k;
    const bool shared = L->shared_gate != nullptr;
    f.ids_flag = reinterpret_cast<int32_t *>(c.take<char>(bm_host::kIdsFlagBytes));
    f.b.counts = c.take<int32_t>(L->E);
    f.b.offsets = c.take<int32_t>(L->E + 1);
    f.b.perm = c.take<int32_t>(std::max<int64_t>(n, 1));
    f.b.active = c.take<int32_t>(L->E);
    f.b.n_active = c.take<int32_t>(1);
    f.b.scratch = reinterpret_cast<int32_t *>(c.take<char>(bm_host::bucket_scratch_bytes(T, L->k, L->E)));
    if (mode == BITMOE_PREFILL) {
        f.b.tile_rows = bm_cfg::kPfRows;
        f.max_tiles = (int)((n + f.b.tile_rows - 1) / f.b.tile_rows + std::min<int64_t>(L->E, n));
        f.b.tiles = c.take<int32_t>(2 * std::max(f.max_tiles, 1));
        f.b.n_tiles = c.take<int32_t>(1);
        f.p.x16 = c.take<uint16_t>((int64_t)T * L->H);
        f.p.xsc = c.take<float>(T);
        f.p.h = c.take<uint16_t>(n * L->I);
        f.p.hexp = c.take<int32_t>(n * (L->I / 256));
        f.p.o16 = c.take<uint16_t>(n * L->H);
        f.p.oexp = c.take<int32_t>(n * ((L->H + bm_cfg::kPfDnCols - 1) / bm_cfg::kPfDnCols));
        if (shared) {
            f.p.hs = c.take<float>((int64_t)T * L->I);
            f.p.os = c.take<float>((int64_t)T * L->H);
        }
    } else {
        f.b.tile_rows = 1;
        const bm_host::DecodePlan p = bm_host::decode_plan(L, T, false);
        bm_host::DecodeBufs &d = f.d;
        d.logits = c.take<float>((int64_t)T * L->E);
        d.h = c.take<uint16_t>(n * L->I);
        d.hsum2 = c.take<float2>(n * (L->I / 16));
        d.hscale = c.take<float>(n * (L->I / 64));
        d.o = c.take<float>(n * L->H);
        d.ycount = c.take<int32_t>(L->H / 64);
        if (p.pf_tiles) {
            d.single = c.take<int4>(p.slots);
            d.n_single = c.take<int32_t>(1);
            d.gctr = c.take<int32_t>(1);
            f.b.tiles = c.take<int32_t>(2 * p.pf_tiles);
            f.b.n_tiles = c.take<int32_t>(1);
            d.pf.x16 = c.take<uint16_t>((int64_t)T * L->H);
            d.pf.xsc = c.take<float>(T);
            d.pf.h = c.take<uint16_t>(n * L->I);
            d.pf.hexp = c.take<int32_t>(n * (L->I / 256));
            d.pf.o = d.o;
        }
        if (shared) {
            d.sgp = c.take<float>((int64_t)p.kc_sg * 2 * T * L->I);
            d.hs = c.take<uint16_t>(2 * (int64_t)T * L->I);
            d.osp = c.take<float>((int64_t)p.kc_sd * T * L->H);
        }
        d.bk = f.b;
        if (T > kFusedRouterMaxT) {
            // the router's scratch for moe_forward_decode (the larger of
            // the two dtypes' needs)
            f.route_ws_bytes = bm_host::route_ws_bytes(L, T, BITMOE_BF16);
            f.route_ws = c.take<char>(f.route_ws_bytes);
        }
    }
    f.bytes = c.off;
    return f;
}

int check_ws(void *ws, size_t have, size_t need) {
    if (need == 0) return BITMOE_OK;
    if (!ws || have < need || !aligned(ws, kAlign)) return BITMOE_EWORKSPACE;
    return BITMOE_OK;
}

// Every argument but the workspace.
int ffn_args(const bitmoe_layer *L, const void *x, int x_dtype, int T, const int32_t *ids, const float *w,
             const float *y) {
    int rc = check_ffn_layer(L);
    if (rc) return rc;
    if (T < 0) return BITMOE_EINVAL;
    if (T > kMaxT) return BITMOE_EUNSUPPORTED;
    if (x_dtype != BITMOE_F32 && x_dtype != BITMOE_BF16) return BITMOE_EINVAL;
    if (T == 0) return BITMOE_OK;
    if (!x || !ids || !w || !y) return BITMOE_EINVAL;
    if (!aligned(x, 16) || !aligned(y, 16)) return BITMOE_EINVAL;
    return BITMOE_OK;
}

int ffn_common(const bitmoe_layer *L, const void *x, int x_dtype, int T, const int32_t *ids,
               const float *w, float *y, void *ws, size_t ws_bytes, int mode, FfnWs *out) {
    int rc = ffn_args(L, x, x_dtype, T, ids, w, y);
    if (rc || T == 0) return rc;
    FfnWs need = carve_ffn(L, T, mode, nullptr);
    rc = check_ws(ws, ws_bytes, need.bytes);
    if (rc) return rc;
    *out = carve_ffn(L, T, mode, ws);
    return BITMOE_OK;
}

}  // namespace

extern "C" {

int moe_set_timing_events(void *start, void *stop, int which) {
    if ((start == nullptr) != (stop == nullptr)) return BITMOE_EINVAL;
    if (which != BITMOE_TIME_GATEUP && which != BITMOE_TIME_DOWN) return BITMOE_EINVAL;
    bm_host::TimingEvents &ev = bm_host::timing_events();
    ev.start = static_cast<hipEvent_t>(start);
    ev.stop = static_cast<hipEvent_t>(stop);
    ev.which = which;
    return BITMOE_OK;
}

const char *moe_strerror(int code) {
    switch (code) {
        case BITMOE_OK: return "ok";
        case BITMOE_EINVAL: return "invalid argument (null pointer, bad dtype or mode, bad size or alignment)";
        case BITMOE_EUNSUPPORTED:
            return "unsupported shape, layout or size (H and I must be multiples of 256, 1<=k<=16, k<=E<=1024; "
                   "the FFN calls read TILED blocks; a cache map needs no more distinct experts than slots)";
        case BITMOE_EWORKSPACE: return "workspace missing, too small or not 256-byte aligned";
        case BITMOE_EHIP: return "a HIP kernel launch failed";
        case BITMOE_ESCRATCH:
            return "the call needs more scratch than the library's static array holds "
                   "(BITMOE_STATIC_SCRATCH_BYTES; use the entry point that takes a workspace)";
        default: return "unknown error code";
    }
}

const char *moe_version(void) {
    return BITMOE_CHECK_IDS ? "bitmoe 0.1.0 (gfx950, caller routing ids checked)" : "bitmoe 0.1.0 (gfx950)";
}

size_t moe_route_workspace_bytes(const bitmoe_layer *L, int T, int x_dtype) {
    if (check_layer_shape(L) || T <= 0) return 0;
    return bm_host::route_ws_bytes(L, T, x_dtype);
}

int moe_route(const bitmoe_layer *L, const void *x, int x_dtype, int T, float *logits, int32_t *ids,
              float *w, void *ws, size_t ws_bytes, void *stream) {
    int rc = check_layer_shape(L);
    if (rc) return rc;
    if (!L->router_w) return BITMOE_EINVAL;
    if (T < 0) return BITMOE_EINVAL;
    if (T > kMaxT) return BITMOE_EUNSUPPORTED;
    if (x_dtype != BITMOE_F32 && x_dtype != BITMOE_BF16) return BITMOE_EINVAL;
    if (T == 0) return BITMOE_OK;
    if (!x || !ids || !w || !aligned(x, 16)) return BITMOE_EINVAL;
    rc = check_ws(ws, ws_bytes, bm_host::route_ws_bytes(L, T, x_dtype));
    if (rc) return rc;
    hipStream_t s = as_stream(stream);
    float *part = static_cast<float *>(ws);
    if (bm_host::route_uses_mfma(T, x_dtype))
        return bm_host::launch_router_mfma(L, x, T, logits, ids, w, part, s);
    // one wave per expert row, token batches of kRouterNT
    const int NT = bm_cfg::kRouterNT;
    const size_t xs = x_dtype == BITMOE_BF16 ? 2 : 4;
    for (int t0 = 0; t0 < T; t0 += NT) {
        int nt = std::min(NT, T - t0);
        const char *xb = static_cast<const char *>(x) + (size_t)t0 * L->H * xs;
        float *lg = logits ? logits + (size_t)t0 * L->E : part;
        if ((rc = bm_host::launch_router_gemv(L, xb, x_dtype, nt, lg, s))) return rc;
        if ((rc = bm_host::launch_topk(lg, nt, L->E, L->k, ids + (size_t)t0 * L->k,
                                       w + (size_t)t0 * L->k, s)))
            return rc;
    }
    return BITMOE_OK;
}

int moe_topk(const float *logits, int T, int E, int k, int32_t *ids, float *w, void *stream) {
    if (T < 0 || E <= 0 || k <= 0) return BITMOE_EINVAL;
    if (k > 16 || k > E || E > 1024) return BITMOE_EUNSUPPORTED;
    if (T > kMaxT) return BITMOE_EUNSUPPORTED;
    if (T == 0) return BITMOE_OK;
    if (!logits || !ids || !w) return BITMOE_EINVAL;
    return bm_host::launch_topk(logits, T, E, k, ids, w, as_stream(stream));
}

size_t moe_bucket_workspace_bytes(int T, int k, int E) {
    if (T <= 0 || k <= 0 || E <= 0) return 0;
    return bm_host::kIdsFlagBytes + bm_host::bucket_scratch_bytes(T, k, E);
}

int moe_bucket(const int32_t *ids, int T, int k, int E, int32_t *counts, int32_t *offsets,
               int32_t *perm, int32_t *active, int32_t *n_active, void *ws, size_t ws_bytes,
               void *stream) {
    if (T < 0 || k <= 0 || E <= 0) return BITMOE_EINVAL;
    if (k > 16 || k > E || E > 1024 || T > kMaxT) return BITMOE_EUNSUPPORTED;
    if (T == 0) return BITMOE_OK;
    if (!ids || !counts || !offsets || !perm || !active || !n_active) return BITMOE_EINVAL;
    int rc = check_ws(ws, ws_bytes, bm_host::kIdsFlagBytes + bm_host::bucket_scratch_bytes(T, k, E));
    if (rc) return rc;
    bm_host::Buckets b{};
    b.counts = counts; b.offsets = offsets; b.perm = perm; b.active = active;
    b.n_active = n_active; b.tiles = nullptr; b.n_tiles = nullptr;
    b.scratch = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + bm_host::kIdsFlagBytes); b.tile_rows = 1;
    hipStream_t s = as_stream(stream);
    if ((rc = bm_host::launch_check_ids(ids, (int64_t)T * k, E, static_cast<int32_t *>(ws), s))) return rc;
    return bm_host::launch_bucket(ids, T, k, E, b, s);
}

size_t moe_workspace_bytes(const bitmoe_layer *L, int T, int mode) {
    if (check_ffn_layer(L) || T <= 0 || T > kMaxT) return 0;
    if (mode != BITMOE_DECODE && mode != BITMOE_PREFILL) return 0;
    return carve_ffn(L, T, mode, nullptr).bytes;
}

int moe_ffn_decode(const bitmoe_layer *L, const void *x, int x_dtype, int T, const int32_t *ids,
                   const float *w, float *y, void *ws, size_t ws_bytes, void *stream) {
    FfnWs f;
    int rc = ffn_common(L, x, x_dtype, T, ids, w, y, ws, ws_bytes, BITMOE_DECODE, &f);
    if (rc || T == 0) return rc;
    bm_host::DecodeBufs b = f.d;
    b.ids = const_cast<int32_t *>(ids);
    b.w = const_cast<float *>(w);
    b.y = y;
    hipStream_t s = as_stream(stream);
    if ((rc = bm_host::launch_check_ids(ids, (int64_t)T * L->k, L->E, f.ids_flag, s))) return rc;
    return bm_host::launch_decode(L, x, x_dtype, T, bm_host::decode_plan(L, T, false), b, s);
}

int moe_forward_decode(const bitmoe_layer *L, const void *x, int x_dtype, int T, int32_t *ids,
                       float *w, float *y, void *ws, size_t ws_bytes, void *stream) {
    return bm_host::forward_decode(L, x, x_dtype, T, ids, w, y, ws, ws_bytes, stream, true);
}

int moe_ffn_prefill(const bitmoe_layer *L, const void *x, int x_dtype, int T, const int32_t *ids,
                    const float *w, float *y, void *ws, size_t ws_bytes, void *stream) {
    FfnWs f;
    int rc = ffn_common(L, x, x_dtype, T, ids, w, y, ws, ws_bytes, BITMOE_PREFILL, &f);
    if (rc || T == 0) return rc;
    hipStream_t s = as_stream(stream);
    if ((rc = bm_host::launch_check_ids(ids, (int64_t)T * L->k, L->E, f.ids_flag, s))) return rc;
    if ((rc = bm_host::launch_bucket(ids, T, L->k, L->E, f.b, s))) return rc;
    return bm_host::launch_prefill_ffn(L, x, x_dtype, T, w, y, f.b, f.max_tiles, f.p, s);
}

int moe_dequant_iq2x(const void *blocks, const void *grid, int64_t nblocks, void *out, int out_dtype,
                     void *stream) {
    if (nblocks < 0) return BITMOE_EINVAL;
    if (out_dtype != BITMOE_F32 && out_dtype != BITMOE_BF16) return BITMOE_EINVAL;
    if (nblocks == 0) return BITMOE_OK;
    if (!blocks || !grid || !out || !aligned(blocks, 2) || !aligned(grid, 8) || !aligned(out, 16))
        return BITMOE_EINVAL;
    return bm_host::launch_dequant_iq2x(blocks, grid, nblocks, out, out_dtype, as_stream(stream));
}

int moe_dequant_q2k(const void *blocks, int64_t nblocks, void *out, int out_dtype, void *stream) {
    if (nblocks < 0) return BITMOE_EINVAL;
    if (out_dtype != BITMOE_F32 && out_dtype != BITMOE_BF16) return BITMOE_EINVAL;
    if (nblocks == 0) return BITMOE_OK;
    if (!blocks || !out || !aligned(blocks, 4) || !aligned(out, 16)) return BITMOE_EINVAL;
    return bm_host::launch_dequant_q2k(blocks, nblocks, out, out_dtype, as_stream(stream));
}

int moe_dequant_mxfp4(const void *blocks, int64_t nblocks, void *out, int out_dtype, void *stream) {
    if (nblocks < 0) return BITMOE_EINVAL;
    if (out_dtype != BITMOE_F32 && out_dtype != BITMOE_BF16) return BITMOE_EINVAL;
    if (nblocks == 0) return BITMOE_OK;
    if (!blocks || !out || !aligned(out, 16)) return BITMOE_EINVAL;
    return bm_host::launch_dequant_mxfp4(blocks, nblocks, out, out_dtype, as_stream(stream));
}

int moe_quantize_iq2x(const float *w, const void *grid, int64_t nblocks, void *blocks, void *stream) {
    if (nblocks < 0) return BITMOE_EINVAL;
    if (nblocks == 0) return BITMOE_OK;
    if (!w || !grid || !blocks || !aligned(w, 16) || !aligned(grid, 8)) return BITMOE_EINVAL;
    return bm_host::launch_quant_iq2x(w, grid, nblocks, blocks, as_stream(stream));
}

int moe_quantize_q2k(const float *w, int64_t nblocks, void *blocks, void *stream) {
    if (nblocks < 0) return BITMOE_EINVAL;
    if (nblocks == 0) return BITMOE_OK;
    if (!w || !blocks || !aligned(w, 16)) return BITMOE_EINVAL;
    return bm_host::launch_quant_q2k(w, nblocks, blocks, as_stream(stream));
}

int moe_quantize_mxfp4(const float *w, int64_t nblocks, void *blocks, void *stream) {
    if (nblocks < 0) return BITMOE_EINVAL;
    if (nblocks == 0) return BITMOE_OK;
    if (!w || !blocks || !aligned(w, 16)) return BITMOE_EINVAL;
    return bm_host::launch_quant_mxfp4(w, nblocks, blocks, as_stream(stream));
}

int moe_pack_iq2x(const void *src, void *dst, int E, int N, int K, void *stream) {
    if (E < 0 || N < 0 || K < 0) return BITMOE_EINVAL;
    if (N % 64 || K % 256) return BITMOE_EUNSUPPORTED;
    if ((int64_t)E * N * K == 0) return BITMOE_OK;
    if (!src || !dst || !aligned(src, 2) || !aligned(dst, 16)) return BITMOE_EINVAL;
    return bm_host::launch_pack_iq2x(src, dst, E, N, K, as_stream(stream));
}

int moe_pack_q2k(const void *src, void *dst, int E, int N, int K, void *stream) {
    if (E < 0 || N < 0 || K < 0) return BITMOE_EINVAL;
    if (N % 64 || K % 256) return BITMOE_EUNSUPPORTED;
    if ((int64_t)E * N * K == 0) return BITMOE_OK;
    if (!src || !dst || !aligned(src, 4) || !aligned(dst, 16)) return BITMOE_EINVAL;
    return bm_host::launch_pack_q2k(src, dst, E, N, K, as_stream(stream));
}

int moe_pack_mxfp4(const void *src, void *dst, int E, int N, int K, void *stream) {
    if (E < 0 || N < 0 || K < 0) return BITMOE_EINVAL;
    if (N % 64 || K % 256) return BITMOE_EUNSUPPORTED;
    if ((int64_t)E * N * K == 0) return BITMOE_OK;
    if (!src || !dst || !aligned(dst, 16)) return BITMOE_EINVAL;
    return bm_host::launch_pack_mxfp4(src, dst, E, N, K, as_stream(stream));
}

int moe_pack_bf16(const void *src, void *dst, int N, int K, void *stream) {
    if (N < 0 || K < 0) return BITMOE_EINVAL;
    if (N % 64 || K % 8) return BITMOE_EUNSUPPORTED;
    if ((int64_t)N * K == 0) return BITMOE_OK;
    if (!src || !dst || !aligned(src, 16) || !aligned(dst, 16)) return BITMOE_EINVAL;
    return bm_host::launch_pack_bf16(src, dst, N, K, as_stream(stream));
}

}  // extern "C"

namespace bm_host {

int forward_decode_check(const bitmoe_layer *L, const void *x, int x_dtype, int T, const int32_t *ids,
                         const float *w, const float *y, size_t *ws_need) {
    if (L && !L->router_w) return BITMOE_EINVAL;
    const int rc = ffn_args(L, x, x_dtype, T, ids, w, y);
    if (rc || T == 0) return rc;
    *ws_need = carve_ffn(L, T, BITMOE_DECODE, nullptr).bytes;
    return BITMOE_OK;
}

int forward_decode(const bitmoe_layer *L, const void *x, int x_dtype, int T, int32_t *ids, float *w, float *y,
                   void *ws, size_t ws_bytes, void *stream, bool fork) {
    if (L && !L->router_w) return BITMOE_EINVAL;
    FfnWs f;
    int rc = ffn_common(L, x, x_dtype, T, ids, w, y, ws, ws_bytes, BITMOE_DECODE, &f);
    if (rc || T == 0) return rc;
    hipStream_t s = as_stream(stream);
    DecodeBufs b = f.d;
    b.ids = ids;
    b.w = w;
    b.y = y;
    const bool fused = T <= kFusedRouterMaxT;
    if (!fused) {
        // the router's scratch is carved from the decode workspace
        rc = moe_route(L, x, x_dtype, T, nullptr, ids, w, f.route_ws, f.route_ws_bytes, stream);
        if (rc) return rc;
    }
    DecodePlan p = decode_plan(L, T, fused);
    p.fork = fork;
    return launch_decode(L, x, x_dtype, T, p, b, s);
}

}  // namespace bm_host
