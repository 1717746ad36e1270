// Launch planning: how a call is split into launches and how much scratch it
// needs.  Host code only (no kernels), shared by the C ABI's validation and
// workspace sizing and by the launchers.
#include <algorithm>
#include <atomic>

#include "host.h"

namespace bm_host {

using namespace bm_cfg;

int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

size_t bucket_scratch_bytes(int T, int k, int E) {
    const int64_t n = (int64_t)T * k;
    if (n <= kSmallPairs) return 256;
    const int64_t nblk = (n + kBT - 1) / kBT;
    return (size_t)(nblk * E * 4 + 255) / 256 * 256;
}

size_t router_mfma_part_floats(int T, int E) { return (size_t)kRouterSplit * T * E; }

bool route_uses_mfma(int T, int x_dtype) { return T >= kMfmaRouterMinT && x_dtype == BITMOE_BF16; }

size_t route_ws_bytes(const bitmoe_layer *L, int T, int x_dtype) {
    const size_t floats = route_uses_mfma(T, x_dtype) ? router_mfma_part_floats(T, L->E)
                                                     : (size_t)std::min(T, kRouterNT) * L->E;
    return (floats * 4 + 255) / 256 * 256;
}

DecodePlan decode_plan(const bitmoe_layer *L, int T, bool with_router) {
    DecodePlan p;
    const bool shared = L->shared_gate != nullptr;
    p.slots = (int)std::min<int64_t>(L->E, (int64_t)T * L->k);
    // one token, 2-bit experts: the k gate/up workgroups of a panel also take
    // 64/k of its shared rows each (k a power of two), streaming beside the
    // routed experts' decode, which is bound by its lookups and arithmetic;
    // the front launch then only computes the router logits, with small
    // workgroups spread over more CUs.  (The MXFP4 gate/up streams at the
    // memory's pace already: its shared gate/up stays in the front launch.)
    p.sg_rows = (shared && T == 1 && L->format == BITMOE_FORMAT_2BIT && L->k <= 16 && 64 % L->k == 0)
                    ? 64 / L->k : 0;
    p.front_waves = (T == 1 && (p.sg_rows || !shared)) ? kFrontRouterWaves : kFrontWaves;
    // router rows per front workgroup: one per wave for one token; for
    // several, kRouterRowWaves waves share a row (a quarter of K each), so
    // that the rows spread over four times the compute units
    const int rows_per_wg = T > 1 ? p.front_waves / kRouterRowWaves : p.front_waves;
    p.n_rwg = with_router ? (L->E + rows_per_wg - 1) / rows_per_wg : 0;
    p.kc_sd = shared ? std::max(1, (L->I + kSharedChunkCols - 1) / kSharedChunkCols) : 0;
    // one token: no more shared-down chunks than leave every down workgroup
    // (k routed + the shared chunks per 64 outputs) resident at once, so that
    // none waits for a second round at the end of the launch (when the routed
    // workgroups alone do not fit, the chunks stay as they are)
    if (shared && T == 1) {
        const int panels = L->H / 64, room = (cu_count() * kDownWavesPerSimd - p.slots * panels) / panels;
        if (room >= 1) p.kc_sd = std::min(p.kc_sd, room);
    }
    p.small = (int64_t)T * L->k <= kWaveBucketMax;
    // several tokens (one row tile per expert): experts chosen by more than
    // one token go through the prefill kernels, which decode each weight once
    // for all of its tokens on the matrix cores, beside the single-token
    // experts on a second stream.  Below kSplitMinT tokens few experts are
    // shared, and one decode launch for all experts (passes of up to four
    // tokens) is faster than the fork, the join and the extra launches.
    p.pf_tiles = (p.small && T >= kSplitMinT && T <= kPfRows) ? (int)std::min<int64_t>(L->E, (int64_t)T * L->k / 2)
                                                              : 0;
    // one token: every gate/up workgroup routes it itself.  More tokens: the
    // gate/up workgroups each take several (expert, panel) items from one
    // bucketing, done by the front launch's first workgroup when the caller
    // gives the ids, else (top-k of the router logits first) by a mid launch.
    // The prefill kernels' fp16 activations (2-bit experts) are prepared by
    // front workgroups too, one per token, up to kFrontPrepMaxT tokens.
    p.bucket_in_front = !with_router && T > 1 && p.small;
    p.xprep_in_front = p.pf_tiles > 0 && L->format == BITMOE_FORMAT_2BIT && T <= kFrontPrepMaxT;
    p.prep_wg = p.xprep_in_front ? T : p.bucket_in_front ? 1 : 0;
    p.need_mid = (!p.small || T > 1) && !p.bucket_in_front;
    // otherwise the shared gate/up's K chunks: as many as fit the compute
    // units beside the other front workgroups (one front workgroup per CU), at
    // most 8
    p.kc_sg = shared && !p.sg_rows
                  ? std::max(1, std::min(kMaxChunks, (cu_count() - p.n_rwg - p.prep_wg) / (L->I / 64)))
                  : 0;
    return p;
}

TimingEvents &timing_events() {
    thread_local TimingEvents ev;
    return ev;
}

TimingEvents timing_for(int which) {
    const TimingEvents &ev = timing_events();
    return ev.which == which ? ev : TimingEvents{};
}

}  // namespace bm_host
