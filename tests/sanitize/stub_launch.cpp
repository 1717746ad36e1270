// Launcher stand-ins for the host sanitizer build of the C ABI (test
// infrastructure): the validation, planning and workspace code of api.cpp
// and plan.cpp run for real; every launcher reports a failed launch instead
// of queueing kernels, so nothing touches a GPU.
#include "../../bit_moe_amd/csrc/host.h"

namespace bm_host {

int launch_dequant_iq2x(const void *, const void *, int64_t, void *, int, hipStream_t) { return BITMOE_EHIP; }
int launch_dequant_q2k(const void *, int64_t, void *, int, hipStream_t) { return BITMOE_EHIP; }
int launch_quant_iq2x(const float *, const void *, int64_t, void *, hipStream_t) { return BITMOE_EHIP; }
int launch_quant_q2k(const float *, int64_t, void *, hipStream_t) { return BITMOE_EHIP; }
int launch_quant_mxfp4(const float *, int64_t, void *, hipStream_t) { return BITMOE_EHIP; }
int launch_pack_iq2x(const void *, void *, int, int, int, hipStream_t) { return BITMOE_EHIP; }
int launch_pack_q2k(const void *, void *, int, int, int, hipStream_t) { return BITMOE_EHIP; }
int launch_pack_bf16(const void *, void *, int, int, hipStream_t) { return BITMOE_EHIP; }
int launch_dequant_mxfp4(const void *, int64_t, void *, int, hipStream_t) { return BITMOE_EHIP; }
int launch_pack_mxfp4(const void *, void *, int, int, int, hipStream_t) { return BITMOE_EHIP; }
int launch_router_gemv(const bitmoe_layer *, const void *, int, int, float *, hipStream_t) { return BITMOE_EHIP; }
int launch_router_mfma(const bitmoe_layer *, const void *, int, float *, int32_t *, float *, float *, hipStream_t) {
    return BITMOE_EHIP;
}
int launch_topk(const float *, int, int, int, int32_t *, float *, hipStream_t) { return BITMOE_EHIP; }
int launch_bucket(const int32_t *, int, int, int, const Buckets &, hipStream_t) { return BITMOE_EHIP; }
// (a release build queues nothing here)
int launch_check_ids(const int32_t *, int64_t, int, int32_t *, hipStream_t) { return BITMOE_OK; }
int launch_decode(const bitmoe_layer *, const void *, int, int, const DecodePlan &, const DecodeBufs &, hipStream_t) {
    return BITMOE_EHIP;
}
int launch_prefill_routed(const bitmoe_layer *, const void *, int, int, const Buckets &, int, const PrefillBufs &,
                          hipStream_t, int) {
    return BITMOE_EHIP;
}
int launch_prefill_ffn(const bitmoe_layer *, const void *, int, int, const float *, float *, const Buckets &, int,
                       const PrefillBufs &, hipStream_t) {
    return BITMOE_EHIP;
}

}  // namespace bm_host
