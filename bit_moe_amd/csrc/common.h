// Internal helpers shared by the HIP sources of libbitmoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bitmoe.h"

#define BM_DEV __device__ __forceinline__

namespace bm {

constexpr int kWave = 64;           // CDNA wavefront width
constexpr int kPanel = 64;          // rows per tiled panel (= lanes per wave)
constexpr int kQK = 256;            // weights per superblock

// ---- scalar conversions -------------------------------------------------

BM_DEV float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
BM_DEV float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
BM_DEV float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

BM_DEV float fp16_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
BM_DEV uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Packed bf16 pair dot product with fp32 accumulation (v_dot2c_f32_bf16).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
BM_DEV float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), acc, false);
}

// ---- wave helpers -------------------------------------------------------

BM_DEV int lane_id() { return __lane_id(); }

BM_DEV float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

BM_DEV float silu(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace bm

// ---- host-side launchers (defined in the .hip files) ----------------------

namespace bm_host {

int launch_dequant_iq2x(const void *blocks, const void *grid, int64_t nblocks,
                        void *out, int out_dtype, hipStream_t s);
int launch_dequant_q2k(const void *blocks, int64_t nblocks, void *out,
                       int out_dtype, hipStream_t s);
int launch_pack_iq2x(const void *src, void *dst, int E, int N, int K, hipStream_t s);
int launch_pack_q2k(const void *src, void *dst, int E, int N, int K, hipStream_t s);
int launch_pack_bf16(const void *src, void *dst, int N, int K, hipStream_t s);

// router logits [T][E] fp32 for at most router_tokens_per_launch() tokens
int router_tokens_per_launch();
int launch_router_gemv(const bitmoe_layer *L, const void *x, int x_dtype, int T,
                       float *logits, hipStream_t s);
int launch_router_mfma(const bitmoe_layer *L, const void *x, int T, float *logits,
                       hipStream_t s);
int launch_topk(const float *part, int KS, int T, int E, int k, float *logits,
                int32_t *ids, float *w, hipStream_t s);

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

// decode FFN
int launch_decode_ffn(const bitmoe_layer *L, const void *x, int x_dtype, int T,
                      const int32_t *ids, const float *w, float *y,
                      const Buckets &b, float *h, float *hsum, float *o,
                      float *hs, float *os, hipStream_t s);

// prefill FFN
int prefill_tile_rows();
int launch_prefill_ffn(const bitmoe_layer *L, const void *x, int x_dtype, int T,
                       const int32_t *ids, const float *w, float *y,
                       const Buckets &b, int max_tiles, uint16_t *xb, uint16_t *h,
                       float *o, float *hs, float *os, hipStream_t s);

// events recorded around the gate/up launch (moe_set_timing_events)
struct TimingEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
TimingEvents &timing_events();
inline void timing_begin(hipStream_t s) {
    if (timing_events().start) (void)hipEventRecord(timing_events().start, s);
}
inline void timing_end(hipStream_t s) {
    if (timing_events().stop) (void)hipEventRecord(timing_events().stop, s);
}

}  // namespace bm_host

#define BM_LAUNCH_CHECK()                                      \
    do {                                                       \
        if (hipGetLastError() != hipSuccess) return BITMOE_EHIP; \
    } while (0)
