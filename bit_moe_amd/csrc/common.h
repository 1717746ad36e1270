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

// ---- tiled IQ2X group fields ---------------------------------------------
// A tiled IQ2X group is four little-endian 16-bit fields F_j (run j of 8
// weights): bits 8-15 the codebook index; bits 4-6 the signs of weights
// 0,1,2 and bit 7 the parity of the signs of weights 0..3; bits 1-3 the
// signs of weights 4,5,6; bit 0 bit j of the 4-bit group scale.  The sign
// of weight 3 is bit7 ^ bits 4..6 and that of weight 7 (even parity over
// the 8) is bit7 ^ bits 1..3.  It is a bijective re-encoding of the
// canonical 8 bytes.
//
// Decode tables (LDS): a 64 KiB main table of 16-byte entries, one per
// (index, F bits 4-7): the 8 magnitudes as bf16 with the signs of weights
// 0..3 applied and weight 7 signed by the parity bit; and an 8-entry mask
// table (F bits 1-3) that flips the signs of weights 4..7.
constexpr int kIq2xMainEntries = 4096;            // uint4 entries
constexpr int kIq2xMaskBytes = 64;                // after the main table
BM_DEV uint32_t iq2x_main_off(uint32_t F) { return F & 0xFFF0u; }
BM_DEV uint32_t iq2x_mask_off(uint32_t F) { return (F << 2) & 0x38u; }
// 4-bit group scale from the two words W0 = F0 | F1 << 16, W1 = F2 | F3 << 16
BM_DEV uint32_t iq2x_scale(uint32_t W0, uint32_t W1) {
    return (W0 & 1u) | ((W0 >> 15) & 2u) | ((W1 & 1u) << 2) | ((W1 >> 13) & 8u);
}
// signs of the 8 weights of a run (bit i = weight i negative)
BM_DEV uint32_t iq2x_signs(uint32_t F) {
    const uint32_t lo3 = (F >> 4) & 7u, hi3 = (F >> 1) & 7u, p = (F >> 7) & 1u;
    const uint32_t s3 = p ^ (__popc(lo3) & 1u), s7 = p ^ (__popc(hi3) & 1u);
    return lo3 | (s3 << 3) | (hi3 << 4) | (s7 << 7);
}
// main table entry e: index e >> 4, F bits 4-7 = e & 15
BM_DEV uint4 iq2x_main_entry(const uint8_t *__restrict__ grid, int e) {
    const int idx = e >> 4;
    const uint32_t q = e & 15, p = q >> 3;
    const uint32_t lo3 = q & 7u;
    const uint32_t signs = lo3 | ((p ^ (__popc(lo3) & 1u)) << 3) | (p << 7);
    const uint2 m8 = *reinterpret_cast<const uint2 *>(grid + 8 * idx);
    uint32_t v[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const uint32_t m = ((i < 4 ? m8.x : m8.y) >> (8 * (i & 3))) & 0xFFu;
        v[i] = (__float_as_uint((float)m) >> 16) | (((signs >> i) & 1u) << 15);   // exact
    }
    return make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
}
// mask table entry m (F bits 1-3): sign flips of weights 4,5 / 6,7
BM_DEV uint2 iq2x_mask_entry(int m) {
    const uint32_t b4 = m & 1, b5 = (m >> 1) & 1, b6 = (m >> 2) & 1;
    return make_uint2((b4 << 15) | (b5 << 31), (b6 << 15) | ((b4 ^ b5 ^ b6) << 31));
}

// ---- small-T router row: one wave per expert row, lanes across K ---------
template <int XBF16, int NT>
BM_DEV void router_row(const uint4 *__restrict__ wrow, const void *__restrict__ x, int H, int T,
                       int E, int e, float *__restrict__ logits) {
    const int lane = lane_id();
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = 0.f;
    const int steps = (H + 511) / 512;          // H is a multiple of 256
#pragma unroll 2
    for (int s = 0; s < steps; s++) {
        const int k = 512 * s + 8 * lane;
        if (k >= H) break;                       // only in a half-width last step
        const uint4 wv = wrow[64 * s + lane];
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const int tt = t < T ? t : 0;
            if (XBF16) {
                const uint4 xv = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + (int64_t)tt * H + k);
                float a = acc[t];
                a = dot2_bf16(wv.x, xv.x, a);
                a = dot2_bf16(wv.y, xv.y, a);
                a = dot2_bf16(wv.z, xv.z, a);
                a = dot2_bf16(wv.w, xv.w, a);
                acc[t] = a;
            } else {
                const float4 *xp = reinterpret_cast<const float4 *>(static_cast<const float *>(x) + (int64_t)tt * H + k);
                const float4 x0 = xp[0], x1 = xp[1];
                float a = acc[t];
                a = fmaf(bf16_lo(wv.x), x0.x, a); a = fmaf(bf16_hi(wv.x), x0.y, a);
                a = fmaf(bf16_lo(wv.y), x0.z, a); a = fmaf(bf16_hi(wv.y), x0.w, a);
                a = fmaf(bf16_lo(wv.z), x1.x, a); a = fmaf(bf16_hi(wv.z), x1.y, a);
                a = fmaf(bf16_lo(wv.w), x1.z, a); a = fmaf(bf16_hi(wv.w), x1.w, a);
                acc[t] = a;
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; t++) {
        const float v = wave_sum(acc[t]);
        if (lane == 0 && t < T) logits[(int64_t)t * E + e] = v;
    }
}

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
int launch_topk(const float *logits, int T, int E, int k, int32_t *ids, float *w, hipStream_t s);

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

// decode FFN (four launches, see decode.hip)
struct DecodePlan {
    int slots = 0;          // workgroup rows reserved for active experts
    int n_rwg = 0;          // router workgroups in the front launch (0: ids given)
    int kc_sg = 0;          // K chunks of the shared gate/up
    int kc_sd = 0;          // K chunks of the shared down
    bool bucket_in_mid = true;
};
struct DecodeBufs {
    float *logits;          // [T][E] (router in the front launch)
    int32_t *ids;           // [T][k]
    float *w;               // [T][k]
    Buckets bk;
    float *sgp;             // [kc_sg][2][T][I] shared gate/up partial sums
    uint16_t *hs;           // [2][T][I] shared h as bf16 hi, lo
    uint16_t *h;            // [2][T*k][I] routed h as bf16 hi, lo (bucket order, quads [0,2,1,3])
    float *hsum;            // [T*k][I/16]
    float *o;               // [T*k][H] routed down outputs, pair order
    float *osp;             // [kc_sd][T][H] shared down partial sums
    uint4 *tab;             // IQ2X decode tables (64 KiB + 64 B)
    float *y;               // [T][H]
};
DecodePlan decode_plan(const bitmoe_layer *L, int T, bool with_router);
int launch_decode(const bitmoe_layer *L, const void *x, int x_dtype, int T, const DecodePlan &p,
                  const DecodeBufs &b, hipStream_t s);

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
