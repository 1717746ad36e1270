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

// Packed fp16 pair dot product with fp32 accumulation (v_dot2_f32_f16).
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
BM_DEV float dot2_f16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
}

// ---- wave helpers -------------------------------------------------------

BM_DEV int lane_id() { return __lane_id(); }

BM_DEV float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Sum over each row of 16 lanes (DPP row shifts; out-of-row sources read 0),
// complete in lane 15 of the row.
template <int CTRL>
BM_DEV float dpp_shr_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
BM_DEV float row16_sum(float v) {
    v = dpp_shr_add<0x111>(v);
    v = dpp_shr_add<0x112>(v);
    v = dpp_shr_add<0x114>(v);
    return dpp_shr_add<0x118>(v);
}

BM_DEV float silu(float z) { return z / (1.0f + __expf(-z)); }

// ---- hand-over between workgroups of one launch -------------------------
// Data read by other workgroups of the same launch is written with
// device-scope (write-through) stores and read with device-scope loads; a
// workgroup waits for its stores to complete before it signals them.
BM_DEV void st_dev(float *p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
BM_DEV void st_dev(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
BM_DEV float ld_dev(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
BM_DEV uint32_t ld_dev(const uint32_t *p) {
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
BM_DEV void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---- tiled IQ2X group words ----------------------------------------------
// A tiled IQ2X group (32 weights, four runs of 8) is two little-endian
// 32-bit words, W0 for runs 0,1 and W1 for runs 2,3.  A run takes two
// bytes of its word, the first run bytes 0-1, the second bytes 2-3: the
// codebook index, then the stored signs of weights 0..6 (bit i set: weight
// i negative) in bits 0-6 and one bit of the 4-bit group scale in bit 7
// (scale bit 0 in byte 1 of W0, bit 1 in byte 3 of W0, bit 2 in byte 1 of
// W1, bit 3 in byte 3 of W1).  The sign of weight 7 makes the number of
// negative weights of the run even.  It is a bijective regrouping of the
// canonical 8 bytes of the group.
BM_DEV uint32_t iq2x_scale(uint32_t W0, uint32_t W1) {
    return ((W0 >> 15) & 1u) | ((W0 >> 30) & 2u) | ((W1 >> 13) & 4u) | ((W1 >> 28) & 8u);
}
// 2 s + 1 of the group scale s: the four scale bits spread to 0x00/0xFF
// bytes by one byte permute, weighted 2, 4, 8, 16 and summed
BM_DEV uint32_t iq2x_scale_odd(uint32_t W0, uint32_t W1) {
    const uint32_t m = __builtin_amdgcn_perm(W1, W0, 0x0B0A0908u);
    return __builtin_amdgcn_sad_u8(m & 0x10080402u, 0u, 1u);
}

// Run lookup tables in LDS.  Each 16-byte entry is kept in 16 copies, one
// per 16-byte slot of a 256-byte line (copy c of entry i at 256 i + 16 c),
// and lane l reads copy l & 15: a 16-lane group whose slots are distinct is
// served without bank conflicts whichever lines it touches, so random
// lookups run at the full LDS rate.
//  magnitudes (at 0, 256 entries): the 8 codebook magnitudes of row i as
//    16-bit floats (bf16 or fp16, both exact for bytes);
//  signs (at 64 KiB): for the sign byte i of a run (bit 7, the scale bit,
//    ignored), four XOR masks, bit 15 / bit 31 of mask p set when weight
//    2p / 2p+1 is negative.  Either all 256 byte values are present (64 KiB)
//    or the 128 without bit 7 (32 KiB; the offset is masked).
// XOR-ing mask p into magnitude word p gives the signed pair (w_2p, w_2p+1).
// The tables sit at LDS address 0 of kernels whose LDS is all dynamic (the
// host checks that they have no static LDS), and lookups read them through
// lds_ld16 at the computed offset as it is: reading through the extern
// array would add its base, a symbol resolved only at link time, with one
// more instruction per lookup.
BM_DEV uint4 lds_ld16(uint32_t a) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    const u32x4_t v = *(const __attribute__((address_space(3))) u32x4_t *)a;
    return make_uint4(v.x, v.y, v.z, v.w);
#else
    (void)a;               // device code only; the host pass sees this body
    return uint4{};
#endif
}
constexpr int kLutMagBytes = 65536;
constexpr int kLutSgnFull = 65536, kLutSgnHalf = 32768;
// per-lane constant of the offset permutes: the lane's slot, and byte 2 = 1
// for the sign table's base
BM_DEV uint32_t lut_lane_const(int lane) { return (uint32_t)(lane & 15) << 4 | 1u << 16; }
// byte offsets of the two lookups of run `second` of word W (one permute
// each: [slot, index byte, 0, 0] and [slot, sign byte, 1, 0])
BM_DEV uint32_t lut_mag_off(uint32_t W, uint32_t lc, int second) {
    return __builtin_amdgcn_perm(W, lc, second ? 0x0C0C0600u : 0x0C0C0400u);
}
BM_DEV uint32_t lut_sgn_off(uint32_t W, uint32_t lc, int second) {
    return __builtin_amdgcn_perm(W, lc, second ? 0x0C020700u : 0x0C020500u);
}
// entry `e` of the sign table: the 8 signs of the stored 7, as XOR masks
BM_DEV uint4 lut_sign_entry(uint32_t e) {
    const uint32_t s7 = e & 0x7Fu, sg = s7 | ((__popc(s7) & 1u) << 7);
    uint32_t m[4];
#pragma unroll
    for (int p = 0; p < 4; p++) m[p] = (((sg >> (2 * p)) & 1u) << 15) | (((sg >> (2 * p + 1)) & 1u) << 31);
    return make_uint4(m[0], m[1], m[2], m[3]);
}
// entry `e` of the magnitude table from the codebook row (8 bytes), as
// bf16 (BF = 1) or fp16 pairs
template <int BF>
BM_DEV uint4 lut_mag_from_row(uint2 g) {
    const uint32_t b[2] = {g.x, g.y};
    uint32_t m[4];
#pragma unroll
    for (int p = 0; p < 4; p++) {
        const uint32_t w = b[p >> 1] >> (16 * (p & 1));
        const float lo = (float)(w & 0xFFu), hi = (float)((w >> 8) & 0xFFu);
        if (BF) {
            m[p] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
        } else {
            m[p] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
        }
    }
    return make_uint4(m[0], m[1], m[2], m[3]);
}
template <int BF>
BM_DEV uint4 lut_mag_entry(const uint8_t *__restrict__ grid, uint32_t e) {
    return lut_mag_from_row<BF>(*reinterpret_cast<const uint2 *>(grid + 8 * e));
}
// The 16 copies of one line (entry `e` of the table at byte `base`), the
// c-th write to slot (c + e) & 15 so that the lanes of a write instruction
// (consecutive entries) hit distinct slots.
BM_DEV void lut_write_line(uint8_t *lut, int base, int e, uint4 v) {
    uint4 *line = reinterpret_cast<uint4 *>(lut + base + 256 * e);
#pragma unroll
    for (int c = 0; c < 16; c++) line[(c + e) & 15] = v;
}
// both tables (SGN = kLutSgnFull or kLutSgnHalf bytes of signs), by the
// threads of the workgroup: one line (16 copies of an entry) per thread
template <int BF, int SGN>
BM_DEV void lut_build(const uint8_t *__restrict__ grid, uint8_t *lut) {
    for (int e = threadIdx.x; e < 256 + SGN / 256; e += blockDim.x) {
        if (e < 256) lut_write_line(lut, 0, e, lut_mag_entry<BF>(grid, e));
        else lut_write_line(lut, kLutMagBytes, e - 256, lut_sign_entry(e - 256));
    }
}

// ---- tiled Q2K quant words -------------------------------------------------
// A tiled Q2K sub-block (16 weights) is one little-endian word: the 2-bit
// quants of the even-indexed weights 0,2,..,14 at bits 0-15 (weight 2p at
// bits 2p), those of the odd-indexed ones at bits 16-31 (weight 2p+1 at
// bits 16+2p).  Piece c (16 bytes) of a block holds sub-blocks 4c..4c+3.
BM_DEV uint32_t q2k_word_quant(uint32_t W, int i) { return (W >> (16 * (i & 1) + (i & ~1))) & 3u; }
// Weights 2p, 2p+1 of word W as the fp16 pair (B_p + q_2p, B_p + q_2p+1),
// B_p = 2^(10 - 2s), s = p for p < 5, else p - 5 (taken from W >> 10): the
// quants sit in the mantissa where one unit is 1, so only a mask and an OR
// are needed.  W10 = W >> 10.
template <int PAIR>
BM_DEV uint32_t q2k_pair_f16(uint32_t W, uint32_t W10) {
    constexpr int s = PAIR < 5 ? PAIR : PAIR - 5;
    constexpr uint32_t base = (uint32_t)(25 - 2 * s) << 10;     // fp16 bits of 2^(10 - 2s)
    return ((PAIR < 5 ? W : W10) & (0x00030003u << (2 * s))) | base | (base << 16);
}
// The 5 masks and 5 bases of q2k_pair_f16 held in registers, so that each
// pair is one v_and_or_b32 (a three-operand op takes no two literals).
struct Q2kPairConsts {
    uint32_t mask[5], base[5];
    BM_DEV Q2kPairConsts() {
#pragma unroll
        for (int s = 0; s < 5; s++) {
            uint32_t m = 0x00030003u << (2 * s), b = ((uint32_t)(25 - 2 * s) << 10) * 0x10001u;
            asm volatile("" : "+v"(m));
            asm volatile("" : "+s"(b));
            mask[s] = m;
            base[s] = b;
        }
    }
    template <int PAIR>
    BM_DEV uint32_t pair(uint32_t W, uint32_t W10) const {
        constexpr int s = PAIR < 5 ? PAIR : PAIR - 5;
        return ((PAIR < 5 ? W : W10) & mask[s]) | base[s];
    }
};
constexpr float q2k_pair_bias(int pair) { return (float)(1 << (10 - 2 * (pair < 5 ? pair : pair - 5))); }

// ---- small-T router row: one wave per expert row, lanes across K ---------
// The row is read in chunks (up to 8 loads of 16 bytes per lane, all in
// flight together), so one row costs about one memory round trip per chunk.
template <int XBF16, int NT>
BM_DEV float router_dot8(uint4 wv, const void *__restrict__ x, int H, int tt, int k, float a) {
    if (XBF16) {
        const uint4 xv = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + (int64_t)tt * H + k);
        a = dot2_bf16(wv.x, xv.x, a);
        a = dot2_bf16(wv.y, xv.y, a);
        a = dot2_bf16(wv.z, xv.z, a);
        a = dot2_bf16(wv.w, xv.w, a);
    } else {
        const float4 *xp = reinterpret_cast<const float4 *>(static_cast<const float *>(x) + (int64_t)tt * H + k);
        const float4 x0 = xp[0], x1 = xp[1];
        a = fmaf(bf16_lo(wv.x), x0.x, a); a = fmaf(bf16_hi(wv.x), x0.y, a);
        a = fmaf(bf16_lo(wv.y), x0.z, a); a = fmaf(bf16_hi(wv.y), x0.w, a);
        a = fmaf(bf16_lo(wv.z), x1.x, a); a = fmaf(bf16_hi(wv.z), x1.y, a);
        a = fmaf(bf16_lo(wv.w), x1.z, a); a = fmaf(bf16_hi(wv.w), x1.w, a);
    }
    return a;
}

template <int XBF16, int NT>
BM_DEV void router_row(const uint4 *__restrict__ wrow, const void *__restrict__ x, int H, int T,
                       int E, int e, float *__restrict__ logits) {
    constexpr int CH = NT == 1 ? 8 : NT <= 4 ? 4 : 2;
    const int lane = lane_id();
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = 0.f;
    const int steps = (H + 511) / 512;          // H is a multiple of 256
    for (int s0 = 0; s0 < steps; s0 += CH) {
        uint4 wv[CH];
#pragma unroll
        for (int i = 0; i < CH; i++) {
            // steps past the row, and the idle half-wave of a half-width
            // last step, re-read the row's first piece and are not used
            const int s = s0 + i, k = 512 * s + 8 * lane;
            wv[i] = wrow[(s < steps && k < H) ? 64 * s + lane : lane];
        }
        // every loaded piece is used (a branch around the extra ones would
        // let the compiler sink their loads next to the use); the extra
        // ones' sums are dropped
#pragma unroll
        for (int i = 0; i < CH; i++) {
            const int s = s0 + i, k = 512 * s + 8 * lane;
            const bool keep = s < steps && k < H;
            if (NT > 1 && !keep) continue;      // (more tokens: registers are short)
            const int kc = keep ? k : 8 * lane;
#pragma unroll
            for (int t = 0; t < NT; t++) {
                const float a = router_dot8<XBF16, NT>(wv[i], x, H, t < T ? t : 0, kc, acc[t]);
                acc[t] = keep ? a : acc[t];
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
size_t router_mfma_part_floats(int T, int E);
int launch_router_mfma(const bitmoe_layer *L, const void *x, int T, float *logits, int32_t *ids, float *w,
                       float *part, hipStream_t s);
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

// decode FFN (three launches for decode batches, see decode.hip)
struct DecodePlan {
    int slots = 0;          // workgroup rows reserved for active experts
    int n_rwg = 0;          // router workgroups in the front launch (0: ids given)
    int kc_sg = 0;          // K chunks of the shared gate/up
    int kc_sd = 0;          // K chunks of the shared down
    bool small = false;     // T*k <= 128: one-wave bucketing
    bool need_mid = true;   // top-k and/or bucketing in a launch of their own
    int pf_tiles = 0;       // > 0: experts chosen by several tokens take the prefill
                            // kernels, one row tile each (at most pf_tiles tiles)
};
// Prefill working buffers (all device memory, carved from the workspace).
struct PrefillBufs {
    uint16_t *x16;      // [T][H] fp16 activations, scaled per token by 1/xsc
    float *xsc;         // [T] power-of-two token scales
    uint16_t *h;        // [T*k][I] fp16 h rows in bucket order, scaled per 256 columns
    int32_t *hexp;      // [T*k][I/256] exponents of those scales
    float *o;           // [T*k][H] per-pair expert outputs
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
DecodePlan decode_plan(const bitmoe_layer *L, int T, bool with_router);
int launch_decode(const bitmoe_layer *L, const void *x, int x_dtype, int T, const DecodePlan &p,
                  const DecodeBufs &b, hipStream_t s);

// prefill FFN
int prefill_tile_rows();
// xprep + routed gate/up + routed down over b's row tiles; o written per pair
int launch_prefill_routed(const bitmoe_layer *L, const void *x, int x_dtype, int T, const Buckets &b,
                          int max_tiles, const PrefillBufs &pb, hipStream_t s);
int launch_prefill_ffn(const bitmoe_layer *L, const void *x, int x_dtype, int T, const float *w, float *y,
                       const Buckets &b, int max_tiles, const PrefillBufs &pb, hipStream_t s);

// events taken at the start and end of the gate/up launch (moe_set_timing_events)
struct TimingEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
TimingEvents &timing_events();

}  // namespace bm_host

#define BM_LAUNCH_CHECK()                                      \
    do {                                                       \
        if (hipGetLastError() != hipSuccess) return BITMOE_EHIP; \
    } while (0)
