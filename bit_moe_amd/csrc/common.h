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

BM_DEV uint32_t f16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// ---- fp16 activations for the matrix-core kernels ------------------------
// Each token row goes to fp16 times 2^-e, one power of two e per token, so
// that the row's largest |x| lands in [2^14, 2^15): any bf16/fp32 range then
// maps onto fp16's normal range (0, inf and NaN give e = 0).
BM_DEV int pf_exponent(float m) {
    const uint32_t u = __float_as_uint(m);
    if (!(m > 0.f) || u >= 0x7F800000u) return 0;
    const int ex = (int)(u >> 23) - 127;
    return max(ex - 14, -100);
}
struct Xp8 { float v[8]; };
// 8 consecutive activations at element offset i (bf16 or fp32), as fp32
template <int XBF16>
BM_DEV Xp8 xprep_load8(const void *x, int64_t i) {
    Xp8 r;
    if (XBF16) {
        const uint4 q = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + i);
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; j++) { r.v[2 * j] = bf16_lo(w[j]); r.v[2 * j + 1] = bf16_hi(w[j]); }
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(x) + i);
        const float4 a = p[0], b = p[1];
        r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
        r.v[4] = b.x; r.v[5] = b.y; r.v[6] = b.z; r.v[7] = b.w;
    }
    return r;
}
BM_DEV float xprep_absmax8(const Xp8 &a) {
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 8; j++) m = fmaxf(m, fabsf(a.v[j]));
    return m;
}
BM_DEV void xprep_store8(uint16_t *dst, const Xp8 &a, int e) {
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; j++) o[j] = f16_bits(ldexpf(a.v[2 * j], -e)) | (f16_bits(ldexpf(a.v[2 * j + 1], -e)) << 16);
    *reinterpret_cast<uint4 *>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
}
// One token row on one workgroup (H a multiple of 8; sm holds a float per
// wave).  Every thread calls it: it holds a block barrier.
template <int XBF16>
BM_DEV void xprep_token_block(int H, const void *x, int t, uint16_t *x16, float *xsc, float *sm) {
    const int tid = threadIdx.x, nt = blockDim.x, nw = nt / kWave;
    const int64_t row = (int64_t)t * H;
    // the thread's first kHold pieces are loaded together and kept in
    // registers for the second pass (H 7168 on 256 threads: all of them)
    constexpr int kHold = 4;
    Xp8 hv[kHold];
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < kHold; i++) {
        const int c = (tid + i * nt) * 8;
        if (c < H) {
            hv[i] = xprep_load8<XBF16>(x, row + c);
            m = fmaxf(m, xprep_absmax8(hv[i]));
        }
    }
    for (int c = (tid + kHold * nt) * 8; c < H; c += nt * 8) m = fmaxf(m, xprep_absmax8(xprep_load8<XBF16>(x, row + c)));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    if ((tid & (kWave - 1)) == 0) sm[tid / kWave] = m;
    __syncthreads();
    m = 0.f;
    for (int w = 0; w < nw; w++) m = fmaxf(m, sm[w]);
    const int e = pf_exponent(m);
    if (tid == 0) xsc[t] = ldexpf(1.f, e);
#pragma unroll
    for (int i = 0; i < kHold; i++) {
        const int c = (tid + i * nt) * 8;
        if (c < H) xprep_store8(x16 + row + c, hv[i], e);
    }
    for (int c = (tid + kHold * nt) * 8; c < H; c += nt * 8) xprep_store8(x16 + row + c, xprep_load8<XBF16>(x, row + c), e);
}

// ---- MXFP4 (OCP Microscaling: E2M1 elements, one E8M0 scale per 32) -----
// v_cvt_scalef32_pk_{bf16,f16,f32}_fp4: byte SEL of w holds two E2M1
// elements, the first in its low nibble; the result holds element * scale
// for both, the first in the low half, rounded to nearest-even (exact in
// fp32, and in bf16 / fp16 within range).  The instruction reads the scale
// operand's exponent field as an E8M0 value, so the fp32 bit pattern X << 23
// stands for 2^(X-127) for every X, 0 and 255 (NaN) included.
BM_DEV float mx_cvt_scale(uint32_t X) { return __uint_as_float(X << 23); }
template <int SEL>
BM_DEV uint32_t fp4x2_bf16s(uint32_t w, float scale) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL));
}
template <int SEL>
BM_DEV uint32_t fp4x2_f16s(uint32_t w, float scale) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, SEL));
}
template <int SEL>
BM_DEV float2 fp4x2_f32s(uint32_t w, float scale) {
    const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, SEL);
    return make_float2(v[0], v[1]);
}
// the two elements themselves (scale 1)
template <int SEL>
BM_DEV uint32_t fp4x2_bf16(uint32_t w) { return fp4x2_bf16s<SEL>(w, 1.f); }
template <int SEL>
BM_DEV uint32_t fp4x2_f16(uint32_t w) { return fp4x2_f16s<SEL>(w, 1.f); }
// The block scale 2^(X-127) as fp32: X << 23 for X = 1..254, the subnormal
// 2^-127 for X = 0 and NaN for X = 255 (both take mantissa bit 22).
BM_DEV float mx_scale(uint32_t X) {
    return __uint_as_float((X << 23) | ((((X + 1u) & 0xFEu) == 0u) ? 0x400000u : 0u));
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
// A tiled Q2K sub-block (16 weights) is one little-endian word whose byte s
// (0..3) holds the 2-bit quants of weights 2s and 2s+1 in bits 0-1 and 4-5,
// and those of weights 8+2s and 9+2s in bits 2-3 and 6-7.  Masking the word
// (q2k_lo: weights 0..7, q2k_hi: weights 8..15) leaves in each byte two
// nibbles that are E2M1 codes 0..3, whose values are q/2; the hardware
// conversion at scale 2 then gives each consecutive pair as exact fp16 quants.
// Piece c (16 bytes) of a block holds sub-blocks 4c..4c+3.
BM_DEV int q2k_word_shift(int i) { return 8 * ((i & 7) >> 1) + 4 * (i & 1) + 2 * (i >> 3); }
BM_DEV uint32_t q2k_word_quant(uint32_t W, int i) { return (W >> q2k_word_shift(i)) & 3u; }
BM_DEV uint32_t q2k_lo(uint32_t W) { return W & 0x33333333u; }
BM_DEV uint32_t q2k_hi(uint32_t W) { return (W >> 2) & 0x33333333u; }
// (q_{2S}, q_{2S+1}) of a masked word as an fp16 pair (E2M1 scale 2^1)
template <int S>
BM_DEV uint32_t q2k_pair_f16(uint32_t spread) { return fp4x2_f16s<S>(spread, 2.f); }

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
    const int spare = lane < H / 8 ? lane : 0;
    for (int s0 = 0; s0 < steps; s0 += CH) {
        uint4 wv[CH];
#pragma unroll
        for (int i = 0; i < CH; i++) {
            // steps past the row, and the idle half-wave of a half-width
            // last step, re-read a piece of the row's first step and are not used
            const int s = s0 + i, k = 512 * s + 8 * lane;
            wv[i] = wrow[(s < steps && k < H) ? 64 * s + lane : spare];
        }
        // every loaded piece is used (a branch around the extra ones would
        // let the compiler sink their loads next to the use); the extra
        // ones' sums are dropped
#pragma unroll
        for (int i = 0; i < CH; i++) {
            const int s = s0 + i, k = 512 * s + 8 * lane;
            const bool keep = s < steps && k < H;
            if (NT > 1 && !keep) continue;      // (more tokens: registers are short)
            const int kc = keep ? k : 8 * spare;
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

#include "host.h"
