// Prefill FFN: grouped GEMMs over the bucketed (token, expert) pairs with the
// routed weights dequantised to bf16 tiles in LDS feeding bf16 MFMA
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation).  Prefill is compute-bound
// (page "Faire tenir un MoE de 284B dans un portable de 128 Go", section "Un
// pre-remplissage a 790 t/s revele le veritable goulot d'etranglement"), so
// the dense contraction goes to the matrix cores.
//
// Work list: the bucketing pass emits tiles (expert e, first row r0) of up to
// BM rows of expert e's bucket; grid.y walks the tiles, grid.x the N tiles.
//  gate/up: A = gathered activation rows (bf16), B = [gate rows | up rows]
//           of the N tile, epilogue h = silu(g) * u (bf16, bucket order).
//  down:    A = h rows of the tile (contiguous), B = Q2K rows, epilogue
//           writes o[pair][n] (fp32); k_combine applies the routing weights.
#include <hip/hip_ext.h>

#include "common.h"

namespace {

using namespace bm;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 64;        // rows per tile (matches the bucket tile list)
constexpr int BK = 128;       // K per LDS stage (half a superblock)
constexpr int LDK = BK + 8;   // padded LDS row stride in bf16 elements

struct PrefillArgs {
    int H, I, k, T;
    const uint8_t *gate, *up, *down, *grid;
    const int32_t *counts, *offsets, *perm, *tiles, *n_tiles;
};

// --- B-tile dequantisation into LDS (bf16 = RNE of the exact fp32 value) ---

// 32 weights of IQ2X group g of block (n, kb) of one expert's tiled slab,
// without the superblock scale: +-(2s+1)*grid[idx][i].  With codebook
// magnitudes in {1,3,5,7} these are odd integers <= 217, exact in bf16; the
// factor d/8 is applied to the fp32 partial sums of each superblock.
BM_DEV void iq2x_group_int_to_lds(const uint8_t *slab, int nb, int n, int kb, int g,
                                  const uint2 *sgrid, uint16_t *dst) {
    const int P = n >> 6, r = n & 63;
    const int64_t pk = (int64_t)P * nb + kb;
    const uint2 gw = reinterpret_cast<const uint2 *>(slab)[((pk * 4 + (g >> 1)) * 64 + r) * 2 + (g & 1)];
    const float s2 = (float)(2u * iq2x_scale(gw.x, gw.y) + 1u);
    uint32_t out[16];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint32_t R = iq2x_run(j < 2 ? gw.x : gw.y, j & 1);
        const uint32_t sig = iq2x_run_signs(R);
        const uint2 row = sgrid[iq2x_run_idx(R)];
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            uint32_t m0 = ((i < 4 ? row.x : row.y) >> (8 * (i & 3))) & 0xFFu;
            uint32_t m1 = ((i < 4 ? row.x : row.y) >> (8 * ((i + 1) & 3))) & 0xFFu;
            uint32_t b0 = f32_to_bf16_rne(s2 * (float)m0) | (((sig >> i) & 1u) << 15);
            uint32_t b1 = f32_to_bf16_rne(s2 * (float)m1) | (((sig >> (i + 1)) & 1u) << 15);
            out[4 * j + i / 2] = b0 | (b1 << 16);
        }
    }
    uint4 *o = reinterpret_cast<uint4 *>(dst);
#pragma unroll
    for (int q = 0; q < 4; q++) o[q] = make_uint4(out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]);
}

// 16 weights of Q2K sub-block b of block (n, kb) without d and the min:
// scale*q, integers 0..45, exact in bf16.  The kernel applies d and the
// -dmin*min*sum(h) term to the fp32 partial sums of each superblock.
BM_DEV void q2k_sub_int_to_lds(const uint8_t *slab, int N, int nb, int n, int kb, int b, uint16_t *dst) {
    const int P = n >> 6, r = n & 63;
    const int64_t pk = (int64_t)P * nb + kb;
    const int64_t S = (int64_t)N * nb;
    const uint32_t W = reinterpret_cast<const uint32_t *>(slab)[((pk * 4 + (b >> 2)) * 64 + r) * 4 + (b & 3)];
    const float sc = (float)(slab[S * 64 + (pk * 64 + r) * 16 + b] & 15u);
    uint32_t out[8];
#pragma unroll
    for (int p = 0; p < 8; p++) {
        const uint32_t v0 = __float_as_uint(sc * (float)((W >> (2 * p)) & 3u)) >> 16;          // exact
        const uint32_t v1 = __float_as_uint(sc * (float)((W >> (16 + 2 * p)) & 3u)) >> 16;
        out[p] = v0 | (v1 << 16);
    }
    uint4 *o = reinterpret_cast<uint4 *>(dst);
    o[0] = make_uint4(out[0], out[1], out[2], out[3]);
    o[1] = make_uint4(out[4], out[5], out[6], out[7]);
}

// MFMA over one BK stage: wave computes 4 M-blocks x NB N-blocks.
template <int NB>
BM_DEV void mfma_stage(const uint16_t *sa, const uint16_t *sb, const int (&bcol)[NB],
                       f32x4 (&acc)[4][NB]) {
    const int lane = lane_id();
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
        const int kof = kk + 8 * (lane >> 4);
        bf16x8 fb[NB];
#pragma unroll
        for (int j = 0; j < NB; j++)
            fb[j] = *reinterpret_cast<const bf16x8 *>(sb + (bcol[j] + (lane & 15)) * LDK + kof);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            bf16x8 fa = *reinterpret_cast<const bf16x8 *>(sa + (16 * i + (lane & 15)) * LDK + kof);
#pragma unroll
            for (int j = 0; j < NB; j++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb[j], acc[i][j], 0, 0, 0);
        }
    }
}

// ---------------------------------------------------------------------------
// gate/up.  grid = (I/64, max_tiles), 256 threads.  N tile: h columns
// n0..n0+63; B rows 0-63 = gate rows n0.., 64-127 = up rows n0..
// ---------------------------------------------------------------------------
template <int XBF16>
__global__ void __launch_bounds__(256)
k_prefill_gateup(int H, int I, int k, const uint8_t *__restrict__ gate,
                 const uint8_t *__restrict__ up, const uint8_t *__restrict__ grid,
                 const void *__restrict__ x, const int32_t *__restrict__ counts,
                 const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm,
                 const int32_t *__restrict__ tiles, const int32_t *__restrict__ n_tiles,
                 uint16_t *__restrict__ h) {
    __shared__ __attribute__((aligned(16))) uint16_t sa[BM * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t sb[128 * LDK];
    __shared__ uint2 sgrid[256];
    __shared__ int stok[BM];
    const int tile = blockIdx.y;
    if (tile >= *n_tiles) return;
    const int e = tiles[2 * tile], r0 = tiles[2 * tile + 1];
    const int off = offsets[e], rows = min(BM, counts[e] - r0);
    const int n0 = blockIdx.x * 64;
    const int tid = threadIdx.x, lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int i = tid; i < 256; i += 256) sgrid[i] = reinterpret_cast<const uint2 *>(grid)[i];
    if (tid < BM) stok[tid] = perm[off + r0 + min(tid, rows - 1)] / k;
    const int nb = H / kQK;
    const int64_t slab = (int64_t)I * nb * 66;
    const uint8_t *G = gate + e * slab, *U = up + e * slab;
    const uint16_t *Gd = reinterpret_cast<const uint16_t *>(G + (int64_t)I * nb * 64);
    const uint16_t *Ud = reinterpret_cast<const uint16_t *>(U + (int64_t)I * nb * 64);
    const int ncol = n0 + 16 * wv + (lane & 15);          // this lane's output column
    const int64_t dbase = (int64_t)(ncol >> 6) * nb * 64 + (ncol & 63);
    f32x4 acc[4][2], part[4][2];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int bcol[2] = {16 * wv, 64 + 16 * wv};
    __syncthreads();
    for (int kb = 0; kb < nb; kb++) {
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) part[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int half = 0; half < 2; half++) {
            const int k0 = kb * kQK + half * BK;
            // A: 64 rows x 128 K -> 1024 pieces of 8 values, 4 per thread
#pragma unroll
            for (int p = 0; p < 4; p++) {
                int piece = tid + 256 * p, r = piece >> 4, c = (piece & 15) * 8;
                const int t = stok[r];
                uint4 v;
                if (XBF16) {
                    v = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + (int64_t)t * H + k0 + c);
                } else {
                    const float4 *xp = reinterpret_cast<const float4 *>(static_cast<const float *>(x) + (int64_t)t * H + k0 + c);
                    float4 a = xp[0], b = xp[1];
                    v = make_uint4(f32_to_bf16_rne(a.x) | (f32_to_bf16_rne(a.y) << 16),
                                   f32_to_bf16_rne(a.z) | (f32_to_bf16_rne(a.w) << 16),
                                   f32_to_bf16_rne(b.x) | (f32_to_bf16_rne(b.y) << 16),
                                   f32_to_bf16_rne(b.z) | (f32_to_bf16_rne(b.w) << 16));
                }
                *reinterpret_cast<uint4 *>(sa + r * LDK + c) = v;
            }
            // B: 128 rows x 4 groups = 512 (row, group) units, 2 per thread
#pragma unroll
            for (int p = 0; p < 2; p++) {
                int u = tid + 256 * p, row = u >> 2, gg = u & 3;
                const uint8_t *S = row < 64 ? G : U;
                iq2x_group_int_to_lds(S, nb, n0 + (row & 63), kb, 4 * half + gg, sgrid, sb + row * LDK + 32 * gg);
            }
            __syncthreads();
            mfma_stage<2>(sa, sb, bcol, part);
            __syncthreads();
        }
        const float dg = 0.125f * fp16_to_f32(Gd[dbase + (int64_t)kb * 64]);
        const float du = 0.125f * fp16_to_f32(Ud[dbase + (int64_t)kb * 64]);
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                acc[i][0][q] = fmaf(dg, part[i][0][q], acc[i][0][q]);
                acc[i][1][q] = fmaf(du, part[i][1][q], acc[i][1][q]);
            }
    }
    // epilogue: lane holds rows 4*(lane/16)+q of each M block, column lane%16
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
            int m = 16 * i + 4 * (lane >> 4) + q;
            if (m < rows) {
                float hv = silu(acc[i][0][q]) * acc[i][1][q];
                h[(int64_t)(off + r0 + m) * I + ncol] = (uint16_t)f32_to_bf16_rne(hv);
            }
        }
}

// ---------------------------------------------------------------------------
// down.  grid = (H/64, max_tiles), 256 threads.  A = h rows (bucket order).
// Per superblock: P = h . (scale*q) on MFMA, Pmin = Hsum . min on one more
// MFMA whose K slots hold the 16 sub-block sums of h split into bf16 high
// and low parts (so the min term keeps ~16 bits), then
// C += d * P - dmin * Pmin in fp32.
// ---------------------------------------------------------------------------
constexpr int HS_LD = 40;     // padded row stride of the sub-block sums (bf16)

__global__ void __launch_bounds__(256)
k_prefill_down(int H, int I, const uint8_t *__restrict__ down, const uint16_t *__restrict__ h,
               const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets,
               const int32_t *__restrict__ perm, const int32_t *__restrict__ tiles,
               const int32_t *__restrict__ n_tiles, float *__restrict__ o) {
    __shared__ __attribute__((aligned(16))) uint16_t sa[BM * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t sb[64 * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t hs[BM * HS_LD];
    const int tile = blockIdx.y;
    if (tile >= *n_tiles) return;
    const int e = tiles[2 * tile], r0 = tiles[2 * tile + 1];
    const int off = offsets[e], rows = min(BM, counts[e] - r0);
    const int n0 = blockIdx.x * 64;
    const int tid = threadIdx.x, lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nb = I / kQK;
    const int64_t S = (int64_t)H * nb;
    const uint8_t *D = down + (int64_t)e * S * 84;
    const int ncol = n0 + 16 * wv + (lane & 15);           // this lane's output column
    const int64_t pbase = (int64_t)(ncol >> 6) * nb * 64 + (ncol & 63);
    f32x4 acc[4][1], part[4][1];
#pragma unroll
    for (int i = 0; i < 4; i++) acc[i][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int bcol[1] = {16 * wv};
    for (int kb = 0; kb < nb; kb++) {
#pragma unroll
        for (int i = 0; i < 4; i++) part[i][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int half = 0; half < 2; half++) {
            const int k0 = kb * kQK + half * BK;
#pragma unroll
            for (int p = 0; p < 4; p++) {
                int piece = tid + 256 * p, r = piece >> 4, c = (piece & 15) * 8;
                int row = off + r0 + min(r, rows - 1);
                *reinterpret_cast<uint4 *>(sa + r * LDK + c) =
                    *reinterpret_cast<const uint4 *>(h + (int64_t)row * I + k0 + c);
            }
            // B: 64 rows x 8 sub-blocks (128 K) = 512 units, 2 per thread
#pragma unroll
            for (int p = 0; p < 2; p++) {
                int u = tid + 256 * p, row = u >> 3, sbk = u & 7;
                q2k_sub_int_to_lds(D, H, nb, n0 + row, kb, 8 * half + sbk, sb + row * LDK + 16 * sbk);
            }
            __syncthreads();
            // sums of 16 h values per (row, sub-block), split hi + lo
#pragma unroll
            for (int p = 0; p < 2; p++) {
                int u = tid + 256 * p, row = u >> 3, j = u & 7;
                const uint4 *src = reinterpret_cast<const uint4 *>(sa + row * LDK + 16 * j);
                uint4 a = src[0], b = src[1];
                uint32_t w8[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                float sum = 0.f;
#pragma unroll
                for (int q = 0; q < 8; q++) sum += bf16_lo(w8[q]) + bf16_hi(w8[q]);
                uint32_t hi = f32_to_bf16_rne(sum);
                uint32_t lo = f32_to_bf16_rne(sum - bf16_to_f32(hi));
                hs[row * HS_LD + 8 * half + j] = (uint16_t)hi;
                hs[row * HS_LD + 16 + 8 * half + j] = (uint16_t)lo;
            }
            mfma_stage<1>(sa, sb, bcol, part);
            __syncthreads();
        }
        // min term: K slots = [Hsum_hi 0..15 | Hsum_lo 0..15] x [min 0..15 | min 0..15]
        const int64_t pk = pbase + (int64_t)kb * 64;
        const int kg = lane >> 4;
        const uint2 scb = *reinterpret_cast<const uint2 *>(D + S * 64 + pk * 16 + 8 * (kg & 1));
        uint32_t mw[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            uint32_t word = q < 2 ? scb.x : scb.y;
            uint32_t m0 = (word >> (16 * (q & 1) + 4)) & 15u, m1 = (word >> (16 * (q & 1) + 12)) & 15u;
            mw[q] = (__float_as_uint((float)m0) >> 16) | (__float_as_uint((float)m1) & 0xFFFF0000u);
        }
        const bf16x8 fbm = __builtin_bit_cast(bf16x8, make_uint4(mw[0], mw[1], mw[2], mw[3]));
        const uint32_t dd = reinterpret_cast<const uint32_t *>(D + S * 80)[pk];
        const float d = fp16_to_f32(dd & 0xFFFFu), dmin = fp16_to_f32(dd >> 16);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const bf16x8 fam = *reinterpret_cast<const bf16x8 *>(hs + (16 * i + (lane & 15)) * HS_LD + 8 * kg);
            const f32x4 pm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fam, fbm, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4; q++) acc[i][0][q] = fmaf(d, part[i][0][q], fmaf(-dmin, pm[q], acc[i][0][q]));
        }
    }
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
            int m = 16 * i + 4 * (lane >> 4) + q;
            if (m < rows) o[(int64_t)perm[off + r0 + m] * H + ncol] = acc[i][0][q];
        }
}

// Shared expert for prefill-mode calls: dense bf16 FFN per token, one
// workgroup per (token, 64-row panel); simple and only used when a shared
// expert is supplied to the prefill entry point.
template <int XBF16>
__global__ void __launch_bounds__(64)
k_shared_gateup_rows(int H, int I, const uint4 *__restrict__ sg, const uint4 *__restrict__ su,
                     const void *__restrict__ x, float *__restrict__ hs) {
    const int P = blockIdx.x, t = blockIdx.y, lane = lane_id(), K8 = H / 8;
    float g = 0.f, u = 0.f;
    for (int c = 0; c < K8; c++) {
        uint4 gw = sg[((int64_t)P * K8 + c) * 64 + lane], uw = su[((int64_t)P * K8 + c) * 64 + lane];
        float xv[8];
        if (XBF16) {
            uint4 xb = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + (int64_t)t * H + 8 * c);
            uint32_t xw[4] = {xb.x, xb.y, xb.z, xb.w};
#pragma unroll
            for (int q = 0; q < 4; q++) { xv[2 * q] = bf16_lo(xw[q]); xv[2 * q + 1] = bf16_hi(xw[q]); }
        } else {
#pragma unroll
            for (int q = 0; q < 8; q++) xv[q] = static_cast<const float *>(x)[(int64_t)t * H + 8 * c + q];
        }
        uint32_t gg[4] = {gw.x, gw.y, gw.z, gw.w}, uu[4] = {uw.x, uw.y, uw.z, uw.w};
#pragma unroll
        for (int q = 0; q < 4; q++) {
            g = fmaf(bf16_lo(gg[q]), xv[2 * q], g); g = fmaf(bf16_hi(gg[q]), xv[2 * q + 1], g);
            u = fmaf(bf16_lo(uu[q]), xv[2 * q], u); u = fmaf(bf16_hi(uu[q]), xv[2 * q + 1], u);
        }
    }
    hs[(int64_t)t * I + P * 64 + lane] = silu(g) * u;
}

__global__ void __launch_bounds__(64)
k_shared_down_rows(int H, int I, const uint4 *__restrict__ sd, const float *__restrict__ hs,
                   float *__restrict__ os) {
    const int P = blockIdx.x, t = blockIdx.y, lane = lane_id(), K8 = I / 8;
    float acc = 0.f;
    for (int c = 0; c < K8; c++) {
        uint4 wv = sd[((int64_t)P * K8 + c) * 64 + lane];
        uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
        const float *hp = hs + (int64_t)t * I + 8 * c;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            acc = fmaf(bf16_lo(ww[q]), hp[2 * q], acc);
            acc = fmaf(bf16_hi(ww[q]), hp[2 * q + 1], acc);
        }
    }
    os[(int64_t)t * H + P * 64 + lane] = acc;
}

__global__ void __launch_bounds__(256)
k_combine_p(const float *__restrict__ o, const float *__restrict__ w, const float *__restrict__ os,
            float *__restrict__ y, int T, int H, int k) {
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * H) return;
    int t = (int)(i / H), n = (int)(i % H);
    float s = 0.f;
    for (int j = 0; j < k; j++) s = fmaf(w[t * k + j], o[((int64_t)t * k + j) * H + n], s);
    if (os) s += os[i];
    y[i] = s;
}

}  // namespace

namespace bm_host {

int prefill_tile_rows() { return BM; }

int launch_prefill_ffn(const bitmoe_layer *L, const void *x, int x_dtype, int T, const int32_t *ids,
                       const float *w, float *y, const Buckets &b, int max_tiles, uint16_t *xb,
                       uint16_t *h, float *o, float *hs, float *os, hipStream_t s) {
    (void)ids; (void)xb;
    const int H = L->H, I = L->I, k = L->k;
    dim3 g1(I / 64, max_tiles);
    {
        // the timing events, when set, are taken by the dispatch itself
        const TimingEvents ev = timing_events();
        auto kg = x_dtype == BITMOE_BF16 ? k_prefill_gateup<1> : k_prefill_gateup<0>;
        hipExtLaunchKernelGGL(kg, g1, dim3(256), 0, s, ev.start, ev.stop, 0, H, I, k, (const uint8_t *)L->gate_q,
                              (const uint8_t *)L->up_q, (const uint8_t *)L->grid, x, (const int32_t *)b.counts,
                              (const int32_t *)b.offsets, (const int32_t *)b.perm, (const int32_t *)b.tiles,
                              (const int32_t *)b.n_tiles, h);
        BM_LAUNCH_CHECK();
    }
    dim3 g2(H / 64, max_tiles);
    k_prefill_down<<<g2, 256, 0, s>>>(H, I, (const uint8_t *)L->down_q, h, b.counts, b.offsets, b.perm,
                                      b.tiles, b.n_tiles, o);
    BM_LAUNCH_CHECK();
    const bool shared = L->shared_gate != nullptr;
    if (shared) {
        dim3 gs1(I / 64, T), gs2(H / 64, T);
        if (x_dtype == BITMOE_BF16)
            k_shared_gateup_rows<1><<<gs1, 64, 0, s>>>(H, I, (const uint4 *)L->shared_gate,
                                                       (const uint4 *)L->shared_up, x, hs);
        else
            k_shared_gateup_rows<0><<<gs1, 64, 0, s>>>(H, I, (const uint4 *)L->shared_gate,
                                                       (const uint4 *)L->shared_up, x, hs);
        BM_LAUNCH_CHECK();
        k_shared_down_rows<<<gs2, 64, 0, s>>>(H, I, (const uint4 *)L->shared_down, hs, os);
        BM_LAUNCH_CHECK();
    }
    int64_t n = (int64_t)T * H;
    k_combine_p<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(o, w, shared ? os : nullptr, y, T, H, k);
    BM_LAUNCH_CHECK();
    return BITMOE_OK;
}

}  // namespace bm_host
