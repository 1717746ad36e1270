// Prefill FFN: grouped GEMMs over the bucketed (token, expert) rows on the
// matrix cores.  Prefill is compute-bound (page "Faire tenir un MoE de 284B
// dans un portable de 128 Go", section "Un pre-remplissage a 790 t/s revele
// le veritable goulot d'etranglement"), so the contraction runs on
// v_mfma_f32_32x32x16_f16 with fp32 accumulation (on gfx950 the 32x32 shape
// issues at the full matrix rate from one wave and leaves room for the
// dequantisation VALU work between MFMAs; 16x16x32 reaches about 80%).
//
// Operands.  Activations enter as fp16 scaled by a power of two per token
// (k_pf_xprep), so any bf16/fp32 range maps onto fp16's normal range; the
// scale is undone in fp32 after the contraction.  Weights are dequantised
// straight into MFMA operand registers, never to memory: each lane owns the
// eight K slots of one codebook run (IQ2X) or of half a Q2K sub-block and
// builds its fp16 operand with one packed fp16 op per weight pair (IQ2X:
// w = c * (+-m), c = d/8 (2s+1) folded per group; Q2K: w = a q - b with
// a = d sc, b = dmin m per sub-block).  The K order inside a stage is
// permuted so that a lane's slots follow the packed layout; the activation
// tile in LDS is read with the same permutation, so the products pair up.
//
// IQ2X runs decode through two LDS tables: the codebook row of the run's
// index as 8 fp16 magnitudes, and the run's 7 stored sign bits (parity signs
// included) as 4 XOR masks over the fp16 pairs.  Both are kept in 16 copies,
// one per 16-byte slot of a 256-byte line, and lane l reads slot l & 15: on
// gfx950 a 16-lane group whose slots are distinct is served without bank
// conflicts whatever lines it touches, so the random lookups run at full
// LDS rate (random 8-byte lookups into one copy lose about half to conflicts).
//
// Work list: the bucketing pass emits tiles (expert e, first row r0) of up to
// 96 rows of e's bucket; a tile runs ceil(rows/32) row blocks (a compile-time
// count chosen per tile).  Workgroups are numbered so that all N-tiles of one
// M-tile land on the same XCD (round-robin dispatch), which keeps the
// activation rows they share in that XCD's L2.
//  gate/up: 8 waves x 32 h columns (gate and up blocks of the same columns
//           in one lane), epilogue h = silu(g) u stored as fp16 with one
//           power-of-two exponent per (row, 256 columns).
//  down:    16 waves x 32 output columns, A = h rows rescaled per 256-column
//           chunk to the row's largest exponent while staged into LDS;
//           epilogue writes o[pair][n] as fp16 with one power-of-two
//           exponent per (pair, 512 columns) (fp32 for decode batches);
//           k_combine_p applies the routing weights.
// MXFP4 routed experts (k_mx_*) keep this tiling and pipeline on the bf16
// matrix cores, with operands from the hardware E2M1 conversion (below).
#include <hip/hip_ext.h>

#include <type_traits>

#include "device_util.h"

namespace {

using namespace bm;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPfWaves = 8;
constexpr int kPfThreads = kPfWaves * kWave;
using bm_cfg::kPfRows;                        // rows per tile (3 blocks of 32)
constexpr int kPfHalf = 128;                  // K per LDS stage
// Activation stage in LDS, chunk-major: 16-byte chunk c (8 K values) of row m
// at (c * kPfRows + m) * 16.  An MFMA operand read (16 lanes = 16 rows of one
// chunk) and a staging write (8 rows x 2 chunks per 16 lanes) then touch
// contiguous 128-byte runs, which gfx950's LDS serves without bank conflicts
// (row-strided layouts, padded or XOR-swizzled, cost 4 extra cycles per read).
constexpr int kPfGuCols = 256;                // h columns per gate/up workgroup
using bm_cfg::kPfDnCols;                      // output columns per down workgroup (one 32-column block per wave)
constexpr int kPfXcds = 8;
constexpr int kPfMagBytes = kLutMagBytes;       // 256 codebook rows x 16 copies x 16 bytes
constexpr int kPfSgnBytes = kLutSgnHalf;        // 128 sign patterns x 16 copies x 16 bytes
constexpr int kPfTabBytes = kPfMagBytes + kPfSgnBytes;
constexpr int kPfABytes = kPfRows * kPfHalf * 2;
constexpr int kPfGuLds = kPfTabBytes + 2 * kPfABytes + kPfRows * (4 + 4 + 4) + kPfWaves * kPfRows * 4;
// fp16 weight operands carry a factor 2^kPfWShift (IQ2X) or 2^kPfDnWShift
// (Q2K), removed in the fp32 epilogues: with it a superblock scale d (and
// dmin) in [2^-19, 8] keeps every nonzero weight in fp16's normal range and
// below its largest finite value.  IQ2X weights lie in [d/8, 217 d/8] (group
// scale (0.5+s)/4 <= 31/8, magnitude <= 7): times 2^8, [2^-14, 55552] at the
// ends of the range.  Q2K terms d sc q <= 45 d and dmin m <= 15 dmin: times
// 2^7, at most 46080, and the smallest nonzero term d sc (or dmin m) is
// 2^-12; a q - b is formed in one fused fp16 operation, so its only
// rounding is that of the result.
constexpr int kPfWShift = 8;
constexpr float kPfWScale = 256.f;
constexpr int kPfDnWShift = 7;
constexpr float kPfDnWScale = 128.f;
static_assert(kPfWScale == (float)(1 << kPfWShift) && kPfDnWScale == (float)(1 << kPfDnWShift), "scale factors");

BM_DEV uint32_t h2u(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
BM_DEV f16x2 u2h(uint32_t v) { return __builtin_bit_cast(f16x2, v); }
BM_DEV uint32_t f16_pair(float f) { const uint32_t b = f16_bits(f); return b | (b << 16); }
BM_DEV uint32_t pk_mul(uint32_t a, uint32_t b) { return h2u(u2h(a) * u2h(b)); }

// fp16 bits of 2^d, d <= 0 (subnormal below 2^-14, zero below 2^-24)
BM_DEV uint32_t f16_pow2(int d) {
    if (d >= -14) return (uint32_t)(15 + d) << 10;
    if (d >= -24) return 1u << (d + 24);
    return 0u;
}

// ---- workgroup -> (M-tile, N-tile), all N-tiles of an M-tile on one XCD ----
struct PfSlot { int tile, ntile; };
BM_DEV PfSlot pf_slot(int nN) {
    const int b = blockIdx.x, xcd = b % kPfXcds, slot = b / kPfXcds;
    return {(slot / nN) * kPfXcds + xcd, slot % nN};
}
int pf_grid(int max_tiles, int nN) { return (max_tiles + kPfXcds - 1) / kPfXcds * kPfXcds * nN; }

// ---------------------------------------------------------------------------
// activations -> fp16, one power-of-two scale per token.  grid = T, 256 thr.
// (decode batches that take these kernels do the same in their front launch)
// ---------------------------------------------------------------------------
template <int XBF16>
__global__ void __launch_bounds__(256)
k_pf_xprep(int H, const void *__restrict__ x, uint16_t *__restrict__ x16, float *__restrict__ xsc) {
    __shared__ float sm[4];
    xprep_token_block<XBF16>(H, x, blockIdx.x, x16, xsc, sm);
}

// ---------------------------------------------------------------------------
// gate/up.  512 threads; wave w owns h columns hc0 + 32w .. +31: blocks 0,1
// are the gate rows of those columns, blocks 2,3 the up rows.
// ---------------------------------------------------------------------------

// The LDS decode tables (layout in common.h): magnitudes as fp16 pairs, and
// the 128 sign entries without the scale bit (32 KiB).  Threads 0..255 each
// write the 16 copies of one magnitude line, threads 256..383 those of one
// sign line.
BM_DEV void pf_build_tables(const uint8_t *__restrict__ grid, uint8_t *lds) {
    const int t = threadIdx.x;
    if (t < 256) lut_write_line(lds, 0, t, lut_mag_entry<0>(grid, t));
    else if (t < 384) lut_write_line(lds, kPfMagBytes, t - 256, lut_sign_entry(t - 256));
}

// Table lookups of run `second` of word W (magnitudes, sign masks); lc =
// lut_lane_const(lane).  The sign offset drops the scale bit (bit 15).
struct RunLut { u32x4 m, g; };
BM_DEV RunLut pf_iq2x_lookup(const uint8_t *lds, uint32_t W, int second, uint32_t lc) {
    (void)lds;
    const uint4 m = lds_ld16(lut_mag_off(W, lc, second)), g = lds_ld16(lut_sgn_off(W, lc, second) & ~0x8000u);
    return {u32x4{m.x, m.y, m.z, m.w}, u32x4{g.x, g.y, g.z, g.w}};
}
// fp16 operand (8 weights, K order) of a looked-up run, times the group's c2
BM_DEV f16x8 pf_iq2x_build(const RunLut &l, uint32_t c2) {
    const uint4 v = make_uint4(pk_mul(c2, l.m.x ^ l.g.x), pk_mul(c2, l.m.y ^ l.g.y), pk_mul(c2, l.m.z ^ l.g.z),
                               pk_mul(c2, l.m.w ^ l.g.w));
    return __builtin_bit_cast(f16x8, v);
}

struct PfTile {
    int e, r0, off, rows;
};
BM_DEV PfTile pf_tile(int tile, const int32_t *tiles, const int32_t *counts, const int32_t *offsets) {
    PfTile t;
    t.e = tiles[2 * tile];
    t.r0 = tiles[2 * tile + 1];
    t.off = offsets[t.e];
    t.rows = min(kPfRows, counts[t.e] - t.r0);
    return t;
}

struct GuArgs {
    int H, I, k;
    const uint8_t *gate, *up, *grid;
    const uint16_t *x16;
    const float *xsc;
    const int32_t *counts, *offsets, *perm, *tiles, *n_tiles;
    uint16_t *h;
    int32_t *hexp;
};

// Activation stages (gate/up: x16 rows, down: h rows) go global -> registers
// -> LDS, chunk-major with R rows: 16-byte chunk c (8 K values) of row m at
// (c R + m) * 16.  R rows x 16 chunks = R/32 loads of 16 bytes per thread,
// each group of 64 lanes taking 8 rows x 8 chunks (a 16-lane group then
// writes two contiguous 128-byte runs).  Operand reads (32 rows of one chunk
// per half-wave) touch contiguous 256-byte runs: no bank conflicts.
struct StageIdx { int row, c; };
BM_DEV StageIdx stage_idx(int p) {
    const int u = threadIdx.x + kPfThreads * p, q = u >> 6, l = u & 63;
    return {8 * (q >> 1) + (l & 7), 8 * (q & 1) + (l >> 3)};
}
template <int R>
BM_DEV void stage_store(uint8_t *dst, const u32x4 (&r)[R / 32]) {
#pragma unroll
    for (int p = 0; p < R / 32; p++) {
        const StageIdx x = stage_idx(p);
        *reinterpret_cast<u32x4 *>(dst + (x.c * R + x.row) * 16) = r[p];
    }
}
template <int R>
BM_DEV void gu_stage_load(const GuArgs &a, const int *stok, int kb, int hf, u32x4 (&r)[R / 32]) {
    const int k0 = kb * kQK + hf * kPfHalf;
#pragma unroll
    for (int p = 0; p < R / 32; p++) {
        const StageIdx x = stage_idx(p);
        r[p] = *reinterpret_cast<const u32x4 *>(a.x16 + (int64_t)stok[x.row] * a.H + k0 + 8 * x.c);
    }
}
// MFMA A operand (32 rows x 16 K): rows 32i + (lane & 31), chunk 8 (lane >> 5) + t
template <int R>
BM_DEV f16x8 frag32(const uint8_t *buf, int i, int lane, int t) {
    return *reinterpret_cast<const f16x8 *>(buf + ((8 * (lane >> 5) + t) * R + 32 * i + (lane & 31)) * 16);
}
BM_DEV f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }
// row of accumulator register r of a 32x32 block in lane half kh
BM_DEV int acc_row(int r, int kh) { return 8 * (r >> 2) + 4 * kh + (r & 3); }

// ---- the stage pipeline of every grouped-GEMM tile ----------------------------
// Stage st (128 K) runs its MFMAs from LDS activation buffer st & 1.  At its
// start it loads the activation pieces of stage st + AHEAD into registers
// (load_a) and the weight slot of stage st + 2 (load_slot); after its MFMAs
// (compute) it writes the activations of stage st + 1 into the other buffer
// (put_a), then a barrier.  AHEAD = 2 keeps two register sets, alternating by
// stage, so that each activation load has two stages' compute to arrive.
// The issue order is pinned (activations, then the slot), so that the wait
// before put_a leaves the slot in flight (memory counters retire in issue
// order).  Slots and register sets rotate by call, never by copy (a copy
// would wait for the loads), and the stages whose prefetches are all in
// range carry no conditionals (a conditional load path there breaks the
// issue order and the compiler then drains every load).
// pre() runs after the prologue's loads are issued and before the first
// put_a: set-up that the first put_a needs may overlap those loads.
struct NoPre {
    BM_DEV void operator()() const {}
};
template <int AHEAD, class Regs, class Slot, class LoadA, class PutA, class LoadSlot, class Compute,
          class Pre = NoPre>
BM_DEV void run_stages(int nsteps, LoadA &&load_a, PutA &&put_a, LoadSlot &&load_slot, Compute &&compute,
                       Pre &&pre = Pre{}) {
    static_assert(AHEAD == 1 || AHEAD == 2, "activation prefetch depth");
    Regs ra, rb;
    Slot q0, q1, q2;
    auto stage = [&](auto full, int st, Slot &cur, Slot &pre, Regs &ld, Regs &sv) {
        const int s1 = st + 1, s2 = st + 2, sa = st + AHEAD;
        asm volatile("" ::: "memory");
        if (full || sa < nsteps) load_a(sa, ld);
        asm volatile("" ::: "memory");
        if (full || s2 < nsteps) load_slot(s2, pre);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        compute(st & 1, cur);
        if (full || s1 < nsteps) put_a(s1 & 1, sv);
        __syncthreads();
    };
    using Full = std::integral_constant<bool, true>;
    using Part = std::integral_constant<bool, false>;
    load_a(0, ra);
    if (AHEAD == 2) load_a(1, rb);
    load_slot(0, q0);
    load_slot(1, q1);                    // nsteps >= 2: K is a multiple of 256
    pre();
    put_a(0, ra);
    // drain the prologue loads: otherwise the compiler merges their pending
    // state into the loop header and waits on the current slot every pass
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int st = 0;
    if constexpr (AHEAD == 1) {
        for (; st + 5 <= nsteps; st += 3) {
            stage(Full{}, st, q0, q2, ra, ra);
            stage(Full{}, st + 1, q1, q0, ra, ra);
            stage(Full{}, st + 2, q2, q1, ra, ra);
        }
        // at most 4 stages remain; the slot rotation continues from q0
        if (st < nsteps) stage(Part{}, st, q0, q2, ra, ra);
        if (st + 1 < nsteps) stage(Part{}, st + 1, q1, q0, ra, ra);
        if (st + 2 < nsteps) stage(Part{}, st + 2, q2, q1, ra, ra);
        if (st + 3 < nsteps) stage(Part{}, st + 3, q0, q2, ra, ra);
    } else {
        for (; st + 8 <= nsteps; st += 6) {
            stage(Full{}, st, q0, q2, ra, rb);
            stage(Full{}, st + 1, q1, q0, rb, ra);
            stage(Full{}, st + 2, q2, q1, ra, rb);
            stage(Full{}, st + 3, q0, q2, rb, ra);
            stage(Full{}, st + 4, q1, q0, ra, rb);
            stage(Full{}, st + 5, q2, q1, rb, ra);
        }
        // at most 7 stages remain
        if (st < nsteps) stage(Part{}, st, q0, q2, ra, rb);
        if (st + 1 < nsteps) stage(Part{}, st + 1, q1, q0, rb, ra);
        if (st + 2 < nsteps) stage(Part{}, st + 2, q2, q1, ra, rb);
        if (st + 3 < nsteps) stage(Part{}, st + 3, q0, q2, rb, ra);
        if (st + 4 < nsteps) stage(Part{}, st + 4, q1, q0, ra, rb);
        if (st + 5 < nsteps) stage(Part{}, st + 5, q2, q1, rb, ra);
        if (st + 6 < nsteps) stage(Part{}, st + 6, q0, q2, ra, rb);
    }
}

// ---------------------------------------------------------------------------
// gate/up.  512 threads; wave w owns h columns hc0 + 32w .. +31: block 0 the
// gate rows, block 1 the up rows of those columns (lane & 31 = column).  In a
// stage (half superblock, 4 groups) lane half kh takes groups 2kh, 2kh+1 -
// one 16-byte piece of the tiled slab - k-step t being run t & 3 of group
// 2kh + (t >> 2), i.e. stage K offset 64 kh + 8 t.
// ---------------------------------------------------------------------------
template <int MB>
BM_DEV void gu_tile(const GuArgs &a, uint8_t *lds, const PfTile &t, int ntile) {
    constexpr int R = 32 * MB;
    uint8_t *const sa = lds + kPfTabBytes;              // A buffer b at sa + b * kPfABytes
    int *stok = reinterpret_cast<int *>(lds + kPfTabBytes + 2 * kPfABytes);
    float *sxs = reinterpret_cast<float *>(stok + kPfRows);
    int *sexp = reinterpret_cast<int *>(sxs + kPfRows);
    float *smax = reinterpret_cast<float *>(sexp + kPfRows);
    const int lane = lane_id(), col = lane & 31, kh = lane >> 5;
    const uint32_t lc = lut_lane_const(lane);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nb = a.H / kQK;
    const int64_t slab = (int64_t)a.I * nb * 66;
    const uint8_t *G = a.gate + t.e * slab, *U = a.up + t.e * slab;
    const int hc = ntile * kPfGuCols + 32 * w + col, P = hc >> 6, pr = hc & 63;
    // byte offsets at superblock 0, half 0 (one expert's slab is below 4 GiB)
    const uint32_t qoff = (uint32_t)((P * nb * 4 + kh) * 64 + pr) * 16;
    const uint32_t doff = (uint32_t)a.I * nb * 64 + (uint32_t)(P * nb * 64 + pr) * 2;
    struct Slot { uint4 g, u; uint32_t dg, du; };       // words of one stage + raw fp16 d
    auto load_slot = [&](int st, Slot &sl) {
        const uint32_t o = qoff + (st >> 1) * 4096 + (st & 1) * 2048, od = doff + (st >> 1) * 128;
        sl.g = *reinterpret_cast<const uint4 *>(G + o);
        sl.u = *reinterpret_cast<const uint4 *>(U + o);
        sl.dg = *reinterpret_cast<const uint16_t *>(G + od);
        sl.du = *reinterpret_cast<const uint16_t *>(U + od);
    };
    f32x16 acc[MB][2];
#pragma unroll
    for (int i = 0; i < MB; i++) acc[i][0] = acc[i][1] = (f32x16)0.f;
    // One stage: 8 k-steps.  K-step s reads its activation operands first,
    // then issues the table lookups of k-step s+2 (LDS reads retire in issue
    // order, so the MFMAs of s wait only for their own operands while the
    // lookups stay in flight), then builds its weight operands from the
    // lookups issued two k-steps earlier and runs its MFMAs.
    auto compute = [&](const uint8_t *A, const Slot &sl) {
        // c = d/8 (2s+1) per (block, group) as fp16 pairs
        const float dg = 0.125f * kPfWScale * fp16_to_f32(sl.dg), du = 0.125f * kPfWScale * fp16_to_f32(sl.du);
        const uint32_t c2[2][2] = {{f16_pair(dg * (float)iq2x_scale_odd(sl.g.x, sl.g.y)),
                                    f16_pair(dg * (float)iq2x_scale_odd(sl.g.z, sl.g.w))},
                                   {f16_pair(du * (float)iq2x_scale_odd(sl.u.x, sl.u.y)),
                                    f16_pair(du * (float)iq2x_scale_odd(sl.u.z, sl.u.w))}};
        auto word = [&](const uint4 &v, int s) {
            const int q = s >> 2, rr = s & 3;
            return rr < 2 ? (q ? v.z : v.x) : (q ? v.w : v.y);
        };
        RunLut lg[8], lu[8];
        lg[0] = pf_iq2x_lookup(lds, word(sl.g, 0), 0, lc);
        lu[0] = pf_iq2x_lookup(lds, word(sl.u, 0), 0, lc);
        lg[1] = pf_iq2x_lookup(lds, word(sl.g, 1), 1, lc);
        lu[1] = pf_iq2x_lookup(lds, word(sl.u, 1), 1, lc);
#pragma unroll
        for (int s = 0; s < 8; s++) {
            f16x8 av[MB];
#pragma unroll
            for (int i = 0; i < MB; i++) av[i] = frag32<R>(A, i, lane, s);
            if (s + 2 < 8) {
                lg[s + 2] = pf_iq2x_lookup(lds, word(sl.g, s + 2), (s + 2) & 1, lc);
                lu[s + 2] = pf_iq2x_lookup(lds, word(sl.u, s + 2), (s + 2) & 1, lc);
            }
            const f16x8 bg = pf_iq2x_build(lg[s], c2[0][s >> 2]);
            const f16x8 bu = pf_iq2x_build(lu[s], c2[1][s >> 2]);
#pragma unroll
            for (int i = 0; i < MB; i++) {
                acc[i][0] = mfma32(av[i], bg, acc[i][0]);
                acc[i][1] = mfma32(av[i], bu, acc[i][1]);
            }
        }
    };
    struct ARegs { u32x4 r[R / 32]; };
    run_stages<2, ARegs, Slot>(
        2 * nb, [&](int st, ARegs &v) { gu_stage_load<R>(a, stok, st >> 1, st & 1, v.r); },
        [&](int buf, ARegs &v) { stage_store<R>(sa + buf * kPfABytes, v.r); }, load_slot,
        [&](int buf, const Slot &sl) { compute(sa + buf * kPfABytes, sl); });
    // epilogue: lane holds rows 32i + acc_row(r, kh), column hc.  h in
    // registers; row maxima over the workgroup's 256 columns (32 lanes of a
    // half-wave, then the 8 waves through LDS) give each row's power of two.
    float hv[MB][16];
#pragma unroll
    for (int i = 0; i < MB; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const float xs = sxs[32 * i + acc_row(r, kh)];
            hv[i][r] = silu(acc[i][0][r] * xs) * (acc[i][1][r] * xs);
        }
    // per row, the max over the half-wave's 32 columns (complete in lanes 31
    // and 63), eight independent reductions at a time so that they interleave
#pragma unroll
    for (int i = 0; i < MB; i++)
#pragma unroll
        for (int r0 = 0; r0 < 16; r0 += 8) {
            float mx[8];
#pragma unroll
            for (int j = 0; j < 8; j++) mx[j] = half_wave_max_abs(hv[i][r0 + j]);
            if (col == 31) {
#pragma unroll
                for (int j = 0; j < 8; j++) smax[w * kPfRows + 32 * i + acc_row(r0 + j, kh)] = mx[j];
            }
        }
    __syncthreads();
    if (threadIdx.x < R) {
        float mx = 0.f;
#pragma unroll
        for (int v = 0; v < kPfWaves; v++) mx = fmaxf(mx, smax[v * kPfRows + threadIdx.x]);
        const int e = pf_exponent(mx);
        sexp[threadIdx.x] = e;
        if ((int)threadIdx.x < t.rows)
            a.hexp[(int64_t)(t.off + t.r0 + threadIdx.x) * (a.I / kPfGuCols) + ntile] = e;
    }
    __syncthreads();
    // (a block whose 32 rows are all in the tile stores without per-row tests)
    uint16_t *hrow = a.h + (int64_t)(t.off + t.r0) * a.I + hc;
    auto store = [&](int i, int r) {
        const int m = 32 * i + acc_row(r, kh);
        hrow[(int64_t)m * a.I] = (uint16_t)f16_bits(ldexpf(hv[i][r], -sexp[m]));
    };
#pragma unroll
    for (int i = 0; i < MB; i++) {
        if (32 * (i + 1) <= t.rows) {
#pragma unroll
            for (int r = 0; r < 16; r++) store(i, r);
        } else {
#pragma unroll
            for (int r = 0; r < 16; r++)
                if (32 * i + acc_row(r, kh) < t.rows) store(i, r);
        }
    }
}

__global__ void __launch_bounds__(kPfThreads)
k_pf_gateup(GuArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // Mentioning an accumulation register makes the compiler pick the MFMA
    // form that keeps C/D in AGPRs (otherwise every MFMA reads and writes 16
    // arch VGPRs, competing with the dequantisation VALU work for them).
    asm volatile("" ::: "a0");
    const PfSlot sl = pf_slot(a.I / kPfGuCols);
    if (sl.tile >= *a.n_tiles) return;
    const PfTile t = pf_tile(sl.tile, a.tiles, a.counts, a.offsets);
    int *stok = reinterpret_cast<int *>(lds + kPfTabBytes + 2 * kPfABytes);
    float *sxs = reinterpret_cast<float *>(stok + kPfRows);
    if (threadIdx.x < kPfRows) {
        const int tok = a.perm[t.off + t.r0 + min((int)threadIdx.x, t.rows - 1)] / a.k;
        stok[threadIdx.x] = tok;
        sxs[threadIdx.x] = a.xsc[tok] * (1.f / kPfWScale);
    }
    pf_build_tables(a.grid, lds);
    __syncthreads();
    switch ((t.rows + 31) >> 5) {
        case 1: gu_tile<1>(a, lds, t, sl.ntile); break;
        case 2: gu_tile<2>(a, lds, t, sl.ntile); break;
        default: gu_tile<3>(a, lds, t, sl.ntile); break;
    }
}

// ---------------------------------------------------------------------------
// down.  1024 threads (16 waves); wave w owns output columns n0 + 32w ..
// +31, one 32-column block, so a wave holds at most 3 x 16 accumulators and
// four waves run on each SIMD: the Q2K decode (VALU) of some waves then runs
// under the MFMAs of others.  (Measured against two 8-wave workgroups of
// 256 columns per compute unit, which stage every activation tile twice:
// slower.)  In a stage (half superblock, 8 sub-blocks) lane
// half kh takes sub-blocks 4kh..4kh+3 - one 16-byte piece - k-step t being
// half t & 1 of sub-block 4kh + (t >> 1): stage K offset 64 kh + 8 t again.
// Outputs: fp16 per pair with one power-of-two exponent per (pair, 512
// columns) (prefill), or fp32 per pair (decode batches).
// ---------------------------------------------------------------------------
constexpr int kDnWaves = 16;
constexpr int kDnThreads = kDnWaves * kWave;
static_assert(kPfDnCols == kDnWaves * 32, "one 32-column block per down wave");
// LDS: two A stages | semax [rows] | output exponents [rows] | pair of each
// row [rows] | row maxima [waves][rows]
constexpr int kPfDnLdsAll = 2 * kPfABytes + kPfRows * (4 + 4 + 4) + kDnWaves * kPfRows * 4;

struct DnArgs {
    int H, I;
    const uint8_t *down;
    const uint16_t *h;
    const int32_t *hexp;
    const int32_t *counts, *offsets, *perm, *tiles, *n_tiles;
    float *o;           // fp32 outputs [pairs][H] (decode batches), or
    uint16_t *o16;      // fp16 outputs [pairs][H] and their
    int32_t *oexp;      // exponents [pairs][H / kPfDnCols, rounded up]
};

// Stage pieces of a down workgroup: R rows x 16 chunks, thread
// threadIdx.x + kDnThreads p taking piece p; the row test is wave-uniform.
template <int R>
constexpr int dn_pieces() { return (16 * R + kDnThreads - 1) / kDnThreads; }
BM_DEV StageIdx dn_stage_idx(int p) {
    const int u = threadIdx.x + kDnThreads * p, q = u >> 6, l = u & 63;
    return {8 * (q >> 1) + (l & 7), 8 * (q & 1) + (l >> 3)};
}

// Raw loads only (h piece and its chunk exponent): a rescale here would make
// the wave wait for these loads before the current stage's MFMAs.  Pieces
// past the tile's R rows re-read a valid row and are never stored.
template <int R>
BM_DEV void dn_stage_load(const DnArgs &a, const PfTile &t, int kb, int hf, u32x4 (&r)[dn_pieces<R>()],
                          int (&ex)[dn_pieces<R>()]) {
    const int k0 = kb * kQK + hf * kPfHalf, nI = a.I / kPfGuCols;
#pragma unroll
    for (int p = 0; p < dn_pieces<R>(); p++) {
        const StageIdx x = dn_stage_idx(p);
        const int64_t gr = t.off + t.r0 + min(min(x.row, R - 1), t.rows - 1);
        r[p] = *reinterpret_cast<const u32x4 *>(a.h + gr * a.I + k0 + 8 * x.c);
        ex[p] = a.hexp[gr * nI + kb];
    }
}

// Rescale the loaded pieces to the row's largest exponent (exact: powers of
// two) and store them into the stage buffer.
template <int R>
BM_DEV void dn_stage_put(uint8_t *dst, const int *semax, const int (&ex)[dn_pieces<R>()],
                         u32x4 (&r)[dn_pieces<R>()]) {
#pragma unroll
    for (int p = 0; p < dn_pieces<R>(); p++) {
        const StageIdx x = dn_stage_idx(p);
        if (x.row < R) {
            const int d = ex[p] - semax[x.row];
            if (d != 0) {
                const uint32_t f = f16_pow2(d) * 0x10001u;
                r[p] = u32x4{pk_mul(r[p].x, f), pk_mul(r[p].y, f), pk_mul(r[p].z, f), pk_mul(r[p].w, f)};
            }
            *reinterpret_cast<u32x4 *>(dst + (x.c * R + x.row) * 16) = r[p];
        }
    }
}

// Down epilogue: lane holds rows 32i + acc_row(r, kh) of output column c0,
// each row's value being acc * 2^(semax[m] - wshift).  fp32 outputs per pair
// (OUT32), or fp16 with one power-of-two exponent per (pair, 512 columns):
// each row's largest |value| over the workgroup's 512 columns (32 lanes of
// a half-wave by DPP, then the 16 waves through LDS) sets its power of two.
template <int MB, int OUT32>
BM_DEV void dn_epilogue(const DnArgs &a, uint8_t *lds, const PfTile &t, int ntile, const f32x16 (&acc)[MB],
                        int c0, bool active, int wshift) {
    const int *semax = reinterpret_cast<const int *>(lds + 2 * kPfABytes);
    int *soex = const_cast<int *>(semax) + kPfRows;
    const int *spair = soex + kPfRows;
    float *smax = reinterpret_cast<float *>(soex + 2 * kPfRows);
    const int lane = lane_id(), col = lane & 31, kh = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (OUT32) {
        if (!active) return;
#pragma unroll
        for (int i = 0; i < MB; i++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = 32 * i + acc_row(r, kh);
                if (m < t.rows) a.o[(int64_t)spair[m] * a.H + c0] = ldexpf(acc[i][r], semax[m] - wshift);
            }
        return;
    }
#pragma unroll
    for (int i = 0; i < MB; i++)
#pragma unroll
        for (int r0 = 0; r0 < 16; r0 += 8) {
            float mx[8];
#pragma unroll
            for (int j = 0; j < 8; j++) mx[j] = half_wave_max_abs(active ? acc[i][r0 + j] : 0.f);
            if (col == 31) {
#pragma unroll
                for (int j = 0; j < 8; j++) smax[w * kPfRows + 32 * i + acc_row(r0 + j, kh)] = mx[j];
            }
        }
    __syncthreads();
    if (threadIdx.x < 32 * MB) {
        float mx = 0.f;
#pragma unroll
        for (int v = 0; v < kDnWaves; v++) mx = fmaxf(mx, smax[v * kPfRows + threadIdx.x]);
        const int e = pf_exponent(mx);
        soex[threadIdx.x] = e;
        if ((int)threadIdx.x < t.rows)
            a.oexp[(int64_t)spair[threadIdx.x] * ((a.H + kPfDnCols - 1) / kPfDnCols) + ntile] =
                e + semax[threadIdx.x] - wshift;
    }
    __syncthreads();
    if (!active) return;
    // (a block whose 32 rows are all in the tile stores without per-row tests)
    auto store = [&](int i, int r) {
        const int m = 32 * i + acc_row(r, kh);
        a.o16[(int64_t)spair[m] * a.H + c0] = (uint16_t)f16_bits(ldexpf(acc[i][r], -soex[m]));
    };
#pragma unroll
    for (int i = 0; i < MB; i++) {
        if (32 * (i + 1) <= t.rows) {
#pragma unroll
            for (int r = 0; r < 16; r++) store(i, r);
        } else {
#pragma unroll
            for (int r = 0; r < 16; r++)
                if (32 * i + acc_row(r, kh) < t.rows) store(i, r);
        }
    }
}

template <int MB, int OUT32>
BM_DEV void dn_tile(const DnArgs &a, uint8_t *lds, const PfTile &t, int ntile) {
    constexpr int R = 32 * MB, DP = dn_pieces<R>();
    uint8_t *const sa = lds;                             // A buffer b at sa + b * kPfABytes
    int *semax = reinterpret_cast<int *>(lds + 2 * kPfABytes);
    const int lane = lane_id(), col = lane & 31, kh = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nb = a.I / kQK;
    const int64_t S = (int64_t)a.H * nb;
    const uint8_t *D = a.down + (int64_t)t.e * S * 84;
    const int c0 = ntile * kPfDnCols + 32 * w + col;
    const bool active = ntile * kPfDnCols + 32 * w < a.H;     // wave-uniform (H is a multiple of 256)
    const int cc = min(c0, a.H - 1), P = cc >> 6, pr = cc & 63;
    const uint32_t pk64 = (uint32_t)(P * nb * 64 + pr);          // (P nb + kb) 64 + r at kb = 0
    const uint32_t qoff = (uint32_t)((P * nb * 4 + kh) * 64 + pr) * 16;
    const uint32_t soff = (uint32_t)(S * 64) + pk64 * 16 + 4 * kh;
    const uint32_t doff = (uint32_t)(S * 80) + pk64 * 4;
    struct Slot { uint4 w; uint32_t sc, dd; };           // words, 4 scale bytes, d|dmin
    auto load_slot = [&](int st, Slot &sl) {
        const int kb = st >> 1, hf = st & 1;
        sl.w = *reinterpret_cast<const uint4 *>(D + qoff + kb * 4096 + hf * 2048);
        sl.sc = *reinterpret_cast<const uint32_t *>(D + soff + kb * 1024 + 8 * hf);
        sl.dd = *reinterpret_cast<const uint32_t *>(D + doff + kb * 256);
    };
    f32x16 acc[MB];
#pragma unroll
    for (int i = 0; i < MB; i++) acc[i] = (f32x16)0.f;
    auto compute = [&](const uint8_t *A, const Slot &sl) {
        // (a, -b) of each sub-block from one packed fma: (16 + sc, 16 + m) times
        // (d', -dmin') minus 16 (d', -dmin'), d' = 2^7 d and dmin' = 2^7 dmin
        // (exact scalings), i.e. one fp16 rounding each of d' sc and -dmin' m
        const f16x2 dm = u2h(sl.dd) * f16x2{kPfDnWScale, -kPfDnWScale};
        const f16x2 c16 = dm * f16x2{-16.f, -16.f};
        const uint32_t slo = sl.sc & 0x0F0F0F0Fu, shi = (sl.sc >> 4) & 0x0F0F0F0Fu;
        const uint32_t wsel[4] = {sl.w.x, sl.w.y, sl.w.z, sl.w.w};
#pragma unroll
        for (int sbk = 0; sbk < 4; sbk++) {                 // sub-block 4kh + sbk: k-steps 2 sbk, 2 sbk + 1
            // sc and m of byte sbk into the two halves, as the fp16 mantissas of 16 + sc, 16 + m
            const uint32_t scm = __builtin_amdgcn_perm(shi, slo, 0x0C040C00u + 0x00010001u * sbk);
            const f16x2 ab = __builtin_elementwise_fma(u2h((scm << 6) | 0x4C004C00u), dm, c16);
            const f16x2 av = ab.xx, bv = ab.yy;
            const uint32_t qlo = q2k_lo(wsel[sbk]), qhi = q2k_hi(wsel[sbk]);
#pragma unroll
            for (int half = 0; half < 2; half++) {
                f16x8 af[MB];
#pragma unroll
                for (int i = 0; i < MB; i++) af[i] = frag32<R>(A, i, lane, 2 * sbk + half);
                const uint32_t src = half ? qhi : qlo;
                const uint32_t qb[4] = {q2k_pair_f16<0>(src), q2k_pair_f16<1>(src), q2k_pair_f16<2>(src),
                                        q2k_pair_f16<3>(src)};                  // exact quant pairs
                uint4 v;
                uint32_t *vv = reinterpret_cast<uint32_t *>(&v);
#pragma unroll
                for (int q = 0; q < 4; q++) vv[q] = h2u(__builtin_elementwise_fma(u2h(qb[q]), av, bv));   // a q - b
                const f16x8 b = __builtin_bit_cast(f16x8, v);
#pragma unroll
                for (int i = 0; i < MB; i++) acc[i] = mfma32(af[i], b, acc[i]);
            }
        }
    };
    struct ARegs { u32x4 r[DP]; int e[DP]; };
    // each row's largest h exponent (the staged pieces are rescaled to it):
    // every (row, 256-column chunk) exponent loaded at once, maxima by LDS
    // atomics, while the first stages' loads are in flight
    auto row_max_exponents = [&]() {
        const int nI = a.I / kPfGuCols;
        if (threadIdx.x < kPfRows) semax[threadIdx.x] = -(1 << 30);
        __syncthreads();
        for (int u = threadIdx.x; u < kPfRows * nI; u += kDnThreads) {
            const int m = u / nI, c = u - m * nI;
            const int64_t gr = t.off + t.r0 + min(m, t.rows - 1);
            atomicMax(&semax[m], a.hexp[gr * nI + c]);
        }
        __syncthreads();
    };
    run_stages<1, ARegs, Slot>(
        2 * nb, [&](int st, ARegs &v) { dn_stage_load<R>(a, t, st >> 1, st & 1, v.r, v.e); },
        [&](int buf, ARegs &v) { dn_stage_put<R>(sa + buf * kPfABytes, semax, v.e, v.r); }, load_slot,
        [&](int buf, const Slot &sl) {
            if (active) compute(sa + buf * kPfABytes, sl);
        },
        row_max_exponents);
    dn_epilogue<MB, OUT32>(a, lds, t, ntile, acc, c0, active, kPfDnWShift);
}

template <int OUT32>
__global__ void __launch_bounds__(kDnThreads)
k_pf_down(DnArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // (no AGPR hint: at most 48 accumulators, which fit beside the decode
    // state in the 128 registers a wave may hold at four waves per SIMD)
    const PfSlot sl = pf_slot((a.H + kPfDnCols - 1) / kPfDnCols);
    if (sl.tile >= *a.n_tiles) return;
    const PfTile t = pf_tile(sl.tile, a.tiles, a.counts, a.offsets);
    // the pair of each row (the epilogue's output rows); the rows' largest h
    // exponents are gathered inside the stage pipeline's prologue
    int *semax = reinterpret_cast<int *>(lds + 2 * kPfABytes);
    if (threadIdx.x < kPfRows)
        semax[2 * kPfRows + threadIdx.x] = a.perm[t.off + t.r0 + min((int)threadIdx.x, t.rows - 1)];
    switch ((t.rows + 31) >> 5) {
        case 1: dn_tile<1, OUT32>(a, lds, t, sl.ntile); break;
        case 2: dn_tile<2, OUT32>(a, lds, t, sl.ntile); break;
        default: dn_tile<3, OUT32>(a, lds, t, sl.ntile); break;
    }
}

// ---------------------------------------------------------------------------
// MXFP4 routed experts.  The operands are bf16: the activations as they
// are (fp32 activations rounded to bf16 first, k_mx_xprep), h rounded to
// bf16, and the weights straight from the hardware conversion, one
// instruction per weight pair with the block scale applied (element *
// 2^(X-127) is exact in bf16 for every X up to 252), so there are no
// tables and no exponent bookkeeping: the k-step's VALU work is eight
// conversions (gate/up) or four (down) against 2 MB or MB MFMAs.
// Tiled MXFP4 slab of an [N][K] matrix: piece c (32 weights) of 256-weight
// chunk kb of row P*64 + r at ((P nb + kb) 8 + c) 64 + r, 16 bytes, byte i
// holding weights 2i (low nibble) and 2i+1; the row's 8 scale bytes of the
// chunk at N K/2 + ((P nb + kb) 64 + r) 8.  In a stage (half chunk: pieces
// 4 hf .. 4 hf + 3) lane half kh takes pieces 4 hf + 2 kh and + 1, k-step t
// reading dword t & 3 of piece 4 hf + 2 kh + (t >> 2): stage K offset
// 64 kh + 8 t, as for the 2-bit formats.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr int kMxGuLds = 2 * kPfABytes + kPfRows * 4;

BM_DEV f32x16 mfma32b(bf16x8 a, bf16x8 b, f32x16 c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }
template <int R>
BM_DEV bf16x8 frag32b(const uint8_t *buf, int i, int lane, int t) {
    return *reinterpret_cast<const bf16x8 *>(buf + ((8 * (lane >> 5) + t) * R + 32 * i + (lane & 31)) * 16);
}
// bf16 operand of 8 weights (one dword) at scale 2^(X-127)
BM_DEV bf16x8 mx_operand(uint32_t W, uint32_t X) {
    const float sc = mx_cvt_scale(X);
    const uint4 v = make_uint4(fp4x2_bf16s<0>(W, sc), fp4x2_bf16s<1>(W, sc), fp4x2_bf16s<2>(W, sc),
                               fp4x2_bf16s<3>(W, sc));
    return __builtin_bit_cast(bf16x8, v);
}
BM_DEV uint32_t u4_word(const uint4 &v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

// fp32 activations -> bf16 (nearest-even), 8 per thread
__global__ void __launch_bounds__(256)
k_mx_xprep(int64_t n8, const float *__restrict__ x, uint16_t *__restrict__ xb) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const float4 *p = reinterpret_cast<const float4 *>(x) + 2 * i;
    const float4 u = p[0], v = p[1];
    reinterpret_cast<uint4 *>(xb)[i] =
        make_uint4(f32_to_bf16_rne(u.x) | (f32_to_bf16_rne(u.y) << 16), f32_to_bf16_rne(u.z) | (f32_to_bf16_rne(u.w) << 16),
                   f32_to_bf16_rne(v.x) | (f32_to_bf16_rne(v.y) << 16), f32_to_bf16_rne(v.z) | (f32_to_bf16_rne(v.w) << 16));
}

// gate/up: 8 waves x 32 h columns as in gu_tile; a.x16 holds the bf16
// activation rows.  Epilogue: h = silu(g) u rounded to bf16.
template <int MB>
BM_DEV void mx_gu_tile(const GuArgs &a, uint8_t *lds, const PfTile &t, int ntile) {
    constexpr int R = 32 * MB;
    uint8_t *const sa = lds;                            // A buffer b at sa + b * kPfABytes
    const int *stok = reinterpret_cast<const int *>(lds + 2 * kPfABytes);
    const int lane = lane_id(), col = lane & 31, kh = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nb = a.H / kQK;
    const int64_t slab = (int64_t)a.I * a.H / 32 * 17;
    const uint8_t *G = a.gate + t.e * slab, *U = a.up + t.e * slab;
    const int hc = ntile * kPfGuCols + 32 * w + col, P = hc >> 6, pr = hc & 63;
    // byte offsets at chunk 0, half 0 (one expert's slab is below 4 GiB)
    const uint32_t qoff = (uint32_t)((P * nb * 8 + 2 * kh) * 64 + pr) * 16;
    const uint32_t soff = (uint32_t)(a.I * a.H / 2) + (uint32_t)(P * nb * 64 + pr) * 8 + 2 * kh;
    struct Slot { uint4 g0, g1, u0, u1; uint32_t sg, su; };
    auto load_slot = [&](int st, Slot &sl) {
        const int kb = st >> 1, hf = st & 1;
        const uint32_t o = qoff + kb * 8192 + hf * 4096, os = soff + kb * 512 + 4 * hf;
        sl.g0 = *reinterpret_cast<const uint4 *>(G + o);
        sl.g1 = *reinterpret_cast<const uint4 *>(G + o + 1024);
        sl.u0 = *reinterpret_cast<const uint4 *>(U + o);
        sl.u1 = *reinterpret_cast<const uint4 *>(U + o + 1024);
        sl.sg = *reinterpret_cast<const uint16_t *>(G + os);
        sl.su = *reinterpret_cast<const uint16_t *>(U + os);
    };
    f32x16 acc[MB][2];
#pragma unroll
    for (int i = 0; i < MB; i++) acc[i][0] = acc[i][1] = (f32x16)0.f;
    auto compute = [&](const uint8_t *A, const Slot &sl) {
#pragma unroll
        for (int s = 0; s < 8; s++) {
            bf16x8 av[MB];
#pragma unroll
            for (int i = 0; i < MB; i++) av[i] = frag32b<R>(A, i, lane, s);
            const bf16x8 bg = mx_operand(u4_word(s < 4 ? sl.g0 : sl.g1, s & 3), s < 4 ? sl.sg & 0xFFu : sl.sg >> 8);
            const bf16x8 bu = mx_operand(u4_word(s < 4 ? sl.u0 : sl.u1, s & 3), s < 4 ? sl.su & 0xFFu : sl.su >> 8);
#pragma unroll
            for (int i = 0; i < MB; i++) {
                acc[i][0] = mfma32b(av[i], bg, acc[i][0]);
                acc[i][1] = mfma32b(av[i], bu, acc[i][1]);
            }
        }
    };
    struct ARegs { u32x4 r[R / 32]; };
    run_stages<2, ARegs, Slot>(
        2 * nb, [&](int st, ARegs &v) { gu_stage_load<R>(a, stok, st >> 1, st & 1, v.r); },
        [&](int buf, ARegs &v) { stage_store<R>(sa + buf * kPfABytes, v.r); }, load_slot,
        [&](int buf, const Slot &sl) { compute(sa + buf * kPfABytes, sl); });
    // (a block whose 32 rows are all in the tile stores without per-row tests)
    uint16_t *hrow = a.h + (int64_t)(t.off + t.r0) * a.I + hc;
    auto store = [&](int i, int r) {
        const int m = 32 * i + acc_row(r, kh);
        hrow[(int64_t)m * a.I] = (uint16_t)f32_to_bf16_rne(silu(acc[i][0][r]) * acc[i][1][r]);
    };
#pragma unroll
    for (int i = 0; i < MB; i++) {
        if (32 * (i + 1) <= t.rows) {
#pragma unroll
            for (int r = 0; r < 16; r++) store(i, r);
        } else {
#pragma unroll
            for (int r = 0; r < 16; r++)
                if (32 * i + acc_row(r, kh) < t.rows) store(i, r);
        }
    }
}

__global__ void __launch_bounds__(kPfThreads)
k_mx_gateup(GuArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    asm volatile("" ::: "a0");           // accumulators in AGPRs (see k_pf_gateup)
    const PfSlot sl = pf_slot(a.I / kPfGuCols);
    if (sl.tile >= *a.n_tiles) return;
    const PfTile t = pf_tile(sl.tile, a.tiles, a.counts, a.offsets);
    int *stok = reinterpret_cast<int *>(lds + 2 * kPfABytes);
    if (threadIdx.x < kPfRows) stok[threadIdx.x] = a.perm[t.off + t.r0 + min((int)threadIdx.x, t.rows - 1)] / a.k;
    __syncthreads();
    switch ((t.rows + 31) >> 5) {
        case 1: mx_gu_tile<1>(a, lds, t, sl.ntile); break;
        case 2: mx_gu_tile<2>(a, lds, t, sl.ntile); break;
        default: mx_gu_tile<3>(a, lds, t, sl.ntile); break;
    }
}

// down: 16 waves x 32 output columns as in dn_tile; A = the bf16 h rows
// copied into the stage as they are.
template <int R>
BM_DEV void mx_dn_stage_load(const DnArgs &a, const PfTile &t, int kb, int hf, u32x4 (&r)[dn_pieces<R>()]) {
    const int k0 = kb * kQK + hf * kPfHalf;
#pragma unroll
    for (int p = 0; p < dn_pieces<R>(); p++) {
        const StageIdx x = dn_stage_idx(p);
        const int64_t gr = t.off + t.r0 + min(min(x.row, R - 1), t.rows - 1);
        r[p] = *reinterpret_cast<const u32x4 *>(a.h + gr * a.I + k0 + 8 * x.c);
    }
}
template <int R>
BM_DEV void mx_dn_stage_put(uint8_t *dst, const u32x4 (&r)[dn_pieces<R>()]) {
#pragma unroll
    for (int p = 0; p < dn_pieces<R>(); p++) {
        const StageIdx x = dn_stage_idx(p);
        if (x.row < R) *reinterpret_cast<u32x4 *>(dst + (x.c * R + x.row) * 16) = r[p];
    }
}

template <int MB, int OUT32>
BM_DEV void mx_dn_tile(const DnArgs &a, uint8_t *lds, const PfTile &t, int ntile) {
    constexpr int R = 32 * MB, DP = dn_pieces<R>();
    uint8_t *const sa = lds;
    const int lane = lane_id(), col = lane & 31, kh = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nb = a.I / kQK;
    const int64_t slab = (int64_t)a.H * a.I / 32 * 17;
    const uint8_t *D = a.down + (int64_t)t.e * slab;
    const int c0 = ntile * kPfDnCols + 32 * w + col;
    const bool active = ntile * kPfDnCols + 32 * w < a.H;     // wave-uniform
    const int cc = min(c0, a.H - 1), P = cc >> 6, pr = cc & 63;
    const uint32_t qoff = (uint32_t)((P * nb * 8 + 2 * kh) * 64 + pr) * 16;
    const uint32_t soff = (uint32_t)(a.H * a.I / 2) + (uint32_t)(P * nb * 64 + pr) * 8 + 2 * kh;
    struct Slot { uint4 w0, w1; uint32_t sc; };
    auto load_slot = [&](int st, Slot &sl) {
        const int kb = st >> 1, hf = st & 1;
        const uint32_t o = qoff + kb * 8192 + hf * 4096;
        sl.w0 = *reinterpret_cast<const uint4 *>(D + o);
        sl.w1 = *reinterpret_cast<const uint4 *>(D + o + 1024);
        sl.sc = *reinterpret_cast<const uint16_t *>(D + soff + kb * 512 + 4 * hf);
    };
    f32x16 acc[MB];
#pragma unroll
    for (int i = 0; i < MB; i++) acc[i] = (f32x16)0.f;
    auto compute = [&](const uint8_t *A, const Slot &sl) {
#pragma unroll
        for (int s = 0; s < 8; s++) {
            bf16x8 af[MB];
#pragma unroll
            for (int i = 0; i < MB; i++) af[i] = frag32b<R>(A, i, lane, s);
            const bf16x8 b = mx_operand(u4_word(s < 4 ? sl.w0 : sl.w1, s & 3), s < 4 ? sl.sc & 0xFFu : sl.sc >> 8);
#pragma unroll
            for (int i = 0; i < MB; i++) acc[i] = mfma32b(af[i], b, acc[i]);
        }
    };
    struct ARegs { u32x4 r[DP]; };
    run_stages<1, ARegs, Slot>(
        2 * nb, [&](int st, ARegs &v) { mx_dn_stage_load<R>(a, t, st >> 1, st & 1, v.r); },
        [&](int buf, ARegs &v) { mx_dn_stage_put<R>(sa + buf * kPfABytes, v.r); }, load_slot,
        [&](int buf, const Slot &sl) {
            if (active) compute(sa + buf * kPfABytes, sl);
        });
    dn_epilogue<MB, OUT32>(a, lds, t, ntile, acc, c0, active, 0);
}

template <int OUT32>
__global__ void __launch_bounds__(kDnThreads)
k_mx_down(DnArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const PfSlot sl = pf_slot((a.H + kPfDnCols - 1) / kPfDnCols);
    if (sl.tile >= *a.n_tiles) return;
    const PfTile t = pf_tile(sl.tile, a.tiles, a.counts, a.offsets);
    // the epilogue's row exponents (0: h is not rescaled) and pairs
    int *semax = reinterpret_cast<int *>(lds + 2 * kPfABytes);
    if (threadIdx.x < kPfRows) {
        semax[threadIdx.x] = 0;
        semax[2 * kPfRows + threadIdx.x] = a.perm[t.off + t.r0 + min((int)threadIdx.x, t.rows - 1)];
    }
    __syncthreads();
    switch ((t.rows + 31) >> 5) {
        case 1: mx_dn_tile<1, OUT32>(a, lds, t, sl.ntile); break;
        case 2: mx_dn_tile<2, OUT32>(a, lds, t, sl.ntile); break;
        default: mx_dn_tile<3, OUT32>(a, lds, t, sl.ntile); break;
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

// y[t][n] = sum_j w[t][j] o[t k + j][n] (+ os[t][n]) with o in fp16 and one
// power-of-two exponent per (pair, 512 columns): eight consecutive outputs
// per thread, the k rows' 16-byte loads issued together (k <= KMAX), slots
// summed in order.
template <int KMAX>
__global__ void __launch_bounds__(256)
k_combine_p(const uint16_t *__restrict__ o16, const int32_t *__restrict__ oexp, const float *__restrict__ w,
            const float *__restrict__ os, float *__restrict__ y, int T, int H, int k) {
    const int H8 = H / 8, nN = (H + kPfDnCols - 1) / kPfDnCols;
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (int64_t)T * H8) return;
    const int t = (int)(q / H8), n8 = (int)(q - (int64_t)t * H8), tile = 8 * n8 / kPfDnCols;
    const uint4 *o4 = reinterpret_cast<const uint4 *>(o16) + (int64_t)t * k * H8 + n8;
    uint4 v[KMAX];
    int e[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; j++) {
        const int jj = min(j, k - 1);
        v[j] = o4[(int64_t)jj * H8];
        e[j] = oexp[((int64_t)t * k + jj) * nN + tile];
    }
    float s[8];
#pragma unroll
    for (int i = 0; i < 8; i++) s[i] = 0.f;
#pragma unroll
    for (int j = 0; j < KMAX; j++)
        if (j < k) {
            const float wj = ldexpf(w[t * k + j], e[j]);
            const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                s[2 * i] = fmaf(wj, fp16_to_f32(u[i] & 0xFFFFu), s[2 * i]);
                s[2 * i + 1] = fmaf(wj, fp16_to_f32(u[i] >> 16), s[2 * i + 1]);
            }
        }
    if (os) {
        const float4 *a4 = reinterpret_cast<const float4 *>(os + (int64_t)t * H + 8 * n8);
        const float4 a = a4[0], b = a4[1];
        s[0] += a.x; s[1] += a.y; s[2] += a.z; s[3] += a.w;
        s[4] += b.x; s[5] += b.y; s[6] += b.z; s[7] += b.w;
    }
    float4 *y4 = reinterpret_cast<float4 *>(y + (int64_t)t * H + 8 * n8);
    y4[0] = make_float4(s[0], s[1], s[2], s[3]);
    y4[1] = make_float4(s[4], s[5], s[6], s[7]);
}

}  // namespace

namespace bm_host {

// MXFP4 routed experts: activation rounding (fp32 input only), gate/up, down
static int launch_prefill_routed_mx(const bitmoe_layer *L, const void *x, int x_dtype, int T, const Buckets &b,
                                    int max_tiles, const PrefillBufs &pb, hipStream_t s, int parts) {
    const int H = L->H, I = L->I, k = L->k;
    static const bool attr =
        hipFuncSetAttribute(reinterpret_cast<const void *>(k_mx_down<0>), hipFuncAttributeMaxDynamicSharedMemorySize,
                            kPfDnLdsAll) == hipSuccess &&
        hipFuncSetAttribute(reinterpret_cast<const void *>(k_mx_down<1>), hipFuncAttributeMaxDynamicSharedMemorySize,
                            kPfDnLdsAll) == hipSuccess;
    if (!attr) return BITMOE_EHIP;
    const uint16_t *xb = x_dtype == BITMOE_BF16 ? static_cast<const uint16_t *>(x) : pb.x16;
    if (x_dtype != BITMOE_BF16 && (parts & kPfPrep)) {
        const int64_t n8 = (int64_t)T * H / 8;
        k_mx_xprep<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(n8, static_cast<const float *>(x), pb.x16);
        BM_LAUNCH_CHECK();
    }
    if (!(parts & kPfRouted)) return BITMOE_OK;
    {
        GuArgs a{H, I, k, (const uint8_t *)L->gate_q, (const uint8_t *)L->up_q, nullptr, xb, nullptr,
                 b.counts, b.offsets, b.perm, b.tiles, b.n_tiles, pb.h, nullptr};
        const TimingEvents ev = timing_for(BITMOE_TIME_GATEUP);
        hipExtLaunchKernelGGL(k_mx_gateup, dim3(pf_grid(max_tiles, I / kPfGuCols)), dim3(kPfThreads), kMxGuLds, s,
                              ev.start, ev.stop, 0, a);
        BM_LAUNCH_CHECK();
    }
    {
        DnArgs a{H, I, (const uint8_t *)L->down_q, pb.h, nullptr, b.counts, b.offsets, b.perm, b.tiles,
                 b.n_tiles, pb.o, pb.o16, pb.oexp};
        const TimingEvents ev = timing_for(BITMOE_TIME_DOWN);
        hipExtLaunchKernelGGL(pb.o16 ? k_mx_down<0> : k_mx_down<1>,
                              dim3(pf_grid(max_tiles, (H + kPfDnCols - 1) / kPfDnCols)), dim3(kDnThreads),
                              kPfDnLdsAll, s, ev.start, ev.stop, 0, a);
        BM_LAUNCH_CHECK();
    }
    return BITMOE_OK;
}

int launch_prefill_routed(const bitmoe_layer *L, const void *x, int x_dtype, int T, const Buckets &b,
                          int max_tiles, const PrefillBufs &pb, hipStream_t s, int parts) {
    if (L->format == BITMOE_FORMAT_MXFP4)
        return launch_prefill_routed_mx(L, x, x_dtype, T, b, max_tiles, pb, s, parts);
    const int H = L->H, I = L->I, k = L->k;
    static const bool attr = [] {
        hipFuncAttributes fa;           // the gate/up tables must start at LDS address 0
        return hipFuncGetAttributes(&fa, reinterpret_cast<const void *>(k_pf_gateup)) == hipSuccess &&
               fa.sharedSizeBytes == 0 &&
               hipFuncSetAttribute(reinterpret_cast<const void *>(k_pf_gateup),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, kPfGuLds) == hipSuccess &&
               hipFuncSetAttribute(reinterpret_cast<const void *>(k_pf_down<0>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, kPfDnLdsAll) == hipSuccess &&
               hipFuncSetAttribute(reinterpret_cast<const void *>(k_pf_down<1>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, kPfDnLdsAll) == hipSuccess;
    }();
    if (!attr) return BITMOE_EHIP;
    if (parts & kPfPrep) {
        if (x_dtype == BITMOE_BF16) k_pf_xprep<1><<<T, 256, 0, s>>>(H, x, pb.x16, pb.xsc);
        else k_pf_xprep<0><<<T, 256, 0, s>>>(H, x, pb.x16, pb.xsc);
        BM_LAUNCH_CHECK();
    }
    if (!(parts & kPfRouted)) return BITMOE_OK;
    {
        GuArgs a{H, I, k, (const uint8_t *)L->gate_q, (const uint8_t *)L->up_q, (const uint8_t *)L->grid,
                 pb.x16, pb.xsc, b.counts, b.offsets, b.perm, b.tiles, b.n_tiles, pb.h, pb.hexp};
        // the timing events, when set, are taken by the dispatch itself
        const TimingEvents ev = timing_for(BITMOE_TIME_GATEUP);
        hipExtLaunchKernelGGL(k_pf_gateup, dim3(pf_grid(max_tiles, I / kPfGuCols)), dim3(kPfThreads), kPfGuLds, s,
                              ev.start, ev.stop, 0, a);
        BM_LAUNCH_CHECK();
    }
    {
        // fp16 outputs with exponents when the buffers are given (prefill),
        // fp32 otherwise (decode batches)
        DnArgs a{H, I, (const uint8_t *)L->down_q, pb.h, pb.hexp, b.counts, b.offsets, b.perm, b.tiles,
                 b.n_tiles, pb.o, pb.o16, pb.oexp};
        const TimingEvents ev = timing_for(BITMOE_TIME_DOWN);
        hipExtLaunchKernelGGL(pb.o16 ? k_pf_down<0> : k_pf_down<1>,
                              dim3(pf_grid(max_tiles, (H + kPfDnCols - 1) / kPfDnCols)), dim3(kDnThreads),
                              kPfDnLdsAll, s, ev.start, ev.stop, 0, a);
        BM_LAUNCH_CHECK();
    }
    return BITMOE_OK;
}

int launch_prefill_ffn(const bitmoe_layer *L, const void *x, int x_dtype, int T, const float *w, float *y,
                       const Buckets &b, int max_tiles, const PrefillBufs &pb, hipStream_t s) {
    const int H = L->H, I = L->I, k = L->k;
    const int rc = launch_prefill_routed(L, x, x_dtype, T, b, max_tiles, pb, s);
    if (rc) return rc;
    const bool shared = L->shared_gate != nullptr;
    if (shared) {
        dim3 gs1(I / 64, T), gs2(H / 64, T);
        if (x_dtype == BITMOE_BF16)
            k_shared_gateup_rows<1><<<gs1, 64, 0, s>>>(H, I, (const uint4 *)L->shared_gate,
                                                       (const uint4 *)L->shared_up, x, pb.hs);
        else
            k_shared_gateup_rows<0><<<gs1, 64, 0, s>>>(H, I, (const uint4 *)L->shared_gate,
                                                       (const uint4 *)L->shared_up, x, pb.hs);
        BM_LAUNCH_CHECK();
        k_shared_down_rows<<<gs2, 64, 0, s>>>(H, I, (const uint4 *)L->shared_down, pb.hs, pb.os);
        BM_LAUNCH_CHECK();
    }
    if (reinterpret_cast<uintptr_t>(y) % 16) return BITMOE_EINVAL;
    const int64_t n8 = (int64_t)T * H / 8;
    auto kc = k <= 8 ? k_combine_p<8> : k_combine_p<16>;
    kc<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(pb.o16, pb.oexp, w, shared ? pb.os : nullptr, y, T, H, k);
    BM_LAUNCH_CHECK();
    return BITMOE_OK;
}

}  // namespace bm_host
