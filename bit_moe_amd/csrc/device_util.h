// Device-side building blocks shared by routing, bucketing and the fused
// decode pipeline: per-wave top-k with renormalised softmax, and the
// stable counting-sort pieces of the token -> expert bucketing.
#pragma once

#include "common.h"

namespace bm {

// Wave-wide max through DPP row shifts and row broadcasts (no LDS round
// trips); lanes without a source lane keep their own value.
template <int CTRL, int ROWS>
BM_DEV float dpp_max(float v) {
    const int o = __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROWS, 0xF, false);
    return fmaxf(v, __int_as_float(o));
}
// Routing ids given by the caller are trusted: values in [0, E).  A build
// with BITMOE_CHECK_IDS = 1 counts the others before the FFN (k_check_ids,
// into the first int32 of the call's workspace) and reads every id clamped
// into range, so that a bad id can only give a wrong result, never an access
// out of bounds.
#ifndef BITMOE_CHECK_IDS
#define BITMOE_CHECK_IDS 0
#endif
BM_DEV int user_id(int v, int E) { return BITMOE_CHECK_IDS ? min(max(v, 0), E - 1) : v; }

// Max of |v| over each half-wave (row shifts, then row 0 -> 1 and 2 -> 3),
// complete in lanes 31 and 63.  Non-negative floats order as their bit
// patterns (a NaN's above +inf), so the steps are integer maxima, each one
// instruction with its DPP move folded in (lanes without a source read 0,
// the maximum's identity; a float max adds canonicalising moves around
// every step).
BM_DEV float half_wave_max_abs(float v) {
    uint32_t u = __float_as_uint(fabsf(v));
#define BM_DPP_UMAX(CTRL, ROWS) u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, CTRL, ROWS, 0xF, false))
    BM_DPP_UMAX(0x111, 0xF);   // row_shr:1
    BM_DPP_UMAX(0x112, 0xF);   // row_shr:2
    BM_DPP_UMAX(0x114, 0xF);   // row_shr:4
    BM_DPP_UMAX(0x118, 0xF);   // row_shr:8: lane 15 of each row holds the row max
    BM_DPP_UMAX(0x142, 0xA);   // row_bcast:15 into rows 1, 3
#undef BM_DPP_UMAX
    return __uint_as_float(u);
}
BM_DEV float wave_max_f32(float v) {
    v = dpp_max<0x111, 0xF>(v);   // row_shr:1
    v = dpp_max<0x112, 0xF>(v);   // row_shr:2
    v = dpp_max<0x114, 0xF>(v);   // row_shr:4
    v = dpp_max<0x118, 0xF>(v);   // row_shr:8: lane 15 of each row holds the row max
    v = dpp_max<0x142, 0xA>(v);   // row_bcast:15 into rows 1, 3
    v = dpp_max<0x143, 0xC>(v);   // row_bcast:31 into rows 2, 3: lane 63 holds the max
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Top-k of one token's logits by one wavefront: k rounds of wave max, the
// lowest index holding it (ballots), then the softmax over the k selected.
// Lane 0 writes ids[0..k) and w[0..k) (either may be null) and, if given,
// the ids to sids[0..k) as well.  E <= 1024, k <= 16.  (NaN logits:
// the result is unspecified but every id is distinct and in range.)
BM_DEV void topk_wave(const float *__restrict__ lrow, int E, int k, int32_t *__restrict__ ids,
                      float *__restrict__ wout, int *sids = nullptr) {
    const int lane = lane_id();
    constexpr int MAXV = 16;
    const int nv = (E + 63) >> 6;
    float v[MAXV];
    uint32_t live = 0;        // bit i: element lane + 64 i exists and is not taken
#pragma unroll
    for (int i = 0; i < MAXV; i++) {
        const int e = lane + 64 * i;
        const int ec = e < E ? e : E - 1;        // every load issued, the extra ones masked
        v[i] = lrow[ec];
        if (e < E) live |= 1u << i;
    }
    float sel[16];
    int sid[16];
    for (int j = 0; j < k; j++) {
        float bv = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < MAXV; i++)
            if ((live >> i) & 1u) bv = fmaxf(bv, v[i]);
        const float m = wave_max_f32(bv);
        int be = -1;
        for (int i = 0; i < nv && be < 0; i++) {
            const uint64_t b = __ballot(((live >> i) & 1u) && v[i] == m);
            if (b) be = 64 * i + (int)__builtin_ctzll(b);
        }
        for (int i = 0; i < nv && be < 0; i++) {      // only reached with NaN logits
            const uint64_t b = __ballot((live >> i) & 1u);
            if (b) be = 64 * i + (int)__builtin_ctzll(b);
        }
        if ((be & 63) == lane) live &= ~(1u << (be >> 6));
        sel[j] = m;
        sid[j] = be;
    }
    if (lane == 0) {
        float z = 0.f, ex[16];
        for (int j = 0; j < k; j++) { ex[j] = __expf(sel[j] - sel[0]); z += ex[j]; }
        const float inv = 1.0f / z;
        for (int j = 0; j < k; j++) {
            if (ids) ids[j] = sid[j];
            if (wout) wout[j] = ex[j] * inv;
            if (sids) sids[j] = sid[j];
        }
    }
}

// Wave-wide minimum of an int (DPP as wave_max_f32).
template <int CTRL, int ROWS>
BM_DEV int dpp_min_i32(int v) {
    return min(v, __builtin_amdgcn_update_dpp(v, v, CTRL, ROWS, 0xF, false));
}
BM_DEV int wave_min_i32(int v) {
    v = dpp_min_i32<0x111, 0xF>(v);
    v = dpp_min_i32<0x112, 0xF>(v);
    v = dpp_min_i32<0x114, 0xF>(v);
    v = dpp_min_i32<0x118, 0xF>(v);
    v = dpp_min_i32<0x142, 0xA>(v);
    v = dpp_min_i32<0x143, 0xC>(v);
    return __builtin_amdgcn_readlane(v, 63);
}

// Key of (logit, expert) for the top-k below, a double in [1, 2) whose
// mantissa is the logit's order-preserving 32-bit pattern (-0 as +0, NaN as
// -inf, experts past E below everything) followed by 255 - expert: the
// largest key is the largest logit, the lowest expert among equal logits.
BM_DEV double topk_key(float v, int e, int E) {
    uint32_t u = 0u;
    if (e < E) {
        const uint32_t b = v == v ? __float_as_uint(v + 0.0f) : 0xFF800000u;
        u = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    }
    const uint64_t m = ((uint64_t)u << 20) | ((uint64_t)(255 - (e & 255)) << 12);
    return __longlong_as_double((long long)(0x3FF0000000000000ull | m));
}
BM_DEV void topk_key_decode(double key, float &v, int &e) {
    const uint64_t m = (uint64_t)__double_as_longlong(key);
    e = 255 - (int)((m >> 12) & 0xFFu);
    const uint32_t u = (uint32_t)(m >> 20);
    v = __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}
template <int CTRL, int ROWS>
BM_DEV double dpp_max_f64(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp((int)b, (int)b, CTRL, ROWS, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp((int)(b >> 32), (int)(b >> 32), CTRL, ROWS, 0xF, false);
    return fmax(v, __longlong_as_double((long long)(uint32_t)lo | ((long long)hi << 32)));
}
BM_DEV double wave_max_f64(double v) {
    v = dpp_max_f64<0x111, 0xF>(v);
    v = dpp_max_f64<0x112, 0xF>(v);
    v = dpp_max_f64<0x114, 0xF>(v);
    v = dpp_max_f64<0x118, 0xF>(v);
    v = dpp_max_f64<0x142, 0xA>(v);
    v = dpp_max_f64<0x143, 0xC>(v);
    const long long b = __double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)b, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(b >> 32), 63);
    return __longlong_as_double((long long)lo | ((long long)hi << 32));
}

// Top-k of one token's logits for E <= 256, by one wavefront, from values
// the caller loaded beforehand: lane l holds the logits of experts l, l+64,
// l+128, l+192 in v[] (anything beyond E is ignored).  Order: logit
// descending, expert index ascending; NaN counts as -inf.  Each (logit,
// expert) becomes one unique key (topk_key); each lane sorts its four keys,
// and every round takes the wave max of the lane heads, whose lane drops its
// head.  Lane j < k keeps the j-th pick, so the softmax over the k picks is
// one row sum.  Lanes j < k write ids[j], w[j] and sids[j] (any may be null)
// and return their pick.
BM_DEV int topk_wave4(float (&v)[4], int E, int k, int32_t *__restrict__ ids, float *__restrict__ wout,
                      int *sids) {
    const int lane = lane_id();
    double key[4];
#pragma unroll
    for (int i = 0; i < 4; i++) key[i] = topk_key(v[i], lane + 64 * i, E);
    auto cx = [&](int a, int b) {          // order slots a > b
        const double hi = fmax(key[a], key[b]), lo = fmin(key[a], key[b]);
        key[a] = hi;
        key[b] = lo;
    };
    cx(0, 1); cx(2, 3); cx(0, 2); cx(1, 3); cx(1, 2);
    double pk = 1.0, k0 = 1.0;
    for (int j = 0; j < k; j++) {
        const double m = wave_max_f64(key[0]);
        if (j == 0) k0 = m;
        if (lane == j) pk = m;
        if (key[0] == m) {
            key[0] = key[1]; key[1] = key[2]; key[2] = key[3]; key[3] = 0.0;
        }
    }
    float pv, m0;
    int pi, e0;
    topk_key_decode(pk, pv, pi);
    topk_key_decode(k0, m0, e0);
    const float ex = lane < k ? __expf(pv - m0) : 0.f;
    const float z = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(row16_sum(ex)), 15));
    if (lane < k) {
        if (ids) ids[lane] = pi;
        if (wout) wout[lane] = ex * (1.0f / z);
        if (sids) sids[lane] = pi;
    }
    return pi;
}

using bm_cfg::kBT;                  // threads per bucketing block = pairs per chunk
using bm_cfg::kBW;                  // waves per block

BM_DEV int key_bits(int E) {        // bits needed for keys 0..E (E = "no pair")
    int b = 1;
    while ((1 << b) <= E) b++;
    return b;
}

// Exclusive scan over the block; returns the prefix of v, sets *total.
BM_DEV int block_exscan(int v, int *swave, int *total) {
    int lane = lane_id(), w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) swave[w] = x;
    __syncthreads();
    if (w == 0) {
        int s = lane < nw ? swave[lane] : 0, c = s;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            int y = __shfl_up(c, o, 64);
            if (lane >= o) c += y;
        }
        if (lane < nw) swave[lane] = c - s;
        if (lane == nw - 1) swave[kBW] = c;
    }
    __syncthreads();
    int r = x - v + swave[w];
    *total = swave[kBW];
    __syncthreads();
    return r;
}

// Match set and rank of this lane's key among the lanes of its wave.
BM_DEV void wave_match(int key, int kbits, uint64_t &match, int &rank) {
    uint64_t m = __ballot(1);
    for (int b = 0; b < kbits; b++) {
        int bit = (key >> b) & 1;
        uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    uint64_t lt = (1ull << lane_id()) - 1ull;
    match = m;
    rank = __popcll(m & lt);
}

// Stable scatter of one chunk of kBT pairs starting at p0.  base[e] holds the
// first perm slot of expert e for this chunk; wcnt is [kBW][E] LDS, zeroed.
BM_DEV void scatter_chunk(const int32_t *__restrict__ ids, int n, int E, int p0, const int *base,
                          int *wcnt, int32_t *__restrict__ perm, int kbits) {
    int tid = threadIdx.x, w = tid >> 6;
    int p = p0 + tid;
    int key = p < n ? user_id(ids[p], E) : E;
    uint64_t match;
    int rank;
    wave_match(key, kbits, match, rank);
    if (key < E && rank == 0) wcnt[w * E + key] = __popcll(match);
    __syncthreads();
    if (key < E) {
        int pos = base[key] + rank;
        for (int v = 0; v < w; v++) pos += wcnt[v * E + key];
        perm[pos] = p;
    }
}

// Active list (ascending experts with pairs) and the row-tile list.  The
// tiles are listed by their count of 32-row blocks, largest first (full
// tiles of every expert in expert order, then each expert's last tile by
// its blocks), so that the grouped GEMMs dispatch the longest tiles first
// and the shortest fill the last round.
BM_DEV int tile_class(int c, int tile_rows, int &nt) {      // blocks of the last tile, at most 3 (0: none)
    nt = (c + tile_rows - 1) / tile_rows;
    return nt ? min((c - (nt - 1) * tile_rows + 31) / 32, 3) : 0;
}
BM_DEV void active_and_tiles(const int *scount, int E, int32_t *__restrict__ active,
                             int32_t *__restrict__ n_active, int32_t *__restrict__ tiles,
                             int32_t *__restrict__ n_tiles, int tile_rows, int *swave) {
    int tid = threadIdx.x;
    const int full_cls = min((tile_rows + 31) / 32, 3);
    if (E <= kBT && full_cls == 3) {
        // one chunk of experts, full tiles of class 3 (the prefill tiles):
        // the class counts come with the positions, from one scan of the
        // class-3 tiles and one of the class-2 and class-1 last tiles packed
        // (at most one per expert each, E <= kBT < 2^16)
        const int e = tid, c = e < E ? scount[e] : 0;
        int tot;
        const int a = block_exscan(c > 0 ? 1 : 0, swave, &tot);
        if (e < E) active[e] = -1;
        __syncthreads();
        if (e < E && c > 0) active[a] = e;
        if (tiles) {
            int nt;
            const int cl = tile_class(c, tile_rows, nt);
            const int n3 = (nt > 1 ? nt - 1 : 0) + (cl == 3 ? 1 : 0);
            int t3, t21;
            const int p3 = block_exscan(n3, swave, &t3);
            const int p21 = block_exscan((cl == 2 ? 1 : 0) | (cl == 1 ? 1 << 16 : 0), swave, &t21);
            const int t2 = t21 & 0xFFFF, t1 = t21 >> 16;
            for (int i = 0; i + 1 < nt; i++) {
                tiles[2 * (p3 + i)] = e;
                tiles[2 * (p3 + i) + 1] = i * tile_rows;
            }
            if (cl > 0) {
                const int pos = cl == 3 ? p3 + nt - 1 : cl == 2 ? t3 + (p21 & 0xFFFF) : t3 + t2 + (p21 >> 16);
                tiles[2 * pos] = e;
                tiles[2 * pos + 1] = (nt - 1) * tile_rows;
            }
            if (tid == 0 && n_tiles) *n_tiles = t3 + t2 + t1;
        }
        if (tid == 0) *n_active = tot;
        return;
    }
    // tiles: first pass, the count of each class (full tiles are of class
    // full_cls; the last tile of an expert of its own blocks)
    int cls_base[4] = {0, 0, 0, 0};
    if (tiles) {
        int tot[4] = {0, 0, 0, 0};
        for (int e0 = 0; e0 < E; e0 += kBT) {
            const int e = e0 + tid, c = e < E ? scount[e] : 0;
            int nt;
            const int cl = tile_class(c, tile_rows, nt);
#pragma unroll
            for (int k = 1; k <= 3; k++) {
                const int m = (k == cl ? 1 : 0) + (k == full_cls && nt > 1 ? nt - 1 : 0);
                int t;
                block_exscan(m, swave, &t);
                tot[k] += t;
            }
        }
        for (int k = 3, acc = 0; k >= 1; k--) {
            cls_base[k] = acc;
            acc += tot[k];
        }
    }
    for (int e0 = 0, abase = 0; e0 < E; e0 += kBT) {
        int e = e0 + tid;
        int c = e < E ? scount[e] : 0;
        int tot;
        int a = block_exscan(c > 0 ? 1 : 0, swave, &tot);
        if (e < E) {
            active[e] = -1;
        }
        __syncthreads();
        if (e < E && c > 0) active[abase + a] = e;
        abase += tot;
        if (tiles) {
            int nt;
            const int cl = tile_class(c, tile_rows, nt);
#pragma unroll
            for (int k = 1; k <= 3; k++) {
                const int nfull = k == full_cls && nt > 1 ? nt - 1 : 0;
                const int m = (k == cl ? 1 : 0) + nfull;
                int t;
                const int t0 = cls_base[k] + block_exscan(m, swave, &t);
                for (int i = 0; i < nfull; i++) {
                    tiles[2 * (t0 + i)] = e;
                    tiles[2 * (t0 + i) + 1] = i * tile_rows;
                }
                if (k == cl) {
                    tiles[2 * (t0 + nfull)] = e;
                    tiles[2 * (t0 + nfull) + 1] = (nt - 1) * tile_rows;
                }
                cls_base[k] += t;
            }
        }
        if (e0 + kBT >= E && tid == 0) {
            *n_active = abase;
            if (n_tiles) *n_tiles = cls_base[1];
        }
    }
}


// ---- small-batch bucketing by one wavefront (n <= 128 pairs) -------------
// Stage 1: the stable rank of every pair among all pairs (key = expert id,
// ties by pair index) from ballots over the key bits, most significant
// first; perm[rank] = pair, and the keys in sorted order into LDS sk[].
// Stage 2 (after a block barrier): the ascending active list, and counts
// and offsets of the active experts only (other entries are not written).
using bm_cfg::kWaveBucketMax;

BM_DEV void bucket_wave_rank(const int32_t *__restrict__ ids, int n, int E, int32_t *__restrict__ perm,
                             int *sk) {
    const int lane = lane_id();
    const int kb = key_bits(E);
    const uint64_t below = (1ull << lane) - 1ull;
    const int M = n > 64 ? 2 : 1;
    int key[2];
#pragma unroll
    for (int m = 0; m < 2; m++) {
        const int p = lane + 64 * m;
        key[m] = p < n ? user_id(ids[p], E) : E;
    }
    for (int m = 0; m < M; m++) {
        int rank = 0;
        for (int m2 = 0; m2 < M; m2++) {
            uint64_t eq = ~0ull;
            int less = 0;
            for (int b = kb - 1; b >= 0; b--) {
                const uint64_t B = __ballot((key[m2] >> b) & 1);
                if ((key[m] >> b) & 1) {
                    less += __popcll(eq & ~B);
                    eq &= B;
                } else {
                    eq &= ~B;
                }
            }
            rank += less + (m2 < m ? __popcll(eq) : m2 == m ? __popcll(eq & below) : 0);
        }
        const int p = lane + 64 * m;
        if (p < n) {
            perm[rank] = p;
            sk[rank] = key[m];
        }
    }
}

BM_DEV void bucket_wave_lists(int n, const int *sk, int32_t *__restrict__ counts,
                              int32_t *__restrict__ offsets, int32_t *__restrict__ active,
                              int32_t *__restrict__ n_active) {
    const int lane = lane_id();
    const uint64_t below = (1ull << lane) - 1ull;
    bool lead[2];
    int key[2];
#pragma unroll
    for (int m = 0; m < 2; m++) {
        const int r = lane + 64 * m;
        key[m] = r < n ? sk[r] : -1;
        lead[m] = r < n && (r == 0 || sk[r - 1] != key[m]);
    }
    const uint64_t L0 = __ballot(lead[0]), L1 = __ballot(lead[1]);
    const int na = __popcll(L0) + __popcll(L1);
#pragma unroll
    for (int m = 0; m < 2; m++) {
        if (!lead[m]) continue;
        const int r = lane + 64 * m;
        const int slot = m == 0 ? __popcll(L0 & below) : __popcll(L0) + __popcll(L1 & below);
        // next leader after r, else n
        int next = n;
        const uint64_t a0 = m == 0 ? (L0 & ~(below | (1ull << lane))) : 0ull;
        const uint64_t a1 = m == 0 ? L1 : (L1 & ~(below | (1ull << lane)));
        if (a0) next = (int)__builtin_ctzll(a0);
        else if (a1) next = 64 + (int)__builtin_ctzll(a1);
        active[slot] = key[m];
        offsets[key[m]] = r;
        counts[key[m]] = next - r;
    }
    if (lane == 0) *n_active = na;
}

// After bucket_wave_rank (sk[] = the n sorted keys): one row tile (e, 0) for
// every expert holding more than one pair, in ascending expert order, and
// their count.  One wavefront; every such expert must hold at most one
// tile's rows.
BM_DEV void bucket_wave_multi_tiles(int n, const int *sk, int32_t *__restrict__ tiles,
                                    int32_t *__restrict__ n_tiles) {
    const int lane = lane_id();
    const uint64_t below = (1ull << lane) - 1ull;
    bool lead[2], multi[2];
    int key[2];
#pragma unroll
    for (int m = 0; m < 2; m++) {
        const int r = lane + 64 * m;
        key[m] = r < n ? sk[r] : -1;
        lead[m] = r < n && (r == 0 || sk[r - 1] != key[m]);
        multi[m] = lead[m] && r + 1 < n && sk[r + 1] == key[m];
    }
    const uint64_t M0 = __ballot(multi[0]), M1 = __ballot(multi[1]);
#pragma unroll
    for (int m = 0; m < 2; m++) {
        if (!multi[m]) continue;
        const int pos = m == 0 ? __popcll(M0 & below) : __popcll(M0) + __popcll(M1 & below);
        tiles[2 * pos] = key[m];
        tiles[2 * pos + 1] = 0;
    }
    if (lane == 0) *n_tiles = __popcll(M0) + __popcll(M1);
}

// Single-workgroup bucketing of n <= a few thousand pairs (kBT threads):
// counts, offsets, stable perm, active list [, row tiles].  smem must hold
// (2 + kBW) * E ints; swave kBW + 1 ints.
BM_DEV void bucket_block(const int32_t *__restrict__ ids, int n, int E, int32_t *__restrict__ counts,
                         int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
                         int32_t *__restrict__ active, int32_t *__restrict__ n_active,
                         int32_t *__restrict__ tiles, int32_t *__restrict__ n_tiles, int tile_rows,
                         int *smem, int *swave) {
    int *scount = smem;               // [E]
    int *sbase = scount + E;          // [E]
    int *wcnt = sbase + E;            // [kBW][E]
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kBT) scount[e] = 0;
    for (int i = tid; i < kBW * E; i += kBT) wcnt[i] = 0;
    __syncthreads();
    for (int p = tid; p < n; p += kBT) atomicAdd(&scount[user_id(ids[p], E)], 1);
    __syncthreads();
    {
        const int c = tid < E ? scount[tid] : 0;
        int tot;
        const int o = block_exscan(c, swave, &tot);
        if (tid < E) {
            counts[tid] = c;
            offsets[tid] = o;
            sbase[tid] = o;
        }
        if (tid == 0) offsets[E] = tot;
    }
    __syncthreads();
    active_and_tiles(scount, E, active, n_active, tiles, n_tiles, tile_rows, swave);
    const int kbits = key_bits(E);
    for (int p0 = 0; p0 < n; p0 += kBT) {
        scatter_chunk(ids, n, E, p0, sbase, wcnt, perm, kbits);
        __syncthreads();
        for (int e = tid; e < E; e += kBT) {
            int s = 0;
            for (int v = 0; v < kBW; v++) {
                s += wcnt[v * E + e];
                wcnt[v * E + e] = 0;
            }
            sbase[e] += s;
        }
        __syncthreads();
    }
}

}  // namespace bm
