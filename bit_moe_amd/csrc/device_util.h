// Device-side building blocks shared by routing, bucketing and the fused
// decode pipeline: per-wave top-k with renormalised softmax, and the
// stable counting-sort pieces of the token -> expert bucketing.
#pragma once

#include "common.h"

namespace bm {

// Top-k of one token's logits by one wavefront: repeated wave argmax
// (larger value, then lower index), then softmax over the k selected.
// Lane 0 writes ids[0..k) and w[0..k).  E <= 1024, k <= 16.
BM_DEV void topk_wave(const float *__restrict__ lrow, int E, int k, int32_t *__restrict__ ids,
                      float *__restrict__ wout) {
    const int lane = lane_id();
    constexpr int MAXV = 16;
    float v[MAXV];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < MAXV; i++) {
        const int e = lane + 64 * i;
        v[i] = e < E ? lrow[e] : 0.f;
    }
    float sel[16];
    int sid[16];
    for (int j = 0; j < k; j++) {
        float bv = 0.f;
        int be = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < MAXV; i++) {
            const int e = lane + 64 * i;
            const bool ok = e < E && !((taken >> i) & 1u);
            if (ok && (be == 0x7FFFFFFF || v[i] > bv)) { bv = v[i]; be = e; }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o, 64);
            const int oe = __shfl_xor(be, o, 64);
            const bool better = (oe != 0x7FFFFFFF) &&
                                (be == 0x7FFFFFFF || ov > bv || (ov == bv && oe < be));
            if (better) { bv = ov; be = oe; }
        }
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        sel[j] = bv;
        sid[j] = be;
    }
    if (lane == 0) {
        float z = 0.f, ex[16];
        for (int j = 0; j < k; j++) { ex[j] = __expf(sel[j] - sel[0]); z += ex[j]; }
        const float inv = 1.0f / z;
        for (int j = 0; j < k; j++) {
            ids[j] = sid[j];
            wout[j] = ex[j] * inv;
        }
    }
}

constexpr int kBT = 1024;           // threads per bucketing block = pairs per chunk
constexpr int kBW = kBT / 64;       // waves per block

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
    int key = p < n ? ids[p] : E;
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

// Active list (ascending experts with pairs) and the row-tile list.
BM_DEV void active_and_tiles(const int *scount, int E, int32_t *__restrict__ active,
                             int32_t *__restrict__ n_active, int32_t *__restrict__ tiles,
                             int32_t *__restrict__ n_tiles, int tile_rows, int *swave) {
    int tid = threadIdx.x;
    for (int e0 = 0, abase = 0, tbase = 0; e0 < E; e0 += kBT) {
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
            int nt = (c + tile_rows - 1) / tile_rows, ttot;
            int t0 = block_exscan(nt, swave, &ttot);
            for (int i = 0; i < nt; i++) {
                tiles[2 * (tbase + t0 + i)] = e;
                tiles[2 * (tbase + t0 + i) + 1] = i * tile_rows;
            }
            tbase += ttot;
        }
        if (e0 + kBT >= E && tid == 0) {
            *n_active = abase;
            if (n_tiles) *n_tiles = tbase;
        }
    }
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
    for (int p = tid; p < n; p += kBT) atomicAdd(&scount[ids[p]], 1);
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
