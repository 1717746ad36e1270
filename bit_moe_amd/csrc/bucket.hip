// Token -> expert bucketing: per-expert counts, exclusive prefix-sum offsets,
// a stable permutation of the (token, slot) pairs grouped by expert, the list
// of active experts (each streamed once however many tokens chose it) and,
// for the grouped GEMM, a list of (expert, first row) tiles.
//
// Stability without sorting: inside a wavefront, lanes holding the same
// expert find each other with one ballot per bit of the expert index; their
// rank is the popcount of the lower lanes in that match set.  Per-wave counts
// go to LDS so each lane also knows how many earlier waves (and, through the
// histogram pass, earlier blocks) hit its expert.
#include "common.h"

namespace {

using namespace bm;

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

// ---- single-block path (small T*k) -----------------------------------------
__global__ void __launch_bounds__(kBT)
k_bucket_small(const int32_t *__restrict__ ids, int n, int E, int32_t *__restrict__ counts,
               int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
               int32_t *__restrict__ active, int32_t *__restrict__ n_active,
               int32_t *__restrict__ tiles, int32_t *__restrict__ n_tiles, int tile_rows) {
    extern __shared__ int smem[];
    int *scount = smem;               // [E]
    int *sbase = scount + E;          // [E]
    int *wcnt = sbase + E;            // [kBW][E]
    __shared__ int swave[kBW + 1];
    int tid = threadIdx.x;
    for (int e = tid; e < E; e += kBT) scount[e] = 0;
    for (int i = tid; i < kBW * E; i += kBT) wcnt[i] = 0;
    __syncthreads();
    for (int p = tid; p < n; p += kBT) atomicAdd(&scount[ids[p]], 1);
    __syncthreads();
    // offsets = exclusive scan of counts (E <= 1024 = kBT)
    {
        int c = tid < E ? scount[tid] : 0, tot;
        int o = block_exscan(c, swave, &tot);
        if (tid < E) {
            counts[tid] = c;
            offsets[tid] = o;
            sbase[tid] = o;
        }
        if (tid == 0) offsets[E] = tot;
    }
    __syncthreads();
    active_and_tiles(scount, E, active, n_active, tiles, n_tiles, tile_rows, swave);
    int kbits = key_bits(E);
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

// ---- multi-block path -------------------------------------------------------
__global__ void __launch_bounds__(kBT)
k_bucket_hist(const int32_t *__restrict__ ids, int n, int E, int32_t *__restrict__ bhist) {
    extern __shared__ int sh[];
    int tid = threadIdx.x;
    for (int e = tid; e < E; e += kBT) sh[e] = 0;
    __syncthreads();
    int p = blockIdx.x * kBT + tid;
    if (p < n) atomicAdd(&sh[ids[p]], 1);
    __syncthreads();
    for (int e = tid; e < E; e += kBT) bhist[(int64_t)blockIdx.x * E + e] = sh[e];
}

__global__ void __launch_bounds__(kBT)
k_bucket_scan(int E, int nblk, int32_t *__restrict__ bhist, int32_t *__restrict__ counts,
              int32_t *__restrict__ offsets, int32_t *__restrict__ active,
              int32_t *__restrict__ n_active, int32_t *__restrict__ tiles,
              int32_t *__restrict__ n_tiles, int tile_rows) {
    extern __shared__ int scount[];   // [E]
    __shared__ int swave[kBW + 1];
    int tid = threadIdx.x;
    int e = tid;
    int run = 0;
    if (e < E)
        for (int b = 0; b < nblk; b++) {
            int c = bhist[(int64_t)b * E + e];
            bhist[(int64_t)b * E + e] = run;        // rows of e in earlier blocks
            run += c;
        }
    int tot;
    int o = block_exscan(e < E ? run : 0, swave, &tot);
    if (e < E) {
        counts[e] = run;
        offsets[e] = o;
        scount[e] = run;
        for (int b = 0; b < nblk; b++) bhist[(int64_t)b * E + e] += o;
    }
    if (tid == 0) offsets[E] = tot;
    __syncthreads();
    active_and_tiles(scount, E, active, n_active, tiles, n_tiles, tile_rows, swave);
}

__global__ void __launch_bounds__(kBT)
k_bucket_scatter(const int32_t *__restrict__ ids, int n, int E, const int32_t *__restrict__ bbase,
                 int32_t *__restrict__ perm) {
    extern __shared__ int smem[];
    int *sbase = smem;               // [E]
    int *wcnt = smem + E;            // [kBW][E]
    int tid = threadIdx.x;
    for (int e = tid; e < E; e += kBT) sbase[e] = bbase[(int64_t)blockIdx.x * E + e];
    for (int i = tid; i < kBW * E; i += kBT) wcnt[i] = 0;
    __syncthreads();
    scatter_chunk(ids, n, E, blockIdx.x * kBT, sbase, wcnt, perm, key_bits(E));
}

}  // namespace

namespace bm_host {

constexpr int kSmallPairs = 4096;

size_t bucket_scratch_bytes(int T, int k, int E) {
    int64_t n = (int64_t)T * k;
    if (n <= kSmallPairs) return 256;
    int64_t nblk = (n + kBT - 1) / kBT;
    return (size_t)(nblk * E * 4 + 255) / 256 * 256;
}

// Dynamic LDS above 64 KiB (E close to 1024) must be opted into per kernel.
template <class K>
static void allow_lds(K kernel, size_t bytes) {
    if (bytes > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

int launch_bucket(const int32_t *ids, int T, int k, int E, const Buckets &b, hipStream_t s) {
    int n = T * k;
    if (n <= kSmallPairs) {
        size_t sh = (size_t)(2 + kBW) * E * sizeof(int);
        allow_lds(k_bucket_small, sh);
        k_bucket_small<<<1, kBT, sh, s>>>(ids, n, E, b.counts, b.offsets, b.perm, b.active,
                                          b.n_active, b.tiles, b.n_tiles, b.tile_rows);
        BM_LAUNCH_CHECK();
        return BITMOE_OK;
    }
    int nblk = (n + kBT - 1) / kBT;
    k_bucket_hist<<<nblk, kBT, E * sizeof(int), s>>>(ids, n, E, b.scratch);
    BM_LAUNCH_CHECK();
    k_bucket_scan<<<1, kBT, E * sizeof(int), s>>>(E, nblk, b.scratch, b.counts, b.offsets, b.active,
                                                 b.n_active, b.tiles, b.n_tiles, b.tile_rows);
    BM_LAUNCH_CHECK();
    const size_t sh = (size_t)(1 + kBW) * E * sizeof(int);
    allow_lds(k_bucket_scatter, sh);
    k_bucket_scatter<<<nblk, kBT, sh, s>>>(ids, n, E, b.scratch, b.perm);
    BM_LAUNCH_CHECK();
    return BITMOE_OK;
}

}  // namespace bm_host
