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
#include "device_util.h"

namespace {

using namespace bm;

// ---- single-block path (small T*k) -----------------------------------------
__global__ void __launch_bounds__(kBT)
k_bucket_small(const int32_t *__restrict__ ids, int n, int E, int32_t *__restrict__ counts,
               int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
               int32_t *__restrict__ active, int32_t *__restrict__ n_active,
               int32_t *__restrict__ tiles, int32_t *__restrict__ n_tiles, int tile_rows) {
    extern __shared__ int smem[];
    __shared__ int swave[kBW + 1];
    bucket_block(ids, n, E, counts, offsets, perm, active, n_active, tiles, n_tiles, tile_rows, smem,
                 swave);
}

// ---- the checked build's count of ids outside [0, E) ------------------------
// One workgroup, a fixed order of partial sums: flag = the count (0: all in
// range).
__global__ void __launch_bounds__(kBT)
k_check_ids(const int32_t *__restrict__ ids, int64_t n, int E, int32_t *__restrict__ flag) {
    __shared__ int swave[kBW + 1];
    int bad = 0;
    for (int64_t p = threadIdx.x; p < n; p += kBT) bad += (ids[p] < 0 || ids[p] >= E) ? 1 : 0;
    int tot;
    (void)block_exscan(bad, swave, &tot);
    if (threadIdx.x == 0) *flag = tot;
}

// ---- multi-block path -------------------------------------------------------
__global__ void __launch_bounds__(kBT)
k_bucket_hist(const int32_t *__restrict__ ids, int n, int E, int32_t *__restrict__ bhist) {
    extern __shared__ int sh[];
    int tid = threadIdx.x;
    for (int e = tid; e < E; e += kBT) sh[e] = 0;
    __syncthreads();
    int p = blockIdx.x * kBT + tid;
    if (p < n) atomicAdd(&sh[user_id(ids[p], E)], 1);
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
    // the blocks' counts in batches of kB loads issued together, then their
    // prefix (a load after each store would wait for it: one round trip per
    // block)
    constexpr int kB = 16;
    if (e < E)
        for (int b0 = 0; b0 < nblk; b0 += kB) {
            int c[kB];
#pragma unroll
            for (int i = 0; i < kB; i++) c[i] = b0 + i < nblk ? bhist[(int64_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < kB; i++)
                if (b0 + i < nblk) {
                    bhist[(int64_t)(b0 + i) * E + e] = run;        // rows of e in earlier blocks
                    run += c[i];
                }
        }
    int tot;
    int o = block_exscan(e < E ? run : 0, swave, &tot);
    if (e < E) {
        counts[e] = run;
        offsets[e] = o;
        scount[e] = run;
        for (int b0 = 0; b0 < nblk; b0 += kB) {
            int v[kB];
#pragma unroll
            for (int i = 0; i < kB; i++) v[i] = b0 + i < nblk ? bhist[(int64_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < kB; i++)
                if (b0 + i < nblk) bhist[(int64_t)(b0 + i) * E + e] = v[i] + o;
        }
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

using bm_cfg::kSmallPairs;

// Dynamic LDS above 64 KiB (E close to 1024) must be opted into per kernel.
template <class K>
static void allow_lds(K kernel, size_t bytes) {
    if (bytes > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

int launch_check_ids(const int32_t *ids, int64_t n, int E, int32_t *flag, hipStream_t s) {
    if (!BITMOE_CHECK_IDS || n == 0) return BITMOE_OK;
    k_check_ids<<<1, kBT, 0, s>>>(ids, n, E, flag);
    BM_LAUNCH_CHECK();
    return BITMOE_OK;
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
