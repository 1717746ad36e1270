// Routed-expert residency cache: the routed experts' packed weights live in
// (pinned) host memory and a pool of HBM slots holds the ones in use; each
// decode step maps its routing onto slots, copying missing experts in on the
// caller's stream.  This is the pages' SSD streaming of routed experts
// through an in-memory expert cache, non-routed weights staying resident
// ("Faire tenir un MoE de 284B dans un portable de 128 Go", section
// "Streaming depuis le SSD quand la memoire fait defaut"; "ds4 : analyse
// pratique pour un usage documente", section "Executer des modeles plus
// grands que la RAM avec le streaming SSD"), one level up: host memory plays
// the SSD and HBM the cache.
//
// Policy (deterministic): a step's distinct experts, in order of first
// appearance in ids, are served from their slot when resident; a missing
// expert takes the lowest-numbered empty slot, else the least recently used
// slot not used by this step (ties to the lower slot).  Host code only.
#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "host.h"

namespace {

constexpr size_t kAlign = 256;
inline size_t up256(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

struct Cache {
    bitmoe_layer dev;                         // router, grid, shared (device); routed slabs: the pool
    const char *host[3];                      // gate, up, down slabs of all E experts (host)
    size_t slab[3];                           // bytes of one expert's slab of each tensor
    char *pool[3];                            // pool regions [slots][slab]
    int slots;
    std::vector<int> slot_of, expert_in;      // expert -> slot (-1), slot -> expert (-1)
    std::vector<int64_t> last_use;            // slot -> step of last use
    int64_t step = 0, hits = 0, misses = 0;
};

void slabs(const bitmoe_layer *L, size_t (&s)[3]) {
    if (L->format == BITMOE_FORMAT_MXFP4) {
        s[0] = s[1] = (size_t)L->I * (L->H / 32) * 17;
        s[2] = (size_t)L->H * (L->I / 32) * 17;
        return;
    }
    s[0] = s[1] = (size_t)L->I * (L->H / 256) * 66;
    s[2] = (size_t)L->H * (L->I / 256) * 84;
}

int check_cache_layer(const bitmoe_layer *L) {
    if (!L) return BITMOE_EINVAL;
    if (L->H <= 0 || L->I <= 0 || L->E <= 0 || L->k <= 0) return BITMOE_EINVAL;
    if (L->format != BITMOE_FORMAT_2BIT && L->format != BITMOE_FORMAT_MXFP4) return BITMOE_EINVAL;
    if (L->H % 256 || L->I % 256 || L->k > 16 || L->k > L->E || L->E > 1024) return BITMOE_EUNSUPPORTED;
    return BITMOE_OK;
}

}  // namespace

extern "C" {

size_t moe_cache_pool_bytes(const bitmoe_layer *L, int slots) {
    if (check_cache_layer(L) || slots < L->k || slots > L->E) return 0;
    size_t s[3];
    slabs(L, s);
    return 3 * kAlign + (size_t)slots * (s[0] + s[1] + s[2]);
}

int moe_cache_create(const bitmoe_layer *L, const void *host_gate, const void *host_up, const void *host_down,
                     int slots, void *pool, size_t pool_bytes, void **cache) {
    int rc = check_cache_layer(L);
    if (rc) return rc;
    if (!cache || !host_gate || !host_up || !host_down || !pool) return BITMOE_EINVAL;
    if (L->format == BITMOE_FORMAT_2BIT && !L->grid) return BITMOE_EINVAL;
    if (slots < L->k || slots > L->E) return BITMOE_EINVAL;
    if ((L->shared_gate != nullptr) != (L->shared_up != nullptr) ||
        (L->shared_up != nullptr) != (L->shared_down != nullptr))
        return BITMOE_EINVAL;
    if (pool_bytes < moe_cache_pool_bytes(L, slots)) return BITMOE_EWORKSPACE;
    Cache *c = new (std::nothrow) Cache;
    if (!c) return BITMOE_EINVAL;
    c->dev = *L;
    c->host[0] = static_cast<const char *>(host_gate);
    c->host[1] = static_cast<const char *>(host_up);
    c->host[2] = static_cast<const char *>(host_down);
    slabs(L, c->slab);
    char *p = reinterpret_cast<char *>(up256(reinterpret_cast<uintptr_t>(pool)));
    for (int t = 0; t < 3; t++) {
        c->pool[t] = p;
        p = reinterpret_cast<char *>(up256(reinterpret_cast<uintptr_t>(p + (size_t)slots * c->slab[t])));
    }
    c->slots = slots;
    c->slot_of.assign(L->E, -1);
    c->expert_in.assign(slots, -1);
    c->last_use.assign(slots, -1);
    c->dev.E = slots;
    c->dev.gate_q = c->pool[0];
    c->dev.up_q = c->pool[1];
    c->dev.down_q = c->pool[2];
    c->dev.layout = BITMOE_LAYOUT_TILED;
    *cache = c;
    return BITMOE_OK;
}

int moe_cache_destroy(void *cache) {
    delete static_cast<Cache *>(cache);
    return BITMOE_OK;
}

int moe_cache_layer(const void *cache, bitmoe_layer *out) {
    if (!cache || !out) return BITMOE_EINVAL;
    const Cache *c = static_cast<const Cache *>(cache);
    *out = c->dev;
    return BITMOE_OK;
}

int moe_cache_map(void *cache, const int32_t *ids, int n, int32_t *slot_ids, int *loaded, void *stream) {
    if (!cache || n < 0) return BITMOE_EINVAL;
    if (n == 0) {
        if (loaded) *loaded = 0;
        return BITMOE_OK;
    }
    if (!ids || !slot_ids) return BITMOE_EINVAL;
    Cache *c = static_cast<Cache *>(cache);
    const int E = (int)c->slot_of.size();
    for (int i = 0; i < n; i++)
        if (ids[i] < 0 || ids[i] >= E) return BITMOE_EINVAL;
    // the step's distinct experts, first appearance first
    std::vector<int> distinct;
    std::vector<char> seen(E, 0);
    for (int i = 0; i < n; i++)
        if (!seen[ids[i]]) {
            seen[ids[i]] = 1;
            distinct.push_back(ids[i]);
        }
    if ((int)distinct.size() > c->slots) return BITMOE_EUNSUPPORTED;
    const int64_t step = ++c->step;
    for (int e : distinct)
        if (c->slot_of[e] >= 0) c->last_use[c->slot_of[e]] = step;
    int nload = 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (int e : distinct) {
        if (c->slot_of[e] >= 0) {
            c->hits++;
            continue;
        }
        int victim = -1;
        for (int j = 0; j < c->slots && victim < 0; j++)
            if (c->expert_in[j] < 0) victim = j;
        if (victim < 0)
            for (int j = 0; j < c->slots; j++)
                if (c->last_use[j] < step && (victim < 0 || c->last_use[j] < c->last_use[victim])) victim = j;
        if (victim < 0) return BITMOE_EUNSUPPORTED;      // (cannot happen: distinct <= slots)
        if (c->expert_in[victim] >= 0) c->slot_of[c->expert_in[victim]] = -1;
        c->expert_in[victim] = e;
        c->slot_of[e] = victim;
        c->last_use[victim] = step;
        for (int t = 0; t < 3; t++)
            if (hipMemcpyAsync(c->pool[t] + (size_t)victim * c->slab[t], c->host[t] + (size_t)e * c->slab[t],
                               c->slab[t], hipMemcpyHostToDevice, s) != hipSuccess) {
                c->slot_of[e] = -1;                    // the slot holds no whole expert now
                c->expert_in[victim] = -1;
                c->last_use[victim] = -1;
                return BITMOE_EHIP;
            }
        c->misses++;
        nload++;
    }
    for (int i = 0; i < n; i++) slot_ids[i] = c->slot_of[ids[i]];
    if (loaded) *loaded = nload;
    return BITMOE_OK;
}

int moe_cache_stats(const void *cache, int64_t *hits, int64_t *misses, int32_t *expert_in_slot) {
    if (!cache) return BITMOE_EINVAL;
    const Cache *c = static_cast<const Cache *>(cache);
    if (hits) *hits = c->hits;
    if (misses) *misses = c->misses;
    if (expert_in_slot) std::copy(c->expert_in.begin(), c->expert_in.end(), expert_in_slot);
    return BITMOE_OK;
}

}  // extern "C"
