// Host sanitizer driver for the routed-expert residency cache (test
// infrastructure): a small layer whose host slabs carry a per-expert byte
// pattern, a host buffer in the pool's place (the HIP stand-in copies with
// memcpy), and a scripted sequence of routing steps.  After every step the
// driver checks that each occupied slot holds exactly its expert's bytes
// (gate, up and down), and prints the slot ids, the copy count and the
// expert of every slot for the test to compare with its own LRU model.
// Ends with the argument checks.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/bitmoe.h"

static int failures = 0;
#define EXPECT(c)                                                       \
    do {                                                                \
        if (!(c)) {                                                     \
            std::printf("FAILED line %d: %s\n", __LINE__, #c);          \
            failures++;                                                 \
        }                                                               \
    } while (0)

static uint8_t pattern(int tensor, int e, size_t i) { return (uint8_t)(31 * tensor + 7 * e + i * 13 + (i >> 9)); }

int main() {
    const int H = 256, I = 256, E = 8, k = 2, slots = 4;
    const size_t sg = (size_t)I * (H / 256) * 66, sd = (size_t)H * (I / 256) * 84;
    std::vector<uint8_t> host[3];
    const size_t sz[3] = {sg, sg, sd};
    for (int t = 0; t < 3; t++) {
        host[t].resize(E * sz[t]);
        for (int e = 0; e < E; e++)
            for (size_t i = 0; i < sz[t]; i++) host[t][e * sz[t] + i] = pattern(t, e, i);
    }
    bitmoe_layer L;
    std::memset(&L, 0, sizeof L);
    L.H = H; L.I = I; L.E = E; L.k = k;
    L.router_w = L.grid = reinterpret_cast<void *>(uintptr_t(4096));
    L.layout = BITMOE_LAYOUT_TILED;
    const size_t pb = moe_cache_pool_bytes(&L, slots);
    EXPECT(pb > 0);
    std::vector<uint8_t> pool(pb);
    void *cache = nullptr;
    EXPECT(moe_cache_create(&L, host[0].data(), host[1].data(), host[2].data(), slots, pool.data(), pb, &cache) == 0);
    bitmoe_layer P;
    EXPECT(moe_cache_layer(cache, &P) == 0);
    EXPECT(P.E == slots && P.k == k && P.layout == BITMOE_LAYOUT_TILED && P.router_w == L.router_w);
    const uint8_t *base[3] = {static_cast<const uint8_t *>(P.gate_q), static_cast<const uint8_t *>(P.up_q),
                              static_cast<const uint8_t *>(P.down_q)};
    // steps of routing ids (n values each)
    const std::vector<std::vector<int>> steps = {
        {3, 5}, {5, 1, 3, 6}, {0, 7}, {7, 0, 3, 3}, {2, 4, 6, 1}, {1, 1}, {5, 6, 7, 0}, {2, 2, 2, 2}, {4, 3}};
    for (const auto &ids : steps) {
        std::vector<int32_t> id(ids.begin(), ids.end()), slot(ids.size(), -9);
        int loaded = -1;
        EXPECT(moe_cache_map(cache, id.data(), (int)id.size(), slot.data(), &loaded, nullptr) == 0);
        int32_t in_slot[slots];
        int64_t hits = 0, misses = 0;
        EXPECT(moe_cache_stats(cache, &hits, &misses, in_slot) == 0);
        std::printf("step");
        for (int32_t s : slot) std::printf(" %d", s);
        std::printf(" | loaded %d | slots", loaded);
        for (int j = 0; j < slots; j++) std::printf(" %d", in_slot[j]);
        std::printf(" | hits %lld misses %lld\n", (long long)hits, (long long)misses);
        for (size_t i = 0; i < id.size(); i++) EXPECT(slot[i] >= 0 && in_slot[slot[i]] == id[i]);
        for (int j = 0; j < slots; j++) {
            if (in_slot[j] < 0) continue;
            for (int t = 0; t < 3; t++)
                EXPECT(std::memcmp(base[t] + j * sz[t], host[t].data() + in_slot[j] * sz[t], sz[t]) == 0);
        }
    }
    // argument checks
    int32_t bad[2] = {0, E}, out[2];
    EXPECT(moe_cache_map(cache, bad, 2, out, nullptr, nullptr) == BITMOE_EINVAL);
    int32_t many[5] = {0, 1, 2, 3, 4};
    EXPECT(moe_cache_map(cache, many, 5, out, nullptr, nullptr) == BITMOE_EUNSUPPORTED);
    EXPECT(moe_cache_map(cache, many, 0, nullptr, nullptr, nullptr) == 0);
    EXPECT(moe_cache_map(nullptr, many, 2, out, nullptr, nullptr) == BITMOE_EINVAL);
    void *c2 = nullptr;
    EXPECT(moe_cache_create(&L, host[0].data(), host[1].data(), host[2].data(), slots, pool.data(), pb - 1, &c2) ==
           BITMOE_EWORKSPACE);
    EXPECT(moe_cache_create(&L, host[0].data(), host[1].data(), host[2].data(), 1, pool.data(), pb, &c2) ==
           BITMOE_EINVAL);                                      // fewer slots than k
    EXPECT(moe_cache_create(&L, nullptr, host[1].data(), host[2].data(), slots, pool.data(), pb, &c2) == BITMOE_EINVAL);
    EXPECT(moe_cache_pool_bytes(&L, E + 1) == 0);
    EXPECT(moe_cache_destroy(cache) == 0);
    std::printf(failures ? "cache sanitizer driver: %d check(s) failed\n" : "cache sanitizer driver: ok\n", failures);
    return failures ? 1 : 0;
}
