// Host sanitizer driver for the C ABI (test infrastructure): every entry
// point's validation, the workspace sizing and carving over a sweep of
// shapes and token counts (up to the largest T a call accepts), under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Device pointers are
// fake aligned addresses that nothing dereferences: with valid arguments the
// calls reach the launcher stand-ins, which report BITMOE_EHIP.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/bitmoe.h"

static int failures = 0;
#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            std::printf("FAILED line %d: %s\n", __LINE__, #cond);           \
            failures++;                                                     \
        }                                                                   \
    } while (0)

static void *fake(uintptr_t a) { return reinterpret_cast<void *>(a); }

static bitmoe_layer layer(int H, int I, int E, int k, bool shared, int layout = BITMOE_LAYOUT_TILED,
                          int format = BITMOE_FORMAT_2BIT) {
    bitmoe_layer L;
    std::memset(&L, 0, sizeof(L));
    L.H = H; L.I = I; L.E = E; L.k = k;
    L.router_w = L.gate_q = L.up_q = L.down_q = L.grid = fake(1 << 20);
    if (shared) L.shared_gate = L.shared_up = L.shared_down = fake(2 << 20);
    L.layout = layout;
    L.format = format;
    if (format == BITMOE_FORMAT_MXFP4) L.grid = nullptr;       // not needed by MXFP4 layers
    return L;
}

int main() {
    const int shapes[][4] = {{256, 512, 8, 2}, {7168, 2048, 256, 8}, {512, 256, 1024, 16}, {256, 256, 1, 1}};
    const int tokens[] = {1, 2, 3, 4, 16, 17, 63, 64, 96, 97, 200, 2048, 8192, 65536, 1 << 20};
    void *x = fake(1 << 24), *out = fake(2 << 24), *ws = fake(3 << 24);
    for (int fmt = 0; fmt < 2; fmt++)
    for (const auto &s : shapes)
        for (int sh = 0; sh < 2; sh++) {
            bitmoe_layer L = layer(s[0], s[1], s[2], s[3], sh, BITMOE_LAYOUT_TILED, fmt);
            size_t prev[2] = {0, 0};
            for (int T : tokens) {
                for (int mode = 0; mode < 2; mode++) {
                    const size_t need = moe_workspace_bytes(&L, T, mode);
                    EXPECT(need > 0 && need % 256 == 0);
                    // prefill scratch grows with T; decode batches of up to 96
                    // tokens also carve the matrix-core path's buffers
                    if (mode == 1) EXPECT(need >= prev[mode]);
                    prev[mode] = need;
                    int32_t *ids = static_cast<int32_t *>(out);
                    float *w = static_cast<float *>(out), *y = static_cast<float *>(out);
                    auto ffn = mode ? moe_ffn_prefill : moe_ffn_decode;
                    EXPECT(ffn(&L, x, BITMOE_BF16, T, ids, w, y, ws, need, nullptr) == BITMOE_EHIP);
                    EXPECT(ffn(&L, x, BITMOE_BF16, T, ids, w, y, ws, need - 1, nullptr) == BITMOE_EWORKSPACE);
                    if (mode == 0) {
                        for (int dt = 0; dt < 2; dt++)
                            EXPECT(moe_forward_decode(&L, x, dt, T, ids, w, y, ws, need, nullptr) == BITMOE_EHIP);
                    }
                }
                for (int dt = 0; dt < 2; dt++) {
                    const size_t rneed = moe_route_workspace_bytes(&L, T, dt);
                    EXPECT(rneed > 0 && rneed % 256 == 0);
                    EXPECT(moe_route(&L, x, dt, T, nullptr, static_cast<int32_t *>(out), static_cast<float *>(out),
                                     ws, rneed, nullptr) == BITMOE_EHIP);
                    EXPECT(moe_route(&L, x, dt, T, nullptr, static_cast<int32_t *>(out), static_cast<float *>(out),
                                     ws, rneed - 1, nullptr) == BITMOE_EWORKSPACE);
                }
                const size_t bneed = moe_bucket_workspace_bytes(T, s[3], s[2]);
                int32_t *o32 = static_cast<int32_t *>(out);
                EXPECT(moe_bucket(o32, T, s[3], s[2], o32, o32, o32, o32, o32, ws, bneed, nullptr) == BITMOE_EHIP);
            }
            EXPECT(moe_workspace_bytes(&L, (1 << 20) + 1, 0) == 0);
            bitmoe_layer C = layer(s[0], s[1], s[2], s[3], sh, BITMOE_LAYOUT_CANONICAL);
            EXPECT(moe_workspace_bytes(&C, 4, 0) == 0);
            EXPECT(moe_ffn_decode(&C, x, 1, 4, static_cast<int32_t *>(out), static_cast<float *>(out),
                                  static_cast<float *>(out), ws, 1 << 30, nullptr) == BITMOE_EUNSUPPORTED);
        }
    // argument checks of every entry point
    bitmoe_layer L = layer(256, 512, 8, 2, false);
    int32_t *o32 = static_cast<int32_t *>(out);
    float *of = static_cast<float *>(out);
    EXPECT(moe_ffn_decode(nullptr, x, 1, 4, o32, of, of, ws, 1 << 20, nullptr) == BITMOE_EINVAL);
    EXPECT(moe_ffn_prefill(&L, x, 3, 4, o32, of, of, ws, 1 << 20, nullptr) == BITMOE_EINVAL);
    EXPECT(moe_ffn_prefill(&L, fake(8), 1, 4, o32, of, of, ws, 1 << 20, nullptr) == BITMOE_EINVAL);
    bitmoe_layer bad = layer(100, 512, 8, 2, false);
    EXPECT(moe_ffn_decode(&bad, x, 1, 4, o32, of, of, ws, 1 << 20, nullptr) == BITMOE_EUNSUPPORTED);
    bad = layer(256, 512, 8, 17, false);
    EXPECT(moe_route(&bad, x, 1, 4, nullptr, o32, of, ws, 1 << 20, nullptr) == BITMOE_EUNSUPPORTED);
    EXPECT(moe_topk(of, 4, 8, 9, o32, of, nullptr) == BITMOE_EUNSUPPORTED);
    EXPECT(moe_topk(of, 4, 8, 2, o32, of, nullptr) == BITMOE_EHIP);
    EXPECT(moe_dequant_iq2x(x, x, -1, out, 0, nullptr) == BITMOE_EINVAL);
    EXPECT(moe_dequant_iq2x(x, x, 1000, out, 1, nullptr) == BITMOE_EHIP);
    EXPECT(moe_dequant_q2k(fake(2), 10, out, 0, nullptr) == BITMOE_EINVAL);
    EXPECT(moe_pack_iq2x(x, out, 2, 64, 256, nullptr) == BITMOE_EHIP);
    EXPECT(moe_pack_q2k(x, out, 2, 64, 100, nullptr) == BITMOE_EUNSUPPORTED);
    EXPECT(moe_pack_bf16(x, out, 64, 12, nullptr) == BITMOE_EUNSUPPORTED);
    EXPECT(moe_dequant_mxfp4(fake(3), 10, out, 0, nullptr) == BITMOE_EHIP);      // blocks: no alignment
    EXPECT(moe_dequant_mxfp4(x, 10, fake(8), 0, nullptr) == BITMOE_EINVAL);
    EXPECT(moe_dequant_mxfp4(x, 10, out, 2, nullptr) == BITMOE_EINVAL);
    EXPECT(moe_pack_mxfp4(fake(3), out, 2, 64, 256, nullptr) == BITMOE_EHIP);
    EXPECT(moe_pack_mxfp4(x, out, 2, 64, 32, nullptr) == BITMOE_EUNSUPPORTED);
    bitmoe_layer nog = layer(256, 512, 8, 2, false);
    nog.grid = nullptr;                                                        // 2-bit layers need the codebook
    EXPECT(moe_ffn_decode(&nog, x, 1, 4, o32, of, of, ws, 1 << 20, nullptr) == BITMOE_EINVAL);
    nog.format = 7;
    EXPECT(moe_ffn_decode(&nog, x, 1, 4, o32, of, of, ws, 1 << 20, nullptr) == BITMOE_EINVAL);
    EXPECT(moe_set_timing_events(nullptr, nullptr, 5) == BITMOE_EINVAL);
    for (int c = 1; c >= -5; c--) EXPECT(std::strlen(moe_strerror(c)) > 0);
    EXPECT(std::strlen(moe_version()) > 0);
    std::printf(failures ? "abi sanitizer driver: %d check(s) failed\n" : "abi sanitizer driver: ok\n", failures);
    return failures ? 1 : 0;
}
