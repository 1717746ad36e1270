// moe_forward_decode_noalloc: the decode step of moe_forward_decode with its
// scratch in a fixed device array of this library instead of a caller
// workspace, for callers that cannot allocate device memory.
//
// The array is a file-scope __device__ variable: each device the library
// runs on holds its own copy from module load until the process ends.  Host
// code never uses the symbol's name as an address (on the host it only
// stands in for the symbol); the device address is looked up once per device
// with hipGetSymbolAddress and kept.  The call never forks onto the
// library's side stream, so it creates no stream and allocates nothing.
// Every call on one device shares that device's array: calls that overlap
// on one device (different streams, several threads) race.  Nothing in the
// array has to start at zero: the decode launches clear their counters
// themselves, as they do in a caller's workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "host.h"

namespace {

constexpr size_t kScratchBytes = BITMOE_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// The device address of `scratch` on the current device, looked up at the
// first call on that device (nullptr if the lookup fails).
void *scratch_on_current_device() {
    static std::mutex mu;
    static void *addr[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        addr[dev] = p;
    }
    return addr[dev];
}

}  // namespace

extern "C" int moe_forward_decode_noalloc(const bitmoe_layer *L, const void *x, int x_dtype, int T, int32_t *ids,
                                          float *w, float *y, void *stream) {
    size_t need = 0;
    int rc = bm_host::forward_decode_check(L, x, x_dtype, T, ids, w, y, &need);
    if (rc || T == 0) return rc;
    if (need > kScratchBytes) return BITMOE_ESCRATCH;
    void *ws = scratch_on_current_device();
    if (!ws) return BITMOE_EHIP;
    return bm_host::forward_decode(L, x, x_dtype, T, ids, w, y, ws, kScratchBytes, stream, false);
}
