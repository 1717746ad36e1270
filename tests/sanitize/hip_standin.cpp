// A stand-in for the few HIP runtime calls the library's host code makes
// (test infrastructure, host sanitizer builds only): no device exists, so
// device queries fail (the library then assumes 256 compute units) and
// asynchronous copies are plain memcpy between host buffers that play the
// device memory.
#include <cstring>

#include <hip/hip_runtime_api.h>

extern "C" {

hipError_t hipGetDevice(int *device) {
    if (device) *device = 0;
    return hipErrorNoDevice;
}

hipError_t hipDeviceGetAttribute(int *value, hipDeviceAttribute_t, int) {
    if (value) *value = 0;
    return hipErrorNoDevice;
}

hipError_t hipMemcpyAsync(void *dst, const void *src, size_t bytes, hipMemcpyKind, hipStream_t) {
    std::memcpy(dst, src, bytes);
    return hipSuccess;
}

}  // extern "C"
