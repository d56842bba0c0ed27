// hbm_probe.hip - measurement aid, not part of the decode path: a plain
// device-to-device copy of known size.  The benchmark times it to report the
// copy bandwidth this GPU sustains, and hardware-counter runs use its known
// byte count to calibrate the FETCH_SIZE / WRITE_SIZE counters.

#include <hip/hip_runtime.h>

#include <cstddef>

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_copy_probe(const f4 *__restrict__ src,
                                                   f4 *__restrict__ dst, size_t n) {
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

}  // namespace

extern "C" {

// Copies `bytes` (a multiple of 16; both pointers 16-byte aligned device
// memory) from src to dst on `stream`.  Returns 0, or -1 on bad arguments,
// or -6 when the launch fails.
int gdn_probe_copy(const void *src, void *dst, size_t bytes, void *stream) {
    if (!src || !dst || bytes % 16 != 0 || reinterpret_cast<size_t>(src) % 16 != 0 ||
        reinterpret_cast<size_t>(dst) % 16 != 0)
        return -1;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    (void)hipGetLastError();
    k_copy_probe<<<dim3(cus * 4), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const f4 *>(src), static_cast<f4 *>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
