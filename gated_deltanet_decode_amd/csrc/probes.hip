// probes.hip - measurement aids, not part of the decode path:
//  - a plain device-to-device copy of known size: the benchmark times it to
//    report the copy bandwidth this GPU sustains, and hardware-counter runs
//    use its known byte count to calibrate the FETCH_SIZE / WRITE_SIZE
//    counters;
//  - an in-place read-modify-write with the state step's memory pattern and
//    none of its arithmetic: the rate the step's access pattern alone
//    reaches, the practical ceiling for the step kernel;
//  - a stream of independent non-packed FP32 FMAs with no memory traffic:
//    the issue rate the VALU sustains at a given number of waves per CU, the
//    practical ceiling for the multi-token kernel.

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

// The gdn_step kernel's memory pattern without its arithmetic: a persistent
// grid of one 8-wave workgroup per CU walks 4 KiB tiles (8 rows of 512 B) in
// grid-stride order; in a tile, lane c of row group g reads the float4 chunks
// 8*i + c (i = 0..3) of row g with nontemporal loads, flips the bits in `key`
// (0: data unchanged) and writes them back with nontemporal stores.
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
constexpr int kProbeWaves = 8;

__global__ __launch_bounds__(kProbeWaves * 64) void k_inplace_probe(f4 *buf, int64_t n_tiles,
                                                                    unsigned key) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = lane >> 3;
    const int c = lane & 7;
    const int G = gridDim.x;
    const int g = blockIdx.x;
    const int lg = (G % 8 == 0) ? (g % 8) * (G / 8) + g / 8 : g;
    const int64_t stride = static_cast<int64_t>(G) * kProbeWaves;
    for (int64_t u = static_cast<int64_t>(lg) * kProbeWaves + wave; u < n_tiles; u += stride) {
        f4 *row = buf + u * 256 + grp * 32;        // a tile is 256 float4, a row 32
        f4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __builtin_nontemporal_load(row + 8 * i + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u4 b = __builtin_bit_cast(u4, v[i]) ^ key;
            __builtin_nontemporal_store(__builtin_bit_cast(f4, b), row + 8 * i + c);
        }
    }
}


// kFmaChains independent fmaf chains per lane, iterated `iters` times; one
// float per thread is stored at the end so nothing is optimised away.  Built,
// like every kernel here, without packed FP32 instructions: each fmaf is one
// v_fmac_f32 (wave64) instruction.
constexpr int kFmaChains = 16;

__global__ void k_fma_probe(float *out, int iters, float x, float y) {
    float acc[kFmaChains];
#pragma unroll
    for (int i = 0; i < kFmaChains; ++i) acc[i] = threadIdx.x * 1e-3f + i;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kFmaChains; ++i) acc[i] = fmaf(acc[i], x, y);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kFmaChains; ++i) s += acc[i];
    out[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

int device_cus() {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    return cus > 0 ? cus : 256;
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
    const int cus = device_cus();
    (void)hipGetLastError();
    k_copy_probe<<<dim3(cus * 4), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const f4 *>(src), static_cast<f4 *>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Reads and rewrites `bytes` (a multiple of 4096; 16-byte aligned device
// memory) in place, XOR-ing every 32-bit word with `key` (0 leaves the data
// unchanged), on `stream`.  Returns 0, -1 on bad arguments, -6 when the
// launch fails.
int gdn_probe_inplace(void *buf, size_t bytes, unsigned key, void *stream) {
    if (!buf || bytes == 0 || bytes % 4096 != 0 || reinterpret_cast<size_t>(buf) % 16 != 0)
        return -1;
    const int64_t tiles = static_cast<int64_t>(bytes / 4096);
    const int64_t need = (tiles + kProbeWaves - 1) / kProbeWaves;
    const int cus = device_cus();
    const int grid = static_cast<int>(need < cus ? need : cus);
    (void)hipGetLastError();
    k_inplace_probe<<<dim3(grid), dim3(kProbeWaves * 64), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<f4 *>(buf), tiles, key);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Runs `workgroups` x `threads` threads (threads a multiple of 64, at most
// 1024), each doing iters x 16 FP32 FMAs, and writes one float per thread to
// `out` (device memory holding at least workgroups x threads floats) on
// `stream`.  Returns 0, -1 on bad arguments, -6 when the launch fails.
int gdn_probe_fma(float *out, size_t out_floats, int workgroups, int threads, int iters,
                  void *stream) {
    if (!out || workgroups < 1 || threads < 64 || threads > 1024 || threads % 64 != 0 ||
        iters < 1 || out_floats < static_cast<size_t>(workgroups) * static_cast<size_t>(threads))
        return -1;
    (void)hipGetLastError();
    k_fma_probe<<<dim3(workgroups), dim3(threads), 0, static_cast<hipStream_t>(stream)>>>(
        out, iters, 0.999f, 1e-3f);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
