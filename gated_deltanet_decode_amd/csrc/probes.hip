// probes.hip - measurement aids, not part of the decode path:
//  - a plain device-to-device copy of known size: the benchmark times it to
//    report the copy bandwidth this GPU sustains, and hardware-counter runs
//    use its known byte count to calibrate the FETCH_SIZE / WRITE_SIZE
//    counters;
//  - an in-place read-modify-write with the staged step kernel's memory
//    pattern and none of its arithmetic: the rate the step's access pattern
//    alone reaches, the practical ceiling for the step kernel;
//  - an in-place read-modify-write with a persistent XCD-aware tile walk
//    (each wave loading and storing its own tile row by row, nontemporal
//    16-byte accesses), the pattern of the pair kernel; the same walk
//    copying between two buffers, reading only, or writing only;
//  - a stream of independent non-packed FP32 FMAs with no memory traffic:
//    the issue rate the VALU sustains at a given number of waves per CU, the
//    practical ceiling for the multi-token kernel;
//  - an empty kernel and the in-place probe with one wave per tile: the
//    floors of a small, latency-bound launch.

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

// The tile walk: a persistent grid of one 8-wave workgroup per CU walks
// 4 KiB tiles (8 rows of 512 B) in grid-stride order; in a tile, lane c of
// row group g reads the float4 chunks 8*i + c (i = 0..3) of row g with
// nontemporal loads, flips the bits in `key` (0: data unchanged) and writes
// them back with nontemporal stores.
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
constexpr int kProbeWaves = 8;

// src == dst: the in-place probe; otherwise a copy with the same walk.  W:
// waves per workgroup (kProbeWaves for the persistent walk; 1 with one
// workgroup per tile, the step kernel's shape for small launches).
template <int W>
__global__ __launch_bounds__(W * 64) void k_inplace_probe(const f4 *src, f4 *dst,
                                                          int64_t n_tiles, unsigned key) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = lane >> 3;
    const int c = lane & 7;
    const int G = gridDim.x;
    const int g = blockIdx.x;
    const int lg = (G % 8 == 0) ? (g % 8) * (G / 8) + g / 8 : g;
    const int64_t stride = static_cast<int64_t>(G) * W;
    for (int64_t u = static_cast<int64_t>(lg) * W + wave; u < n_tiles; u += stride) {
        const int64_t row = u * 256 + grp * 32;    // a tile is 256 float4, a row 32
        f4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __builtin_nontemporal_load(src + row + 8 * i + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u4 b = __builtin_bit_cast(u4, v[i]) ^ key;
            __builtin_nontemporal_store(__builtin_bit_cast(f4, b), dst + row + 8 * i + c);
        }
    }
}

// The staged step kernel's memory pattern without its arithmetic: a
// workgroup of 8 waves takes two consecutive tiles; every thread loads one
// float4 (nontemporal, 1 KiB contiguous per wave instruction) into LDS; after
// a barrier waves 0 and 4 read their tile back in the row layout (lane c of
// row group g: float4 chunks 8*i + c of row g), flip the bits in `key` and
// store the rows with nontemporal stores.
__global__ __launch_bounds__(512) void k_staged_probe(f4 *buf, unsigned key) {
    __shared__ f4 tile[2][256];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = lane >> 3;
    const int c = lane & 7;
    const int mine = wave / 4;
    f4 *T = buf + (static_cast<int64_t>(blockIdx.x) * 2 + mine) * 256;
    tile[mine][(wave % 4) * 64 + lane] = __builtin_nontemporal_load(T + (wave % 4) * 64 + lane);
    __syncthreads();
    if (wave % 4 != 0) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = grp * 32 + 8 * i + c;
        const u4 b = __builtin_bit_cast(u4, tile[mine][q]) ^ key;
        __builtin_nontemporal_store(__builtin_bit_cast(f4, b), T + q);
    }
}

// One direction only, with the same walk, lanes and nontemporal accesses:
// reads every tile and folds its bits into one word per thread, written to
// sink[thread] at the end (so the loads are kept); or writes every tile with
// `key`.  Together with the in-place probe they show what mixing reads and
// writes in one stream costs.
__global__ __launch_bounds__(kProbeWaves * 64) void k_read_probe(const f4 *src, unsigned *sink,
                                                                 int64_t n_tiles) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = lane >> 3;
    const int c = lane & 7;
    const int G = gridDim.x;
    const int g = blockIdx.x;
    const int lg = (G % 8 == 0) ? (g % 8) * (G / 8) + g / 8 : g;
    const int64_t stride = static_cast<int64_t>(G) * kProbeWaves;
    unsigned acc = 0;
    for (int64_t u = static_cast<int64_t>(lg) * kProbeWaves + wave; u < n_tiles; u += stride) {
        const int64_t row = u * 256 + grp * 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u4 b = __builtin_bit_cast(u4, __builtin_nontemporal_load(src + row + 8 * i + c));
            acc ^= b.x ^ b.y ^ b.z ^ b.w;
        }
    }
    sink[static_cast<int64_t>(g) * blockDim.x + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kProbeWaves * 64) void k_write_probe(f4 *dst, int64_t n_tiles,
                                                                  unsigned key) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = lane >> 3;
    const int c = lane & 7;
    const int G = gridDim.x;
    const int g = blockIdx.x;
    const int lg = (G % 8 == 0) ? (g % 8) * (G / 8) + g / 8 : g;
    const int64_t stride = static_cast<int64_t>(G) * kProbeWaves;
    const u4 b = {key, key, key, key};
    for (int64_t u = static_cast<int64_t>(lg) * kProbeWaves + wave; u < n_tiles; u += stride) {
        const int64_t row = u * 256 + grp * 32;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_nontemporal_store(__builtin_bit_cast(f4, b), dst + row + 8 * i + c);
    }
}

// Does nothing: the cost of a launch of a given shape.
__global__ void k_empty_probe() {}

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
    k_inplace_probe<kProbeWaves>
        <<<dim3(grid), dim3(kProbeWaves * 64), 0, static_cast<hipStream_t>(stream)>>>(
            static_cast<const f4 *>(buf), static_cast<f4 *>(buf), tiles, key);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Copies `bytes` (a multiple of 4096; both pointers 16-byte aligned device
// memory, not overlapping) from src to dst with the in-place probe's walk.
// Returns 0, -1 on bad arguments, -6 when the launch fails.
int gdn_probe_copy_nt(const void *src, void *dst, size_t bytes, void *stream) {
    if (!src || !dst || bytes == 0 || bytes % 4096 != 0 ||
        reinterpret_cast<size_t>(src) % 16 != 0 || reinterpret_cast<size_t>(dst) % 16 != 0)
        return -1;
    const int64_t tiles = static_cast<int64_t>(bytes / 4096);
    const int64_t need = (tiles + kProbeWaves - 1) / kProbeWaves;
    const int cus = device_cus();
    const int grid = static_cast<int>(need < cus ? need : cus);
    (void)hipGetLastError();
    k_inplace_probe<kProbeWaves>
        <<<dim3(grid), dim3(kProbeWaves * 64), 0, static_cast<hipStream_t>(stream)>>>(
            static_cast<const f4 *>(src), static_cast<f4 *>(dst), tiles, 0u);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Reads `bytes` (a multiple of 4096, 16-byte aligned device memory) with
// the in-place probe's walk; each thread writes one 32-bit word to `sink`,
// which must hold sink_bytes >= 4 x (one 512-thread workgroup per compute
// unit, at most one per 8 tiles) bytes.  Returns 0, -1 on bad arguments, -6
// when the launch fails.
int gdn_probe_read(const void *buf, size_t bytes, void *sink, size_t sink_bytes, void *stream) {
    if (!buf || !sink || bytes == 0 || bytes % 4096 != 0 ||
        reinterpret_cast<size_t>(buf) % 16 != 0 || reinterpret_cast<size_t>(sink) % 4 != 0)
        return -1;
    const int64_t tiles = static_cast<int64_t>(bytes / 4096);
    const int64_t need = (tiles + kProbeWaves - 1) / kProbeWaves;
    const int cus = device_cus();
    const int grid = static_cast<int>(need < cus ? need : cus);
    if (sink_bytes < static_cast<size_t>(grid) * kProbeWaves * 64 * sizeof(unsigned)) return -1;
    (void)hipGetLastError();
    k_read_probe<<<dim3(grid), dim3(kProbeWaves * 64), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const f4 *>(buf), static_cast<unsigned *>(sink), tiles);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Writes `bytes` (a multiple of 4096, 16-byte aligned device memory) with
// the in-place probe's walk, every 32-bit word set to `key`.  Returns 0, -1
// on bad arguments, -6 when the launch fails.
int gdn_probe_write(void *buf, size_t bytes, unsigned key, void *stream) {
    if (!buf || bytes == 0 || bytes % 4096 != 0 || reinterpret_cast<size_t>(buf) % 16 != 0)
        return -1;
    const int64_t tiles = static_cast<int64_t>(bytes / 4096);
    const int64_t need = (tiles + kProbeWaves - 1) / kProbeWaves;
    const int cus = device_cus();
    const int grid = static_cast<int>(need < cus ? need : cus);
    (void)hipGetLastError();
    k_write_probe<<<dim3(grid), dim3(kProbeWaves * 64), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<f4 *>(buf), tiles, key);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Reads and rewrites `bytes` (a multiple of 8192, at most 2^35, 16-byte
// aligned device memory) in place with the staged step kernel's pattern,
// XOR-ing every 32-bit word with `key`.  Returns 0, -1 on bad arguments, -6
// when the launch fails.
int gdn_probe_inplace_staged(void *buf, size_t bytes, unsigned key, void *stream) {
    if (!buf || bytes == 0 || bytes % 8192 != 0 || bytes > (size_t(1) << 35) ||
        reinterpret_cast<size_t>(buf) % 16 != 0)
        return -1;
    (void)hipGetLastError();
    k_staged_probe<<<dim3(static_cast<unsigned>(bytes / 8192)), dim3(512), 0,
                     static_cast<hipStream_t>(stream)>>>(static_cast<f4 *>(buf), key);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// The in-place probe with one one-wave workgroup per 4 KiB tile, the shape
// the step kernel takes for small launches: `bytes` a multiple of 4096, at
// most 2^36 (2^24 tiles).  Returns 0, -1 on bad arguments, -6 when the
// launch fails.
int gdn_probe_inplace_small(void *buf, size_t bytes, unsigned key, void *stream) {
    if (!buf || bytes == 0 || bytes % 4096 != 0 || bytes > (size_t(1) << 36) ||
        reinterpret_cast<size_t>(buf) % 16 != 0)
        return -1;
    const int64_t tiles = static_cast<int64_t>(bytes / 4096);
    (void)hipGetLastError();
    k_inplace_probe<1><<<dim3(static_cast<unsigned>(tiles)), dim3(64), 0,
                         static_cast<hipStream_t>(stream)>>>(
        static_cast<const f4 *>(buf), static_cast<f4 *>(buf), tiles, key);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Launches an empty kernel of `workgroups` x `threads` threads (threads a
// multiple of 64, at most 1024).  Returns 0, -1 on bad arguments, -6 when
// the launch fails.
int gdn_probe_empty(int workgroups, int threads, void *stream) {
    if (workgroups < 1 || threads < 64 || threads > 1024 || threads % 64 != 0) return -1;
    (void)hipGetLastError();
    k_empty_probe<<<dim3(workgroups), dim3(threads), 0, static_cast<hipStream_t>(stream)>>>();
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
