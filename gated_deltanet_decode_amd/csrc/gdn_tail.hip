// gdn_tail.hip - gdn_layer_tail: conv1d prestate, gated RMSNorm, the
// beta/alpha parameter transforms and the single-launch fused tail.

#include <atomic>
#include <mutex>

#include "gdn_device.hpp"

namespace gdn {
namespace {

// Scratch of gdn_layer_tail_noalloc, for callers that cannot allocate: the
// three-launch tail stages its normalised Q|K|V and step output here instead
// of in a caller's workspace.  Each GPU the library runs on holds its own
// copy until the process ends, and every call on that GPU shares it.  Host
// code never uses this name as an address: noalloc_scratch() returns the
// device address that hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mutex;

// --------------------------------------------------------- tail helpers
// Block-wide sum for a block of NW waves; every thread gets the same bits.
template <int NW>
__device__ __forceinline__ float block_sum(float x, float *red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += red[w];
    return s;
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// beta/alpha parameter transforms (Red Lite dev15a, "Validation boundary":
// named as the stage before the update; the formula is the reading of the
// Gated DeltaNet paper's Mamba-2 style gating):
//   beta = 1 / (1 + exp(-b)),  gate = -exp(a_log) * softplus(a + dt_bias),
// softplus(x) = log(1 + exp(x)), evaluated as x + log1p(exp(-x)) for x > 0.
__device__ __forceinline__ float softplus(float x) {
    return x > 0.0f ? x + log1pf(expf(-x)) : log1pf(expf(x));
}

__device__ __forceinline__ void beta_gate(float b, float a, float a_log, float dt_bias,
                                          float &beta, float &gate) {
    beta = 1.0f / (1.0f + expf(-b));
    gate = -expf(a_log) * softplus(a + dt_bias);
}

// conv-state shift + causal conv1d + SiLU for one 128-channel chunk of one
// sequence; chunks inside the Q and K parts are also L2-normalised (the head
// dim is 128, so a chunk is exactly one head).
template <int K>
__global__ __launch_bounds__(D) void k_prestate(PrestateArgs a) {
    __shared__ float red[D / 64];
    const int n_chunks = a.C / D;
    const int64_t b = blockIdx.x / n_chunks;
    const int chunk = static_cast<int>(blockIdx.x - b * n_chunks);
    const int c = chunk * D + threadIdx.x;
    float *cs = a.conv_state + b * (K - 1) * static_cast<int64_t>(a.C);

    float win[K];
#pragma unroll
    for (int t = 0; t < K - 1; ++t) win[t] = cs[static_cast<int64_t>(t) * a.C + c];
    win[K - 1] = a.x[b * a.C + c];

    const float *w = a.conv_w + static_cast<int64_t>(c) * K;
    float acc = 0.0f;
#pragma unroll
    for (int t = 0; t < K; ++t) acc = fmaf(w[t], win[t], acc);
#pragma unroll
    for (int t = 0; t < K - 1; ++t) cs[static_cast<int64_t>(t) * a.C + c] = win[t + 1];

    float s = silu(acc);
    if (chunk * D < a.n_qk) {        // block-uniform: a Q or K head
        const float ss = block_sum<D / 64>(s * s, red);
        const float nrm = fmaxf(sqrtf(ss), 1e-6f);
        s = s / nrm;
    }
    a.qkv[b * a.C + c] = s;
}

// Gated RMSNorm x SiLU(z) over one group of one row.
constexpr int kNormThreads = kGatedNormThreads;
__global__ __launch_bounds__(kNormThreads) void k_gated_norm(GatedNormArgs a) {
    __shared__ float red[kNormThreads / 64];
    const int groups = a.n / a.group;
    const int64_t row = blockIdx.x / groups;
    const int64_t base = row * a.n + static_cast<int64_t>(blockIdx.x - row * groups) * a.group;
    float ss = 0.0f;
    for (int i = threadIdx.x; i < a.group; i += kNormThreads) {
        const float o = a.o[base + i];
        ss = fmaf(o, o, ss);
    }
    ss = block_sum<kNormThreads / 64>(ss, red);
    const float rms = sqrtf(ss / static_cast<float>(a.group) + a.eps);
    for (int i = threadIdx.x; i < a.group; i += kNormThreads)
        a.y[base + i] = (a.o[base + i] / rms) * a.w[i] * silu(a.z[base + i]);
}

// beta/alpha parameter transforms, one thread per (sequence, value head).
constexpr int kGateThreads = 256;
__global__ __launch_bounds__(kGateThreads) void k_gate_transform(GateArgs a) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kGateThreads + threadIdx.x;
    if (i >= static_cast<int64_t>(a.B) * a.Hv) return;
    const int64_t b = i / a.Hv;
    const int h = static_cast<int>(i - b * a.Hv);
    const float *row = a.ba + b * 2 * a.Hv;
    beta_gate(row[h], row[a.Hv + h], a.a_log[h], a.dt_bias[h], a.beta[i], a.gate[i]);
}


// ------------------------------------------------------ fused layer tail
// The whole recurrent-branch tail for one token in one launch.  One
// workgroup per (sequence b, key head kh) owns every channel that key head's
// value heads need: Q head kh, K head kh and the V channels of the RV value
// heads h = kh + i*Hk.  Owning them outright makes the conv-cache shift
// race-free, and lets the step read Q, K and V from LDS.  The workgroup issues
// the nontemporal loads of its RV x 64 KiB of state first and computes the
// prestate while they are in flight.  Every reduction keeps the order of the
// three-launch path (k_prestate, k_step, k_gated_norm), so both paths give
// the same bits.  With kRaw the lanes also make their heads' beta and gate
// from the raw gate inputs with beta_gate(), as k_gate_transform does.
constexpr int kTailThreads = 256;

template <int RV, int K, bool kRaw>
__global__ __launch_bounds__(kTailThreads) void k_tail_fused(TailFusedArgs a) {
    constexpr int kCh = (2 + RV) * D;               // owned channels
    constexpr int kTiles = RV * kTilesPerHead;      // state tiles of the workgroup
    constexpr int kTilesPerWave = kTiles / (kTailThreads / 64);
    __shared__ alignas(16) float act[kCh];          // Q | K | V_0 .. V_{RV-1}
    __shared__ float core[RV * D];
    __shared__ float red[kTailThreads / 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = lane >> 3;
    const int c = lane & 7;
    const int b = blockIdx.x / a.Hk;
    const int kh = blockIdx.x - b * a.Hk;
    const int nq = a.Hk * D;

    // 1. state loads in flight, with the wave's beta and gate (or, with kRaw,
    //    the raw logits and per-head parameters they are made from).  All
    //    tiles of a wave lie in one value head.
    static_assert(kTilesPerHead % kTilesPerWave == 0, "a wave's tiles must share a head");
    const int hw = kh + (wave * kTilesPerWave / kTilesPerHead) * a.Hk;
    RowSlice r[kTilesPerWave];
    int64_t roff[kTilesPerWave];
#pragma unroll
    for (int j = 0; j < kTilesPerWave; ++j) {
        const int t = wave * kTilesPerWave + j;
        const int row = (t % kTilesPerHead) * kRowsPerTile + grp;
        roff[j] = (static_cast<int64_t>(b) * a.Hv + hw) * (D * D) + row * D;
        load_row<true>(r[j], a.state + roff[j], c);
    }
    float bt = 0.0f, gt = 0.0f, raw_b = 0.0f, raw_a = 0.0f, raw_l = 0.0f, raw_d = 0.0f;
    if constexpr (kRaw) {
        const float *ba = a.ba + static_cast<int64_t>(b) * 2 * a.Hv;
        raw_b = ba[hw];
        raw_a = ba[a.Hv + hw];
        raw_l = a.a_log[hw];
        raw_d = a.dt_bias[hw];
    } else {
        bt = a.beta[static_cast<int64_t>(b) * a.Hv + hw];
        gt = a.gate[static_cast<int64_t>(b) * a.Hv + hw];
    }

    // 2. conv-state shift + conv1d + SiLU on the owned channels; the first
    //    pass holds Q (threads 0..127) and K (threads 128..255), which are
    //    L2-normalised per head with the reduction order of k_prestate.
    float *cs = a.conv_state + static_cast<int64_t>(b) * (K - 1) * a.C;
#pragma unroll
    for (int pass = 0; pass < (kCh + kTailThreads - 1) / kTailThreads; ++pass) {
        const int slot = tid + pass * kTailThreads;
        if (pass > 0 && slot >= kCh) continue;     // only in a partial last pass
        int ch;
        if (slot < D)
            ch = kh * D + slot;
        else if (slot < 2 * D)
            ch = nq + kh * D + (slot - D);
        else
            ch = 2 * nq + (kh + ((slot - 2 * D) / D) * a.Hk) * D + (slot % D);
        float win[K];
#pragma unroll
        for (int t = 0; t < K - 1; ++t) win[t] = cs[static_cast<int64_t>(t) * a.C + ch];
        win[K - 1] = a.x[static_cast<int64_t>(b) * a.C + ch];
        const float *w = a.conv_w + static_cast<int64_t>(ch) * K;
        float acc = 0.0f;
#pragma unroll
        for (int t = 0; t < K; ++t) acc = fmaf(w[t], win[t], acc);
#pragma unroll
        for (int t = 0; t < K - 1; ++t) cs[static_cast<int64_t>(t) * a.C + ch] = win[t + 1];
        float s = silu(acc);
        if (pass == 0) {
            float x2 = s * s;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) x2 += __shfl_xor(x2, off, 64);
            if (lane == 0) red[wave] = x2;
            __syncthreads();
            const int h2 = wave >> 1;              // 0: Q, 1: K
            const float ss = (0.0f + red[2 * h2]) + red[2 * h2 + 1];
            s = s / fmaxf(sqrtf(ss), 1e-6f);
        }
        act[slot] = s;
        if (a.dbg_qkv) a.dbg_qkv[static_cast<int64_t>(b) * a.C + ch] = s;
    }
    if constexpr (kRaw) beta_gate(raw_b, raw_a, raw_l, raw_d, bt, gt);
    const float e = expf(gt);
    __syncthreads();

    // 3. the state step on the preloaded rows; k and q come from LDS
    VecSlice kv, qv;
    load_vec(kv, act + D, c);
    load_vec(qv, act, c);
#pragma unroll
    for (int j = 0; j < kTilesPerWave; ++j) {
        const int t = wave * kTilesPerWave + j;
        const int i = t / kTilesPerHead;
        const int row = (t % kTilesPerHead) * kRowsPerTile + grp;
        const float o = row_token(r[j], kv, qv, e, bt, act[(2 + i) * D + row]);
        store_row<true>(a.state + roff[j], r[j], c);
        if (c == 0) core[i * D + row] = o;
    }
    __syncthreads();

    // 4. gated RMSNorm x SiLU(z), one 128-element group per value head, with
    //    the reduction order of k_gated_norm (128 threads per group); with
    //    RV = 1 the upper 128 threads carry zeros through the barriers.
    {
        const int i = tid / D;                     // value head slot
        const int j = tid - i * D;
        const bool live = tid < RV * D;
        const float o = live ? core[tid] : 0.0f;
        float x2 = fmaf(o, o, 0.0f);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) x2 += __shfl_xor(x2, off, 64);
        if (lane == 0) red[wave] = x2;
        __syncthreads();
        if (live) {
            const float ss = (0.0f + red[2 * i]) + red[2 * i + 1];
            const float rms = sqrtf(ss / static_cast<float>(D) + a.eps);
            const int h = kh + i * a.Hk;
            const int64_t yo = static_cast<int64_t>(b) * a.Hv * D + static_cast<int64_t>(h) * D + j;
            a.y[yo] = (o / rms) * a.norm_w[j] * silu(a.z[yo]);
            if (a.dbg_core) a.dbg_core[yo] = o;
        }
    }
}

}  // namespace

hipError_t noalloc_scratch(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            // with device `dev` current: its own copy of the array
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

bool tail_fused_supported(int32_t Hv, int32_t Hk, int32_t K, int32_t group) {
    const int32_t rv = Hv / Hk;
    return (rv == 1 || rv == 2) && K == 4 && group == D;
}

hipError_t launch_tail_fused(const TailFusedArgs &a, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hk));
    const bool raw = a.ba != nullptr;
    if (a.Hv == a.Hk && a.K == 4) {
        if (raw)
            k_tail_fused<1, 4, true><<<grid, dim3(kTailThreads), 0, s>>>(a);
        else
            k_tail_fused<1, 4, false><<<grid, dim3(kTailThreads), 0, s>>>(a);
    } else if (a.Hv == 2 * a.Hk && a.K == 4) {
        if (raw)
            k_tail_fused<2, 4, true><<<grid, dim3(kTailThreads), 0, s>>>(a);
        else
            k_tail_fused<2, 4, false><<<grid, dim3(kTailThreads), 0, s>>>(a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_prestate(const PrestateArgs &a, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.C / D) * a.B));
    switch (a.K) {
    case 2: k_prestate<2><<<grid, dim3(D), 0, s>>>(a); break;
    case 3: k_prestate<3><<<grid, dim3(D), 0, s>>>(a); break;
    case 4: k_prestate<4><<<grid, dim3(D), 0, s>>>(a); break;
    case 5: k_prestate<5><<<grid, dim3(D), 0, s>>>(a); break;
    case 6: k_prestate<6><<<grid, dim3(D), 0, s>>>(a); break;
    case 7: k_prestate<7><<<grid, dim3(D), 0, s>>>(a); break;
    case 8: k_prestate<8><<<grid, dim3(D), 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gated_norm(const GatedNormArgs &a, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.n / a.group) * a.rows));
    k_gated_norm<<<grid, dim3(kNormThreads), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_gate_transform(const GateArgs &a, hipStream_t s) {
    const int64_t n = static_cast<int64_t>(a.B) * a.Hv;
    const dim3 grid(static_cast<unsigned>((n + kGateThreads - 1) / kGateThreads));
    k_gate_transform<<<grid, dim3(kGateThreads), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace gdn
