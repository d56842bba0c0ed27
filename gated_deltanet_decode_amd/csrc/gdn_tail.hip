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
// The whole recurrent-branch tail for NP consecutive positions in one launch
// (NP = 1: one token; NP = 2: the speculative pair, docs.rs "Module
// linear_core", gdn_pair: position 1 commits ring and state, position 2
// moves them together into the tentative buffers).  One workgroup per
// (sequence b, key head kh) owns every channel that key head's value heads
// need: Q head kh, K head kh and the V channels of the RV value heads
// h = kh + i*Hk.  Owning them outright makes the conv-ring update race-free
// and lets the step read Q, K and V from LDS.
//
// Order of work, chosen by measurement on MI355X (B = 32, states streamed
// from HBM): each wave issues the nontemporal loads of its state tiles, then
// every conv input of the workgroup's channels at once (the K-1 ring slots,
// the NP new inputs and the K taps of both channel passes), so conv, SiLU
// and L2 run as soon as the wave's loads are back and no further memory
// round trip sits between the state loads and the step.  Fetching the V
// channels' inputs after the Q/K barrier measured 6 % slower, fetching the
// conv inputs ahead of the state 5 % slower, and 8 waves of 4 tiles 4 %
// slower.
//
// Every reduction keeps the order of the three-launch path (k_prestate,
// gdn_step's kernel, k_gated_norm), so both paths give the same bits, and position 2
// of a pair gives the bits of a one-position call on the ring and state
// that position 1 committed.  With kRaw the lanes also make their heads'
// beta and gate from the raw gate inputs with beta_gate(), as
// k_gate_transform does.
constexpr int kTailThreads = 256;

// Channel of owned slot `slot` of key head kh: Q head kh, K head kh, then
// the V channels of value heads kh, kh + Hk, ...  Slots beyond the owned
// ones (a partial last pass) map to a Q channel, so their loads stay in
// bounds; nothing computed from them is stored.
template <int RV>
__device__ __forceinline__ int owned_channel(int slot, int kh, int Hk) {
    const int nq = Hk * D;
    if (slot < D) return kh * D + slot;
    if (slot < 2 * D) return nq + kh * D + (slot - D);
    if (slot < (2 + RV) * D) return 2 * nq + (kh + ((slot - 2 * D) / D) * Hk) * D + (slot % D);
    return kh * D + (slot % D);
}

template <int RV, int K, bool kRaw, int NP>
__global__ __launch_bounds__(kTailThreads) void k_tail(TailFusedArgs a) {
    constexpr int kW = kTailThreads / 64;
    constexpr int kCh = (2 + RV) * D;               // owned channels
    constexpr int kPasses = (kCh + kTailThreads - 1) / kTailThreads;
    constexpr int kTiles = RV * kTilesPerHead;      // state tiles of the workgroup
    constexpr int kTPW = kTiles / kW;
    constexpr int kWin = K - 1 + NP;                // ring slots, then the NP inputs
    __shared__ alignas(16) float act[NP][kCh];      // Q | K | V_0 .. V_{RV-1} per position
    __shared__ float core[NP][RV * D];
    __shared__ float red[NP][kW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = lane >> 3;
    const int c = lane & 7;
    const int b = blockIdx.x / a.Hk;
    const int kh = blockIdx.x - b * a.Hk;

    // 1. state loads in flight, with each position's beta and gate (or, with
    //    kRaw, the raw logits and per-head parameters they are made from).
    //    All tiles of a wave lie in one value head.
    static_assert(kTilesPerHead % kTPW == 0, "a wave's tiles must share a head");
    static_assert(NP == 1 || !kRaw, "the pair takes beta and gate as given");
    const int hw = kh + (wave * kTPW / kTilesPerHead) * a.Hk;
    RowSlice r[kTPW];
    int64_t roff[kTPW];
#pragma unroll
    for (int j = 0; j < kTPW; ++j) {
        const int t = wave * kTPW + j;
        const int row = (t % kTilesPerHead) * kRowsPerTile + grp;
        roff[j] = (static_cast<int64_t>(b) * a.Hv + hw) * (D * D) + row * D;
        load_row<true>(r[j], a.state + roff[j], c);
    }
    float bt[NP], gt[NP];
    float raw_b = 0.0f, raw_a = 0.0f, raw_l = 0.0f, raw_d = 0.0f;
    if constexpr (kRaw) {
        const float *ba = a.ba + static_cast<int64_t>(b) * 2 * a.Hv;
        raw_b = ba[hw];
        raw_a = ba[a.Hv + hw];
        raw_l = a.a_log[hw];
        raw_d = a.dt_bias[hw];
    } else {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int64_t bp = static_cast<int64_t>(b) * NP + p;
            bt[p] = a.beta[bp * a.Hv + hw];
            gt[p] = a.gate[bp * a.Hv + hw];
        }
    }

    // 2. every conv input of the owned channels
    float *cs = a.conv_state + static_cast<int64_t>(b) * (K - 1) * a.C;
    float win[kPasses][kWin], wt[kPasses][K];
    int chs[kPasses];
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
        const int ch = owned_channel<RV>(tid + pass * kTailThreads, kh, a.Hk);
        chs[pass] = ch;
#pragma unroll
        for (int t = 0; t < K - 1; ++t) win[pass][t] = cs[static_cast<int64_t>(t) * a.C + ch];
#pragma unroll
        for (int p = 0; p < NP; ++p)
            win[pass][K - 1 + p] = a.x[(static_cast<int64_t>(b) * NP + p) * a.C + ch];
        const float *w = a.conv_w + static_cast<int64_t>(ch) * K;
#pragma unroll
        for (int t = 0; t < K; ++t) wt[pass][t] = w[t];
    }

    // 3. conv1d over each position's window (oldest first) + SiLU; the ring
    //    after position 1 goes to conv_state and, for a pair, the ring after
    //    position 2 to conv_state_next.  The first pass holds Q (threads
    //    0..127) and K (threads 128..255), which are L2-normalised per head
    //    with the reduction order of k_prestate.
    float *csn = NP == 2 ? a.conv_state_next + static_cast<int64_t>(b) * (K - 1) * a.C : nullptr;
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
        const int slot = tid + pass * kTailThreads;
        const bool live = slot < kCh;
        const int ch = chs[pass];
        float sv[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            float acc = 0.0f;
#pragma unroll
            for (int t = 0; t < K; ++t) acc = fmaf(wt[pass][t], win[pass][p + t], acc);
            sv[p] = silu(acc);
        }
        if (live) {
#pragma unroll
            for (int t = 0; t < K - 1; ++t)
                cs[static_cast<int64_t>(t) * a.C + ch] = win[pass][t + 1];
            if constexpr (NP == 2) {
#pragma unroll
                for (int t = 0; t < K - 1; ++t)
                    csn[static_cast<int64_t>(t) * a.C + ch] = win[pass][t + 2];
            }
        }
        if (pass == 0) {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                float x2 = sv[p] * sv[p];
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) x2 += __shfl_xor(x2, off, 64);
                if (lane == 0) red[p][wave] = x2;
            }
            __syncthreads();
            const int h2 = wave >> 1;              // 0: Q, 1: K
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const float ss = (0.0f + red[p][2 * h2]) + red[p][2 * h2 + 1];
                sv[p] = sv[p] / fmaxf(sqrtf(ss), 1e-6f);
            }
        }
        if (live) {
#pragma unroll
            for (int p = 0; p < NP; ++p) act[p][slot] = sv[p];
            if (NP == 1 && a.dbg_qkv) a.dbg_qkv[static_cast<int64_t>(b) * a.C + ch] = sv[0];
        }
    }
    if constexpr (kRaw) beta_gate(raw_b, raw_a, raw_l, raw_d, bt[0], gt[0]);
    float e[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) e[p] = expf(gt[p]);
    __syncthreads();

    // 4. the state step on the preloaded rows; k and q come from LDS.  All of
    //    the wave's rows take position 1 and go back to `state`; a pair's
    //    rows then take position 2 and go to `state_next` (2 % faster at
    //    B = 32 than both positions tile by tile; same bits).
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        VecSlice kv, qv;
        load_vec(kv, act[p] + D, c);
        load_vec(qv, act[p], c);
        float *dst = p == 0 ? a.state : a.state_next;
#pragma unroll
        for (int j = 0; j < kTPW; ++j) {
            const int t = wave * kTPW + j;
            const int i = t / kTilesPerHead;
            const int row = (t % kTilesPerHead) * kRowsPerTile + grp;
            const float o = row_token(r[j], kv, qv, e[p], bt[p], act[p][(2 + i) * D + row]);
            store_row<true>(dst + roff[j], r[j], c);
            if (c == 0) core[p][i * D + row] = o;
        }
    }
    __syncthreads();

    // 5. gated RMSNorm x SiLU(z), one 128-element group per value head and
    //    position, with the reduction order of k_gated_norm (128 threads per
    //    group); with RV = 1 the upper 128 threads carry zeros through the
    //    barrier.
    {
        const int i = tid / D;                     // value head slot
        const int j = tid - i * D;
        const bool live = tid < RV * D;
        float o[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            o[p] = live ? core[p][tid] : 0.0f;
            float x2 = fmaf(o[p], o[p], 0.0f);
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) x2 += __shfl_xor(x2, off, 64);
            if (lane == 0) red[p][wave] = x2;
        }
        __syncthreads();
        if (live) {
            const int h = kh + i * a.Hk;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const float ss = (0.0f + red[p][2 * i]) + red[p][2 * i + 1];
                const float rms = sqrtf(ss / static_cast<float>(D) + a.eps);
                const int64_t yo = (static_cast<int64_t>(b) * NP + p) * a.Hv * D +
                                   static_cast<int64_t>(h) * D + j;
                a.y[yo] = (o[p] / rms) * a.norm_w[j] * silu(a.z[yo]);
                if (NP == 1 && a.dbg_core) a.dbg_core[yo] = o[p];
            }
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

hipError_t launch_tail_fused(const TailFusedArgs &a, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hk));
    const bool raw = a.ba != nullptr;
    if (a.Hv == a.Hk && a.K == 4) {
        if (raw)
            k_tail<1, 4, true, 1><<<grid, dim3(kTailThreads), 0, s>>>(a);
        else
            k_tail<1, 4, false, 1><<<grid, dim3(kTailThreads), 0, s>>>(a);
    } else if (a.Hv == 2 * a.Hk && a.K == 4) {
        if (raw)
            k_tail<2, 4, true, 1><<<grid, dim3(kTailThreads), 0, s>>>(a);
        else
            k_tail<2, 4, false, 1><<<grid, dim3(kTailThreads), 0, s>>>(a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_tail_pair(const TailFusedArgs &a, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hk));
    if (a.ba != nullptr || !a.state_next || !a.conv_state_next) return hipErrorInvalidValue;
    if (a.Hv == a.Hk && a.K == 4)
        k_tail<1, 4, false, 2><<<grid, dim3(kTailThreads), 0, s>>>(a);
    else if (a.Hv == 2 * a.Hk && a.K == 4)
        k_tail<2, 4, false, 2><<<grid, dim3(kTailThreads), 0, s>>>(a);
    else
        return hipErrorInvalidValue;
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
