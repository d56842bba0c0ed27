// gdn_kernels.hip - gfx950 (CDNA4) kernels of the Gated DeltaNet decode path.
//
// The per-token update (Red Lite dev15c, "Pinned llama.cpp semantics"):
//   M *= exp(gate); sk = M k; delta = (v - sk) beta; M += delta k^T;
//   out = M q / sqrt(128)     on the transposed state M[j][i] = S[i][j].
//
// Work decomposition.  Row j of a head's state depends only on that row,
// on the head's k and q, and on v[j], beta and gate: rows never exchange
// data, not even across tokens.  Every kernel here therefore gives one state
// row (128 floats, 512 contiguous bytes) to a quad of four lanes:
//   lane c (0..3) of the quad owns the float4 chunks 4*i + c, i = 0..7,
//   i.e. 32 of the 128 columns, interleaved so that one vector-memory
//   instruction of the quad covers 64 contiguous bytes of the row.
// A wave64 therefore works on 16 rows at a time (a "tile", 8 KiB of state).
// The two row dot products (M k and M q) are a 32-term FMA chain per lane
// followed by a two-step quad reduction over DPP quad_perm; the quad then
// holds bitwise-identical sums in all four lanes, so delta is identical in
// every lane that applies it.
//
// All kernels share row_token(), so a row's arithmetic is the same in the
// single-step kernel, the multi-token kernel and the tail: a T-token gdn_seq
// is bitwise equal to T gdn_step calls.
//
// No MFMA: the update is a sequence of rank-1 updates and matrix-vector
// products (one multiply-add per state element per operation), which is
// memory-bound in the one-token case and VALU-bound when the state is held
// on chip.

#include <hip/hip_runtime.h>

#include "gdn_launch.hpp"

namespace gdn {
namespace {

constexpr int D = kHeadDim;            // 128
constexpr int kLanesPerRow = 4;        // a quad owns a row
constexpr int kF4PerLane = D / 4 / kLanesPerRow;  // 8 float4 = 32 floats per lane
constexpr int kRowsPerTile = 64 / kLanesPerRow;    // 16 rows per wave
// 1/sqrt(128) rounded to binary32; the output is scaled by it.
constexpr float kInvSqrtD = 0.08838834764831845f;

// ----------------------------------------------------------------- helpers
// DPP move within a quad; CTRL is a quad_perm selector.
template <int CTRL>
__device__ __forceinline__ float dpp_quad(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the 4 lanes of a quad; every lane of the quad gets the same bits.
__device__ __forceinline__ float quad_sum(float x) {
    x = x + dpp_quad<0xB1>(x);  // quad_perm [1,0,3,2]: partner lane c^1
    x = x + dpp_quad<0x4E>(x);  // quad_perm [2,3,0,1]: partner lane c^2
    return x;
}

struct RowSlice {   // the 32 state elements of one row that this lane owns
    float4 m[kF4PerLane];
};
struct VecSlice {   // the matching 32 entries of k or q
    float4 x[kF4PerLane];
};

__device__ __forceinline__ void load_row(RowSlice &r, const float *row, int c) {
    const float4 *p = reinterpret_cast<const float4 *>(row);
#pragma unroll
    for (int i = 0; i < kF4PerLane; ++i) r.m[i] = p[4 * i + c];
}

__device__ __forceinline__ void store_row(float *row, const RowSlice &r, int c) {
    float4 *p = reinterpret_cast<float4 *>(row);
#pragma unroll
    for (int i = 0; i < kF4PerLane; ++i) p[4 * i + c] = r.m[i];
}

__device__ __forceinline__ void load_vec(VecSlice &v, const float *src, int c) {
    const float4 *p = reinterpret_cast<const float4 *>(src);
#pragma unroll
    for (int i = 0; i < kF4PerLane; ++i) v.x[i] = p[4 * i + c];
}

// This lane's partial of dot(row, w): a sequential FMA chain over its 32 columns.
__device__ __forceinline__ float dot_part(const RowSlice &r, const VecSlice &w) {
    float p = 0.0f;
#pragma unroll
    for (int i = 0; i < kF4PerLane; ++i) {
        p = fmaf(r.m[i].x, w.x[i].x, p);
        p = fmaf(r.m[i].y, w.x[i].y, p);
        p = fmaf(r.m[i].z, w.x[i].z, p);
        p = fmaf(r.m[i].w, w.x[i].w, p);
    }
    return p;
}

// One token on one state row j (steps 1-5), in the page's order.
// Returns out[j].
__device__ __forceinline__ float row_token(RowSlice &r, const VecSlice &k, const VecSlice &q,
                                           float e, float beta, float vj) {
#pragma unroll
    for (int i = 0; i < kF4PerLane; ++i) {           // 1. decay
        r.m[i].x *= e;
        r.m[i].y *= e;
        r.m[i].z *= e;
        r.m[i].w *= e;
    }
    const float sk = quad_sum(dot_part(r, k));        // 2. sk = M[j] . k
    const float d = (vj - sk) * beta;                 // 3. delta
#pragma unroll
    for (int i = 0; i < kF4PerLane; ++i) {           // 4. rank-1 update
        r.m[i].x = fmaf(d, k.x[i].x, r.m[i].x);
        r.m[i].y = fmaf(d, k.x[i].y, r.m[i].y);
        r.m[i].z = fmaf(d, k.x[i].z, r.m[i].z);
        r.m[i].w = fmaf(d, k.x[i].w, r.m[i].w);
    }
    return quad_sum(dot_part(r, q)) * kInvSqrtD;      // 5. output, updated state
}

// ------------------------------------------------------------- gdn_step
// One workgroup = kWaves waves x kTiles tiles x 16 rows.  With kTiles = 2 a
// workgroup is exactly one head (128 rows, 64 KiB of state): all 16 state
// loads of a lane are issued before any arithmetic, so a workgroup keeps
// 64 KiB in flight.
constexpr int kStepWaves = 4;
constexpr int kStepTiles = 2;
constexpr int kStepRowsPerWG = kStepWaves * kStepTiles * kRowsPerTile;  // 128
static_assert(kStepRowsPerWG == D, "one head per workgroup");

__global__ __launch_bounds__(kStepWaves * 64) void k_step(StepArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int quad = lane >> 2;
    const int c = lane & 3;

    // head = b * Hv + h; the host guarantees B * Hv fits in 31 bits
    const unsigned hd = blockIdx.x;
    const unsigned bu = hd / static_cast<unsigned>(a.Hv);
    const int h = static_cast<int>(hd - bu * static_cast<unsigned>(a.Hv));
    const int kh = h % a.Hk;                      // key-head broadcast
    const int64_t head = hd;
    const int64_t b = bu;

    float *M = a.state + head * (D * D);
    int rows[kStepTiles];
    RowSlice r[kStepTiles];
#pragma unroll
    for (int t = 0; t < kStepTiles; ++t) {
        rows[t] = (wave * kStepTiles + t) * kRowsPerTile + quad;
        load_row(r[t], M + rows[t] * D, c);
    }

    VecSlice kv, qv;
    load_vec(kv, a.k + b * a.qk_bstride + kh * D, c);
    load_vec(qv, a.q + b * a.qk_bstride + kh * D, c);
    const float e = expf(a.gate[head]);
    const float bt = a.beta[head];
    const float *vh = a.v + b * a.v_bstride + static_cast<int64_t>(h) * D;
    float vj[kStepTiles];
#pragma unroll
    for (int t = 0; t < kStepTiles; ++t) vj[t] = vh[rows[t]];

    float *out = a.out + head * D;
#pragma unroll
    for (int t = 0; t < kStepTiles; ++t) {
        const float o = row_token(r[t], kv, qv, e, bt, vj[t]);
        store_row(M + rows[t] * D, r[t], c);
        if (c == 0) out[rows[t]] = o;
    }
}

// -------------------------------------------------------------- gdn_seq
// One workgroup per (sequence, value head): 8 waves x one 16-row tile each,
// so the whole 64 KiB head state lives in VGPRs (32 floats per lane) for all
// T tokens and is read and written once per call.  The per-token inputs
// (k, q, v, gate, beta: 1.5 KiB per token) are staged through LDS in chunks
// of kChunk tokens, double-buffered: the global loads of chunk c+1 are issued
// before chunk c is computed and written to LDS after it, so their latency
// hides behind kChunk tokens of arithmetic and there is one barrier per chunk.
constexpr int kSeqWaves = D / kRowsPerTile;   // 8
constexpr int kSeqThreads = kSeqWaves * 64;   // 512
constexpr int kChunk = 16;

struct alignas(16) TokenLds {
    float k[D];
    float q[D];
    float v[D];
    float gate;
    float beta;
    float pad[2];
};
static_assert(sizeof(TokenLds) % 16 == 0, "float4 aligned token slots");

// float4 loads needed per token: k (32) + q (32) + v (32)
constexpr int kTokF4 = 3 * D / 4;
constexpr int kChunkF4 = kChunk * kTokF4;                    // 1536
constexpr int kF4PerThread = (kChunkF4 + kSeqThreads - 1) / kSeqThreads;  // 3
static_assert(kChunkF4 % kSeqThreads == 0, "even staging split");

struct ChunkRegs {
    float4 f[kF4PerThread];
    float s;   // gate or beta of one token (threads 0 .. 2*kChunk-1)
};

__device__ __forceinline__ void seq_fetch(ChunkRegs &cr, const SeqArgs &a, int64_t b, int h,
                                          int kh, int t0, int tid) {
#pragma unroll
    for (int j = 0; j < kF4PerThread; ++j) {
        const int e = tid + j * kSeqThreads;
        const int tt = e / kTokF4;
        const int w = e - tt * kTokF4;
        const int t = t0 + tt;
        float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < a.T) {
            const int64_t bt = b * a.T + t;
            const float *src;
            if (w < 32)
                src = a.k + (bt * a.Hk + kh) * D + 4 * w;
            else if (w < 64)
                src = a.q + (bt * a.Hk + kh) * D + 4 * (w - 32);
            else
                src = a.v + (bt * a.Hv + h) * D + 4 * (w - 64);
            val = *reinterpret_cast<const float4 *>(src);
        }
        cr.f[j] = val;
    }
    cr.s = 0.0f;
    if (tid < 2 * kChunk) {
        const int tt = tid < kChunk ? tid : tid - kChunk;
        const int t = t0 + tt;
        if (t < a.T) {
            const int64_t idx = (b * a.T + t) * a.Hv + h;
            cr.s = tid < kChunk ? a.gate[idx] : a.beta[idx];
        }
    }
}

__device__ __forceinline__ void seq_stage(TokenLds *buf, const ChunkRegs &cr, int tid) {
#pragma unroll
    for (int j = 0; j < kF4PerThread; ++j) {
        const int e = tid + j * kSeqThreads;
        const int tt = e / kTokF4;
        const int w = e - tt * kTokF4;
        float *dst = w < 32 ? buf[tt].k + 4 * w
                   : w < 64 ? buf[tt].q + 4 * (w - 32)
                            : buf[tt].v + 4 * (w - 64);
        *reinterpret_cast<float4 *>(dst) = cr.f[j];
    }
    if (tid < kChunk)
        buf[tid].gate = cr.s;
    else if (tid < 2 * kChunk)
        buf[tid - kChunk].beta = cr.s;
}

__global__ __launch_bounds__(kSeqThreads) void k_seq(SeqArgs a) {
    __shared__ TokenLds lds[2][kChunk];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int quad = lane >> 2;
    const int c = lane & 3;

    const unsigned hd = blockIdx.x;               // b * Hv + h
    const unsigned bu = hd / static_cast<unsigned>(a.Hv);
    const int h = static_cast<int>(hd - bu * static_cast<unsigned>(a.Hv));
    const int kh = h % a.Hk;
    const int64_t head = hd;
    const int64_t b = bu;
    const int row = wave * kRowsPerTile + quad;

    float *Mrow = a.state + head * (D * D) + row * D;
    RowSlice r;
    load_row(r, Mrow, c);

    ChunkRegs cr;
    seq_fetch(cr, a, b, h, kh, 0, tid);
    seq_stage(lds[0], cr, tid);
    __syncthreads();

    const int n_chunks = (a.T + kChunk - 1) / kChunk;
    for (int ch = 0; ch < n_chunks; ++ch) {
        const bool more = ch + 1 < n_chunks;
        if (more) seq_fetch(cr, a, b, h, kh, (ch + 1) * kChunk, tid);

        const TokenLds *buf = lds[ch & 1];
        const int t0 = ch * kChunk;
        const int nt = min(kChunk, a.T - t0);
        for (int tt = 0; tt < nt; ++tt) {
            const TokenLds &tok = buf[tt];
            VecSlice kv, qv;
            load_vec(kv, tok.k, c);
            load_vec(qv, tok.q, c);
            const float e = expf(tok.gate);
            const float o = row_token(r, kv, qv, e, tok.beta, tok.v[row]);
            if (c == 0) a.out[((b * a.T + t0 + tt) * a.Hv + h) * D + row] = o;
        }

        if (more) {
            seq_stage(lds[(ch + 1) & 1], cr, tid);
            __syncthreads();
        }
    }
    store_row(Mrow, r, c);
}

// --------------------------------------------------------- tail kernels
// Block-wide sum for a block of NW waves; every thread gets the same bits.
template <int NW>
__device__ __forceinline__ float block_sum(float x, float *scratch) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = x;
    __syncthreads();
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += scratch[w];
    return s;
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// conv-state shift + causal conv1d + SiLU for one 128-channel chunk of one
// sequence; chunks inside the Q and K parts are also L2-normalised (the head
// dim is 128, so a chunk is exactly one head).
template <int K>
__global__ __launch_bounds__(D) void k_prestate(PrestateArgs a) {
    __shared__ float scratch[D / 64];
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
        const float ss = block_sum<D / 64>(s * s, scratch);
        const float nrm = fmaxf(sqrtf(ss), 1e-6f);
        s = s / nrm;
    }
    a.qkv[b * a.C + c] = s;
}

// Gated RMSNorm x SiLU(z) over one group of one row.
constexpr int kNormThreads = 128;
__global__ __launch_bounds__(kNormThreads) void k_gated_norm(GatedNormArgs a) {
    __shared__ float scratch[kNormThreads / 64];
    const int groups = a.n / a.group;
    const int64_t row = blockIdx.x / groups;
    const int64_t base = row * a.n + static_cast<int64_t>(blockIdx.x - row * groups) * a.group;
    float ss = 0.0f;
    for (int i = threadIdx.x; i < a.group; i += kNormThreads) {
        const float o = a.o[base + i];
        ss = fmaf(o, o, ss);
    }
    ss = block_sum<kNormThreads / 64>(ss, scratch);
    const float rms = sqrtf(ss / static_cast<float>(a.group) + a.eps);
    for (int i = threadIdx.x; i < a.group; i += kNormThreads)
        a.y[base + i] = (a.o[base + i] / rms) * a.w[i] * silu(a.z[base + i]);
}

}  // namespace

// ---------------------------------------------------------------- launch
hipError_t launch_step(const StepArgs &a, hipStream_t s) {
    const int64_t heads = static_cast<int64_t>(a.B) * a.Hv;
    k_step<<<dim3(static_cast<unsigned>(heads)), dim3(kStepWaves * 64), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_seq(const SeqArgs &a, hipStream_t s) {
    const int64_t heads = static_cast<int64_t>(a.B) * a.Hv;
    k_seq<<<dim3(static_cast<unsigned>(heads)), dim3(kSeqThreads), 0, s>>>(a);
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

}  // namespace gdn
