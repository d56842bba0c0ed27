// gdn_kernels.hip - gfx950 (CDNA4) kernels of the Gated DeltaNet decode path.
//
// The per-token update (Red Lite dev15c, "Pinned llama.cpp semantics"):
//   M *= exp(gate); sk = M k; delta = (v - sk) beta; M += delta k^T;
//   out = M q / sqrt(128)     on the transposed state M[j][i] = S[i][j].
//
// Work decomposition.  Row j of a head's state depends only on that row,
// on the head's k and q, and on v[j], beta and gate: rows never exchange
// data, not even across tokens.  Every kernel here therefore gives one state
// row (128 floats, 512 contiguous bytes) to a group of eight lanes:
//   lane c (0..7) of the group owns the float4 chunks 8*i + c, i = 0..3,
//   i.e. 16 of the 128 columns, interleaved so that one vector-memory
//   instruction of the group covers one whole 128-byte line of the row.
// A wave64 therefore works on 8 rows at a time (a "tile", 4 KiB of state).
// The two row dot products (M k and M q) are a 16-term FMA chain per lane
// followed by a three-step reduction over the group with DPP
// (row_half_mirror, then two quad_perm swaps); all eight lanes end with
// bitwise-identical sums, so delta is the same in every lane that applies it.
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

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int D = kHeadDim;                        // 128
constexpr int kLanesPerRow = 8;                    // a lane group owns a row
constexpr int kF4PerLane = D / 4 / kLanesPerRow;   // 4 float4 = 16 floats per lane
constexpr int kRowsPerTile = 64 / kLanesPerRow;    // 8 rows per wave
constexpr int kTilesPerHead = D / kRowsPerTile;    // 16
// 1/sqrt(128) rounded to binary32; the output is scaled by it.
constexpr float kInvSqrtD = 0.08838834764831845f;

// ----------------------------------------------------------------- helpers
// DPP move; CTRL is a row_half_mirror or quad_perm selector.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the 8 lanes of a row group; every lane gets the same bits
// (each step adds a value to its partner's copy of the same value).
__device__ __forceinline__ float group_sum(float x) {
    x = x + dpp<0x141>(x);   // row_half_mirror: lane i <-> 7-i within 8
    x = x + dpp<0xB1>(x);    // quad_perm [1,0,3,2]: lane c^1
    x = x + dpp<0x4E>(x);    // quad_perm [2,3,0,1]: lane c^2
    return x;
}

struct RowSlice {   // the 16 state elements of one row that this lane owns
    f4 m[kF4PerLane];
};
struct VecSlice {   // the matching 16 entries of k or q
    f4 x[kF4PerLane];
};

// State rows are streamed with nontemporal loads and stores when NT: they
// are touched once per call and need not displace other data in the caches.
template <bool NT>
__device__ __forceinline__ void load_row(RowSlice &r, const float *row, int c) {
    const f4 *p = reinterpret_cast<const f4 *>(row);
#pragma unroll
    for (int i = 0; i < kF4PerLane; ++i) {
        if constexpr (NT)
            r.m[i] = __builtin_nontemporal_load(p + kLanesPerRow * i + c);
        else
            r.m[i] = p[kLanesPerRow * i + c];
    }
}

template <bool NT>
__device__ __forceinline__ void store_row(float *row, const RowSlice &r, int c) {
    f4 *p = reinterpret_cast<f4 *>(row);
#pragma unroll
    for (int i = 0; i < kF4PerLane; ++i) {
        if constexpr (NT)
            __builtin_nontemporal_store(r.m[i], p + kLanesPerRow * i + c);
        else
            p[kLanesPerRow * i + c] = r.m[i];
    }
}

__device__ __forceinline__ void load_vec(VecSlice &v, const float *src, int c) {
    const f4 *p = reinterpret_cast<const f4 *>(src);
#pragma unroll
    for (int i = 0; i < kF4PerLane; ++i) v.x[i] = p[kLanesPerRow * i + c];
}

// This lane's partial of dot(row, w): a sequential FMA chain over its 16 columns.
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
    const float sk = group_sum(dot_part(r, k));       // 2. sk = M[j] . k
    const float d = (vj - sk) * beta;                 // 3. delta
#pragma unroll
    for (int i = 0; i < kF4PerLane; ++i) {           // 4. rank-1 update
        r.m[i].x = fmaf(d, k.x[i].x, r.m[i].x);
        r.m[i].y = fmaf(d, k.x[i].y, r.m[i].y);
        r.m[i].z = fmaf(d, k.x[i].z, r.m[i].z);
        r.m[i].w = fmaf(d, k.x[i].w, r.m[i].w);
    }
    return group_sum(dot_part(r, q)) * kInvSqrtD;     // 5. output, updated state
}

// The same arithmetic split at the token boundary, for the multi-token
// kernel: head_part() is steps 1-2 of a token, body_part() steps 4-5, and
// pass() runs steps 4-5 of token t and steps 1-2 of token t+1 in one sweep
// over the row.  Every element sees exactly the operations of row_token(),
// in the same order, and the partial sums accumulate in the same element
// order, so the results are bitwise those of row_token().
__device__ __forceinline__ float head_part(RowSlice &r, const VecSlice &k, float e) {
    float p = 0.0f;
#pragma unroll
    for (int i = 0; i < kF4PerLane; ++i) {
        r.m[i].x *= e;
        r.m[i].y *= e;
        r.m[i].z *= e;
        r.m[i].w *= e;
        p = fmaf(r.m[i].x, k.x[i].x, p);
        p = fmaf(r.m[i].y, k.x[i].y, p);
        p = fmaf(r.m[i].z, k.x[i].z, p);
        p = fmaf(r.m[i].w, k.x[i].w, p);
    }
    return p;
}

__device__ __forceinline__ float body_part(RowSlice &r, float d, const VecSlice &k,
                                           const VecSlice &q) {
    float o = 0.0f;
#pragma unroll
    for (int i = 0; i < kF4PerLane; ++i) {
        r.m[i].x = fmaf(d, k.x[i].x, r.m[i].x);
        r.m[i].y = fmaf(d, k.x[i].y, r.m[i].y);
        r.m[i].z = fmaf(d, k.x[i].z, r.m[i].z);
        r.m[i].w = fmaf(d, k.x[i].w, r.m[i].w);
        o = fmaf(r.m[i].x, q.x[i].x, o);
        o = fmaf(r.m[i].y, q.x[i].y, o);
        o = fmaf(r.m[i].z, q.x[i].z, o);
        o = fmaf(r.m[i].w, q.x[i].w, o);
    }
    return o;
}

// Steps 4-5 of token t (delta d, k, q) and steps 1-2 of token t+1 (decay en,
// key kn): this lane's output partial of t goes to o, its key partial of t+1
// to p.
__device__ __forceinline__ void pass(RowSlice &r, float d, const VecSlice &k, const VecSlice &q,
                                     float en, const VecSlice &kn, float &o, float &p) {
    o = 0.0f;
    p = 0.0f;
#pragma unroll
    for (int i = 0; i < kF4PerLane; ++i) {
#define GDN_PASS_LANE(X)                          \
        r.m[i].X = fmaf(d, k.x[i].X, r.m[i].X);   \
        o = fmaf(r.m[i].X, q.x[i].X, o);          \
        r.m[i].X *= en;                           \
        p = fmaf(r.m[i].X, kn.x[i].X, p);
        GDN_PASS_LANE(x)
        GDN_PASS_LANE(y)
        GDN_PASS_LANE(z)
        GDN_PASS_LANE(w)
#undef GDN_PASS_LANE
    }
}

// ------------------------------------------------------------- gdn_step
// HBM-bound: the state is streamed once in and once out.  A persistent grid
// of one 8-wave workgroup per CU walks the tiles (8 rows = 4 KiB each) of all
// heads in a grid-stride loop, one tile per wave per iteration, so the
// addresses in flight at any moment form one contiguous window of ~8 MiB
// that advances through the state.  Measured on MI355X this beats one
// workgroup per head, more or fewer waves per CU, deeper per-wave queues and
// prefetching the next tile.  Workgroup g runs on XCD g % 8; the tile order
// is remapped so that the 16 tiles of a head go to workgroups of one XCD and
// its k and q are fetched into one L2 only.
constexpr int kStepWaves = 8;
constexpr int kXcds = 8;

__global__ __launch_bounds__(kStepWaves * 64) void k_step(StepArgs a, int n_tiles) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = lane >> 3;
    const int c = lane & 7;

    const int G = gridDim.x;
    const int g = blockIdx.x;
    const int lg = (G % kXcds == 0) ? (g % kXcds) * (G / kXcds) + g / kXcds : g;
    const int stride = G * kStepWaves;

    for (int u = lg * kStepWaves + wave; u < n_tiles; u += stride) {
        const int head = u / kTilesPerHead;                   // b * Hv + h
        const int row = (u % kTilesPerHead) * kRowsPerTile + grp;
        const int b = head / a.Hv;
        const int h = head - b * a.Hv;
        const int kh = h % a.Hk;                              // key-head broadcast

        float *Mrow = a.state + static_cast<int64_t>(head) * (D * D) + row * D;
        RowSlice r;
        load_row<true>(r, Mrow, c);
        VecSlice kv, qv;
        load_vec(kv, a.k + b * a.qk_bstride + kh * D, c);
        load_vec(qv, a.q + b * a.qk_bstride + kh * D, c);
        const float e = expf(a.gate[head]);
        const float bt = a.beta[head];
        const float vj = a.v[b * a.v_bstride + h * D + row];

        const float o = row_token(r, kv, qv, e, bt, vj);
        store_row<true>(Mrow, r, c);
        if (c == 0) a.out[static_cast<int64_t>(head) * D + row] = o;
    }
}

// ------------------------------------------------------------- gdn_pair
// Speculative two-position step (docs.rs "Module linear_core", gdn_pair):
// the same persistent tile walk as k_step; each row is read once, advanced
// by position 1 and written back to `state` (committed), then advanced by
// position 2 in registers and written to `state_next` (tentative).  Three
// state transfers instead of the four of two separate steps.
__global__ __launch_bounds__(kStepWaves * 64) void k_pair(PairArgs a, int n_tiles) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = lane >> 3;
    const int c = lane & 7;

    const int G = gridDim.x;
    const int g = blockIdx.x;
    const int lg = (G % kXcds == 0) ? (g % kXcds) * (G / kXcds) + g / kXcds : g;
    const int stride = G * kStepWaves;

    for (int u = lg * kStepWaves + wave; u < n_tiles; u += stride) {
        const int head = u / kTilesPerHead;
        const int row = (u % kTilesPerHead) * kRowsPerTile + grp;
        const int b = head / a.Hv;
        const int h = head - b * a.Hv;
        const int kh = h % a.Hk;
        const int64_t roff = static_cast<int64_t>(head) * (D * D) + row * D;

        RowSlice r;
        load_row<true>(r, a.state + roff, c);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int64_t bp = static_cast<int64_t>(b) * 2 + p;
            VecSlice kv, qv;
            load_vec(kv, a.k + (bp * a.Hk + kh) * D, c);
            load_vec(qv, a.q + (bp * a.Hk + kh) * D, c);
            const int64_t hp = bp * a.Hv + h;
            const float e = expf(a.gate[hp]);
            const float o = row_token(r, kv, qv, e, a.beta[hp], a.v[hp * D + row]);
            store_row<true>((p == 0 ? a.state : a.state_next) + roff, r, c);
            if (c == 0) a.out[hp * D + row] = o;
        }
    }
}

// -------------------------------------------------------------- gdn_seq
// One workgroup per (sequence, value head): 8 waves x 2 tiles, so the whole
// 64 KiB head state lives in VGPRs (32 floats per lane) for all T tokens and
// is read and written once per call.  The per-token inputs (k, q, v,
// exp(gate), beta: 1.5 KiB per token) are staged through LDS in chunks of
// kChunk = 32 tokens, double-buffered (97 KiB of LDS; gfx950 allows 160 KiB
// per workgroup): the global loads of chunk c+1 are issued before chunk c is
// computed and written to LDS after it, so their latency hides behind 32
// tokens of arithmetic.  Outputs overwrite the consumed v entries in LDS
// (row j's v is read only by row j's lanes, before its output exists) and are
// flushed to HBM with coalesced 16-byte stores once per chunk.  Two barriers
// per chunk; none per token.
//
// Within a chunk the row update is software-pipelined (pass()): the update
// and output of token t share one sweep over the registers with the decay and
// key dot product of token t+1, so only the key reduction sits on the
// critical path between tokens.  Full chunks are unrolled, so every LDS
// address is an immediate offset and no loop bookkeeping runs per token.
// The kernel is VALU-issue bound (measured: VALU busy ~97 %), so every
// instruction per token counts.
#ifndef GDN_SEQ_CHUNK
#define GDN_SEQ_CHUNK 32
#endif
#ifndef GDN_SEQ_TILES_PER_WAVE
#define GDN_SEQ_TILES_PER_WAVE 2
#endif
constexpr int kChunk = GDN_SEQ_CHUNK;
constexpr int kSeqTilesPerWave = GDN_SEQ_TILES_PER_WAVE;
constexpr int kSeqWaves = kTilesPerHead / kSeqTilesPerWave;   // 8
constexpr int kSeqThreads = kSeqWaves * 64;                   // 512

struct alignas(16) TokenLds {
    float k[D];
    float q[D];
    float v[D];       // v on entry; the token's output once computed
    float e;          // exp(gate)
    float beta;
    float pad[2];
};
static_assert(sizeof(TokenLds) % 16 == 0, "float4 aligned token slots");

// float4 loads per token: k (32) + q (32) + v (32)
constexpr int kTokF4 = 3 * D / 4;
constexpr int kChunkF4 = kChunk * kTokF4;                     // 3072
constexpr int kFetchPer = (kChunkF4 + kSeqThreads - 1) / kSeqThreads;   // 6
constexpr int kFlushPer = (kChunk * D / 4 + kSeqThreads - 1) / kSeqThreads; // 2
static_assert(2 * kChunk <= kSeqThreads, "one thread per gate and per beta");

struct ChunkRegs {
    f4 f[kFetchPer];
    float s;   // gate or beta of one token (threads 0 .. 2*kChunk-1)
};

__device__ __forceinline__ void seq_fetch(ChunkRegs &cr, const SeqArgs &a, int64_t b, int h,
                                          int kh, int t0, int tid) {
#pragma unroll
    for (int j = 0; j < kFetchPer; ++j) {
        const int e = tid + j * kSeqThreads;
        const int tt = e / kTokF4;
        const int w = e - tt * kTokF4;
        const int t = t0 + tt;
        f4 val = {0.f, 0.f, 0.f, 0.f};
        if (e < kChunkF4 && t < a.T) {
            const int64_t bt = b * a.T + t;
            const float *src;
            if (w < 32)
                src = a.k + (bt * a.Hk + kh) * D + 4 * w;
            else if (w < 64)
                src = a.q + (bt * a.Hk + kh) * D + 4 * (w - 32);
            else
                src = a.v + (bt * a.Hv + h) * D + 4 * (w - 64);
            val = *reinterpret_cast<const f4 *>(src);
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
    for (int j = 0; j < kFetchPer; ++j) {
        const int e = tid + j * kSeqThreads;
        if (e >= kChunkF4) break;
        const int tt = e / kTokF4;
        const int w = e - tt * kTokF4;
        float *dst = w < 32 ? buf[tt].k + 4 * w
                   : w < 64 ? buf[tt].q + 4 * (w - 32)
                            : buf[tt].v + 4 * (w - 64);
        *reinterpret_cast<f4 *>(dst) = cr.f[j];
    }
    if (tid < kChunk)
        buf[tid].e = expf(cr.s);          // the token's decay factor, computed once
    else if (tid < 2 * kChunk)
        buf[tid - kChunk].beta = cr.s;
}

// Token tt of a chunk: steps 3-5 of tt and, when `next`, steps 1-2 of tt+1
// (kv holds k of token tt on entry and of tt+1 on exit; p the key partials).
template <int TPW>
__device__ __forceinline__ void seq_token(TokenLds *buf, int tt, bool next, const int (&rows)[TPW],
                                          RowSlice (&r)[TPW], VecSlice &kv, float (&p)[TPW],
                                          int c) {
    TokenLds &tok = buf[tt];
    float d[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t)                              // step 3
        d[t] = (tok.v[rows[t]] - group_sum(p[t])) * tok.beta;
    VecSlice qv;
    load_vec(qv, tok.q, c);
    float o[TPW];
    if (next) {
        VecSlice kn;
        load_vec(kn, buf[tt + 1].k, c);
        const float en = buf[tt + 1].e;
#pragma unroll
        for (int t = 0; t < TPW; ++t) pass(r[t], d[t], kv, qv, en, kn, o[t], p[t]);
        kv = kn;
    } else {
#pragma unroll
        for (int t = 0; t < TPW; ++t) o[t] = body_part(r[t], d[t], kv, qv);
    }
    // every lane of the row group holds the same output bits
#pragma unroll
    for (int t = 0; t < TPW; ++t) tok.v[rows[t]] = group_sum(o[t]) * kInvSqrtD;
}

__global__ __launch_bounds__(kSeqThreads) void k_seq(SeqArgs a) {
    constexpr int TPW = kSeqTilesPerWave;
    __shared__ TokenLds lds[2][kChunk];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = lane >> 3;
    const int c = lane & 7;

    const int head = blockIdx.x;                  // b * Hv + h
    const int b = head / a.Hv;
    const int h = head - b * a.Hv;
    const int kh = h % a.Hk;

    float *M = a.state + static_cast<int64_t>(head) * (D * D);
    int rows[TPW];
    RowSlice r[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        rows[t] = (wave * TPW + t) * kRowsPerTile + grp;
        load_row<false>(r[t], M + rows[t] * D, c);
    }

    ChunkRegs cr;
    seq_fetch(cr, a, b, h, kh, 0, tid);
    seq_stage(lds[0], cr, tid);
    __syncthreads();

    const int n_chunks = (a.T + kChunk - 1) / kChunk;
    for (int ch = 0; ch < n_chunks; ++ch) {
        const bool more = ch + 1 < n_chunks;
        if (more) seq_fetch(cr, a, b, h, kh, (ch + 1) * kChunk, tid);

        TokenLds *buf = lds[ch & 1];
        const int t0 = ch * kChunk;
        const int nt = min(kChunk, a.T - t0);

        // steps 1-2 of the chunk's first token
        VecSlice kv;
        load_vec(kv, buf[0].k, c);
        float p[TPW];
        {
            const float e0 = buf[0].e;
#pragma unroll
            for (int t = 0; t < TPW; ++t) p[t] = head_part(r[t], kv, e0);
        }
        if (nt == kChunk) {
            // full chunk: unrolled, so every LDS address is an immediate offset
#pragma unroll
            for (int tt = 0; tt < kChunk; ++tt) seq_token(buf, tt, tt + 1 < kChunk, rows, r, kv, p, c);
        } else {
            for (int tt = 0; tt < nt; ++tt) seq_token(buf, tt, tt + 1 < nt, rows, r, kv, p, c);
        }
        __syncthreads();                 // outputs of chunk ch complete in LDS

#pragma unroll
        for (int j = 0; j < kFlushPer; ++j) {   // flush: float4s of the outputs
            const int e = tid + j * kSeqThreads;
            const int tt = e / (D / 4);
            const int col = (e % (D / 4)) * 4;
            if (tt < nt) {
                const int64_t o = ((static_cast<int64_t>(b) * a.T + t0 + tt) * a.Hv + h) * D + col;
                *reinterpret_cast<f4 *>(a.out + o) = *reinterpret_cast<const f4 *>(buf[tt].v + col);
            }
        }
        if (more) seq_stage(lds[(ch + 1) & 1], cr, tid);
        __syncthreads();                 // chunk ch+1 staged; chunk ch flushed
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) store_row<false>(M + rows[t] * D, r[t], c);
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


// ------------------------------------------------------ fused layer tail
// The whole recurrent-branch tail for one token in one launch.  One
// workgroup per (sequence b, key head kh) owns every channel that key head's
// value heads need: Q head kh, K head kh and the V channels of the RV value
// heads h = kh + i*Hk.  Owning them outright makes the conv-cache shift
// race-free, and lets the step read Q, K and V from LDS.  The workgroup issues
// the nontemporal loads of its RV x 64 KiB of state first and computes the
// prestate while they are in flight.  Every reduction keeps the order of the
// three-launch path (k_prestate, k_step, k_gated_norm), so both paths give
// the same bits.
constexpr int kTailThreads = 256;

template <int RV, int K>
__global__ __launch_bounds__(kTailThreads) void k_tail_fused(TailFusedArgs a) {
    constexpr int kCh = (2 + RV) * D;               // owned channels
    constexpr int kTiles = RV * kTilesPerHead;      // state tiles of the workgroup
    constexpr int kTilesPerWave = kTiles / (kTailThreads / 64);
    __shared__ alignas(16) float act[kCh];          // Q | K | V_0 .. V_{RV-1}
    __shared__ float core[RV * D];
    __shared__ float scratch[kTailThreads / 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = lane >> 3;
    const int c = lane & 7;
    const int b = blockIdx.x / a.Hk;
    const int kh = blockIdx.x - b * a.Hk;
    const int nq = a.Hk * D;

    // 1. state loads in flight
    RowSlice r[kTilesPerWave];
    int64_t roff[kTilesPerWave];
#pragma unroll
    for (int j = 0; j < kTilesPerWave; ++j) {
        const int t = wave * kTilesPerWave + j;
        const int h = kh + (t / kTilesPerHead) * a.Hk;
        const int row = (t % kTilesPerHead) * kRowsPerTile + grp;
        roff[j] = (static_cast<int64_t>(b) * a.Hv + h) * (D * D) + row * D;
        load_row<true>(r[j], a.state + roff[j], c);
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
            if (lane == 0) scratch[wave] = x2;
            __syncthreads();
            const int h2 = wave >> 1;              // 0: Q, 1: K
            const float ss = (0.0f + scratch[2 * h2]) + scratch[2 * h2 + 1];
            s = s / fmaxf(sqrtf(ss), 1e-6f);
        }
        act[slot] = s;
        if (a.dbg_qkv) a.dbg_qkv[static_cast<int64_t>(b) * a.C + ch] = s;
    }
    __syncthreads();

    // 3. the state step on the preloaded rows; k and q come from LDS
    VecSlice kv, qv;
    load_vec(kv, act + D, c);
    load_vec(qv, act, c);
#pragma unroll
    for (int j = 0; j < kTilesPerWave; ++j) {
        const int t = wave * kTilesPerWave + j;
        const int i = t / kTilesPerHead;
        const int h = kh + i * a.Hk;
        const int row = (t % kTilesPerHead) * kRowsPerTile + grp;
        const int bh = b * a.Hv + h;
        const float e = expf(a.gate[bh]);
        const float o = row_token(r[j], kv, qv, e, a.beta[bh], act[(2 + i) * D + row]);
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
        if (lane == 0) scratch[wave] = x2;
        __syncthreads();
        if (live) {
            const float ss = (0.0f + scratch[2 * i]) + scratch[2 * i + 1];
            const float rms = sqrtf(ss / static_cast<float>(D) + a.eps);
            const int h = kh + i * a.Hk;
            const int64_t yo = static_cast<int64_t>(b) * a.Hv * D + static_cast<int64_t>(h) * D + j;
            a.y[yo] = (o / rms) * a.norm_w[j] * silu(a.z[yo]);
            if (a.dbg_core) a.dbg_core[yo] = o;
        }
    }
}

}  // namespace

// ---------------------------------------------------------------- launch
#ifndef GDN_STEP_WGS_PER_CU
#define GDN_STEP_WGS_PER_CU 1
#endif

// Compute units of the current device (read once per device; a value that
// never changes, so concurrent first calls race harmlessly).
static int device_cus() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

hipError_t launch_step(const StepArgs &a, hipStream_t s) {
    const int64_t tiles = static_cast<int64_t>(a.B) * a.Hv * kTilesPerHead;
    const int64_t full = device_cus() * static_cast<int64_t>(GDN_STEP_WGS_PER_CU);
    const int64_t need = (tiles + kStepWaves - 1) / kStepWaves;
    const int grid = static_cast<int>(need < full ? need : full);
    k_step<<<dim3(grid), dim3(kStepWaves * 64), 0, s>>>(a, static_cast<int>(tiles));
    return hipGetLastError();
}

hipError_t launch_pair(const PairArgs &a, hipStream_t s) {
    const int64_t tiles = static_cast<int64_t>(a.B) * a.Hv * kTilesPerHead;
    const int64_t full = device_cus() * static_cast<int64_t>(GDN_STEP_WGS_PER_CU);
    const int64_t need = (tiles + kStepWaves - 1) / kStepWaves;
    const int grid = static_cast<int>(need < full ? need : full);
    k_pair<<<dim3(grid), dim3(kStepWaves * 64), 0, s>>>(a, static_cast<int>(tiles));
    return hipGetLastError();
}

hipError_t launch_seq(const SeqArgs &a, hipStream_t s) {
    const int64_t heads = static_cast<int64_t>(a.B) * a.Hv;
    k_seq<<<dim3(static_cast<unsigned>(heads)), dim3(kSeqThreads), 0, s>>>(a);
    return hipGetLastError();
}

bool tail_fused_supported(int32_t Hv, int32_t Hk, int32_t K, int32_t group) {
    const int32_t rv = Hv / Hk;
    return (rv == 1 || rv == 2) && K == 4 && group == D;
}

hipError_t launch_tail_fused(const TailFusedArgs &a, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hk));
    if (a.Hv == a.Hk && a.K == 4)
        k_tail_fused<1, 4><<<grid, dim3(kTailThreads), 0, s>>>(a);
    else if (a.Hv == 2 * a.Hk && a.K == 4)
        k_tail_fused<2, 4><<<grid, dim3(kTailThreads), 0, s>>>(a);
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

}  // namespace gdn
