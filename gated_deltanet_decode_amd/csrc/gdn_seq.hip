// gdn_seq.hip - gdn_seq: the multi-token kernel with the state resident in
// registers.

#include "gdn_device.hpp"

namespace gdn {
namespace {

// -------------------------------------------------------------- gdn_seq
// One workgroup per (sequence, value head), or per half head for short
// sequences, of waves holding 2 tiles each: the head's state lives in VGPRs
// (32 floats per lane) for all T tokens and is read and written once per
// call.  Rows never exchange data, so a head splits across workgroups
// freely; each part stages the head's k and q and flushes only its own rows'
// outputs.
//
// The per-token inputs (k, q, v, exp(gate), beta: 1.5 KiB per token) are
// staged through LDS in chunks of CH tokens (8, 16 or 32 by sequence length),
// double-buffered (97 KiB of LDS for CH = 32; gfx950 allows 160 KiB per
// workgroup): the global loads of chunk c+1 are issued before chunk c is
// computed and written to LDS after it, so their latency hides behind CH
// tokens of arithmetic.  Outputs overwrite the consumed v entries in LDS (row
// j's v is read only by row j's lanes, before its output exists) and are
// flushed to HBM with coalesced 16-byte stores once per chunk.  Two barriers
// per chunk; none per token.
//
// Within a chunk the row update is software-pipelined (pass()): the update
// and output of token t share one sweep over the registers with the decay and
// key dot product of token t+1, so only the key reduction sits on the
// critical path between tokens.  Full chunks are unrolled, so every LDS
// address is an immediate offset and no loop bookkeeping runs per token.
// Long sequences are VALU-issue bound (measured: VALU busy ~97 %), so every
// instruction per token counts.

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

// Sizes of a chunk of CH tokens staged by NTH threads (CH = 32, NTH = 512:
// 3072 float4, 6 per thread).
template <int CH, int NTH>
struct Chunk {
    static constexpr int kF4 = CH * kTokF4;
    static constexpr int kFetchPer = (kF4 + NTH - 1) / NTH;
    static_assert(2 * CH <= NTH, "one thread per gate and per beta");
};

template <int CH, int NTH>
struct ChunkRegs {
    f4 f[Chunk<CH, NTH>::kFetchPer];
    float s;   // gate or beta of one token (threads 0 .. 2*CH-1)
};

template <int CH, int NTH>
__device__ __forceinline__ void seq_fetch(ChunkRegs<CH, NTH> &cr, const SeqArgs &a, int64_t b, int h,
                                          int kh, int t0, int tid) {
#pragma unroll
    for (int j = 0; j < Chunk<CH, NTH>::kFetchPer; ++j) {
        const int e = tid + j * NTH;
        const int tt = e / kTokF4;
        const int w = e - tt * kTokF4;
        const int t = t0 + tt;
        f4 val = {0.f, 0.f, 0.f, 0.f};
        if (e < Chunk<CH, NTH>::kF4 && t < a.T) {
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
    if (tid < 2 * CH) {
        const int tt = tid < CH ? tid : tid - CH;
        const int t = t0 + tt;
        if (t < a.T) {
            const int64_t idx = (b * a.T + t) * a.Hv + h;
            cr.s = tid < CH ? a.gate[idx] : a.beta[idx];
        }
    }
}

template <int CH, int NTH>
__device__ __forceinline__ void seq_stage(TokenLds *buf, const ChunkRegs<CH, NTH> &cr, int tid) {
#pragma unroll
    for (int j = 0; j < Chunk<CH, NTH>::kFetchPer; ++j) {
        const int e = tid + j * NTH;
        if (e >= Chunk<CH, NTH>::kF4) break;
        const int tt = e / kTokF4;
        const int w = e - tt * kTokF4;
        float *dst = w < 32 ? buf[tt].k + 4 * w
                   : w < 64 ? buf[tt].q + 4 * (w - 32)
                            : buf[tt].v + 4 * (w - 64);
        *reinterpret_cast<f4 *>(dst) = cr.f[j];
    }
    if (tid < CH)
        buf[tid].e = expf(cr.s);          // the token's decay factor, computed once
    else if (tid < 2 * CH)
        buf[tid - CH].beta = cr.s;
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

// CH: tokens per LDS chunk; NT: nontemporal state load and store; a head's
// 128 rows are split over PARTS workgroups of 16 / (TPW * PARTS) waves with
// TPW tiles each.
template <int CH, bool NT, int TPW, int PARTS>
__global__ __launch_bounds__(64 * 16 / (TPW * PARTS)) void k_seq(SeqArgs a) {
    constexpr int NTH = 64 * 16 / (TPW * PARTS);
    constexpr int R = D / PARTS;                  // rows of this workgroup
    __shared__ TokenLds lds[2][CH];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = lane >> 3;
    const int c = lane & 7;

    const int head = blockIdx.x / PARTS;          // b * Hv + h
    const int part = blockIdx.x - head * PARTS;
    const int b = head / a.Hv;
    const int h = head - b * a.Hv;
    const int kh = h % a.Hk;

    float *M = a.state + static_cast<int64_t>(head) * (D * D);
    int rows[TPW];
    RowSlice r[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        rows[t] = part * R + (wave * TPW + t) * kRowsPerTile + grp;
        load_row<NT>(r[t], M + rows[t] * D, c);
    }

    ChunkRegs<CH, NTH> cr;
    seq_fetch(cr, a, b, h, kh, 0, tid);
    seq_stage(lds[0], cr, tid);
    __syncthreads();

    const int n_chunks = (a.T + CH - 1) / CH;
    for (int ch = 0; ch < n_chunks; ++ch) {
        const bool more = ch + 1 < n_chunks;
        if (more) seq_fetch(cr, a, b, h, kh, (ch + 1) * CH, tid);

        TokenLds *buf = lds[ch & 1];
        const int t0 = ch * CH;
        const int nt = min(CH, a.T - t0);

        // steps 1-2 of the chunk's first token
        VecSlice kv;
        load_vec(kv, buf[0].k, c);
        float p[TPW];
        {
            const float e0 = buf[0].e;
#pragma unroll
            for (int t = 0; t < TPW; ++t) p[t] = head_part(r[t], kv, e0);
        }
        if (nt == CH) {
            // full chunk: unrolled, so every LDS address is an immediate offset
#pragma unroll
            for (int tt = 0; tt < CH; ++tt) seq_token(buf, tt, tt + 1 < CH, rows, r, kv, p, c);
        } else {
            for (int tt = 0; tt < nt; ++tt) seq_token(buf, tt, tt + 1 < nt, rows, r, kv, p, c);
        }
        __syncthreads();                 // outputs of chunk ch complete in LDS

#pragma unroll
        for (int j = 0; j < (CH * R / 4 + NTH - 1) / NTH; ++j) {   // flush this part's outputs
            const int e = tid + j * NTH;
            const int tt = e / (R / 4);
            const int col = part * R + (e % (R / 4)) * 4;
            if (tt < nt) {
                const int64_t o = ((static_cast<int64_t>(b) * a.T + t0 + tt) * a.Hv + h) * D + col;
                *reinterpret_cast<f4 *>(a.out + o) = *reinterpret_cast<const f4 *>(buf[tt].v + col);
            }
        }
        if (more) seq_stage(lds[(ch + 1) & 1], cr, tid);
        __syncthreads();                 // chunk ch+1 staged; chunk ch flushed
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) store_row<NT>(M + rows[t] * D, r[t], c);
}

}  // namespace

// Chunk size and state access by sequence length (measured on MI355X):
// long sequences stage 32 tokens per chunk and keep the plain state access;
// short ones are dominated by the state transfer, which the nontemporal hint
// speeds up by up to ~15 %, and by the last, partial chunk, which a smaller
// chunk (fully unrolled more often) shortens.
// Launch shape by sequence length (measured on MI355X):
// - T = 1 runs the single-step kernel (in gdn_api.cpp);
// - T <= 32: the state transfer dominates; two workgroups of 4 waves per head
//   (64 rows each) let two heads' halves share a CU, so one's state transfer
//   overlaps the other's arithmetic (15-24 % faster at B = 256, T = 2..8);
//   the nontemporal hint speeds the transfer up; chunks of 8 (T < 16) or 16
//   tokens shorten the last, partial chunk;
// - longer sequences are VALU-bound: one 8-wave workgroup per head, 32-token
//   chunks, plain state access (two parts per head measured 40 % slower).
hipError_t launch_seq(const SeqArgs &a, hipStream_t s) {
    const int64_t heads = static_cast<int64_t>(a.B) * a.Hv;
    const dim3 split(static_cast<unsigned>(heads * 2)), whole(static_cast<unsigned>(heads));
    if (a.T < 16)
        k_seq<8, true, 2, 2><<<split, dim3(256), 0, s>>>(a);
    else if (a.T <= 32)
        k_seq<16, true, 2, 2><<<split, dim3(256), 0, s>>>(a);
    else
        k_seq<32, false, 2, 1><<<whole, dim3(512), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace gdn
