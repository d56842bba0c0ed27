// gdn_seq.hip - gdn_seq: the multi-token kernel with the state resident in
// registers.

#include <cstddef>

#include "gdn_device.hpp"

namespace gdn {
namespace {

// -------------------------------------------------------------- gdn_seq
// One workgroup per (sequence, value head), or per half head for short
// sequences and for more heads than CUs, of waves holding 2 tiles each: the
// head's state lives in VGPRs (32 floats per lane) for all T tokens and is
// read and written once per call.  Rows never exchange data, so a head splits
// across workgroups freely; each part stages the head's k and q and flushes
// only its own rows' outputs.
//
// The per-token inputs (k, q, v, exp(gate), beta, and for the scaled decay
// below two per-token factors: 1.5 KiB per token) are
// staged through LDS in chunks of CH tokens (8, 16 or 32 by sequence length),
// double-buffered (97 KiB of LDS for CH = 32; gfx950 allows 160 KiB per
// workgroup): the global loads of chunk c+1 are issued before chunk c is
// computed and written to LDS after it, so their latency hides behind CH
// tokens of arithmetic.  With DMA, k, q and v go from global memory straight
// into LDS (global_load_lds_dwordx4) and hold no registers meanwhile.
// Outputs overwrite the consumed v entries in LDS (row j's v is read only by
// row j's lanes, before its output exists) and are flushed to HBM with
// coalesced 16-byte stores once per chunk.  Two barriers per chunk; none per
// token.
//
// Within a chunk the row update is software-pipelined (pass()): the update
// and output of token t share one sweep over the registers with the decay and
// key dot product of token t+1, so only the key reduction sits on the
// critical path between tokens.  Full chunks are unrolled, so every LDS
// address is an immediate offset and no loop bookkeeping runs per token.
// With PAIR, a wave's two tiles are reduced together (seq_token, pair_sum):
// per token and lane that is 3 DPP adds for both key sums and 3 for both
// outputs, one delta and one output, instead of 6 + 6, two and two.
// Long sequences are VALU-issue bound (measured: VALU instructions issue
// 81-96 % of the time), so every instruction per token counts: 16- and
// 32-token chunks also carry the decay as a scale (scaled decay, below).

struct alignas(16) TokenLds {
    float k[D];
    float q[D];
    float v[D];       // v on entry; the token's output once computed
    float e;          // exp(gate)
    float beta;
    float w;          // scaled decay: beta / c_t
    float os;         // scaled decay: c_t / sqrt(d)
};
static_assert(sizeof(TokenLds) % 16 == 0, "float4 aligned token slots");

// Chunk staging: every thread fetches float4 column 4 * (tid % 32) of k, q
// and v for tokens tid / 32 + n * NTH / 32 of the chunk, kSlots tokens per
// array (CH = 32, NTH = 512: 2 tokens, 6 float4 per thread).  A slot's array
// and token offset are compile-time constants, so a chunk's addresses are a
// few pointer increments.
template <int CH, int NTH>
struct Chunk {
    static constexpr int kTokStride = NTH / 32;          // tokens apart of a thread's slots
    static constexpr int kSlots = CH / kTokStride;       // slots per array
    static constexpr int kFetchPer = 3 * kSlots;
    static_assert(NTH % 32 == 0 && CH % kTokStride == 0, "whole token rows per slot");
    static_assert(2 * CH <= NTH, "one thread per gate and per beta");
};

template <int CH, int NTH, bool DMA>
struct ChunkRegs {
    f4 f[DMA ? 1 : Chunk<CH, NTH>::kFetchPer];   // k slots, then q, then v (unused with DMA)
    float s;    // gate or beta of one token (threads 0 .. 2*CH-1); with the
    float s2;   // scaled decay, thread t < CH holds token t's gate and beta
};

// Global-to-LDS load of 16 bytes per lane (global_load_lds_dwordx4): lane l's
// bytes land at dst + 16 l.  dst must be the same in every lane of the wave;
// the data is in LDS once the wave's vector-memory counter has drained
// (s_waitcnt with kWaitVmcnt0, the gfx9 encoding of vmcnt(0) alone).
constexpr int kWaitVmcnt0 = 0x0F70;
__device__ __forceinline__ void load_lds16(const float *src, float *dst) {
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void *)(src),
                                     (__attribute__((address_space(3))) void *)(dst), 16, 0, 0);
}

// kClamp: the chunk may run past token T - 1 (only a sequence's last chunk
// can); slots past the end load token T - 1 again, which nothing reads (a
// partial chunk computes, flushes and takes the next key of its first nt
// tokens only).  Every load is unconditional and in bounds.
// DMA: token tt of the chunk is fetched by wave tt % NW straight into its
// LDS slot (buf): k and q, adjacent there, with one instruction (lanes 0-31
// k, 32-63 q: 1 KiB), v with a second one on lanes 0-31 (512 B).
template <int CH, int NTH, bool kClamp, bool SC, bool DMA>
__device__ __forceinline__ void seq_fetch(ChunkRegs<CH, NTH, DMA> &cr, TokenLds *buf, const SeqArgs &a,
                                          int64_t b, int h, int kh, int t0, int tid) {
    using C = Chunk<CH, NTH>;
    if constexpr (DMA) {
        constexpr int NW = NTH / 64;
        static_assert(CH % NW == 0, "whole tokens per wave");
        static_assert(offsetof(TokenLds, q) == offsetof(TokenLds, k) + D * sizeof(float),
                      "k and q adjacent: one 1 KiB transfer");
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const bool lo = lane < 32;
        const int c4 = 4 * (lane & 31);
#pragma unroll
        for (int n = 0; n < CH / NW; ++n) {
            const int tt = wave + n * NW;
            const int t = kClamp ? min(t0 + tt, a.T - 1) : t0 + tt;
            const int64_t bt = b * a.T + t;
            load_lds16((lo ? a.k : a.q) + (bt * a.Hk + kh) * D + c4, buf[tt].k);
            if (lo) load_lds16(a.v + (bt * a.Hv + h) * D + c4, buf[tt].v);
        }
    }
    const int col = 4 * (tid & 31);
    const int t = t0 + (tid >> 5);                      // token of slot 0
    const int64_t bt = b * a.T + t;
    const int64_t koff = (bt * a.Hk + kh) * D + col;    // k and q share the layout
    const int64_t voff = (bt * a.Hv + h) * D + col;
    const int64_t ktok = static_cast<int64_t>(a.Hk) * D;   // one token apart
    const int64_t vtok = static_cast<int64_t>(a.Hv) * D;
#pragma unroll
    for (int n = 0; n < (DMA ? 0 : C::kSlots); ++n) {
        const int dt = kClamp ? min(t + n * C::kTokStride, a.T - 1) - t : n * C::kTokStride;
        cr.f[n] = *reinterpret_cast<const f4 *>(a.k + koff + dt * ktok);
        cr.f[C::kSlots + n] = *reinterpret_cast<const f4 *>(a.q + koff + dt * ktok);
        cr.f[2 * C::kSlots + n] = *reinterpret_cast<const f4 *>(a.v + voff + dt * vtok);
    }
    cr.s = 0.0f;
    cr.s2 = 0.0f;
    if constexpr (SC) {
        if (tid < CH) {
            const int tg = kClamp ? min(t0 + tid, a.T - 1) : t0 + tid;
            const int64_t idx = (b * a.T + tg) * a.Hv + h;
            cr.s = a.gate[idx];
            cr.s2 = a.beta[idx];
        }
    } else if (tid < 2 * CH) {
        const int tt = tid < CH ? tid : tid - CH;
        const int tg = kClamp ? min(t0 + tt, a.T - 1) : t0 + tt;
        const int64_t idx = (b * a.T + tg) * a.Hv + h;
        cr.s = tid < CH ? a.gate[idx] : a.beta[idx];
    }
}

template <int CH, int NTH, bool SC, bool DMA>
__device__ __forceinline__ void fetch_chunk(ChunkRegs<CH, NTH, DMA> &cr, TokenLds *buf, const SeqArgs &a,
                                            int64_t b, int h, int kh, int t0, int tid) {
    // 8-token chunks (sequences under 16 tokens) always clamp: one code path
    // measured 1-3 % faster at T = 3..6.
    if (CH > 8 && t0 + CH <= a.T)
        seq_fetch<CH, NTH, false, SC, DMA>(cr, buf, a, b, h, kh, t0, tid);
    else
        seq_fetch<CH, NTH, true, SC, DMA>(cr, buf, a, b, h, kh, t0, tid);
}

// Scaled decay.  The decay multiplies every state element by the same
// factor, so within a group of kScaleGroup tokens the registers may hold
// S / c_t, with c_t the product of the group's decays up to token t: a
// token's decay then changes c_t instead of the registers, the key product
// is c_t (S / c_t) . k, the delta is applied as delta / c_t, and the output
// is c_t (S / c_t) . q.  That takes the decay multiply, one of the four VALU
// instructions per element and token, off the registers; c of the group's
// last token is multiplied back in at its end.  Staging computes c_t (a
// prefix product over the group's lanes), w_t = beta_t / c_t and
// c_t / sqrt(d) once per group, so a token's delta is
// v w - ((S / c_t) . k) beta and its output scale one multiply.
// A group runs scaled only when it is complete, all its gates are <= 0 (no
// NaN) and its decay product is >= kMinScale (2^-63), so c_t stays normal
// and S / c_t at most 2^63.5 |S| (finite for |S| up to about 1e19; larger
// states need the per-token form); otherwise it runs with the per-token
// multiply.  Groups are counted from the call's first token in every launch
// shape, so results do not depend on the shape (or on B); but a scaled
// group's rounding differs from the per-token multiply, so its results are
// not bitwise those of gdn_step.
constexpr int kScaleGroup = 16;
constexpr float kMinScale = 0x1p-63f;

// DPP move that keeps `old` in lanes without a source (row shifts).
template <int CTRL>
__device__ __forceinline__ float dpp_or(float old, float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                                 __builtin_bit_cast(int, x), CTRL,
                                                                 0xF, 0xF, false));
}

__device__ __forceinline__ float lane_value(float x, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// Stages a fetched chunk into LDS (with DMA, its per-token scalars only).
// With SC, info[2 g] says whether group g of the chunk may run scaled (1 or
// 0) and info[2 g + 1] is its decay product.
template <int CH, int NTH, bool SC, bool DMA>
__device__ __forceinline__ void seq_stage(TokenLds *buf, float *info, const ChunkRegs<CH, NTH, DMA> &cr,
                                          int tid) {
    using C = Chunk<CH, NTH>;
    const int col = 4 * (tid & 31);
    TokenLds *tok = buf + (tid >> 5);
#pragma unroll
    for (int n = 0; n < (DMA ? 0 : C::kSlots); ++n) {
        TokenLds &tk = tok[n * C::kTokStride];
        *reinterpret_cast<f4 *>(tk.k + col) = cr.f[n];
        *reinterpret_cast<f4 *>(tk.q + col) = cr.f[C::kSlots + n];
        *reinterpret_cast<f4 *>(tk.v + col) = cr.f[2 * C::kSlots + n];
    }
    if constexpr (SC) {
        static_assert(kScaleGroup == 16 && CH % kScaleGroup == 0 && CH <= 64,
                      "a group is one row of 16 lanes of wave 0");
        if (tid < 64) {                   // wave 0: lane t < CH holds token t's gate and beta
            const bool mine = tid < CH;
            const float g = mine ? cr.s : 0.0f;
            const float e = expf(g);      // the token's decay factor (1 past the chunk)
            float c = e;                  // inclusive prefix product over each row of 16
            c *= dpp_or<0x111>(1.0f, c);  // row_shr:1
            c *= dpp_or<0x112>(1.0f, c);  // row_shr:2
            c *= dpp_or<0x114>(1.0f, c);  // row_shr:4
            c *= dpp_or<0x118>(1.0f, c);  // row_shr:8
            // every lane of wave 0 takes part in the ballot and the reads
            const uint64_t bad = __ballot(!(g <= 0.0f));           // positive or NaN gates
            float last[CH / kScaleGroup];
#pragma unroll
            for (int gi = 0; gi < CH / kScaleGroup; ++gi) last[gi] = lane_value(c, gi * 16 + 15);
            if (mine) {
                TokenLds &tk = buf[tid];
                tk.e = e;
                tk.beta = cr.s2;
                tk.w = cr.s2 / c;
                tk.os = c * kInvSqrtD;
            }
            if (tid == 0) {
#pragma unroll
                for (int gi = 0; gi < CH / kScaleGroup; ++gi) {
                    const bool ok = ((bad >> (gi * 16)) & 0xFFFFu) == 0 && last[gi] >= kMinScale;
                    info[2 * gi] = ok ? 1.0f : 0.0f;
                    info[2 * gi + 1] = last[gi];
                }
            }
        }
    } else {
        if (tid < CH)
            buf[tid].e = expf(cr.s);      // the token's decay factor, computed once
        else if (tid < 2 * CH)
            buf[tid - CH].beta = cr.s;
    }
}

// Plain DPP move (no `old` operand to materialise); every lane of the
// patterns used here has a source lane, so none reads the bound value.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// group_sum() of two rows A and B at once, for a row group whose lanes hold
// both rows in swapped register slots: lanes 0-3 have A's partial in `own`
// and B's in `other`, lanes 4-7 the reverse.  Returns A's sum in lanes 0-3
// and B's in lanes 4-7, with group_sum()'s bits: the first level adds the
// same pairs of partials (lane i and lane 7-i), and the other two stay
// within lanes 0-3 or 4-7.
__device__ __forceinline__ float pair_sum(float own, float other) {
    float x = own + dpp<0x141>(other);
    x = x + dpp<0xB1>(x);
    x = x + dpp<0x4E>(x);
    return x;
}

// dst = s ? a : b, element by element.
__device__ __forceinline__ void select_row(RowSlice &dst, bool s, const RowSlice &a,
                                           const RowSlice &b) {
#pragma unroll
    for (int i = 0; i < kF4PerLane; ++i) {
        dst.m[i].x = s ? a.m[i].x : b.m[i].x;
        dst.m[i].y = s ? a.m[i].y : b.m[i].y;
        dst.m[i].z = s ? a.m[i].z : b.m[i].z;
        dst.m[i].w = s ? a.m[i].w : b.m[i].w;
    }
}

// pass() without the decay multiply (the scaled form).
__device__ __forceinline__ void pass_scaled(RowSlice &r, float d, const VecSlice &k,
                                            const VecSlice &q, const VecSlice &kn, float &o,
                                            float &p) {
    o = 0.0f;
    p = 0.0f;
#pragma unroll
    for (int i = 0; i < kF4PerLane; ++i) {
#define GDN_PASS_LANE(X)                          \
        r.m[i].X = fmaf(d, k.x[i].X, r.m[i].X);   \
        o = fmaf(r.m[i].X, q.x[i].X, o);          \
        p = fmaf(r.m[i].X, kn.x[i].X, p);
        GDN_PASS_LANE(x)
        GDN_PASS_LANE(y)
        GDN_PASS_LANE(z)
        GDN_PASS_LANE(w)
#undef GDN_PASS_LANE
    }
}

__device__ __forceinline__ void scale_row(RowSlice &r, float f) {
#pragma unroll
    for (int i = 0; i < kF4PerLane; ++i) {
        r.m[i].x *= f;
        r.m[i].y *= f;
        r.m[i].z *= f;
        r.m[i].w *= f;
    }
}

// Token tt of a chunk: correction, rank-1 update and read-out of tt and,
// when `next`, the decay and key product of tt+1
// (kv holds k of token tt on entry and of tt+1 on exit; p the key partials).
// kPair: a lane's two rows sit in swapped slots (slot 0 is row A in lanes 0-3
// of the row group and row B in lanes 4-7), so pair_sum() reduces both rows
// with one set of DPP adds, each lane computes the delta of its slot-0 row
// only and takes the other row's from its mirror lane, and writes one output.
// Otherwise each slot is reduced on its own.  Both give the same bits.
// kScaled: the registers hold S / c_t (scaled decay above); kFold: see below.
template <bool kPair, int TPW, bool kScaled, bool kFold = false>
__device__ __forceinline__ void seq_token(TokenLds *buf, int tt, bool next, const int (&rows)[TPW],
                                          RowSlice (&r)[TPW], VecSlice &kv, float (&p)[TPW],
                                          int c, float fold = 1.0f) {
    static_assert(!kPair || TPW == 2, "pairing needs two tiles per wave");
    TokenLds &tok = buf[tt];
    float d[TPW];                                              // correction
    if constexpr (kScaled) {
        // v w - ((S / c) . k) beta = (v - S . k) beta / c = delta / c
        if constexpr (kPair) {
            d[0] = fmaf(-pair_sum(p[0], p[1]), tok.beta, tok.v[rows[0]] * tok.w);
            d[1] = dpp_mov<0x141>(d[0]);
        } else {
#pragma unroll
            for (int t = 0; t < TPW; ++t) d[t] = fmaf(-group_sum(p[t]), tok.beta, tok.v[rows[t]] * tok.w);
        }
    } else if constexpr (kPair) {
        d[0] = (tok.v[rows[0]] - pair_sum(p[0], p[1])) * tok.beta;
        d[1] = dpp_mov<0x141>(d[0]);                           // from lane 7-c: the other row
    } else {
#pragma unroll
        for (int t = 0; t < TPW; ++t) d[t] = (tok.v[rows[t]] - group_sum(p[t])) * tok.beta;
    }
    const float oscale = kScaled ? tok.os : kInvSqrtD;
    VecSlice qv;
    load_vec(qv, tok.q, c);
    float o[TPW];
    if (next) {
        VecSlice kn;
        load_vec(kn, buf[tt + 1].k, c);
        const float en = buf[tt + 1].e;
        if constexpr (kFold) {
            // last token of a scaled group followed by another: the registers
            // take the group's c back (the same bits as body_part(), then
            // scale_row(), then the next group's dot_part())
#pragma unroll
            for (int t = 0; t < TPW; ++t) pass(r[t], d[t], kv, qv, fold, kn, o[t], p[t]);
        } else if constexpr (kScaled) {
#pragma unroll
            for (int t = 0; t < TPW; ++t) pass_scaled(r[t], d[t], kv, qv, kn, o[t], p[t]);
        } else {
#pragma unroll
            for (int t = 0; t < TPW; ++t) pass(r[t], d[t], kv, qv, en, kn, o[t], p[t]);
        }
        kv = kn;
    } else {
#pragma unroll
        for (int t = 0; t < TPW; ++t) o[t] = body_part(r[t], d[t], kv, qv);
    }
    // every lane holding a row in a written slot has the same output bits
    if constexpr (kPair) {
        tok.v[rows[0]] = pair_sum(o[0], o[1]) * oscale;
    } else {
#pragma unroll
        for (int t = 0; t < TPW; ++t) tok.v[rows[t]] = group_sum(o[t]) * oscale;
    }
}

// Tokens [0, nt) of the CH staged tokens at buf, with the per-token decay
// multiply: decay and key product of the first, then seq_token() for each;
// when nt == CH the loop is unrolled, so every LDS address is an immediate
// offset.
template <int CH, bool PAIR, int TPW>
__device__ __forceinline__ void seq_chunk(TokenLds *buf, int nt, const int (&rows)[TPW],
                                          RowSlice (&r)[TPW], int c) {
    VecSlice kv;
    load_vec(kv, buf[0].k, c);
    float p[TPW];
    const float e0 = buf[0].e;
#pragma unroll
    for (int t = 0; t < TPW; ++t) p[t] = head_part(r[t], kv, e0);
    if (nt == CH) {
#pragma unroll
        for (int tt = 0; tt < CH; ++tt)
            seq_token<PAIR, TPW, false>(buf, tt, tt + 1 < CH, rows, r, kv, p, c);
    } else {
        for (int tt = 0; tt < nt; ++tt)
            seq_token<PAIR, TPW, false>(buf, tt, tt + 1 < nt, rows, r, kv, p, c);
    }
}

// A complete group of kScaleGroup tokens with the scaled decay.  On entry
// the registers hold the state before the group's first token, which is
// S / c_0 of the decayed state (c_0 = e_0).  `carried`: kv and p already
// hold that token's key and key partials (the previous group folded with a
// pipelined pass).  `next_scaled`: the group after it (at buf[kScaleGroup],
// in the same chunk) runs scaled too; the last token then folds c back in
// with the next token's key product in the same sweep and leaves kv and p
// for it.  On exit the registers hold the state after the group.
template <bool PAIR, int TPW>
__device__ __forceinline__ void seq_group_scaled(TokenLds *buf, const float *info, bool carried,
                                                 bool next_scaled, const int (&rows)[TPW],
                                                 RowSlice (&r)[TPW], int c, VecSlice &kv,
                                                 float (&p)[TPW]) {
    constexpr int N = kScaleGroup;
    if (!carried) {
        load_vec(kv, buf[0].k, c);
#pragma unroll
        for (int t = 0; t < TPW; ++t) p[t] = dot_part(r[t], kv);
    }
#pragma unroll
    for (int tt = 0; tt < N - 1; ++tt) seq_token<PAIR, TPW, true>(buf, tt, true, rows, r, kv, p, c);
    const float last = info[1];
    if (next_scaled) {
        seq_token<PAIR, TPW, true, true>(buf, N - 1, true, rows, r, kv, p, c, last);
    } else {
        seq_token<PAIR, TPW, true>(buf, N - 1, false, rows, r, kv, p, c);
#pragma unroll
        for (int t = 0; t < TPW; ++t) scale_row(r[t], last);
    }
}

__device__ __forceinline__ bool group_scaled(const float *info, int gi) {
    return __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, info[2 * gi])) != 0;
}

// CH: tokens per LDS chunk; NT: nontemporal state load and store; PAIR:
// paired row reductions (seq_token); a head's 128 rows are split over PARTS
// workgroups of 16 / (TPW * PARTS) waves with TPW tiles each; WPS: waves per
// SIMD the register allocation must allow (3 caps it at 168 VGPRs); SC: the
// scaled decay; DMA: chunks go from global memory straight into LDS.
template <int CH, bool NT, bool PAIR, int PARTS, int WPS, int TPW = 2, bool SC = false, bool DMA = false>
__global__ __launch_bounds__(64 * 16 / (TPW * PARTS), WPS) void k_seq(SeqArgs a) {
    constexpr int NTH = 64 * 16 / (TPW * PARTS);
    constexpr int R = D / PARTS;                  // rows of this workgroup
    __shared__ TokenLds lds[2][CH];
    __shared__ float info[2][2 * (CH / 8)];       // per buffer, with SC (seq_stage)

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
    // The wave's TPW tiles.  The state moves in tile order (whole 128-byte
    // lines per instruction); with PAIR, lanes 4-7 of each row group swap
    // the two slots in registers, as seq_token() expects.  rows[] is per slot.
    // (Two-tile kernels keep the swap path even unpaired, where it swaps
    // nothing: the code it compiles to is the measured one.)
    const bool swap = PAIR && c >= 4;
    int tile_row[TPW], rows[TPW];
    RowSlice r[TPW];
    if constexpr (TPW == 2) {
        RowSlice m[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            tile_row[t] = part * R + (wave * 2 + t) * kRowsPerTile + grp;
            load_row<NT>(m[t], M + tile_row[t] * D, c);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            rows[t] = swap ? tile_row[t ^ 1] : tile_row[t];
            select_row(r[t], swap, m[t ^ 1], m[t]);
        }
    } else {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            tile_row[t] = part * R + (wave * TPW + t) * kRowsPerTile + grp;
            rows[t] = tile_row[t];
            load_row<NT>(r[t], M + tile_row[t] * D, c);
        }
    }

    ChunkRegs<CH, NTH, DMA> cr;
    fetch_chunk<CH, NTH, SC, DMA>(cr, lds[0], a, b, h, kh, 0, tid);
    seq_stage<CH, NTH, SC, DMA>(lds[0], info[0], cr, tid);
    if constexpr (DMA) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // this wave's transfers are in LDS
    __syncthreads();

    const int n_chunks = (a.T + CH - 1) / CH;
    for (int ch = 0; ch < n_chunks; ++ch) {
        const bool more = ch + 1 < n_chunks;
        if (more) fetch_chunk<CH, NTH, SC, DMA>(cr, lds[(ch + 1) & 1], a, b, h, kh, (ch + 1) * CH, tid);

        TokenLds *buf = lds[ch & 1];
        const int t0 = ch * CH;
        const int nt = min(CH, a.T - t0);

        if constexpr (SC) {
            // group by group: complete groups that pass the check run scaled
            constexpr int G = CH / kScaleGroup;
            const float *inf = info[ch & 1];
            VecSlice kv;
            float p[TPW];
            bool carried = false;
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                const int ng = min(kScaleGroup, nt - gi * kScaleGroup);
                if (ng <= 0) break;
                TokenLds *gb = buf + gi * kScaleGroup;
                if (ng == kScaleGroup && group_scaled(inf, gi)) {
                    const bool next_scaled = gi + 1 < G && nt - (gi + 1) * kScaleGroup >= kScaleGroup &&
                                             group_scaled(inf, gi + 1);
                    seq_group_scaled<PAIR, TPW>(gb, inf + 2 * gi, carried, next_scaled, rows, r, c, kv, p);
                    carried = next_scaled;
                } else {
                    seq_chunk<kScaleGroup, PAIR, TPW>(gb, ng, rows, r, c);
                    carried = false;
                }
            }
        } else if constexpr (CH < 32 && TPW == 2) {
            seq_chunk<CH, PAIR, TPW>(buf, nt, rows, r, c);
        } else {
            // seq_chunk()'s steps written out here: the long-sequence kernels
            // (32-token chunks, one-tile waves) compile to a faster schedule
            // this way (2-5 % at T = 1024-4096); the half-head kernels to a
            // faster one through seq_chunk() (4-6 % at T <= 64, many heads)
            VecSlice kv;
            load_vec(kv, buf[0].k, c);
            float p[TPW];
            {
                const float e0 = buf[0].e;
#pragma unroll
                for (int t = 0; t < TPW; ++t) p[t] = head_part(r[t], kv, e0);
            }
            if (nt == CH) {
#pragma unroll
                for (int tt = 0; tt < CH; ++tt)
                    seq_token<PAIR, TPW, false>(buf, tt, tt + 1 < CH, rows, r, kv, p, c);
            } else {
                for (int tt = 0; tt < nt; ++tt)
                    seq_token<PAIR, TPW, false>(buf, tt, tt + 1 < nt, rows, r, kv, p, c);
            }
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
        if (more) seq_stage<CH, NTH, SC, DMA>(lds[(ch + 1) & 1], info[(ch + 1) & 1], cr, tid);
        if constexpr (DMA) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // chunk ch+1's transfers
        __syncthreads();                 // chunk ch+1 staged; chunk ch flushed
    }
    if constexpr (TPW == 2) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            RowSlice m;
            select_row(m, swap, r[t ^ 1], r[t]);
            store_row<NT>(M + tile_row[t] * D, m, c);
        }
    } else {
#pragma unroll
        for (int t = 0; t < TPW; ++t) store_row<NT>(M + tile_row[t] * D, r[t], c);
    }
}

}  // namespace

// Launch shape (measured on MI355X, 256 CUs, 32 heads):
// - T = 1 runs the single-step kernel (in gdn_api.cpp).
// - At most CUs / 4 heads (B <= 2), any T: heads split into one-tile waves,
//   16 one-wave workgroups per head (B = 1) or 8 of two waves (B = 2), so a
//   wave's instruction stream per token is short; 8-token chunks with
//   nontemporal state access below 16 tokens, 16-token chunks and plain
//   access from there.  Against the half-head routes below, device time
//   per call (graph replays): B = 1 T = 2 4.44 -> 4.17 us, T = 8 6.26 ->
//   5.06, T = 15 9.42 -> 7.84, T = 64 24.7 -> 19.2; B = 2 7-17 % faster.
// - T <= 64: half heads (two workgroups of 4 waves, 64 rows each, per head),
//   so that several share a CU and one's state transfer overlaps the
//   others' arithmetic; nontemporal state access; 8-token chunks below 16
//   tokens, 16-token chunks from there.  Whole heads are 3-30 % slower here
//   except at B = 6..8 and T near 64 (up to 4 % faster; not special-cased).
//   With few heads, paired reductions: fewer instructions, and occupancy
//   does not matter.  With many, registers for three workgroups per CU
//   (168 VGPRs): the 8-token kernel unpaired (164; 180 paired), the
//   16-token kernel paired with its chunks fetched straight into LDS (DMA:
//   168 VGPRs, no spill; 194 with the chunk in registers).
//   Thresholds: T < 16, paired up to `CUs` heads (2-5 % faster at B <= 8,
//   5-25 % slower from B = 32); T >= 16, DMA and three per CU beyond `CUs`
//   heads (next item), two per CU with the chunk in registers up to `CUs`
//   heads (the DMA kernel measured equal or up to 3 % slower at B <= 8).
//   DMA measured equal or slower for T < 16.
// - 16 tokens or more with more heads than CUs, at any length: the DMA
//   half-head kernel, three workgroups (12 waves) per CU.  Against the
//   unpaired register-staged kernel held to 168 VGPRs (28 bytes of spill per
//   lane) at T <= 64: 5-14 % faster from B = 12 to 512.  Against whole heads
//   (next item, 8 waves per CU) beyond 64 tokens: 7-10 % faster where both
//   fill their rounds of workgroups alike (B = 24 T = 512 665 -> 596 us,
//   B = 40 T = 1024 2083 -> 1916), 20-31 % where whole heads leave most of a
//   round empty (B = 9 T = 4096 3383 -> 2347 us, B = 12 T = 2048 1643 ->
//   1192, B = 20 T = 2048 2490 -> 1989).  Whole heads stay where they fill
//   every round and the half heads do not (heads a multiple of CUs, twice
//   the heads not of 3 x CUs) beyond 1024 tokens: B = 16 T = 4096 3303
//   against 3560 us (at T = 1024 the half heads are 3 % ahead there).
// - Longer sequences with at most `CUs` heads: whole heads, one 8-wave
//   workgroup per head, 32-token chunks, plain state access, paired
//   reductions.  They are VALU-bound; half heads at two per CU duplicate the
//   staging without adding waves (40 % slower at B = 8, T = 4096; 1.72
//   against 1.67 ms with the DMA kernel).
//   With fewer heads than CUs, whole heads leave CUs idle, and a head is
//   split while the parts still fit the CUs:
//   - B = 1, 2: the one-tile splits above.  A lone wave on its SIMD issues
//     one instruction per 4 cycles, so halving its rows nearly halves its
//     instruction stream: 1.74 -> 1.07 ms at B = 1, T = 4096 (1.39 ms with
//     two tiles per wave); 1.76 -> 1.21 ms at B = 2 (1.40 ms with 4 parts of
//     two tiles);
//   - up to CUs / 2 heads (B = 3, 4): 2 parts of four two-tile waves (paired,
//     32-token chunks): 1.84 -> 1.47 ms at B = 4, T = 4096; one-tile parts
//     there measured 20 % slower, and two-tile splits no better than the
//     half-head routes below 65 tokens.
// - 16- and 32-token chunks run their groups with the scaled decay (SC):
//   per call, B = 8 T = 4096 1.77 -> 1.67 ms, B = 1 T = 4096 1.03 -> 0.93,
//   B = 4 T = 4096 1.36 -> 1.26, B = 64 T = 64 248 -> 219 us, B = 256
//   T = 64 1.00 -> 0.89 ms (graph replays).  Folding c once per 32 tokens
//   where a chunk has 32 was another 1-2 % faster but makes the bits depend
//   on the launch shape.  8-token chunks (T < 16) keep the per-token form,
//   and gdn_seq_exact (launch_seq's `exact`) runs every chunk per token.
static_assert(2 * 256 == kSeqThreadsPerHead && 512 == kSeqThreadsPerHead,
              "the API bounds B * Hv by this launch's work-items per head");

namespace {

// Workgroups of the DMA half-head kernel that fit on a CU: 168 VGPRs (three
// waves per SIMD) and 49 KiB of LDS.
constexpr int kDmaWgsPerCu = 3;

// SC: the 16- and 32-token kernels run qualifying groups scaled.
template <bool SC>
hipError_t launch_seq_as(const SeqArgs &a, hipStream_t s) {
    const int64_t heads = static_cast<int64_t>(a.B) * a.Hv;
    const int64_t cus = device_cus();
    const dim3 split(static_cast<unsigned>(heads * 2)), whole(static_cast<unsigned>(heads));
    if (8 * heads <= cus) {
        // 16 one-wave parts of one tile each (1024 work-items per head; taken
        // only for heads <= CUs / 8)
        const dim3 grid(static_cast<unsigned>(heads * 16)), block(64);
        if (a.T < 16)
            k_seq<8, true, false, 16, 1, 1><<<grid, block, 0, s>>>(a);
        else
            k_seq<16, false, false, 16, 1, 1, SC><<<grid, block, 0, s>>>(a);
    } else if (4 * heads <= cus) {
        // 8 two-wave parts of one tile per wave (1024 work-items per head;
        // heads <= CUs / 4)
        const dim3 grid(static_cast<unsigned>(heads * 8)), block(128);
        if (a.T < 16)
            k_seq<8, true, false, 8, 1, 1><<<grid, block, 0, s>>>(a);
        else
            k_seq<16, false, false, 8, 1, 1, SC><<<grid, block, 0, s>>>(a);
    } else if (a.T < 16) {
        if (heads <= cus)
            k_seq<8, true, true, 2, 1><<<split, dim3(256), 0, s>>>(a);
        else
            k_seq<8, true, false, 2, 1><<<split, dim3(256), 0, s>>>(a);
    } else if (heads > cus && !(a.T > 1024 && heads % cus == 0 &&
                                  (2 * heads) % (kDmaWgsPerCu * cus) != 0)) {
        k_seq<16, true, true, 2, kDmaWgsPerCu, 2, SC, true><<<split, dim3(256), 0, s>>>(a);
    } else if (a.T <= 64) {
        k_seq<16, true, true, 2, 1, 2, SC><<<split, dim3(256), 0, s>>>(a);
    } else if (2 * heads <= cus) {
        k_seq<32, false, true, 2, 1, 2, SC><<<split, dim3(256), 0, s>>>(a);
    } else {
        k_seq<32, false, true, 1, 1, 2, SC><<<whole, dim3(512), 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_seq(const SeqArgs &a, hipStream_t s, bool exact) {
    return exact ? launch_seq_as<false>(a, s) : launch_seq_as<true>(a, s);
}

}  // namespace gdn
