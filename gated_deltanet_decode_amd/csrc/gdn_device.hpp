// gdn_device.hpp - device-side building blocks shared by every gfx950 kernel
// of the decode path: the row layout, the DPP reduction and the per-row
// arithmetic of the state update.  Included by the kernel sources only.
//
// The per-token update (Red Lite dev15c, "Pinned llama.cpp semantics") on the
// transposed state M = S^T (M[j][i] = S[i][j]), with e = exp(gate):
//   M' = e M + beta (v - e M k) k^T,   out = M' q / sqrt(128).
// Row j of it, the unit every kernel here works on: the decay of the row,
// its key product sk = (e M[j]) . k, the correction delta = (v[j] - sk) beta,
// the rank-1 update e M[j] + delta k, and the read-out M'[j] . q / sqrt(128).
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
// All kernels share this arithmetic (row_token() or the parts it is split
// into below), so a row's arithmetic is the same in the single-step kernel,
// the multi-token kernels and the tail: gdn_seq_exact over T tokens is
// bitwise equal to T gdn_step calls, and so is gdn_seq wherever it does not
// carry a 16-token group's decay as one scale (the scaled-decay note in
// gdn_seq.hip says when it does).
//
// No MFMA: the update is a sequence of rank-1 updates and matrix-vector
// products (one multiply-add per state element per operation), which is
// memory-bound in the one-token case and VALU-bound when the state is held
// on chip.
#pragma once

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

// The rank-1 update alone: M[j] += d k^T on this lane's columns.
__device__ __forceinline__ void update_part(RowSlice &r, float d, const VecSlice &k) {
#pragma unroll
    for (int i = 0; i < kF4PerLane; ++i) {
        r.m[i].x = fmaf(d, k.x[i].x, r.m[i].x);
        r.m[i].y = fmaf(d, k.x[i].y, r.m[i].y);
        r.m[i].z = fmaf(d, k.x[i].z, r.m[i].z);
        r.m[i].w = fmaf(d, k.x[i].w, r.m[i].w);
    }
}

// One token on one state row j: decay, key product, correction, rank-1
// update, then the read-out from the updated row.
// Returns out[j].
__device__ __forceinline__ float row_token(RowSlice &r, const VecSlice &k, const VecSlice &q,
                                           float e, float beta, float vj) {
#pragma unroll
    for (int i = 0; i < kF4PerLane; ++i) {           // decay
        r.m[i].x *= e;
        r.m[i].y *= e;
        r.m[i].z *= e;
        r.m[i].w *= e;
    }
    const float sk = group_sum(dot_part(r, k));       // key product M[j] . k
    const float d = (vj - sk) * beta;                 // correction delta
    update_part(r, d, k);                             // rank-1 update
    return group_sum(dot_part(r, q)) * kInvSqrtD;     // read-out, updated row
}

// The same arithmetic split into parts, for kernels that interleave it with
// memory traffic or with the next token: head_part() is the decay and key
// partial of a token, update_part() its rank-1 update, body_part() the rank-1
// update and read-out partial, and pass() the rank-1 update and read-out of
// token t with the decay and key partial of token t+1 in one sweep
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

// Rank-1 update and read-out of token t (delta d, k, q), then the decay and
// key product of token t+1 (decay en, key kn): this lane's output partial of
// t goes to o, its key partial of t+1 to p.
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

}  // namespace
}  // namespace gdn
