// gdn_launch.hpp - internal interface between the C-ABI layer (gdn_api.cpp)
// and the gfx950 kernels (gdn_step.hip, gdn_seq.hip, gdn_tail.hip).  Not
// installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace gdn {

// Only head size supported by the kernels: d_k = d_v = 128 (the page's model).
constexpr int kHeadDim = 128;

// One token of the state step for B sequences.  q/k/v may live inside a larger
// per-sequence row (the layer tail reads them from its [B][C] buffer), hence
// the explicit per-sequence strides (in floats).
struct StepArgs {
    const float *q;
    const float *k;
    const float *v;
    const float *beta;
    const float *gate;
    float *state;
    float *out;
    int64_t qk_bstride;  // floats between sequences in q and k
    int64_t v_bstride;   // floats between sequences in v
    int32_t B;
    int32_t Hv;
    int32_t Hk;
};

struct SeqArgs {
    const float *q;
    const float *k;
    const float *v;
    const float *beta;
    const float *gate;
    float *state;
    float *out;
    int32_t B;
    int32_t T;
    int32_t Hv;
    int32_t Hk;
};

// Two positions: position 1 commits into `state`, position 2 (computed from
// the committed state) goes to `state_next`.  q/k [B][2][Hk][D], v/out
// [B][2][Hv][D], beta/gate [B][2][Hv].
struct PairArgs {
    const float *q;
    const float *k;
    const float *v;
    const float *beta;
    const float *gate;
    float *state;
    float *state_next;
    float *out;
    int32_t B;
    int32_t Hv;
    int32_t Hk;
};

// conv-state shift + causal conv1d + SiLU + per-head L2 of the Q and K parts.
struct PrestateArgs {
    const float *x;
    const float *conv_w;
    float *conv_state;
    float *qkv;        // [B][C] output
    int32_t B;
    int32_t C;
    int32_t K;
    int32_t n_qk;      // channels of Q plus K (2 * Hk * d_k); these get L2-normalised
};

// Threads per workgroup of the gated-norm kernel (one workgroup per sequence
// and group); the API checks that its launch fits the 32-bit dispatch grid.
constexpr int kGatedNormThreads = 128;

// Work-items of a gdn_seq launch per head (two 256-thread halves or one
// 512-thread workgroup).
constexpr int kSeqThreadsPerHead = 512;

struct GatedNormArgs {
    const float *o;
    const float *z;
    const float *w;
    float *y;
    int32_t rows;
    int32_t n;
    int32_t group;
    float eps;
};

// beta/alpha parameter transforms: beta, gate [B][Hv] from the raw projection
// ba [B][2*Hv] ([beta logits | alpha logits]) and a_log, dt_bias [Hv].
struct GateArgs {
    const float *ba;
    const float *a_log;
    const float *dt_bias;
    float *beta;
    float *gate;
    int32_t B;
    int32_t Hv;
};

// The whole tail in one launch (one workgroup per sequence and key head).
// beta/gate are used as given, or, when ba is set, computed in the kernel
// from ba, a_log and dt_bias as in GateArgs.  The pair (launch_tail_pair)
// takes two positions per sequence: x [B][2][C], beta/gate [B][2][Hv],
// z/y [B][2][Hv*D]; position 1 commits conv_state and state, position 2
// writes conv_state_next and state_next.
struct TailFusedArgs {
    const float *x;
    const float *conv_w;
    float *conv_state;
    float *conv_state_next;   // pair only
    const float *beta;
    const float *gate;
    const float *ba;       // optional raw gate inputs (then beta/gate are unused)
    const float *a_log;
    const float *dt_bias;
    float *state;
    float *state_next;        // pair only
    const float *z;
    const float *norm_w;
    float *y;
    float *dbg_qkv;    // optional
    float *dbg_core;   // optional
    int32_t B;
    int32_t Hv;
    int32_t Hk;
    int32_t C;
    int32_t K;
    float eps;
};

// Bytes of the per-GPU static scratch array of gdn_layer_tail_noalloc.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;

// The device address of that array on the current device, looked up with
// hipGetSymbolAddress on the first call per device and cached.
hipError_t noalloc_scratch(void **ptr);

// True when launch_tail_fused and launch_tail_pair have a kernel for these
// sizes: value heads per key head 1 or 2 (Hv a multiple of Hk, Hk >= 1, as
// the ABI checks first), conv kernel 4, gated-norm group equal to the head
// dimension.
inline bool tail_fused_supported(int32_t Hv, int32_t Hk, int32_t K, int32_t group) {
    return (Hv == Hk || Hv == 2 * Hk) && K == 4 && group == kHeadDim;
}

// Compute units of the current device, read once per device and cached
// (256 on MI355X; 256 too if the query fails).
int device_cus();

// cached: state loads and stores with the default cache policy instead of
// nontemporal ones (same arithmetic, same bits).
hipError_t launch_step(const StepArgs &a, hipStream_t s, bool cached = false);
hipError_t launch_tail_fused(const TailFusedArgs &a, hipStream_t s);
hipError_t launch_tail_pair(const TailFusedArgs &a, hipStream_t s);
// exact: every token multiplies the decay into the state (no scaled groups).
hipError_t launch_seq(const SeqArgs &a, hipStream_t s, bool exact);
hipError_t launch_pair(const PairArgs &a, hipStream_t s);
hipError_t launch_prestate(const PrestateArgs &a, hipStream_t s);
hipError_t launch_gated_norm(const GatedNormArgs &a, hipStream_t s);
hipError_t launch_gate_transform(const GateArgs &a, hipStream_t s);

}  // namespace gdn
