/*
 * gdn.h - C ABI of libgdn.so, the MI355X (gfx950) Gated DeltaNet decode path.
 *
 * Operation (Red Lite dev15c "Gated DeltaNet recurrent-state parity",
 * section "Pinned llama.cpp semantics"): for every sequence b and value head
 * h, with key head kh = h % n_k_heads, e = exp(gate[b][h]), beta = beta[b][h]
 * and the state kept transposed, M = S^T (row j = value coordinate, column
 * i = key coordinate; M[j][i] = S[i][j]), one token does
 *     M' = e M + beta (v - e M k) k^T,        out = M' q / sqrt(d_k)
 * with k = k[kh], q = q[kh], v = v[h]: the delta rule applied to the decayed
 * state, and the read-out taken from the new state.  The page's geometry is
 * d_k = d_v = 128, 16 key heads, 32 value heads, a 2 MiB F32 state per
 * sequence and layer.
 *
 * Conventions shared by every call
 *   - All tensors are float32 (IEEE binary32), row-major and contiguous.
 *   - Every pointer is a device pointer (hipMalloc'd or torch CUDA memory)
 *     that the caller owns; the library keeps no reference after the call.
 *   - Tensor pointers must be 16-byte aligned; per-head vectors (beta, gate,
 *     the raw gate inputs, conv_w, norm_w) 4-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls enqueue their kernels on it and return without synchronising.
 *   - Inputs are read-only; `state` and `conv_state` are updated in place.
 *     Outputs must not overlap any input or state buffer.
 *   - Supported on the GPU path: d_k = d_v = 128, n_k_heads >= 1,
 *     n_v_heads a multiple of n_k_heads, B >= 1, 1 <= T <= 1073741824,
 *     B * n_v_heads <= 134213631 (gdn_seq, gdn_seq_exact: <= 8388607).
 *     Launches must fit the dispatch's 32-bit work-item count; the limits
 *     here and in gdn_layer_tail guarantee it (a state that large would not
 *     fit in memory anyway).
 *   - Results are bitwise deterministic for identical inputs, independent of
 *     B and of the other sequences in the batch.  gdn_seq_exact over T
 *     tokens is bitwise equal to T calls of gdn_step; so is gdn_seq for
 *     T < 16 (longer calls: see gdn_seq).
 *   - NaN and Inf inputs are not checked; they propagate.
 *
 * Errors: every call returns GDN_OK (0) or a negative code.  Argument errors
 * are detected before anything is enqueued and leave every buffer untouched;
 * gdn_last_error() then returns a message describing the failure (thread
 * local, valid until the next call on the same thread).  GDN_ERR_HIP reports
 * a failed kernel launch (hipGetLastError); work already enqueued by that
 * call may have run.
 *
 * Thread safety: every call may be made concurrently from several host
 * threads.  The library's mutable global state is the thread-local error
 * text, a per-device cache of the compute-unit count and, for
 * gdn_layer_tail_noalloc only, a static per-GPU scratch array with a
 * per-device cache of its address (see there for the calls that share it).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_VERSION 10300 /* 1.3.0 */

#define GDN_OK 0
#define GDN_ERR_NULL (-1)      /* a required pointer is NULL                  */
#define GDN_ERR_SHAPE (-2)     /* unsupported sizes (B, T, heads, dims, tail) */
#define GDN_ERR_ALIGN (-3)     /* a pointer is not suitably aligned           */
#define GDN_ERR_ALIAS (-4)     /* an output overlaps an input or a state      */
#define GDN_ERR_WORKSPACE (-5) /* workspace missing or too small              */
#define GDN_ERR_HIP (-6)       /* the HIP runtime reported a launch error     */

/* Head geometry.  The page's model: {32, 16, 128, 128}. */
typedef struct gdn_dims {
    int32_t n_v_heads; /* value / recurrent heads                   */
    int32_t n_k_heads; /* key / query heads; value head h uses h % n_k_heads */
    int32_t d_k;       /* key dimension (state row length)          */
    int32_t d_v;       /* value dimension (state rows per head)     */
} gdn_dims;

/* Tail parameters.  The page's model: {4, 128, 1e-6f, 0}. */
typedef struct gdn_tail_params {
    int32_t conv_kernel;   /* causal conv1d taps, 2..8; cache holds conv_kernel-1 inputs */
    int32_t norm_group;    /* gated RMSNorm group size; must divide n_v_heads*d_v        */
    float norm_eps;        /* added to mean(o^2) inside the square root, >= 0            */
    int32_t force_unfused; /* 0: one launch when supported (conv_kernel 4, norm_group
                              = d_v, n_v_heads = n_k_heads or 2*n_k_heads), otherwise
                              three; non-zero: always three launches.  Both give the
                              same bits.                                                */
} gdn_tail_params;

/*
 * gdn_step - one token for B sequences (dev15c, the update above).
 *   q, k   [B][n_k_heads][d_k]   (L2-normalised by the caller)
 *   v      [B][n_v_heads][d_v]
 *   beta   [B][n_v_heads]        update strength, used as given
 *   gate   [B][n_v_heads]        log-decay; the step applies exp()
 *   state  [B][n_v_heads][d_v][d_k]   transposed state M, updated in place
 *   out    [B][n_v_heads][d_v]
 * Each state element is read once and written once.
 */
int gdn_step(const gdn_dims *dims, int32_t B,
             const float *q, const float *k, const float *v,
             const float *beta, const float *gate,
             float *state, float *out, void *stream);

/* gdn_step_ex flags */
#define GDN_STATE_CACHED 1u /* state through the caches instead of streamed */

/*
 * gdn_step_ex - gdn_step with a cache-policy hint for the state.
 *   flags  0: as gdn_step (the state is streamed with nontemporal loads and
 *             stores, which keeps it from displacing other data: right when
 *             the states a decode loop cycles through exceed the GPU's
 *             256 MB Infinity Cache, e.g. many layers of a large batch);
 *          GDN_STATE_CACHED: state loads and stores use the default cache
 *             policy, for callers whose whole working set of states stays
 *             resident in the Infinity Cache from call to call (e.g. one
 *             128 MiB state stepped repeatedly).
 * Results are bitwise equal for both policies.  Unknown flag bits:
 * GDN_ERR_SHAPE.  Other arguments, layouts and errors as gdn_step.
 */
int gdn_step_ex(const gdn_dims *dims, int32_t B,
                const float *q, const float *k, const float *v,
                const float *beta, const float *gate,
                float *state, float *out, uint32_t flags, void *stream);

/*
 * gdn_seq - T tokens for B sequences, run in order with the state carried
 * (docs.rs "Module linear_core", gdn_forward_batch: the recurrence runs
 * over the positions one after another, with the same elementwise results
 * as single steps).
 *   q, k   [B][T][n_k_heads][d_k]
 *   v      [B][T][n_v_heads][d_v]
 *   beta, gate [B][T][n_v_heads]
 *   state  [B][n_v_heads][d_v][d_k]   in: state before token 0, out: after T-1
 *   out    [B][T][n_v_heads][d_v]
 * The state stays on chip for all T tokens: it is read once and written once
 * per call.
 * Tokens are taken in groups of 16 counted from token 0.  A complete group
 * whose gates are all <= 0 and whose decay product (the product of
 * exp(gate) over the group) is at least 2^-63 runs with the decay carried
 * as one scale c for the whole state, which holds S / c during the group:
 * the step's arithmetic without the decay multiply on each state element,
 * rounded differently from gdn_step (the same recurrence to float32
 * rounding, not the same bits).  Every other group, and a trailing partial
 * one, multiplies per token as gdn_step does: a call in which no group
 * qualifies (T < 16, or decay stronger than that floor) is bitwise equal to
 * T gdn_step calls.  Splitting T into consecutive calls at multiples of 16
 * tokens gives bitwise the same result.  Inside a scaled group the state is
 * held up to 2^63.5 times larger, so states or values beyond about 1e19 in
 * magnitude overflow there; gdn_seq_exact has the full float32 range.
 */
int gdn_seq(const gdn_dims *dims, int32_t B, int32_t T,
            const float *q, const float *k, const float *v,
            const float *beta, const float *gate,
            float *state, float *out, void *stream);

/*
 * gdn_seq_exact - gdn_seq with no scaled groups: every token multiplies the
 * decay into the state as gdn_step does, so the results are bitwise equal to
 * T gdn_step calls at any T, and to any split of T into consecutive calls
 * (docs.rs "Module linear_core", gdn_forward_batch: elementwise identical to
 * single steps).  Same arguments, layout, limits and errors as gdn_seq; on
 * long sequences it is 5-12 % slower.
 */
int gdn_seq_exact(const gdn_dims *dims, int32_t B, int32_t T,
                  const float *q, const float *k, const float *v,
                  const float *beta, const float *gate,
                  float *state, float *out, void *stream);

/*
 * gdn_pair - two consecutive positions for B sequences, fused for speculative
 * verification (docs.rs "Module linear_core", gdn_pair: the first position's
 * update is kept, the second's is held aside until the draft is accepted or
 * rejected).  Position 1 advances `state`
 * in place (committed); position 2 advances the committed state into
 * `state_next` (tentative: the caller adopts it on acceptance, e.g. by
 * swapping the buffers, or drops it on rejection).
 *   q, k        [B][2][n_k_heads][d_k]     position 1 then position 2
 *   v           [B][2][n_v_heads][d_v]
 *   beta, gate  [B][2][n_v_heads]
 *   state       [B][n_v_heads][d_v][d_k]   in: before position 1, out: after it
 *   state_next  [B][n_v_heads][d_v][d_k]   out: after position 2 (caller-owned)
 *   out         [B][2][n_v_heads][d_v]
 * The state is read once and written twice.  Results are bitwise equal to
 * gdn_step on position 1 and to gdn_seq over both positions.
 */
int gdn_pair(const gdn_dims *dims, int32_t B,
             const float *q, const float *k, const float *v,
             const float *beta, const float *gate,
             float *state, float *state_next, float *out, void *stream);

/*
 * gdn_layer_tail - the recurrent branch around the step for one token
 * (Red Lite dev15e "complete recurrent DeltaNet layer composition", stage
 * list; dev15a "Validation boundary", prestate order), with C = 2*n_k_heads*d_k
 * + n_v_heads*d_v channels (8192 for the page's model):
 *   1. conv-state shift + causal conv1d over the window
 *      [conv_state slot 0 .. slot K-2, x] (oldest first, tap t on window
 *      element t, no bias); conv_state then holds the last K-1 raw inputs;
 *   2. SiLU;  3. split [Q | K | V];  4. per-head L2 norm of Q and K
 *      (u / max(||u||, 1e-6));  5. gdn_step;
 *   6. gated RMSNorm: y = o / sqrt(mean_group(o^2) + eps) * norm_w[pos] * SiLU(z).
 *   x          [B][C]          raw pre-conv channels
 *   conv_w     [C][conv_kernel]
 *   conv_state [B][conv_kernel-1][C]   in/out
 *   beta, gate [B][n_v_heads]
 *   state      [B][n_v_heads][d_v][d_k] in/out
 *   z          [B][n_v_heads*d_v]
 *   norm_w     [norm_group]
 *   y          [B][n_v_heads*d_v]      output
 *   dbg_qkv    [B][C] optional (NULL = skip): normalised Q | K | V fed to the step
 *   dbg_core   [B][n_v_heads][d_v] optional: step output before the gated norm
 *   workspace  device scratch of gdn_layer_tail_workspace_bytes() bytes
 *              (16-byte aligned), used only by the three-launch path: it
 *              may be NULL (workspace_bytes 0) when the single launch
 *              applies (see gdn_tail_params) or both dbg buffers are given
 * Size limits (GDN_ERR_SHAPE beyond): B * C <= 1073741823 and
 * B * n_v_heads * d_v / norm_group <= 33554431 (gated-norm groups).
 */
int gdn_layer_tail(const gdn_dims *dims, const gdn_tail_params *params, int32_t B,
                   const float *x, const float *conv_w, float *conv_state,
                   const float *beta, const float *gate, float *state,
                   const float *z, const float *norm_w, float *y,
                   float *dbg_qkv, float *dbg_core,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_layer_tail_pair - gdn_layer_tail for two consecutive positions fused
 * for speculative verification (docs.rs "Module linear_core", gdn_pair: the
 * first position's update is kept, the second's is held aside, and the
 * conv ring is held aside with the recurrent state).  Position 1 advances
 * `conv_state` and `state` in place (committed); position 2 starts from the
 * committed ring and state and writes its ring to `conv_state_next` and its
 * state to `state_next` (tentative: the caller adopts both on acceptance,
 * e.g. by swapping the buffers, or drops them on rejection).
 *   x            [B][2][C]              raw pre-conv channels, position 1 then 2
 *   conv_w       [C][conv_kernel]
 *   conv_state   [B][conv_kernel-1][C]  in: before position 1, out: after it
 *   conv_state_next [B][conv_kernel-1][C]  out: after position 2
 *   beta, gate   [B][2][n_v_heads]
 *   state        [B][n_v_heads][d_v][d_k]  in: before position 1, out: after it
 *   state_next   [B][n_v_heads][d_v][d_k]  out: after position 2
 *   z            [B][2][n_v_heads*d_v]
 *   norm_w       [norm_group]
 *   y            [B][2][n_v_heads*d_v]  output of both positions
 * One launch; supports the single-launch geometry only (conv_kernel 4,
 * norm_group = d_v, n_v_heads = n_k_heads or 2*n_k_heads; GDN_ERR_SHAPE
 * otherwise; force_unfused is ignored) and needs no workspace.  The state is
 * read once and written twice, and so is the conv ring.  Results are bitwise
 * equal to gdn_layer_tail on position 1 followed by gdn_layer_tail on
 * position 2 (on copies of the committed ring and state).
 * Size limit (GDN_ERR_SHAPE beyond): B * 2 * C <= 1073741823.
 */
int gdn_layer_tail_pair(const gdn_dims *dims, const gdn_tail_params *params, int32_t B,
                        const float *x, const float *conv_w, float *conv_state,
                        float *conv_state_next, const float *beta, const float *gate,
                        float *state, float *state_next, const float *z,
                        const float *norm_w, float *y, void *stream);

/* Bytes of workspace the three-launch path of gdn_layer_tail needs when no
 * dbg buffer is given: enough for every path (0 on invalid arguments). */
size_t gdn_layer_tail_workspace_bytes(const gdn_dims *dims, int32_t B);

/*
 * Raw inputs of the beta/alpha parameter transforms (Red Lite dev15a,
 * "Validation boundary": the stage before the recurrent update;
 * "DeltaNet projection parity - real layer 0": the beta/alpha projection has
 * 64 outputs per token, two per value head).
 *   ba       [B][2*n_v_heads]  projection outputs: the n_v_heads beta logits,
 *                              then the n_v_heads alpha logits
 *   a_log    [n_v_heads]       per-head log decay rate
 *   dt_bias  [n_v_heads]       per-head bias of the alpha logit
 */
typedef struct {
    const float *ba;
    const float *a_log;
    const float *dt_bias;
} gdn_gate_inputs;

/*
 * gdn_gate_transform - beta and gate from the raw inputs:
 *   beta[b][h] = 1 / (1 + exp(-ba[b][h]))
 *   gate[b][h] = -exp(a_log[h]) * softplus(ba[b][n_v_heads + h] + dt_bias[h]),
 *   softplus(x) = log(1 + exp(x)).
 * The pages name these transforms but print no formula; this is the
 * Mamba-2 style gating of the Gated DeltaNet paper (sigmoid write strength,
 * log-decay -exp(A_log) * softplus(alpha + dt_bias)).  gate <= 0, so the
 * per-token decay exp(gate) lies in (0, 1].  Computed in binary32.
 *   beta, gate [B][n_v_heads] outputs (must not overlap the inputs)
 */
int gdn_gate_transform(const gdn_dims *dims, int32_t B, const gdn_gate_inputs *in,
                       float *beta, float *gate, void *stream);

/*
 * gdn_layer_tail_ba - gdn_layer_tail with beta and gate computed from the
 * raw gate inputs as in gdn_gate_transform (the whole recurrent branch of
 * one token from the projection outputs x, ba and z to y).  Arguments as in
 * gdn_layer_tail; the three-launch path needs a workspace of
 * gdn_layer_tail_ba_workspace_bytes() bytes, of which it uses the last
 * 2*B*n_v_heads floats for beta and gate (the single launch needs none, so
 * the workspace may then be NULL).  Results are bitwise equal to
 * gdn_gate_transform followed by gdn_layer_tail.
 */
int gdn_layer_tail_ba(const gdn_dims *dims, const gdn_tail_params *params, int32_t B,
                      const float *x, const float *conv_w, float *conv_state,
                      const gdn_gate_inputs *gates, float *state,
                      const float *z, const float *norm_w, float *y,
                      float *dbg_qkv, float *dbg_core,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace the three-launch path of gdn_layer_tail_ba needs when
 * no dbg buffer is given: enough for every path (0 on invalid arguments). */
size_t gdn_layer_tail_ba_workspace_bytes(const gdn_dims *dims, int32_t B);

/* Size of the static scratch of gdn_layer_tail_noalloc, per GPU. */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * gdn_layer_tail_noalloc - gdn_layer_tail without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Where the
 * three-launch path needs staging (it runs when the single launch does not
 * apply or force_unfused is set, and no dbg buffers are given), it uses a
 * static scratch array of GDN_NOALLOC_SCRATCH_BYTES that each GPU holds from
 * the first such call until the process ends; the single launch needs none.
 * The call allocates nothing.  Arguments, results (bitwise) and errors are
 * those of gdn_layer_tail, plus GDN_ERR_WORKSPACE, before anything is
 * enqueued, when the staging would exceed the scratch
 * (gdn_layer_tail_workspace_bytes(dims, B) > GDN_NOALLOC_SCRATCH_BYTES: B >
 * 341 at the page geometry on the three-launch path), and GDN_ERR_HIP if the
 * scratch's address cannot be obtained.  Every call on one GPU shares the
 * scratch, which keeps the last call's contents: calls that overlap on one
 * GPU (on different streams, or from threads without ordering between them)
 * race when they take the three-launch path; calls on one stream do not.
 * The first call on a device looks the scratch's address up
 * (hipGetSymbolAddress): a caller that captures the call into a HIP graph
 * makes one call before capturing.
 */
int gdn_layer_tail_noalloc(const gdn_dims *dims, const gdn_tail_params *params, int32_t B,
                           const float *x, const float *conv_w, float *conv_state,
                           const float *beta, const float *gate, float *state,
                           const float *z, const float *norm_w, float *y,
                           float *dbg_qkv, float *dbg_core, void *stream);

/* Message for the last non-zero return on this thread ("" if none). */
const char *gdn_last_error(void);

/* GDN_VERSION of the loaded library. */
int gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
