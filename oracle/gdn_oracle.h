/*
 * gdn_oracle.h - plain C99 CPU oracle for the Gated DeltaNet recurrent-state
 * step and the recurrent-branch tail around it.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the yardstick the HIP path is
 * checked against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  The product library never calls it, and the
 * two share no source, header, table or helper.
 *
 * Sources (the pages this follows; cited by page title and section):
 *   [dev15c]  "Red Lite dev15c - Gated DeltaNet recurrent-state parity",
 *             sections "Scope" (geometry) and "Pinned llama.cpp semantics"
 *             (head broadcast, transposed layout, the per-token update,
 *             output from the updated state).
 *   [dev15e]  "Red Lite dev15e - complete recurrent DeltaNet layer
 *             composition", the stage list at the top of the page and
 *             "M4 field result" (geometry, cache sizes).
 *   [dev15a]  "Red Lite dev15a - DeltaNet projection field validation",
 *             "Validation boundary" (order of the prestate stages) and
 *             "DeltaNet projection parity - real layer 0" (RMS epsilon).
 *   [linear_core] docs.rs "Module linear_core" (cortiq_engine), functions
 *             gdn_forward / gdn_forward_batch (a call moves the state on by
 *             one position; the batch form takes the positions one after
 *             another and gives the single-position results element for
 *             element), gdn_pair.
 *
 * Precision: the pages fix F32 for the state, the vectors and the conv path,
 * so the authority functions compute in binary32 with sequential sums and no
 * contraction (the library is built with -ffp-contract=off, no fast-math).
 * oracle_gdn_step_f64 is a binary64 shadow used only as an error yardstick.
 *
 * Every function here is pinned by CPU tests to facts other than itself
 * (closed forms, invariants, brute force, exact dyadic arithmetic, the pages'
 * printed geometry); none is "parity unpinned".
 *
 * Layouts (all row-major, contiguous, caller-owned):
 *   q, k   [B][Hk][dk]          (seq: [B][T][Hk][dk])
 *   v      [B][Hv][dv]          (seq: [B][T][Hv][dv])
 *   beta   [B][Hv]              (seq: [B][T][Hv])   post-transform, used as is
 *   gate   [B][Hv]              (seq: [B][T][Hv])   log-decay; exp() applied here
 *   M      [B][Hv][dv][dk]      transposed state, M[j][i] = S[i][j]
 *   S      [B][Hv][dk][dv]      non-transposed state (oracle_gdn_step_S only)
 *   out    [B][Hv][dv]          (seq: [B][T][Hv][dv])
 *   delta  [B][Hv][dv]          optional debug output: the correction
 *                               coefficient beta (v - e M k); NULL = skip
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* [dev15c] one token on the transposed state M (the authority):
 *   M' = e M + beta (v - e M k) k^T, out = M' q / sqrt(dk), e = exp(gate). */
void oracle_gdn_step_M(int32_t B, int32_t Hv, int32_t Hk, int32_t dk, int32_t dv,
                       const float *q, const float *k, const float *v,
                       const float *beta, const float *gate,
                       float *M, float *out, float *delta);

/* [dev15c] the same token written on the non-transposed state S[i][j]. */
void oracle_gdn_step_S(int32_t B, int32_t Hv, int32_t Hk, int32_t dk, int32_t dv,
                       const float *q, const float *k, const float *v,
                       const float *beta, const float *gate,
                       float *S, float *out, float *delta);

/* [dev15c] binary64 shadow of oracle_gdn_step_M: f32 inputs promoted, state
 * and output in double. */
void oracle_gdn_step_f64(int32_t B, int32_t Hv, int32_t Hk, int32_t dk, int32_t dv,
                         const float *q, const float *k, const float *v,
                         const float *beta, const float *gate,
                         double *M, double *out);

/* [linear_core] the binary64 shadow over T positions in order (state and
 * outputs in double; f32 inputs promoted), used as the error yardstick of
 * long sequences. */
void oracle_gdn_seq_f64(int32_t B, int32_t T, int32_t Hv, int32_t Hk, int32_t dk, int32_t dv,
                        const float *q, const float *k, const float *v,
                        const float *beta, const float *gate,
                        double *M, double *out);

/* [linear_core] gdn_forward_batch: T positions in order, state carried. */
void oracle_gdn_seq(int32_t B, int32_t T, int32_t Hv, int32_t Hk, int32_t dk, int32_t dv,
                    const float *q, const float *k, const float *v,
                    const float *beta, const float *gate,
                    float *M, float *out);

/* [linear_core] gdn_pair: two positions fused for speculative verification.
 * Position 1 commits into M; position 2 starts from that committed state and
 * its state goes to M_next (tentative), leaving M as after position 1.
 *   q, k [B][2][Hk][dk]; v [B][2][Hv][dv]; beta, gate [B][2][Hv]
 *   M [B][Hv][dv][dk] in/out; M_next [B][Hv][dv][dk] out; out [B][2][Hv][dv] */
void oracle_gdn_pair(int32_t B, int32_t Hv, int32_t Hk, int32_t dk, int32_t dv,
                     const float *q, const float *k, const float *v,
                     const float *beta, const float *gate,
                     float *M, float *M_next, float *out);

/* [dev15a] the conv stage of the prestate for one token: shift of the conv
 * cache, causal conv1d with the F32 weights, then SiLU.
 *   x          [B][C]        raw pre-conv channels of this token
 *   conv_w     [C][K]        tap 0 is applied to the oldest input
 *   conv_state [B][K-1][C]   slot 0 = oldest; in/out (shifted by one)
 *   act        [B][C]        SiLU(conv) */
void oracle_conv_silu(int32_t B, int32_t C, int32_t K,
                      const float *x, const float *conv_w, float *conv_state,
                      float *act);

/* [dev15a, Validation boundary] the L2 norm stage of the Q and K heads: each
 * of the n rows of length d is divided by its Euclidean norm (floored at
 * 1e-6).  In place. */
void oracle_l2norm_rows(int32_t n, int32_t d, float *u);

/* [dev15e] the tail's normalisation: RMSNorm per group, scaled by the norm
 * weight and gated by SiLU(z).
 *   o, z, y [rows][n]; the norm runs over consecutive groups of `group`
 *   elements; w [group] is indexed by the position inside the group.
 *   y = o / sqrt(mean(o^2) + eps) * w * SiLU(z). */
void oracle_gated_rmsnorm(int32_t rows, int32_t n, int32_t group, float eps,
                          const float *o, const float *z, const float *w,
                          float *y);

/* [dev15e] recurrent-branch tail for one token, stages in page order:
 * conv-state shift + conv1d + SiLU; the channels cut into contiguous
 * [Q | K | V]; each Q and K head scaled to unit L2 norm; the state update;
 * gated RMSNorm x SiLU(z).
 *   x [B][C] with C = 2*Hk*dk + Hv*dv; conv_w [C][K]; conv_state [B][K-1][C]
 *   beta, gate [B][Hv]; M [B][Hv][dv][dk]; z, y [B][Hv*dv]; norm_w [group]
 *   qkv_out  [B][C]        optional: normalized Q | K | V fed to the step
 *   core_out [B][Hv][dv]   optional: step output before the gated norm */
void oracle_layer_tail(int32_t B, int32_t Hv, int32_t Hk, int32_t dk, int32_t dv,
                       int32_t K, int32_t group, float eps,
                       const float *x, const float *conv_w, float *conv_state,
                       const float *beta, const float *gate, float *M,
                       const float *z, const float *norm_w, float *y,
                       float *qkv_out, float *core_out);

/* [linear_core] gdn_pair over the whole tail, conv ring and state together:
 * position 1 commits conv ring and state; position 2 runs from the committed
 * ones and writes its ring and state to the tentative buffers.
 *   x [B][2][C]; beta, gate [B][2][Hv]; z, y [B][2][Hv*dv]
 *   conv_state [B][K-1][C] in/out; conv_state_next [B][K-1][C] out
 *   M [B][Hv][dv][dk] in/out; M_next [B][Hv][dv][dk] out */
void oracle_layer_tail_pair(int32_t B, int32_t Hv, int32_t Hk, int32_t dk, int32_t dv,
                            int32_t K, int32_t group, float eps,
                            const float *x, const float *conv_w,
                            float *conv_state, float *conv_state_next,
                            const float *beta, const float *gate,
                            float *M, float *M_next,
                            const float *z, const float *norm_w, float *y);

/* [dev15a] beta/alpha parameter transforms (the pages name them; the
 * formula is a reading, see the definition):
 *   beta[b][h] = sigmoid(ba[b][h]),
 *   gate[b][h] = -exp(a_log[h]) * softplus(ba[b][Hv + h] + dt_bias[h]).
 * ba [B][2*Hv]; a_log, dt_bias [Hv]; beta, gate [B][Hv]. */
void oracle_gate_transform(int32_t B, int32_t Hv, const float *ba, const float *a_log,
                           const float *dt_bias, float *beta, float *gate);

#ifdef __cplusplus
}
#endif

#endif /* GDN_ORACLE_H */
