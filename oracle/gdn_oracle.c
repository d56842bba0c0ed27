/*
 * gdn_oracle.c - plain C99 CPU oracle (TEST INFRASTRUCTURE ONLY; see
 * gdn_oracle.h for the sources, the layouts and who may call this).
 *
 * Written to be read against the pages, not to be fast: sequential binary32
 * sums, a separate multiply and add (the build uses -ffp-contract=off), libm
 * expf/sqrtf.
 */
#include "gdn_oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

/* Sequential binary32 dot product of a[0], a[step], ..., a[(n-1)*step]
 * with b[0..n-1]: one rounded product and one rounded sum per term, in
 * index order. */
static float dot(const float *a, size_t step, const float *b, int32_t n)
{
    float s = 0.0f;
    int32_t i;
    for (i = 0; i < n; ++i)
        s = s + a[(size_t)i * step] * b[i];
    return s;
}

/*
 * One value head, one token ([dev15c] "Pinned llama.cpp semantics").
 *
 * The head's state is a dk x dv matrix S (key coordinate i, value coordinate
 * j), stored transposed as M = S^T, so that M[j] (row j, dk contiguous
 * floats) is everything value coordinate j remembers.  With e = exp(gate),
 * the token's effect in matrix form is
 *
 *     M' = e M + beta (v - e M k) k^T          (delta rule on the decayed state)
 *     out = M' q / sqrt(dk)                    (read-out from the new state)
 *
 * dk is the state/key dimension, 128 on the page; it is a parameter only so
 * that tiny heads can be brute-forced.  Row j of M' depends on row j of M,
 * on the shared k, q, beta, e and on v[j] alone, so the update is evaluated
 * row by row: the decayed row r = e M[j], its correction coefficient
 * c = beta (v[j] - r.k) (the value the page calls delta), the new row
 * r + c k, and out[j] = (r + c k).q / sqrt(dk).
 */
static void head_token_M(int32_t dk, int32_t dv,
                         const float *q, const float *k, const float *v,
                         float beta, float gate, float *M, float *out,
                         float *delta)
{
    const float e = expf(gate);
    const float rs = sqrtf((float)dk);
    int32_t i, j;

    for (j = 0; j < dv; ++j) {
        float *m = M + (size_t)j * dk;
        float c;
        for (i = 0; i < dk; ++i)
            m[i] = m[i] * e;
        c = (v[j] - dot(m, 1, k, dk)) * beta;
        if (delta)
            delta[j] = c;
        for (i = 0; i < dk; ++i)
            m[i] = m[i] + c * k[i];
        out[j] = dot(m, 1, q, dk) / rs;
    }
}

/* Value head h reads Q/K of key head h % Hk: the page lists the broadcast as
 * value_head % key_heads, i.e. key heads 0..15 then 0..15 again. */
static int32_t key_head_of(int32_t h, int32_t Hk) { return h % Hk; }

void oracle_gdn_step_M(int32_t B, int32_t Hv, int32_t Hk, int32_t dk, int32_t dv,
                       const float *q, const float *k, const float *v,
                       const float *beta, const float *gate,
                       float *M, float *out, float *delta)
{
    int32_t b, h;
    for (b = 0; b < B; ++b) {
        for (h = 0; h < Hv; ++h) {
            const int32_t kh = key_head_of(h, Hk);
            const size_t bh = (size_t)b * Hv + h;
            head_token_M(dk, dv,
                         q + ((size_t)b * Hk + kh) * dk,
                         k + ((size_t)b * Hk + kh) * dk,
                         v + bh * dv,
                         beta[bh], gate[bh],
                         M + bh * dv * dk,
                         out + bh * dv,
                         delta ? delta + bh * dv : NULL);
        }
    }
}

/*
 * The same token on the non-transposed state S (dk rows of dv floats), in
 * whole-matrix order rather than row by row:
 *     S <- e S;   c = beta (v - S^T k);   S <- S + k c^T;   out = S^T q / sqrt(dk).
 * The products S^T k and S^T q run down the columns of S.
 */
static void head_token_S(int32_t dk, int32_t dv,
                         const float *q, const float *k, const float *v,
                         float beta, float gate, float *S, float *out,
                         float *delta)
{
    const float e = expf(gate);
    const float rs = sqrtf((float)dk);
    float *c = (float *)malloc((size_t)dv * sizeof(float));
    int32_t i, j;

    for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] = S[(size_t)i * dv + j] * e;
    for (j = 0; j < dv; ++j) {
        c[j] = (v[j] - dot(S + j, (size_t)dv, k, dk)) * beta;
        if (delta)
            delta[j] = c[j];
    }
    for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] = S[(size_t)i * dv + j] + k[i] * c[j];
    for (j = 0; j < dv; ++j)
        out[j] = dot(S + j, (size_t)dv, q, dk) / rs;
    free(c);
}

void oracle_gdn_step_S(int32_t B, int32_t Hv, int32_t Hk, int32_t dk, int32_t dv,
                       const float *q, const float *k, const float *v,
                       const float *beta, const float *gate,
                       float *S, float *out, float *delta)
{
    int32_t b, h;
    for (b = 0; b < B; ++b) {
        for (h = 0; h < Hv; ++h) {
            const int32_t kh = key_head_of(h, Hk);
            const size_t bh = (size_t)b * Hv + h;
            head_token_S(dk, dv,
                         q + ((size_t)b * Hk + kh) * dk,
                         k + ((size_t)b * Hk + kh) * dk,
                         v + bh * dv,
                         beta[bh], gate[bh],
                         S + bh * dk * dv,
                         out + bh * dv,
                         delta ? delta + bh * dv : NULL);
        }
    }
}

/* Binary64 shadow of head_token_M: the same row form with f32 inputs
 * promoted and the state, sums and output in double. */
static double dot64(const double *a, const float *b, int32_t n)
{
    double s = 0.0;
    int32_t i;
    for (i = 0; i < n; ++i)
        s = s + a[i] * (double)b[i];
    return s;
}

static void head_token_f64(int32_t dk, int32_t dv,
                           const float *q, const float *k, const float *v,
                           float beta, float gate, double *M, double *out)
{
    const double e = exp((double)gate);
    const double rs = sqrt((double)dk);
    int32_t i, j;

    for (j = 0; j < dv; ++j) {
        double *m = M + (size_t)j * dk;
        double c;
        for (i = 0; i < dk; ++i)
            m[i] = m[i] * e;
        c = ((double)v[j] - dot64(m, k, dk)) * (double)beta;
        for (i = 0; i < dk; ++i)
            m[i] = m[i] + c * (double)k[i];
        out[j] = dot64(m, q, dk) / rs;
    }
}

void oracle_gdn_step_f64(int32_t B, int32_t Hv, int32_t Hk, int32_t dk, int32_t dv,
                         const float *q, const float *k, const float *v,
                         const float *beta, const float *gate,
                         double *M, double *out)
{
    int32_t b, h;
    for (b = 0; b < B; ++b) {
        for (h = 0; h < Hv; ++h) {
            const int32_t kh = key_head_of(h, Hk);
            const size_t bh = (size_t)b * Hv + h;
            head_token_f64(dk, dv,
                           q + ((size_t)b * Hk + kh) * dk,
                           k + ((size_t)b * Hk + kh) * dk,
                           v + bh * dv,
                           beta[bh], gate[bh],
                           M + bh * dv * dk,
                           out + bh * dv);
        }
    }
}

/* [linear_core] the binary64 shadow over T positions in order, state carried
 * (the yardstick for long sequences). */
void oracle_gdn_seq_f64(int32_t B, int32_t T, int32_t Hv, int32_t Hk, int32_t dk, int32_t dv,
                        const float *q, const float *k, const float *v,
                        const float *beta, const float *gate,
                        double *M, double *out)
{
    int32_t b, t, h;
    for (b = 0; b < B; ++b) {
        for (t = 0; t < T; ++t) {
            const size_t bt = (size_t)b * T + t;
            for (h = 0; h < Hv; ++h) {
                const int32_t kh = key_head_of(h, Hk);
                head_token_f64(dk, dv,
                               q + (bt * Hk + kh) * dk,
                               k + (bt * Hk + kh) * dk,
                               v + (bt * Hv + h) * dv,
                               beta[bt * Hv + h], gate[bt * Hv + h],
                               M + ((size_t)b * Hv + h) * dv * dk,
                               out + (bt * Hv + h) * dv);
            }
        }
    }
}

/* [linear_core] the batch path takes the positions one after another; each
 * position is one single-token step on the carried state. */
void oracle_gdn_seq(int32_t B, int32_t T, int32_t Hv, int32_t Hk, int32_t dk, int32_t dv,
                    const float *q, const float *k, const float *v,
                    const float *beta, const float *gate,
                    float *M, float *out)
{
    int32_t b, t, h;
    for (b = 0; b < B; ++b) {
        for (t = 0; t < T; ++t) {
            const size_t bt = (size_t)b * T + t;
            for (h = 0; h < Hv; ++h) {
                const int32_t kh = key_head_of(h, Hk);
                head_token_M(dk, dv,
                            q + (bt * Hk + kh) * dk,
                            k + (bt * Hk + kh) * dk,
                            v + (bt * Hv + h) * dv,
                            beta[bt * Hv + h], gate[bt * Hv + h],
                            M + ((size_t)b * Hv + h) * dv * dk,
                            out + (bt * Hv + h) * dv,
                            NULL);
            }
        }
    }
}

/* [linear_core] gdn_pair: position 1 is an ordinary step on the committed
 * state; position 2 is a step on a copy of the result (the tentative lane). */
void oracle_gdn_pair(int32_t B, int32_t Hv, int32_t Hk, int32_t dk, int32_t dv,
                     const float *q, const float *k, const float *v,
                     const float *beta, const float *gate,
                     float *M, float *M_next, float *out)
{
    int32_t b, h, p;
    for (b = 0; b < B; ++b) {
        for (h = 0; h < Hv; ++h) {
            const int32_t kh = key_head_of(h, Hk);
            float *Mh = M + ((size_t)b * Hv + h) * dv * dk;
            float *Nh = M_next + ((size_t)b * Hv + h) * dv * dk;
            for (p = 0; p < 2; ++p) {
                const size_t bp = (size_t)b * 2 + p;
                if (p == 1)
                    memcpy(Nh, Mh, (size_t)dv * dk * sizeof(float));
                head_token_M(dk, dv,
                            q + (bp * Hk + kh) * dk,
                            k + (bp * Hk + kh) * dk,
                            v + (bp * Hv + h) * dv,
                            beta[bp * Hv + h], gate[bp * Hv + h],
                            p == 0 ? Mh : Nh,
                            out + (bp * Hv + h) * dv,
                            NULL);
            }
        }
    }
}

static float silu(float x) { return x / (1.0f + expf(-x)); }

/*
 * [dev15a] conv-state shift + causal conv1d + SiLU, one token.  The window
 * of channel c is [cache slot 0 .. slot K-2, x] (oldest first); tap t of the
 * weight multiplies window element t; there is no bias.  Afterwards the
 * cache holds the last K-1 raw inputs (the new x in the last slot).
 */
void oracle_conv_silu(int32_t B, int32_t C, int32_t K,
                      const float *x, const float *conv_w, float *conv_state,
                      float *act)
{
    float *win = (float *)malloc((size_t)K * sizeof(float));
    int32_t b, c, t;
    for (b = 0; b < B; ++b) {
        float *cs = conv_state + (size_t)b * (K - 1) * C;
        for (c = 0; c < C; ++c) {
            float acc = 0.0f;
            for (t = 0; t < K - 1; ++t)
                win[t] = cs[(size_t)t * C + c];
            win[K - 1] = x[(size_t)b * C + c];
            for (t = 0; t < K; ++t)
                acc = acc + conv_w[(size_t)c * K + t] * win[t];
            for (t = 0; t < K - 1; ++t)
                cs[(size_t)t * C + c] = win[t + 1];
            act[(size_t)b * C + c] = silu(acc);
        }
    }
    free(win);
}

void oracle_l2norm_rows(int32_t n, int32_t d, float *u)
{
    int32_t r, i;
    for (r = 0; r < n; ++r) {
        float *row = u + (size_t)r * d;
        float ss = 0.0f, nrm;
        for (i = 0; i < d; ++i)
            ss = ss + row[i] * row[i];
        nrm = sqrtf(ss);
        if (nrm < 1e-6f)
            nrm = 1e-6f;
        for (i = 0; i < d; ++i)
            row[i] = row[i] / nrm;
    }
}

void oracle_gated_rmsnorm(int32_t rows, int32_t n, int32_t group, float eps,
                          const float *o, const float *z, const float *w,
                          float *y)
{
    int32_t r, g, i;
    for (r = 0; r < rows; ++r) {
        for (g = 0; g < n; g += group) {
            const size_t base = (size_t)r * n + g;
            float ss = 0.0f, rms;
            for (i = 0; i < group; ++i)
                ss = ss + o[base + i] * o[base + i];
            rms = sqrtf(ss / (float)group + eps);
            for (i = 0; i < group; ++i)
                y[base + i] = (o[base + i] / rms) * w[i] * silu(z[base + i]);
        }
    }
}

void oracle_layer_tail(int32_t B, int32_t Hv, int32_t Hk, int32_t dk, int32_t dv,
                       int32_t K, int32_t group, float eps,
                       const float *x, const float *conv_w, float *conv_state,
                       const float *beta, const float *gate, float *M,
                       const float *z, const float *norm_w, float *y,
                       float *qkv_out, float *core_out)
{
    const int32_t nq = Hk * dk, nv = Hv * dv;
    const int32_t C = 2 * nq + nv;
    float *act = (float *)malloc((size_t)B * C * sizeof(float));
    float *q = (float *)malloc((size_t)B * nq * sizeof(float));
    float *k = (float *)malloc((size_t)B * nq * sizeof(float));
    float *v = (float *)malloc((size_t)B * nv * sizeof(float));
    float *o = (float *)malloc((size_t)B * nv * sizeof(float));
    int32_t b;

    /* conv-state shift, conv1d, SiLU */
    oracle_conv_silu(B, C, K, x, conv_w, conv_state, act);

    /* Q/K/V split, [Q | K | V], then per-head L2 of Q and K */
    for (b = 0; b < B; ++b) {
        memcpy(q + (size_t)b * nq, act + (size_t)b * C, (size_t)nq * sizeof(float));
        memcpy(k + (size_t)b * nq, act + (size_t)b * C + nq, (size_t)nq * sizeof(float));
        memcpy(v + (size_t)b * nv, act + (size_t)b * C + 2 * nq, (size_t)nv * sizeof(float));
    }
    oracle_l2norm_rows(B * Hk, dk, q);
    oracle_l2norm_rows(B * Hk, dk, k);

    if (qkv_out) {
        for (b = 0; b < B; ++b) {
            memcpy(qkv_out + (size_t)b * C, q + (size_t)b * nq, (size_t)nq * sizeof(float));
            memcpy(qkv_out + (size_t)b * C + nq, k + (size_t)b * nq, (size_t)nq * sizeof(float));
            memcpy(qkv_out + (size_t)b * C + 2 * nq, v + (size_t)b * nv, (size_t)nv * sizeof(float));
        }
    }

    /* the recurrent state step */
    oracle_gdn_step_M(B, Hv, Hk, dk, dv, q, k, v, beta, gate, M, o, NULL);
    if (core_out)
        memcpy(core_out, o, (size_t)B * nv * sizeof(float));

    /* gated RMSNorm x SiLU(z) */
    oracle_gated_rmsnorm(B, nv, group, eps, o, z, norm_w, y);

    free(act);
    free(q);
    free(k);
    free(v);
    free(o);
}

/*
 * [linear_core] gdn_pair applied to the whole recurrent branch: the first
 * position's update is kept, the second's is held aside, and the conv ring
 * is held aside together with the state.  Position 1 is one layer tail on
 * the committed conv ring and state.  Position 2 is one layer tail that
 * starts from what position 1 committed, run on copies: its ring and state
 * go to the tentative buffers, so the committed ones stay as position 1 left
 * them.
 *   x [B][2][C]; beta, gate [B][2][Hv]; z, y [B][2][Hv*dv]
 *   conv_state [B][K-1][C] in/out (committed), conv_state_next out (tentative)
 *   M [B][Hv][dv][dk] in/out (committed), M_next out (tentative)
 */
void oracle_layer_tail_pair(int32_t B, int32_t Hv, int32_t Hk, int32_t dk, int32_t dv,
                            int32_t K, int32_t group, float eps,
                            const float *x, const float *conv_w,
                            float *conv_state, float *conv_state_next,
                            const float *beta, const float *gate,
                            float *M, float *M_next,
                            const float *z, const float *norm_w, float *y)
{
    const int32_t nv = Hv * dv;
    const int32_t C = 2 * Hk * dk + nv;
    const size_t ring = (size_t)(K - 1) * C;
    const size_t st = (size_t)Hv * dv * dk;
    int32_t b, p;
    for (b = 0; b < B; ++b) {
        for (p = 0; p < 2; ++p) {
            const size_t bp = 2 * (size_t)b + p;
            float *cs = (p == 0 ? conv_state : conv_state_next) + (size_t)b * ring;
            float *Mb = (p == 0 ? M : M_next) + (size_t)b * st;
            if (p == 1) {
                memcpy(cs, conv_state + (size_t)b * ring, ring * sizeof(float));
                memcpy(Mb, M + (size_t)b * st, st * sizeof(float));
            }
            oracle_layer_tail(1, Hv, Hk, dk, dv, K, group, eps,
                              x + bp * C, conv_w, cs,
                              beta + bp * Hv, gate + bp * Hv, Mb,
                              z + bp * nv, norm_w, y + bp * nv, NULL, NULL);
        }
    }
}

/* ---------------------------------------------------------------------
 * [dev15a] "Validation boundary" names the beta/alpha parameter transforms
 * as the stage before the recurrent update, and "DeltaNet projection parity -
 * real layer 0" gives their projection 64 outputs per token, i.e. one beta
 * and one alpha logit per value head.  The pages print no formula.  Reading
 * taken (the Mamba-2 style gating of the Gated DeltaNet paper, Yang, Kautz
 * and Hatamizadeh, restated): per sequence b and value head h,
 *   beta = sigmoid(b_h) = 1 / (1 + exp(-b_h))
 *   gate = -exp(A_log[h]) * softplus(a_h + dt_bias[h]),
 *          softplus(x) = log(1 + exp(x)),
 * with the projection row laid out [b_0 .. b_{Hv-1} | a_0 .. a_{Hv-1}].
 * softplus is evaluated as x + log1p(exp(-x)) for x > 0, the same function
 * without the overflow of exp(x).
 */
static float softplus(float x) { return x > 0.0f ? x + log1pf(expf(-x)) : log1pf(expf(x)); }

void oracle_gate_transform(int32_t B, int32_t Hv, const float *ba, const float *a_log,
                           const float *dt_bias, float *beta, float *gate)
{
    int32_t b, h;
    for (b = 0; b < B; ++b) {
        const float *row = ba + (size_t)b * 2 * Hv;
        for (h = 0; h < Hv; ++h) {
            const float bl = row[h];
            const float al = row[Hv + h];
            beta[(size_t)b * Hv + h] = 1.0f / (1.0f + expf(-bl));
            gate[(size_t)b * Hv + h] = -expf(a_log[h]) * softplus(al + dt_bias[h]);
        }
    }
}
