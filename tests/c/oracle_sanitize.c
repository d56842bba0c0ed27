/* Drives every oracle function on small inputs; built with AddressSanitizer
 * and UndefinedBehaviorSanitizer by tests/test_cpu_aux.py (CPU only).  Exits
 * non-zero on a non-finite result; the sanitizers abort on any out-of-bounds
 * access or undefined behaviour. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "gdn_oracle.h"

static float *rnd(size_t n, unsigned *s, float scale) {
    float *a = (float *)malloc(n * sizeof(float));
    size_t i;
    for (i = 0; i < n; ++i) {
        *s = *s * 1664525u + 1013904223u;
        a[i] = scale * ((float)((*s >> 8) & 0xFFFF) / 65536.0f - 0.5f);
    }
    return a;
}

static int finite_all(const float *a, size_t n) {
    size_t i;
    for (i = 0; i < n; ++i)
        if (!isfinite(a[i])) return 0;
    return 1;
}

int main(void) {
    unsigned s = 12345u;
    const int B = 2, Hv = 4, Hk = 2, d = 8, T = 3, K = 4;
    const int C = 2 * Hk * d + Hv * d;
    float *q = rnd((size_t)B * 2 * Hk * d, &s, 1.0f), *k = rnd((size_t)B * 2 * Hk * d, &s, 1.0f);
    float *v = rnd((size_t)B * 2 * Hv * d, &s, 2.0f);
    float *beta = rnd((size_t)B * 2 * Hv, &s, 1.0f), *gate = rnd((size_t)B * 2 * Hv, &s, 1.0f);
    float *M = rnd((size_t)B * Hv * d * d, &s, 0.2f), *Mn = rnd((size_t)B * Hv * d * d, &s, 0.2f);
    float *out = rnd((size_t)B * 2 * Hv * d, &s, 1.0f), *delta = rnd((size_t)B * Hv * d, &s, 1.0f);
    double *M64 = (double *)calloc((size_t)B * Hv * d * d, sizeof(double));
    double *o64 = (double *)calloc((size_t)B * Hv * d, sizeof(double));
    float *qs = rnd((size_t)B * T * Hk * d, &s, 1.0f), *ks = rnd((size_t)B * T * Hk * d, &s, 1.0f);
    float *vs = rnd((size_t)B * T * Hv * d, &s, 1.0f), *bs = rnd((size_t)B * T * Hv, &s, 1.0f);
    float *gs = rnd((size_t)B * T * Hv, &s, 1.0f), *os = rnd((size_t)B * T * Hv * d, &s, 1.0f);
    float *x = rnd((size_t)B * C, &s, 2.0f), *w = rnd((size_t)C * K, &s, 0.2f);
    float *cs = rnd((size_t)B * (K - 1) * C, &s, 2.0f), *act = rnd((size_t)B * C, &s, 1.0f);
    float *z = rnd((size_t)B * Hv * d, &s, 2.0f), *nw = rnd((size_t)d, &s, 1.0f);
    float *nw_all = rnd((size_t)Hv * d, &s, 1.0f);   /* weight for one group over all heads */
    float *y = rnd((size_t)B * Hv * d, &s, 1.0f), *qkv = rnd((size_t)B * C, &s, 1.0f);
    float *core = rnd((size_t)B * Hv * d, &s, 1.0f);

    oracle_gdn_step_M(B, Hv, Hk, d, d, q, k, v, beta, gate, M, out, delta);
    oracle_gdn_step_M(B, Hv, Hk, d, d, q, k, v, beta, gate, M, out, NULL);
    oracle_gdn_step_S(B, Hv, Hk, d, d, q, k, v, beta, gate, Mn, out, delta);
    oracle_gdn_step_f64(B, Hv, Hk, d, d, q, k, v, beta, gate, M64, o64);
    oracle_gdn_seq(B, T, Hv, Hk, d, d, qs, ks, vs, bs, gs, M, os);
    oracle_gdn_pair(B, Hv, Hk, d, d, q, k, v, beta, gate, M, Mn, out);
    oracle_conv_silu(B, C, K, x, w, cs, act);
    oracle_l2norm_rows(B * Hk, d, act);
    oracle_gated_rmsnorm(B, Hv * d, d, 1e-6f, out, z, nw, y);
    oracle_layer_tail(B, Hv, Hk, d, d, K, d, 1e-6f, x, w, cs, beta, gate, M, z, nw, y, qkv, core);
    oracle_layer_tail(B, Hv, Hk, d, d, K, Hv * d, 1e-6f, x, w, cs, beta, gate, M, z, nw_all, y, NULL,
                      NULL);

    if (!finite_all(M, (size_t)B * Hv * d * d) || !finite_all(y, (size_t)B * Hv * d) ||
        !finite_all(os, (size_t)B * T * Hv * d) || !finite_all(Mn, (size_t)B * Hv * d * d)) {
        fprintf(stderr, "non-finite result\n");
        return 1;
    }
    free(q); free(k); free(v); free(beta); free(gate); free(M); free(Mn); free(out); free(delta);
    free(M64); free(o64); free(qs); free(ks); free(vs); free(bs); free(gs); free(os);
    free(x); free(w); free(cs); free(act); free(z); free(nw); free(nw_all); free(y); free(qkv);
    free(core);
    printf("oracle sanitizer run ok\n");
    return 0;
}
