/*
 * gdn_c_check.c - calls libgdn.so through its C ABI only (no Python), the
 * way the Red Lite pages test their native path, and checks results that
 * have closed forms on the host:
 *   1. pure decay (beta = 0):       M' = exp(gate) M,   out = exp(gate) M q / sqrt(128)
 *   2. delta rule (beta=1, gate=0, unit k):  M' k = v  for every value head
 *   3. full forget (gate = -1e4):   M' = beta v k^T
 *   4. gdn_seq over 3 tokens == 3 gdn_step calls, bit for bit, and
 *      gdn_seq_exact over 20 tokens == 20 gdn_step calls
 *   5. argument errors: GDN_ERR_ALIGN / GDN_ERR_ALIAS before any work
 *   6. gdn_gate_transform: sigmoid(0) = 1/2 exactly, sigmoid(ln 3) = 3/4,
 *      gate = -ln 2 at a zero softplus argument, exp(gate) = 1 - beta when
 *      a_log = dt_bias = 0 and the alpha logit equals the beta logit
 *   7. gdn_step_ex with GDN_STATE_CACHED == gdn_step, bit for bit, and an
 *      unknown flag bit is refused
 * Exits 0 on success; prints the first failure otherwise.
 */
#include <hip/hip_runtime_api.h>

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gdn.h"

#define B 2
#define HV 32
#define HK 16
#define D 128
#define NS ((size_t)B * HV * D * D)

#define HIP_OK(x)                                                              \
    do {                                                                       \
        hipError_t e_ = (x);                                                   \
        if (e_ != hipSuccess) {                                                \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));     \
            exit(2);                                                           \
        }                                                                      \
    } while (0)

static unsigned rng = 2024u;
static float uni(void) {            /* deterministic, in (-0.5, 0.5) */
    rng = rng * 1664525u + 1013904223u;
    return (float)((rng >> 8) & 0xFFFFFF) / 16777216.0f - 0.5f;
}

static void unit_rows(float *a, int rows) {
    for (int r = 0; r < rows; ++r) {
        double s = 0;
        for (int i = 0; i < D; ++i) s += (double)a[r * D + i] * a[r * D + i];
        for (int i = 0; i < D; ++i) a[r * D + i] = (float)(a[r * D + i] / sqrt(s));
    }
}

typedef struct { float *q, *k, *v, *beta, *gate, *M, *out; } Dev;

static void upload(Dev *d, const float *q, const float *k, const float *v, const float *beta,
                   const float *gate, const float *M) {
    HIP_OK(hipMemcpy(d->q, q, (size_t)B * HK * D * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d->k, k, (size_t)B * HK * D * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d->v, v, (size_t)B * HV * D * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d->beta, beta, (size_t)B * HV * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d->gate, gate, (size_t)B * HV * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d->M, M, NS * 4, hipMemcpyHostToDevice));
}

static int fail(const char *what, double err) {
    fprintf(stderr, "FAIL %s (error %.3e)\n", what, err);
    return 1;
}

int main(void) {
    const gdn_dims dims = {HV, HK, D, D};
    float *q = malloc((size_t)B * HK * D * 4), *k = malloc((size_t)B * HK * D * 4);
    float *v = malloc((size_t)B * HV * D * 4), *beta = malloc(B * HV * 4), *gate = malloc(B * HV * 4);
    float *M = malloc(NS * 4), *M2 = malloc(NS * 4), *out = malloc((size_t)B * HV * D * 4);
    Dev d;
    HIP_OK(hipMalloc((void **)&d.q, (size_t)B * HK * D * 4));
    HIP_OK(hipMalloc((void **)&d.k, (size_t)B * HK * D * 4));
    HIP_OK(hipMalloc((void **)&d.v, (size_t)B * HV * D * 4));
    HIP_OK(hipMalloc((void **)&d.beta, B * HV * 4));
    HIP_OK(hipMalloc((void **)&d.gate, B * HV * 4));
    HIP_OK(hipMalloc((void **)&d.M, NS * 4));
    HIP_OK(hipMalloc((void **)&d.out, (size_t)B * HV * D * 4));

    for (size_t i = 0; i < (size_t)B * HK * D; ++i) { q[i] = uni(); k[i] = uni(); }
    unit_rows(q, B * HK);
    unit_rows(k, B * HK);
    for (size_t i = 0; i < (size_t)B * HV * D; ++i) v[i] = 2.0f * uni();
    for (size_t i = 0; i < NS; ++i) M[i] = 0.2f * uni();

    /* 1. pure decay */
    for (int i = 0; i < B * HV; ++i) { beta[i] = 0.0f; gate[i] = -0.5f + 0.4f * uni(); }
    upload(&d, q, k, v, beta, gate, M);
    if (gdn_step(&dims, B, d.q, d.k, d.v, d.beta, d.gate, d.M, d.out, NULL) != GDN_OK)
        return fail(gdn_last_error(), 0);
    HIP_OK(hipMemcpy(M2, d.M, NS * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(out, d.out, (size_t)B * HV * D * 4, hipMemcpyDeviceToHost));
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < HV; ++h) {
            const double e = exp((double)gate[b * HV + h]);
            const float *Mh = M + ((size_t)b * HV + h) * D * D, *Nh = M2 + ((size_t)b * HV + h) * D * D;
            const float *qh = q + ((size_t)b * HK + h % HK) * D;
            for (int j = 0; j < D; ++j) {
                double s = 0;
                for (int i = 0; i < D; ++i) {
                    const double want = e * Mh[j * D + i];
                    if (fabs(Nh[j * D + i] - want) > 1e-6) return fail("pure decay state", Nh[j * D + i] - want);
                    s += want * qh[i];
                }
                const double o = out[((size_t)b * HV + h) * D + j] - s / sqrt(128.0);
                if (fabs(o) > 1e-6) return fail("pure decay out", o);
            }
        }

    /* 2. delta rule */
    for (int i = 0; i < B * HV; ++i) { beta[i] = 1.0f; gate[i] = 0.0f; }
    upload(&d, q, k, v, beta, gate, M);
    if (gdn_step(&dims, B, d.q, d.k, d.v, d.beta, d.gate, d.M, d.out, NULL) != GDN_OK)
        return fail(gdn_last_error(), 0);
    HIP_OK(hipMemcpy(M2, d.M, NS * 4, hipMemcpyDeviceToHost));
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < HV; ++h) {
            const float *Nh = M2 + ((size_t)b * HV + h) * D * D;
            const float *kh = k + ((size_t)b * HK + h % HK) * D;
            for (int j = 0; j < D; ++j) {
                double s = 0;
                for (int i = 0; i < D; ++i) s += (double)Nh[j * D + i] * kh[i];
                if (fabs(s - v[((size_t)b * HV + h) * D + j]) > 2e-6) return fail("delta rule", s - v[((size_t)b * HV + h) * D + j]);
            }
        }

    /* 3. full forget */
    for (int i = 0; i < B * HV; ++i) { beta[i] = 0.25f + 0.5f * (uni() + 0.5f); gate[i] = -1e4f; }
    upload(&d, q, k, v, beta, gate, M);
    if (gdn_step(&dims, B, d.q, d.k, d.v, d.beta, d.gate, d.M, d.out, NULL) != GDN_OK)
        return fail(gdn_last_error(), 0);
    HIP_OK(hipMemcpy(M2, d.M, NS * 4, hipMemcpyDeviceToHost));
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < HV; ++h)
            for (int j = 0; j < D; ++j) {
                const float bv = v[((size_t)b * HV + h) * D + j] * beta[b * HV + h];
                for (int i = 0; i < D; ++i) {
                    const float want = bv * k[((size_t)b * HK + h % HK) * D + i];
                    if (M2[(((size_t)b * HV + h) * D + j) * D + i] != want) return fail("full forget", 0);
                }
            }

    /* 4. gdn_seq over 3 tokens == 3 gdn_step calls, bit for bit; the same
     *    for gdn_seq_exact over 20 tokens (past the 16-token groups) */
    typedef int (*seq_fn)(const gdn_dims *, int32_t, int32_t, const float *, const float *,
                          const float *, const float *, const float *, float *, float *, void *);
    const seq_fn seq_fns[2] = {gdn_seq, gdn_seq_exact};
    const int seq_T[2] = {3, 20};
    for (int which = 0; which < 2; ++which) {
        const int T = seq_T[which];
        float *qs, *ks, *vs, *bs, *gs, *os, *Ms;
        HIP_OK(hipMalloc((void **)&qs, (size_t)B * T * HK * D * 4));
        HIP_OK(hipMalloc((void **)&ks, (size_t)B * T * HK * D * 4));
        HIP_OK(hipMalloc((void **)&vs, (size_t)B * T * HV * D * 4));
        HIP_OK(hipMalloc((void **)&bs, (size_t)B * T * HV * 4));
        HIP_OK(hipMalloc((void **)&gs, (size_t)B * T * HV * 4));
        HIP_OK(hipMalloc((void **)&os, (size_t)B * T * HV * D * 4));
        HIP_OK(hipMalloc((void **)&Ms, NS * 4));
        for (int i = 0; i < B * HV; ++i) { beta[i] = 0.3f + 0.4f * (uni() + 0.5f); gate[i] = -0.7f + 0.5f * uni(); }
        for (int b = 0; b < B; ++b)            /* the same token repeated: [b][t] = token b */
            for (int t = 0; t < T; ++t) {
                const size_t bt = (size_t)b * T + t;
                HIP_OK(hipMemcpy(qs + bt * HK * D, q + (size_t)b * HK * D, HK * D * 4, hipMemcpyHostToDevice));
                HIP_OK(hipMemcpy(ks + bt * HK * D, k + (size_t)b * HK * D, HK * D * 4, hipMemcpyHostToDevice));
                HIP_OK(hipMemcpy(vs + bt * HV * D, v + (size_t)b * HV * D, HV * D * 4, hipMemcpyHostToDevice));
                HIP_OK(hipMemcpy(bs + bt * HV, beta + b * HV, HV * 4, hipMemcpyHostToDevice));
                HIP_OK(hipMemcpy(gs + bt * HV, gate + b * HV, HV * 4, hipMemcpyHostToDevice));
            }
        upload(&d, q, k, v, beta, gate, M);
        HIP_OK(hipMemcpy(Ms, M, NS * 4, hipMemcpyHostToDevice));
        if (seq_fns[which](&dims, B, T, qs, ks, vs, bs, gs, Ms, os, NULL) != GDN_OK)
            return fail(gdn_last_error(), 0);
        for (int t = 0; t < T; ++t)
            if (gdn_step(&dims, B, d.q, d.k, d.v, d.beta, d.gate, d.M, d.out, NULL) != GDN_OK)
                return fail(gdn_last_error(), 0);
        HIP_OK(hipDeviceSynchronize());
        HIP_OK(hipMemcpy(M2, d.M, NS * 4, hipMemcpyDeviceToHost));
        float *Mseq = malloc(NS * 4);
        HIP_OK(hipMemcpy(Mseq, Ms, NS * 4, hipMemcpyDeviceToHost));
        if (memcmp(M2, Mseq, NS * 4) != 0)
            return fail(which ? "gdn_seq_exact != 20 x gdn_step" : "gdn_seq != 3 x gdn_step", 0);
        free(Mseq);
        hipFree(qs); hipFree(ks); hipFree(vs); hipFree(bs); hipFree(gs); hipFree(os); hipFree(Ms);
    }

    /* 5. argument errors are returned before any work */
    if (gdn_step(&dims, B, (const float *)((char *)d.q + 4), d.k, d.v, d.beta, d.gate, d.M, d.out,
                 NULL) != GDN_ERR_ALIGN)
        return fail("misaligned q not rejected", 0);
    if (gdn_step(&dims, B, d.q, d.k, d.v, d.beta, d.gate, d.M, d.M, NULL) != GDN_ERR_ALIAS)
        return fail("out aliasing state not rejected", 0);

    /* 6. beta/alpha parameter transforms */
    {
        float ba[B * 2 * HV], al[HV], dt[HV], hb[B * HV], hg[B * HV];
        for (int h = 0; h < HV; ++h) {
            al[h] = 0.0f;
            dt[h] = 0.0f;
            ba[h] = (h % 2) ? 0.0f : (float)log(3.0);       /* sequence 0: beta logits */
            ba[HV + h] = 0.0f;                              /* sequence 0: alpha logits */
            ba[2 * HV + h] = 0.25f * (float)(h - 16);       /* sequence 1: b = a = x */
            ba[3 * HV + h] = 0.25f * (float)(h - 16);
        }
        float *dba, *dal, *ddt, *db, *dg;
        HIP_OK(hipMalloc((void **)&dba, sizeof ba));
        HIP_OK(hipMalloc((void **)&dal, sizeof al));
        HIP_OK(hipMalloc((void **)&ddt, sizeof dt));
        HIP_OK(hipMalloc((void **)&db, sizeof hb));
        HIP_OK(hipMalloc((void **)&dg, sizeof hg));
        HIP_OK(hipMemcpy(dba, ba, sizeof ba, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(dal, al, sizeof al, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(ddt, dt, sizeof dt, hipMemcpyHostToDevice));
        const gdn_gate_inputs gin = {dba, dal, ddt};
        if (gdn_gate_transform(&dims, B, &gin, db, dg, NULL) != GDN_OK) return fail(gdn_last_error(), 0);
        HIP_OK(hipMemcpy(hb, db, sizeof hb, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(hg, dg, sizeof hg, hipMemcpyDeviceToHost));
        for (int h = 0; h < HV; ++h) {
            const double want_b = (h % 2) ? 0.5 : 0.75;
            if ((h % 2) && hb[h] != 0.5f) return fail("sigmoid(0) != 1/2", fabs(hb[h] - 0.5));
            if (fabs(hb[h] - want_b) > 3e-7) return fail("sigmoid(ln 3) != 3/4", fabs(hb[h] - want_b));
            if (fabs(hg[h] + log(2.0)) > 3e-7) return fail("softplus(0) != ln 2", fabs(hg[h] + log(2.0)));
            const double e = exp((double)hg[HV + h]) - (1.0 - (double)hb[HV + h]);
            if (fabs(e) > 3e-7) return fail("exp(gate) != 1 - beta", fabs(e));
        }
        if (gdn_gate_transform(&dims, B, &gin, db, dba, NULL) != GDN_ERR_ALIAS)
            return fail("gate aliasing ba not rejected", 0);
        hipFree(dba); hipFree(dal); hipFree(ddt); hipFree(db); hipFree(dg);
    }

    /* 7. the cached-state policy gives the bits of the default */
    {
        float *M1, *M2d, *o1, *o2;
        HIP_OK(hipMalloc((void **)&M1, NS * 4));
        HIP_OK(hipMalloc((void **)&M2d, NS * 4));
        HIP_OK(hipMalloc((void **)&o1, (size_t)B * HV * D * 4));
        HIP_OK(hipMalloc((void **)&o2, (size_t)B * HV * D * 4));
        HIP_OK(hipMemcpy(M1, d.M, NS * 4, hipMemcpyDeviceToDevice));
        HIP_OK(hipMemcpy(M2d, d.M, NS * 4, hipMemcpyDeviceToDevice));
        if (gdn_step(&dims, B, d.q, d.k, d.v, d.beta, d.gate, M1, o1, NULL) != GDN_OK ||
            gdn_step_ex(&dims, B, d.q, d.k, d.v, d.beta, d.gate, M2d, o2, GDN_STATE_CACHED,
                        NULL) != GDN_OK)
            return fail(gdn_last_error(), 0);
        if (gdn_step_ex(&dims, B, d.q, d.k, d.v, d.beta, d.gate, M2d, o2, 2u, NULL) !=
            GDN_ERR_SHAPE)
            return fail("unknown gdn_step_ex flag not rejected", 0);
        float *h1 = (float *)malloc(NS * 4), *h2 = (float *)malloc(NS * 4);
        HIP_OK(hipMemcpy(h1, M1, NS * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(h2, M2d, NS * 4, hipMemcpyDeviceToHost));
        if (memcmp(h1, h2, NS * 4) != 0) return fail("cached-policy state != gdn_step", 0);
        HIP_OK(hipMemcpy(h1, o1, (size_t)B * HV * D * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(h2, o2, (size_t)B * HV * D * 4, hipMemcpyDeviceToHost));
        if (memcmp(h1, h2, (size_t)B * HV * D * 4) != 0) return fail("cached-policy out != gdn_step", 0);
        free(h1); free(h2);
        hipFree(M1); hipFree(M2d); hipFree(o1); hipFree(o2);
    }

    HIP_OK(hipDeviceSynchronize());
    printf("C ABI check ok (version %d)\n", gdn_version());
    free(q); free(k); free(v); free(beta); free(gate); free(M); free(M2); free(out);
    hipFree(d.q); hipFree(d.k); hipFree(d.v); hipFree(d.beta); hipFree(d.gate); hipFree(d.M); hipFree(d.out);
    return 0;
}
