/* gdn_api_check.c - the C-ABI layer of libgdn (gdn_api.cpp) on the host
 * alone, built with AddressSanitizer and UndefinedBehaviorSanitizer and
 * linked with launcher stubs (gdn_api_stubs.cpp) instead of the kernels.
 * It drives every entry point through its argument checks (NULL pointers,
 * alignment, overlapping buffers, size limits at and one past their
 * boundary, workspace sizes, flags) and checks what a call that passes them
 * hands to the launchers: the kernel chosen, sizes, strides, and how the
 * workspace or the static scratch is split between the intermediates.  A
 * launch error reported by the runtime must come back as GDN_ERR_HIP and
 * stop the remaining launches of the call.
 *
 * Device buffers are stand-in addresses 2^44 bytes apart: the ABI layer
 * only compares and offsets them and never reads through them, so sizes up
 * to the largest the checks accept can be given without memory behind them. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gdn.h"
#include "gdn_api_stubs.h"

static int failures = 0;
static int checks = 0;

#define EXPECT(c)                                                       \
    do {                                                                \
        ++checks;                                                       \
        if (!(c)) {                                                     \
            fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                 \
        }                                                               \
    } while (0)

/* rc must be `want`; for an error, the message must hold `needle`; for
 * GDN_OK, the message must be empty. */
static void expect_rc(int rc, int want, const char *needle, int line) {
    ++checks;
    const char *msg = gdn_last_error();
    int ok = rc == want;
    if (ok && want == GDN_OK) ok = msg[0] == '\0';
    if (ok && want != GDN_OK && needle) ok = strstr(msg, needle) != NULL;
    if (!ok) {
        fprintf(stderr, "%s:%d: rc %d (want %d), message \"%s\" (want \"%s\")\n", __FILE__, line,
                rc, want, msg, needle ? needle : "");
        ++failures;
    }
}
#define EXPECT_RC(call, want, needle) expect_rc((call), (want), (needle), __LINE__)

/* stand-in device buffer number `slot` */
static float *F(int slot) { return (float *)(uintptr_t)((uint64_t)(slot + 1) << 44); }

#define STREAM ((void *)(uintptr_t)0x5eed0)

/* the i-th recorded launch, or an empty record (kind "") when there is none,
 * so that a missing launch fails its checks instead of stopping the run */
static const stub_launch *L(int i) {
    static const stub_launch none;
    const stub_launch *l = stub_launch_at(i);
    return l ? l : &none;
}
static int kind_is(int i, const char *k) { return strcmp(L(i)->kind, k) == 0; }

static const gdn_dims PAGE = {32, 16, 128, 128};

static void check_step(void) {
    float *q = F(0), *k = F(1), *v = F(2), *beta = F(3), *gate = F(4), *state = F(5),
          *out = F(6);
    const size_t ns = (size_t)3 * 32 * 128 * 128; /* floats of state at B = 3 */

    stub_reset();
    EXPECT_RC(gdn_step(&PAGE, 3, q, k, v, beta, gate, state, out, STREAM), GDN_OK, NULL);
    EXPECT(stub_n_launches() == 1 && kind_is(0, "step"));
    EXPECT(L(0)->p[0] == q && L(0)->p[1] == k && L(0)->p[2] == v && L(0)->p[3] == beta &&
           L(0)->p[4] == gate && L(0)->p[5] == state && L(0)->p[6] == out);
    EXPECT(L(0)->i[0] == 3 && L(0)->i[1] == 32 && L(0)->i[2] == 16 && L(0)->i[3] == 0);
    EXPECT(L(0)->l[0] == 16 * 128 && L(0)->l[1] == 32 * 128);
    EXPECT(L(0)->stream == STREAM);

    /* the cache-policy flag reaches the launcher; other bits are refused */
    stub_reset();
    EXPECT_RC(gdn_step_ex(&PAGE, 3, q, k, v, beta, gate, state, out, GDN_STATE_CACHED, STREAM),
              GDN_OK, NULL);
    EXPECT(stub_n_launches() == 1 && L(0)->i[3] == 1);
    EXPECT_RC(gdn_step_ex(&PAGE, 3, q, k, v, beta, gate, state, out, 2u, STREAM), GDN_ERR_SHAPE,
              "unknown flags 0x2");
    EXPECT_RC(gdn_step_ex(&PAGE, 3, q, k, v, beta, gate, state, out, 0x80000001u, STREAM),
              GDN_ERR_SHAPE, "unknown flags 0x80000000");
    EXPECT(stub_n_launches() == 1);

    /* each pointer NULL in turn, named in the message */
    {
        const char *names[7] = {"q", "k", "v", "beta", "gate", "state", "out"};
        for (int i = 0; i < 7; ++i) {
            float *p[7] = {q, k, v, beta, gate, state, out};
            char want[32];
            p[i] = NULL;
            snprintf(want, sizeof want, "%s is NULL", names[i]);
            EXPECT_RC(gdn_step(&PAGE, 3, p[0], p[1], p[2], p[3], p[4], p[5], p[6], STREAM),
                      GDN_ERR_NULL, want);
        }
    }
    /* vectors need 16 bytes, per-head scalars 4 */
    EXPECT_RC(gdn_step(&PAGE, 3, q + 1, k, v, beta, gate, state, out, STREAM), GDN_ERR_ALIGN,
              "q (");
    EXPECT_RC(gdn_step(&PAGE, 3, q, k, v, beta, gate, state + 2, out, STREAM), GDN_ERR_ALIGN,
              "state (");
    EXPECT_RC(gdn_step(&PAGE, 3, q, k, v, (float *)((char *)beta + 2), gate, state, out, STREAM),
              GDN_ERR_ALIGN, "beta (");
    EXPECT_RC(gdn_step(&PAGE, 3, q, k, v, beta + 1, gate + 3, state, out, STREAM), GDN_OK, NULL);
    /* outputs must not overlap anything; read-only inputs may */
    EXPECT_RC(gdn_step(&PAGE, 3, q, k, v, beta, gate, state, state + ns - 4, STREAM),
              GDN_ERR_ALIAS, "state overlaps out");
    EXPECT_RC(gdn_step(&PAGE, 3, q, k, v, beta, gate, state, v, STREAM), GDN_ERR_ALIAS,
              "overlaps v");
    EXPECT_RC(gdn_step(&PAGE, 3, q, k, v, beta, gate, state, (float *)gate, STREAM),
              GDN_ERR_ALIAS, "out overlaps gate");
    EXPECT_RC(gdn_step(&PAGE, 3, q, q, v, beta, beta, state, state + ns, STREAM), GDN_OK, NULL);

    /* shapes */
    EXPECT_RC(gdn_step(NULL, 3, q, k, v, beta, gate, state, out, STREAM), GDN_ERR_NULL,
              "dims is NULL");
    EXPECT_RC(gdn_step(&PAGE, 0, q, k, v, beta, gate, state, out, STREAM), GDN_ERR_SHAPE,
              "B must be >= 1");
    EXPECT_RC(gdn_step(&PAGE, -5, q, k, v, beta, gate, state, out, STREAM), GDN_ERR_SHAPE,
              "B must be >= 1");
    {
        const gdn_dims bad[] = {{0, 16, 128, 128}, {32, 0, 128, 128}, {33, 16, 128, 128},
                                {16, 32, 128, 128}, {32, 16, 64, 128}, {32, 16, 128, 256}};
        for (int i = 0; i < 6; ++i)
            EXPECT_RC(gdn_step(&bad[i], 1, q, k, v, beta, gate, state, out, STREAM),
                      GDN_ERR_SHAPE, NULL);
    }
    /* B * n_v_heads up to (INT32_MAX - 65536) / 16, at and one past the limit */
    {
        const gdn_dims one = {1, 1, 128, 128};
        EXPECT_RC(gdn_step(&one, 134213631, q, k, v, beta, gate, state, out, STREAM), GDN_OK,
                  NULL);
        EXPECT_RC(gdn_step(&one, 134213632, q, k, v, beta, gate, state, out, STREAM),
                  GDN_ERR_SHAPE, "exceeds 134213631");
        EXPECT_RC(gdn_step(&PAGE, 4194175, q, k, v, beta, gate, state, out, STREAM), GDN_OK,
                  NULL);
        EXPECT_RC(gdn_step(&PAGE, 4194176, q, k, v, beta, gate, state, out, STREAM),
                  GDN_ERR_SHAPE, "134213632");
        EXPECT_RC(gdn_step(&PAGE, INT32_MAX, q, k, v, beta, gate, state, out, STREAM),
                  GDN_ERR_SHAPE, "exceeds");
    }
}

static void check_seq(void) {
    float *q = F(0), *k = F(1), *v = F(2), *beta = F(3), *gate = F(4), *state = F(5),
          *out = F(6);
    stub_reset();
    /* one token takes the single-step kernel (same bits, faster) */
    EXPECT_RC(gdn_seq(&PAGE, 4, 1, q, k, v, beta, gate, state, out, STREAM), GDN_OK, NULL);
    EXPECT(stub_n_launches() == 1 && kind_is(0, "step"));
    EXPECT(L(0)->i[0] == 4 && L(0)->l[0] == 2048 && L(0)->l[1] == 4096 && L(0)->i[3] == 0);
    EXPECT_RC(gdn_seq_exact(&PAGE, 4, 1, q, k, v, beta, gate, state, out, STREAM), GDN_OK, NULL);
    EXPECT(stub_n_launches() == 2 && kind_is(1, "step"));
    EXPECT_RC(gdn_seq(&PAGE, 4, 7, q, k, v, beta, gate, state, out, STREAM), GDN_OK, NULL);
    EXPECT(kind_is(2, "seq") && L(2)->i[0] == 4 && L(2)->i[3] == 7 && L(2)->p[6] == out);
    EXPECT_RC(gdn_seq_exact(&PAGE, 4, 7, q, k, v, beta, gate, state, out, STREAM), GDN_OK, NULL);
    EXPECT(kind_is(3, "seq_exact") && L(3)->i[1] == 32 && L(3)->i[2] == 16);

    EXPECT_RC(gdn_seq(&PAGE, 4, 0, q, k, v, beta, gate, state, out, STREAM), GDN_ERR_SHAPE,
              "T must be in");
    EXPECT_RC(gdn_seq(&PAGE, 1, (1 << 30) + 1, q, k, v, beta, gate, state, out, STREAM),
              GDN_ERR_SHAPE, "T must be in");
    {
        const gdn_dims one = {1, 1, 128, 128};
        EXPECT_RC(gdn_seq(&one, 1, 1 << 30, q, k, v, beta, gate, state, out, STREAM), GDN_OK,
                  NULL);
        /* B * n_v_heads * 512 work-items must fit 32 bits */
        EXPECT_RC(gdn_seq(&one, 8388607, 2, q, k, v, beta, gate, state, out, STREAM), GDN_OK,
                  NULL);
        EXPECT_RC(gdn_seq_exact(&one, 8388608, 2, q, k, v, beta, gate, state, out, STREAM),
                  GDN_ERR_SHAPE, "gdn_seq_exact: B * n_v_heads = 8388608 exceeds 8388607");
    }
    /* out covers B*T tokens: the last token's row must not reach the state */
    EXPECT_RC(gdn_seq(&PAGE, 2, 3, q, k, v, beta, gate, state, state - 2 * 3 * 4096 + 4, STREAM),
              GDN_ERR_ALIAS, "overlaps");
    EXPECT_RC(gdn_seq(&PAGE, 2, 3, q, k, v, beta, gate, state, state - 2 * 3 * 4096, STREAM),
              GDN_OK, NULL);
    EXPECT_RC(gdn_seq(&PAGE, 2, 3, q, k, v, beta, NULL, state, out, STREAM), GDN_ERR_NULL,
              "gate is NULL");
    EXPECT_RC(gdn_seq(NULL, 2, 3, q, k, v, beta, gate, state, out, STREAM), GDN_ERR_NULL,
              "dims");
}

static void check_pair(void) {
    float *q = F(0), *k = F(1), *v = F(2), *beta = F(3), *gate = F(4), *state = F(5),
          *out = F(6), *state_next = F(7);
    stub_reset();
    EXPECT_RC(gdn_pair(&PAGE, 5, q, k, v, beta, gate, state, state_next, out, STREAM), GDN_OK,
              NULL);
    EXPECT(stub_n_launches() == 1 && kind_is(0, "pair") && L(0)->p[7] == state_next &&
           L(0)->p[5] == state && L(0)->i[0] == 5);
    EXPECT_RC(gdn_pair(&PAGE, 5, q, k, v, beta, gate, state, state, out, STREAM), GDN_ERR_ALIAS,
              "state overlaps state_next");
    EXPECT_RC(gdn_pair(&PAGE, 5, q, k, v, beta, gate, state, NULL, out, STREAM), GDN_ERR_NULL,
              "state_next is NULL");
    /* out holds two positions per sequence: 2 * 5 * 4096 floats */
    EXPECT_RC(gdn_pair(&PAGE, 5, q, k, v, beta, gate, state, out + 2 * 5 * 4096 - 4, out,
                       STREAM),
              GDN_ERR_ALIAS, "overlaps");
    EXPECT_RC(gdn_pair(&PAGE, 5, q, k, v, beta, gate, state, out + 2 * 5 * 4096, out, STREAM),
              GDN_OK, NULL);
    EXPECT(stub_n_launches() == 2);
}

static gdn_tail_params tail_params(int K, int group, float eps, int unfused) {
    gdn_tail_params p;
    memset(&p, 0, sizeof p);
    p.conv_kernel = K;
    p.norm_group = group;
    p.norm_eps = eps;
    p.force_unfused = unfused;
    return p;
}

static void check_tail(void) {
    float *x = F(0), *cw = F(1), *cs = F(2), *beta = F(3), *gate = F(4), *state = F(5),
          *z = F(6), *nw = F(7), *y = F(8), *ws = F(9), *dq = F(10), *dc = F(11);
    const int B = 3, C = 8192;
    const gdn_tail_params fused = tail_params(4, 128, 1e-6f, 0);
    const gdn_tail_params unf = tail_params(4, 128, 1e-6f, 1);
    const size_t wsb = gdn_layer_tail_workspace_bytes(&PAGE, B);

    EXPECT(gdn_layer_tail_workspace_bytes(NULL, B) == 0);
    EXPECT(gdn_layer_tail_workspace_bytes(&PAGE, 0) == 0);
    EXPECT(wsb == (size_t)B * (C + 4096) * 4);
    EXPECT(gdn_layer_tail_ba_workspace_bytes(&PAGE, B) == wsb + (size_t)2 * B * 32 * 4);
    EXPECT(gdn_layer_tail_ba_workspace_bytes(NULL, B) == 0);

    EXPECT(stub_tail_fused_supported(32, 16, 4, 128) && stub_tail_fused_supported(16, 16, 4, 128));
    EXPECT(!stub_tail_fused_supported(48, 16, 4, 128) && !stub_tail_fused_supported(32, 16, 3, 128));
    EXPECT(!stub_tail_fused_supported(32, 16, 4, 64) && !stub_tail_fused_supported(64, 16, 4, 128));

    /* single launch: no workspace needed */
    stub_reset();
    EXPECT_RC(gdn_layer_tail(&PAGE, &fused, B, x, cw, cs, beta, gate, state, z, nw, y, NULL, NULL,
                             NULL, 0, STREAM),
              GDN_OK, NULL);
    EXPECT(stub_n_launches() == 1 && kind_is(0, "tail_fused"));
    EXPECT(L(0)->p[0] == x && L(0)->p[1] == cw && L(0)->p[2] == cs && L(0)->p[3] == beta &&
           L(0)->p[4] == gate && L(0)->p[5] == state && L(0)->p[6] == z && L(0)->p[7] == nw &&
           L(0)->p[8] == y && L(0)->p[9] == NULL && L(0)->p[12] == NULL && L(0)->p[14] == NULL);
    EXPECT(L(0)->i[0] == B && L(0)->i[1] == 32 && L(0)->i[2] == 16 && L(0)->i[3] == C &&
           L(0)->i[4] == 4 && L(0)->f == 1e-6f);
    EXPECT_RC(gdn_layer_tail(&PAGE, &fused, B, x, cw, cs, beta, gate, state, z, nw, y, dq, dc,
                             NULL, 0, STREAM),
              GDN_OK, NULL);
    EXPECT(stub_n_launches() == 2 && L(1)->p[12] == dq && L(1)->p[13] == dc);

    /* three launches: the workspace holds Q|K|V, then the step output */
    stub_reset();
    EXPECT_RC(gdn_layer_tail(&PAGE, &unf, B, x, cw, cs, beta, gate, state, z, nw, y, NULL, NULL,
                             NULL, 0, STREAM),
              GDN_ERR_WORKSPACE, "workspace is NULL (147456 bytes needed)");
    EXPECT_RC(gdn_layer_tail(&PAGE, &unf, B, x, cw, cs, beta, gate, state, z, nw, y, NULL, NULL,
                             ws, wsb - 1, STREAM),
              GDN_ERR_WORKSPACE, "147455 bytes, 147456 needed");
    EXPECT_RC(gdn_layer_tail(&PAGE, &unf, B, x, cw, cs, beta, gate, state, z, nw, y, NULL, NULL,
                             ws + 1, wsb, STREAM),
              GDN_ERR_ALIGN, "workspace");
    EXPECT(stub_n_launches() == 0);
    EXPECT_RC(gdn_layer_tail(&PAGE, &unf, B, x, cw, cs, beta, gate, state, z, nw, y, NULL, NULL,
                             ws, wsb, STREAM),
              GDN_OK, NULL);
    EXPECT(stub_n_launches() == 3 && kind_is(0, "prestate") && kind_is(1, "step") &&
           kind_is(2, "gated_norm"));
    EXPECT(L(0)->p[0] == x && L(0)->p[2] == cs && L(0)->p[3] == ws && L(0)->i[1] == C &&
           L(0)->i[2] == 4 && L(0)->i[3] == 4096);
    EXPECT(L(1)->p[0] == ws && L(1)->p[1] == ws + 2048 && L(1)->p[2] == ws + 4096 &&
           L(1)->p[3] == beta && L(1)->p[5] == state && L(1)->p[6] == ws + (size_t)B * C &&
           L(1)->l[0] == C && L(1)->l[1] == C && L(1)->i[0] == B);
    EXPECT(L(2)->p[0] == ws + (size_t)B * C && L(2)->p[1] == z && L(2)->p[3] == y &&
           L(2)->i[0] == B && L(2)->i[1] == 4096 && L(2)->i[2] == 128 && L(2)->f == 1e-6f);

    /* debug buffers take the place of their part of the workspace */
    stub_reset();
    EXPECT_RC(gdn_layer_tail(&PAGE, &unf, B, x, cw, cs, beta, gate, state, z, nw, y, dq, NULL, ws,
                             (size_t)B * 4096 * 4, STREAM),
              GDN_OK, NULL);
    EXPECT(L(0)->p[3] == dq && L(1)->p[0] == dq && L(1)->p[6] == ws && L(2)->p[0] == ws);
    EXPECT_RC(gdn_layer_tail(&PAGE, &unf, B, x, cw, cs, beta, gate, state, z, nw, y, dq, dc, NULL,
                             0, STREAM),
              GDN_OK, NULL);
    EXPECT(stub_n_launches() == 6 && L(3)->p[3] == dq && L(4)->p[6] == dc && L(5)->p[0] == dc);
    EXPECT_RC(gdn_layer_tail(&PAGE, &unf, B, x, cw, cs, beta, gate, state, z, nw, y, dq + 2, dc,
                             NULL, 0, STREAM),
              GDN_ERR_ALIGN, "dbg_qkv");

    /* sizes without a single-launch kernel take the three launches */
    {
        const gdn_tail_params g64 = tail_params(4, 64, 1e-6f, 0);
        const gdn_tail_params k3 = tail_params(3, 128, 1e-6f, 0);
        const gdn_dims h48 = {48, 16, 128, 128};
        stub_reset();
        EXPECT_RC(gdn_layer_tail(&PAGE, &g64, B, x, cw, cs, beta, gate, state, z, nw, y, NULL,
                                 NULL, ws, wsb, STREAM),
                  GDN_OK, NULL);
        EXPECT(stub_n_launches() == 3 && L(2)->i[2] == 64);
        EXPECT_RC(gdn_layer_tail(&PAGE, &k3, B, x, cw, cs, beta, gate, state, z, nw, y, NULL,
                                 NULL, ws, wsb, STREAM),
                  GDN_OK, NULL);
        EXPECT(stub_n_launches() == 6 && L(3)->i[2] == 3);
        EXPECT_RC(gdn_layer_tail(&h48, &fused, B, x, cw, cs, beta, gate, state, z, nw, y, NULL,
                                 NULL, ws, gdn_layer_tail_workspace_bytes(&h48, B), STREAM),
                  GDN_OK, NULL);
        EXPECT(stub_n_launches() == 9 && kind_is(6, "prestate") && L(6)->i[1] == 4096 + 6144 &&
               L(7)->l[0] == 4096 + 6144 && L(7)->p[2] == ws + 4096);
    }

    /* parameter checks */
    {
        const gdn_tail_params bad[] = {tail_params(1, 128, 1e-6f, 0),
                                       tail_params(9, 128, 1e-6f, 0),
                                       tail_params(4, 0, 1e-6f, 0),
                                       tail_params(4, 100, 1e-6f, 0),
                                       tail_params(4, 128, -1e-6f, 0),
                                       tail_params(4, 128, NAN, 0),
                                       tail_params(4, 128, INFINITY, 0)};
        const char *want[] = {"conv_kernel", "conv_kernel", "norm_group", "norm_group",
                              "norm_eps", "norm_eps", "norm_eps"};
        for (int i = 0; i < 7; ++i)
            EXPECT_RC(gdn_layer_tail(&PAGE, &bad[i], B, x, cw, cs, beta, gate, state, z, nw, y,
                                     NULL, NULL, ws, wsb, STREAM),
                      GDN_ERR_SHAPE, want[i]);
        const gdn_tail_params eps0 = tail_params(4, 128, 0.0f, 0);
        EXPECT_RC(gdn_layer_tail(&PAGE, &eps0, B, x, cw, cs, beta, gate, state, z, nw, y, NULL,
                                 NULL, NULL, 0, STREAM),
                  GDN_OK, NULL);
        EXPECT_RC(gdn_layer_tail(&PAGE, NULL, B, x, cw, cs, beta, gate, state, z, nw, y, NULL,
                                 NULL, NULL, 0, STREAM),
                  GDN_ERR_NULL, "params is NULL");
    }
    /* B * channels up to INT32_MAX / 2, one gated-norm grid within 32 bits */
    EXPECT_RC(gdn_layer_tail(&PAGE, &fused, 131071, x, cw, cs, beta, gate, state, z, nw, y, NULL,
                             NULL, NULL, 0, STREAM),
              GDN_OK, NULL);
    EXPECT_RC(gdn_layer_tail(&PAGE, &fused, 131072, x, cw, cs, beta, gate, state, z, nw, y, NULL,
                             NULL, NULL, 0, STREAM),
              GDN_ERR_SHAPE, "too large");
    {
        const gdn_tail_params g1 = tail_params(4, 1, 1e-6f, 0);
        EXPECT_RC(gdn_layer_tail(&PAGE, &g1, 8191, x, cw, cs, beta, gate, state, z, nw, y, NULL,
                                 NULL, ws, (size_t)1 << 40, STREAM),
                  GDN_OK, NULL);
        EXPECT_RC(gdn_layer_tail(&PAGE, &g1, 8192, x, cw, cs, beta, gate, state, z, nw, y, NULL,
                                 NULL, ws, (size_t)1 << 40, STREAM),
                  GDN_ERR_SHAPE, "groups too many");
    }

    /* written buffers must be disjoint from everything */
    EXPECT_RC(gdn_layer_tail(&PAGE, &fused, B, x, cw, cs, beta, gate, state, z, nw, z, NULL, NULL,
                             NULL, 0, STREAM),
              GDN_ERR_ALIAS, "overlaps");
    EXPECT_RC(gdn_layer_tail(&PAGE, &fused, B, x, cw, x + (size_t)B * C - 4, beta, gate, state, z,
                             nw, y, NULL, NULL, NULL, 0, STREAM),
              GDN_ERR_ALIAS, "conv_state overlaps x");
    EXPECT_RC(gdn_layer_tail(&PAGE, &unf, B, x, cw, cs, beta, gate, state, z, nw, y, NULL, NULL,
                             state + 64, wsb, STREAM),
              GDN_ERR_ALIAS, "state overlaps qkv buffer");
    EXPECT_RC(gdn_layer_tail(&PAGE, &unf, B, x, cw, cs, beta, gate, state, z, nw, y, dq, y + 4,
                             NULL, 0, STREAM),
              GDN_ERR_ALIAS, "y overlaps core buffer");
    EXPECT_RC(gdn_layer_tail(&PAGE, &fused, B, x, cw, cs, beta, gate, state, z, nw, y, NULL, NULL,
                             state, 0, STREAM),
              GDN_OK, NULL); /* an unused workspace is not looked at */
}

static void check_tail_ba(void) {
    float *x = F(0), *cw = F(1), *cs = F(2), *state = F(5), *z = F(6), *nw = F(7), *y = F(8),
          *ws = F(9), *ba = F(12), *alog = F(13), *dtb = F(14);
    const int B = 2, C = 8192;
    const gdn_tail_params fused = tail_params(4, 128, 1e-6f, 0);
    const gdn_tail_params unf = tail_params(4, 128, 1e-6f, 1);
    const gdn_gate_inputs gin = {ba, alog, dtb};
    const size_t wsb = gdn_layer_tail_ba_workspace_bytes(&PAGE, B);

    stub_reset();
    EXPECT_RC(gdn_layer_tail_ba(&PAGE, &fused, B, x, cw, cs, &gin, state, z, nw, y, NULL, NULL,
                                NULL, 0, STREAM),
              GDN_OK, NULL);
    EXPECT(stub_n_launches() == 1 && kind_is(0, "tail_fused") && L(0)->p[3] == NULL &&
           L(0)->p[4] == NULL && L(0)->p[9] == ba && L(0)->p[10] == alog && L(0)->p[11] == dtb);

    /* three launches after the gate transform: beta and gate at the end of the workspace */
    stub_reset();
    EXPECT_RC(gdn_layer_tail_ba(&PAGE, &unf, B, x, cw, cs, &gin, state, z, nw, y, NULL, NULL, ws,
                                wsb - 4, STREAM),
              GDN_ERR_WORKSPACE, "needed");
    EXPECT_RC(gdn_layer_tail_ba(&PAGE, &unf, B, x, cw, cs, &gin, state, z, nw, y, NULL, NULL, ws,
                                wsb, STREAM),
              GDN_OK, NULL);
    {
        const float *wbeta = ws + (size_t)B * C + (size_t)B * 4096;
        EXPECT(stub_n_launches() == 4 && kind_is(0, "gate") && kind_is(1, "prestate") &&
               kind_is(2, "step") && kind_is(3, "gated_norm"));
        EXPECT(L(0)->p[0] == ba && L(0)->p[3] == wbeta && L(0)->p[4] == wbeta + B * 32 &&
               L(0)->i[0] == B && L(0)->i[1] == 32);
        EXPECT(L(2)->p[3] == wbeta && L(2)->p[4] == wbeta + B * 32);
        EXPECT((const char *)(wbeta + 2 * B * 32) == (const char *)ws + wsb);
    }

    EXPECT_RC(gdn_layer_tail_ba(&PAGE, &fused, B, x, cw, cs, NULL, state, z, nw, y, NULL, NULL,
                                NULL, 0, STREAM),
              GDN_ERR_NULL, "gates is NULL");
    {
        const gdn_gate_inputs nob = {NULL, alog, dtb}, nod = {ba, alog, NULL};
        EXPECT_RC(gdn_layer_tail_ba(&PAGE, &fused, B, x, cw, cs, &nob, state, z, nw, y, NULL,
                                    NULL, NULL, 0, STREAM),
                  GDN_ERR_NULL, "ba is NULL");
        EXPECT_RC(gdn_layer_tail_ba(&PAGE, &fused, B, x, cw, cs, &nod, state, z, nw, y, NULL,
                                    NULL, NULL, 0, STREAM),
                  GDN_ERR_NULL, "dt_bias is NULL");
        const gdn_gate_inputs onstate = {ba, state, dtb};
        EXPECT_RC(gdn_layer_tail_ba(&PAGE, &fused, B, x, cw, cs, &onstate, state, z, nw, y, NULL,
                                    NULL, NULL, 0, STREAM),
                  GDN_ERR_ALIAS, "state overlaps a_log");
    }
}

static void check_tail_pair(void) {
    float *x = F(0), *cw = F(1), *cs = F(2), *beta = F(3), *gate = F(4), *state = F(5),
          *z = F(6), *nw = F(7), *y = F(8), *csn = F(9), *sn = F(10);
    const int B = 6;
    const gdn_tail_params p = tail_params(4, 128, 1e-6f, 0);
    stub_reset();
    EXPECT_RC(gdn_layer_tail_pair(&PAGE, &p, B, x, cw, cs, csn, beta, gate, state, sn, z, nw, y,
                                  STREAM),
              GDN_OK, NULL);
    EXPECT(stub_n_launches() == 1 && kind_is(0, "tail_pair") && L(0)->p[14] == csn &&
           L(0)->p[15] == sn && L(0)->p[2] == cs && L(0)->p[5] == state && L(0)->i[0] == B &&
           L(0)->i[3] == 8192 && L(0)->i[4] == 4 && L(0)->p[9] == NULL);
    /* force_unfused has no meaning for the pair */
    {
        const gdn_tail_params pu = tail_params(4, 128, 1e-6f, 1);
        EXPECT_RC(gdn_layer_tail_pair(&PAGE, &pu, B, x, cw, cs, csn, beta, gate, state, sn, z,
                                      nw, y, STREAM),
                  GDN_OK, NULL);
        EXPECT(stub_n_launches() == 2 && kind_is(1, "tail_pair"));
    }
    {
        const gdn_tail_params k3 = tail_params(3, 128, 1e-6f, 0),
                              g64 = tail_params(4, 64, 1e-6f, 0),
                              bad_eps = tail_params(4, 128, -1.0f, 0);
        const gdn_dims h48 = {48, 16, 128, 128};
        EXPECT_RC(gdn_layer_tail_pair(&PAGE, &k3, B, x, cw, cs, csn, beta, gate, state, sn, z,
                                      nw, y, STREAM),
                  GDN_ERR_SHAPE, "supports conv_kernel 4");
        EXPECT_RC(gdn_layer_tail_pair(&PAGE, &g64, B, x, cw, cs, csn, beta, gate, state, sn, z,
                                      nw, y, STREAM),
                  GDN_ERR_SHAPE, "supports conv_kernel 4");
        EXPECT_RC(gdn_layer_tail_pair(&h48, &p, B, x, cw, cs, csn, beta, gate, state, sn, z, nw,
                                      y, STREAM),
                  GDN_ERR_SHAPE, "supports conv_kernel 4");
        EXPECT_RC(gdn_layer_tail_pair(&PAGE, &bad_eps, B, x, cw, cs, csn, beta, gate, state, sn,
                                      z, nw, y, STREAM),
                  GDN_ERR_SHAPE, "norm_eps");
        EXPECT_RC(gdn_layer_tail_pair(&PAGE, NULL, B, x, cw, cs, csn, beta, gate, state, sn, z,
                                      nw, y, STREAM),
                  GDN_ERR_NULL, "params is NULL");
    }
    EXPECT_RC(gdn_layer_tail_pair(&PAGE, &p, B, x, cw, cs, cs, beta, gate, state, sn, z, nw, y,
                                  STREAM),
              GDN_ERR_ALIAS, "conv_state overlaps conv_state_next");
    EXPECT_RC(gdn_layer_tail_pair(&PAGE, &p, B, x, cw, cs, csn, beta, gate, state, NULL, z, nw, y,
                                  STREAM),
              GDN_ERR_NULL, "state_next is NULL");
    /* y holds two positions: 2 * B * 4096 floats */
    EXPECT_RC(gdn_layer_tail_pair(&PAGE, &p, B, x, cw, cs, csn, beta, gate, state,
                                  y + 2 * B * 4096 - 4, z, nw, y, STREAM),
              GDN_ERR_ALIAS, "overlaps");
    EXPECT_RC(gdn_layer_tail_pair(&PAGE, &p, B, x, cw, cs, csn, beta, gate, state,
                                  y + 2 * B * 4096, z, nw, y, STREAM),
              GDN_OK, NULL);
    EXPECT_RC(gdn_layer_tail_pair(&PAGE, &p, B, x, cw, cs, csn, beta + 1, gate, state, sn, z, nw,
                                  y, STREAM),
              GDN_OK, NULL);
    EXPECT_RC(gdn_layer_tail_pair(&PAGE, &p, B, x + 1, cw, cs, csn, beta, gate, state, sn, z, nw,
                                  y, STREAM),
              GDN_ERR_ALIGN, "x (");
    /* 2 * B * channels up to INT32_MAX / 2 */
    EXPECT_RC(gdn_layer_tail_pair(&PAGE, &p, 65535, x, cw, cs, csn, beta, gate, state, sn, z, nw,
                                  y, STREAM),
              GDN_OK, NULL);
    EXPECT_RC(gdn_layer_tail_pair(&PAGE, &p, 65536, x, cw, cs, csn, beta, gate, state, sn, z, nw,
                                  y, STREAM),
              GDN_ERR_SHAPE, "too large");
}

static void check_noalloc(void) {
    float *x = F(0), *cw = F(1), *cs = F(2), *beta = F(3), *gate = F(4), *state = F(5),
          *z = F(6), *nw = F(7), *y = F(8), *dq = F(10), *dc = F(11);
    const gdn_tail_params fused = tail_params(4, 128, 1e-6f, 0);
    const gdn_tail_params unf = tail_params(4, 128, 1e-6f, 1);
    const float *scr = (const float *)stub_scratch();

    EXPECT(stub_scratch_bytes() == GDN_NOALLOC_SCRATCH_BYTES);
    /* the single launch needs no scratch and does not look it up */
    stub_reset();
    EXPECT_RC(gdn_layer_tail_noalloc(&PAGE, &fused, 7, x, cw, cs, beta, gate, state, z, nw, y,
                                     NULL, NULL, STREAM),
              GDN_OK, NULL);
    EXPECT(stub_n_launches() == 1 && kind_is(0, "tail_fused") && stub_scratch_lookups() == 0);
    /* the three launches split the static scratch as they split a workspace */
    EXPECT_RC(gdn_layer_tail_noalloc(&PAGE, &unf, 7, x, cw, cs, beta, gate, state, z, nw, y, NULL,
                                     NULL, STREAM),
              GDN_OK, NULL);
    EXPECT(stub_n_launches() == 4 && stub_scratch_lookups() == 1);
    EXPECT(L(1)->p[3] == scr && L(2)->p[0] == scr && L(2)->p[6] == scr + 7 * 8192 &&
           L(3)->p[0] == scr + 7 * 8192);
    /* 16 MiB hold 341 sequences at 49152 bytes each; 342 are refused */
    EXPECT_RC(gdn_layer_tail_noalloc(&PAGE, &unf, 341, x, cw, cs, beta, gate, state, z, nw, y,
                                     NULL, NULL, STREAM),
              GDN_OK, NULL);
    EXPECT_RC(gdn_layer_tail_noalloc(&PAGE, &unf, 342, x, cw, cs, beta, gate, state, z, nw, y,
                                     NULL, NULL, STREAM),
              GDN_ERR_WORKSPACE, "needs 16809984 bytes of scratch; the static scratch holds 16777216");
    EXPECT(stub_n_launches() == 7);
    /* with both debug buffers the scratch is not needed at any B */
    EXPECT_RC(gdn_layer_tail_noalloc(&PAGE, &unf, 5000, x, cw, cs, beta, gate, state, z, nw, y,
                                     dq, dc, STREAM),
              GDN_OK, NULL);
    EXPECT(stub_scratch_lookups() == 2 && L(7)->p[3] == dq && L(8)->p[6] == dc);
    EXPECT_RC(gdn_layer_tail_noalloc(&PAGE, &unf, 7, x, cw, cs, beta, gate, (float *)scr + 4, z,
                                     nw, y, NULL, NULL, STREAM),
              GDN_ERR_ALIAS, "state overlaps qkv buffer");
}

static void check_gate_transform(void) {
    float *ba = F(0), *alog = F(1), *dtb = F(2), *beta = F(3), *gate = F(4);
    const gdn_gate_inputs gin = {ba, alog, dtb};
    stub_reset();
    EXPECT_RC(gdn_gate_transform(&PAGE, 9, &gin, beta, gate, STREAM), GDN_OK, NULL);
    EXPECT(stub_n_launches() == 1 && kind_is(0, "gate") && L(0)->p[3] == beta &&
           L(0)->p[4] == gate && L(0)->i[0] == 9 && L(0)->i[1] == 32);
    EXPECT_RC(gdn_gate_transform(&PAGE, 9, NULL, beta, gate, STREAM), GDN_ERR_NULL,
              "gate inputs are NULL");
    EXPECT_RC(gdn_gate_transform(&PAGE, 9, &gin, ba + 5, gate, STREAM), GDN_ERR_ALIAS,
              "beta overlaps ba");
    EXPECT_RC(gdn_gate_transform(&PAGE, 9, &gin, beta, beta + 9 * 32 - 1, STREAM), GDN_ERR_ALIAS,
              "overlaps");
    EXPECT_RC(gdn_gate_transform(&PAGE, 9, &gin, beta, beta + 9 * 32, STREAM), GDN_OK, NULL);
    EXPECT_RC(gdn_gate_transform(&PAGE, 9, &gin, beta, (float *)((char *)gate + 2), STREAM),
              GDN_ERR_ALIGN, "gate (");
    EXPECT_RC(gdn_gate_transform(&PAGE, 0, &gin, beta, gate, STREAM), GDN_ERR_SHAPE, "B must");
}

/* A launch error from the runtime is reported with the launch named, and the
 * launches after it in the same call are not made. */
static void check_launch_errors(void) {
    float *q = F(0), *k = F(1), *v = F(2), *beta = F(3), *gate = F(4), *state = F(5),
          *out = F(6), *ws = F(9);
    const gdn_tail_params unf = tail_params(4, 128, 1e-6f, 1);
    stub_reset();
    stub_fail_launch(0);
    EXPECT_RC(gdn_step(&PAGE, 2, q, k, v, beta, gate, state, out, STREAM), GDN_ERR_HIP,
              "gdn_step launch: stubbed launch failure");
    EXPECT_RC(gdn_step(&PAGE, 2, q, k, v, beta, gate, state, out, STREAM), GDN_OK, NULL);

    stub_reset();
    stub_fail_launch(1);
    EXPECT_RC(gdn_layer_tail(&PAGE, &unf, 2, q, k, v, beta, gate, state, out, F(7), F(8), NULL,
                             NULL, ws, gdn_layer_tail_workspace_bytes(&PAGE, 2), STREAM),
              GDN_ERR_HIP, "gdn_layer_tail step launch");
    EXPECT(stub_n_launches() == 2 && kind_is(0, "prestate") && kind_is(1, "step"));

    stub_reset();
    stub_fail_launch(0);
    EXPECT_RC(gdn_seq(&PAGE, 2, 9, q, k, v, beta, gate, state, out, STREAM), GDN_ERR_HIP,
              "gdn_seq: stubbed");
    stub_reset();
    stub_fail_launch(0);
    EXPECT_RC(gdn_layer_tail_pair(&PAGE, &unf, 2, q, k, v, F(10), beta, gate, state, F(11), out,
                                  F(7), F(8), STREAM),
              GDN_ERR_HIP, "gdn_layer_tail_pair launch");
}

int main(void) {
    EXPECT(gdn_version() == GDN_VERSION);
    check_step();
    check_seq();
    check_pair();
    check_tail();
    check_tail_ba();
    check_tail_pair();
    check_noalloc();
    check_gate_transform();
    check_launch_errors();
    if (failures) {
        printf("C ABI host check: %d of %d checks failed\n", failures, checks);
        return 1;
    }
    printf("C ABI host check ok (%d checks)\n", checks);
    return 0;
}
