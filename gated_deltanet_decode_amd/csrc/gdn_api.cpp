// gdn_api.cpp - the C ABI declared in include/gdn.h: argument validation,
// error reporting and kernel dispatch.  All validation happens on the host
// before anything is enqueued, so a rejected call leaves every buffer as it
// was and never touches the GPU.

#include "gdn.h"

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "gdn_launch.hpp"

namespace gdn {

// A value that never changes; relaxed atomics make concurrent first calls
// from several host threads well defined.
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace gdn

namespace {

thread_local char g_error[512];

void clear_error() { g_error[0] = '\0'; }

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return code;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Do [a, a+na) and [b, b+nb) share a byte?
bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

struct Buf {
    const char *name;
    const void *p;
    size_t bytes;
};

// Every output must be disjoint from every other listed buffer.
int check_alias(const Buf *outs, int n_out, const Buf *all, int n_all) {
    for (int i = 0; i < n_out; ++i)
        for (int j = 0; j < n_all; ++j) {
            if (outs[i].p == all[j].p && outs[i].name == all[j].name) continue;  // itself
            if (overlap(outs[i].p, outs[i].bytes, all[j].p, all[j].bytes))
                return fail(GDN_ERR_ALIAS, "%s overlaps %s", outs[i].name, all[j].name);
        }
    return GDN_OK;
}

int check_dims(const gdn_dims *d) {
    if (!d) return fail(GDN_ERR_NULL, "dims is NULL");
    if (d->n_v_heads < 1 || d->n_k_heads < 1)
        return fail(GDN_ERR_SHAPE, "head counts must be >= 1 (n_v_heads=%d, n_k_heads=%d)",
                    d->n_v_heads, d->n_k_heads);
    if (d->n_v_heads % d->n_k_heads != 0)
        return fail(GDN_ERR_SHAPE, "n_v_heads=%d is not a multiple of n_k_heads=%d",
                    d->n_v_heads, d->n_k_heads);
    if (d->d_k != gdn::kHeadDim || d->d_v != gdn::kHeadDim)
        return fail(GDN_ERR_SHAPE, "only d_k = d_v = %d is supported (got d_k=%d, d_v=%d)",
                    gdn::kHeadDim, d->d_k, d->d_v);
    return GDN_OK;
}

// Heads of one call map to workgroups along grid x, and the persistent
// kernels count 16 row tiles per head in a 32-bit index that may run up to
// one grid stride (at most 65536 tiles) past the last tile.
int check_batch(const gdn_dims *d, int64_t B, const char *what) {
    if (B < 1) return fail(GDN_ERR_SHAPE, "%s must be >= 1 (got %lld)", what, (long long)B);
    const int64_t limit = (static_cast<int64_t>(INT32_MAX) - 65536) / 16;   // 134213631
    if (B * d->n_v_heads > limit)
        return fail(GDN_ERR_SHAPE, "B * n_v_heads = %lld exceeds %lld",
                    (long long)(B * d->n_v_heads), (long long)limit);
    return GDN_OK;
}

#define GDN_TRY(expr)               \
    do {                            \
        const int rc__ = (expr);    \
        if (rc__ != GDN_OK) return rc__; \
    } while (0)

int check_ptrs(const Buf *bufs, int n, uintptr_t align) {
    for (int i = 0; i < n; ++i) {
        if (!bufs[i].p) return fail(GDN_ERR_NULL, "%s is NULL", bufs[i].name);
        if (!aligned(bufs[i].p, align))
            return fail(GDN_ERR_ALIGN, "%s (%p) is not %u-byte aligned", bufs[i].name, bufs[i].p,
                        static_cast<unsigned>(align));
    }
    return GDN_OK;
}

int hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess)
        return fail(GDN_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), static_cast<int>(e));
    return GDN_OK;
}

// gdn_seq and gdn_seq_exact: checks, then the launch (exact: no scaled groups).
int seq_call(const char *name, bool exact, const gdn_dims *dims, int32_t B, int32_t T,
             const float *q, const float *k, const float *v, const float *beta,
             const float *gate, float *state, float *out, void *stream) {
    clear_error();
    GDN_TRY(check_dims(dims));
    GDN_TRY(check_batch(dims, B, "B"));
    // 2^30 keeps the kernels' 32-bit token arithmetic (t + chunk length)
    // clear of overflow; no buffer of that many tokens fits a GPU.
    if (T < 1 || T > (1 << 30))
        return fail(GDN_ERR_SHAPE, "T must be in [1, 1073741824] (got %d)", T);
    // the launch must fit the dispatch's 32-bit work-item count
    if (static_cast<int64_t>(B) * dims->n_v_heads * gdn::kSeqThreadsPerHead > UINT32_MAX)
        return fail(GDN_ERR_SHAPE, "%s: B * n_v_heads = %lld exceeds %lld", name,
                    (long long)(static_cast<int64_t>(B) * dims->n_v_heads),
                    (long long)(UINT32_MAX / gdn::kSeqThreadsPerHead));
    const size_t f = sizeof(float);
    const size_t BT = static_cast<size_t>(B) * T;
    const size_t nqk = BT * dims->n_k_heads * dims->d_k * f;
    const size_t nv = BT * dims->n_v_heads * dims->d_v * f;
    const size_t nh = BT * dims->n_v_heads * f;
    const size_t ns = static_cast<size_t>(B) * dims->n_v_heads * dims->d_v * dims->d_k * f;
    const Buf vec[] = {{"q", q, nqk}, {"k", k, nqk}, {"v", v, nv}, {"state", state, ns},
                       {"out", out, nv}};
    const Buf sc[] = {{"beta", beta, nh}, {"gate", gate, nh}};
    GDN_TRY(check_ptrs(vec, 5, 16));
    GDN_TRY(check_ptrs(sc, 2, 4));
    const Buf all[] = {vec[0], vec[1], vec[2], vec[3], vec[4], sc[0], sc[1]};
    const Buf outs[] = {vec[3], vec[4]};
    GDN_TRY(check_alias(outs, 2, all, 7));

    gdn::SeqArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.gate = gate;
    a.state = state;
    a.out = out;
    a.B = B;
    a.T = T;
    a.Hv = dims->n_v_heads;
    a.Hk = dims->n_k_heads;
    (void)hipGetLastError();
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 1) {
        // one token is gdn_step (same per-row arithmetic, same bits): the
        // streaming kernel moves the state faster than the multi-token one
        gdn::StepArgs sa{};
        sa.q = q;
        sa.k = k;
        sa.v = v;
        sa.beta = beta;
        sa.gate = gate;
        sa.state = state;
        sa.out = out;
        sa.qk_bstride = static_cast<int64_t>(dims->n_k_heads) * dims->d_k;
        sa.v_bstride = static_cast<int64_t>(dims->n_v_heads) * dims->d_v;
        sa.B = B;
        sa.Hv = dims->n_v_heads;
        sa.Hk = dims->n_k_heads;
        return hip_status(gdn::launch_step(sa, s), name);
    }
    return hip_status(gdn::launch_seq(a, s, exact), name);
}

}  // namespace

extern "C" {

int gdn_version(void) { return GDN_VERSION; }

const char *gdn_last_error(void) { return g_error; }

int gdn_step(const gdn_dims *dims, int32_t B, const float *q, const float *k, const float *v,
             const float *beta, const float *gate, float *state, float *out, void *stream) {
    return gdn_step_ex(dims, B, q, k, v, beta, gate, state, out, 0u, stream);
}

int gdn_step_ex(const gdn_dims *dims, int32_t B, const float *q, const float *k, const float *v,
                const float *beta, const float *gate, float *state, float *out, uint32_t flags,
                void *stream) {
    clear_error();
    if (flags & ~static_cast<uint32_t>(GDN_STATE_CACHED))
        return fail(GDN_ERR_SHAPE, "unknown flags 0x%x", flags & ~GDN_STATE_CACHED);
    GDN_TRY(check_dims(dims));
    GDN_TRY(check_batch(dims, B, "B"));
    const size_t f = sizeof(float);
    const size_t nqk = static_cast<size_t>(B) * dims->n_k_heads * dims->d_k * f;
    const size_t nv = static_cast<size_t>(B) * dims->n_v_heads * dims->d_v * f;
    const size_t nh = static_cast<size_t>(B) * dims->n_v_heads * f;
    const size_t ns = static_cast<size_t>(B) * dims->n_v_heads * dims->d_v * dims->d_k * f;
    const Buf vec[] = {{"q", q, nqk}, {"k", k, nqk}, {"v", v, nv}, {"state", state, ns},
                       {"out", out, nv}};
    const Buf sc[] = {{"beta", beta, nh}, {"gate", gate, nh}};
    GDN_TRY(check_ptrs(vec, 5, 16));
    GDN_TRY(check_ptrs(sc, 2, 4));
    const Buf all[] = {vec[0], vec[1], vec[2], vec[3], vec[4], sc[0], sc[1]};
    const Buf outs[] = {vec[3], vec[4]};  // state and out are written
    GDN_TRY(check_alias(outs, 2, all, 7));

    gdn::StepArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.gate = gate;
    a.state = state;
    a.out = out;
    a.qk_bstride = static_cast<int64_t>(dims->n_k_heads) * dims->d_k;
    a.v_bstride = static_cast<int64_t>(dims->n_v_heads) * dims->d_v;
    a.B = B;
    a.Hv = dims->n_v_heads;
    a.Hk = dims->n_k_heads;
    (void)hipGetLastError();  // do not report an earlier, unrelated error
    return hip_status(gdn::launch_step(a, static_cast<hipStream_t>(stream),
                                       (flags & GDN_STATE_CACHED) != 0),
                      "gdn_step launch");
}

int gdn_seq(const gdn_dims *dims, int32_t B, int32_t T, const float *q, const float *k,
            const float *v, const float *beta, const float *gate, float *state, float *out,
            void *stream) {
    return seq_call("gdn_seq", false, dims, B, T, q, k, v, beta, gate, state, out, stream);
}

int gdn_seq_exact(const gdn_dims *dims, int32_t B, int32_t T, const float *q, const float *k,
                  const float *v, const float *beta, const float *gate, float *state, float *out,
                  void *stream) {
    return seq_call("gdn_seq_exact", true, dims, B, T, q, k, v, beta, gate, state, out, stream);
}

int gdn_pair(const gdn_dims *dims, int32_t B, const float *q, const float *k, const float *v,
             const float *beta, const float *gate, float *state, float *state_next, float *out,
             void *stream) {
    clear_error();
    GDN_TRY(check_dims(dims));
    GDN_TRY(check_batch(dims, B, "B"));
    const size_t f = sizeof(float);
    const size_t B2 = static_cast<size_t>(B) * 2;
    const size_t nqk = B2 * dims->n_k_heads * dims->d_k * f;
    const size_t nv = B2 * dims->n_v_heads * dims->d_v * f;
    const size_t nh = B2 * dims->n_v_heads * f;
    const size_t ns = static_cast<size_t>(B) * dims->n_v_heads * dims->d_v * dims->d_k * f;
    const Buf vec[] = {{"q", q, nqk},     {"k", k, nqk},
                       {"v", v, nv},      {"state", state, ns},
                       {"out", out, nv},  {"state_next", state_next, ns}};
    const Buf sc[] = {{"beta", beta, nh}, {"gate", gate, nh}};
    GDN_TRY(check_ptrs(vec, 6, 16));
    GDN_TRY(check_ptrs(sc, 2, 4));
    const Buf all[] = {vec[0], vec[1], vec[2], vec[3], vec[4], vec[5], sc[0], sc[1]};
    const Buf outs[] = {vec[3], vec[4], vec[5]};
    GDN_TRY(check_alias(outs, 3, all, 8));

    gdn::PairArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.gate = gate;
    a.state = state;
    a.state_next = state_next;
    a.out = out;
    a.B = B;
    a.Hv = dims->n_v_heads;
    a.Hk = dims->n_k_heads;
    (void)hipGetLastError();
    return hip_status(gdn::launch_pair(a, static_cast<hipStream_t>(stream)), "gdn_pair launch");
}

size_t gdn_layer_tail_workspace_bytes(const gdn_dims *dims, int32_t B) {
    if (!dims || B < 1 || dims->n_v_heads < 1 || dims->n_k_heads < 1 || dims->d_k < 1 ||
        dims->d_v < 1)
        return 0;
    const size_t C = 2 * static_cast<size_t>(dims->n_k_heads) * dims->d_k +
                     static_cast<size_t>(dims->n_v_heads) * dims->d_v;
    const size_t qkv = static_cast<size_t>(B) * C * sizeof(float);
    const size_t core = static_cast<size_t>(B) * dims->n_v_heads * dims->d_v * sizeof(float);
    return qkv + core;  // both parts are multiples of 16 bytes (d_k = d_v = 128)
}

}  // extern "C"

namespace {

// Checks the raw gate inputs of B sequences.
int check_gate_inputs(const gdn_dims *dims, int32_t B, const gdn_gate_inputs *in, Buf *bufs) {
    if (!in) return fail(GDN_ERR_NULL, "gate inputs are NULL");
    const size_t f = sizeof(float);
    bufs[0] = {"ba", in->ba, static_cast<size_t>(B) * 2 * dims->n_v_heads * f};
    bufs[1] = {"a_log", in->a_log, static_cast<size_t>(dims->n_v_heads) * f};
    bufs[2] = {"dt_bias", in->dt_bias, static_cast<size_t>(dims->n_v_heads) * f};
    return check_ptrs(bufs, 3, 4);
}

// The layer tail with beta/gate given (raw == NULL) or computed from the raw
// gate inputs.  With raw inputs the unfused path writes beta and gate to the
// end of the workspace first.  noalloc: the workspace is the library's static
// per-GPU scratch instead of a caller's buffer.
int layer_tail(const char *name, const gdn_dims *dims, const gdn_tail_params *params, int32_t B,
               const float *x, const float *conv_w, float *conv_state, const float *beta,
               const float *gate, const gdn_gate_inputs *raw, float *state, const float *z,
               const float *norm_w, float *y, float *dbg_qkv, float *dbg_core, void *workspace,
               size_t workspace_bytes, void *stream, bool noalloc = false) {
    GDN_TRY(check_dims(dims));
    if (!params) return fail(GDN_ERR_NULL, "params is NULL");
    GDN_TRY(check_batch(dims, B, "B"));
    const int K = params->conv_kernel;
    if (K < 2 || K > 8) return fail(GDN_ERR_SHAPE, "conv_kernel must be in 2..8 (got %d)", K);
    const int64_t nvw = static_cast<int64_t>(dims->n_v_heads) * dims->d_v;
    if (params->norm_group < 1 || nvw % params->norm_group != 0)
        return fail(GDN_ERR_SHAPE, "norm_group=%d must be >= 1 and divide n_v_heads*d_v=%lld",
                    params->norm_group, (long long)nvw);
    if (!(params->norm_eps >= 0.0f) || params->norm_eps > 3.0e38f)
        return fail(GDN_ERR_SHAPE, "norm_eps must be finite and >= 0");
    const int64_t C = 2 * static_cast<int64_t>(dims->n_k_heads) * dims->d_k + nvw;
    if (C * B > INT32_MAX / 2)
        return fail(GDN_ERR_SHAPE, "B * channels = %lld too large", (long long)(C * B));
    // one gated-norm workgroup per sequence and group: its launch must fit the
    // dispatch's 32-bit work-item count
    if (static_cast<int64_t>(B) * (nvw / params->norm_group) * gdn::kGatedNormThreads > UINT32_MAX)
        return fail(GDN_ERR_SHAPE, "B * n_v_heads * d_v / norm_group = %lld groups too many",
                    (long long)(static_cast<int64_t>(B) * (nvw / params->norm_group)));

    const size_t f = sizeof(float);
    const size_t nx = static_cast<size_t>(B) * C * f;
    const size_t nw = static_cast<size_t>(C) * K * f;
    const size_t ncs = static_cast<size_t>(B) * (K - 1) * C * f;
    const size_t nh = static_cast<size_t>(B) * dims->n_v_heads * f;
    const size_t ns = static_cast<size_t>(B) * dims->n_v_heads * dims->d_v * dims->d_k * f;
    const size_t nz = static_cast<size_t>(B) * nvw * f;
    const size_t nnw = static_cast<size_t>(params->norm_group) * f;

    const Buf vec[] = {{"x", x, nx}, {"conv_state", conv_state, ncs}, {"state", state, ns},
                       {"z", z, nz}, {"y", y, nz}};
    Buf sc[6] = {{"conv_w", conv_w, nw}, {"norm_w", norm_w, nnw}, {"beta", beta, nh},
                 {"gate", gate, nh}};
    int n_sc = 4;
    if (raw) {
        GDN_TRY(check_gate_inputs(dims, B, raw, sc + 2));
        n_sc = 5;
    }
    GDN_TRY(check_ptrs(vec, 5, 16));
    GDN_TRY(check_ptrs(sc, n_sc, 4));
    if (dbg_qkv && !aligned(dbg_qkv, 16)) return fail(GDN_ERR_ALIGN, "dbg_qkv is not 16-byte aligned");
    if (dbg_core && !aligned(dbg_core, 16))
        return fail(GDN_ERR_ALIGN, "dbg_core is not 16-byte aligned");

    // The single launch keeps Q|K|V, the step output and beta/gate on chip;
    // only the three-launch path stages them in the workspace (or in the
    // debug buffers when they are given).
    const bool fused = !params->force_unfused &&
                       gdn::tail_fused_supported(dims->n_v_heads, dims->n_k_heads, K,
                                                 params->norm_group);
    const size_t need =
        fused ? 0 : (dbg_qkv ? 0 : nx) + (dbg_core ? 0 : nz) + (raw ? 2 * nh : 0);
    if (noalloc && need > 0) {
        if (need > gdn::kNoAllocScratchBytes)
            return fail(GDN_ERR_WORKSPACE,
                        "%s needs %zu bytes of scratch; the static scratch holds %zu", name, need,
                        gdn::kNoAllocScratchBytes);
        GDN_TRY(hip_status(gdn::noalloc_scratch(&workspace), "static scratch lookup"));
        workspace_bytes = gdn::kNoAllocScratchBytes;
    }
    if (need > 0) {
        if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
        if (!aligned(workspace, 16)) return fail(GDN_ERR_ALIGN, "workspace is not 16-byte aligned");
        if (workspace_bytes < need)
            return fail(GDN_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes,
                        need);
    }
    float *ws = need > 0 ? static_cast<float *>(workspace) : nullptr;
    float *qkv = dbg_qkv ? dbg_qkv : ws;
    float *core = dbg_core ? dbg_core : (ws ? ws + (dbg_qkv ? 0 : nx / f) : nullptr);
    float *wbeta = (raw && ws) ? ws + ((dbg_qkv ? 0 : nx) + (dbg_core ? 0 : nz)) / f : nullptr;
    float *wgate = wbeta ? wbeta + nh / f : nullptr;
    if (raw && !fused) {
        beta = wbeta;
        gate = wgate;
    }

    // Every written buffer (conv_state, state, y and the intermediates) must be
    // disjoint from every other buffer; outputs are copies of entries of all[].
    Buf all[16];
    int n_all = 0;
    for (const Buf &b : vec) all[n_all++] = b;
    for (int i = 0; i < n_sc; ++i) all[n_all++] = sc[i];
    const int i_mid = n_all;
    all[n_all++] = {"qkv buffer", qkv, nx};
    all[n_all++] = {"core buffer", core, nz};
    if (raw) {
        all[n_all++] = {"beta buffer", wbeta, nh};
        all[n_all++] = {"gate buffer", wgate, nh};
    }
    Buf outs[7] = {vec[1], vec[2], vec[4]};
    int n_out = 3;
    for (int i = i_mid; i < n_all; ++i) outs[n_out++] = all[i];
    GDN_TRY(check_alias(outs, n_out, all, n_all));

    const hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    char what[96];

    if (fused) {
        gdn::TailFusedArgs fa{};
        fa.x = x;
        fa.conv_w = conv_w;
        fa.conv_state = conv_state;
        fa.beta = raw ? nullptr : beta;
        fa.gate = raw ? nullptr : gate;
        fa.ba = raw ? raw->ba : nullptr;
        fa.a_log = raw ? raw->a_log : nullptr;
        fa.dt_bias = raw ? raw->dt_bias : nullptr;
        fa.state = state;
        fa.z = z;
        fa.norm_w = norm_w;
        fa.y = y;
        fa.dbg_qkv = dbg_qkv;
        fa.dbg_core = dbg_core;
        fa.B = B;
        fa.Hv = dims->n_v_heads;
        fa.Hk = dims->n_k_heads;
        fa.C = static_cast<int32_t>(C);
        fa.K = K;
        fa.eps = params->norm_eps;
        snprintf(what, sizeof what, "%s fused launch", name);
        return hip_status(gdn::launch_tail_fused(fa, s), what);
    }

    if (raw) {
        gdn::GateArgs ga{};
        ga.ba = raw->ba;
        ga.a_log = raw->a_log;
        ga.dt_bias = raw->dt_bias;
        ga.beta = wbeta;
        ga.gate = wgate;
        ga.B = B;
        ga.Hv = dims->n_v_heads;
        snprintf(what, sizeof what, "%s gate-transform launch", name);
        GDN_TRY(hip_status(gdn::launch_gate_transform(ga, s), what));
    }

    gdn::PrestateArgs pa{};
    pa.x = x;
    pa.conv_w = conv_w;
    pa.conv_state = conv_state;
    pa.qkv = qkv;
    pa.B = B;
    pa.C = static_cast<int32_t>(C);
    pa.K = K;
    pa.n_qk = 2 * dims->n_k_heads * dims->d_k;
    snprintf(what, sizeof what, "%s prestate launch", name);
    GDN_TRY(hip_status(gdn::launch_prestate(pa, s), what));

    gdn::StepArgs sa{};
    sa.q = qkv;
    sa.k = qkv + static_cast<int64_t>(dims->n_k_heads) * dims->d_k;
    sa.v = qkv + pa.n_qk;
    sa.beta = beta;
    sa.gate = gate;
    sa.state = state;
    sa.out = core;
    sa.qk_bstride = C;
    sa.v_bstride = C;
    sa.B = B;
    sa.Hv = dims->n_v_heads;
    sa.Hk = dims->n_k_heads;
    snprintf(what, sizeof what, "%s step launch", name);
    GDN_TRY(hip_status(gdn::launch_step(sa, s), what));

    gdn::GatedNormArgs na{};
    na.o = core;
    na.z = z;
    na.w = norm_w;
    na.y = y;
    na.rows = B;
    na.n = static_cast<int32_t>(nvw);
    na.group = params->norm_group;
    na.eps = params->norm_eps;
    snprintf(what, sizeof what, "%s gated-norm launch", name);
    return hip_status(gdn::launch_gated_norm(na, s), what);
}

}  // namespace

extern "C" {

int gdn_layer_tail(const gdn_dims *dims, const gdn_tail_params *params, int32_t B,
                   const float *x, const float *conv_w, float *conv_state, const float *beta,
                   const float *gate, float *state, const float *z, const float *norm_w, float *y,
                   float *dbg_qkv, float *dbg_core, void *workspace, size_t workspace_bytes,
                   void *stream) {
    clear_error();
    return layer_tail("gdn_layer_tail", dims, params, B, x, conv_w, conv_state, beta, gate,
                      nullptr, state, z, norm_w, y, dbg_qkv, dbg_core, workspace,
                      workspace_bytes, stream);
}

int gdn_layer_tail_ba(const gdn_dims *dims, const gdn_tail_params *params, int32_t B,
                      const float *x, const float *conv_w, float *conv_state,
                      const gdn_gate_inputs *gates, float *state, const float *z,
                      const float *norm_w, float *y, float *dbg_qkv, float *dbg_core,
                      void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    if (!gates) return fail(GDN_ERR_NULL, "gates is NULL");
    return layer_tail("gdn_layer_tail_ba", dims, params, B, x, conv_w, conv_state, nullptr,
                      nullptr, gates, state, z, norm_w, y, dbg_qkv, dbg_core, workspace,
                      workspace_bytes, stream);
}

int gdn_layer_tail_pair(const gdn_dims *dims, const gdn_tail_params *params, int32_t B,
                        const float *x, const float *conv_w, float *conv_state,
                        float *conv_state_next, const float *beta, const float *gate,
                        float *state, float *state_next, const float *z, const float *norm_w,
                        float *y, void *stream) {
    clear_error();
    GDN_TRY(check_dims(dims));
    if (!params) return fail(GDN_ERR_NULL, "params is NULL");
    GDN_TRY(check_batch(dims, B, "B"));
    const int K = params->conv_kernel;
    if (!gdn::tail_fused_supported(dims->n_v_heads, dims->n_k_heads, K, params->norm_group))
        return fail(GDN_ERR_SHAPE,
                    "gdn_layer_tail_pair supports conv_kernel 4, norm_group = d_v and n_v_heads "
                    "= n_k_heads or 2 * n_k_heads (got %d, %d, %d, %d)",
                    K, params->norm_group, dims->n_v_heads, dims->n_k_heads);
    if (!(params->norm_eps >= 0.0f) || params->norm_eps > 3.0e38f)
        return fail(GDN_ERR_SHAPE, "norm_eps must be finite and >= 0");
    const int64_t nvw = static_cast<int64_t>(dims->n_v_heads) * dims->d_v;
    const int64_t C = 2 * static_cast<int64_t>(dims->n_k_heads) * dims->d_k + nvw;
    if (2 * C * B > INT32_MAX / 2)
        return fail(GDN_ERR_SHAPE, "B * 2 * channels = %lld too large", (long long)(2 * C * B));

    const size_t f = sizeof(float);
    const size_t nx = static_cast<size_t>(B) * 2 * C * f;
    const size_t nw = static_cast<size_t>(C) * K * f;
    const size_t ncs = static_cast<size_t>(B) * (K - 1) * C * f;
    const size_t nh = static_cast<size_t>(B) * 2 * dims->n_v_heads * f;
    const size_t ns = static_cast<size_t>(B) * dims->n_v_heads * dims->d_v * dims->d_k * f;
    const size_t nz = static_cast<size_t>(B) * 2 * nvw * f;
    const size_t nnw = static_cast<size_t>(params->norm_group) * f;
    const Buf vec[] = {{"x", x, nx},
                       {"conv_state", conv_state, ncs},
                       {"conv_state_next", conv_state_next, ncs},
                       {"state", state, ns},
                       {"state_next", state_next, ns},
                       {"z", z, nz},
                       {"y", y, nz}};
    const Buf sc[] = {{"conv_w", conv_w, nw}, {"norm_w", norm_w, nnw}, {"beta", beta, nh},
                      {"gate", gate, nh}};
    GDN_TRY(check_ptrs(vec, 7, 16));
    GDN_TRY(check_ptrs(sc, 4, 4));
    const Buf all[] = {vec[0], vec[1], vec[2], vec[3], vec[4], vec[5], vec[6],
                       sc[0],  sc[1],  sc[2],  sc[3]};
    const Buf outs[] = {vec[1], vec[2], vec[3], vec[4], vec[6]};
    GDN_TRY(check_alias(outs, 5, all, 11));

    gdn::TailFusedArgs fa{};
    fa.x = x;
    fa.conv_w = conv_w;
    fa.conv_state = conv_state;
    fa.conv_state_next = conv_state_next;
    fa.beta = beta;
    fa.gate = gate;
    fa.state = state;
    fa.state_next = state_next;
    fa.z = z;
    fa.norm_w = norm_w;
    fa.y = y;
    fa.B = B;
    fa.Hv = dims->n_v_heads;
    fa.Hk = dims->n_k_heads;
    fa.C = static_cast<int32_t>(C);
    fa.K = K;
    fa.eps = params->norm_eps;
    (void)hipGetLastError();
    return hip_status(gdn::launch_tail_pair(fa, static_cast<hipStream_t>(stream)),
                      "gdn_layer_tail_pair launch");
}

int gdn_layer_tail_noalloc(const gdn_dims *dims, const gdn_tail_params *params, int32_t B,
                           const float *x, const float *conv_w, float *conv_state,
                           const float *beta, const float *gate, float *state, const float *z,
                           const float *norm_w, float *y, float *dbg_qkv, float *dbg_core,
                           void *stream) {
    clear_error();
    return layer_tail("gdn_layer_tail_noalloc", dims, params, B, x, conv_w, conv_state, beta,
                      gate, nullptr, state, z, norm_w, y, dbg_qkv, dbg_core, nullptr, 0, stream,
                      true);
}

size_t gdn_layer_tail_ba_workspace_bytes(const gdn_dims *dims, int32_t B) {
    const size_t base = gdn_layer_tail_workspace_bytes(dims, B);
    if (base == 0) return 0;
    return base + 2 * static_cast<size_t>(B) * dims->n_v_heads * sizeof(float);
}

int gdn_gate_transform(const gdn_dims *dims, int32_t B, const gdn_gate_inputs *in, float *beta,
                       float *gate, void *stream) {
    clear_error();
    GDN_TRY(check_dims(dims));
    GDN_TRY(check_batch(dims, B, "B"));
    Buf inb[3];
    GDN_TRY(check_gate_inputs(dims, B, in, inb));
    const size_t nh = static_cast<size_t>(B) * dims->n_v_heads * sizeof(float);
    const Buf ob[] = {{"beta", beta, nh}, {"gate", gate, nh}};
    GDN_TRY(check_ptrs(ob, 2, 4));
    const Buf all[] = {inb[0], inb[1], inb[2], ob[0], ob[1]};
    GDN_TRY(check_alias(ob, 2, all, 5));

    gdn::GateArgs a{};
    a.ba = in->ba;
    a.a_log = in->a_log;
    a.dt_bias = in->dt_bias;
    a.beta = beta;
    a.gate = gate;
    a.B = B;
    a.Hv = dims->n_v_heads;
    (void)hipGetLastError();
    return hip_status(gdn::launch_gate_transform(a, static_cast<hipStream_t>(stream)),
                      "gdn_gate_transform launch");
}

}  // extern "C"
