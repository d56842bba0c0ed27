// gdn_api_stubs.cpp - host-only stand-ins for the kernel launchers and the
// four HIP runtime calls that gdn_api.cpp makes, so that the C-ABI layer can
// be built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and
// driven on a machine without a GPU (tests/c/gdn_api_check.c).  Every launch
// is recorded instead of enqueued; the check program reads the records back
// to check what the ABI layer passed on.  Test infrastructure, never part of
// libgdn.

#include <hip/hip_runtime_api.h>

#include <cstring>

#include "gdn_launch.hpp"
#include "gdn_api_stubs.h"

namespace {

stub_launch g_log[STUB_MAX_LAUNCHES];
int g_n = 0;
int g_fail_at = -1;  // index of the launch that reports an error, -1: none
int g_scratch_lookups = 0;
alignas(256) unsigned char g_scratch[gdn::kNoAllocScratchBytes];

hipError_t record(const stub_launch &l) {
    const int i = g_n;
    if (g_n < STUB_MAX_LAUNCHES) g_log[g_n++] = l;
    return i == g_fail_at ? hipErrorLaunchFailure : hipSuccess;
}

stub_launch blank(const char *kind, hipStream_t s) {
    stub_launch l;
    std::memset(&l, 0, sizeof l);
    std::strncpy(l.kind, kind, sizeof l.kind - 1);
    l.stream = s;
    return l;
}

}  // namespace

extern "C" {

void stub_reset(void) {
    g_n = 0;
    g_fail_at = -1;
    g_scratch_lookups = 0;
}

void stub_fail_launch(int index) { g_fail_at = g_n + index; }

int stub_n_launches(void) { return g_n; }

const stub_launch *stub_launch_at(int i) { return (i >= 0 && i < g_n) ? &g_log[i] : nullptr; }

int stub_scratch_lookups(void) { return g_scratch_lookups; }

const void *stub_scratch(void) { return g_scratch; }

size_t stub_scratch_bytes(void) { return gdn::kNoAllocScratchBytes; }

int stub_tail_fused_supported(int32_t Hv, int32_t Hk, int32_t K, int32_t group) {
    return gdn::tail_fused_supported(Hv, Hk, K, group) ? 1 : 0;
}

// The HIP runtime calls of gdn_api.cpp: one device, 256 compute units, and
// an error string that names the stub.
hipError_t hipGetDevice(int *d) {
    *d = 0;
    return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t attr, int) {
    *v = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
    return hipSuccess;
}

hipError_t hipGetLastError(void) { return hipSuccess; }

const char *hipGetErrorString(hipError_t e) {
    return e == hipErrorLaunchFailure ? "stubbed launch failure" : "stubbed HIP error";
}

}  // extern "C"

namespace gdn {

hipError_t noalloc_scratch(void **ptr) {
    ++g_scratch_lookups;
    *ptr = g_scratch;
    return hipSuccess;
}

hipError_t launch_step(const StepArgs &a, hipStream_t s, bool cached) {
    stub_launch l = blank("step", s);
    l.p[0] = a.q;
    l.p[1] = a.k;
    l.p[2] = a.v;
    l.p[3] = a.beta;
    l.p[4] = a.gate;
    l.p[5] = a.state;
    l.p[6] = a.out;
    l.i[0] = a.B;
    l.i[1] = a.Hv;
    l.i[2] = a.Hk;
    l.i[3] = cached ? 1 : 0;
    l.l[0] = a.qk_bstride;
    l.l[1] = a.v_bstride;
    return record(l);
}

hipError_t launch_seq(const SeqArgs &a, hipStream_t s, bool exact) {
    stub_launch l = blank(exact ? "seq_exact" : "seq", s);
    l.p[0] = a.q;
    l.p[1] = a.k;
    l.p[2] = a.v;
    l.p[3] = a.beta;
    l.p[4] = a.gate;
    l.p[5] = a.state;
    l.p[6] = a.out;
    l.i[0] = a.B;
    l.i[1] = a.Hv;
    l.i[2] = a.Hk;
    l.i[3] = a.T;
    return record(l);
}

hipError_t launch_pair(const PairArgs &a, hipStream_t s) {
    stub_launch l = blank("pair", s);
    l.p[0] = a.q;
    l.p[1] = a.k;
    l.p[2] = a.v;
    l.p[3] = a.beta;
    l.p[4] = a.gate;
    l.p[5] = a.state;
    l.p[6] = a.out;
    l.p[7] = a.state_next;
    l.i[0] = a.B;
    l.i[1] = a.Hv;
    l.i[2] = a.Hk;
    return record(l);
}

static stub_launch tail_record(const char *kind, const TailFusedArgs &a, hipStream_t s) {
    stub_launch l = blank(kind, s);
    l.p[0] = a.x;
    l.p[1] = a.conv_w;
    l.p[2] = a.conv_state;
    l.p[3] = a.beta;
    l.p[4] = a.gate;
    l.p[5] = a.state;
    l.p[6] = a.z;
    l.p[7] = a.norm_w;
    l.p[8] = a.y;
    l.p[9] = a.ba;
    l.p[10] = a.a_log;
    l.p[11] = a.dt_bias;
    l.p[12] = a.dbg_qkv;
    l.p[13] = a.dbg_core;
    l.p[14] = a.conv_state_next;
    l.p[15] = a.state_next;
    l.i[0] = a.B;
    l.i[1] = a.Hv;
    l.i[2] = a.Hk;
    l.i[3] = a.C;
    l.i[4] = a.K;
    l.f = a.eps;
    return l;
}

hipError_t launch_tail_fused(const TailFusedArgs &a, hipStream_t s) {
    return record(tail_record("tail_fused", a, s));
}

hipError_t launch_tail_pair(const TailFusedArgs &a, hipStream_t s) {
    return record(tail_record("tail_pair", a, s));
}

hipError_t launch_prestate(const PrestateArgs &a, hipStream_t s) {
    stub_launch l = blank("prestate", s);
    l.p[0] = a.x;
    l.p[1] = a.conv_w;
    l.p[2] = a.conv_state;
    l.p[3] = a.qkv;
    l.i[0] = a.B;
    l.i[1] = a.C;
    l.i[2] = a.K;
    l.i[3] = a.n_qk;
    return record(l);
}

hipError_t launch_gated_norm(const GatedNormArgs &a, hipStream_t s) {
    stub_launch l = blank("gated_norm", s);
    l.p[0] = a.o;
    l.p[1] = a.z;
    l.p[2] = a.w;
    l.p[3] = a.y;
    l.i[0] = a.rows;
    l.i[1] = a.n;
    l.i[2] = a.group;
    l.f = a.eps;
    return record(l);
}

hipError_t launch_gate_transform(const GateArgs &a, hipStream_t s) {
    stub_launch l = blank("gate", s);
    l.p[0] = a.ba;
    l.p[1] = a.a_log;
    l.p[2] = a.dt_bias;
    l.p[3] = a.beta;
    l.p[4] = a.gate;
    l.i[0] = a.B;
    l.i[1] = a.Hv;
    return record(l);
}

}  // namespace gdn
