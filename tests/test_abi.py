"""CPU: the C-ABI library loads, exports every entry point include/gdn.h
declares, and rejects bad arguments with the documented codes before it
touches the GPU (no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def g():
    import gated_deltanet_decode_amd as g
    return g


def declared_functions():
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol(g):
    names = declared_functions()
    assert {"gdn_step", "gdn_seq", "gdn_pair", "gdn_layer_tail", "gdn_layer_tail_workspace_bytes",
            "gdn_gate_transform", "gdn_layer_tail_ba", "gdn_layer_tail_ba_workspace_bytes",
            "gdn_last_error", "gdn_version"} <= set(names)
    for n in names:
        assert hasattr(g.lib, n), f"{n} not exported"
    nm = os.popen(f"nm -D --defined-only {g.LIBRARY}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", nm), f"{n} missing from the dynamic symbol table"


def test_version_and_codes_match_header(g):
    hdr = open(os.path.join(ROOT, "include", "gdn.h")).read()
    assert g.version() == int(re.search(r"#define GDN_VERSION (\d+)", hdr).group(1))
    for name, val in re.findall(r"#define (GDN_(?:OK|ERR_\w+))\s+\(?(-?\d+)\)?", hdr):
        assert g.ERRORS[int(val)] == name


# Fake, well-aligned, disjoint "device" addresses: validation only looks at
# the numbers, and every case below fails before any launch.
B, HV, HK, D = 2, 32, 16, 128
BASE = 1 << 40


def addrs():
    sz = {"q": B * HK * D * 4, "k": B * HK * D * 4, "v": B * HV * D * 4,
          "beta": B * HV * 4, "gate": B * HV * 4, "state": B * HV * D * D * 4,
          "out": B * HV * D * 4}
    a, p = {}, BASE
    for n in ("q", "k", "v", "beta", "gate", "state", "out"):
        a[n] = p
        p += (sz[n] + 4095) // 4096 * 4096
    return a, sz


def call_step(g, dims, Bv, a):
    return g.lib.gdn_step(ctypes.byref(dims) if dims is not None else None, Bv,
                          a["q"], a["k"], a["v"], a["beta"], a["gate"], a["state"], a["out"], None)


def expect(g, rc, code, needle):
    assert rc == code, f"rc={rc} ({g.ERRORS.get(rc)}), expected {g.ERRORS[code]}: {g.last_error()}"
    assert needle in g.last_error(), g.last_error()


def test_step_validation(g):
    a, sz = addrs()
    d = g.Dims(HV, HK, D, D)
    expect(g, call_step(g, None, B, a), -1, "dims")
    for n in a:
        bad = dict(a, **{n: None})
        expect(g, call_step(g, d, B, bad), -1, n)
    expect(g, call_step(g, d, 0, a), -2, "B")
    expect(g, call_step(g, d, -3, a), -2, "B")
    expect(g, call_step(g, g.Dims(32, 12, D, D), B, a), -2, "multiple")
    expect(g, call_step(g, g.Dims(32, 16, 64, 64), B, a), -2, "d_k")
    expect(g, call_step(g, g.Dims(32, 16, 128, 64), B, a), -2, "d_v")
    expect(g, call_step(g, g.Dims(0, 16, 128, 128), B, a), -2, "head")
    expect(g, call_step(g, d, (1 << 31) // 32 + 1, a), -2, "exceeds")
    # one past the largest accepted B * n_v_heads (134213631, which leaves one
    # grid stride of headroom below INT32_MAX for the 32-bit tile index)
    expect(g, call_step(g, d, 134213631 // 32 + 1, a), -2, "exceeds")
    for n in ("q", "k", "v", "state", "out"):
        expect(g, call_step(g, d, B, dict(a, **{n: a[n] + 8})), -3, n)
    for n in ("beta", "gate"):
        expect(g, call_step(g, d, B, dict(a, **{n: a[n] + 2})), -3, n)
    # out overlapping state, q, or the tail of v; state overlapping k
    expect(g, call_step(g, d, B, dict(a, out=a["state"] + 4096)), -4, "out")
    expect(g, call_step(g, d, B, dict(a, out=a["q"])), -4, "out")
    expect(g, call_step(g, d, B, dict(a, out=a["v"] + sz["v"] - 16)), -4, "out")
    expect(g, call_step(g, d, B, dict(a, state=a["k"] - 16)), -4, "state")


@pytest.mark.parametrize("name", ["gdn_seq", "gdn_seq_exact"])
def test_seq_validation(g, name):
    a, _ = addrs()
    d = g.Dims(HV, HK, D, D)
    fn = getattr(g.lib, name)
    f = lambda T, aa: fn(ctypes.byref(d), B, T, aa["q"], aa["k"], aa["v"],
                         aa["beta"], aa["gate"], aa["state"], aa["out"], None)
    expect(g, f(0, a), -2, "T")
    expect(g, f(-1, a), -2, "T")
    expect(g, f((1 << 30) + 1, a), -2, "T")
    expect(g, f(2**31 - 1, a), -2, "T")
    # 2^23 heads: 512 work-items each would overflow the 32-bit dispatch grid
    big = lambda Bv: fn(ctypes.byref(d), Bv, 4, a["q"], a["k"], a["v"], a["beta"],
                        a["gate"], a["state"], a["out"], None)
    expect(g, big((1 << 23) // HV), -2, f"{name}: B * n_v_heads")
    expect(g, f(4, dict(a, gate=None)), -1, "gate")
    expect(g, f(4, dict(a, v=a["v"] + 4)), -3, "v")
    expect(g, f(1, dict(a, out=a["state"] - 16)), -4, "out")
    # the fake layout is sized for T = 1: with T = 4, k runs into the state
    expect(g, f(4, a), -4, "state")


def test_pair_validation(g):
    a, sz = addrs()
    d = g.Dims(HV, HK, D, D)
    nxt = BASE + (1 << 36)

    def f(aa, n=nxt, Bv=1):
        return g.lib.gdn_pair(ctypes.byref(d), Bv, aa["q"], aa["k"], aa["v"], aa["beta"],
                              aa["gate"], aa["state"], n, aa["out"], None)
    expect(g, f(a, n=None), -1, "state_next")
    expect(g, f(a, n=nxt + 8), -3, "state_next")
    expect(g, f(a, n=a["state"]), -4, "state")
    expect(g, f(a, n=a["state"] + sz["state"] // 2 - 4096), -4, "state")
    expect(g, f(a, Bv=0), -2, "B")
    # with B = 1 the two positions fill exactly the B = 2 single-step slots
    expect(g, f(dict(a, out=a["k"])), -4, "out")


def test_step_ex_flags(g):
    """gdn_step_ex refuses unknown flag bits before anything else happens;
    with a known flag it validates like gdn_step."""
    a, sz = addrs()
    d = g.Dims(HV, HK, D, D)

    def f(flags, **over):
        x = dict(a, **over)
        return g.lib.gdn_step_ex(ctypes.byref(d), B, x["q"], x["k"], x["v"], x["beta"], x["gate"],
                                 x["state"], x["out"], flags, None)

    expect(g, f(2), -2, "unknown flags 0x2")
    expect(g, f(0x80000001), -2, "unknown flags 0x80000000")
    expect(g, f(1, q=None), -1, "q")
    expect(g, f(1, out=a["state"]), -4, "out")


def test_tail_validation(g):
    d = g.Dims(HV, HK, D, D)
    C = 2 * HK * D + HV * D
    p = g.TailParams(4, 128, 1e-6)
    pu = g.TailParams(4, 128, 1e-6, 1)      # three launches: the workspace is used
    base = {"x": BASE, "conv_w": BASE + (1 << 24), "cs": BASE + (2 << 24), "beta": BASE + (3 << 24),
            "gate": BASE + (4 << 24), "state": BASE + (5 << 24), "z": BASE + (8 << 24),
            "nw": BASE + (9 << 24), "y": BASE + (10 << 24), "ws": BASE + (11 << 24)}
    need = g.layer_tail_workspace_bytes(B)
    assert need == B * (C + HV * D) * 4

    def f(pp=p, dd=d, Bv=B, ws_bytes=need, dq=None, dc=None, **over):
        a = dict(base, **over)
        return g.lib.gdn_layer_tail(
            ctypes.byref(dd), ctypes.byref(pp) if pp is not None else None, Bv,
            a["x"], a["conv_w"], a["cs"], a["beta"], a["gate"], a["state"], a["z"], a["nw"],
            a["y"], dq, dc, a["ws"], ws_bytes, None)

    expect(g, f(pp=None), -1, "params")
    expect(g, f(x=None), -1, "x")
    expect(g, f(nw=None), -1, "norm_w")
    expect(g, f(pp=g.TailParams(1, 128, 1e-6)), -2, "conv_kernel")
    expect(g, f(pp=g.TailParams(9, 128, 1e-6)), -2, "conv_kernel")
    expect(g, f(pp=g.TailParams(4, 100, 1e-6)), -2, "norm_group")
    expect(g, f(pp=g.TailParams(4, 128, -1.0)), -2, "norm_eps")
    expect(g, f(pp=g.TailParams(4, 128, float("nan"))), -2, "norm_eps")
    expect(g, f(Bv=0), -2, "B")
    # one-element groups at B = 8193: 8193 * 4096 gated-norm workgroups of 128
    # threads would overflow the 32-bit dispatch grid
    expect(g, f(pp=g.TailParams(4, 1, 1e-6), Bv=8193), -2, "groups too many")
    expect(g, f(pp=pu, ws_bytes=need - 4), -5, "workspace")
    expect(g, f(pp=pu, ws=None), -5, "workspace")
    expect(g, f(cs=base["cs"] + 4), -3, "conv_state")
    expect(g, f(pp=pu, ws=base["ws"] + 4), -3, "workspace")
    expect(g, f(y=base["z"]), -4, "y")
    expect(g, f(y=base["x"] + 64), -4, "y")
    expect(g, f(pp=pu, ws=base["state"]), -4, "buffer")
    # the single launch never touches the workspace, so an unused one that
    # overlaps a buffer is not checked (the GPU tests run it with NULL)
    # both debug buffers given -> no workspace needed, but they must not collide
    dq, dc = BASE + (12 << 24), BASE + (13 << 24)
    expect(g, f(ws=None, ws_bytes=0, dq=dq, dc=dq + 64), -4, "buffer")
    expect(g, f(pp=pu, ws=None, ws_bytes=0, dq=dq, dc=dq + 64), -4, "buffer")
    expect(g, f(dq=dq + 4), -3, "dbg_qkv")
    # a three-launch tail at a shape the single launch does not take (conv
    # kernel 3) needs the workspace too
    expect(g, f(pp=g.TailParams(3, 128, 1e-6), ws=None), -5, "workspace")


def test_tail_noalloc_validation(g):
    """gdn_layer_tail_noalloc: the checks of gdn_layer_tail, and a three-launch
    call whose staging exceeds the static scratch is refused before anything
    else happens (B = 342 at the page geometry needs 16.03 MiB)."""
    d = g.Dims(HV, HK, D, D)
    assert g.layer_tail_workspace_bytes(341) <= 16 << 20 < g.layer_tail_workspace_bytes(342)
    step = 1 << 30                          # room for B = 342 in every buffer
    base = {"x": BASE, "conv_w": BASE + step, "cs": BASE + 2 * step, "beta": BASE + 3 * step,
            "gate": BASE + 4 * step, "state": BASE + 5 * step, "z": BASE + 6 * step,
            "nw": BASE + 7 * step, "y": BASE + 8 * step}

    def f(pp, Bv=B, dq=None, dc=None, **over):
        a = dict(base, **over)
        return g.lib.gdn_layer_tail_noalloc(
            ctypes.byref(d), ctypes.byref(pp), Bv, a["x"], a["conv_w"], a["cs"], a["beta"],
            a["gate"], a["state"], a["z"], a["nw"], a["y"], dq, dc, None)

    pu = g.TailParams(4, 128, 1e-6, 1)
    expect(g, f(pu, Bv=342), -5, "static scratch holds 16777216")
    expect(g, f(g.TailParams(3, 128, 1e-6), Bv=342), -5, "static scratch")
    expect(g, f(pu, x=None), -1, "x")
    expect(g, f(g.TailParams(4, 128, 1e-6), y=base["z"]), -4, "y")
    expect(g, f(pu, Bv=0), -2, "B")


def test_tail_pair_validation(g):
    d = g.Dims(HV, HK, D, D)
    p = g.TailParams(4, 128, 1e-6)
    step = 1 << 26
    names = ("x", "conv_w", "cs", "csn", "beta", "gate", "state", "sn", "z", "nw", "y")
    base = {n: BASE + i * step for i, n in enumerate(names)}

    def f(pp=p, dd=d, Bv=B, **over):
        a = dict(base, **over)
        return g.lib.gdn_layer_tail_pair(
            ctypes.byref(dd), ctypes.byref(pp) if pp is not None else None, Bv,
            *(a[n] for n in names), None)

    expect(g, f(pp=None), -1, "params")
    expect(g, f(csn=None), -1, "conv_state_next")
    expect(g, f(sn=None), -1, "state_next")
    expect(g, f(pp=g.TailParams(3, 128, 1e-6)), -2, "conv_kernel 4")
    expect(g, f(pp=g.TailParams(4, 64, 1e-6)), -2, "norm_group")
    expect(g, f(dd=g.Dims(64, 16, D, D)), -2, "n_v_heads")
    expect(g, f(pp=g.TailParams(4, 128, float("inf"))), -2, "norm_eps")
    expect(g, f(Bv=0), -2, "B")
    expect(g, f(x=base["x"] + 4), -3, "x")
    expect(g, f(beta=base["beta"] + 2), -3, "beta")
    expect(g, f(csn=base["cs"]), -4, "conv_state")
    expect(g, f(sn=base["state"] + 64), -4, "state")
    expect(g, f(y=base["z"]), -4, "y")
    expect(g, f(csn=base["x"]), -4, "conv_state_next")


def test_gate_transform_validation(g):
    d = g.Dims(HV, HK, D, D)
    base = {"ba": BASE, "a_log": BASE + (1 << 20), "dt": BASE + (2 << 20),
            "beta": BASE + (3 << 20), "gate": BASE + (4 << 20)}

    def f(dd=d, Bv=B, null_in=False, **over):
        a = dict(base, **over)
        gi = g.GateInputs(a["ba"], a["a_log"], a["dt"])
        return g.lib.gdn_gate_transform(ctypes.byref(dd), Bv, None if null_in else ctypes.byref(gi),
                                        a["beta"], a["gate"], None)

    expect(g, f(null_in=True), -1, "gate inputs")
    expect(g, f(ba=None), -1, "ba")
    expect(g, f(a_log=None), -1, "a_log")
    expect(g, f(dt=None), -1, "dt_bias")
    expect(g, f(beta=None), -1, "beta")
    expect(g, f(gate=base["ba"] + 2), -3, "gate")
    expect(g, f(Bv=0), -2, "B")
    expect(g, f(dd=g.Dims(HV, HK, 64, 64)), -2, "d_k")
    # beta over the second half of ba, gate over a_log
    expect(g, f(beta=base["ba"] + B * HV * 4), -4, "beta")
    expect(g, f(gate=base["a_log"]), -4, "gate")
    expect(g, f(gate=base["beta"] + 4), -4, "beta")


def test_tail_ba_validation(g):
    d = g.Dims(HV, HK, D, D)
    C = 2 * HK * D + HV * D
    p = g.TailParams(4, 128, 1e-6)
    base = {"x": BASE, "conv_w": BASE + (1 << 24), "cs": BASE + (2 << 24), "ba": BASE + (3 << 24),
            "a_log": BASE + (4 << 24), "dt": BASE + (4 << 24) + 4096, "state": BASE + (5 << 24),
            "z": BASE + (8 << 24), "nw": BASE + (9 << 24), "y": BASE + (10 << 24),
            "ws": BASE + (11 << 24)}
    need = g.layer_tail_ba_workspace_bytes(B)
    assert need == B * (C + HV * D) * 4 + 2 * B * HV * 4
    assert need == g.layer_tail_workspace_bytes(B) + 2 * B * HV * 4

    pu = g.TailParams(4, 128, 1e-6, 1)      # three launches: the workspace is used

    def f(ws_bytes=need, null_gates=False, dq=None, dc=None, pp=pu, **over):
        a = dict(base, **over)
        gi = g.GateInputs(a["ba"], a["a_log"], a["dt"])
        return g.lib.gdn_layer_tail_ba(
            ctypes.byref(d), ctypes.byref(pp), B, a["x"], a["conv_w"], a["cs"],
            None if null_gates else ctypes.byref(gi), a["state"], a["z"], a["nw"], a["y"],
            dq, dc, a["ws"], ws_bytes, None)

    expect(g, f(null_gates=True), -1, "gates")
    expect(g, f(ba=None), -1, "ba")
    expect(g, f(dt=None), -1, "dt_bias")
    expect(g, f(ws_bytes=need - 4), -5, "workspace")
    # the dbg buffers replace the qkv and core parts; beta/gate still need room
    dq, dc = BASE + (12 << 24), BASE + (13 << 24)
    expect(g, f(ws=None, ws_bytes=0, dq=dq, dc=dc), -5, "workspace")
    expect(g, f(ws_bytes=2 * B * HV * 4 - 4, dq=dq, dc=dc), -5, "workspace")
    # the beta/gate part of the workspace must not overlap the inputs
    expect(g, f(ws=base["ba"] - need + 16, ws_bytes=need), -4, "buffer")
    expect(g, f(y=base["x"] + 64), -4, "y")


def test_workspace_bytes_invalid(g):
    assert g.lib.gdn_layer_tail_workspace_bytes(None, 4) == 0
    assert g.lib.gdn_layer_tail_workspace_bytes(ctypes.byref(g.PAGE_DIMS), 0) == 0
    assert g.lib.gdn_layer_tail_ba_workspace_bytes(None, 4) == 0
    assert g.lib.gdn_layer_tail_ba_workspace_bytes(ctypes.byref(g.PAGE_DIMS), 0) == 0


def test_binding_rejects_cpu_tensors(g):
    import torch
    q = torch.zeros(1, 16, 128)
    with pytest.raises(ValueError, match="GPU"):
        g.step(q, q, torch.zeros(1, 32, 128), torch.zeros(1, 32), torch.zeros(1, 32),
               torch.zeros(1, 32, 128, 128), torch.zeros(1, 32, 128))
    with pytest.raises(TypeError, match="float32"):
        g.step(q.double(), q, torch.zeros(1, 32, 128), torch.zeros(1, 32), torch.zeros(1, 32),
               torch.zeros(1, 32, 128, 128), torch.zeros(1, 32, 128))


def test_product_never_imports_the_oracle():
    """The product package and the oracle share no source: nothing under the
    package mentions the oracle module or its library."""
    pkg = os.path.join(ROOT, "gated_deltanet_decode_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".cpp", ".hip", ".hpp", ".h")):
                txt = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in txt and "liboracle" not in txt \
                    and "gdn_oracle" not in txt, f"{fn} references the oracle"
    hdr = open(os.path.join(ROOT, "include", "gdn.h")).read()
    assert "oracle" not in hdr


def test_probe_library_rejects_bad_arguments():
    """The measurement probes validate before launching anything."""
    from gated_deltanet_decode_amd._build import PROBE_LIBRARY
    lib = ctypes.CDLL(PROBE_LIBRARY)
    lib.gdn_probe_inplace.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint, ctypes.c_void_p]
    lib.gdn_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert lib.gdn_probe_inplace(None, 4096, 0, None) == -1
    assert lib.gdn_probe_inplace(BASE, 4000, 0, None) == -1
    assert lib.gdn_probe_inplace(BASE + 8, 4096, 0, None) == -1
    assert lib.gdn_probe_copy(None, BASE, 16, None) == -1
    assert lib.gdn_probe_copy(BASE, BASE + (1 << 20), 20, None) == -1
    lib.gdn_probe_fma.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_void_p]
    assert lib.gdn_probe_fma(None, 1 << 20, 256, 512, 10, None) == -1      # no buffer
    assert lib.gdn_probe_fma(BASE, 1 << 20, 256, 500, 10, None) == -1      # not whole waves
    assert lib.gdn_probe_fma(BASE, 1 << 20, 256, 2048, 10, None) == -1     # over 1024 threads
    assert lib.gdn_probe_fma(BASE, 1 << 20, 0, 512, 10, None) == -1        # no workgroup
    assert lib.gdn_probe_fma(BASE, 1 << 20, 256, 512, 0, None) == -1       # no iteration
    assert lib.gdn_probe_fma(BASE, 256 * 512 - 1, 256, 512, 10, None) == -1  # buffer too small
