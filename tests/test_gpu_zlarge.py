"""GPU: every kernel on a state past 2^31 floats (8 GiB), the size at which a
32-bit element offset would wrap.  B = 4104 sequences of 32 value heads are
131,328 heads of 16,384 floats, so the heads of the last 8 sequences start
beyond float index 2^31; and gdn_step at B = 16400, whose 34 GB of state
take two launches of the staged kernel.

Inputs and states of G = 8 seeded sequences are tiled over the batch on the
GPU: sequence b gets the inputs and starting state of sequence b % 8.  Each
sequence's result depends only on its own inputs and state, so every group
of 8 must come out bit for bit equal to the first group (checked over the
whole batch on the GPU), and the first group must match the oracle within
the per-step tolerances.  A mis-addressed head anywhere in the batch, in
particular past the 2^31 boundary, breaks the first check."""
import numpy as np
import pytest

import gdn_inputs as gi
import ref

pytestmark = pytest.mark.gpu

G = 8                      # distinct sequences
B = 4104                   # 513 groups; 131,328 heads > 2^31 / (128 * 128)
NG = B // G
assert B * 32 * 128 * 128 > 2 ** 31 and (B - G) * 32 * 128 * 128 >= 2 ** 31


@pytest.fixture(scope="module")
def g():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_deltanet_decode_amd as g
    return g


@pytest.fixture(autouse=True)
def _release():
    yield
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def tiled(a):
    """numpy [G][...] -> GPU [B][...], sequence b holding a[b % G]."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.repeat((NG,) + (1,) * (t.dim() - 1))


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def first(t):
    return t[:G].cpu().numpy()


def assert_groups_bitwise(name, t, ng=NG):
    """Every group of G sequences of t ([ng * G][...]) equals the first group
    bit for bit (compared as 32-bit patterns)."""
    import torch
    rows = t.reshape(ng, -1).view(torch.int32)
    bad = 0
    for s in range(1, ng, 32):
        bad += int((rows[s:s + 32] != rows[0]).any(dim=1).sum())
    ref.record(name=f"{name}: {ng} groups bitwise", mismatched_groups=bad, passed=bad == 0)
    print(f"    {name:>14s}: {ng} groups of {G} bitwise equal: {bad == 0}", flush=True)
    assert bad == 0, f"{name}: {bad} of {ng - 1} groups differ from the first"


def test_step_cached_past_2_31(g, orc):
    """gdn_step_ex with GDN_STATE_CACHED (the one-shot kernel) and the default
    staged kernel over the same 8.6 GB state."""
    import torch
    print(f"\n  gdn_step_ex cached / gdn_step B={B}", flush=True)
    si = gi.step_inputs(7101, 0, G)
    M0 = gi.state(7101, 0, G)
    t = {n: tiled(x) for n, x in si.items()}
    for cached in (True, False):
        Md = tiled(M0)
        o = torch.empty((B, 32, 128), device="cuda")
        g.step(t["q"], t["k"], t["v"], t["beta"], t["gate"], Md, o, cached=cached)
        torch.cuda.synchronize()
        tag = "cached" if cached else "default"
        assert_groups_bitwise(f"{tag} state", Md)
        assert_groups_bitwise(f"{tag} out", o)
        M = M0.copy()
        want = orc.step_M(si["q"], si["k"], si["v"], si["beta"], si["gate"], M)
        ref.assert_close(f"{tag} state", first(Md), M, 1e-6)
        ref.assert_close(f"{tag} out", first(o), want, 1e-5)
        del Md


def test_step_split_launch_past_32_gib(g, orc):
    """gdn_step at B = 16400 (34 GB of state): the staged kernel covers 2^22
    tile pairs (32 GiB) per launch, so this call takes two launches and its
    last 16 sequences come from the second one."""
    import torch
    Bs = 16400
    ng = Bs // G
    assert Bs * 32 * 16 // 2 > 1 << 22
    print(f"\n  gdn_step B={Bs} (two staged launches)", flush=True)
    si = gi.step_inputs(7102, 0, G)
    M0 = gi.state(7102, 0, G)
    t = {n: dev(x).repeat((ng,) + (1,) * (x.ndim - 1)) for n, x in si.items()}
    Md = dev(M0).repeat(ng, 1, 1, 1)
    o = torch.empty((Bs, 32, 128), device="cuda")
    g.step(t["q"], t["k"], t["v"], t["beta"], t["gate"], Md, o)
    torch.cuda.synchronize()
    assert_groups_bitwise("state", Md, ng)
    assert_groups_bitwise("out", o, ng)
    M = M0.copy()
    want = orc.step_M(si["q"], si["k"], si["v"], si["beta"], si["gate"], M)
    ref.assert_close("state", first(Md), M, 1e-6)
    ref.assert_close("out", first(o), want, 1e-5)
    del Md


@pytest.mark.parametrize("T,exact", [(3, False), (20, False), (20, True), (65, False)])
def test_seq_past_2_31(g, orc, T, exact):
    """The many-heads gdn_seq routes: 8-token chunks (T < 16) and the
    half-head kernel with its chunks fetched straight into LDS (16-token
    chunks; T = 20 scaled and exact, T = 65 with a partial last chunk)."""
    import torch
    print(f"\n  gdn_seq{'_exact' if exact else ''} B={B} T={T}", flush=True)
    si = gi.step_inputs(7200 + T, 0, G, T=T)
    M0 = gi.state(7200 + T, 0, G)
    t = {n: tiled(x) for n, x in si.items()}
    Md = tiled(M0)
    o = torch.empty((B, T, 32, 128), device="cuda")
    g.seq(t["q"], t["k"], t["v"], t["beta"], t["gate"], Md, o, exact=exact)
    torch.cuda.synchronize()
    assert_groups_bitwise("state", Md)
    assert_groups_bitwise("out", o)
    M = M0.copy()
    want = orc.seq(si["q"], si["k"], si["v"], si["beta"], si["gate"], M)
    ref.assert_close("state", first(Md), M, 1e-6)
    ref.assert_close("out", first(o), want, 1e-5)


def test_pair_past_2_31(g, orc):
    import torch
    print(f"\n  gdn_pair B={B}", flush=True)
    si = gi.step_inputs(7301, 0, G, T=2)
    M0 = gi.state(7301, 0, G)
    t = {n: tiled(x) for n, x in si.items()}
    Md = tiled(M0)
    Mn = torch.empty_like(Md)
    o = torch.empty((B, 2, 32, 128), device="cuda")
    g.pair(t["q"], t["k"], t["v"], t["beta"], t["gate"], Md, Mn, o)
    torch.cuda.synchronize()
    for name, x in (("committed", Md), ("tentative", Mn), ("out", o)):
        assert_groups_bitwise(name, x)
    M = M0.copy()
    want, Mn_o = orc.pair(si["q"], si["k"], si["v"], si["beta"], si["gate"], M)
    ref.assert_close("committed", first(Md), M, 1e-6)
    ref.assert_close("tentative", first(Mn), Mn_o, 1e-6)
    ref.assert_close("out", first(o), want, 1e-5)


@pytest.mark.parametrize("path", ["single", "three", "raw_gates", "noalloc"])
def test_tail_past_2_31(g, orc, path):
    """gdn_layer_tail (single launch and three launches), gdn_layer_tail_ba
    and gdn_layer_tail_noalloc (single launch: no scratch at this B)."""
    import torch
    print(f"\n  layer tail ({path}) B={B}", flush=True)
    ti = gi.tail_inputs(7400, G)
    gin = gi.gate_inputs(7400, G)
    M0 = gi.state(7400, 0, G)
    x, z = tiled(ti["x"]), tiled(ti["z"])
    cs = tiled(ti["conv_state"])
    cw, nw = dev(ti["conv_w"]), dev(ti["norm_w"])
    Md = tiled(M0)
    y = torch.empty((B, 4096), device="cuda")
    if path == "raw_gates":
        g.layer_tail_ba(x, cw, cs, tiled(gin["ba"]), dev(gin["a_log"]), dev(gin["dt_bias"]), Md,
                        z, nw, y)
        beta, gate = orc.gate_transform(gin["ba"], gin["a_log"], gin["dt_bias"])
    else:
        beta, gate = ti["beta"], ti["gate"]
        bd, gd = tiled(beta), tiled(gate)
        if path == "single":
            g.layer_tail(x, cw, cs, bd, gd, Md, z, nw, y)
        elif path == "three":
            ws = torch.empty(g.layer_tail_workspace_bytes(B), dtype=torch.uint8, device="cuda")
            params = g.TailParams(4, 128, 1e-6, 1)
            g.layer_tail(x, cw, cs, bd, gd, Md, z, nw, y, workspace=ws, params=params)
        else:
            g.layer_tail_noalloc(x, cw, cs, bd, gd, Md, z, nw, y)
    torch.cuda.synchronize()
    for name, t in (("conv ring", cs), ("state", Md), ("y", y)):
        assert_groups_bitwise(name, t)
    M = M0.copy()
    ring = ti["conv_state"].copy()
    want, _, _ = orc.layer_tail(ti["x"], ti["conv_w"], ring, beta, gate, M, ti["z"],
                                ti["norm_w"], 16, 128)
    assert np.array_equal(first(cs), ring), "conv ring not bitwise"
    ref.assert_close("state", first(Md), M, 1e-6)
    ref.assert_close("y", first(y), want, 1e-5)


def test_tail_pair_past_2_31(g, orc):
    import torch
    print(f"\n  gdn_layer_tail_pair B={B}", flush=True)
    t1 = gi.tail_inputs(7500, G, slot=0)
    t2 = gi.tail_inputs(7500, G, slot=1)
    pr = {n: np.ascontiguousarray(np.stack([t1[n], t2[n]], axis=1))
          for n in ("x", "beta", "gate", "z")}
    M0 = gi.state(7500, 0, G)
    Md = tiled(M0)
    Mn = torch.empty_like(Md)
    cs = tiled(t1["conv_state"])
    csn = torch.empty_like(cs)
    y = torch.empty((B, 2, 4096), device="cuda")
    g.layer_tail_pair(tiled(pr["x"]), dev(t1["conv_w"]), cs, csn, tiled(pr["beta"]),
                      tiled(pr["gate"]), Md, Mn, tiled(pr["z"]), dev(t1["norm_w"]), y)
    torch.cuda.synchronize()
    for name, t in (("ring", cs), ("ring next", csn), ("committed", Md), ("tentative", Mn),
                    ("y", y)):
        assert_groups_bitwise(name, t)
    M = M0.copy()
    ring = t1["conv_state"].copy()
    want, csn_o, Mn_o = orc.layer_tail_pair(pr["x"], t1["conv_w"], ring, pr["beta"], pr["gate"],
                                            M, pr["z"], t1["norm_w"], 16, 128)
    assert np.array_equal(first(cs), ring), "committed ring not bitwise"
    assert np.array_equal(first(csn), csn_o), "tentative ring not bitwise"
    ref.assert_close("committed", first(Md), M, 1e-6)
    ref.assert_close("tentative", first(Mn), Mn_o, 1e-6)
    ref.assert_close("y", first(y), want, 1e-5)
