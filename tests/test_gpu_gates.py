"""GPU: the beta/alpha parameter transforms (gdn_gate_transform) and the
layer tail that starts from the raw gate inputs (gdn_layer_tail_ba), against
the oracle (oracle_gate_transform, then oracle_layer_tail), and bitwise
against the library's own two-call route (gdn_gate_transform, then
gdn_layer_tail) on both the single-launch and the three-launch tail."""
import numpy as np
import pytest

import gdn_inputs as gi
import ref

pytestmark = pytest.mark.gpu

HV = 32


@pytest.fixture(scope="module")
def g():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_deltanet_decode_amd as g
    return g


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_gates(g, gin):
    import torch
    B = gin["ba"].shape[0]
    beta = torch.empty((B, HV), device="cuda")
    gate = torch.empty((B, HV), device="cuda")
    g.gate_transform(dev(gin["ba"]), dev(gin["a_log"]), dev(gin["dt_bias"]), beta, gate)
    torch.cuda.synchronize()
    return beta.cpu().numpy(), gate.cpu().numpy()


def close_rel(name, got, want, rel=1e-6, abs_=1e-7):
    """Within rel * |want| + abs_ elementwise (a few binary32 ulps: the GPU
    and the host libm may differ by an ulp or two in exp and log1p)."""
    got = got.astype(np.float64)
    want = want.astype(np.float64)
    err = np.abs(got - want)
    lim = rel * np.abs(want) + abs_
    i = int(np.argmax(err - lim))
    assert np.all(err <= lim), f"{name}: |{got.flat[i]} - {want.flat[i]}| = {err.flat[i]:.3e} > {lim.flat[i]:.3e}"


@pytest.mark.parametrize("B", [1, 3, 257])
def test_gate_transform_matches_oracle(g, orc, B):
    print(f"\n  gdn_gate_transform B={B}", flush=True)
    gin = gi.gate_inputs(5000 + B, B)
    beta, gate = gpu_gates(g, gin)
    wb, wg = orc.gate_transform(gin["ba"], gin["a_log"], gin["dt_bias"])
    close_rel("beta", beta, wb)
    close_rel("gate", gate, wg)
    assert np.all(gate < 0) and np.all((beta > 0) & (beta < 1))


def test_gate_transform_extremes(g, orc):
    """Logits far in both tails, exact zeros and large per-head parameters:
    no overflow, no NaN, same values as the oracle."""
    print("\n  gdn_gate_transform extreme logits", flush=True)
    rng = np.random.default_rng(3)
    B = 8
    ba = (30.0 * rng.standard_normal((B, 2 * HV))).astype(np.float32)
    ba[0, :] = 0.0
    ba[1, :HV] = 100.0
    ba[1, HV:] = -100.0
    ba[2, :HV] = -100.0
    ba[2, HV:] = 100.0
    a_log = np.linspace(-4, 4, HV).astype(np.float32)
    dt_bias = np.linspace(-8, 8, HV).astype(np.float32)
    gin = dict(ba=ba, a_log=a_log, dt_bias=dt_bias)
    beta, gate = gpu_gates(g, gin)
    wb, wg = orc.gate_transform(ba, a_log, dt_bias)
    assert np.all(np.isfinite(beta)) and np.all(np.isfinite(gate))
    close_rel("beta", beta, wb, abs_=1e-30)
    close_rel("gate", gate, wg, abs_=1e-30)
    assert np.all(beta[0] == np.float32(0.5))


def tail_inputs_ba(seed, B, Hv=HV, Hk=16):
    ti = gi.tail_inputs(seed, B, Hv=Hv, Hk=Hk)
    gin = gi.gate_inputs(seed, B, Hv=Hv)
    return ti, gin


def run_tail_ba(g, ti, gin, M, force_unfused=0, use_dbg=False, Hv=HV, Hk=16):
    import torch
    B, C = ti["x"].shape
    dims = g.Dims(Hv, Hk, 128, 128)
    t = {n: dev(x) for n, x in ti.items()}
    gd = {n: dev(x) for n, x in gin.items()}
    Md = dev(M)
    y = torch.empty((B, Hv * 128), device="cuda")
    dq = torch.empty((B, C), device="cuda") if use_dbg else None
    dc = torch.empty((B, Hv, 128), device="cuda") if use_dbg else None
    # the single launch needs no workspace: it runs with none
    ws = torch.empty(g.layer_tail_ba_workspace_bytes(B, dims), dtype=torch.uint8, device="cuda") \
        if force_unfused else None
    params = g.TailParams(4, 128, 1e-6, force_unfused)
    g.layer_tail_ba(t["x"], t["conv_w"], t["conv_state"], gd["ba"], gd["a_log"], gd["dt_bias"],
                    Md, t["z"], t["norm_w"], y, dbg_qkv=dq, dbg_core=dc, workspace=ws,
                    dims=dims, params=params)
    torch.cuda.synchronize()
    return dict(y=y.cpu().numpy(), state=Md.cpu().numpy(),
                conv_state=t["conv_state"].cpu().numpy(),
                qkv=None if dq is None else dq.cpu().numpy(),
                core=None if dc is None else dc.cpu().numpy())


def run_two_calls(g, ti, gin, M, force_unfused=0):
    """gdn_gate_transform, then gdn_layer_tail with its beta and gate."""
    import torch
    B, C = ti["x"].shape
    beta, gate = gpu_gates(g, gin)
    t = {n: dev(x) for n, x in ti.items()}
    Md = dev(M)
    y = torch.empty((B, HV * 128), device="cuda")
    ws = torch.empty(g.layer_tail_workspace_bytes(B), dtype=torch.uint8, device="cuda")
    g.layer_tail(t["x"], t["conv_w"], t["conv_state"], dev(beta), dev(gate), Md, t["z"],
                 t["norm_w"], y, workspace=ws, params=g.TailParams(4, 128, 1e-6, force_unfused))
    torch.cuda.synchronize()
    return dict(y=y.cpu().numpy(), state=Md.cpu().numpy(),
                conv_state=t["conv_state"].cpu().numpy())


def oracle_tail_ba(orc, ti, gin, M, Hk=16):
    beta, gate = orc.gate_transform(gin["ba"], gin["a_log"], gin["dt_bias"])
    cs = ti["conv_state"].copy()
    y, qkv, core = orc.layer_tail(ti["x"], ti["conv_w"], cs, beta, gate, M, ti["z"],
                                  ti["norm_w"], Hk, 128)
    return dict(y=y, qkv=qkv, core=core, conv_state=cs, state=M)


@pytest.mark.parametrize("B,force_unfused", [(1, 0), (5, 0), (32, 0), (5, 1), (32, 1)])
def test_tail_ba_matches_oracle(g, orc, B, force_unfused):
    print(f"\n  gdn_layer_tail_ba B={B} unfused={force_unfused}", flush=True)
    ti, gin = tail_inputs_ba(5100 + B, B)
    M = gi.state(5100 + B, 0, B)
    got = run_tail_ba(g, ti, gin, M, force_unfused, use_dbg=(B == 5))
    want = oracle_tail_ba(orc, ti, gin, M)
    if got["qkv"] is not None:
        ref.assert_close("qkv", got["qkv"], want["qkv"], 1e-5)
        ref.assert_close("core", got["core"], want["core"], 1e-5)
    ref.assert_close("y", got["y"], want["y"], 1e-5)
    ref.assert_close("state", got["state"], want["state"], 1e-6)
    assert np.array_equal(got["conv_state"], want["conv_state"]), "conv cache not bitwise"


@pytest.mark.parametrize("force_unfused", [0, 1])
def test_tail_ba_bitwise_equals_transform_then_tail(g, force_unfused):
    print(f"\n  gdn_layer_tail_ba == gate_transform + layer_tail, unfused={force_unfused}", flush=True)
    B = 7
    ti, gin = tail_inputs_ba(5200, B)
    M = gi.state(5200, 0, B)
    a = run_tail_ba(g, ti, gin, M.copy(), force_unfused)
    b = run_two_calls(g, ti, gin, M.copy(), force_unfused)
    for k in ("y", "state", "conv_state"):
        assert np.array_equal(a[k], b[k]), f"{k} differs"


def test_tail_ba_fused_equals_unfused(g):
    print("\n  gdn_layer_tail_ba fused == three-launch", flush=True)
    B = 9
    ti, gin = tail_inputs_ba(5300, B)
    M = gi.state(5300, 0, B)
    a = run_tail_ba(g, ti, gin, M.copy(), 0)
    b = run_tail_ba(g, ti, gin, M.copy(), 1)
    for k in ("y", "state", "conv_state"):
        assert np.array_equal(a[k], b[k]), f"{k} differs"


@pytest.mark.parametrize("force_unfused", [0, 1])
def test_tail_ba_one_value_head_per_key_head(g, orc, force_unfused):
    """Hv = Hk = 16 (the single-launch tail's one-value-head specialisation)."""
    print(f"\n  gdn_layer_tail_ba Hv=Hk=16 unfused={force_unfused}", flush=True)
    B, Hv, Hk = 4, 16, 16
    ti, gin = tail_inputs_ba(5400, B, Hv, Hk)
    M = gi.state(5400, 0, B, Hv=Hv)
    got = run_tail_ba(g, ti, gin, M, force_unfused, Hv=Hv, Hk=Hk)
    want = oracle_tail_ba(orc, ti, gin, M, Hk=Hk)
    ref.assert_close("y", got["y"], want["y"], 1e-5)
    ref.assert_close("state", got["state"], want["state"], 1e-6)
    assert np.array_equal(got["conv_state"], want["conv_state"]), "conv cache not bitwise"
