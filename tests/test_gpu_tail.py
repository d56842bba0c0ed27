"""GPU: gdn_layer_tail against the oracle, stage by stage in the chained,
non-reset style of Red Lite dev15e (each side feeds its own stage outputs to
its next stage): normalised Q|K|V, core output, y, the conv cache (bitwise)
and the recurrent state."""
import numpy as np
import pytest

import gdn_inputs as gi
import ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_deltanet_decode_amd as g
    return g


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_tail(g, ti, M, dims=None, params=None, use_dbg=True, use_ws=True):
    import torch
    dims = dims or g.PAGE_DIMS
    params = params or g.PAGE_TAIL
    B, C = ti["x"].shape
    t = {n: dev(x) for n, x in ti.items()}
    Md = dev(M)
    nv = dims.n_v_heads * dims.d_v
    y = torch.empty((B, nv), device="cuda")
    dq = torch.empty((B, C), device="cuda") if use_dbg else None
    dc = torch.empty((B, dims.n_v_heads, dims.d_v), device="cuda") if use_dbg else None
    ws = torch.empty(g.layer_tail_workspace_bytes(B, dims), dtype=torch.uint8, device="cuda") \
        if use_ws else None
    g.layer_tail(t["x"], t["conv_w"], t["conv_state"], t["beta"], t["gate"], Md, t["z"],
                 t["norm_w"], y, dbg_qkv=dq, dbg_core=dc, workspace=ws, dims=dims, params=params)
    torch.cuda.synchronize()
    return dict(y=y.cpu().numpy(), state=Md.cpu().numpy(), conv_state=t["conv_state"].cpu().numpy(),
                qkv=None if dq is None else dq.cpu().numpy(),
                core=None if dc is None else dc.cpu().numpy())


def oracle_tail(orc, ti, M, Hk=16, d=128, group=128):
    cs = ti["conv_state"].copy()
    y, qkv, core = orc.layer_tail(ti["x"], ti["conv_w"], cs, ti["beta"], ti["gate"], M,
                                  ti["z"], ti["norm_w"], Hk, d, group=group)
    return dict(y=y, qkv=qkv, core=core, conv_state=cs, state=M)


def check(got, want, state_tol=1e-6):
    if got["qkv"] is not None:
        ref.assert_close("qkv", got["qkv"], want["qkv"], 1e-5)
        ref.assert_close("core", got["core"], want["core"], 1e-5)
    ref.assert_close("y", got["y"], want["y"], 1e-5)
    ref.assert_close("state", got["state"], want["state"], state_tol)
    assert np.array_equal(got["conv_state"], want["conv_state"]), "conv cache not bitwise"


def test_tail_b32_layer_tail(g, orc, workload):
    """B=32, 8192 channels, kernel 4, group 128, eps 1e-6."""
    workload("tail_b32")
    c = gi.WORKLOADS["tail_b32"]
    print("\n  gdn_layer_tail B=32 (tail_b32)", flush=True)
    ti = gi.tail_inputs(c["seed"], c["B"])
    M = gi.state(c["seed"], 0, c["B"])
    got = run_tail(g, ti, M)
    want = oracle_tail(orc, ti, M)
    check(got, want)


@pytest.mark.parametrize("use_dbg,use_ws,unfused", [(False, True, 0), (True, False, 0),
                                                    (False, False, 0), (False, True, 1),
                                                    (True, False, 1)])
def test_tail_workspace_and_debug_buffers(g, orc, use_dbg, use_ws, unfused):
    """The result does not depend on whether intermediates go to the
    workspace or to the debug buffers; the single launch runs without any
    workspace."""
    print(f"\n  gdn_layer_tail B=3 dbg={use_dbg} workspace={use_ws} three launches={unfused}",
          flush=True)
    ti = gi.tail_inputs(4100, 3)
    M = gi.state(4100, 0, 3)
    got = run_tail(g, ti, M, use_dbg=use_dbg, use_ws=use_ws,
                   params=g.TailParams(4, 128, 1e-6, unfused))
    want = oracle_tail(orc, ti, M)
    check(got, want)


@pytest.mark.parametrize("K,group", [(2, 4096), (3, 64), (8, 256)])
def test_tail_other_kernel_and_group_sizes(g, orc, K, group):
    print(f"\n  gdn_layer_tail K={K} group={group}", flush=True)
    ti = gi.tail_inputs(4200 + K, 2, K=K, group=group)
    M = gi.state(4200 + K, 0, 2)
    got = run_tail(g, ti, M, params=g.TailParams(K, group, 1e-6))
    want = oracle_tail(orc, ti, M, group=group)
    check(got, want)


@pytest.mark.parametrize("Hv,Hk", [(32, 16), (16, 16)])
def test_fused_and_three_launch_paths_agree_bitwise(g, orc, Hv, Hk):
    """The single-launch tail and the three-launch tail give the same bits on
    every output (they share the per-element arithmetic and the reduction
    order), and both match the oracle."""
    print(f"\n  gdn_layer_tail fused vs three launches Hv={Hv} Hk={Hk}", flush=True)
    dims = g.Dims(Hv, Hk, 128, 128)
    ti = gi.tail_inputs(4400 + Hv, 4, Hv, Hk)
    M = gi.state(4400 + Hv, 0, 4, Hv)
    fused = run_tail(g, ti, M, dims=dims, params=g.TailParams(4, 128, 1e-6, 0))
    three = run_tail(g, ti, M, dims=dims, params=g.TailParams(4, 128, 1e-6, 1))
    for n in ("y", "state", "conv_state", "qkv", "core"):
        assert np.array_equal(fused[n], three[n]), f"{n} differs between the two paths"
    want = oracle_tail(orc, ti, M, Hk=Hk)
    check(fused, want)


def test_tail_three_tokens_fill_the_cache(g, orc):
    """After kernel-1 = 3 tokens the conv cache holds exactly the last three
    raw inputs; the chained GPU and oracle states stay within tolerance."""
    import torch
    print("\n  gdn_layer_tail three tokens", flush=True)
    B = 2
    ti = gi.tail_inputs(4300, B)
    M = gi.state(4300, 0, B)
    t = {n: dev(x) for n, x in ti.items()}
    Md = dev(M)
    y = torch.empty((B, 4096), device="cuda")
    ws = torch.empty(g.layer_tail_workspace_bytes(B), dtype=torch.uint8, device="cuda")
    cs = ti["conv_state"].copy()
    xs = []
    for step in range(3):
        x = gi.tail_inputs(4300, B, slot=step + 1)["x"]
        xs.append(x)
        g.layer_tail(dev(x), t["conv_w"], t["conv_state"], t["beta"], t["gate"], Md, t["z"],
                     t["norm_w"], y, workspace=ws)
        yo, _, _ = orc.layer_tail(x, ti["conv_w"], cs, ti["beta"], ti["gate"], M, ti["z"],
                                  ti["norm_w"], 16, 128)
    torch.cuda.synchronize()
    assert np.array_equal(t["conv_state"].cpu().numpy(), np.stack(xs, 1))
    ref.assert_close("y", y.cpu().numpy(), yo, 1e-5)
    ref.assert_close("state", Md.cpu().numpy(), M, 1e-6)


@pytest.mark.parametrize("Hv,Hk", [(22, 11), (11, 11)])
def test_tail_other_head_counts(g, orc, Hv, Hk):
    """Key-head counts other than the page's (5632 / 4224 channels), single
    launch and three launches, against the oracle."""
    print(f"\n  gdn_layer_tail Hv={Hv} Hk={Hk}", flush=True)
    dims = g.Dims(Hv, Hk, 128, 128)
    ti = gi.tail_inputs(4600 + Hv, 3, Hv, Hk)
    M = gi.state(4600 + Hv, 0, 3, Hv)
    for fu in (0, 1):
        got = run_tail(g, ti, M, dims=dims, params=g.TailParams(4, 128, 1e-6, fu))
        want = oracle_tail(orc, ti, M.copy(), Hk=Hk)
        check(got, want)


def test_tail_degenerate_inputs(g, orc):
    """Degenerate cases of the branch: one sequence's channels all zero (its
    Q and K heads hit the L2 floor and stay zero, so the step sees a zero key
    and only decays), another's gates at -80 (the decay underflows towards a
    full forget), and a zero state, against the oracle on both launch paths."""
    print("\n  gdn_layer_tail degenerate inputs", flush=True)
    B = 4
    ti = gi.tail_inputs(4700, B)
    ti["x"][1] = 0.0
    ti["conv_state"][1] = 0.0
    ti["gate"][2] = -80.0
    M = gi.state(4700, 0, B)
    M[3] = 0.0
    for fu in (0, 1):
        got = run_tail(g, ti, M, params=g.TailParams(4, 128, 1e-6, fu))
        want = oracle_tail(orc, ti, M.copy())
        check(got, want)
        assert np.all(got["qkv"][1] == 0.0), "zero channels must stay zero through L2"


def test_tail_b128(g, orc):
    """A larger batch (B=128: 2048 workgroups of the single-launch tail)."""
    print("\n  gdn_layer_tail B=128", flush=True)
    ti = gi.tail_inputs(4500, 128)
    M = gi.state(4500, 0, 128)
    got = run_tail(g, ti, M)
    want = oracle_tail(orc, ti, M)
    check(got, want)
