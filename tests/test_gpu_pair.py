"""GPU: gdn_pair (speculative two-position step; docs.rs "Module
linear_core", gdn_pair) against the oracle, and its bitwise contract with
gdn_step (committed position) and gdn_seq (tentative position)."""
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


def run_pair(g, si, M):
    import torch
    t = {n: dev(x) for n, x in si.items()}
    Md = dev(M)
    Mn = torch.full_like(Md, float("nan"))
    out = torch.empty(si["v"].shape, dtype=torch.float32, device="cuda")
    g.pair(t["q"], t["k"], t["v"], t["beta"], t["gate"], Md, Mn, out)
    torch.cuda.synchronize()
    return Md.cpu().numpy(), Mn.cpu().numpy(), out.cpu().numpy()


# B = 1, 3: one wave per tile; B = 5: one epoch of the walk; B = 64: four
# epochs; B = 70 x 33 heads: 36,960 tiles in 5 epochs, the last ragged.
@pytest.mark.parametrize("B,Hv,Hk", [(1, 32, 16), (3, 32, 16), (2, 4, 2), (5, 32, 16),
                                     (64, 32, 16), (70, 33, 11)])
def test_pair_matches_oracle(g, orc, B, Hv, Hk):
    print(f"\n  gdn_pair B={B} Hv={Hv} Hk={Hk}", flush=True)
    si = gi.step_inputs(5000 + B, 0, B, Hv, Hk, T=2)
    M = gi.state(5000 + B, 0, B, Hv)
    Mg, Mng, og = run_pair(g, si, M)
    want, Mn = orc.pair(si["q"], si["k"], si["v"], si["beta"], si["gate"], M)
    ref.assert_close("committed", Mg, M, 1e-6)
    ref.assert_close("tentative", Mng, Mn, 1e-6)
    ref.assert_close("out", og, want, 1e-5)


def test_pair_is_bitwise_step_then_seq(g):
    """Position 1 == gdn_step; position 2's state and both outputs ==
    gdn_seq over the two positions (shared row arithmetic)."""
    import torch
    print("\n  gdn_pair == gdn_step + gdn_seq(T=2)", flush=True)
    B = 5
    si = gi.step_inputs(5100, 0, B, T=2)
    M = gi.state(5100, 0, B)
    Mg, Mng, og = run_pair(g, si, M)
    t = {n: dev(x) for n, x in si.items()}
    Ms = dev(M)
    os_ = torch.empty((B, 2, 32, 128), device="cuda")
    g.seq(t["q"], t["k"], t["v"], t["beta"], t["gate"], Ms, os_)
    t1 = {n: dev(np.ascontiguousarray(x[:, 0])) for n, x in si.items()}
    M1 = dev(M)
    o1 = torch.empty((B, 32, 128), device="cuda")
    g.step(t1["q"], t1["k"], t1["v"], t1["beta"], t1["gate"], M1, o1)
    torch.cuda.synchronize()
    assert np.array_equal(Mg, M1.cpu().numpy()), "committed state != gdn_step"
    assert np.array_equal(Mng, Ms.cpu().numpy()), "tentative state != gdn_seq(T=2)"
    assert np.array_equal(og, os_.cpu().numpy()), "outputs != gdn_seq(T=2)"


def test_pair_reject_then_accept(g, orc):
    """Speculative use: reject keeps the committed state; a later pair on the
    same committed state and an accepted swap chain match the oracle."""
    import torch
    print("\n  gdn_pair reject / accept", flush=True)
    B = 2
    M = gi.state(5200, 0, B)
    Md = dev(M)
    Mn = torch.empty_like(Md)
    out = torch.empty((B, 2, 32, 128), device="cuda")
    # first verification: draft rejected -> only position 1 counts
    s1 = gi.step_inputs(5200, 1, B, T=2)
    t = {n: dev(x) for n, x in s1.items()}
    g.pair(t["q"], t["k"], t["v"], t["beta"], t["gate"], Md, Mn, out)
    orc.step_M(*(np.ascontiguousarray(s1[n][:, 0]) for n in ("q", "k", "v", "beta", "gate")), M)
    # second verification: draft accepted -> adopt the tentative state
    s2 = gi.step_inputs(5200, 2, B, T=2)
    t = {n: dev(x) for n, x in s2.items()}
    g.pair(t["q"], t["k"], t["v"], t["beta"], t["gate"], Md, Mn, out)
    Md, Mn = Mn, Md
    orc.seq(s2["q"], s2["k"], s2["v"], s2["beta"], s2["gate"], M)
    torch.cuda.synchronize()
    ref.assert_close("state", Md.cpu().numpy(), M, 1e-6)
