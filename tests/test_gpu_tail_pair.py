"""GPU: gdn_layer_tail_pair, the speculative pair over the whole recurrent
branch (docs.rs "Module linear_core", gdn_pair: the first position is kept,
the second held aside with its conv ring and state), against the oracle
(oracle_layer_tail_pair), and its bitwise contract with two gdn_layer_tail
calls."""
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


def pair_inputs(seed, B, Hv=32, Hk=16):
    """Two positions of tail inputs (slots 0 and 1); the conv weight, norm
    weight and starting ring are those of the first."""
    t1 = gi.tail_inputs(seed, B, Hv=Hv, Hk=Hk, slot=0)
    t2 = gi.tail_inputs(seed, B, Hv=Hv, Hk=Hk, slot=1)
    pr = lambda n: np.ascontiguousarray(np.stack([t1[n], t2[n]], axis=1))
    return dict(x=pr("x"), beta=pr("beta"), gate=pr("gate"), z=pr("z"), conv_w=t1["conv_w"],
                norm_w=t1["norm_w"], conv_state=t1["conv_state"]), t1, t2


def run_pair(g, pi, M, dims):
    import torch
    t = {n: dev(x) for n, x in pi.items()}
    Md = dev(M)
    Mn = torch.full_like(Md, float("nan"))
    csn = torch.full_like(t["conv_state"], float("nan"))
    B = M.shape[0]
    y = torch.full((B, 2, dims.n_v_heads * 128), float("nan"), device="cuda")
    g.layer_tail_pair(t["x"], t["conv_w"], t["conv_state"], csn, t["beta"], t["gate"], Md, Mn,
                      t["z"], t["norm_w"], y, dims=dims)
    torch.cuda.synchronize()
    return dict(cs=t["conv_state"].cpu().numpy(), csn=csn.cpu().numpy(), M=Md.cpu().numpy(),
                Mn=Mn.cpu().numpy(), y=y.cpu().numpy())


# B = 32: the page's tail batch; B = 1, 5: small and odd; Hv = Hk: one value
# head per key head (the other single-launch shape)
@pytest.mark.parametrize("B,Hv,Hk", [(32, 32, 16), (1, 32, 16), (5, 32, 16), (3, 16, 16),
                                     (7, 22, 11)])
def test_tail_pair_matches_oracle(g, orc, B, Hv, Hk):
    print(f"\n  gdn_layer_tail_pair B={B} Hv={Hv} Hk={Hk}", flush=True)
    dims = g.Dims(Hv, Hk, 128, 128)
    pi, _, _ = pair_inputs(6200 + B + Hv, B, Hv, Hk)
    M = gi.state(6200 + B + Hv, 0, B, Hv)
    got = run_pair(g, pi, M, dims)
    cs = pi["conv_state"].copy()
    y, csn, Mn = orc.layer_tail_pair(pi["x"], pi["conv_w"], cs, pi["beta"], pi["gate"], M,
                                     pi["z"], pi["norm_w"], Hk, 128)
    assert np.array_equal(got["cs"], cs), "committed ring not bitwise"
    assert np.array_equal(got["csn"], csn), "tentative ring not bitwise"
    ref.assert_close("committed", got["M"], M, 1e-6)
    ref.assert_close("tentative", got["Mn"], Mn, 1e-6)
    ref.assert_close("y", got["y"], y, 1e-5)


def test_tail_pair_is_bitwise_two_tails(g):
    """Position 1 == gdn_layer_tail on the committed ring and state;
    position 2 == gdn_layer_tail on what position 1 committed."""
    import torch
    print("\n  gdn_layer_tail_pair == two gdn_layer_tail calls", flush=True)
    B = 32
    pi, t1, t2 = pair_inputs(6300, B)
    M = gi.state(6300, 0, B)
    got = run_pair(g, pi, M, g.PAGE_DIMS)
    cs = dev(pi["conv_state"])
    Md = dev(M)
    ys = []
    for t in (t1, t2):
        y = torch.empty((B, 4096), device="cuda")
        g.layer_tail(dev(t["x"]), dev(pi["conv_w"]), cs, dev(t["beta"]), dev(t["gate"]), Md,
                     dev(t["z"]), dev(pi["norm_w"]), y)
        ys.append(y)
        if t is t1:
            cs1, M1 = cs.clone(), Md.clone()
    torch.cuda.synchronize()
    assert np.array_equal(got["cs"], cs1.cpu().numpy()), "committed ring"
    assert np.array_equal(got["M"], M1.cpu().numpy()), "committed state"
    assert np.array_equal(got["csn"], cs.cpu().numpy()), "tentative ring"
    assert np.array_equal(got["Mn"], Md.cpu().numpy()), "tentative state"
    assert np.array_equal(got["y"][:, 0], ys[0].cpu().numpy()), "y of position 1"
    assert np.array_equal(got["y"][:, 1], ys[1].cpu().numpy()), "y of position 2"


def test_tail_pair_reject_then_accept(g, orc):
    """Speculative use over three verifications: reject (only position 1
    counts: ring and state stay committed), accept (adopt the tentative ring
    and state by swapping buffers), reject again; the chain matches the
    oracle's sequence of single tails."""
    import torch
    print("\n  gdn_layer_tail_pair reject / accept / reject", flush=True)
    B = 4
    base = gi.tail_inputs(6400, B)
    M = gi.state(6400, 0, B)
    cs = base["conv_state"].copy()
    Md, Mn = dev(M), torch.empty((B, 32, 128, 128), device="cuda")
    csd, csn = dev(cs), torch.empty((B, 3, 8192), device="cuda")
    cw, nw = dev(base["conv_w"]), dev(base["norm_w"])
    y = torch.empty((B, 2, 4096), device="cuda")
    for step, accept in enumerate((False, True, False)):
        t1 = gi.tail_inputs(6400, B, slot=2 * step + 1)
        t2 = gi.tail_inputs(6400, B, slot=2 * step + 2)
        pr = lambda n: dev(np.stack([t1[n], t2[n]], axis=1))
        g.layer_tail_pair(pr("x"), cw, csd, csn, pr("beta"), pr("gate"), Md, Mn, pr("z"), nw, y)
        yo1, _, _ = orc.layer_tail(t1["x"], base["conv_w"], cs, t1["beta"], t1["gate"], M,
                                   t1["z"], base["norm_w"], 16, 128)
        torch.cuda.synchronize()
        ref.assert_close(f"y1[{step}]", y[:, 0].cpu().numpy(), yo1, 1e-5)
        if accept:
            Md, Mn = Mn, Md
            csd, csn = csn, csd
            yo2, _, _ = orc.layer_tail(t2["x"], base["conv_w"], cs, t2["beta"], t2["gate"], M,
                                       t2["z"], base["norm_w"], 16, 128)
            ref.assert_close(f"y2[{step}]", y[:, 1].cpu().numpy(), yo2, 1e-5)
    torch.cuda.synchronize()
    assert np.array_equal(csd.cpu().numpy(), cs), "ring after the chain"
    ref.assert_close("state", Md.cpu().numpy(), M, 1e-6)
