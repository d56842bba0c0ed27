"""GPU: the full-size workloads, in the launch configuration the benchmark
times, checked against the oracle element by element (every sequence of every
layer for step_b256_x36, whose pre-states are regenerated on the host layer
by layer).

  step_b64_x100: B=64 decode, 100 gdn_step calls with fresh inputs
  step_b256_x36: B=256 x 36 layers (18 GiB of state), one gdn_step per
                 layer, plus the same 36 layers flattened into one B=9216 call
  seq_b8_t4096:  gdn_seq B=8 x T=4096 from a zero state
"""
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


@pytest.mark.timeout(600)
def test_step_b64_x100(g, orc):
    import torch
    c = gi.WORKLOADS["step_b64_x100"]
    B, calls = c["B"], c["calls"]
    print(f"\n  step_b64_x100: gdn_step B={B} x {calls} calls", flush=True)
    M = gi.state(c["seed"], 0, B)
    Md = dev(M)
    inputs = [gi.step_inputs(c["seed"], i, B) for i in range(calls)]
    dins = [{n: dev(x) for n, x in si.items()} for si in inputs]
    outs = torch.empty((calls, B, 32, 128), device="cuda")
    M1 = None
    for i in range(calls):
        t = dins[i]
        g.step(t["q"], t["k"], t["v"], t["beta"], t["gate"], Md, outs[i])
        if i == 0:
            M1 = Md.cpu().numpy()
    torch.cuda.synchronize()
    Mg, og = Md.cpu().numpy(), outs.cpu().numpy()
    worst = 0.0
    for i in range(calls):
        want = ref.step_mt(orc, inputs[i], M)
        if i == 0:
            ref.assert_close("state@1", M1, M, 1e-6)
        worst = max(worst, ref.max_err(og[i], want)[0])
        assert worst <= 1e-5, f"call {i}: out error {worst:.3e}"
    print(f"    all {calls} outputs: max abs {worst:.3e}", flush=True)
    ref.assert_close("state@100", Mg, M, 1e-6)


@pytest.mark.timeout(900)
def test_step_b256_x36_layers(g, orc):
    import torch
    c = gi.WORKLOADS["step_b256_x36"]
    B, L, seed = c["B"], c["layers"], c["seed"]
    print(f"\n  step_b256_x36: gdn_step B={B} x {L} layers (18 GiB state)", flush=True)
    states = torch.empty((L, B, 32, 128, 128), device="cuda")
    stage = torch.empty((B, 32, 128, 128), pin_memory=True)
    sn = stage.numpy()
    ins = []
    for l in range(L):
        gi.state_into(sn, seed, l)
        states[l].copy_(stage)
        ins.append(gi.step_inputs(seed, l, B))
    torch.cuda.synchronize()
    dins = {n: dev(np.stack([ins[l][n] for l in range(L)])) for n in ins[0]}
    outs = torch.empty((L, B, 32, 128), device="cuda")
    print("    inputs resident; running 36 layer calls", flush=True)
    for l in range(L):
        g.step(dins["q"][l], dins["k"][l], dins["v"][l], dins["beta"][l], dins["gate"][l],
               states[l], outs[l])
    torch.cuda.synchronize()

    # every sequence of every layer: regenerate the layer's pre-state on the
    # host, advance it with the oracle, compare the whole 512 MiB layer
    worst_s = worst_o = 0.0
    og = outs.cpu().numpy()
    for l in range(L):
        gi.state_into(sn, seed, l)
        M = sn.copy()
        want = ref.step_mt(orc, ins[l], M)
        worst_s = max(worst_s, ref.max_abs_err(states[l].cpu().numpy(), M))
        worst_o = max(worst_o, ref.max_abs_err(og[l], want))
        if l % 6 == 5:
            print(f"    layers 0..{l} checked: state {worst_s:.3e} out {worst_o:.3e}", flush=True)
    assert worst_s <= 1e-6 and worst_o <= 1e-5, (worst_s, worst_o)

    # The same memory as one flattened B=9216 call (one more token), checked
    # in full the same way.
    print("    flattened B=9216 call", flush=True)
    flat = states.view(L * B, 32, 128, 128)
    ins2 = [gi.step_inputs(seed + 100, l, B) for l in range(L)]
    d2 = {n: dev(np.concatenate([ins2[l][n] for l in range(L)])) for n in ins2[0]}
    out2 = torch.empty((L * B, 32, 128), device="cuda")
    g.step(d2["q"], d2["k"], d2["v"], d2["beta"], d2["gate"], flat, out2)
    torch.cuda.synchronize()
    o2 = out2.cpu().numpy()
    worst_s = worst_o = 0.0
    for l in range(L):
        gi.state_into(sn, seed, l)
        M = sn.copy()
        ref.step_mt(orc, ins[l], M)                  # the layer's first token
        want = ref.step_mt(orc, ins2[l], M)          # the flattened call's token
        worst_s = max(worst_s, ref.max_abs_err(flat[l * B:(l + 1) * B].cpu().numpy(), M))
        worst_o = max(worst_o, ref.max_abs_err(o2[l * B:(l + 1) * B], want))
        if l % 6 == 5:
            print(f"    flattened, layers 0..{l} checked: state {worst_s:.3e} out {worst_o:.3e}",
                  flush=True)
    assert worst_s <= 1e-6 and worst_o <= 1e-5, (worst_s, worst_o)


@pytest.mark.timeout(600)
def test_seq_b8_t4096(g, orc):
    import torch
    c = gi.WORKLOADS["seq_b8_t4096"]
    B, T = c["B"], c["T"]
    print(f"\n  seq_b8_t4096: gdn_seq B={B} T={T} from zero state", flush=True)
    si = gi.step_inputs(c["seed"], 0, B, T=T)
    M = np.zeros((B, 32, 128, 128), np.float32)
    t = {n: dev(x) for n, x in si.items()}
    Md = dev(M)
    out = torch.empty((B, T, 32, 128), device="cuda")
    g.seq(t["q"], t["k"], t["v"], t["beta"], t["gate"], Md, out)
    torch.cuda.synchronize()
    print("    GPU done; oracle running", flush=True)
    want = ref.seq_mt(orc, si, M)
    ref.assert_close("state", Md.cpu().numpy(), M, 1e-4)
    ref.assert_close("out", out.cpu().numpy(), want, 1e-4)
