"""GPU: the full-size workloads, in the launch configuration the benchmark
times, checked against the oracle element by element (every sequence of every
layer for step_b256_x36, whose pre-states are regenerated on the host layer
by layer).

  step_b64_x100: B=64 decode, 100 gdn_step calls with fresh inputs (both
                 cache policies the benchmark times)
  step_b256_x36: B=256 x 36 layers (18 GiB of state), one gdn_step per
                 layer, plus the same 36 layers flattened into one B=9216 call
  seq_b8_t4096:  gdn_seq B=8 x T=4096 from a zero state
  seq_b256_t64:  gdn_seq B=256 x T=64 from seeded states (the benchmark's
                 many-heads short-sequence line)
  seq_b40_t1024: gdn_seq B=40 x T=1024 from seeded states (the benchmark's
                 many-heads long-sequence line; 8 of the sequences checked)
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
def test_step_b64_x100(g, orc, workload):
    import torch
    workload("step_b64_x100")
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
    # the same 100 calls with GDN_STATE_CACHED (the benchmark's cached line):
    # bitwise the default policy's results
    Mc = dev(M)
    outs_c = torch.empty_like(outs)
    for i in range(calls):
        t = dins[i]
        g.step(t["q"], t["k"], t["v"], t["beta"], t["gate"], Mc, outs_c[i], cached=True)
    torch.cuda.synchronize()
    Mg, og = Md.cpu().numpy(), outs.cpu().numpy()
    assert np.array_equal(Mc.cpu().numpy(), Mg) and np.array_equal(outs_c.cpu().numpy(), og), \
        "cached policy differs from the default over 100 calls"
    worst = 0.0
    M64 = M.astype(np.float64)
    e_gpu = e_orc = 0.0
    for i in range(calls):
        want = ref.step_mt(orc, inputs[i], M)
        out64 = ref.step_f64_mt(orc, inputs[i], M64)
        if i == 0:
            ref.assert_close("state@1", M1, M, 1e-6)
        worst = max(worst, ref.max_err(og[i], want)[0])
        e_gpu = max(e_gpu, ref.max_abs_err64(og[i], out64))
        e_orc = max(e_orc, ref.max_abs_err64(want, out64))
        assert worst <= 1e-5, f"call {i}: out error {worst:.3e}"
    ref.assert_abs_bound(f"all {calls} outs", worst, 1e-5)
    ref.assert_close("state@100", Mg, M, 1e-6)
    ref.assert_f64_ratio(f"all {calls} outs", e_gpu, e_orc)
    ref.assert_vs_f64("state@100", Mg, M, M64)


@pytest.mark.timeout(900)
def test_step_b256_x36_layers(g, orc, workload):
    import torch
    workload("step_b256_x36")
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
    f64 = {"gs": 0.0, "os": 0.0, "go": 0.0, "oo": 0.0}
    for l in range(L):
        gi.state_into(sn, seed, l)
        M = sn.copy()
        if l in (0, L - 1):     # the binary64 yardstick on the first and last layer
            M64 = sn.astype(np.float64)
            out64 = ref.step_f64_mt(orc, ins[l], M64)
        want = ref.step_mt(orc, ins[l], M)
        Ml = states[l].cpu().numpy()
        worst_s = max(worst_s, ref.max_abs_err(Ml, M))
        worst_o = max(worst_o, ref.max_abs_err(og[l], want))
        if l in (0, L - 1):
            f64["gs"] = max(f64["gs"], ref.max_abs_err64(Ml, M64))
            f64["os"] = max(f64["os"], ref.max_abs_err64(M, M64))
            f64["go"] = max(f64["go"], ref.max_abs_err64(og[l], out64))
            f64["oo"] = max(f64["oo"], ref.max_abs_err64(want, out64))
        if l % 6 == 5:
            print(f"    layers 0..{l} checked: state {worst_s:.3e} out {worst_o:.3e}", flush=True)
    ref.assert_abs_bound("state, 36 layers", worst_s, 1e-6)
    ref.assert_abs_bound("out, 36 layers", worst_o, 1e-5)
    ref.assert_f64_ratio("state, layers 0 and 35", f64["gs"], f64["os"])
    ref.assert_f64_ratio("out, layers 0 and 35", f64["go"], f64["oo"])

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
    ref.assert_abs_bound("flattened B=9216 state", worst_s, 1e-6)
    ref.assert_abs_bound("flattened B=9216 out", worst_o, 1e-5)


@pytest.mark.timeout(900)
def test_seq_b8_t4096(g, orc, workload):
    """gdn_seq (scaled decay) and gdn_seq_exact at full size against the
    oracle (1e-4), both against the binary64 shadow (within the yardstick
    factor of the f32 oracle's own error), and the gap between the two forms
    (within twice that)."""
    import torch
    workload("seq_b8_t4096")
    c = gi.WORKLOADS["seq_b8_t4096"]
    B, T = c["B"], c["T"]
    print(f"\n  seq_b8_t4096: gdn_seq and gdn_seq_exact B={B} T={T} from zero state", flush=True)
    si = gi.step_inputs(c["seed"], 0, B, T=T)
    M = np.zeros((B, 32, 128, 128), np.float32)
    t = {n: dev(x) for n, x in si.items()}
    res = {}
    for exact in (False, True):
        Md = dev(M)
        out = torch.empty((B, T, 32, 128), device="cuda")
        g.seq(t["q"], t["k"], t["v"], t["beta"], t["gate"], Md, out, exact=exact)
        torch.cuda.synchronize()
        res[exact] = (Md.cpu().numpy(), out.cpu().numpy())
        del Md, out
    print("    GPU done; oracle (f32 and f64) running", flush=True)
    M64 = M.astype(np.float64)
    want = ref.seq_mt(orc, si, M)
    out64 = ref.seq_f64_mt(orc, si, M64)
    for exact, tag in ((False, "seq"), (True, "seq_exact")):
        Mg, og = res[exact]
        ref.assert_close(f"{tag} state", Mg, M, 1e-4)
        ref.assert_close(f"{tag} out", og, want, 1e-4)
        ref.assert_vs_f64(f"{tag} state", Mg, M, M64)
        ref.assert_vs_f64(f"{tag} out", og, want, out64)
    for i, what, o32, o64 in ((0, "state", M, M64), (1, "out", want, out64)):
        gap = ref.max_abs_err(res[False][i], res[True][i])
        e_orc = ref.max_abs_err64(o32, o64)
        bound = 2 * ref.F64_FACTOR * e_orc + 1e-12
        ref.record(name=f"seq vs seq_exact {what}", max_abs=gap, bound=bound, passed=gap <= bound)
        print(f"    seq vs seq_exact {what}: {gap:.3e} (bound {bound:.3e})", flush=True)
        assert gap <= bound, f"gdn_seq and gdn_seq_exact differ by {gap:.3e} in {what}"


@pytest.mark.timeout(600)
def test_seq_b256_t64(g, orc, workload):
    """gdn_seq at the benchmark's B=256 x T=64 (8192 heads: half heads, three
    workgroups per CU) against the oracle, every element, and the binary64
    yardstick on 8 of the sequences; gdn_seq_exact likewise."""
    import torch
    workload("seq_b256_t64")
    c = gi.WORKLOADS["seq_b256_t64"]
    B, T = c["B"], c["T"]
    print(f"\n  seq_b256_t64: gdn_seq and gdn_seq_exact B={B} T={T}", flush=True)
    si = gi.step_inputs(c["seed"], 0, B, T=T)
    M = gi.state(c["seed"], 0, B)
    t = {n: dev(x) for n, x in si.items()}
    res = {}
    for exact in (False, True):
        Md = dev(M)
        out = torch.empty((B, T, 32, 128), device="cuda")
        g.seq(t["q"], t["k"], t["v"], t["beta"], t["gate"], Md, out, exact=exact)
        torch.cuda.synchronize()
        res[exact] = (Md.cpu().numpy(), out.cpu().numpy())
        del Md, out
    Mo = M.copy()
    want = ref.seq_mt(orc, si, Mo)
    s8 = {n: np.ascontiguousarray(x[:8]) for n, x in si.items()}
    M64 = M[:8].astype(np.float64)
    Mo8 = M[:8].copy()
    want8 = ref.seq_mt(orc, s8, Mo8)
    out64 = ref.seq_f64_mt(orc, s8, M64)
    for exact, tag in ((False, "seq"), (True, "seq_exact")):
        Mg, og = res[exact]
        ref.assert_close(f"{tag} state", Mg, Mo, 1e-6)
        ref.assert_close(f"{tag} out", og, want, 1e-5)
        ref.assert_vs_f64(f"{tag} state[:8]", Mg[:8], Mo8, M64)
        ref.assert_vs_f64(f"{tag} out[:8]", og[:8], want8, out64)


@pytest.mark.timeout(600)
def test_seq_b40_t1024(g, orc, workload):
    """gdn_seq at the benchmark's B=40 x T=1024 (1280 heads: half heads with
    their chunks fetched into LDS, three workgroups per CU), the whole batch
    in one launch; sequences 0-3 and 36-39 against the oracle, every element,
    and the binary64 yardstick on two of them; gdn_seq_exact likewise."""
    import torch
    workload("seq_b40_t1024")
    c = gi.WORKLOADS["seq_b40_t1024"]
    B, T = c["B"], c["T"]
    print(f"\n  seq_b40_t1024: gdn_seq and gdn_seq_exact B={B} T={T}", flush=True)
    si = gi.step_inputs(c["seed"], 0, B, T=T)
    M = gi.state(c["seed"], 0, B)
    t = {n: dev(x) for n, x in si.items()}
    res = {}
    for exact in (False, True):
        Md = dev(M)
        out = torch.empty((B, T, 32, 128), device="cuda")
        g.seq(t["q"], t["k"], t["v"], t["beta"], t["gate"], Md, out, exact=exact)
        torch.cuda.synchronize()
        res[exact] = (Md.cpu().numpy(), out.cpu().numpy())
        del Md, out
    del t
    pick = np.r_[0:4, B - 4:B]
    sp = {n: np.ascontiguousarray(x[pick]) for n, x in si.items()}
    Mo = M[pick].copy()
    want = ref.seq_mt(orc, sp, Mo)
    s2 = {n: np.ascontiguousarray(x[[0, B - 1]]) for n, x in si.items()}
    M64 = M[[0, B - 1]].astype(np.float64)
    out64 = ref.seq_f64_mt(orc, s2, M64)
    for exact, tag in ((False, "seq"), (True, "seq_exact")):
        Mg, og = res[exact]
        ref.assert_close(f"{tag} state", Mg[pick], Mo, 1e-4)
        ref.assert_close(f"{tag} out", og[pick], want, 1e-4)
        ref.assert_vs_f64(f"{tag} state[0,-1]", Mg[[0, B - 1]], Mo[[0, -1]], M64)
        ref.assert_vs_f64(f"{tag} out[0,-1]", og[[0, B - 1]], want[[0, -1]], out64)
