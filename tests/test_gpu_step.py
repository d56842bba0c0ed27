"""GPU: gdn_step (through the C ABI) against the oracle, element by element,
plus the properties the pages fix: h % 16 broadcast, the delta-rule
invariant, batch invariance and run-to-run determinism."""
import numpy as np
import pytest

import gdn_inputs as gi
import ref

pytestmark = pytest.mark.gpu

STATE_TOL = 1e-6   # per-step tolerances (absolute)
OUT_TOL = 1e-5


@pytest.fixture(scope="module")
def g():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_deltanet_decode_amd as g
    return g


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_step(g, si, M):
    import torch
    t = {n: dev(x) for n, x in si.items()}
    Md = dev(M)
    out = torch.empty(si["v"].shape, dtype=torch.float32, device="cuda")
    g.step(t["q"], t["k"], t["v"], t["beta"], t["gate"], Md, out)
    torch.cuda.synchronize()
    return Md.cpu().numpy(), out.cpu().numpy()


@pytest.mark.parametrize("B,Hv,Hk", [(1, 32, 16), (3, 32, 16), (5, 4, 2), (2, 1, 1),
                                     (2, 64, 16), (7, 16, 16), (1, 96, 32)])
def test_step_matches_oracle(g, orc, B, Hv, Hk):
    print(f"\n  gdn_step B={B} Hv={Hv} Hk={Hk}", flush=True)
    si = gi.step_inputs(2000 + B, Hv, B, Hv, Hk)
    M = gi.state(2000 + B, Hv, B, Hv)
    Mg, og = run_step(g, si, M)
    want = ref.step_mt(orc, si, M)
    ref.assert_close("state", Mg, M, STATE_TOL)
    ref.assert_close("out", og, want, OUT_TOL)


def test_step_large_launch_matches_oracle(g, orc):
    # 257 x 33 heads = 135,696 tiles in 67,848 staged workgroups of two
    # tiles, with head counts (33 value, 11 key) that are not powers of two.
    B, Hv, Hk = 257, 33, 11
    print(f"\n  gdn_step large launch B={B} Hv={Hv} Hk={Hk}", flush=True)
    si = gi.step_inputs(2600, Hv, B, Hv, Hk)
    M = gi.state(2600, Hv, B, Hv)
    Mg, og = run_step(g, si, M)
    want = ref.step_mt(orc, si, M)
    ref.assert_close("state", Mg, M, STATE_TOL)
    ref.assert_close("out", og, want, OUT_TOL)


def test_step_b1_single_sequence(g, orc, workload):
    """One sequence, one token, the page geometry."""
    workload("step_b1")
    c = gi.WORKLOADS["step_b1"]
    print("\n  gdn_step B=1 (step_b1)", flush=True)
    si = gi.step_inputs(c["seed"], 0, 1)
    M = gi.state(c["seed"], 0, 1)
    M64 = M.astype(np.float64)
    Mg, og = run_step(g, si, M)
    want = orc.step_M(si["q"], si["k"], si["v"], si["beta"], si["gate"], M)
    out64 = orc.step_f64(si["q"], si["k"], si["v"], si["beta"], si["gate"], M64)
    ref.assert_close("state", Mg, M, STATE_TOL)
    ref.assert_close("out", og, want, OUT_TOL)
    # the binary64 yardstick: GPU error within a small factor of the f32 oracle's
    ref.assert_vs_f64("state", Mg, M, M64)
    ref.assert_vs_f64("out", og, want, out64)


def test_broadcast_and_delta_rule_on_gpu(g):
    """beta=1, gate=0, unit k: the GPU's updated state satisfies M'k = v with
    the key head h % 16; heads h and h+16 fed the same v and state agree
    bitwise."""
    print("\n  gdn_step broadcast / delta rule", flush=True)
    si = gi.step_inputs(2100, 0, 2)
    si["beta"][:] = 1.0
    si["gate"][:] = 0.0
    si["v"][:, 16:] = si["v"][:, :16]
    M = gi.state(2100, 0, 2)
    M[:, 16:] = M[:, :16]
    Mg, og = run_step(g, si, M)
    for b in range(2):
        for h in range(32):
            r = Mg[b, h].astype(np.float64) @ si["k"][b, h % 16].astype(np.float64)
            assert np.max(np.abs(r - si["v"][b, h])) <= 2e-6, (b, h)
            if h % 16 != h // 2:
                r2 = Mg[b, h].astype(np.float64) @ si["k"][b, h // 2].astype(np.float64)
                assert np.max(np.abs(r2 - si["v"][b, h])) > 1e-3, (b, h)
        assert np.array_equal(Mg[b, :16], Mg[b, 16:]) and np.array_equal(og[b, :16], og[b, 16:])


def test_batch_invariance_and_determinism(g):
    """A sequence's result is bitwise independent of the batch it runs in, and
    two runs on the same inputs are bitwise equal."""
    print("\n  gdn_step batch invariance", flush=True)
    si = gi.step_inputs(2200, 0, 6)
    M = gi.state(2200, 0, 6)
    M6, o6 = run_step(g, si, M)
    M6b, o6b = run_step(g, si, M)
    assert np.array_equal(M6, M6b) and np.array_equal(o6, o6b), "not deterministic"
    s1 = gi.step_inputs(2200, 0, 1, b0=4)      # sequence 4 alone, regenerated
    M1 = gi.state(2200, 0, 1, b0=4)
    M1g, o1g = run_step(g, s1, M1)
    assert np.array_equal(M1g[0], M6[4]) and np.array_equal(o1g[0], o6[4]), "batch dependence"


def test_special_cases_on_gpu(g, orc):
    """Full forget (gate=-1e4), pure decay (beta=0), zero state, zero k."""
    print("\n  gdn_step special cases", flush=True)
    for case in ("forget", "decay", "zero_state", "zero_k"):
        si = gi.step_inputs(2300, 0, 2)
        M = gi.state(2300, 0, 2)
        if case == "forget":
            si["gate"][:] = -1e4
        elif case == "decay":
            si["beta"][:] = 0
        elif case == "zero_state":
            M[:] = 0
        else:
            si["k"][:] = 0
        Mg, og = run_step(g, si, M)
        want = ref.step_mt(orc, si, M)
        ref.assert_close(case + " state", Mg, M, STATE_TOL)
        ref.assert_close(case + " out", og, want, OUT_TOL)


def test_rejected_call_leaves_buffers_untouched(g):
    """An argument error is reported before anything is enqueued."""
    import ctypes
    import torch
    print("\n  gdn_step rejected call", flush=True)
    si = gi.step_inputs(2400, 0, 2)
    M = gi.state(2400, 0, 2)
    t = {n: dev(x) for n, x in si.items()}
    Md = dev(M)
    out = torch.full((2, 32, 128), 7.0, device="cuda")
    rc = g.lib.gdn_step(ctypes.byref(g.PAGE_DIMS), 2, t["q"].data_ptr() + 4, t["k"].data_ptr(),
                        t["v"].data_ptr(), t["beta"].data_ptr(), t["gate"].data_ptr(),
                        Md.data_ptr(), out.data_ptr(), None)
    torch.cuda.synchronize()
    assert rc == -3 and "q" in g.last_error()
    assert np.array_equal(Md.cpu().numpy(), M) and bool((out == 7.0).all())


def test_unaligned_to_cache_lines(g, orc):
    """Buffers that are 16-byte aligned but not 128-byte aligned (views at a
    16-byte offset into larger allocations) give the same results."""
    import torch
    print("\n  gdn_step at 16-byte offsets", flush=True)
    B = 3
    si = gi.step_inputs(2500, 0, B)
    M = gi.state(2500, 0, B)
    want_M = M.copy()
    want = ref.step_mt(orc, si, want_M)

    def shifted(a):
        buf = torch.zeros(a.size + 4, dtype=torch.float32, device="cuda")
        view = buf[4:].view(a.shape)
        view.copy_(torch.from_numpy(np.ascontiguousarray(a)))
        return view
    t = {n: shifted(x) for n, x in si.items()}
    Md = shifted(M)
    out = torch.zeros(B * 32 * 128 + 4, device="cuda")[4:].view(B, 32, 128)
    assert Md.data_ptr() % 128 == 16
    g.step(t["q"], t["k"], t["v"], t["beta"], t["gate"], Md, out)
    torch.cuda.synchronize()
    ref.assert_close("state", Md.cpu().numpy(), want_M, STATE_TOL)
    ref.assert_close("out", out.cpu().numpy(), want, OUT_TOL)


def test_nan_stays_in_its_row(g):
    """A NaN in one v entry (sequence 1, head 5, row 7) reaches exactly that
    state row and that output; every other row, head and sequence is
    bitwise what it is without the NaN (rows never exchange data)."""
    print("\n  gdn_step NaN isolation", flush=True)
    si = gi.step_inputs(2600, 0, 3)
    M = gi.state(2600, 0, 3)
    clean_M, clean_o = run_step(g, si, M)
    si["v"][1, 5, 7] = np.nan
    Mg, og = run_step(g, si, M)
    assert np.all(np.isnan(Mg[1, 5, 7])) and np.isnan(og[1, 5, 7])
    mask = np.ones(Mg.shape[:3], bool)
    mask[1, 5, 7] = False
    assert np.array_equal(Mg[mask], clean_M[mask]) and np.array_equal(og[mask], clean_o[mask])


# B = 1: one wave per tile (both policies); 64: the Infinity-Cache resident
# decode (cached: 8 tiles per wave, 4 waves per workgroup; default: the
# staged kernel); 17 x 33 heads: the last cached workgroup half empty;
# 300 x 33 heads: a large staged launch
@pytest.mark.parametrize("B,Hv,Hk", [(1, 32, 16), (64, 32, 16), (17, 33, 11), (300, 33, 11)])
def test_step_cached_policy_is_bitwise(g, orc, B, Hv, Hk):
    """gdn_step_ex with GDN_STATE_CACHED (state through the caches) gives the
    bits of gdn_step (nontemporal state), over two chained calls, and matches
    the oracle."""
    import torch
    print(f"\n  gdn_step_ex cached B={B} Hv={Hv} Hk={Hk}", flush=True)
    M = gi.state(2700 + B, 0, B, Hv)
    Mn, Mc = dev(M), dev(M)
    outs = []
    for call in range(2):
        si = gi.step_inputs(2700 + B, call + 1, B, Hv, Hk)
        t = {n: dev(x) for n, x in si.items()}
        on = torch.empty((B, Hv, 128), device="cuda")
        oc = torch.empty_like(on)
        g.step(t["q"], t["k"], t["v"], t["beta"], t["gate"], Mn, on)
        g.step(t["q"], t["k"], t["v"], t["beta"], t["gate"], Mc, oc, cached=True)
        want = ref.step_mt(orc, si, M)
        outs.append((on, oc, want))
    torch.cuda.synchronize()
    assert np.array_equal(Mn.cpu().numpy(), Mc.cpu().numpy()), "state differs between policies"
    for on, oc, want in outs:
        assert np.array_equal(on.cpu().numpy(), oc.cpu().numpy()), "out differs between policies"
        ref.assert_close("out", oc.cpu().numpy(), want, OUT_TOL)
    ref.assert_close("state", Mc.cpu().numpy(), M, STATE_TOL)
