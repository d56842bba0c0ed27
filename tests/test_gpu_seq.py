"""GPU: gdn_seq (state resident on chip over T tokens) against the oracle,
and its contract with gdn_step (docs.rs "Module linear_core",
gdn_forward_batch: sequential over positions, elementwise identical)."""
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


def run_seq(g, si, M, exact=False):
    import torch
    t = {n: dev(x) for n, x in si.items()}
    Md = dev(M)
    out = torch.empty(si["v"].shape, dtype=torch.float32, device="cuda")
    g.seq(t["q"], t["k"], t["v"], t["beta"], t["gate"], Md, out, exact=exact)
    torch.cuda.synchronize()
    return Md.cpu().numpy(), out.cpu().numpy()


def token(si, t):
    return {n: np.ascontiguousarray(x[:, t]) for n, x in si.items()}


# B, T cover every route on a 256-CU MI355X: T = 1 (the single-step
# kernel); up to 64 heads (B = 1, 2), heads split into 16 one-wave or 8
# two-wave workgroups of one tile per wave, with 8-token chunks below 16
# tokens and 16-token chunks from there; otherwise T < 16 (half heads,
# 8-token chunks, full and partial) paired up to 256 heads (B = 4, 8) and
# unpaired beyond (B = 12: 384 heads); 16 <= T <= 64 (half heads, 16-token
# chunks, paired) with the chunk staged through registers up to 256 heads
# (B = 8) and fetched straight into LDS beyond (B = 12: 384 heads, B = 24:
# 768, at any length); beyond 64 tokens with at most 256 heads, 2 parts per
# head while they fit the CUs (B = 3) and whole heads (B = 8).
@pytest.mark.parametrize("B,T,Hv,Hk", [(1, 1, 32, 16), (2, 5, 32, 16), (2, 8, 32, 16),
                                       (1, 17, 32, 16), (1, 24, 32, 16), (2, 32, 32, 16),
                                       (3, 33, 4, 2), (2, 16, 1, 1), (1, 48, 64, 16),
                                       (1, 64, 32, 16), (2, 65, 32, 16), (8, 24, 32, 16),
                                       (12, 9, 32, 16), (24, 20, 32, 16), (1, 70, 32, 16),
                                       (3, 70, 32, 16), (8, 66, 32, 16), (1, 7, 32, 16),
                                       (4, 5, 32, 16), (8, 40, 32, 16), (12, 33, 32, 16)])
def test_seq_matches_oracle(g, orc, B, T, Hv, Hk):
    print(f"\n  gdn_seq B={B} T={T} Hv={Hv} Hk={Hk}", flush=True)
    si = gi.step_inputs(3000 + T, 0, B, Hv, Hk, T=T)
    M = gi.state(3000 + T, 0, B, Hv)
    Mg, og = run_seq(g, si, M)
    M64 = M.astype(np.float64)
    want = ref.seq_mt(orc, si, M)
    out64 = ref.seq_f64_mt(orc, si, M64)
    # The recurrence contracts (0 < exp(gate) < 1, 0 < beta < 1, unit k), so
    # rounding differences do not build up over short runs: the per-step
    # tolerances apply.
    ref.assert_close("state", Mg, M, 1e-6)
    ref.assert_close("out", og, want, 1e-5)
    ref.assert_vs_f64("state", Mg, M, M64)
    ref.assert_vs_f64("out", og, want, out64)


def strong_decay(si):
    """Gates <= -3 everywhere: every 16-token group's decay product is at
    most e^-48, below the scaled form's 2^-63 floor, so every group runs with
    the per-token decay multiply."""
    si = dict(si)
    si["gate"] = (si["gate"] - np.float32(3.0)).astype(np.float32)
    return si


def repeated_steps(g, si, M):
    import torch
    B, T = si["q"].shape[:2]
    Md = dev(M)
    outs = []
    for t in range(T):
        tk = {n: dev(x) for n, x in token(si, t).items()}
        o = torch.empty(tk["v"].shape, device="cuda")
        g.step(tk["q"], tk["k"], tk["v"], tk["beta"], tk["gate"], Md, o)
        outs.append(o)
    torch.cuda.synchronize()
    return Md.cpu().numpy(), torch.stack(outs, 1).cpu().numpy()


@pytest.mark.parametrize("B,T", [(2, 2), (2, 8), (2, 15), (2, 24), (2, 32), (2, 37), (2, 65),
                                 (12, 9), (24, 20), (1, 70), (3, 70), (8, 66), (1, 9), (1, 24),
                                 (4, 8), (8, 32), (2, 16), (4, 64)])
def test_seq_is_bitwise_repeated_step(g, B, T):
    """T tokens in one gdn_seq == T gdn_step calls, bit for bit, whenever no
    group runs scaled: below 16 tokens always, and from 16 tokens on with
    strong decay (every group under the scaled form's floor).  Both paths
    share the per-row arithmetic.  Every route: half heads with 8- and
    16-token chunks, paired and unpaired, heads split in 16, 8 or 2 parts,
    and whole heads."""
    print(f"\n  gdn_seq == repeated gdn_step, B={B} T={T}", flush=True)
    si = gi.step_inputs(3100, 0, B, T=T)
    if T >= 16:
        si = strong_decay(si)
    M = gi.state(3100, 0, B)
    Ms, os_ = run_seq(g, si, M)
    Md, od = repeated_steps(g, si, M)
    assert np.array_equal(Md, Ms), "state differs"
    assert np.array_equal(od, os_), "outputs differ"


@pytest.mark.parametrize("B,T", [(2, 24), (2, 32), (2, 37), (2, 65), (24, 20), (1, 70), (3, 70),
                                 (8, 66), (1, 24), (8, 32), (4, 64), (1, 16), (12, 33), (12, 70)])
def test_seq_exact_is_bitwise_repeated_step(g, B, T):
    """gdn_seq_exact: T tokens == T gdn_step calls, bit for bit, at any T and
    with ordinary gates (no scaled groups), in every launch shape that takes
    16 or more tokens."""
    print(f"\n  gdn_seq_exact == repeated gdn_step, B={B} T={T}", flush=True)
    si = gi.step_inputs(3150, 0, B, T=T)
    M = gi.state(3150, 0, B)
    Ms, os_ = run_seq(g, si, M, exact=True)
    Md, od = repeated_steps(g, si, M)
    assert np.array_equal(Md, Ms), "state differs"
    assert np.array_equal(od, os_), "outputs differ"


# other head counts on the many-heads routes (more heads than CUs): 64 value
# heads per key head group of 16, one head of each kind, 4 value heads per
# key head
@pytest.mark.parametrize("B,T,Hv,Hk", [(5, 80, 64, 16), (300, 16, 1, 1), (64, 20, 32, 8)])
def test_seq_exact_other_head_counts(g, B, T, Hv, Hk):
    """gdn_seq_exact == T gdn_step calls, bit for bit, with head counts other
    than the page's on the half-head kernel that fetches its chunks into
    LDS."""
    print(f"\n  gdn_seq_exact == repeated gdn_step, B={B} T={T} Hv={Hv} Hk={Hk}", flush=True)
    si = gi.step_inputs(3170, 0, B, Hv, Hk, T=T)
    M = gi.state(3170, 0, B, Hv)
    Ms, os_ = run_seq(g, si, M, exact=True)
    Md, od = repeated_steps(g, si, M)
    assert np.array_equal(Md, Ms), "state differs"
    assert np.array_equal(od, os_), "outputs differ"


def test_seq_exact_matches_oracle_and_resumes_anywhere(g, orc):
    """gdn_seq_exact against the oracle, and split at token 13 (not a
    multiple of 16) it is still bitwise one call."""
    print("\n  gdn_seq_exact B=3 T=40, resume at 13", flush=True)
    B, T, T1 = 3, 40, 13
    si = gi.step_inputs(3250, 0, B, T=T)
    M = gi.state(3250, 0, B)
    Mfull, ofull = run_seq(g, si, M, exact=True)
    a = {n: np.ascontiguousarray(x[:, :T1]) for n, x in si.items()}
    b = {n: np.ascontiguousarray(x[:, T1:]) for n, x in si.items()}
    M1, o1 = run_seq(g, a, M, exact=True)
    M2, o2 = run_seq(g, b, M1, exact=True)
    assert np.array_equal(M2, Mfull) and np.array_equal(np.concatenate([o1, o2], 1), ofull)
    Mo = M.copy()
    want = ref.seq_mt(orc, si, Mo)
    ref.assert_close("state", Mfull, Mo, 1e-6)
    ref.assert_close("out", ofull, want, 1e-5)


def mixed_groups(si):
    """Gates that send the 16-token groups down both paths in one call:
    group 1 holds a full forget (gate = -1e4, exp = 0) and group 2 a positive
    gate (0.3), so both run with the per-token multiply; every other complete
    group runs scaled, and a trailing partial group with the multiply."""
    si = dict(si)
    gate = si["gate"].copy()
    T = gate.shape[1]
    if T > 20:
        gate[:, 20] = -1e4
    if T > 40:
        gate[:, 40] = 0.3
    si["gate"] = gate
    return si


# sequence 0 of each batch size below runs through a different launch shape
# (B = 1: 16 one-tile parts, 16-token chunks; B = 2: 8 parts; B = 3: 2 parts,
# 32-token chunks; B = 8: whole heads, 32-token chunks; T <= 64 with B = 4:
# half heads with the chunk in registers; B = 12, 24: half heads with the
# chunk fetched straight into LDS, 16-token chunks; T = 1040 with B = 16:
# whole heads, kept beyond 1024 tokens where they fill their rounds)
@pytest.mark.parametrize("T,Bs", [(100, (1, 2, 3, 8, 12)), (64, (1, 2, 4, 24)), (37, (1, 4, 24)),
                                  (1040, (1, 12, 16))])
def test_seq_bits_do_not_depend_on_launch_shape(g, orc, T, Bs):
    """The scaled groups are counted from the call's first token in every
    launch shape, and a fold inside a 32-token chunk (pipelined with the next
    token's key product) gives the bits of one at a chunk's end: a sequence's
    results are bitwise the same whatever B (and so the launch shape) it runs
    in.  T = 100 mixes the paths: scaled then per-token within a chunk
    (groups 0, 1), per-token then scaled (2, 3), two scaled (4, 5), and a
    partial group (6); all checked against the oracle."""
    print(f"\n  gdn_seq launch-shape independence T={T} B={Bs}", flush=True)
    res = {}
    for B in Bs:
        si = mixed_groups(gi.step_inputs(3500, 0, B, T=T))
        M = gi.state(3500, 0, B)
        res[B] = run_seq(g, si, M)
    first = res[Bs[0]]
    for B in Bs[1:]:
        assert np.array_equal(res[B][0][:1], first[0][:1]), f"state of sequence 0 differs at B={B}"
        assert np.array_equal(res[B][1][:1], first[1][:1]), f"outputs of sequence 0 differ at B={B}"
    si = mixed_groups(gi.step_inputs(3500, 0, 1, T=T))
    M = gi.state(3500, 0, 1)
    want = ref.seq_mt(orc, si, M)
    ref.assert_close("state", first[0], M, 1e-6)
    ref.assert_close("out", first[1], want, 1e-5)


@pytest.mark.parametrize("B", [1, 8])
def test_seq_scaled_group_floor(g, orc, B):
    """The 2^-63 floor on a group's decay product.  Gates of -2.7 (product
    e^-43.2, above it) run scaled, with the registers holding S / c up to
    6e18 |S|: within tolerance of the oracle, and not bitwise the per-token
    path.  Gates of -2.75 (e^-44, below it) run with the per-token multiply:
    bitwise equal to repeated gdn_step."""
    T = 32
    for gate, scaled in ((-2.7, True), (-2.75, False)):
        print(f"\n  gdn_seq B={B} T={T} gate={gate}", flush=True)
        si = gi.step_inputs(3600, 0, B, T=T)
        si["gate"] = np.full_like(si["gate"], np.float32(gate))
        M = gi.state(3600, 0, B)
        Ms, os_ = run_seq(g, si, M)
        Md, od = repeated_steps(g, si, M)
        if scaled:
            assert not (np.array_equal(Md, Ms) and np.array_equal(od, os_)), \
                "a scaled group gave the per-token bits (not taken?)"
            Mo = M.copy()
            want = ref.seq_mt(orc, si, Mo)
            ref.assert_close("state", Ms, Mo, 1e-6)
            ref.assert_close("out", os_, want, 1e-5)
        else:
            assert np.array_equal(Md, Ms) and np.array_equal(od, os_), "per-token group not bitwise"


@pytest.mark.parametrize("T,T1", [(40, 16), (40, 32), (80, 48), (12, 5)])
def test_seq_chunked_resume_is_bitwise(g, T, T1):
    """Checkpoint/resume: seq(T) == seq(T1) then seq(T - T1) from the saved
    state, bit for bit, when T1 is a multiple of 16 (the scaled groups line
    up) or T < 16."""
    print(f"\n  gdn_seq chunked resume T={T} T1={T1}", flush=True)
    B = 3
    si = gi.step_inputs(3200, 0, B, T=T)
    M = gi.state(3200, 0, B)
    Mfull, ofull = run_seq(g, si, M)
    a = {n: np.ascontiguousarray(x[:, :T1]) for n, x in si.items()}
    b = {n: np.ascontiguousarray(x[:, T1:]) for n, x in si.items()}
    M1, o1 = run_seq(g, a, M)
    M2, o2 = run_seq(g, b, M1)
    assert np.array_equal(M2, Mfull) and np.array_equal(np.concatenate([o1, o2], 1), ofull)


def test_seq_resume_at_any_token_matches_oracle(g, orc):
    """Resume at a token that is not a multiple of 16: the groups shift, so
    the bits may differ from one call, but both match the oracle."""
    print("\n  gdn_seq resume at token 13", flush=True)
    B, T, T1 = 3, 40, 13
    si = gi.step_inputs(3200, 0, B, T=T)
    M = gi.state(3200, 0, B)
    a = {n: np.ascontiguousarray(x[:, :T1]) for n, x in si.items()}
    b = {n: np.ascontiguousarray(x[:, T1:]) for n, x in si.items()}
    M1, o1 = run_seq(g, a, M)
    M2, o2 = run_seq(g, b, M1)
    Mo = M.copy()
    want = ref.seq_mt(orc, si, Mo)
    ref.assert_close("state", M2, Mo, 1e-6)
    ref.assert_close("out", np.concatenate([o1, o2], 1), want, 1e-5)


def test_seq_contraction_from_zero_state(g, orc):
    """Zero initial state (as in the B=8 x T=4096 workload) over a ragged T."""
    print("\n  gdn_seq zero state T=70", flush=True)
    B, T = 2, 70
    si = gi.step_inputs(3300, 0, B, T=T)
    M = np.zeros((B, 32, 128, 128), np.float32)
    Mg, og = run_seq(g, si, M)
    want = ref.seq_mt(orc, si, M)
    ref.assert_close("state", Mg, M, 1e-6)
    ref.assert_close("out", og, want, 1e-5)


def test_seq_keeps_all_associations_with_orthonormal_keys(g):
    """beta=1, gate=0 and T = 128 mutually orthonormal keys per key head:
    every token writes v_t along k_t without disturbing the other
    directions, so after the whole sequence the GPU state satisfies
    M k_s = v_s for all 128 tokens (a full-rank delta-rule check)."""
    print("\n  gdn_seq orthonormal keys T=128", flush=True)
    rng = np.random.default_rng(31)
    B, T, Hv, Hk, d = 2, 128, 32, 16, 128
    q = np.empty((B, T, Hk, d), np.float32)
    k = np.empty((B, T, Hk, d), np.float32)
    for b in range(B):
        for h in range(Hk):
            Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
            k[b, :, h] = Q.T.astype(np.float32)
            qq = rng.standard_normal((T, d))
            q[b, :, h] = (qq / np.linalg.norm(qq, axis=1, keepdims=True)).astype(np.float32)
    si = dict(q=q, k=k, v=rng.standard_normal((B, T, Hv, d)).astype(np.float32),
              beta=np.ones((B, T, Hv), np.float32), gate=np.zeros((B, T, Hv), np.float32))
    M = (0.1 * rng.standard_normal((B, Hv, d, d))).astype(np.float32)
    Mg, _ = run_seq(g, si, M)
    worst = 0.0
    for b in range(B):
        for h in range(Hv):
            R = Mg[b, h].astype(np.float64) @ k[b, :, h % Hk].astype(np.float64).T
            worst = max(worst, ref.max_err(R, si["v"][b, :, h].T)[0])   # NaN -> inf
    print(f"    max |M k_s - v_s| over 128 tokens: {worst:.3e}", flush=True)
    assert worst <= 5e-5


def test_seq_more_heads_than_compute_units(g, orc):
    """B=16 x 32 heads = 512 workgroups (two per CU in turn), ragged T."""
    print("\n  gdn_seq B=16 T=40 (512 heads)", flush=True)
    si = gi.step_inputs(3400, 0, 16, T=40)
    M = gi.state(3400, 0, 16)
    Mg, og = run_seq(g, si, M)
    want = ref.seq_mt(orc, si, M)
    ref.assert_close("state", Mg, M, 1e-6)
    ref.assert_close("out", og, want, 1e-5)


def test_seq_nan_isolation(g):
    """NaN inputs stay where the recurrence puts them (B=3, T=70: 32-token
    chunks, scaled groups).
    - A NaN in v (sequence 0, head 2, row 7, token 40) reaches that state row
      and that row's outputs from token 40 on; everything else is bitwise
      the clean run.
    - A NaN gate (sequence 1, head 5, token 20) fails its group's check, so
      that group multiplies per token, and the NaN decay reaches the whole
      head from token 20 on; the head's first group is bitwise the clean run
      and every other head and sequence is bitwise the clean run."""
    print("\n  gdn_seq NaN isolation B=3 T=70", flush=True)
    B, T = 3, 70
    si = gi.step_inputs(3700, 0, B, T=T)
    M = gi.state(3700, 0, B)
    clean_M, clean_o = run_seq(g, si, M)
    si["v"][0, 40, 2, 7] = np.nan
    si["gate"][1, 20, 5] = np.nan
    Mg, og = run_seq(g, si, M)
    assert np.all(np.isnan(Mg[0, 2, 7])) and np.all(np.isnan(og[0, 40:, 2, 7]))
    assert np.all(np.isnan(Mg[1, 5])) and np.all(np.isnan(og[1, 20:, 5]))
    assert np.all(np.isfinite(og[1, 16:20, 5]))
    assert np.array_equal(og[1, :16, 5], clean_o[1, :16, 5])
    keep_M = np.ones(Mg.shape[:3], bool)
    keep_M[0, 2, 7] = False
    keep_M[1, 5, :] = False
    assert np.array_equal(Mg[keep_M], clean_M[keep_M]), "state changed outside the NaN's reach"
    keep_o = np.ones(og.shape, bool)
    keep_o[0, 40:, 2, 7] = False
    keep_o[1, 16:, 5, :] = False
    assert np.array_equal(og[keep_o], clean_o[keep_o]), "outputs changed outside the NaN's reach"
