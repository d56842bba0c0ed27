"""Pins of the CPU oracle to facts other than itself.

Each ``pin_*`` function takes a loaded ``oracle.Oracle`` and raises
``AssertionError`` when the oracle disagrees with a closed form, an invariant,
brute force on tiny inputs, exact dyadic arithmetic, a textbook library
routine or a value the pages print (``golden/page_geometry.json``).

The same functions run against copies of the oracle with planted mistakes
(``test_oracle_mutants.py``): every planted mistake must trip at least one pin.

Sources, by page title and section:
  dev15c  "Red Lite dev15c - Gated DeltaNet recurrent-state parity",
          "Scope" and "Pinned llama.cpp semantics".
  dev15e  "Red Lite dev15e - complete recurrent DeltaNet layer composition".
  dev15a  "Red Lite dev15a - DeltaNet projection field validation".
  linear_core  docs.rs "Module linear_core", gdn_forward / gdn_forward_batch.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
from scipy.special import expit

import gdn_inputs as gi

GOLDEN = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                     "golden", "page_geometry.json")))


def G(name):
    return GOLDEN[name]["value"]


def _rand_step(rng, B, Hv, Hk, d, state_scale=0.1):
    """Small seeded inputs with the page distributions (arbitrary dims)."""
    def unit(n):
        u = rng.standard_normal(n + (d,))
        return (u / np.linalg.norm(u, axis=-1, keepdims=True)).astype(np.float32)
    q = unit((B, Hk))
    k = unit((B, Hk))
    v = rng.standard_normal((B, Hv, d)).astype(np.float32)
    beta = expit(rng.standard_normal((B, Hv))).astype(np.float32)
    gate = (-np.log1p(np.exp(rng.standard_normal((B, Hv))))).astype(np.float32)
    M = (state_scale * rng.standard_normal((B, Hv, d, d))).astype(np.float32)
    return q, k, v, beta, gate, M


# --------------------------------------------------------------------- step
def pin_exact_dyadic(o):
    """The dev15c update on a 4x4 head whose every intermediate is an exact
    binary32 dyadic: gate=0 (decay factor exactly 1), beta=1/2, sqrt(4)=2.
    Expected values come from the matrix closed form
        S' = e (I - beta k k^T) S + beta k v^T,   out = S'^T q / sqrt(d)
    evaluated in exact rational arithmetic; the oracle must match bit for bit."""
    d = 4
    F = Fraction
    k = [F(1, 2), F(-1, 2), F(1, 2), F(1, 2)]
    q = [F(1), F(1, 2), F(-1, 4), F(0)]
    v = [F(1), F(-2), F(1, 2), F(1, 4)]
    beta = F(1, 2)
    # M[j][i] = S[i][j]
    Mx = [[F((3 * j - 2 * i) % 7 - 3, 4) for i in range(d)] for j in range(d)]
    S = [[Mx[j][i] for j in range(d)] for i in range(d)]
    # closed form on S
    kkS = [[sum(k[i] * k[m] * S[m][j] for m in range(d)) for j in range(d)] for i in range(d)]
    Sn = [[S[i][j] - beta * kkS[i][j] + beta * k[i] * v[j] for j in range(d)] for i in range(d)]
    outx = [sum(Sn[i][j] * q[i] for i in range(d)) / 2 for j in range(d)]
    deltax = [(v[j] - sum(S[i][j] * k[i] for i in range(d))) * beta for j in range(d)]

    f32 = lambda a: np.array(a, dtype=np.float64).astype(np.float32)
    qa = f32([[q]]).reshape(1, 1, d)
    ka = f32([[k]]).reshape(1, 1, d)
    va = f32([[v]]).reshape(1, 1, d)
    ba = np.array([[0.5]], np.float32)
    ga = np.zeros((1, 1), np.float32)
    M = f32(Mx).reshape(1, 1, d, d)
    out, delta = o.step_M(qa, ka, va, ba, ga, M, want_delta=True)
    want_M = np.array([[float(Sn[i][j]) for i in range(d)] for j in range(d)], np.float32)
    assert np.array_equal(M[0, 0], want_M), "state differs from exact arithmetic"
    assert np.array_equal(out[0, 0], f32(outx)), "out differs from exact arithmetic"
    assert np.array_equal(delta[0, 0], f32(deltax)), "delta differs from exact arithmetic"

    Sa = np.ascontiguousarray(f32(Mx).T).reshape(1, 1, d, d)
    outS = o.step_S(qa, ka, va, ba, ga, Sa)
    assert np.array_equal(Sa[0, 0].T, want_M) and np.array_equal(outS[0, 0], f32(outx)), \
        "S-layout step differs from exact arithmetic"


def pin_closed_form_tiny_heads(o):
    """Brute force in long double of the dense closed form derived from the
    dev15c update, on tiny heads (d in 1,2,3,4,8; 2 key heads, 4 value
    heads, value head h on key head h % 2): f32 oracle within 1e-6 abs,
    f64 shadow within 1e-12."""
    rng = np.random.default_rng(11)
    LD = np.longdouble
    for d in (1, 2, 3, 4, 8):
        B, Hv, Hk = 2, 4, 2
        q, k, v, beta, gate, M = _rand_step(rng, B, Hv, Hk, d, state_scale=0.5)
        M0 = M.copy()
        M64 = M.astype(np.float64)
        out = o.step_M(q, k, v, beta, gate, M)
        out64 = o.step_f64(q, k, v, beta, gate, M64)
        for b in range(B):
            for h in range(Hv):
                kh = h % Hk
                kk = k[b, kh].astype(LD)
                qq = q[b, kh].astype(LD)
                S = M0[b, h].T.astype(LD)
                e = np.exp(LD(gate[b, h]))
                bt = LD(beta[b, h])
                Sn = e * (np.eye(d, dtype=LD) - bt * np.outer(kk, kk)) @ S \
                    + bt * np.outer(kk, v[b, h].astype(LD))
                on = Sn.T @ qq / np.sqrt(LD(d))
                assert np.max(np.abs(M[b, h].T - Sn)) <= 1e-6, f"state d={d} b={b} h={h}"
                assert np.max(np.abs(out[b, h] - on)) <= 1e-6, f"out d={d} b={b} h={h}"
                assert np.max(np.abs(M64[b, h].T - Sn)) <= 1e-12, f"f64 state d={d}"
                assert np.max(np.abs(out64[b, h] - on)) <= 1e-12, f"f64 out d={d}"


def pin_delta_rule_invariant(o):
    """beta=1, gate=0, ||k||=1  =>  after the update M' k = v exactly in real
    arithmetic (M'k = Mk + (v - Mk) k.k); page geometry, checked in f64 on the
    f32 result within 1e-6."""
    d, Hv, Hk, B = G("state_key_dim"), G("value_heads"), G("key_heads"), 2
    si = gi.step_inputs(7, 0, B, Hv, Hk, d)
    si["beta"][:] = 1.0
    si["gate"][:] = 0.0
    M = gi.state(7, 0, B, Hv, d)
    o.step_M(si["q"], si["k"], si["v"], si["beta"], si["gate"], M)
    for b in range(B):
        for h in range(Hv):
            r = M[b, h].astype(np.float64) @ si["k"][b, h % Hk].astype(np.float64)
            assert np.max(np.abs(r - si["v"][b, h])) <= 1e-6, f"M'k != v at b={b} h={h}"


def pin_broadcast_h_mod_16(o):
    """dev15c: value head h uses Q/K of key head h % 16 (0..15, 0..15).
    Each key head gets a distinct k; the delta-rule invariant identifies
    which key head each value head used, and that map must equal the printed
    one.  Heads h and h+16 fed identical v, beta, gate and state must give
    bitwise-identical results."""
    d, Hv, Hk = G("state_key_dim"), G("value_heads"), G("key_heads")
    si = gi.step_inputs(8, 0, 1, Hv, Hk, d)
    si["beta"][:] = 1.0
    si["gate"][:] = 0.0
    # heads h and h+16 share v and state
    si["v"][0, Hk:] = si["v"][0, :Hk]
    M = gi.state(8, 0, 1, Hv, d)
    M[0, Hk:] = M[0, :Hk]
    out = o.step_M(si["q"], si["k"], si["v"], si["beta"], si["gate"], M)
    K64 = si["k"][0].astype(np.float64)
    found = []
    for h in range(Hv):
        res = [np.max(np.abs(M[0, h].astype(np.float64) @ K64[c] - si["v"][0, h])) for c in range(Hk)]
        c = int(np.argmin(res))
        assert res[c] <= 1e-6, f"no key head satisfies M'k=v for value head {h}"
        found.append(c)
    assert found == G("broadcast"), f"broadcast map {found} != printed map"
    for h in range(Hk):
        assert np.array_equal(M[0, h], M[0, h + Hk]) and np.array_equal(out[0, h], out[0, h + Hk]), \
            f"heads {h} and {h + Hk} differ"


def pin_pure_decay(o):
    """beta=0: the update is M' = e M and out = e (M q)/sqrt(128), a plain
    matrix-vector product (numpy matmul in f64) - within 1e-6."""
    d, Hv, Hk, B = 128, 32, 16, 2
    si = gi.step_inputs(9, 0, B, Hv, Hk, d)
    si["beta"][:] = 0.0
    M = gi.state(9, 0, B, Hv, d)
    M0 = M.astype(np.float64)
    out = o.step_M(si["q"], si["k"], si["v"], si["beta"], si["gate"], M)
    e = np.exp(si["gate"].astype(np.float64))[:, :, None, None]
    assert np.max(np.abs(M - e * M0) / np.maximum(np.abs(e * M0), 1e-30)) <= 1e-6, "decay"
    qh = si["q"].astype(np.float64)[:, np.arange(Hv) % Hk]           # [B][Hv][d]
    want = (e[..., 0] * np.einsum("bhji,bhi->bhj", M0, qh)) / np.sqrt(128.0)
    assert np.max(np.abs(out - want)) <= 1e-6, "pure-decay output"


def pin_full_forget(o):
    """gate = -1e4: exp underflows to 0, so the old state is forgotten:
    M' = (beta v) k^T (bitwise: one rounding per product, as in float32 numpy)
    and out = beta v (k.q)/sqrt(128)."""
    d, Hv, Hk, B = 128, 32, 16, 2
    si = gi.step_inputs(10, 0, B, Hv, Hk, d)
    si["gate"][:] = -1e4
    M = gi.state(10, 0, B, Hv, d)
    out = o.step_M(si["q"], si["k"], si["v"], si["beta"], si["gate"], M)
    kh = si["k"][:, np.arange(Hv) % Hk]                              # f32
    bv = si["v"] * si["beta"][:, :, None]                             # f32, one rounding
    want = bv[:, :, :, None] * kh[:, :, None, :]
    assert np.array_equal(M, want), "full-forget state is not beta v k^T"
    kq = np.einsum("bhi,bhi->bh", kh.astype(np.float64),
                   si["q"][:, np.arange(Hv) % Hk].astype(np.float64))
    wo = bv.astype(np.float64) * kq[:, :, None] / np.sqrt(128.0)
    assert np.max(np.abs(out - wo)) <= 1e-6, "full-forget output"


def pin_scalar_recurrence(o):
    """d = 1, k = +-1: the step reduces to the scalar recurrence
    m_t = (1 - beta_t) e_t m_{t-1} + beta_t v_t k_t,  out_t = m_t q_t,
    checked over 64 positions of gdn_seq within 1e-5."""
    rng = np.random.default_rng(12)
    T = 64
    k = rng.choice([-1.0, 1.0], size=(1, T, 1, 1)).astype(np.float32)
    q = rng.choice([-1.0, 1.0], size=(1, T, 1, 1)).astype(np.float32)
    v = rng.standard_normal((1, T, 1, 1)).astype(np.float32)
    beta = expit(rng.standard_normal((1, T, 1))).astype(np.float32)
    gate = (-np.log1p(np.exp(rng.standard_normal((1, T, 1))))).astype(np.float32)
    M = np.full((1, 1, 1, 1), 0.3, np.float32)
    out = o.seq(q, k, v, beta, gate, M)
    m = 0.3
    for t in range(T):
        e = np.exp(float(gate[0, t, 0]))
        b = float(beta[0, t, 0])
        m = (1 - b) * e * m + b * float(v[0, t, 0, 0]) * float(k[0, t, 0, 0])
        assert abs(out[0, t, 0, 0] - m * float(q[0, t, 0, 0])) <= 1e-5, f"out at t={t}"
    assert abs(M[0, 0, 0, 0] - m) <= 1e-5, "final scalar state"


def pin_orthonormal_keys_are_all_remembered(o):
    """With beta=1, gate=0 and T mutually orthonormal keys, each delta-rule
    update writes v_t along k_t without disturbing the other directions, so
    after the whole sequence M k_s = v_s for every s <= T (and the output of
    token t is M_t q_t / sqrt(d)).  Checked on gdn_seq at the page geometry
    with T = 24 tokens, each key head getting its own orthonormal set."""
    rng = np.random.default_rng(21)
    B, T, Hv, Hk, d = 2, 24, 32, 16, 128
    q = np.empty((B, T, Hk, d), np.float32)
    k = np.empty((B, T, Hk, d), np.float32)
    for b in range(B):
        for h in range(Hk):
            Q, _ = np.linalg.qr(rng.standard_normal((d, T)))       # orthonormal columns
            k[b, :, h] = Q.T.astype(np.float32)
            qq = rng.standard_normal((T, d))
            q[b, :, h] = (qq / np.linalg.norm(qq, axis=1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((B, T, Hv, d)).astype(np.float32)
    beta = np.ones((B, T, Hv), np.float32)
    gate = np.zeros((B, T, Hv), np.float32)
    M = (0.1 * rng.standard_normal((B, Hv, d, d))).astype(np.float32)
    o.seq(q, k, v, beta, gate, M)
    for b in range(B):
        for h in range(Hv):
            kh = h % Hk
            R = M[b, h].astype(np.float64) @ k[b, :, kh].astype(np.float64).T    # [d][T]
            assert np.max(np.abs(R - v[b, :, h].astype(np.float64).T)) <= 2e-5, \
                f"association lost at b={b} h={h}"


def pin_seq_is_repeated_step(o):
    """linear_core: the batch path is the single-token step applied to the
    positions in order, elementwise identical (bitwise here)."""
    rng = np.random.default_rng(13)
    B, T, Hv, Hk, d = 2, 5, 4, 2, 8
    qs, ks, vs, bs, gs = [], [], [], [], []
    for _ in range(T):
        q, k, v, beta, gate, M0 = _rand_step(rng, B, Hv, Hk, d)
        qs.append(q); ks.append(k); vs.append(v); bs.append(beta); gs.append(gate)
    st = lambda xs: np.ascontiguousarray(np.stack(xs, axis=1))
    Ms = M0.copy()
    out = o.seq(st(qs), st(ks), st(vs), st(bs), st(gs), Ms)
    Mr = M0.copy()
    for t in range(T):
        ot = o.step_M(qs[t], ks[t], vs[t], bs[t], gs[t], Mr)
        assert np.array_equal(out[:, t], ot), f"seq out differs from step at t={t}"
    assert np.array_equal(Ms, Mr), "seq final state differs from repeated steps"


def pin_seq_f64_closed_form(o):
    """The binary64 sequence: over 6 positions on tiny heads (d in 1, 3, 8;
    2 key / 4 value heads) it follows the dense closed form
    S_t = e_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
    out_t = S_t^T q_t / sqrt(d), iterated in long double, within 1e-12; and
    at the page geometry it equals the binary64 step applied to the positions
    in order (bitwise)."""
    rng = np.random.default_rng(24)
    LD = np.longdouble
    T = 6
    for d in (1, 3, 8):
        B, Hv, Hk = 2, 4, 2
        steps = [_rand_step(rng, B, Hv, Hk, d, state_scale=0.5) for _ in range(T)]
        M0 = steps[0][5]
        st = lambda i: np.ascontiguousarray(np.stack([s[i] for s in steps], axis=1))
        q, k, v, beta, gate = (st(i) for i in range(5))
        M64 = M0.astype(np.float64)
        out = o.seq_f64(q, k, v, beta, gate, M64)
        for b in range(B):
            for h in range(Hv):
                kh = h % Hk
                S = M0[b, h].T.astype(LD)
                for t in range(T):
                    kk = k[b, t, kh].astype(LD)
                    e = np.exp(LD(gate[b, t, h]))
                    bt = LD(beta[b, t, h])
                    S = e * (np.eye(d, dtype=LD) - bt * np.outer(kk, kk)) @ S \
                        + bt * np.outer(kk, v[b, t, h].astype(LD))
                    on = S.T @ q[b, t, kh].astype(LD) / np.sqrt(LD(d))
                    assert np.max(np.abs(out[b, t, h] - on)) <= 1e-12, f"f64 seq out d={d} t={t}"
                assert np.max(np.abs(M64[b, h].T - S)) <= 1e-12, f"f64 seq state d={d}"
    B, T, Hv, Hk, d = 1, 3, 32, 16, 128
    si = gi.step_inputs(25, 0, B, T=T)
    M0 = gi.state(25, 0, B).astype(np.float64)
    Ms = M0.copy()
    out = o.seq_f64(si["q"], si["k"], si["v"], si["beta"], si["gate"], Ms)
    Mr = M0.copy()
    for t in range(T):
        ot = o.step_f64(*(np.ascontiguousarray(si[n][:, t]) for n in ("q", "k", "v", "beta", "gate")),
                        Mr)
        assert np.array_equal(out[:, t], ot), f"f64 seq out differs from f64 step at t={t}"
    assert np.array_equal(Ms, Mr), "f64 seq state differs from repeated f64 steps"


def pin_pair_is_commit_then_tentative_step(o):
    """linear_core gdn_pair: position 1 commits (the state equals one step),
    position 2 runs from the committed state into the tentative buffer (it
    equals the two-position sequence), and the outputs are those of the
    two-position sequence - bitwise.  With d = 1, k = +-1 both positions also
    follow the scalar closed form m' = (1 - beta) e m + beta v k."""
    rng = np.random.default_rng(20)
    B, Hv, Hk, d = 2, 4, 2, 8
    steps = [_rand_step(rng, B, Hv, Hk, d) for _ in range(2)]
    M0 = steps[0][5]
    st = lambda i: np.ascontiguousarray(np.stack([steps[0][i], steps[1][i]], axis=1))
    q, k, v, beta, gate = (st(i) for i in range(5))
    M = M0.copy()
    out, Mn = o.pair(q, k, v, beta, gate, M)
    M1 = M0.copy()
    o1 = o.step_M(*steps[0][:5], M1)
    M2 = M0.copy()
    o2 = o.seq(q, k, v, beta, gate, M2)
    assert np.array_equal(M, M1), "committed state is not one step"
    assert np.array_equal(Mn, M2), "tentative state is not the two-position sequence"
    assert np.array_equal(out[:, 0], o1) and np.array_equal(out, o2), "pair outputs"
    # scalar closed form
    kk = np.array([1.0, -1.0], np.float32).reshape(1, 2, 1, 1)
    qq = np.array([-1.0, 1.0], np.float32).reshape(1, 2, 1, 1)
    vv = np.array([0.7, -1.3], np.float32).reshape(1, 2, 1, 1)
    bb = np.array([0.25, 0.6], np.float32).reshape(1, 2, 1)
    gg = np.array([-0.3, -1.1], np.float32).reshape(1, 2, 1)
    M = np.full((1, 1, 1, 1), 0.4, np.float32)
    out, Mn = o.pair(qq, kk, vv, bb, gg, M)
    m1 = (1 - 0.25) * np.exp(np.float64(np.float32(-0.3))) * 0.4 + 0.25 * float(np.float32(0.7))
    m2 = (1 - 0.6) * np.exp(np.float64(np.float32(-1.1))) * m1 + 0.6 * float(np.float32(-1.3)) * -1
    assert abs(M[0, 0, 0, 0] - m1) <= 1e-6 and abs(Mn[0, 0, 0, 0] - m2) <= 1e-6, "scalar pair"
    assert abs(out[0, 0, 0, 0] - (-m1)) <= 1e-6 and abs(out[0, 1, 0, 0] - m2) <= 1e-6, "scalar pair out"


def pin_batch_invariance(o):
    """Sequences are independent: sequence b's result does not depend on the
    batch it is computed in (bitwise)."""
    d, Hv, Hk, B = 128, 32, 16, 3
    si = gi.step_inputs(14, 0, B, Hv, Hk, d)
    M = gi.state(14, 0, B, Hv, d)
    M1 = M[1:2].copy()
    out = o.step_M(si["q"], si["k"], si["v"], si["beta"], si["gate"], M)
    s1 = {n: np.ascontiguousarray(a[1:2]) for n, a in si.items()}
    out1 = o.step_M(s1["q"], s1["k"], s1["v"], s1["beta"], s1["gate"], M1)
    assert np.array_equal(out[1:2], out1) and np.array_equal(M[1:2], M1), "batch dependence"


def pin_transposed_layout(o):
    """dev15c: the state is stored transposed, M[j][i] = S[i][j].  The step on
    M and the step on S = M^T agree (within 1e-7; equal here)."""
    d, Hv, Hk, B = 128, 32, 16, 2
    si = gi.step_inputs(15, 0, B, Hv, Hk, d)
    M = gi.state(15, 0, B, Hv, d)
    S = np.ascontiguousarray(np.swapaxes(M, 2, 3))
    outM, dM = o.step_M(si["q"], si["k"], si["v"], si["beta"], si["gate"], M, want_delta=True)
    outS, dS = o.step_S(si["q"], si["k"], si["v"], si["beta"], si["gate"], S, want_delta=True)
    assert np.max(np.abs(np.swapaxes(S, 2, 3) - M)) <= 1e-7, "M vs S state"
    assert np.max(np.abs(outM - outS)) <= 1e-7 and np.max(np.abs(dM - dS)) <= 1e-7, "M vs S out"


# --------------------------------------------------------------------- tail
def _silu64(x):
    x = np.asarray(x, np.float64)
    return x * expit(x)


def pin_conv_special_cases(o):
    """dev15a conv-state shift + causal conv1d (kernel 4, 3-slot cache) + SiLU:
    taps [0,0,0,1] give SiLU(x); taps [1,0,0,0] give SiLU(oldest cache slot);
    after three tokens the cache holds exactly those three raw inputs; and a
    run over six tokens equals numpy's 'valid' convolution of the whole
    sequence [cache, x_1..x_6] with the reversed taps, through SiLU."""
    rng = np.random.default_rng(16)
    B, C, K = 2, 24, 4
    xs = rng.standard_normal((6, B, C)).astype(np.float32)
    cs0 = rng.standard_normal((B, K - 1, C)).astype(np.float32)

    w = np.zeros((C, K), np.float32); w[:, 3] = 1
    cs = cs0.copy()
    act = o.conv_silu(xs[0], w, cs)
    assert np.max(np.abs(act - _silu64(xs[0])) / (1e-30 + np.abs(_silu64(xs[0])))) <= 1e-6, "tap 3"
    w = np.zeros((C, K), np.float32); w[:, 0] = 1
    cs = cs0.copy()
    act = o.conv_silu(xs[0], w, cs)
    assert np.max(np.abs(act - _silu64(cs0[:, 0]))) <= 1e-6, "tap 0 reads oldest slot"

    w = (0.05 * rng.standard_normal((C, K))).astype(np.float32)
    cs = cs0.copy()
    acts = []
    for t in range(6):
        acts.append(o.conv_silu(xs[t], w, cs))
        if t == 2:
            assert np.array_equal(cs, np.stack(xs[:3], axis=1)), "cache != last 3 raw inputs"
    assert np.array_equal(cs, np.stack(xs[3:6], axis=1)), "cache after 6 tokens"
    zero = o.conv_silu(np.zeros((B, C), np.float32), np.ones((C, K), np.float32),
                       np.zeros((B, K - 1, C), np.float32))
    assert np.all(zero == 0.0), "SiLU(0) != 0"
    for b in range(B):
        for c in range(C):
            seqv = np.concatenate([cs0[b, :, c], xs[:, b, c]]).astype(np.float64)
            conv = np.convolve(seqv, w[c, ::-1].astype(np.float64), mode="valid")
            got = np.array([acts[t][b, c] for t in range(6)])
            assert np.max(np.abs(got - _silu64(conv))) <= 1e-6, f"conv b={b} c={c}"


def pin_l2_norm(o):
    """dev15a, the L2 norm of each Q and K head: every row gets unit Euclidean
    norm (within 1e-6) and keeps its direction (numpy.linalg.norm in f64);
    an all-zero row stays zero instead of turning into NaN."""
    rng = np.random.default_rng(17)
    u = rng.standard_normal((5, 128)).astype(np.float32) * np.float32(3.0)
    u[2] *= np.float32(1e-3)
    u[4] = 0
    n = o.l2norm_rows(u)
    for r in range(4):
        assert abs(np.linalg.norm(n[r].astype(np.float64)) - 1) <= 1e-6, f"norm row {r}"
        want = u[r].astype(np.float64) / np.linalg.norm(u[r].astype(np.float64))
        assert np.max(np.abs(n[r] - want)) <= 1e-6, f"direction row {r}"
    assert np.all(n[4] == 0), "zero row"


def pin_gated_rmsnorm(o):
    """dev15e gated RMSNorm x SiLU(z), eps 1e-6 (dev15a prints 9.99999997e-07):
      * w=1, z=c: mean((y/SiLU(c))^2) over a group = m/(m+eps), m = mean(o^2),
        at m ~ 1 and at m ~ 1e-6 where eps matters;
      * o=1, z=c: y/(SiLU(c)/sqrt(1+eps)) reproduces w by position in group;
      * o=1, w=1: y = SiLU(z)/sqrt(1+eps) (scipy expit in f64);
      * groups are independent (changing one group leaves the others bitwise)."""
    rng = np.random.default_rng(18)
    eps = float(np.float32(1e-6))
    group, n, rows = 128, 512, 3
    c = 0.7
    sc = _silu64(np.float32(c))
    for scale in (1.0, 1e-3):
        o_ = (scale * rng.standard_normal((rows, n))).astype(np.float32)
        y = o.gated_rmsnorm(o_, np.full((rows, n), c, np.float32), np.ones(group, np.float32), group)
        for r in range(rows):
            for g in range(0, n, group):
                m = np.mean(o_[r, g:g + group].astype(np.float64) ** 2)
                got = np.mean((y[r, g:g + group].astype(np.float64) / sc) ** 2)
                assert abs(got - m / (m + eps)) <= 1e-5 * m / (m + eps), f"rms scale={scale}"
    w = (1 + 0.02 * rng.standard_normal(group)).astype(np.float32)
    y = o.gated_rmsnorm(np.ones((rows, n), np.float32), np.full((rows, n), c, np.float32), w, group)
    ratio = y.astype(np.float64) / (sc / np.sqrt(1 + eps))
    assert np.max(np.abs(ratio - np.tile(w, n // group))) <= 2e-6, "weight indexing"
    z = rng.standard_normal((rows, n)).astype(np.float32) * np.float32(3)
    y = o.gated_rmsnorm(np.ones((rows, n), np.float32), z, np.ones(group, np.float32), group)
    assert np.max(np.abs(y - _silu64(z) / np.sqrt(1 + eps))) <= 2e-6, "SiLU(z) gate"
    o_ = rng.standard_normal((rows, n)).astype(np.float32)
    y1 = o.gated_rmsnorm(o_, z, w, group)
    o2 = o_.copy(); o2[:, group:2 * group] *= 5
    y2 = o.gated_rmsnorm(o2, z, w, group)
    keep = np.r_[0:group, 2 * group:n]
    assert np.array_equal(y1[:, keep], y2[:, keep]), "groups not independent"


def pin_tail_composition(o):
    """dev15e stage order on the page geometry: conv-state shift + conv1d +
    SiLU, split [Q | K | V] with the printed widths qk=2048 / value=4096 of
    8192 channels, per-head L2 of Q and K, the state step, gated RMSNorm x
    SiLU(z).  The one-call tail equals the stages called one by one
    (bitwise), and the printed cache sizes hold."""
    Hv, Hk, d = G("value_heads"), G("key_heads"), G("state_key_dim")
    qk, vw, C = G("qk_width"), G("value_width"), G("channels")
    assert Hk * d == qk and Hv * d == vw and 2 * qk + vw == C, "geometry"
    assert (gi.CONV_K - 1) * C * 4 == G("conv_cache_bytes"), "conv cache size"
    assert Hv * d * d * 4 == G("recurrent_cache_bytes"), "recurrent cache size"
    B = 2
    ti = gi.tail_inputs(19, B)
    M = gi.state(19, 0, B)
    cs = ti["conv_state"].copy()
    M1, cs1 = M.copy(), cs.copy()
    y, qkv, core = o.layer_tail(ti["x"], ti["conv_w"], cs, ti["beta"], ti["gate"], M,
                                ti["z"], ti["norm_w"], Hk, d)
    act = o.conv_silu(ti["x"], ti["conv_w"], cs1)
    Q = o.l2norm_rows(act[:, :qk].reshape(B, Hk, d))
    Kk = o.l2norm_rows(act[:, qk:2 * qk].reshape(B, Hk, d))
    V = np.ascontiguousarray(act[:, 2 * qk:].reshape(B, Hv, d))
    out = o.step_M(Q, Kk, V, ti["beta"], ti["gate"], M1)
    y1 = o.gated_rmsnorm(out.reshape(B, vw), ti["z"], ti["norm_w"], gi.NORM_GROUP)
    assert np.array_equal(cs, cs1) and np.array_equal(M, M1), "tail caches"
    assert np.array_equal(qkv, np.concatenate([Q.reshape(B, qk), Kk.reshape(B, qk), V.reshape(B, vw)], 1)), "qkv"
    assert np.array_equal(core, out) and np.array_equal(y, y1), "tail outputs"


def pin_tail_pair_ring_and_state_move_together(o):
    """linear_core gdn_pair over the tail, conv ring and state held aside together:
      * the committed conv ring holds [cs_1, cs_2, x_1] and the tentative one
        [cs_2, x_1, x_2] (the last K-1 raw inputs after each position,
        bitwise, independent of any arithmetic);
      * the committed ring, state and y_1 are those of one layer tail at
        position 1, and the tentative ring, state and y_2 those of one layer
        tail at position 2 started from them (bitwise);
      * with beta = 0 at both positions the state only decays: committed
        e_1 M, tentative e_2 e_1 M (f64, within 1e-6 relative)."""
    Hv, Hk, d = G("value_heads"), G("key_heads"), G("state_key_dim")
    B = 2
    t1, t2 = gi.tail_inputs(26, B, slot=0), gi.tail_inputs(26, B, slot=1)
    cs0 = t1["conv_state"].copy()
    M0 = gi.state(26, 0, B)
    pr = lambda n: np.ascontiguousarray(np.stack([t1[n], t2[n]], axis=1))
    x, beta, gate, z = pr("x"), pr("beta"), pr("gate"), pr("z")
    cs, M = cs0.copy(), M0.copy()
    y, csn, Mn = o.layer_tail_pair(x, t1["conv_w"], cs, beta, gate, M, z, t1["norm_w"], Hk, d)
    assert np.array_equal(cs, np.concatenate([cs0[:, 1:], t1["x"][:, None]], axis=1)), \
        "committed ring is not [cs_1, cs_2, x_1]"
    assert np.array_equal(csn, np.concatenate([cs0[:, 2:], t1["x"][:, None], t2["x"][:, None]],
                                              axis=1)), "tentative ring is not [cs_2, x_1, x_2]"
    cs1, M1 = cs0.copy(), M0.copy()
    y1, _, _ = o.layer_tail(t1["x"], t1["conv_w"], cs1, t1["beta"], t1["gate"], M1, t1["z"],
                            t1["norm_w"], Hk, d)
    cs2, M2 = cs1.copy(), M1.copy()
    y2, _, _ = o.layer_tail(t2["x"], t1["conv_w"], cs2, t2["beta"], t2["gate"], M2, t2["z"],
                            t1["norm_w"], Hk, d)
    assert np.array_equal(cs, cs1) and np.array_equal(M, M1), "committed lane is not position 1"
    assert np.array_equal(csn, cs2) and np.array_equal(Mn, M2), "tentative lane is not position 2"
    assert np.array_equal(y[:, 0], y1) and np.array_equal(y[:, 1], y2), "pair outputs"
    beta0 = np.zeros_like(beta)
    M = M0.copy()
    _, _, Mn = o.layer_tail_pair(x, t1["conv_w"], cs0.copy(), beta0, gate, M, z, t1["norm_w"],
                                 Hk, d)
    e = np.exp(gate.astype(np.float64))
    w1 = e[:, 0, :, None, None] * M0
    w2 = e[:, 1, :, None, None] * w1
    rel = lambda a, w: np.max(np.abs(a - w) / np.maximum(np.abs(w), 1e-30))
    assert rel(M, w1) <= 1e-6 and rel(Mn, w2) <= 1e-6, "decay-only pair"


def pin_printed_constants(o):
    """The generator's geometry and the tail epsilon are the printed ones."""
    assert (gi.HV, gi.HK, gi.D) == (G("value_heads"), G("key_heads"), G("state_key_dim"))
    assert gi.D * gi.D * gi.HV * 4 == G("state_bytes_per_layer")
    assert "%.8e" % np.float32(gi.NORM_EPS) == G("rms_epsilon_f32_printed")
    assert gi.D == G("output_scale_divisor_squared")
    assert gi.WORKLOADS["step_b256_x36"]["layers"] == G("recurrent_layers")



# ---------------------------------------------------------- gate transforms
# dev15a names the beta/alpha parameter transforms and prints a 64-output
# projection for them; the formula is a reading (sigmoid for beta, the
# Mamba-2 style gate -exp(A_log) * softplus(alpha + dt_bias)).  These pins tie
# the oracle to closed forms and identities of sigmoid and softplus, not to a
# retyped formula.
def _ulps(x, n):
    return n * np.spacing(np.abs(np.float32(x))).astype(np.float64)


def pin_gate_transform_closed_forms(o):
    """sigmoid(ln m) = m / (1 + m), softplus(ln m) = ln(1 + m), exp(ln n) = n,
    with a different m, n per head (head indexing and the [beta | alpha]
    split of the projection row), plus sigmoid(0) = 1/2 exactly."""
    Hv = G("value_heads")
    assert 2 * Hv == G("beta_alpha_outputs"), "beta/alpha projection width"
    h = np.arange(Hv, dtype=np.float64)
    a_log = np.log(h + 1).astype(np.float32)                    # exp -> h + 1
    dt_bias = (0.25 * (h % 4) - 0.5).astype(np.float32)
    ba = np.empty((2, 2 * Hv), np.float32)
    ba[0, :Hv] = np.log((h + 1) / 2)                            # beta -> (h+1)/(h+3)
    ba[0, Hv:] = (np.log(h + 1) - dt_bias.astype(np.float64))  # a + dt_bias -> ln(h+1)
    ba[1, :Hv] = 0.0                                            # beta -> 1/2 exactly
    ba[1, Hv:] = -dt_bias                                       # softplus(0) = ln 2
    beta, gate = o.gate_transform(ba, a_log, dt_bias)
    want_b = (h + 1) / (h + 3)
    # softplus(ln(h+1)) = ln(h+2); the argument is rounded to f32 on the way
    x = ba[0, Hv:].astype(np.float32) + dt_bias                 # f32 sum, as computed
    want_g = -(h + 1) * np.log(h + 2)
    slack = (h + 1) * np.abs(x.astype(np.float64) - np.log(h + 1)) * ((h + 1) / (h + 2))
    assert np.all(np.abs(beta[0] - want_b) <= _ulps(want_b, 4) + 2e-8), "sigmoid(ln m)"
    assert np.all(np.abs(gate[0] - want_g) <= _ulps(want_g, 8) + slack), "gate closed form"
    assert np.all(beta[1] == np.float32(0.5)), "sigmoid(0)"
    want1 = -(h + 1) * np.log(2.0)                              # -dt_bias + dt_bias = 0 exactly
    assert np.all(np.abs(gate[1] - want1) <= _ulps(want1, 8)), "softplus(0) = ln 2"


def pin_gate_transform_identities(o):
    """With A_log = 0 and dt_bias = 0: exp(gate) = 1 - beta (softplus and
    sigmoid agree), sigmoid(x) + sigmoid(-x) = 1, softplus(x) - softplus(-x)
    = x, max(x, 0) <= softplus(x) <= max(x, 0) + ln 2, d softplus / dx =
    sigmoid (central difference), and finite values at |x| = 100."""
    Hv = G("value_heads")
    rng = np.random.default_rng(23)
    x = (8.0 * rng.standard_normal((6, Hv))).astype(np.float32)
    x[0, :4] = [100.0, -100.0, 0.0, 30.0]
    z = np.zeros(Hv, np.float32)
    rows = np.concatenate([x, -x])
    ba = np.concatenate([rows, rows], axis=1)                   # b = a = x
    beta, gate = o.gate_transform(ba, z, z)
    assert np.all(np.isfinite(beta)) and np.all(np.isfinite(gate)), "finite"
    n = len(x)
    bp, bm, gp, gm = (beta[:n].astype(np.float64), beta[n:].astype(np.float64),
                      gate[:n].astype(np.float64), gate[n:].astype(np.float64))
    assert np.all(np.abs(np.exp(gp) - (1.0 - bp)) <= 3e-7), "exp(gate) = 1 - beta"
    assert np.all(np.abs(bp + bm - 1.0) <= 3e-7), "sigmoid symmetry"
    xd = x.astype(np.float64)
    assert np.all(np.abs((gm - gp) - xd) <= _ulps(xd, 4) + 4e-7), "softplus(x) - softplus(-x) = x"
    sp = -gp
    assert np.all(sp >= np.maximum(xd, 0) - _ulps(xd, 2)) and \
        np.all(sp <= np.maximum(xd, 0) + np.log(2.0) + 4e-7), "softplus bounds"
    # derivative: (softplus(x + e) - softplus(x - e)) / 2e = sigmoid(x)
    eps = 2.0 ** -6
    xs = np.linspace(-4, 4, Hv).astype(np.float32)
    bad = np.stack([xs + eps, xs - eps, xs]).astype(np.float32)
    b2, g2 = o.gate_transform(np.concatenate([bad, bad], axis=1), z, z)
    slope = (-(g2[0].astype(np.float64)) + g2[1].astype(np.float64)) / (2 * eps)
    assert np.all(np.abs(slope - b2[2]) <= 5e-5), "d softplus/dx = sigmoid"


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


def run_all(path):
    """Run every pin against the oracle library at `path`; returns the list
    of (pin name, failure message) pairs."""
    import oracle
    o = oracle.Oracle(path)
    fails = []
    for p in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                p(o)
        except AssertionError as e:
            fails.append((p.__name__, str(e)))
    return fails


if __name__ == "__main__":
    import sys
    fails = run_all(sys.argv[1])
    for n, m in fails:
        print(f"FAIL {n}: {m}")
    sys.exit(1 if fails else 0)
