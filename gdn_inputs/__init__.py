"""Seeded synthetic inputs for the GDN state step and the layer tail.

This module is shared by the tests, the smoke check and the benchmark.  It
holds none of the method's arithmetic: it only draws numbers with the stated
distributions.  Both the oracle and the HIP path receive the same arrays.

Generator
---------
Every block of numbers comes from numpy's Philox4x32-10 counter-based
generator, keyed by ``(seed, stream, slot, index)``:

* ``stream`` names the tensor (``STREAMS`` below);
* ``slot`` is the layer (or, for repeated decode calls, the call number);
* ``index`` is the sequence ``b`` (or 0 for tensors shared by all sequences).

Sequence ``b``'s numbers therefore do not depend on the batch size or on the
other sequences, and any slice can be regenerated on its own (that is how a
state of many GiB is checked without holding a host copy of all of it).

Distributions (one token per call unless stated):

* state        N(0, 0.1^2), float32 (a float32 N(0,1) draw times 0.1f), or zero
* q, k         N(0,1) per head, then scaled to unit L2 norm in float64
               (input shaping: unit-norm keys/queries), rounded to float32
* v            N(0,1)
* beta         sigmoid(N(0,1)), computed in float64, rounded to float32
* gate         -softplus(N(0,1)) = -log1p(exp(n)) < 0, float64 -> float32
* x            N(0,1)  raw pre-conv channels (distribution not stated by the
               pages; standard normal is the reading taken)
* conv_w       N(0, 0.05^2)
* conv_state   N(0,1)
* z            N(0,1)
* norm_w       1 + N(0, 0.02^2)
* ba           N(0,1)  raw beta/alpha projection outputs, [B][2*Hv]
* a_log        log U(1, 16) per value head
* dt_bias      softplus^-1(dt), dt = exp(U(log 1e-3, log 1e-1)) per value head
               (the pages give no values for a_log and dt_bias; these ranges
               follow the published Mamba-2 initialisation; synthetic)
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

STREAMS = {
    "state": 1, "q": 2, "k": 3, "v": 4, "beta": 5, "gate": 6,
    "x": 7, "z": 8, "conv_w": 9, "conv_state": 10, "norm_w": 11,
    "ba": 12, "a_log": 13, "dt_bias": 14,
}

# The page geometry (value heads, key heads, head dim) and the tail geometry.
HV, HK, D = 32, 16, 128
CONV_K = 4
NORM_GROUP = 128
NORM_EPS = 1e-6

# The workloads, by what they are; each has its own seed.
WORKLOADS = {
    # gdn_step, one sequence, one token
    "step_b1": dict(B=1, seed=1000),
    # gdn_step, 64 sequences, 100 calls with fresh inputs (slot = call)
    "step_b64_x100": dict(B=64, calls=100, seed=1001),
    # gdn_step, 256 sequences x 36 recurrent layers (slot = layer), 18 GiB of state
    "step_b256_x36": dict(B=256, layers=36, seed=1002),
    # gdn_seq, 8 sequences x 4096 tokens from a zero state
    "seq_b8_t4096": dict(B=8, T=4096, seed=1003),
    # gdn_layer_tail, 32 sequences, 8192 channels
    "tail_b32": dict(B=32, seed=1004),
    # gdn_seq with many heads and a short sequence: 256 sequences x 64 tokens
    # from seeded states (a secondary line, not one of the five configs)
    "seq_b256_t64": dict(B=256, T=64, seed=1005),
    # gdn_seq with more heads than compute units and a longer sequence: 40
    # sequences x 1024 tokens from seeded states (a secondary line)
    "seq_b40_t1024": dict(B=40, T=1024, seed=1006),
}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _gen(seed: int, stream: str, slot: int, index: int) -> np.random.Generator:
    s = STREAMS[stream]
    assert 0 <= slot < (1 << 24) and 0 <= index < (1 << 24)
    key = np.array([seed, (s << 48) | (slot << 24) | index], dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key))


def normal64(seed, stream, slot, index, n) -> np.ndarray:
    """n standard normals (float64) of one keyed block."""
    return _gen(seed, stream, slot, index).standard_normal(n, dtype=np.float64)


def normal32_into(out: np.ndarray, seed, stream, slot, index, scale=None) -> None:
    """Fill a contiguous float32 array with one keyed block of N(0,1)*scale."""
    flat = out.reshape(-1)
    _gen(seed, stream, slot, index).standard_normal(out=flat, dtype=np.float32)
    if scale is not None:
        np.multiply(flat, np.float32(scale), out=flat)


def _unit_heads(n: np.ndarray, heads: int, d: int) -> np.ndarray:
    h = n.reshape(heads, d)
    return (h / np.sqrt((h * h).sum(axis=1, keepdims=True))).astype(np.float32)


def _sigmoid64(n):
    return 1.0 / (1.0 + np.exp(-n))


def _neg_softplus64(n):
    return -np.log1p(np.exp(n))


# ---------------------------------------------------------------- step inputs
def step_inputs(seed, slot, B, Hv=HV, Hk=HK, d=D, b0=0, T=None):
    """Per-token inputs for sequences b0 .. b0+B-1.

    T=None gives the single-token layout (q,k [B][Hk][d], v [B][Hv][d],
    beta/gate [B][Hv]); an integer T gives [B][T][...]."""
    tt = 1 if T is None else T
    q = np.empty((B, tt, Hk, d), np.float32)
    k = np.empty_like(q)
    v = np.empty((B, tt, Hv, d), np.float32)
    beta = np.empty((B, tt, Hv), np.float32)
    gate = np.empty((B, tt, Hv), np.float32)

    def one(i):
        b = b0 + i
        q[i] = _unit_heads(normal64(seed, "q", slot, b, tt * Hk * d), tt * Hk, d).reshape(tt, Hk, d)
        k[i] = _unit_heads(normal64(seed, "k", slot, b, tt * Hk * d), tt * Hk, d).reshape(tt, Hk, d)
        normal32_into(v[i], seed, "v", slot, b)
        beta[i] = _sigmoid64(normal64(seed, "beta", slot, b, tt * Hv)).astype(np.float32).reshape(tt, Hv)
        gate[i] = _neg_softplus64(normal64(seed, "gate", slot, b, tt * Hv)).astype(np.float32).reshape(tt, Hv)

    _parallel(one, B)
    if T is None:
        q, k, v, beta, gate = (a[:, 0] for a in (q, k, v, beta, gate))
        q, k, v, beta, gate = (np.ascontiguousarray(a) for a in (q, k, v, beta, gate))
    return dict(q=q, k=k, v=v, beta=beta, gate=gate)


def state_into(out: np.ndarray, seed, slot, b0=0, scale=0.1) -> None:
    """Fill out[B][Hv][d][d] (float32, contiguous) with sequence b0+i's state."""
    B = out.shape[0]
    _parallel(lambda i: normal32_into(out[i], seed, "state", slot, b0 + i, scale), B)


def state(seed, slot, B, Hv=HV, d=D, b0=0, scale=0.1) -> np.ndarray:
    out = np.empty((B, Hv, d, d), np.float32)
    state_into(out, seed, slot, b0, scale)
    return out


# ---------------------------------------------------------------- tail inputs
def tail_inputs(seed, B, Hv=HV, Hk=HK, d=D, K=CONV_K, group=NORM_GROUP, b0=0, slot=0):
    """Inputs of the recurrent-branch tail for sequences b0 .. b0+B-1."""
    C = 2 * Hk * d + Hv * d
    x = np.empty((B, C), np.float32)
    cs = np.empty((B, K - 1, C), np.float32)
    z = np.empty((B, Hv * d), np.float32)

    def one(i):
        b = b0 + i
        normal32_into(x[i], seed, "x", slot, b)
        normal32_into(cs[i], seed, "conv_state", slot, b)
        normal32_into(z[i], seed, "z", slot, b)

    _parallel(one, B)
    conv_w = np.empty((C, K), np.float32)
    normal32_into(conv_w, seed, "conv_w", slot, 0, 0.05)
    norm_w = (1.0 + 0.02 * normal64(seed, "norm_w", slot, 0, group)).astype(np.float32)
    si = step_inputs(seed, slot, B, Hv, Hk, d, b0)
    return dict(x=x, conv_w=conv_w, conv_state=cs, z=z, norm_w=norm_w,
                beta=si["beta"], gate=si["gate"])


# ---------------------------------------------------------------- gate inputs
def gate_inputs(seed, B, Hv=HV, b0=0, slot=0):
    """Raw inputs of the beta/alpha parameter transforms for sequences
    b0 .. b0+B-1: ba [B][2*Hv] and the per-head a_log, dt_bias [Hv]."""
    ba = np.empty((B, 2 * Hv), np.float32)
    _parallel(lambda i: normal32_into(ba[i], seed, "ba", slot, b0 + i), B)
    u = _gen(seed, "a_log", slot, 0).uniform(1.0, 16.0, Hv)
    a_log = np.log(u).astype(np.float32)
    dt = np.exp(_gen(seed, "dt_bias", slot, 0).uniform(np.log(1e-3), np.log(1e-1), Hv))
    dt_bias = (dt + np.log(-np.expm1(-dt))).astype(np.float32)
    return dict(ba=ba, a_log=a_log, dt_bias=dt_bias)


def _parallel(fn, n):
    if n <= 1:
        for i in range(n):
            fn(i)
        return
    with ThreadPoolExecutor(min(_threads(), n)) as ex:
        list(ex.map(fn, range(n)))
