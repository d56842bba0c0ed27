"""Test-side helpers: the oracle run over independent sequences in host
threads (ctypes releases the GIL during the C call), and error reporting."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

THREADS = max(1, min(16, os.cpu_count() or 1))


def _split(n, parts):
    parts = max(1, min(parts, n))
    edges = np.linspace(0, n, parts + 1).astype(int)
    return [(edges[i], edges[i + 1]) for i in range(parts)]


def step_mt(o: oracle.Oracle, si: dict, M: np.ndarray, threads: int = THREADS) -> np.ndarray:
    """oracle step_M over the batch in host threads; M updated in place."""
    B = M.shape[0]
    out = np.empty((B, M.shape[1], M.shape[2]), np.float32)

    def run(rng):
        a, b = rng
        sl = {n: np.ascontiguousarray(x[a:b]) for n, x in si.items()}
        Mb = np.ascontiguousarray(M[a:b])
        out[a:b] = o.step_M(sl["q"], sl["k"], sl["v"], sl["beta"], sl["gate"], Mb)
        M[a:b] = Mb

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(run, _split(B, threads)))
    return out


def seq_mt(o: oracle.Oracle, si: dict, M: np.ndarray, threads: int = THREADS) -> np.ndarray:
    """oracle seq over the batch in host threads (one block of sequences per
    thread); M updated in place."""
    B, T = si["q"].shape[:2]
    out = np.empty((B, T, M.shape[1], M.shape[2]), np.float32)

    def run(rng):
        a, b = rng
        sl = {n: np.ascontiguousarray(x[a:b]) for n, x in si.items()}
        Mb = np.ascontiguousarray(M[a:b])
        out[a:b] = o.seq(sl["q"], sl["k"], sl["v"], sl["beta"], sl["gate"], Mb)
        M[a:b] = Mb

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(run, _split(B, threads)))
    return out


def max_err(got, want):
    """(max absolute error, max relative error); NaN or Inf anywhere gives
    inf, so that max() over several results cannot drop it."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    d = np.abs(got - want)
    rel = d / np.maximum(np.abs(want), 1e-30)
    a, r = float(d.max(initial=0.0)), float(rel.max(initial=0.0))
    return (a if np.isfinite(a) else np.inf), (r if np.isfinite(r) else np.inf)


def max_abs_err(got, want, chunk=1 << 24):
    """Max |got - want| over large float32 arrays, in chunks and in float32
    (the difference of two binary32 values within a factor 2 of each other is
    exact); NaN or Inf anywhere gives inf."""
    g = np.asarray(got).reshape(-1)
    w = np.asarray(want).reshape(-1)
    assert g.shape == w.shape
    worst = 0.0
    for i in range(0, g.size, chunk):
        m = float(np.max(np.abs(g[i:i + chunk] - w[i:i + chunk]), initial=0.0))
        if not np.isfinite(m):
            return np.inf
        worst = max(worst, m)
    return worst


def assert_close(name, got, want, atol):
    """Absolute-error gate (relative error is reported, not gated: it blows up
    near zero)."""
    assert got.shape == want.shape, f"{name}: shape {got.shape} != {want.shape}"
    a, r = max_err(got, want)
    print(f"    {name:>12s}: max abs {a:.3e}  max rel {r:.3e}  (tol abs {atol:g})", flush=True)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert a <= atol, f"{name}: max abs error {a:.3e} > {atol:g}"
    return a, r
