"""Test-side helpers: the oracle run over independent sequences in host
threads (ctypes releases the GIL during the C call), error reporting, and the
parity records every check appends to (written out as JSON lines at the end
of a GPU session, one record per compared quantity: max abs, max rel, the
tolerance and whether it passed, with the workload named where the test is one)."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

THREADS = max(1, min(16, os.cpu_count() or 1))

# The GPU path computes in binary32 with FMA and tree reductions, the oracle
# in binary32 with sequential unfused sums; against the binary64 shadow both
# carry rounding error of the same order.  A GPU error more than this many
# times the f32 oracle's own error (plus a floor of 1e-12 for exact cases)
# points at a reduction-order or precision regression far below the
# absolute tolerances.
F64_FACTOR = 4.0

RECORDS: list = []
WORKLOAD = {"name": None}


def _test_id():
    return os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]


def record(**kw):
    kw.setdefault("test", _test_id())
    if WORKLOAD["name"]:
        kw.setdefault("workload", WORKLOAD["name"])
    RECORDS.append(kw)


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


def step_f64_mt(o: oracle.Oracle, si: dict, M64: np.ndarray, threads: int = THREADS):
    """The binary64 shadow step over the batch in host threads; M64 updated
    in place."""
    B = M64.shape[0]
    out = np.empty((B, M64.shape[1], M64.shape[2]), np.float64)

    def run(rng):
        a, b = rng
        sl = {n: np.ascontiguousarray(x[a:b]) for n, x in si.items()}
        Mb = np.ascontiguousarray(M64[a:b])
        out[a:b] = o.step_f64(sl["q"], sl["k"], sl["v"], sl["beta"], sl["gate"], Mb)
        M64[a:b] = Mb

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(run, _split(B, threads)))
    return out


def seq_f64_mt(o: oracle.Oracle, si: dict, M64: np.ndarray, threads: int = THREADS):
    """The binary64 shadow sequence over the batch in host threads; M64
    updated in place."""
    B, T = si["q"].shape[:2]
    out = np.empty((B, T, M64.shape[1], M64.shape[2]), np.float64)

    def run(rng):
        a, b = rng
        sl = {n: np.ascontiguousarray(x[a:b]) for n, x in si.items()}
        Mb = np.ascontiguousarray(M64[a:b])
        out[a:b] = o.seq_f64(sl["q"], sl["k"], sl["v"], sl["beta"], sl["gate"], Mb)
        M64[a:b] = Mb

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
    ok = bool(np.all(np.isfinite(got))) and a <= atol
    record(name=name, max_abs=a, max_rel=r, tol_abs=atol, passed=ok)
    print(f"    {name:>12s}: max abs {a:.3e}  max rel {r:.3e}  (tol abs {atol:g})", flush=True)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert a <= atol, f"{name}: max abs error {a:.3e} > {atol:g}"
    return a, r


def assert_abs_bound(name, worst, atol):
    """The same gate for an error already reduced to its maximum (large
    arrays compared chunk by chunk)."""
    ok = bool(np.isfinite(worst)) and worst <= atol
    record(name=name, max_abs=float(worst), tol_abs=atol, passed=ok)
    print(f"    {name:>12s}: max abs {worst:.3e}  (tol abs {atol:g})", flush=True)
    assert ok, f"{name}: max abs error {worst:.3e} > {atol:g}"


def assert_vs_f64(name, got, oracle32, ref64, factor=F64_FACTOR):
    """The binary64 yardstick: |GPU - f64| <= factor x |f32 oracle - f64|
    (+1e-12), maxima over all elements."""
    e_gpu = max_abs_err64(got, ref64)
    e_orc = max_abs_err64(oracle32, ref64)
    bound = factor * e_orc + 1e-12
    ok = bool(np.isfinite(e_gpu)) and e_gpu <= bound
    record(name=name + " vs f64", gpu_vs_f64=e_gpu, oracle_vs_f64=e_orc,
           ratio=e_gpu / max(e_orc, 1e-300), factor=factor, passed=ok)
    print(f"    {name:>12s}: vs f64 gpu {e_gpu:.3e}  oracle {e_orc:.3e}  "
          f"ratio {e_gpu / max(e_orc, 1e-300):.2f} (gate {factor:g}x)", flush=True)
    assert ok, f"{name}: GPU error vs f64 {e_gpu:.3e} > {factor:g} x oracle's {e_orc:.3e}"


def assert_f64_ratio(name, e_gpu, e_orc, factor=F64_FACTOR):
    """assert_vs_f64 for errors already reduced to their maxima."""
    bound = factor * e_orc + 1e-12
    ok = bool(np.isfinite(e_gpu)) and e_gpu <= bound
    record(name=name + " vs f64", gpu_vs_f64=float(e_gpu), oracle_vs_f64=float(e_orc),
           ratio=e_gpu / max(e_orc, 1e-300), factor=factor, passed=ok)
    print(f"    {name:>12s}: vs f64 gpu {e_gpu:.3e}  oracle {e_orc:.3e}  "
          f"ratio {e_gpu / max(e_orc, 1e-300):.2f} (gate {factor:g}x)", flush=True)
    assert ok, f"{name}: GPU error vs f64 {e_gpu:.3e} > {factor:g} x oracle's {e_orc:.3e}"


def max_abs_err64(got, ref64, chunk=1 << 22):
    """Max |got - ref64| with got promoted to float64, in chunks; NaN or Inf
    gives inf."""
    g = np.asarray(got).reshape(-1)
    w = np.asarray(ref64).reshape(-1)
    assert g.shape == w.shape
    worst = 0.0
    for i in range(0, g.size, chunk):
        m = float(np.max(np.abs(g[i:i + chunk].astype(np.float64) - w[i:i + chunk]), initial=0.0))
        if not np.isfinite(m):
            return np.inf
        worst = max(worst, m)
    return worst
