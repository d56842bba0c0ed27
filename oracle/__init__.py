"""ctypes view of the plain C99 oracle (``oracle/gdn_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The product package
never imports it, and the oracle shares no source with the HIP path.

Every wrapper takes and returns numpy arrays in the layouts documented in
``gdn_oracle.h``; state arrays are updated in place, exactly as the C calls do.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "gdn_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

# Plain, IEEE-faithful build: no fast-math, no FMA contraction.
CFLAGS = ["-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
          "-shared", "-Wall", "-Wextra"]


def build(source: str = SOURCE, output: str = LIBRARY, extra=()) -> str:
    """Compile the oracle with gcc into ``output``; returns the path."""
    cmd = ["gcc", *CFLAGS, *extra, source, "-o", output, "-lm"]
    subprocess.run(cmd, check=True, cwd=HERE)
    return output


_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32 = ctypes.c_int32


def _p32(a):
    if a is None:
        return None
    assert a.dtype == np.float32 and a.flags.c_contiguous, "need contiguous float32"
    return a.ctypes.data_as(_f32p)


def _p64(a):
    assert a.dtype == np.float64 and a.flags.c_contiguous, "need contiguous float64"
    return a.ctypes.data_as(_f64p)


class Oracle:
    """One loaded copy of the oracle library (the default one, or a variant
    compiled from a modified source for the planted-mistake tests)."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            raise FileNotFoundError(f"{path} not built (run __graft_entry__.build())")
        self.path = path
        L = ctypes.CDLL(path)
        dims5 = [_i32] * 5
        vec5 = [_f32p] * 5
        L.oracle_gdn_step_M.argtypes = [_i32, *dims5[1:], *vec5, _f32p, _f32p, _f32p]
        L.oracle_gdn_step_S.argtypes = L.oracle_gdn_step_M.argtypes
        L.oracle_gdn_step_f64.argtypes = [_i32, *dims5[1:], *vec5, _f64p, _f64p]
        L.oracle_gdn_seq.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, *vec5, _f32p, _f32p]
        L.oracle_gdn_seq_f64.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, *vec5, _f64p, _f64p]
        L.oracle_gdn_pair.argtypes = [_i32, *dims5[1:], *vec5, _f32p, _f32p, _f32p]
        L.oracle_conv_silu.argtypes = [_i32, _i32, _i32, _f32p, _f32p, _f32p, _f32p]
        L.oracle_l2norm_rows.argtypes = [_i32, _i32, _f32p]
        L.oracle_gated_rmsnorm.argtypes = [_i32, _i32, _i32, ctypes.c_float,
                                           _f32p, _f32p, _f32p, _f32p]
        L.oracle_layer_tail.argtypes = [_i32] * 7 + [ctypes.c_float] + [_f32p] * 11
        L.oracle_layer_tail_pair.argtypes = [_i32] * 7 + [ctypes.c_float] + [_f32p] * 11
        L.oracle_gate_transform.argtypes = [_i32, _i32] + [_f32p] * 5
        for name in ("oracle_gdn_step_M", "oracle_gdn_step_S", "oracle_gdn_step_f64",
                     "oracle_gdn_seq", "oracle_gdn_seq_f64", "oracle_gdn_pair", "oracle_conv_silu",
                     "oracle_l2norm_rows", "oracle_gated_rmsnorm", "oracle_layer_tail",
                     "oracle_layer_tail_pair", "oracle_gate_transform"):
            getattr(L, name).restype = None
        self.lib = L

    # -- the state step -------------------------------------------------
    @staticmethod
    def _dims(q, v, M):
        B, Hk, dk = q.shape
        _, Hv, dv = v.shape
        assert M.shape[0] == B and M.shape[1] == Hv, "state batch/head mismatch"
        return B, Hv, Hk, dk, dv

    def step_M(self, q, k, v, beta, gate, M, want_delta=False):
        """[dev15c] one token on the transposed state; M updated in place.
        Returns out (and delta when asked)."""
        B, Hv, Hk, dk, dv = self._dims(q, v, M)
        assert M.shape == (B, Hv, dv, dk)
        out = np.empty((B, Hv, dv), np.float32)
        delta = np.empty((B, Hv, dv), np.float32) if want_delta else None
        self.lib.oracle_gdn_step_M(B, Hv, Hk, dk, dv, _p32(q), _p32(k), _p32(v),
                                   _p32(beta), _p32(gate), _p32(M), _p32(out),
                                   _p32(delta))
        return (out, delta) if want_delta else out

    def step_S(self, q, k, v, beta, gate, S, want_delta=False):
        """The same step on the non-transposed state S [B][Hv][dk][dv]."""
        B, Hk, dk = q.shape
        _, Hv, dv = v.shape
        assert S.shape == (B, Hv, dk, dv)
        out = np.empty((B, Hv, dv), np.float32)
        delta = np.empty((B, Hv, dv), np.float32) if want_delta else None
        self.lib.oracle_gdn_step_S(B, Hv, Hk, dk, dv, _p32(q), _p32(k), _p32(v),
                                   _p32(beta), _p32(gate), _p32(S), _p32(out),
                                   _p32(delta))
        return (out, delta) if want_delta else out

    def step_f64(self, q, k, v, beta, gate, M64):
        """Binary64 shadow; M64 (float64) updated in place, returns float64 out."""
        B, Hv, Hk, dk, dv = self._dims(q, v, M64)
        assert M64.shape == (B, Hv, dv, dk)
        out = np.empty((B, Hv, dv), np.float64)
        self.lib.oracle_gdn_step_f64(B, Hv, Hk, dk, dv, _p32(q), _p32(k), _p32(v),
                                     _p32(beta), _p32(gate), _p64(M64), _p64(out))
        return out

    def seq(self, q, k, v, beta, gate, M):
        """[linear_core] T positions in order; q,k [B][T][Hk][dk],
        v [B][T][Hv][dv], beta/gate [B][T][Hv]; M updated in place."""
        B, T, Hk, dk = q.shape
        _, _, Hv, dv = v.shape
        assert M.shape == (B, Hv, dv, dk)
        out = np.empty((B, T, Hv, dv), np.float32)
        self.lib.oracle_gdn_seq(B, T, Hv, Hk, dk, dv, _p32(q), _p32(k), _p32(v),
                                _p32(beta), _p32(gate), _p32(M), _p32(out))
        return out

    def seq_f64(self, q, k, v, beta, gate, M64):
        """Binary64 shadow of seq: M64 (float64) updated in place; returns
        float64 out [B][T][Hv][dv]."""
        B, T, Hk, dk = q.shape
        _, _, Hv, dv = v.shape
        assert M64.shape == (B, Hv, dv, dk)
        out = np.empty((B, T, Hv, dv), np.float64)
        self.lib.oracle_gdn_seq_f64(B, T, Hv, Hk, dk, dv, _p32(q), _p32(k), _p32(v),
                                    _p32(beta), _p32(gate), _p64(M64), _p64(out))
        return out

    def pair(self, q, k, v, beta, gate, M):
        """[linear_core] gdn_pair: q,k [B][2][Hk][dk], v [B][2][Hv][dv],
        beta/gate [B][2][Hv].  M is committed in place (position 1); returns
        (out [B][2][Hv][dv], M_next) with M_next the tentative state."""
        B, two, Hk, dk = q.shape
        assert two == 2
        _, _, Hv, dv = v.shape
        assert M.shape == (B, Hv, dv, dk)
        out = np.empty((B, 2, Hv, dv), np.float32)
        Mn = np.empty_like(M)
        self.lib.oracle_gdn_pair(B, Hv, Hk, dk, dv, _p32(q), _p32(k), _p32(v),
                                 _p32(beta), _p32(gate), _p32(M), _p32(Mn), _p32(out))
        return out, Mn

    # -- tail stages ------------------------------------------------------
    def conv_silu(self, x, conv_w, conv_state):
        B, C = x.shape
        K = conv_w.shape[1]
        assert conv_w.shape == (C, K) and conv_state.shape == (B, K - 1, C)
        act = np.empty((B, C), np.float32)
        self.lib.oracle_conv_silu(B, C, K, _p32(x), _p32(conv_w), _p32(conv_state), _p32(act))
        return act

    def l2norm_rows(self, u):
        """Normalises the last axis of a copy of u; returns the copy."""
        u = np.ascontiguousarray(u, dtype=np.float32).copy()
        d = u.shape[-1]
        self.lib.oracle_l2norm_rows(u.size // d, d, _p32(u))
        return u

    def gated_rmsnorm(self, o, z, w, group, eps=1e-6):
        rows = o.shape[0]
        n = o.size // rows
        y = np.empty_like(o, dtype=np.float32)
        self.lib.oracle_gated_rmsnorm(rows, n, group, eps, _p32(o), _p32(z), _p32(w), _p32(y))
        return y

    def layer_tail(self, x, conv_w, conv_state, beta, gate, M, z, norm_w,
                   Hk, dk, group=128, eps=1e-6):
        """Whole tail; conv_state and M updated in place.  Returns
        (y, qkv, core) with qkv the normalized [Q|K|V] and core the step output."""
        B, C = x.shape
        K = conv_w.shape[1]
        _, Hv, dv, _ = M.shape
        assert C == 2 * Hk * dk + Hv * dv
        y = np.empty((B, Hv * dv), np.float32)
        qkv = np.empty((B, C), np.float32)
        core = np.empty((B, Hv, dv), np.float32)
        self.lib.oracle_layer_tail(B, Hv, Hk, dk, dv, K, group, eps,
                                   _p32(x), _p32(conv_w), _p32(conv_state),
                                   _p32(beta), _p32(gate), _p32(M), _p32(z),
                                   _p32(norm_w), _p32(y), _p32(qkv), _p32(core))
        return y, qkv, core

    def layer_tail_pair(self, x, conv_w, conv_state, beta, gate, M, z, norm_w,
                        Hk, dk, group=128, eps=1e-6):
        """[linear_core] gdn_pair over the whole tail.  x [B][2][C],
        beta/gate [B][2][Hv], z [B][2][Hv*dv].  conv_state and M are
        committed in place (position 1); returns (y [B][2][Hv*dv],
        conv_state_next, M_next), the tentative ring and state after
        position 2."""
        B, two, C = x.shape
        assert two == 2
        K = conv_w.shape[1]
        _, Hv, dv, _ = M.shape
        assert C == 2 * Hk * dk + Hv * dv
        assert conv_state.shape == (B, K - 1, C)
        y = np.empty((B, 2, Hv * dv), np.float32)
        csn = np.empty_like(conv_state)
        Mn = np.empty_like(M)
        self.lib.oracle_layer_tail_pair(B, Hv, Hk, dk, dv, K, group, eps,
                                        _p32(x), _p32(conv_w), _p32(conv_state), _p32(csn),
                                        _p32(beta), _p32(gate), _p32(M), _p32(Mn),
                                        _p32(z), _p32(norm_w), _p32(y))
        return y, csn, Mn

    # -- the beta/alpha parameter transforms ------------------------------
    def gate_transform(self, ba, a_log, dt_bias):
        """beta, gate [B][Hv] from the raw projection ba [B][2*Hv] and the
        per-head a_log, dt_bias [Hv]."""
        ba = np.ascontiguousarray(ba, dtype=np.float32)
        a_log = np.ascontiguousarray(a_log, dtype=np.float32)
        dt_bias = np.ascontiguousarray(dt_bias, dtype=np.float32)
        B, two_hv = ba.shape
        Hv = two_hv // 2
        assert two_hv == 2 * Hv and a_log.shape == (Hv,) and dt_bias.shape == (Hv,)
        beta = np.empty((B, Hv), np.float32)
        gate = np.empty((B, Hv), np.float32)
        self.lib.oracle_gate_transform(B, Hv, _p32(ba), _p32(a_log), _p32(dt_bias),
                                       _p32(beta), _p32(gate))
        return beta, gate


_default = None


def get() -> Oracle:
    """The default oracle, loaded once."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
