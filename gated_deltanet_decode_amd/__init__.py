"""Python binding of libgdn.so (the C ABI in include/gdn.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch provides device memory and streams.  The names mirror the
C entry points:

    step(q, k, v, beta, gate, state, out)        -> gdn_step
    step(..., cached=True)                       -> gdn_step_ex(GDN_STATE_CACHED)
    bind_step(q, k, v, beta, gate, state, out)   -> a prepared gdn_step call
    seq(q, k, v, beta, gate, state, out)         -> gdn_seq
    seq(..., exact=True)                         -> gdn_seq_exact
    pair(q, k, v, beta, gate, state, state_next, out) -> gdn_pair
    layer_tail(x, conv_w, conv_state, beta, gate, state, z, norm_w, y, ...)
                                                 -> gdn_layer_tail
    layer_tail_workspace_bytes(B)                -> gdn_layer_tail_workspace_bytes
    layer_tail_noalloc(x, conv_w, conv_state, beta, gate, state, z, norm_w, y, ...)
                                                 -> gdn_layer_tail_noalloc
    layer_tail_pair(x, conv_w, conv_state, conv_state_next, beta, gate, state,
                    state_next, z, norm_w, y)    -> gdn_layer_tail_pair
    gate_transform(ba, a_log, dt_bias, beta, gate) -> gdn_gate_transform
    layer_tail_ba(x, conv_w, conv_state, ba, a_log, dt_bias, state, z, norm_w, y, ...)
                                                 -> gdn_layer_tail_ba
    layer_tail_ba_workspace_bytes(B)             -> gdn_layer_tail_ba_workspace_bytes
    last_error(), version()

If the library has not been built, importing this package raises: there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os

from ._build import LIBRARY

__all__ = ["GdnError", "Dims", "TailParams", "GateInputs", "lib", "step", "bind_step", "seq",
           "pair",
           "layer_tail", "layer_tail_workspace_bytes", "layer_tail_noalloc", "layer_tail_pair",
           "gate_transform",
           "layer_tail_ba",
           "layer_tail_ba_workspace_bytes", "last_error", "version", "PAGE_DIMS",
           "PAGE_TAIL", "ERRORS"]

if not os.path.exists(LIBRARY):
    raise ImportError(f"{LIBRARY} is not built; run __graft_entry__.build() "
                      "(hipcc --offload-arch=gfx950) first")


class Dims(ctypes.Structure):
    """gdn_dims"""
    _fields_ = [("n_v_heads", ctypes.c_int32), ("n_k_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32)]


class TailParams(ctypes.Structure):
    """gdn_tail_params"""
    _fields_ = [("conv_kernel", ctypes.c_int32), ("norm_group", ctypes.c_int32),
                ("norm_eps", ctypes.c_float), ("force_unfused", ctypes.c_int32)]


class GateInputs(ctypes.Structure):
    """gdn_gate_inputs (device pointers)"""
    _fields_ = [("ba", ctypes.c_void_p), ("a_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p)]


PAGE_DIMS = Dims(32, 16, 128, 128)
PAGE_TAIL = TailParams(4, 128, 1e-6, 0)

ERRORS = {0: "GDN_OK", -1: "GDN_ERR_NULL", -2: "GDN_ERR_SHAPE", -3: "GDN_ERR_ALIGN",
          -4: "GDN_ERR_ALIAS", -5: "GDN_ERR_WORKSPACE", -6: "GDN_ERR_HIP"}

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_DP = ctypes.POINTER(Dims)
_TP = ctypes.POINTER(TailParams)
_GP = ctypes.POINTER(GateInputs)

lib = ctypes.CDLL(LIBRARY)
lib.gdn_version.restype = ctypes.c_int
lib.gdn_version.argtypes = []
lib.gdn_last_error.restype = ctypes.c_char_p
lib.gdn_last_error.argtypes = []
lib.gdn_step.restype = ctypes.c_int
lib.gdn_step.argtypes = [_DP, _i32] + [_vp] * 7 + [_vp]
lib.gdn_step_ex.restype = ctypes.c_int
lib.gdn_step_ex.argtypes = [_DP, _i32] + [_vp] * 7 + [ctypes.c_uint32, _vp]
STATE_CACHED = 1
lib.gdn_seq.restype = ctypes.c_int
lib.gdn_seq.argtypes = [_DP, _i32, _i32] + [_vp] * 7 + [_vp]
lib.gdn_seq_exact.restype = ctypes.c_int
lib.gdn_seq_exact.argtypes = [_DP, _i32, _i32] + [_vp] * 7 + [_vp]
lib.gdn_pair.restype = ctypes.c_int
lib.gdn_pair.argtypes = [_DP, _i32] + [_vp] * 8 + [_vp]
lib.gdn_layer_tail.restype = ctypes.c_int
lib.gdn_layer_tail.argtypes = [_DP, _TP, _i32] + [_vp] * 11 + [_vp, ctypes.c_size_t, _vp]
lib.gdn_layer_tail_pair.restype = ctypes.c_int
lib.gdn_layer_tail_pair.argtypes = [_DP, _TP, _i32] + [_vp] * 11 + [_vp]
lib.gdn_layer_tail_noalloc.restype = ctypes.c_int
lib.gdn_layer_tail_noalloc.argtypes = [_DP, _TP, _i32] + [_vp] * 11 + [_vp]
lib.gdn_layer_tail_workspace_bytes.restype = ctypes.c_size_t
lib.gdn_layer_tail_workspace_bytes.argtypes = [_DP, _i32]
lib.gdn_gate_transform.restype = ctypes.c_int
lib.gdn_gate_transform.argtypes = [_DP, _i32, _GP, _vp, _vp, _vp]
lib.gdn_layer_tail_ba.restype = ctypes.c_int
lib.gdn_layer_tail_ba.argtypes = [_DP, _TP, _i32] + [_vp] * 3 + [_GP] + [_vp] * 6 + \
    [_vp, ctypes.c_size_t, _vp]
lib.gdn_layer_tail_ba_workspace_bytes.restype = ctypes.c_size_t
lib.gdn_layer_tail_ba_workspace_bytes.argtypes = [_DP, _i32]


class GdnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERRORS.get(code, code)}: {message}")
        self.code = code


def version() -> int:
    return lib.gdn_version()


def last_error() -> str:
    return lib.gdn_last_error().decode()


def _check(rc: int) -> None:
    if rc != 0:
        raise GdnError(rc, last_error())


try:
    import torch as _torch
    _F32 = _torch.float32
except ImportError:       # the checks below then raise the import error
    _F32 = None


def _ptr(t, name, shape=None, optional=False):
    """Device address of a contiguous float32 GPU tensor of the given shape.
    The common case is tested in one expression; anything else goes through
    the checks one by one, which name what is wrong."""
    try:
        if (t.dtype is _F32 and t.is_cuda and t.is_contiguous()
                and (shape is None or t.shape == shape)):
            return t.data_ptr()
    except AttributeError:
        pass
    return _ptr_checked(t, name, shape, optional)


def _ptr_checked(t, name, shape, optional):
    import torch
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dims_of(q, v):
    Hk, dk = q.shape[-2], q.shape[-1]
    Hv, dv = v.shape[-2], v.shape[-1]
    return Dims(Hv, Hk, dk, dv)


def step(q, k, v, beta, gate, state, out, stream=None, cached=False) -> None:
    """gdn_step: q,k [B][Hk][dk], v [B][Hv][dv], beta/gate [B][Hv],
    state [B][Hv][dv][dk] (updated in place), out [B][Hv][dv].  cached=True
    calls gdn_step_ex with GDN_STATE_CACHED (states resident in the Infinity
    Cache across calls)."""
    B = q.shape[0]
    d = _dims_of(q, v)
    args = (ctypes.byref(d), B,
            _ptr(q, "q", (B, d.n_k_heads, d.d_k)), _ptr(k, "k", (B, d.n_k_heads, d.d_k)),
            _ptr(v, "v", (B, d.n_v_heads, d.d_v)),
            _ptr(beta, "beta", (B, d.n_v_heads)), _ptr(gate, "gate", (B, d.n_v_heads)),
            _ptr(state, "state", (B, d.n_v_heads, d.d_v, d.d_k)),
            _ptr(out, "out", (B, d.n_v_heads, d.d_v)))
    if cached:
        _check(lib.gdn_step_ex(*args, STATE_CACHED, _stream(stream)))
    else:
        _check(lib.gdn_step(*args, _stream(stream)))


def bind_step(q, k, v, beta, gate, state, out, stream=None, cached=False):
    """A prepared gdn_step call for latency-bound decode loops that step the
    same buffers again and again (new token values written into q, k, v,
    beta and gate between calls): the tensors are checked once here and the
    returned function only re-issues the C call with the converted
    arguments.  The tensors must stay alive and in place while it is used.
    The library still validates every call."""
    B = q.shape[0]
    d = _dims_of(q, v)
    ptrs = (_ptr(q, "q", (B, d.n_k_heads, d.d_k)), _ptr(k, "k", (B, d.n_k_heads, d.d_k)),
            _ptr(v, "v", (B, d.n_v_heads, d.d_v)),
            _ptr(beta, "beta", (B, d.n_v_heads)), _ptr(gate, "gate", (B, d.n_v_heads)),
            _ptr(state, "state", (B, d.n_v_heads, d.d_v, d.d_k)),
            _ptr(out, "out", (B, d.n_v_heads, d.d_v)))
    args = [ctypes.byref(d), ctypes.c_int32(B), *(ctypes.c_void_p(p) for p in ptrs)]
    if cached:
        fn = lib.gdn_step_ex
        args.append(ctypes.c_uint32(STATE_CACHED))
    else:
        fn = lib.gdn_step
    args.append(ctypes.c_void_p(_stream(stream)))
    args = tuple(args)
    keep = (d, q, k, v, beta, gate, state, out)

    def call() -> None:
        rc = fn(*args)
        if rc != 0:
            raise GdnError(rc, last_error())
    call.tensors = keep
    return call


def seq(q, k, v, beta, gate, state, out, stream=None, exact=False) -> None:
    """gdn_seq (gdn_seq_exact with exact=True): q,k [B][T][Hk][dk],
    v [B][T][Hv][dv], beta/gate [B][T][Hv], state [B][Hv][dv][dk] (in/out),
    out [B][T][Hv][dv]."""
    B, T = q.shape[0], q.shape[1]
    d = _dims_of(q, v)
    _check((lib.gdn_seq_exact if exact else lib.gdn_seq)(
        ctypes.byref(d), B, T,
        _ptr(q, "q", (B, T, d.n_k_heads, d.d_k)), _ptr(k, "k", (B, T, d.n_k_heads, d.d_k)),
        _ptr(v, "v", (B, T, d.n_v_heads, d.d_v)),
        _ptr(beta, "beta", (B, T, d.n_v_heads)), _ptr(gate, "gate", (B, T, d.n_v_heads)),
        _ptr(state, "state", (B, d.n_v_heads, d.d_v, d.d_k)),
        _ptr(out, "out", (B, T, d.n_v_heads, d.d_v)), _stream(stream)))


def pair(q, k, v, beta, gate, state, state_next, out, stream=None) -> None:
    """gdn_pair: q,k [B][2][Hk][dk], v [B][2][Hv][dv], beta/gate [B][2][Hv];
    state [B][Hv][dv][dk] is committed with position 1 in place;
    state_next (same shape) receives the tentative state after position 2;
    out [B][2][Hv][dv]."""
    B = q.shape[0]
    d = _dims_of(q, v)
    _check(lib.gdn_pair(
        ctypes.byref(d), B,
        _ptr(q, "q", (B, 2, d.n_k_heads, d.d_k)), _ptr(k, "k", (B, 2, d.n_k_heads, d.d_k)),
        _ptr(v, "v", (B, 2, d.n_v_heads, d.d_v)),
        _ptr(beta, "beta", (B, 2, d.n_v_heads)), _ptr(gate, "gate", (B, 2, d.n_v_heads)),
        _ptr(state, "state", (B, d.n_v_heads, d.d_v, d.d_k)),
        _ptr(state_next, "state_next", (B, d.n_v_heads, d.d_v, d.d_k)),
        _ptr(out, "out", (B, 2, d.n_v_heads, d.d_v)), _stream(stream)))


def layer_tail_workspace_bytes(B: int, dims: Dims = PAGE_DIMS) -> int:
    return int(lib.gdn_layer_tail_workspace_bytes(ctypes.byref(dims), B))


def _workspace(workspace):
    import torch
    if workspace is None:
        return None, 0
    if not (isinstance(workspace, torch.Tensor) and workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def layer_tail(x, conv_w, conv_state, beta, gate, state, z, norm_w, y,
               dbg_qkv=None, dbg_core=None, workspace=None,
               dims: Dims = PAGE_DIMS, params: TailParams = PAGE_TAIL, stream=None) -> None:
    """gdn_layer_tail.  workspace: a GPU tensor of at least
    layer_tail_workspace_bytes(B) bytes (any dtype), or None when both dbg
    buffers are given."""
    B, C = x.shape
    K = params.conv_kernel
    nv = dims.n_v_heads * dims.d_v
    ws_ptr, ws_bytes = _workspace(workspace)
    _check(lib.gdn_layer_tail(
        ctypes.byref(dims), ctypes.byref(params), B,
        _ptr(x, "x", (B, C)), _ptr(conv_w, "conv_w", (C, K)),
        _ptr(conv_state, "conv_state", (B, K - 1, C)),
        _ptr(beta, "beta", (B, dims.n_v_heads)), _ptr(gate, "gate", (B, dims.n_v_heads)),
        _ptr(state, "state", (B, dims.n_v_heads, dims.d_v, dims.d_k)),
        _ptr(z, "z", (B, nv)), _ptr(norm_w, "norm_w", (params.norm_group,)),
        _ptr(y, "y", (B, nv)),
        _ptr(dbg_qkv, "dbg_qkv", (B, C), optional=True),
        _ptr(dbg_core, "dbg_core", (B, dims.n_v_heads, dims.d_v), optional=True),
        ws_ptr, ws_bytes, _stream(stream)))


def layer_tail_noalloc(x, conv_w, conv_state, beta, gate, state, z, norm_w, y,
                       dbg_qkv=None, dbg_core=None,
                       dims: Dims = PAGE_DIMS, params: TailParams = PAGE_TAIL,
                       stream=None) -> None:
    """gdn_layer_tail_noalloc: layer_tail with the library's static per-GPU
    scratch in place of a workspace (allocates nothing)."""
    B, C = x.shape
    K = params.conv_kernel
    nv = dims.n_v_heads * dims.d_v
    _check(lib.gdn_layer_tail_noalloc(
        ctypes.byref(dims), ctypes.byref(params), B,
        _ptr(x, "x", (B, C)), _ptr(conv_w, "conv_w", (C, K)),
        _ptr(conv_state, "conv_state", (B, K - 1, C)),
        _ptr(beta, "beta", (B, dims.n_v_heads)), _ptr(gate, "gate", (B, dims.n_v_heads)),
        _ptr(state, "state", (B, dims.n_v_heads, dims.d_v, dims.d_k)),
        _ptr(z, "z", (B, nv)), _ptr(norm_w, "norm_w", (params.norm_group,)),
        _ptr(y, "y", (B, nv)),
        _ptr(dbg_qkv, "dbg_qkv", (B, C), optional=True),
        _ptr(dbg_core, "dbg_core", (B, dims.n_v_heads, dims.d_v), optional=True),
        _stream(stream)))


def layer_tail_pair(x, conv_w, conv_state, conv_state_next, beta, gate, state, state_next,
                    z, norm_w, y, dims: Dims = PAGE_DIMS, params: TailParams = PAGE_TAIL,
                    stream=None) -> None:
    """gdn_layer_tail_pair: x [B][2][C], beta/gate [B][2][Hv], z/y [B][2][Hv*dv].
    conv_state and state are committed with position 1 in place;
    conv_state_next and state_next receive the tentative ring and state after
    position 2."""
    B, _, C = x.shape
    K = params.conv_kernel
    nv = dims.n_v_heads * dims.d_v
    st = (B, dims.n_v_heads, dims.d_v, dims.d_k)
    _check(lib.gdn_layer_tail_pair(
        ctypes.byref(dims), ctypes.byref(params), B,
        _ptr(x, "x", (B, 2, C)), _ptr(conv_w, "conv_w", (C, K)),
        _ptr(conv_state, "conv_state", (B, K - 1, C)),
        _ptr(conv_state_next, "conv_state_next", (B, K - 1, C)),
        _ptr(beta, "beta", (B, 2, dims.n_v_heads)), _ptr(gate, "gate", (B, 2, dims.n_v_heads)),
        _ptr(state, "state", st), _ptr(state_next, "state_next", st),
        _ptr(z, "z", (B, 2, nv)), _ptr(norm_w, "norm_w", (params.norm_group,)),
        _ptr(y, "y", (B, 2, nv)), _stream(stream)))


def _gate_inputs(ba, a_log, dt_bias, B, Hv):
    return GateInputs(_ptr(ba, "ba", (B, 2 * Hv)), _ptr(a_log, "a_log", (Hv,)),
                      _ptr(dt_bias, "dt_bias", (Hv,)))


def gate_transform(ba, a_log, dt_bias, beta, gate, dims: Dims = PAGE_DIMS, stream=None) -> None:
    """gdn_gate_transform: ba [B][2*Hv] (beta logits | alpha logits), a_log and
    dt_bias [Hv] -> beta, gate [B][Hv]."""
    B = ba.shape[0]
    Hv = dims.n_v_heads
    gi = _gate_inputs(ba, a_log, dt_bias, B, Hv)
    _check(lib.gdn_gate_transform(ctypes.byref(dims), B, ctypes.byref(gi),
                                  _ptr(beta, "beta", (B, Hv)), _ptr(gate, "gate", (B, Hv)),
                                  _stream(stream)))


def layer_tail_ba_workspace_bytes(B: int, dims: Dims = PAGE_DIMS) -> int:
    return int(lib.gdn_layer_tail_ba_workspace_bytes(ctypes.byref(dims), B))


def layer_tail_ba(x, conv_w, conv_state, ba, a_log, dt_bias, state, z, norm_w, y,
                  dbg_qkv=None, dbg_core=None, workspace=None,
                  dims: Dims = PAGE_DIMS, params: TailParams = PAGE_TAIL, stream=None) -> None:
    """gdn_layer_tail_ba: layer_tail with beta and gate made from the raw gate
    inputs.  workspace: at least layer_tail_ba_workspace_bytes(B) bytes."""
    B, C = x.shape
    K = params.conv_kernel
    nv = dims.n_v_heads * dims.d_v
    gi = _gate_inputs(ba, a_log, dt_bias, B, dims.n_v_heads)
    ws_ptr, ws_bytes = _workspace(workspace)
    _check(lib.gdn_layer_tail_ba(
        ctypes.byref(dims), ctypes.byref(params), B,
        _ptr(x, "x", (B, C)), _ptr(conv_w, "conv_w", (C, K)),
        _ptr(conv_state, "conv_state", (B, K - 1, C)), ctypes.byref(gi),
        _ptr(state, "state", (B, dims.n_v_heads, dims.d_v, dims.d_k)),
        _ptr(z, "z", (B, nv)), _ptr(norm_w, "norm_w", (params.norm_group,)),
        _ptr(y, "y", (B, nv)),
        _ptr(dbg_qkv, "dbg_qkv", (B, C), optional=True),
        _ptr(dbg_core, "dbg_core", (B, dims.n_v_heads, dims.d_v), optional=True),
        ws_ptr, ws_bytes, _stream(stream)))
