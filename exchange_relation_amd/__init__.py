"""Python binding of librelation (exact causal Full / Multi-Head Relation on
MI355X / gfx950).

Argument marshalling only: tensors are checked and passed as device pointers
to the C ABI declared in include/relation.h, on torch's current HIP stream.
Every step of the operator runs in the library's HIP kernels. There is no
fallback: if librelation.so is missing or fails to load, every call raises.

Build the library with ``python -m exchange_relation_amd.build``.
"""
import ctypes
import math
import os

import torch

__all__ = [
    "RelationError",
    "lib_path",
    "load_library",
    "relation_fwd",
    "relation_fwd_workspace_bytes",
    "relation_bwd",
    "relation_bwd_workspace_bytes",
    "relation_cache_decode",
    "relation_cache_decode_noalloc",
    "relation_decode_workspace_bytes",
    "relation_cache_decode_ragged",
    "relation_cache_prefill",
    "relation_prefill_workspace_bytes",
    "relation_mhr_fwd",
    "relation_mhr_bwd",
    "relation_linear_fwd",
    "relation_linear_bwd",
    "linear_states_shape",
    "LinearRelationFunction",
    "linear_relation",
    "relation_linear_step",
    "relation_status_string",
    "relation_version",
    "RelationFunction",
    "relation",
    "MultiHeadRelationFunction",
    "mhr_relation",
    "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
REL_F32, REL_BF16 = 0, 1
EXPORTED_SYMBOLS = (
    "relation_fwd_workspace_bytes",
    "relation_fwd",
    "relation_bwd_workspace_bytes",
    "relation_bwd",
    "relation_bwd_events",
    "relation_decode_workspace_bytes",
    "relation_cache_decode",
    "relation_cache_decode_noalloc",
    "relation_cache_decode_ragged",
    "relation_prefill_workspace_bytes",
    "relation_cache_prefill",
    "relation_mhr_fwd_workspace_bytes",
    "relation_mhr_fwd",
    "relation_mhr_bwd_workspace_bytes",
    "relation_mhr_bwd",
    "relation_linear_fwd",
    "relation_linear_states_bytes",
    "relation_linear_bwd_workspace_bytes",
    "relation_linear_bwd_reuse_workspace_bytes",
    "relation_linear_bwd",
    "relation_linear_step",
    "relation_status_string",
    "relation_version",
)


class RelationError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {relation_status_string(status)} (status {status})")


def lib_path():
    return os.path.join(_HERE, "librelation.so")


_LIB = None


def load_library():
    """Loads librelation.so (once) and declares the C signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m exchange_relation_amd.build`")
    lib = ctypes.CDLL(path)
    c_int, c_float, c_size, vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
    lib.relation_fwd_workspace_bytes.restype = c_size
    lib.relation_fwd_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int]
    lib.relation_fwd.restype = c_int
    lib.relation_fwd.argtypes = [c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, vp,
                                 vp, c_size, c_float, c_float, c_float, vp, vp]
    lib.relation_bwd_workspace_bytes.restype = c_size
    lib.relation_bwd_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int]
    lib.relation_bwd.restype = c_int
    lib.relation_bwd.argtypes = [c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, vp,
                                 vp, vp, vp, vp, vp, c_size, c_float, c_float, c_float, vp, vp]
    lib.relation_bwd_events.restype = c_int
    lib.relation_bwd_events.argtypes = lib.relation_bwd.argtypes + [vp, vp]
    lib.relation_decode_workspace_bytes.restype = c_size
    lib.relation_decode_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int]
    lib.relation_cache_decode.restype = c_int
    lib.relation_cache_decode.argtypes = [c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, c_int,
                                          c_int, vp, vp, vp, c_size, c_float, c_float, c_float,
                                          vp]
    lib.relation_cache_decode_noalloc.restype = c_int
    lib.relation_cache_decode_noalloc.argtypes = [c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp,
                                                  c_int, c_int, vp, vp, c_float, c_float,
                                                  c_float, vp]
    lib.relation_cache_decode_ragged.restype = c_int
    lib.relation_cache_decode_ragged.argtypes = [c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp,
                                                 c_int, vp, c_int, vp, vp, vp, c_size, c_float,
                                                 c_float, c_float, vp]
    lib.relation_prefill_workspace_bytes.restype = c_size
    lib.relation_prefill_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int,
                                                     c_int]
    lib.relation_cache_prefill.restype = c_int
    lib.relation_cache_prefill.argtypes = [c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp,
                                           c_int, vp, c_int, vp, vp, vp, vp, c_size, c_float,
                                           c_float, c_float, vp]
    lib.relation_mhr_fwd_workspace_bytes.restype = c_size
    lib.relation_mhr_fwd_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int]
    lib.relation_mhr_fwd.restype = c_int
    lib.relation_mhr_fwd.argtypes = [c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, vp,
                                     c_int, vp, vp, vp, vp, c_size, c_float, c_float, c_float, vp,
                                     vp]
    lib.relation_mhr_bwd_workspace_bytes.restype = c_size
    lib.relation_mhr_bwd_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int]
    lib.relation_mhr_bwd.restype = c_int
    lib.relation_mhr_bwd.argtypes = [c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, vp,
                                     c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, c_size,
                                     c_float, c_float, c_float, vp, vp]
    lib.relation_linear_fwd.restype = c_int
    lib.relation_linear_fwd.argtypes = [c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, vp,
                                        vp, vp, vp, vp, c_float, c_float, vp]
    for fn in ("relation_linear_states_bytes", "relation_linear_bwd_workspace_bytes",
               "relation_linear_bwd_reuse_workspace_bytes"):
        getattr(lib, fn).restype = c_size
        getattr(lib, fn).argtypes = [c_int, c_int, c_int, c_int, c_int]
    lib.relation_linear_bwd.restype = c_int
    lib.relation_linear_bwd.argtypes = [c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, vp,
                                        vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, c_size, c_float,
                                        c_float, vp]
    lib.relation_linear_step.restype = c_int
    lib.relation_linear_step.argtypes = [c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, vp, vp,
                                         vp, c_float, c_float, vp]
    lib.relation_status_string.restype = ctypes.c_char_p
    lib.relation_status_string.argtypes = [c_int]
    lib.relation_version.restype = c_int
    lib.relation_version.argtypes = []
    _LIB = lib
    return lib


def relation_status_string(status):
    return load_library().relation_status_string(int(status)).decode()


def relation_version():
    return load_library().relation_version()


def _dtype_code(t):
    if t.dtype == torch.float32:
        return REL_F32
    if t.dtype == torch.bfloat16:
        return REL_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _check(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _scale(D, scale):
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def _lam(lam, dev):
    """lambda as (value, device pointer): a number is passed by value; a
    one-element float32 tensor on the inputs' device is read by the kernels
    when they run (no host synchronisation)."""
    if isinstance(lam, torch.Tensor):
        if lam.device != dev or lam.dtype != torch.float32 or lam.numel() != 1:
            raise ValueError("a tensor lambda must be one float32 element on the inputs' device")
        if not lam.is_contiguous():
            raise ValueError("lambda tensor must be contiguous")
        return 0.0, _ptr(lam)
    return float(lam), None


def relation_fwd_workspace_bytes(dtype, B, H, T, D):
    code = REL_BF16 if dtype == torch.bfloat16 else REL_F32
    return int(load_library().relation_fwd_workspace_bytes(code, B, H, T, D))


def _workspace(t, need, dev):
    """The caller's workspace tensor (checked), or a new one when need > 0."""
    if t is None:
        return torch.empty((need,), device=dev, dtype=torch.uint8) if need > 0 else None
    if t.device != dev or not t.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    return t


def relation_fwd(q, k, v, lam=0.0, scale=None, tau_s=2.0, y=None, lse=None, gate=None,
                 want_lse=True, want_gate=False, workspace=None, split=True, stream=None):
    """Multi-Head Relation forward. q, k, v: [B, H, T, D] on a GPU, float32 or
    bfloat16, contiguous. Returns (y, lse, gate); lse / gate are float32
    [B, H, T] or None. Outputs may be passed in to avoid allocation. With
    split (default) a grid too small to fill the GPU splits its long query
    blocks over keys, in a workspace allocated here unless one is given."""
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, D]")
    B, H, T, D = q.shape
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for name, t in (("k", k), ("v", v)):
        _check(t, name, dt, q.shape, dev)
    _check(q, "q", dt, q.shape, dev)
    if y is None:
        y = torch.empty_like(q)
    _check(y, "y", dt, q.shape, dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H, T), device=dev, dtype=torch.float32)
    if gate is None and want_gate:
        gate = torch.empty((B, H, T), device=dev, dtype=torch.float32)
    for name, t in (("lse", lse), ("gate", gate)):
        if t is not None:
            _check(t, name, torch.float32, (B, H, T), dev)
    ws = _workspace(workspace, relation_fwd_workspace_bytes(dt, B, H, T, D), dev) if split else None
    lv, lp = _lam(lam, dev)
    st = lib.relation_fwd(code, B, H, T, D, _ptr(q), _ptr(k), _ptr(v), _ptr(y), _ptr(lse),
                          _ptr(gate), _ptr(ws), _nbytes(ws), _scale(D, scale), float(tau_s),
                          lv, lp, _stream(dev, stream))
    if st != 0:
        raise RelationError(st, "relation_fwd")
    return y, lse, gate


def relation_bwd_workspace_bytes(dtype, B, H, T, D):
    code = REL_BF16 if dtype == torch.bfloat16 else REL_F32
    return int(load_library().relation_bwd_workspace_bytes(code, B, H, T, D))


def relation_bwd(q, k, v, y, dy, lse, lam=0.0, scale=None, tau_s=2.0, dq=None, dk=None, dv=None,
                 dlambda=None, workspace=None, want_dlambda=True, stream=None, main_events=None):
    """Backward of relation_fwd. Returns (dq, dk, dv, dlambda) where dlambda is
    a float32 device tensor of shape [1] (or None). main_events: an optional
    pair of torch.cuda.Event(enable_timing=True) that the library records on
    its stream right before and after the main backward kernel(s)
    (relation_bwd_events), for timing that part alone."""
    lib = load_library()
    B, H, T, D = q.shape
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("y", y), ("dy", dy)):
        _check(t, name, dt, q.shape, dev)
    _check(lse, "lse", torch.float32, (B, H, T), dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(t, name, dt, q.shape, dev)
    if dlambda is None and want_dlambda:
        dlambda = torch.empty((1,), device=dev, dtype=torch.float32)
    need = int(lib.relation_bwd_workspace_bytes(code, B, H, T, D))
    if workspace is None:
        workspace = torch.empty((max(need, 1),), device=dev, dtype=torch.uint8)
    lv, lp = _lam(lam, dev)
    args = (code, B, H, T, D, _ptr(q), _ptr(k), _ptr(v), _ptr(y), _ptr(dy), _ptr(lse), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(dlambda), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _scale(D, scale), float(tau_s), lv, lp,
            _stream(dev, stream))
    if main_events is None:
        st = lib.relation_bwd(*args)
    else:
        handles = []
        for e in main_events:
            if e.cuda_event == 0:  # torch creates the HIP event at its first record
                e.record(torch.cuda.current_stream(dev))
            handles.append(ctypes.c_void_p(e.cuda_event))
        st = lib.relation_bwd_events(*args, *handles)
    if st != 0:
        raise RelationError(st, "relation_bwd")
    return dq, dk, dv, dlambda


def relation_decode_workspace_bytes(dtype, B, H, D, capacity):
    code = REL_BF16 if dtype == torch.bfloat16 else REL_F32
    return int(load_library().relation_decode_workspace_bytes(code, B, H, D, capacity))


def relation_cache_decode(q, k_new, v_new, k_cache, v_cache, n_hist, lam=0.0, scale=None,
                          tau_s=2.0, y=None, gate=None, workspace=None, want_gate=False,
                          stream=None):
    """One decode step: q, k_new, v_new [B, H, D]; k_cache, v_cache
    [B, H, capacity, D] (updated in place at slot n_hist). Returns (y, gate)."""
    lib = load_library()
    B, H, D = q.shape
    capacity = k_cache.shape[2]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new)):
        _check(t, name, dt, (B, H, D), dev)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _check(t, name, dt, (B, H, capacity, D), dev)
    y = torch.empty_like(q) if y is None else y
    _check(y, "y", dt, (B, H, D), dev)
    if gate is None and want_gate:
        gate = torch.empty((B, H), device=dev, dtype=torch.float32)
    if gate is not None:
        _check(gate, "gate", torch.float32, (B, H), dev)
    need = int(lib.relation_decode_workspace_bytes(code, B, H, D, capacity))
    if workspace is None:
        workspace = torch.empty((max(need, 1),), device=dev, dtype=torch.uint8)
    st = lib.relation_cache_decode(code, B, H, D, _ptr(q), _ptr(k_new), _ptr(v_new),
                                   _ptr(k_cache), _ptr(v_cache), capacity, int(n_hist), _ptr(y),
                                   _ptr(gate), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(),
                                   _scale(D, scale), float(tau_s), float(lam),
                                   _stream(dev, stream))
    if st != 0:
        raise RelationError(st, "relation_cache_decode")
    return y, gate


def relation_cache_decode_noalloc(q, k_new, v_new, k_cache, v_cache, n_hist, y, lam=0.0,
                                  scale=None, tau_s=2.0, gate=None, stream=None):
    """relation_cache_decode without a workspace: the library's static
    per-GPU scratch serves instead, and nothing is allocated (y and gate are
    the caller's). Calls that overlap in time on one GPU race. Returns
    (y, gate)."""
    lib = load_library()
    B, H, D = q.shape
    capacity = k_cache.shape[2]
    dev, dt = q.device, q.dtype
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("y", y)):
        _check(t, name, dt, (B, H, D), dev)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _check(t, name, dt, (B, H, capacity, D), dev)
    if gate is not None:
        _check(gate, "gate", torch.float32, (B, H), dev)
    st = lib.relation_cache_decode_noalloc(_dtype_code(q), B, H, D, _ptr(q), _ptr(k_new),
                                           _ptr(v_new), _ptr(k_cache), _ptr(v_cache), capacity,
                                           int(n_hist), _ptr(y), _ptr(gate), _scale(D, scale),
                                           float(tau_s), float(lam), _stream(dev, stream))
    if st != 0:
        raise RelationError(st, "relation_cache_decode_noalloc")
    return y, gate


def relation_cache_decode_ragged(q, k_new, v_new, k_cache, v_cache, n_hist, max_n_hist=None,
                                 lam=0.0, scale=None, tau_s=2.0, y=None, gate=None,
                                 workspace=None, want_gate=False, stream=None):
    """One decode step over a ragged cache: as relation_cache_decode, with
    n_hist a device int32 tensor [B] of per-sequence history lengths (not
    modified) and max_n_hist a host bound of them (default capacity - 1).
    Returns (y, gate)."""
    lib = load_library()
    B, H, D = q.shape
    capacity = k_cache.shape[2]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new)):
        _check(t, name, dt, (B, H, D), dev)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _check(t, name, dt, (B, H, capacity, D), dev)
    _check(n_hist, "n_hist", torch.int32, (B,), dev)
    bound = capacity - 1 if max_n_hist is None else int(max_n_hist)
    y = torch.empty_like(q) if y is None else y
    _check(y, "y", dt, (B, H, D), dev)
    if gate is None and want_gate:
        gate = torch.empty((B, H), device=dev, dtype=torch.float32)
    if gate is not None:
        _check(gate, "gate", torch.float32, (B, H), dev)
    need = int(lib.relation_decode_workspace_bytes(code, B, H, D, capacity))
    if workspace is None:
        workspace = torch.empty((max(need, 1),), device=dev, dtype=torch.uint8)
    st = lib.relation_cache_decode_ragged(code, B, H, D, _ptr(q), _ptr(k_new), _ptr(v_new),
                                          _ptr(k_cache), _ptr(v_cache), capacity, _ptr(n_hist),
                                          bound, _ptr(y), _ptr(gate), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          _scale(D, scale), float(tau_s), float(lam),
                                          _stream(dev, stream))
    if st != 0:
        raise RelationError(st, "relation_cache_decode_ragged")
    return y, gate


def relation_prefill_workspace_bytes(dtype, B, H, D, m, n_hist, per_sequence):
    code = REL_BF16 if dtype == torch.bfloat16 else REL_F32
    return int(load_library().relation_prefill_workspace_bytes(code, B, H, D, m, n_hist,
                                                                1 if per_sequence else 0))


def relation_cache_prefill(q, k_new, v_new, k_cache, v_cache, n_hist, max_n_hist=None, lam=0.0,
                           scale=None, tau_s=2.0, y=None, lse=None, gate=None, want_stats=False,
                           workspace=None, split=True, stream=None):
    """m new tokens per sequence: q, k_new, v_new [B, H, m, D] appended at
    slot n_hist (an int, or a device int32 tensor [B] with max_n_hist its
    bound, default capacity - m) of k_cache, v_cache [B, H, capacity, D].
    Returns (y, lse, gate); lse and gate only with want_stats. With split
    (default) long histories are split over workgroups in a workspace."""
    lib = load_library()
    B, H, m, D = q.shape
    capacity = k_cache.shape[2]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new)):
        _check(t, name, dt, (B, H, m, D), dev)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _check(t, name, dt, (B, H, capacity, D), dev)
    if isinstance(n_hist, torch.Tensor):
        _check(n_hist, "n_hist", torch.int32, (B,), dev)
        nh, n = n_hist, capacity - m if max_n_hist is None else int(max_n_hist)
    else:
        nh, n = None, int(n_hist)
    y = torch.empty_like(q) if y is None else y
    _check(y, "y", dt, (B, H, m, D), dev)
    if want_stats:
        lse = torch.empty((B, H, m), device=dev, dtype=torch.float32) if lse is None else lse
        gate = torch.empty((B, H, m), device=dev, dtype=torch.float32) if gate is None else gate
    ws = None
    if split and n >= 0:
        ws = _workspace(workspace, relation_prefill_workspace_bytes(dt, B, H, D, m, n,
                                                                    nh is not None), dev)
    st = lib.relation_cache_prefill(code, B, H, D, m, _ptr(q), _ptr(k_new), _ptr(v_new),
                                    _ptr(k_cache), _ptr(v_cache), capacity, _ptr(nh), n, _ptr(y),
                                    _ptr(lse), _ptr(gate), _ptr(ws), _nbytes(ws),
                                    _scale(D, scale), float(tau_s), float(lam),
                                    _stream(dev, stream))
    if st != 0:
        raise RelationError(st, "relation_cache_prefill")
    return y, lse, gate


def _mhr_maps(p1, rope_cos, rope_sin, theta):
    B, H, T, D = p1.shape
    if (rope_cos is None) != (rope_sin is None):
        raise ValueError("rope_cos and rope_sin go together")
    if rope_cos is not None:
        _check(rope_cos, "rope_cos", torch.float32, (T, D // 2), p1.device)
        _check(rope_sin, "rope_sin", torch.float32, (T, D // 2), p1.device)
    if theta is not None:
        _check(theta, "theta", torch.float32, (H // 2,), p1.device)


def relation_mhr_fwd(p1, p2, I, rope_cos=None, rope_sin=None, theta=None, pairing=0, lam=0.0,
                     scale=None, tau_s=2.0, y=None, lse=None, gate=None, want_gate=False,
                     workspace=None, stream=None):
    """Multi-Head Relation forward with RoPE of p1, p2 (tables [T, D/2]) and
    Givens mixing of I (angles [H/2], pairing 0 or 1). Returns (y, lse, gate)."""
    lib = load_library()
    B, H, T, D = p1.shape
    dev, dt = p1.device, p1.dtype
    code = _dtype_code(p1)
    for name, t in (("p1", p1), ("p2", p2), ("I", I)):
        _check(t, name, dt, (B, H, T, D), dev)
    _mhr_maps(p1, rope_cos, rope_sin, theta)
    y = torch.empty_like(I) if y is None else y
    lse = torch.empty((B, H, T), device=dev, dtype=torch.float32) if lse is None else lse
    _check(y, "y", dt, (B, H, T, D), dev)
    _check(lse, "lse", torch.float32, (B, H, T), dev)
    if gate is None and want_gate:
        gate = torch.empty((B, H, T), device=dev, dtype=torch.float32)
    need = int(lib.relation_mhr_fwd_workspace_bytes(code, B, H, T, D))
    if workspace is None and need:
        workspace = torch.empty((need,), device=dev, dtype=torch.uint8)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.relation_mhr_fwd(code, B, H, T, D, _ptr(p1), _ptr(p2), _ptr(I), _ptr(rope_cos),
                              _ptr(rope_sin), _ptr(theta), int(pairing), _ptr(y), _ptr(lse),
                              _ptr(gate), _ptr(workspace), wsb, _scale(D, scale), float(tau_s),
                              *_lam(lam, dev), _stream(dev, stream))
    if st != 0:
        raise RelationError(st, "relation_mhr_fwd")
    return y, lse, gate


def relation_mhr_bwd(p1, p2, I, y, dy, lse, rope_cos=None, rope_sin=None, theta=None, pairing=0,
                     lam=0.0, scale=None, tau_s=2.0, dp1=None, dp2=None, dI=None, dlambda=None,
                     dtheta=None, workspace=None, fwd_workspace=None, stream=None):
    """Gradients of relation_mhr_fwd. Returns (dp1, dp2, dI, dlambda [1],
    dtheta [H/2] or None). fwd_workspace: the workspace tensor the forward
    used (unchanged since), whose rotated keys and mixed values are then
    reused instead of formed again."""
    lib = load_library()
    B, H, T, D = p1.shape
    dev, dt = p1.device, p1.dtype
    code = _dtype_code(p1)
    for name, t in (("p1", p1), ("p2", p2), ("I", I), ("y", y), ("dy", dy)):
        _check(t, name, dt, (B, H, T, D), dev)
    _check(lse, "lse", torch.float32, (B, H, T), dev)
    _mhr_maps(p1, rope_cos, rope_sin, theta)
    dp1 = torch.empty_like(p1) if dp1 is None else dp1
    dp2 = torch.empty_like(p2) if dp2 is None else dp2
    dI = torch.empty_like(I) if dI is None else dI
    dlambda = torch.empty((1,), device=dev, dtype=torch.float32) if dlambda is None else dlambda
    if theta is not None and dtheta is None:
        dtheta = torch.empty((H // 2,), device=dev, dtype=torch.float32)
    need = int(lib.relation_mhr_bwd_workspace_bytes(code, B, H, T, D))
    if workspace is None:
        workspace = torch.empty((max(need, 1),), device=dev, dtype=torch.uint8)
    st = lib.relation_mhr_bwd(code, B, H, T, D, _ptr(p1), _ptr(p2), _ptr(I), _ptr(rope_cos),
                              _ptr(rope_sin), _ptr(theta), int(pairing), _ptr(y), _ptr(dy),
                              _ptr(lse), _ptr(dp1), _ptr(dp2), _ptr(dI), _ptr(dlambda),
                              _ptr(dtheta), _ptr(fwd_workspace), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _scale(D, scale),
                              float(tau_s), *_lam(lam, dev), _stream(dev, stream))
    if st != 0:
        raise RelationError(st, "relation_mhr_bwd")
    return dp1, dp2, dI, dlambda, dtheta


def relation_linear_fwd(p1, p2, I, g, rope_cos=None, rope_sin=None, state_in=None,
                        want_state=False, scale=None, tau_s=2.0, y=None, state_out=None,
                        states=None, stream=None):
    """Linear Relation forward (bf16 p1, p2, I [B, H, T, 64]; fp32 log
    retention g of the same shape). Optional RoPE tables [T, 32] and initial
    state [B, H, 64, 64] fp32. `states` (optional, fp32
    [B, H, ceil(T / 128) + 1, 64, 64]) receives the state before every chunk
    and the final state, for relation_linear_bwd(fwd_states=...). Returns
    (y, state_out or None)."""
    lib = load_library()
    B, H, T, D = p1.shape
    dev, dt = p1.device, p1.dtype
    for name, t in (("p1", p1), ("p2", p2), ("I", I)):
        _check(t, name, dt, (B, H, T, D), dev)
    _check(g, "g", torch.float32, (B, H, T, D), dev)
    _mhr_maps(p1, rope_cos, rope_sin, None)
    if state_in is not None:
        _check(state_in, "state_in", torch.float32, (B, H, D, D), dev)
    y = torch.empty_like(I) if y is None else y
    _check(y, "y", dt, (B, H, T, D), dev)
    if state_out is None and want_state:
        state_out = torch.empty((B, H, D, D), device=dev, dtype=torch.float32)
    if state_out is not None:
        _check(state_out, "state_out", torch.float32, (B, H, D, D), dev)
    if states is not None:
        _check(states, "states", torch.float32, linear_states_shape(B, H, T, D), dev)
    st = lib.relation_linear_fwd(_dtype_code(p1), B, H, T, D, _ptr(p1), _ptr(p2), _ptr(I), _ptr(g),
                                 _ptr(rope_cos), _ptr(rope_sin), _ptr(state_in), _ptr(y),
                                 _ptr(state_out), _ptr(states), _scale(D, scale), float(tau_s),
                                 _stream(dev, stream))
    if st != 0:
        raise RelationError(st, "relation_linear_fwd")
    return y, state_out


def linear_states_shape(B, H, T, D=64):
    """Shape of the per-chunk states relation_linear_fwd can store: the state
    before every chunk, then the final state ([B, H, nchunks + 1, D, D] fp32;
    the library's relation_linear_states_bytes gives the size)."""
    n = int(load_library().relation_linear_states_bytes(REL_BF16, B, H, T, D))
    if n == 0:
        raise ValueError(f"no Linear Relation states for B={B} H={H} T={T} D={D}")
    return (B, H, n // (B * H * D * D * 4), D, D)


def relation_linear_bwd(p1, p2, I, g, dy, rope_cos=None, rope_sin=None, state_in=None,
                        dstate_out=None, want_dstate_in=False, scale=None, tau_s=2.0,
                        workspace=None, fwd_states=None, stream=None):
    """Gradients of relation_linear_fwd. Returns (dp1, dp2, dI, dg,
    dstate_in or None); dg is fp32 like g. fwd_states: the `states` the
    forward stored for these same inputs (skips the backward's state pass)."""
    lib = load_library()
    B, H, T, D = p1.shape
    dev, dt = p1.device, p1.dtype
    for name, t in (("p1", p1), ("p2", p2), ("I", I), ("dy", dy)):
        _check(t, name, dt, (B, H, T, D), dev)
    _check(g, "g", torch.float32, (B, H, T, D), dev)
    _mhr_maps(p1, rope_cos, rope_sin, None)
    for name, t in (("state_in", state_in), ("dstate_out", dstate_out)):
        if t is not None:
            _check(t, name, torch.float32, (B, H, D, D), dev)
    if fwd_states is not None:
        _check(fwd_states, "fwd_states", torch.float32, linear_states_shape(B, H, T, D), dev)
    dp1, dp2, dI = torch.empty_like(p1), torch.empty_like(p2), torch.empty_like(I)
    dg = torch.empty_like(g)
    dstate_in = (torch.empty((B, H, D, D), device=dev, dtype=torch.float32)
                 if want_dstate_in else None)
    query = (lib.relation_linear_bwd_workspace_bytes if fwd_states is None
             else lib.relation_linear_bwd_reuse_workspace_bytes)
    need = int(query(_dtype_code(p1), B, H, T, D))
    if workspace is None:
        workspace = torch.empty((max(need, 1),), device=dev, dtype=torch.uint8)
    st = lib.relation_linear_bwd(_dtype_code(p1), B, H, T, D, _ptr(p1), _ptr(p2), _ptr(I), _ptr(g),
                                 _ptr(rope_cos), _ptr(rope_sin), _ptr(state_in), _ptr(dy),
                                 _ptr(dstate_out), _ptr(dp1), _ptr(dp2), _ptr(dI), _ptr(dg),
                                 _ptr(dstate_in), _ptr(fwd_states), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _scale(D, scale),
                                 float(tau_s), _stream(dev, stream))
    if st != 0:
        raise RelationError(st, "relation_linear_bwd")
    return dp1, dp2, dI, dg, dstate_in


def relation_linear_step(p1, p2, I, g, state, rope_cos=None, rope_sin=None, scale=None,
                         tau_s=2.0, y=None, stream=None):
    """One Linear Relation decode step: p1, p2, I [B, H, 64] bf16, g [B, H, 64]
    fp32, state [B, H, 64, 64] fp32 updated in place; rope rows [32] or None.
    Returns y [B, H, 64]."""
    lib = load_library()
    B, H, D = p1.shape
    dev, dt = p1.device, p1.dtype
    for name, t in (("p1", p1), ("p2", p2), ("I", I)):
        _check(t, name, dt, (B, H, D), dev)
    _check(g, "g", torch.float32, (B, H, D), dev)
    _check(state, "state", torch.float32, (B, H, D, D), dev)
    if (rope_cos is None) != (rope_sin is None):
        raise ValueError("rope_cos and rope_sin go together")
    if rope_cos is not None:
        _check(rope_cos, "rope_cos", torch.float32, (D // 2,), dev)
        _check(rope_sin, "rope_sin", torch.float32, (D // 2,), dev)
    y = torch.empty_like(I) if y is None else y
    _check(y, "y", dt, (B, H, D), dev)
    st = lib.relation_linear_step(_dtype_code(p1), B, H, D, _ptr(p1), _ptr(p2), _ptr(I), _ptr(g),
                                  _ptr(rope_cos), _ptr(rope_sin), _ptr(state), _ptr(y),
                                  _scale(D, scale), float(tau_s), _stream(dev, stream))
    if st != 0:
        raise RelationError(st, "relation_linear_step")
    return y


def _lam_tensor(lam, dev):
    """The learnable lambda as a one-element float32 tensor on `dev` (a copy
    only when its dtype, device or layout differ; no host round trip)."""
    t = lam.detach().reshape(1)
    if t.device != dev or t.dtype != torch.float32:
        t = t.to(device=dev, dtype=torch.float32)
    return t.contiguous()


class RelationFunction(torch.autograd.Function):
    """autograd wrapper: y = Relation(q, k, v; lambda) with gradients for q,
    k, v and the layer's lambda (a one-element tensor)."""

    @staticmethod
    def forward(ctx, q, k, v, lam, scale, tau_s):
        # lambda stays on the device: the kernels read it when they run
        lam_d = _lam_tensor(lam, q.device)
        y, lse, _ = relation_fwd(q, k, v, lam=lam_d, scale=scale, tau_s=tau_s)
        ctx.save_for_backward(q, k, v, y, lse, lam_d)
        ctx.scale, ctx.tau_s, ctx.lam_shape = scale, tau_s, lam.shape
        return y

    @staticmethod
    def backward(ctx, dy):
        q, k, v, y, lse, lam_d = ctx.saved_tensors
        dq, dk, dv, dlam = relation_bwd(q, k, v, y, dy.contiguous(), lse, lam=lam_d,
                                        scale=ctx.scale, tau_s=ctx.tau_s)
        return dq, dk, dv, dlam.reshape(ctx.lam_shape), None, None


def relation(q, k, v, lam, scale=None, tau_s=2.0):
    """Differentiable Multi-Head Relation; lam is a scalar tensor (learnable)."""
    return RelationFunction.apply(q, k, v, lam, scale, tau_s)


class MultiHeadRelationFunction(torch.autograd.Function):
    """autograd wrapper of relation_mhr_fwd / relation_mhr_bwd: gradients for
    p1, p2, I, lambda and the Givens angles theta. The forward's workspace
    (rotated keys, mixed values) is kept for the backward, which reads it
    instead of forming the maps again."""

    @staticmethod
    def forward(ctx, p1, p2, I, lam, theta, rope_cos, rope_sin, pairing, scale, tau_s):
        B, H, T, D = p1.shape
        need = int(load_library().relation_mhr_fwd_workspace_bytes(_dtype_code(p1), B, H, T, D))
        ws = torch.empty((need,), device=p1.device, dtype=torch.uint8) if need else None
        lam_d = _lam_tensor(lam, p1.device)
        y, lse, _ = relation_mhr_fwd(p1, p2, I, rope_cos, rope_sin, theta, pairing,
                                     lam=lam_d, scale=scale, tau_s=tau_s, workspace=ws)
        ctx.save_for_backward(p1, p2, I, y, lse, theta, rope_cos, rope_sin, ws, lam_d)
        ctx.scale, ctx.tau_s, ctx.pairing = scale, tau_s, pairing
        ctx.lam_shape = lam.shape
        return y

    @staticmethod
    def backward(ctx, dy):
        p1, p2, I, y, lse, theta, rope_cos, rope_sin, ws, lam_d = ctx.saved_tensors
        dp1, dp2, dI, dlam, dth = relation_mhr_bwd(
            p1, p2, I, y, dy.contiguous(), lse, rope_cos, rope_sin, theta, ctx.pairing,
            lam=lam_d, scale=ctx.scale, tau_s=ctx.tau_s, fwd_workspace=ws)
        return (dp1, dp2, dI, dlam.reshape(ctx.lam_shape), dth, None, None, None, None, None)


class LinearRelationFunction(torch.autograd.Function):
    """autograd wrapper of relation_linear_fwd / relation_linear_bwd:
    gradients for p1, p2, I, the log retention g and the initial state. The
    forward stores the state before every chunk, and the backward reads them
    instead of running its own state pass."""

    @staticmethod
    def forward(ctx, p1, p2, I, g, state_in, rope_cos, rope_sin, scale, tau_s):
        B, H, T, D = p1.shape
        states = torch.empty(linear_states_shape(B, H, T, D), device=p1.device,
                             dtype=torch.float32)
        y, state_out = relation_linear_fwd(p1, p2, I, g, rope_cos, rope_sin, state_in,
                                           want_state=True, scale=scale, tau_s=tau_s,
                                           states=states)
        ctx.save_for_backward(p1, p2, I, g, state_in, rope_cos, rope_sin, states)
        ctx.scale, ctx.tau_s = scale, tau_s
        ctx.set_materialize_grads(False)
        return y, state_out

    @staticmethod
    def backward(ctx, dy, dstate_out):
        p1, p2, I, g, state_in, rope_cos, rope_sin, states = ctx.saved_tensors
        if dy is None:
            dy = torch.zeros_like(I)
        want_dsin = state_in is not None and ctx.needs_input_grad[4]
        dp1, dp2, dI, dg, dsin = relation_linear_bwd(
            p1, p2, I, g, dy.contiguous(), rope_cos, rope_sin, state_in,
            dstate_out=None if dstate_out is None else dstate_out.contiguous(),
            want_dstate_in=want_dsin, scale=ctx.scale, tau_s=ctx.tau_s, fwd_states=states)
        return dp1, dp2, dI, dg, dsin, None, None, None, None


def linear_relation(p1, p2, I, g, state_in=None, rope_cos=None, rope_sin=None, scale=None,
                    tau_s=2.0):
    """Differentiable Linear Relation: returns (y, state_out), both with
    gradients (state_out continues into a later call)."""
    return LinearRelationFunction.apply(p1, p2, I, g, state_in, rope_cos, rope_sin, scale, tau_s)


def mhr_relation(p1, p2, I, lam, theta=None, rope_cos=None, rope_sin=None, pairing=0, scale=None,
                 tau_s=2.0):
    """Differentiable Multi-Head Relation with RoPE tables [T, D/2] and
    Givens angles theta [H/2] (learnable); lam is a scalar tensor."""
    return MultiHeadRelationFunction.apply(p1, p2, I, lam, theta, rope_cos, rope_sin, pairing,
                                           scale, tau_s)
