"""ctypes binding of libvla.so (include/vla.h): argument marshalling only.

Every step of the recurrence runs in the library's HIP kernels.  PyTorch is
used only for device memory and the current stream.  There is no fallback: if
the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# VLA_LIB names another build of the same sources (the sanitizer test's)
LIB_PATH = os.environ.get("VLA_LIB") or os.path.join(PKG, "libvla.so")

VLA_OK, VLA_ERR_INVALID_ARG, VLA_ERR_UNSUPPORTED, VLA_ERR_HIP = 0, 1, 2, 3
VLA_F32, VLA_BF16 = 0, 1
NOALLOC_SCRATCH_BYTES = 64 << 20   # VLA_NOALLOC_SCRATCH_BYTES of include/vla.h

_vp = ctypes.c_void_p
_lib = None


class VLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def load() -> ctypes.CDLL:
    """Load libvla.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; build it with "
                "`python -m long_context_sequence_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.vla_forward.restype = ctypes.c_int
        lib.vla_forward.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_float,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        lib.vla_forward_penalty.restype = ctypes.c_int
        lib.vla_forward_penalty.argtypes = [_vp, _vp, _vp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                            ctypes.c_float, _vp, _vp, _vp, _vp, _vp,
                                            ctypes.c_size_t, _vp]
        lib.vla_forward_memory.restype = ctypes.c_int
        lib.vla_forward_memory.argtypes = [_vp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _vp,
                                           ctypes.c_size_t, _vp]
        lib.vla_forward_noalloc.restype = ctypes.c_int
        lib.vla_forward_noalloc.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_float, ctypes.c_float, _vp, _vp, _vp, _vp,
                                            _vp, _vp, _vp, _vp]
        lib.vla_forward_workspace_size.restype = ctypes.c_int
        lib.vla_forward_workspace_size.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                   ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
        lib.vla_step.restype = ctypes.c_int
        lib.vla_step.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_float, _vp, _vp, _vp, _vp, _vp]
        lib.vla_forward_scan.restype = ctypes.c_int
        lib.vla_forward_scan.argtypes = lib.vla_forward.argtypes
        lib.vla_forward_scan_workspace_size.restype = ctypes.c_int
        lib.vla_forward_scan_workspace_size.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                        ctypes.c_int,
                                                        ctypes.POINTER(ctypes.c_size_t)]
        lib.vla_backward.restype = ctypes.c_int
        lib.vla_backward.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_float,
                                     _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _vp, _vp, ctypes.c_size_t, _vp]
        lib.vla_backward_workspace_size.restype = ctypes.c_int
        lib.vla_backward_workspace_size.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                    ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
        lib.vla_baseline_forward.restype = ctypes.c_int
        lib.vla_baseline_forward.argtypes = [ctypes.c_int, _vp, _vp, _vp, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_float, ctypes.c_float, _vp,
                                             _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        lib.vla_baseline_workspace_size.restype = ctypes.c_int
        lib.vla_baseline_workspace_size.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                    ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
        lib.vla_status_string.restype = ctypes.c_char_p
        lib.vla_status_string.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().vla_status_string(int(status)).decode()


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return VLA_F32
    if t.dtype == torch.bfloat16:
        return VLA_BF16
    raise TypeError(f"unsupported input dtype {t.dtype} (float32 or bfloat16)")


def _check(t, name, shape, dtype=None, device=None):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def workspace_size(B: int, H: int, T: int, d_h: int) -> int:
    """Bytes of device workspace vla_forward needs for these sizes."""
    n = ctypes.c_size_t(0)
    st = load().vla_forward_workspace_size(int(B), int(H), int(T), int(d_h), ctypes.byref(n))
    if st != VLA_OK:
        raise VLAError(st, "vla_forward_workspace_size")
    return n.value


def vla_forward(q, k, v, u, lambda0: float = 0.1, eps: float = 1e-4, *,
                o=None, S_out=None, A_out=None, zkey_out=None,
                S0=None, A0=None, zkey0=None, return_state: bool = False, stream=None,
                workspace=None):
    """VLA forward over [B, H, T, d_h] device tensors (float32 or bfloat16).

    Returns ``o`` ([B, H, T, d_h] float32), or ``(o, S, A, zkey)`` when
    ``return_state`` is set or any state output is passed.  ``S0, A0, zkey0``
    continue from a given state.  ``workspace`` is an optional device byte
    tensor of at least ``workspace_size(B, H, T, d_h)`` bytes (allocated here
    when not given).  Launches on ``stream`` (default: PyTorch's current
    stream) without synchronising.
    """
    torch = _torch()
    B, H, T, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("u", u)):
        _check(t, name, (B, H, T, d), q.dtype, dev)
    f32 = torch.float32
    if o is None:
        o = torch.empty((B, H, T, d), dtype=f32, device=dev)
    want_state = return_state or any(x is not None for x in (S_out, A_out, zkey_out))
    if return_state:
        S_out = torch.empty((B, H, d, d), dtype=f32, device=dev) if S_out is None else S_out
        A_out = torch.empty((B, H, d, d), dtype=f32, device=dev) if A_out is None else A_out
        zkey_out = torch.empty((B, H, d), dtype=f32, device=dev) if zkey_out is None else zkey_out
    _check(o, "o", (B, H, T, d), f32, dev)
    for name, t, shp in (("S_out", S_out, (B, H, d, d)), ("A_out", A_out, (B, H, d, d)),
                         ("zkey_out", zkey_out, (B, H, d)), ("S0", S0, (B, H, d, d)),
                         ("A0", A0, (B, H, d, d)), ("zkey0", zkey0, (B, H, d))):
        _check(t, name, shp, f32, dev)
    workspace = _workspace(workspace, B, H, T, d, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().vla_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(u), _dtype_code(q), B, H, T, d,
                            float(lambda0), float(eps), _ptr(o), _ptr(S_out), _ptr(A_out),
                            _ptr(zkey_out), _ptr(S0), _ptr(A0), _ptr(zkey0),
                            _ptr(workspace), ws_bytes, _stream(stream))
    if st != VLA_OK:
        raise VLAError(st, "vla_forward")
    return (o, S_out, A_out, zkey_out) if want_state else o


def _workspace(workspace, B, H, T, d, dev):
    torch = _torch()
    need = workspace_size(B, H, T, d)
    if workspace is None:
        return torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    if need:
        if not workspace.is_cuda or workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the inputs' device")
        if workspace.numel() * workspace.element_size() < need:
            raise ValueError(f"workspace: need {need} bytes")
    return workspace


def vla_forward_penalty(q, k, u, lambda0: float = 0.1, eps: float = 1e-4, *, workspace,
                        A_out=None, zkey_out=None, A0=None, zkey0=None, stream=None):
    """First pass of the forward (d_h in {64, 96, 128}): the penalty chain and the
    per-chunk factors, left in ``workspace`` (a device byte tensor of at least
    ``workspace_size(B, H, T, d_h)`` bytes).  Writes ``A_out``/``zkey_out`` if given."""
    B, H, T, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("u", u)):
        _check(t, name, (B, H, T, d), q.dtype, dev)
    f32 = _torch().float32
    for name, t, shp in (("A_out", A_out, (B, H, d, d)), ("zkey_out", zkey_out, (B, H, d)),
                         ("A0", A0, (B, H, d, d)), ("zkey0", zkey0, (B, H, d))):
        _check(t, name, shp, f32, dev)
    workspace = _workspace(workspace, B, H, T, d, dev)
    st = load().vla_forward_penalty(_ptr(q), _ptr(k), _ptr(u), _dtype_code(q), B, H, T, d,
                                    float(lambda0), float(eps), _ptr(A_out), _ptr(zkey_out),
                                    _ptr(A0), _ptr(zkey0), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream))
    if st != VLA_OK:
        raise VLAError(st, "vla_forward_penalty")


def vla_forward_memory(v, *, workspace, o=None, S_out=None, S0=None, stream=None):
    """Second pass of the forward: the memory chain and the readout from the
    factors (and k^, phi(q)) ``vla_forward_penalty`` left in ``workspace``, and v.
    Returns ``o``."""
    torch = _torch()
    B, H, T, d = v.shape
    dev = v.device
    _check(v, "v", (B, H, T, d), v.dtype, dev)
    f32 = torch.float32
    if o is None:
        o = torch.empty((B, H, T, d), dtype=f32, device=dev)
    _check(o, "o", (B, H, T, d), f32, dev)
    _check(S_out, "S_out", (B, H, d, d), f32, dev)
    _check(S0, "S0", (B, H, d, d), f32, dev)
    workspace = _workspace(workspace, B, H, T, d, dev)
    st = load().vla_forward_memory(_ptr(v), _dtype_code(v), B, H, T, d, _ptr(o), _ptr(S_out),
                                   _ptr(S0), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream))
    if st != VLA_OK:
        raise VLAError(st, "vla_forward_memory")
    return o


def vla_forward_noalloc(q, k, v, u, lambda0: float = 0.1, eps: float = 1e-4, *, o, S_out=None,
                        A_out=None, zkey_out=None, S0=None, A0=None, zkey0=None, stream=None):
    """``vla_forward`` with the library's own fixed workspace: nothing is
    allocated, so every output is passed in (``o`` [B, H, T, d_h] float32 and
    any of the final-state outputs).  Sizes needing more workspace than
    ``NOALLOC_SCRATCH_BYTES`` raise VLAError (VLA_ERR_UNSUPPORTED)."""
    B, H, T, d = q.shape
    dev = q.device
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v), ("u", u)):
        _check(t, name, (B, H, T, d), q.dtype, dev)
    f32 = torch.float32
    _check(o, "o", (B, H, T, d), f32, dev)
    for name, t, shp in (("S_out", S_out, (B, H, d, d)), ("A_out", A_out, (B, H, d, d)),
                         ("zkey_out", zkey_out, (B, H, d)), ("S0", S0, (B, H, d, d)),
                         ("A0", A0, (B, H, d, d)), ("zkey0", zkey0, (B, H, d))):
        _check(t, name, shp, f32, dev)
    st = load().vla_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(u), _dtype_code(q), B, H, T, d,
                                    float(lambda0), float(eps), _ptr(o), _ptr(S_out),
                                    _ptr(A_out), _ptr(zkey_out), _ptr(S0), _ptr(A0), _ptr(zkey0),
                                    _stream(stream))
    if st != VLA_OK:
        raise VLAError(st, "vla_forward_noalloc")
    return o


BASELINES = {"linear": 0, "delta": 1}   # vla_baseline of include/vla.h


def baseline_workspace_size(B: int, H: int, T: int, d_h: int) -> int:
    """Bytes of device workspace vla_baseline needs for these sizes."""
    n = ctypes.c_size_t(0)
    st = load().vla_baseline_workspace_size(int(B), int(H), int(T), int(d_h), ctypes.byref(n))
    if st != VLA_OK:
        raise VLAError(st, "vla_baseline_workspace_size")
    return n.value


def vla_baseline(kind: str, q, k, v, beta: float = 1.0, eps: float = 1e-4, *, o=None,
                 S_out=None, zkey_out=None, S0=None, zkey0=None, return_state: bool = False,
                 stream=None, workspace=None):
    """A baseline on the same [B, H, T, d_h] inputs: kind "linear" (cumulative-sum
    linear attention) or "delta" (DeltaNet, gate beta on the unit key).  Returns
    ``o``, or ``(o, S, zkey)`` with ``return_state`` or a state output."""
    torch = _torch()
    B, H, T, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, (B, H, T, d), q.dtype, dev)
    f32 = torch.float32
    if o is None:
        o = torch.empty((B, H, T, d), dtype=f32, device=dev)
    want_state = return_state or S_out is not None or zkey_out is not None
    if return_state:
        S_out = torch.empty((B, H, d, d), dtype=f32, device=dev) if S_out is None else S_out
        zkey_out = torch.empty((B, H, d), dtype=f32, device=dev) if zkey_out is None else zkey_out
    _check(o, "o", (B, H, T, d), f32, dev)
    for name, t, shp in (("S_out", S_out, (B, H, d, d)), ("zkey_out", zkey_out, (B, H, d)),
                         ("S0", S0, (B, H, d, d)), ("zkey0", zkey0, (B, H, d))):
        _check(t, name, shp, f32, dev)
    need = baseline_workspace_size(B, H, T, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace: need {need} bytes")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().vla_baseline_forward(BASELINES[kind], _ptr(q), _ptr(k), _ptr(v), _dtype_code(q),
                                     B, H, T, d, float(beta), float(eps), _ptr(o), _ptr(S_out),
                                     _ptr(zkey_out), _ptr(S0), _ptr(zkey0), _ptr(workspace),
                                     ws_bytes, _stream(stream))
    if st != VLA_OK:
        raise VLAError(st, "vla_baseline_forward")
    return (o, S_out, zkey_out) if want_state else o


def vla_step(q, k, v, u, S, A, zkey, eps: float = 1e-4, *, o=None, stream=None):
    """One decode token: q, k, v, u are [B, H, d_h]; S, A ([B, H, d, d]) and
    zkey ([B, H, d]) float32 state tensors are updated in place.  Returns o
    ([B, H, d_h] float32)."""
    torch = _torch()
    B, H, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("u", u)):
        _check(t, name, (B, H, d), q.dtype, dev)
    f32 = torch.float32
    if o is None:
        o = torch.empty((B, H, d), dtype=f32, device=dev)
    _check(o, "o", (B, H, d), f32, dev)
    _check(S, "S", (B, H, d, d), f32, dev)
    _check(A, "A", (B, H, d, d), f32, dev)
    _check(zkey, "zkey", (B, H, d), f32, dev)
    st = load().vla_step(_ptr(q), _ptr(k), _ptr(v), _ptr(u), _dtype_code(q), B, H, d,
                         float(eps), _ptr(S), _ptr(A), _ptr(zkey), _ptr(o), _stream(stream))
    if st != VLA_OK:
        raise VLAError(st, "vla_step")
    return o


def vla_status_string(status: int) -> str:
    return status_string(status)


def backward_workspace_size(B: int, H: int, T: int, d_h: int) -> int:
    """Bytes of device workspace vla_backward needs for these sizes."""
    n = ctypes.c_size_t(0)
    st = load().vla_backward_workspace_size(int(B), int(H), int(T), int(d_h), ctypes.byref(n))
    if st != VLA_OK:
        raise VLAError(st, "vla_backward_workspace_size")
    return n.value


def vla_backward(q, k, v, u, dO, lambda0: float = 0.1, eps: float = 1e-4, *,
                 S0=None, A0=None, zkey0=None, dS_T=None, dA_T=None, dzkey_T=None,
                 want_state_grads: bool = True, workspace=None, stream=None):
    """Gradients through vla_forward for [B, H, T, d_h] device inputs.

    ``dO`` ([B, H, T, d_h] float32) is dL/do; ``dS_T, dA_T, dzkey_T`` are the
    adjoints of the final state (None for zero).  Returns ``(dq, dk, dv, du,
    dS0, dA0, dzkey0)`` (float32; the last three None unless
    ``want_state_grads``); ``dA0`` is the gradient with respect to A0 as a
    symmetric matrix.  Launches on ``stream`` without synchronising.
    """
    torch = _torch()
    B, H, T, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("u", u)):
        _check(t, name, (B, H, T, d), q.dtype, dev)
    f32 = torch.float32
    _check(dO, "dO", (B, H, T, d), f32, dev)
    for name, t, shp in (("S0", S0, (B, H, d, d)), ("A0", A0, (B, H, d, d)),
                         ("zkey0", zkey0, (B, H, d)), ("dS_T", dS_T, (B, H, d, d)),
                         ("dA_T", dA_T, (B, H, d, d)), ("dzkey_T", dzkey_T, (B, H, d))):
        _check(t, name, shp, f32, dev)
    dq, dk, dv, du = (torch.empty((B, H, T, d), dtype=f32, device=dev) for _ in range(4))
    dS0 = dA0 = dzk0 = None
    if want_state_grads:
        dS0 = torch.empty((B, H, d, d), dtype=f32, device=dev)
        dA0 = torch.empty((B, H, d, d), dtype=f32, device=dev)
        dzk0 = torch.empty((B, H, d), dtype=f32, device=dev)
    need = backward_workspace_size(B, H, T, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    elif need and (not workspace.is_cuda or workspace.device != dev
                   or not workspace.is_contiguous()
                   or workspace.numel() * workspace.element_size() < need):
        raise ValueError(f"workspace: need a contiguous device tensor of {need} bytes")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().vla_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(u), _dtype_code(q), B, H, T, d,
                             float(lambda0), float(eps), _ptr(S0), _ptr(A0), _ptr(zkey0),
                             _ptr(dO), _ptr(dS_T), _ptr(dA_T), _ptr(dzkey_T), _ptr(dq), _ptr(dk),
                             _ptr(dv), _ptr(du), _ptr(dS0), _ptr(dA0), _ptr(dzk0),
                             _ptr(workspace), ws_bytes, _stream(stream))
    if st != VLA_OK:
        raise VLAError(st, "vla_backward")
    return dq, dk, dv, du, dS0, dA0, dzk0


def scan_workspace_size(B: int, H: int, T: int, d_h: int) -> int:
    """Bytes of device workspace vla_forward_scan needs for these sizes."""
    n = ctypes.c_size_t(0)
    st = load().vla_forward_scan_workspace_size(int(B), int(H), int(T), int(d_h), ctypes.byref(n))
    if st != VLA_OK:
        raise VLAError(st, "vla_forward_scan_workspace_size")
    return n.value


def vla_forward_scan(q, k, v, u, lambda0: float = 0.1, eps: float = 1e-4, *, o=None,
                     S0=None, A0=None, zkey0=None, workspace=None, stream=None):
    """vla_forward with the memory chain as a scan over chunks (d_h in {64, 96, 128}).
    Returns ``(o, S, A, zkey)`` (float32)."""
    torch = _torch()
    B, H, T, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("u", u)):
        _check(t, name, (B, H, T, d), q.dtype, dev)
    f32 = torch.float32
    if o is None:
        o = torch.empty((B, H, T, d), dtype=f32, device=dev)
    _check(o, "o", (B, H, T, d), f32, dev)
    S = torch.empty((B, H, d, d), dtype=f32, device=dev)
    A = torch.empty((B, H, d, d), dtype=f32, device=dev)
    zk = torch.empty((B, H, d), dtype=f32, device=dev)
    for name, t, shp in (("S0", S0, (B, H, d, d)), ("A0", A0, (B, H, d, d)),
                         ("zkey0", zkey0, (B, H, d))):
        _check(t, name, shp, f32, dev)
    need = scan_workspace_size(B, H, T, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif (not workspace.is_cuda or workspace.device != dev or not workspace.is_contiguous()
          or workspace.numel() * workspace.element_size() < need):
        raise ValueError(f"workspace: need a contiguous device tensor of {need} bytes")
    st = load().vla_forward_scan(_ptr(q), _ptr(k), _ptr(v), _ptr(u), _dtype_code(q), B, H, T, d,
                                 float(lambda0), float(eps), _ptr(o), _ptr(S), _ptr(A), _ptr(zk),
                                 _ptr(S0), _ptr(A0), _ptr(zkey0), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    if st != VLA_OK:
        raise VLAError(st, "vla_forward_scan")
    return o, S, A, zk
