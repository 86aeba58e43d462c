"""ctypes binding of libselscan (C ABI in include/selscan.h).

Argument marshalling only: dtype and device checks, ``.contiguous()``,
allocation of outputs and workspace with torch, the current HIP stream, and
status codes turned into exceptions.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

SELSCAN_F32 = 0
SELSCAN_BF16 = 1
SELSCAN_FLAG_ZOH_EXACT = 1
SELSCAN_FLAG_REVERSE = 2
SELSCAN_FLAG_REUSE_FWD_STATE = 4
SELSCAN_FLAG_KEEP_CHECKPOINTS = 8
SELSCAN_MAX_CONV_WIDTH = 4

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libselscan.so")
_lib = None


class SelscanError(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0):
        msg = "%s failed: status %d (%s)" % (where, status, status_string(status))
        if hip_error:
            msg += ", hipError %d" % hip_error
        super().__init__(msg)
        self.status = status
        self.hip_error = hip_error


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libselscan.so with argument types set; raises if not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libselscan.so is not built (%s); run "
                               "`python -m selective_state_space_selscan_amd.build`" % _LIB_PATH)
        L = ctypes.CDLL(_LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.selscan_abi_version.restype = I
        L.selscan_abi_version.argtypes = []
        L.selscan_status_string.restype = ctypes.c_char_p
        L.selscan_status_string.argtypes = [I]
        L.selscan_last_hip_error.restype = I
        L.selscan_last_hip_error.argtypes = []
        L.selscan_supports_n.restype = I
        L.selscan_supports_n.argtypes = [I64]
        L.selscan_fwd_status.restype = I
        L.selscan_fwd_status.argtypes = [P, P]
        L.selscan_fwd_noalloc.restype = I
        L.selscan_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, I, P, P, P, I64, I64, I64,
                                          I64, I, P]
        L.selscan_fwd_workspace_bytes.restype = ctypes.c_size_t
        L.selscan_fwd_workspace_bytes.argtypes = [I64, I64, I64, I64, I]
        L.selscan_fwd.restype = I
        L.selscan_fwd.argtypes = [P, P, P, P, P, P, P, P, I, P, P, P, I64, I64, I64, I64, I,
                                  P, ctypes.c_size_t, P]
        L.selscan_fwd_ex.restype = I
        L.selscan_fwd_ex.argtypes = [P, P, P, P, P, P, P, P, I, P, P, P, I64, I64, I64, I64, I,
                                     I, P, P, I64, P, ctypes.c_size_t, P]
        L.selscan_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.selscan_bwd_workspace_bytes.argtypes = [I64, I64, I64, I64, I]
        L.selscan_bwd.restype = I
        L.selscan_bwd.argtypes = [P] * 12 + [P] * 9 + [I64, I64, I64, I64, I, P,
                                                      ctypes.c_size_t, P]
        L.selscan_bwd.argtypes[8] = I
        L.selscan_bwd_ex.restype = I
        L.selscan_bwd_ex.argtypes = [P] * 12 + [P] * 9 + [I, P, P, I64, P, P] + \
            [I64, I64, I64, I64, I, P, ctypes.c_size_t, P]
        L.selscan_bwd_ex.argtypes[8] = I
        L.selscan_state_update.restype = I
        L.selscan_state_update.argtypes = [P, P, P, P, P, P, P, P, P, I, P, I64, I64, I64, I, P]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().selscan_status_string(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SELSCAN_F32
    if t.dtype == torch.bfloat16:
        return SELSCAN_BF16
    raise TypeError("u/delta/Bm/Cm/z must be float32 or bfloat16, got %s" % t.dtype)


def _prep(t: Optional[torch.Tensor], dtype, device, name: str, shape) -> Optional[torch.Tensor]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    t = t.contiguous()
    if t.data_ptr() % 16:
        t = t.clone()
    return t


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def selscan_fwd_status(workspace: torch.Tensor, stream=None) -> None:
    """Waits for ``stream`` and raises SelscanError (SELSCAN_ERR_TIMEOUT) if a
    bounded wait of the look-back plan gave up during the last forward in
    ``workspace``; returns at once under any other plan."""
    st = lib().selscan_fwd_status(_ptr(workspace), _stream(workspace.device, stream))
    if st != 0:
        raise SelscanError(st, "selscan_fwd_status", lib().selscan_last_hip_error())


def selscan_fwd_workspace_bytes(batch: int, L: int, dim: int, N: int, dtype: int) -> int:
    return int(lib().selscan_fwd_workspace_bytes(batch, L, dim, N, dtype))


def selscan_fwd(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor,
                Cm: torch.Tensor, D_skip: Optional[torch.Tensor] = None,
                z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                delta_softplus: bool = True, h0: Optional[torch.Tensor] = None,
                return_last_state: bool = False, y: Optional[torch.Tensor] = None,
                h_last: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                stream: Optional[torch.cuda.Stream] = None):
    """Selective-scan forward through ``selscan_fwd`` (asynchronous on the stream).

    u, delta, z: (batch, L, dim); Bm, Cm: (batch, L, N) in float32 or bfloat16;
    A: (dim, N), D_skip, delta_bias: (dim,), h0: (batch, dim, N) in float32.
    Returns y, or (y, h_last) when ``return_last_state``."""
    return _fwd(u, delta, A, Bm, Cm, D_skip, z, delta_bias, delta_softplus, h0,
                return_last_state, y, h_last, workspace, stream, None)


def selscan_fwd_noalloc(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor,
                        Bm: torch.Tensor, Cm: torch.Tensor, y: torch.Tensor,
                        D_skip: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                        delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = True,
                        h0: Optional[torch.Tensor] = None, h_last: Optional[torch.Tensor] = None,
                        stream: Optional[torch.cuda.Stream] = None) -> None:
    """``selscan_fwd`` through ``selscan_fwd_noalloc``: the library's fixed
    device scratch is the workspace, and the caller provides y (and h_last)
    as well as the inputs, so the call allocates nothing.  Inputs must
    already be dense, 16-byte aligned and of the right dtypes (no copies are
    made here)."""
    L_ = lib()
    dev = u.device
    dt = u.dtype
    code = _dtype_code(u)
    batch, L, dim = u.shape
    N = A.shape[-1]
    ins = dict(u=(u, dt, (batch, L, dim)), delta=(delta, dt, (batch, L, dim)),
               A=(A, torch.float32, (dim, N)), Bm=(Bm, dt, (batch, L, N)),
               Cm=(Cm, dt, (batch, L, N)), D_skip=(D_skip, torch.float32, (dim,)),
               z=(z, dt, (batch, L, dim)), delta_bias=(delta_bias, torch.float32, (dim,)),
               h0=(h0, torch.float32, (batch, dim, N)))
    for name, (t, tdt, shape) in ins.items():
        if t is not None:
            _check_out(t, tdt, dev, name, shape)
    _check_out(y, dt, dev, "y", (batch, L, dim))
    if h_last is not None:
        _check_out(h_last, torch.float32, dev, "h_last", (batch, dim, N))
    rc = L_.selscan_fwd_noalloc(_ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D_skip),
                                _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)), _ptr(h0),
                                _ptr(y), _ptr(h_last), batch, L, dim, N, code,
                                _stream(dev, stream))
    if rc != 0:
        raise SelscanError(rc, "selscan_fwd_noalloc", L_.selscan_last_hip_error())


def selscan_fwd_ex(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor,
                   Cm: torch.Tensor, D_skip: Optional[torch.Tensor] = None,
                   z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                   delta_softplus: bool = True, h0: Optional[torch.Tensor] = None,
                   return_last_state: bool = False, flags: int = 0,
                   conv_weight: Optional[torch.Tensor] = None,
                   conv_bias: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                   h_last: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None,
                   stream: Optional[torch.cuda.Stream] = None):
    """Forward with variants through ``selscan_fwd_ex``: ``flags`` is an OR of
    SELSCAN_FLAG_ZOH_EXACT and SELSCAN_FLAG_REVERSE, or
    SELSCAN_FLAG_KEEP_CHECKPOINTS, alone or with REVERSE (the backward's
    checkpoints kept in
    ``workspace``, which must then be given, of at least
    selscan_bwd_workspace_bytes); ``conv_weight`` (dim, k) float32 with k <= 4
    (and ``conv_bias`` (dim,)) enables the causal conv1d + SiLU prologue on u.
    Other arguments and the result as ``selscan_fwd``."""
    return _fwd(u, delta, A, Bm, Cm, D_skip, z, delta_bias, delta_softplus, h0,
                return_last_state, y, h_last, workspace, stream,
                (int(flags), conv_weight, conv_bias))


def _fwd(u, delta, A, Bm, Cm, D_skip, z, delta_bias, delta_softplus, h0, return_last_state, y,
         h_last, workspace, stream, ex):
    L_ = lib()
    dev = u.device
    dt = u.dtype
    code = _dtype_code(u)
    batch, L, dim = u.shape
    N = A.shape[-1]
    u = _prep(u, dt, dev, "u", (batch, L, dim))
    delta = _prep(delta, dt, dev, "delta", (batch, L, dim))
    Bm = _prep(Bm, dt, dev, "Bm", (batch, L, N))
    Cm = _prep(Cm, dt, dev, "Cm", (batch, L, N))
    z = _prep(z, dt, dev, "z", (batch, L, dim))
    A = _prep(A, torch.float32, dev, "A", (dim, N))
    D_skip = _prep(D_skip, torch.float32, dev, "D_skip", (dim,))
    delta_bias = _prep(delta_bias, torch.float32, dev, "delta_bias", (dim,))
    h0 = _prep(h0, torch.float32, dev, "h0", (batch, dim, N))
    if y is None:
        y = torch.empty((batch, L, dim), dtype=dt, device=dev)
    else:
        y = _check_out(y, dt, dev, "y", (batch, L, dim))
    if return_last_state and h_last is None:
        h_last = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    elif h_last is not None:
        h_last = _check_out(h_last, torch.float32, dev, "h_last", (batch, dim, N))
    ws_bytes = int(L_.selscan_fwd_workspace_bytes(batch, L, dim, N, code))
    if ex is not None and ex[0] & SELSCAN_FLAG_KEEP_CHECKPOINTS:
        # the checkpoints are for a later backward: they go to the caller's workspace
        ws_bytes = int(L_.selscan_bwd_workspace_bytes(batch, L, dim, N, code))
        if workspace is None or workspace.numel() * workspace.element_size() < ws_bytes:
            raise ValueError("SELSCAN_FLAG_KEEP_CHECKPOINTS needs a workspace of at least "
                             "selscan_bwd_workspace_bytes (%d)" % ws_bytes)
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_ptr = _ptr(workspace) if ws_bytes else None
    ws_len = workspace.numel() * workspace.element_size() if ws_bytes else 0
    common = (_ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D_skip), _ptr(z),
              _ptr(delta_bias), int(bool(delta_softplus)), _ptr(h0), _ptr(y), _ptr(h_last),
              batch, L, dim, N, code)
    if ex is None:
        name = "selscan_fwd"
        rc = L_.selscan_fwd(*common, ws_ptr, ws_len, _stream(dev, stream))
    else:
        name = "selscan_fwd_ex"
        flags, conv_weight, conv_bias = ex
        k = 0
        if conv_weight is not None:
            if conv_weight.dim() != 2:
                raise ValueError("conv_weight must be (dim, k), got %s" % (tuple(conv_weight.shape),))
            k = conv_weight.shape[1]
            conv_weight = _prep(conv_weight, torch.float32, dev, "conv_weight", (dim, k))
            conv_bias = _prep(conv_bias, torch.float32, dev, "conv_bias", (dim,))
        elif conv_bias is not None:
            raise ValueError("conv_bias given without conv_weight")
        rc = L_.selscan_fwd_ex(*common, flags, _ptr(conv_weight), _ptr(conv_bias), k, ws_ptr,
                               ws_len, _stream(dev, stream))
    if rc != 0:
        raise SelscanError(rc, name, L_.selscan_last_hip_error())
    return (y, h_last) if return_last_state else y


def selscan_bwd_workspace_bytes(batch: int, L: int, dim: int, N: int, dtype: int) -> int:
    return int(lib().selscan_bwd_workspace_bytes(batch, L, dim, N, dtype))


def selscan_bwd(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor,
                Cm: torch.Tensor, dy: torch.Tensor, D_skip: Optional[torch.Tensor] = None,
                z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                delta_softplus: bool = True, h0: Optional[torch.Tensor] = None,
                dh_last: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                stream: Optional[torch.cuda.Stream] = None) -> dict:
    """Gradients of ``selscan_fwd`` through ``selscan_bwd`` (asynchronous on the
    stream).  dy: (batch, L, dim) in the input dtype; dh_last: (batch, dim, N)
    float32 or None.  Returns a dict with du, ddelta, dz (None without z) in the
    input dtype and dA, dB, dC, dD, ddelta_bias, dh0 in float32."""
    return _bwd(u, delta, A, Bm, Cm, dy, D_skip, z, delta_bias, delta_softplus, h0, dh_last,
                workspace, stream, None)


def selscan_bwd_ex(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor,
                   Cm: torch.Tensor, dy: torch.Tensor, D_skip: Optional[torch.Tensor] = None,
                   z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                   delta_softplus: bool = True, h0: Optional[torch.Tensor] = None,
                   dh_last: Optional[torch.Tensor] = None, flags: int = 0,
                   conv_weight: Optional[torch.Tensor] = None,
                   conv_bias: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None,
                   stream: Optional[torch.cuda.Stream] = None) -> dict:
    """Gradients of ``selscan_fwd_ex`` (same ``flags``, ``conv_weight``,
    ``conv_bias``) through ``selscan_bwd_ex``.  The dict of ``selscan_bwd``,
    plus dconv_weight (dim, k) and dconv_bias (dim,) in float32 with the conv
    prologue (None without); du is then the gradient of the conv's input u.

    With SELSCAN_FLAG_REUSE_FWD_STATE in ``flags`` (plain or REVERSE alone),
    ``workspace`` must be the tensor the matching forward (``selscan_fwd``,
    or ``selscan_fwd_ex`` with the same REVERSE flag) last ran in, on the
    same inputs, h0 and sizes, at least ``selscan_bwd_workspace_bytes``
    long; the backward then reads that forward's part summaries and entry
    states instead of recomputing them (same result, bit for bit).  With
    SELSCAN_FLAG_KEEP_CHECKPOINTS as well, that forward was
    ``selscan_fwd_ex`` with SELSCAN_FLAG_KEEP_CHECKPOINTS, and its kept
    checkpoint states replace the backward's checkpoint pass (the same
    gradients up to rounding)."""
    return _bwd(u, delta, A, Bm, Cm, dy, D_skip, z, delta_bias, delta_softplus, h0, dh_last,
                workspace, stream, (int(flags), conv_weight, conv_bias))


def _bwd(u, delta, A, Bm, Cm, dy, D_skip, z, delta_bias, delta_softplus, h0, dh_last, workspace,
         stream, ex):
    L_ = lib()
    dev = u.device
    dt = u.dtype
    code = _dtype_code(u)
    batch, L, dim = u.shape
    N = A.shape[-1]
    u = _prep(u, dt, dev, "u", (batch, L, dim))
    delta = _prep(delta, dt, dev, "delta", (batch, L, dim))
    Bm = _prep(Bm, dt, dev, "Bm", (batch, L, N))
    Cm = _prep(Cm, dt, dev, "Cm", (batch, L, N))
    z = _prep(z, dt, dev, "z", (batch, L, dim))
    dy = _prep(dy, dt, dev, "dy", (batch, L, dim))
    A = _prep(A, torch.float32, dev, "A", (dim, N))
    D_skip = _prep(D_skip, torch.float32, dev, "D_skip", (dim,))
    delta_bias = _prep(delta_bias, torch.float32, dev, "delta_bias", (dim,))
    h0 = _prep(h0, torch.float32, dev, "h0", (batch, dim, N))
    dh_last = _prep(dh_last, torch.float32, dev, "dh_last", (batch, dim, N))
    f32 = torch.float32
    g = dict(du=torch.empty((batch, L, dim), dtype=dt, device=dev),
             ddelta=torch.empty((batch, L, dim), dtype=dt, device=dev),
             dz=torch.empty((batch, L, dim), dtype=dt, device=dev) if z is not None else None,
             dA=torch.empty((dim, N), dtype=f32, device=dev),
             dB=torch.empty((batch, L, N), dtype=f32, device=dev),
             dC=torch.empty((batch, L, N), dtype=f32, device=dev),
             dD=torch.empty((dim,), dtype=f32, device=dev),
             ddelta_bias=torch.empty((dim,), dtype=f32, device=dev),
             dh0=torch.empty((batch, dim, N), dtype=f32, device=dev))
    ws_bytes = int(L_.selscan_bwd_workspace_bytes(batch, L, dim, N, code))
    if ex is not None and ex[0] & SELSCAN_FLAG_REUSE_FWD_STATE:
        # the forward's part state is in the caller's workspace: never replace it
        if workspace is None or workspace.numel() * workspace.element_size() < ws_bytes:
            raise ValueError("SELSCAN_FLAG_REUSE_FWD_STATE needs the forward's workspace, "
                             "at least selscan_bwd_workspace_bytes (%d) long" % ws_bytes)
    elif workspace is None or workspace.numel() * workspace.element_size() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    common = (_ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D_skip), _ptr(z),
              _ptr(delta_bias), int(bool(delta_softplus)), _ptr(h0), _ptr(dy), _ptr(dh_last),
              _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
              _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["ddelta_bias"]), _ptr(g["dh0"]))
    tail = (batch, L, dim, N, code, _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(dev, stream))
    if ex is None:
        name = "selscan_bwd"
        rc = L_.selscan_bwd(*common, *tail)
    else:
        name = "selscan_bwd_ex"
        flags, conv_weight, conv_bias = ex
        k = 0
        g["dconv_weight"] = g["dconv_bias"] = None
        if conv_weight is not None:
            if conv_weight.dim() != 2:
                raise ValueError("conv_weight must be (dim, k), got %s" % (tuple(conv_weight.shape),))
            k = conv_weight.shape[1]
            conv_weight = _prep(conv_weight, f32, dev, "conv_weight", (dim, k))
            conv_bias = _prep(conv_bias, f32, dev, "conv_bias", (dim,))
            g["dconv_weight"] = torch.empty((dim, k), dtype=f32, device=dev)
            g["dconv_bias"] = torch.empty((dim,), dtype=f32, device=dev)
        elif conv_bias is not None:
            raise ValueError("conv_bias given without conv_weight")
        rc = L_.selscan_bwd_ex(*common, flags, _ptr(conv_weight), _ptr(conv_bias), k,
                               _ptr(g["dconv_weight"]), _ptr(g["dconv_bias"]), *tail)
    if rc != 0:
        raise SelscanError(rc, name, L_.selscan_last_hip_error())
    return g


def selscan_state_update(state: torch.Tensor, u: torch.Tensor, delta: torch.Tensor,
                         A: torch.Tensor, Bm: torch.Tensor, Cm: torch.Tensor,
                         D_skip: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                         delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = True,
                         y: Optional[torch.Tensor] = None,
                         stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """One decode step through ``selscan_state_update``; ``state`` (batch, dim, N)
    float32 is updated in place.  u, delta, z: (batch, dim); Bm, Cm: (batch, N)."""
    L_ = lib()
    dev = u.device
    dt = u.dtype
    code = _dtype_code(u)
    batch, dim = u.shape
    N = A.shape[-1]
    state = _check_out(state, torch.float32, dev, "state", (batch, dim, N))
    u = _prep(u, dt, dev, "u", (batch, dim))
    delta = _prep(delta, dt, dev, "delta", (batch, dim))
    Bm = _prep(Bm, dt, dev, "Bm", (batch, N))
    Cm = _prep(Cm, dt, dev, "Cm", (batch, N))
    z = _prep(z, dt, dev, "z", (batch, dim))
    A = _prep(A, torch.float32, dev, "A", (dim, N))
    D_skip = _prep(D_skip, torch.float32, dev, "D_skip", (dim,))
    delta_bias = _prep(delta_bias, torch.float32, dev, "delta_bias", (dim,))
    if y is None:
        y = torch.empty((batch, dim), dtype=dt, device=dev)
    else:
        y = _check_out(y, dt, dev, "y", (batch, dim))
    rc = L_.selscan_state_update(_ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm),
                                 _ptr(D_skip), _ptr(z), _ptr(delta_bias),
                                 int(bool(delta_softplus)), _ptr(y), batch, dim, N, code,
                                 _stream(dev, stream))
    if rc != 0:
        raise SelscanError(rc, "selscan_state_update", L_.selscan_last_hip_error())
    return y


def _check_out(t: torch.Tensor, dtype, device, name: str, shape) -> torch.Tensor:
    """Outputs are written in place, so they must already be dense and aligned."""
    if t.device != device or t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError("%s must be %s %s on %s" % (name, dtype, tuple(shape), device))
    if not t.is_contiguous() or t.data_ptr() % 16:
        raise ValueError("%s must be contiguous and 16-byte aligned" % name)
    return t
