"""CPU oracle for the S6 selective scan -- test infrastructure only.

Only ``tests/``, the smoke check of the build entry point and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code with the HIP library.

``selscan_oracle.c`` is the sequential fp64 definition of the scan (see its
header for the page citations).  ``build()`` compiles it with gcc + OpenMP;
``fwd``, ``bwd`` and ``state_update`` wrap it for numpy arrays.

Parity status: every function here is pinned by tests/test_oracle_pins.py
(LTI convolution, closed-form double sum, associative scan, Delta limits,
softplus round trip, skip path, split invariance, decode = forward,
causality, permutation and linearity); the variants of ``fwd`` by the LTI
convolution with the exact zero-order-hold kernel, its A -> 0 limit, the
suffix closed form of the reverse direction, torch's conv1d for the conv
prologue and the flip identity of the reverse direction; ``bwd`` by torch
autograd over a plain fp64 loop of the recurrence and by central finite
differences of ``fwd`` on dyadic inputs.  The pages print no worked numeric
example, so no value is pinned to a number printed on the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "selscan_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle shared library in place (gcc, -O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
                               "-std=c11", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_fwd.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_int, P, P, P,
                                   I64, I64, I64, I64, ctypes.c_int]
        lib.oracle_fwd.restype = ctypes.c_int
        lib.oracle_fwd_ex.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_int, P, P, P,
                                      I64, I64, I64, I64, ctypes.c_int, P, P, I64, ctypes.c_int]
        lib.oracle_fwd_ex.restype = ctypes.c_int
        lib.oracle_bwd.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_int, P, P, P,
                                   P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, ctypes.c_int]
        lib.oracle_bwd.restype = ctypes.c_int
        lib.oracle_bwd_ex.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_int, P, P, P,
                                      P, P, P, P, P, P, P, P, P, I64, I64, I64, I64,
                                      ctypes.c_int, P, P, I64, P, P, ctypes.c_int]
        lib.oracle_bwd_ex.restype = ctypes.c_int
        lib.oracle_state_update.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.c_int, P,
                                            I64, I64, I64, ctypes.c_int]
        lib.oracle_state_update.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


ZOH_EXACT = 1
REVERSE = 2


def fwd(u, delta, A, Bm, Cm, D_skip=None, z=None, delta_bias=None, delta_softplus=True,
        h0=None, threads: Optional[int] = None, flags: int = 0, conv_w=None, conv_b=None):
    """Sequential fp64 forward scan.

    u, delta, z: (batch, L, dim); Bm, Cm: (batch, L, N); A: (dim, N);
    D_skip, delta_bias: (dim,); h0: (batch, dim, N).
    flags: ZOH_EXACT and/or REVERSE.  conv_w (dim, k), conv_b (dim,): causal
    depthwise conv1d + SiLU prologue applied to u (then u is the conv input).
    Returns (y (batch, L, dim) float64, h_last (batch, dim, N) float64)."""
    u, delta, A, Bm, Cm = map(_f32, (u, delta, A, Bm, Cm))
    D_skip, z, delta_bias = map(_f32, (D_skip, z, delta_bias))
    conv_w, conv_b = _f32(conv_w), _f32(conv_b)
    conv_k = 0 if conv_w is None else conv_w.shape[1]
    assert conv_w is None or conv_w.shape == (u.shape[2], conv_k)
    batch, L, dim = u.shape
    N = A.shape[1]
    assert delta.shape == u.shape and A.shape == (dim, N)
    assert Bm.shape == (batch, L, N) and Cm.shape == (batch, L, N)
    assert z is None or z.shape == u.shape
    h0a = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
    assert h0a is None or h0a.shape == (batch, dim, N)
    y = np.empty((batch, L, dim), dtype=np.float64)
    h_last = np.empty((batch, dim, N), dtype=np.float64)
    rc = _load().oracle_fwd_ex(_ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm),
                               _ptr(D_skip), _ptr(z), _ptr(delta_bias),
                               int(bool(delta_softplus)), _ptr(h0a), _ptr(y), _ptr(h_last),
                               batch, L, dim, N, int(flags), _ptr(conv_w), _ptr(conv_b),
                               conv_k, threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_fwd failed with code %d" % rc)
    return y, h_last


def bwd(u, delta, A, Bm, Cm, dy, D_skip=None, z=None, delta_bias=None, delta_softplus=True,
        h0=None, dh_last=None, threads: Optional[int] = None, flags: int = 0, conv_w=None,
        conv_b=None):
    """fp64 gradients of ``fwd`` (with the same flags and conv prologue) for the
    upstream gradients dy (batch, L, dim) and dh_last (batch, dim, N) or None.

    Returns a dict of float64 arrays: du (of the raw input when the conv
    prologue is on), ddelta, dz (None without z), dA, dB, dC, dD, dbias, dh0,
    and dconv_w, dconv_b (None without the conv prologue)."""
    u, delta, A, Bm, Cm, dy = map(_f32, (u, delta, A, Bm, Cm, dy))
    D_skip, z, delta_bias = map(_f32, (D_skip, z, delta_bias))
    conv_w, conv_b = _f32(conv_w), _f32(conv_b)
    conv_k = 0 if conv_w is None else conv_w.shape[1]
    batch, L, dim = u.shape
    N = A.shape[1]
    assert delta.shape == u.shape and dy.shape == u.shape and A.shape == (dim, N)
    assert Bm.shape == (batch, L, N) and Cm.shape == (batch, L, N)
    assert z is None or z.shape == u.shape
    h0a = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
    dhl = None if dh_last is None else np.ascontiguousarray(dh_last, dtype=np.float64)
    out = dict(du=np.empty((batch, L, dim)), ddelta=np.empty((batch, L, dim)),
               dz=np.empty((batch, L, dim)) if z is not None else None,
               dA=np.empty((dim, N)), dB=np.empty((batch, L, N)), dC=np.empty((batch, L, N)),
               dD=np.empty(dim), dbias=np.empty(dim), dh0=np.empty((batch, dim, N)),
               dconv_w=np.empty((dim, conv_k)) if conv_k else None,
               dconv_b=np.empty(dim) if conv_k else None)
    rc = _load().oracle_bwd_ex(_ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D_skip),
                               _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)), _ptr(h0a),
                               _ptr(dy), _ptr(dhl), _ptr(out["du"]), _ptr(out["ddelta"]),
                               _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]),
                               _ptr(out["dD"]), _ptr(out["dz"]), _ptr(out["dbias"]),
                               _ptr(out["dh0"]), batch, L, dim, N, int(flags), _ptr(conv_w),
                               _ptr(conv_b), conv_k, _ptr(out["dconv_w"]), _ptr(out["dconv_b"]),
                               threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_bwd failed with code %d" % rc)
    return out


def state_update(state, u, delta, A, Bm, Cm, D_skip=None, z=None, delta_bias=None,
                 delta_softplus=True, threads: Optional[int] = None):
    """One fp64 decode step, in place on ``state`` (batch, dim, N) float64.

    u, delta, z: (batch, dim); Bm, Cm: (batch, N).  Returns y (batch, dim)."""
    assert state.dtype == np.float64 and state.flags.c_contiguous
    u, delta, A, Bm, Cm = map(_f32, (u, delta, A, Bm, Cm))
    D_skip, z, delta_bias = map(_f32, (D_skip, z, delta_bias))
    batch, dim, N = state.shape
    assert u.shape == (batch, dim) and delta.shape == (batch, dim) and A.shape == (dim, N)
    assert Bm.shape == (batch, N) and Cm.shape == (batch, N)
    y = np.empty((batch, dim), dtype=np.float64)
    rc = _load().oracle_state_update(_ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(Bm),
                                     _ptr(Cm), _ptr(D_skip), _ptr(z), _ptr(delta_bias),
                                     int(bool(delta_softplus)), _ptr(y), batch, dim, N,
                                     threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_state_update failed with code %d" % rc)
    return y


def fwd_inputs(inp, h0=None, threads=None, flags=0, conv_w=None, conv_b=None):
    """Run ``fwd`` on a ``selscan_inputs.FwdInputs`` bundle."""
    return fwd(inp.u.value, inp.delta.value, inp.A, inp.Bm.value, inp.Cm.value, inp.D_skip,
               None if inp.z is None else inp.z.value, inp.delta_bias, True,
               inp.h0 if h0 is None else h0, threads=threads, flags=flags, conv_w=conv_w,
               conv_b=conv_b)
