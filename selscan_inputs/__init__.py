"""Seeded synthetic inputs for the S6 selective scan, shared by the oracle side
and the HIP side.

This module only draws numbers and rounds them to the storage precision. It
holds none of the scan's arithmetic (no softplus, no discretisation, no
recurrence). Every workload here is synthetic; no dataset is involved.

Recipe (per workload; see ``WORKLOADS``):

* dt[d] = exp(U(ln 1e-3, ln 0.1)) and bias[d] = log(expm1(dt[d])), i.e. the
  inverse of softplus, so that softplus(0 + bias) = dt.  This is the dt
  initialisation the Mamba tutorial (pwwt.cn) gives in its §6.2 table and the
  Mamba selection-mechanism article (discosf.com) repeats in §5.1.
* u, B_t, C_t, z ~ N(0, 1) per (b, l, d) and per (b, l, n); Delta_raw ~ N(0, 0.5^2).
* A[d, n] = -(n + 1), the S4D-real initialisation A = -exp(A_log) with
  A_log = log(1..N) of the tutorial's §4.2 listing.
* D_skip = 1 (the listing initialises D to ones).
* bf16 workloads draw in fp32 and round to bf16 with round-to-nearest-even;
  the oracle receives the exact fp32 widening of those bf16 values.

Draw order for the forward: dt, u, Delta_raw, B, C, z (z only when gated).
Decode step k draws u, Delta_raw, B, C, z from ``default_rng([seed, k])``.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"

BASE_SEED = 20261203


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    L: int
    dim: int
    N: int
    dtype: str
    gate: bool
    want_last_state: bool
    seed: int
    decode_steps: int = 0          # >0 marks a decode workload (L is then 1 per call)
    check_every: int = 0


WORKLOADS = {
    # tiny S6 forward, fp32 throughout, no gate
    "tiny_f32": Workload("tiny_f32", 1, 256, 64, 16, F32, False, True, BASE_SEED + 0),
    # one Mamba-130M layer (d_model 768, expand 2)
    "mamba130m_layer": Workload("mamba130m_layer", 8, 2048, 1536, 16, BF16, True, False,
                                BASE_SEED + 1),
    # long sequence, exercises the cross-chunk carry, returns h_L
    "long_seq": Workload("long_seq", 1, 131072, 2048, 16, BF16, True, True, BASE_SEED + 2),
    # large layer (d_model 2560, expand 2)
    "large_layer": Workload("large_layer", 16, 2048, 5120, 16, BF16, True, False,
                            BASE_SEED + 3),
    # recurrent decode: 1024 single-token steps on a resident fp32 state
    "decode": Workload("decode", 256, 1, 5120, 16, BF16, True, False, BASE_SEED + 4,
                       decode_steps=1024, check_every=64),
}


def bf16_round_np(x: np.ndarray):
    """Round fp32 to bf16 (round to nearest, ties to even), in numpy.

    Returns (bits, widened): ``bits`` is the uint16 bf16 pattern, ``widened``
    the exact fp32 value of that bf16 number.  Inputs are finite draws."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    bits = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    widened = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return bits, widened


def bf16_round(x: np.ndarray):
    """Same result as ``bf16_round_np`` (checked in the tests), through torch's
    multi-threaded CPU conversion, which is much faster on large draws."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    widened = t.to(torch.float32).numpy()
    return bits, widened


@dataclasses.dataclass
class Tensor:
    """One input array in both representations.

    ``value`` is fp32 (exact value of the stored number); ``bits`` is the
    uint16 bf16 pattern when the storage dtype is bf16, else None."""
    value: np.ndarray
    bits: Optional[np.ndarray] = None


def _store(x: np.ndarray, dtype: str) -> Tensor:
    if dtype == BF16:
        bits, widened = bf16_round(x)
        return Tensor(widened, bits)
    return Tensor(np.ascontiguousarray(x, dtype=np.float32), None)


@dataclasses.dataclass
class FwdInputs:
    dtype: str
    batch: int
    L: int
    dim: int
    N: int
    u: Tensor
    delta: Tensor
    Bm: Tensor
    Cm: Tensor
    z: Optional[Tensor]
    A: np.ndarray            # (dim, N) fp32
    D_skip: Optional[np.ndarray]   # (dim,) fp32
    delta_bias: Optional[np.ndarray]  # (dim,) fp32
    h0: Optional[np.ndarray] = None   # (batch, dim, N) fp32


def dt_bias(rng: np.random.Generator, dim: int, dt_min=1e-3, dt_max=0.1) -> np.ndarray:
    dt = np.exp(rng.uniform(np.log(dt_min), np.log(dt_max), size=dim))
    return np.log(np.expm1(dt)).astype(np.float32)


def s4d_real_A(dim: int, N: int) -> np.ndarray:
    return np.ascontiguousarray(
        np.broadcast_to(-(np.arange(N, dtype=np.float32) + 1.0), (dim, N)), dtype=np.float32)


def perturbed_A(dim: int, N: int, seed: int, sigma: float = 0.25) -> np.ndarray:
    """A general diagonal A: the S4D-real values -(n+1), each scaled by
    exp(eps) with eps ~ N(0, sigma^2) per (d, n), as a learned A = -exp(A_log)
    drifts from its initialisation.  No A[d, n] is then (n+1) A[d, 0], so the
    kernels take the per-(t, n) exponential path."""
    rng = np.random.default_rng([seed, 31337])
    eps = rng.standard_normal((dim, N)).astype(np.float32) * np.float32(sigma)
    return (s4d_real_A(dim, N) * np.exp(eps)).astype(np.float32)


def mixed_A(dim: int, N: int, seed: int) -> np.ndarray:
    """S4D-real A on the even 64-channel groups and perturbed_A on the odd
    ones, plus one perturbed channel in group 2 (when dim reaches it): a
    call whose channel groups take both the power chain and the per-(t, n)
    exponential, one group general through a single channel."""
    A = s4d_real_A(dim, N)
    pert = perturbed_A(dim, N, seed)
    for g0 in range(64, dim, 128):
        A[g0:g0 + 64] = pert[g0:g0 + 64]
    if dim > 133:
        A[133] = pert[133]
    return A


def make_fwd_inputs(batch: int, L: int, dim: int, N: int, dtype: str = BF16, gate: bool = True,
                    seed: int = BASE_SEED, delta_std: float = 0.5, D_value: Optional[float] = 1.0,
                    with_bias: bool = True, h0: bool = False) -> FwdInputs:
    """Forward-scan inputs with the recipe in the module docstring.

    ``D_value=None`` draws D_skip ~ N(0,1) per channel; ``h0=True`` adds an
    initial state ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    bias = dt_bias(rng, dim)
    u = rng.standard_normal((batch, L, dim), dtype=np.float32)
    delta = rng.standard_normal((batch, L, dim), dtype=np.float32) * np.float32(delta_std)
    Bm = rng.standard_normal((batch, L, N), dtype=np.float32)
    Cm = rng.standard_normal((batch, L, N), dtype=np.float32)
    z = rng.standard_normal((batch, L, dim), dtype=np.float32) if gate else None
    if D_value is None:
        D_skip = rng.standard_normal(dim, dtype=np.float32)
    else:
        D_skip = np.full(dim, D_value, dtype=np.float32)
    h0_arr = rng.standard_normal((batch, dim, N), dtype=np.float32) if h0 else None
    return FwdInputs(
        dtype=dtype, batch=batch, L=L, dim=dim, N=N,
        u=_store(u, dtype), delta=_store(delta, dtype), Bm=_store(Bm, dtype),
        Cm=_store(Cm, dtype), z=_store(z, dtype) if gate else None,
        A=s4d_real_A(dim, N), D_skip=D_skip, delta_bias=bias if with_bias else None,
        h0=h0_arr)


def workload_fwd_inputs(w: Workload, **overrides) -> FwdInputs:
    kw = dict(batch=w.batch, L=w.L, dim=w.dim, N=w.N, dtype=w.dtype, gate=w.gate, seed=w.seed)
    kw.update(overrides)
    return make_fwd_inputs(**kw)


@dataclasses.dataclass
class StepInputs:
    u: Tensor        # (batch, dim)
    delta: Tensor    # (batch, dim)
    Bm: Tensor       # (batch, N)
    Cm: Tensor       # (batch, N)
    z: Optional[Tensor]


def decode_params(w: Workload):
    """Per-channel parameters of a decode workload: (A, D_skip, delta_bias)."""
    rng = np.random.default_rng(w.seed)
    bias = dt_bias(rng, w.dim)
    return s4d_real_A(w.dim, w.N), np.ones(w.dim, dtype=np.float32), bias


def decode_step_inputs(w: Workload, k: int, batch: Optional[int] = None) -> StepInputs:
    """Inputs of decode step ``k`` (0-based); seeded by (seed, k)."""
    b = w.batch if batch is None else batch
    rng = np.random.default_rng([w.seed, k])
    u = rng.standard_normal((b, w.dim), dtype=np.float32)
    delta = rng.standard_normal((b, w.dim), dtype=np.float32) * np.float32(0.5)
    Bm = rng.standard_normal((b, w.N), dtype=np.float32)
    Cm = rng.standard_normal((b, w.N), dtype=np.float32)
    z = rng.standard_normal((b, w.dim), dtype=np.float32) if w.gate else None
    return StepInputs(_store(u, w.dtype), _store(delta, w.dtype), _store(Bm, w.dtype),
                      _store(Cm, w.dtype), _store(z, w.dtype) if w.gate else None)


def to_torch(t: Optional[Tensor], dtype: str, device):
    """Upload one input array in its storage dtype (bf16 bits or fp32)."""
    import torch
    if t is None:
        return None
    if dtype == BF16:
        return torch.from_numpy(t.bits.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(t.value).to(device)


def fwd_tensors(inp: FwdInputs, device) -> dict:
    """The forward inputs as device tensors, keyed like the ABI arguments."""
    import torch
    f = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return dict(u=to_torch(inp.u, inp.dtype, device), delta=to_torch(inp.delta, inp.dtype, device),
                A=f(inp.A), Bm=to_torch(inp.Bm, inp.dtype, device),
                Cm=to_torch(inp.Cm, inp.dtype, device), D_skip=f(inp.D_skip),
                z=to_torch(inp.z, inp.dtype, device), delta_bias=f(inp.delta_bias), h0=f(inp.h0))


def step_tensors(st: StepInputs, dtype: str, device) -> dict:
    return dict(u=to_torch(st.u, dtype, device), delta=to_torch(st.delta, dtype, device),
                Bm=to_torch(st.Bm, dtype, device), Cm=to_torch(st.Cm, dtype, device),
                z=to_torch(st.z, dtype, device))


def channel_slice(inp: FwdInputs, channels: np.ndarray) -> FwdInputs:
    """The inputs restricted to a subset of channels.  Channels are independent
    in the scan, so the oracle on the slice gives those channels' outputs."""
    c = np.asarray(channels)
    sl = lambda t: None if t is None else Tensor(np.ascontiguousarray(t.value[..., c]),
                                                 None if t.bits is None else
                                                 np.ascontiguousarray(t.bits[..., c]))
    return FwdInputs(dtype=inp.dtype, batch=inp.batch, L=inp.L, dim=len(c), N=inp.N,
                     u=sl(inp.u), delta=sl(inp.delta), Bm=inp.Bm, Cm=inp.Cm, z=sl(inp.z),
                     A=np.ascontiguousarray(inp.A[c]),
                     D_skip=None if inp.D_skip is None else np.ascontiguousarray(inp.D_skip[c]),
                     delta_bias=None if inp.delta_bias is None else
                     np.ascontiguousarray(inp.delta_bias[c]),
                     h0=None if inp.h0 is None else np.ascontiguousarray(inp.h0[:, c]))


def decode_block(w: Workload, k0: int, k1: int, threads: int = 8):
    """Inputs of decode steps k0..k1-1, drawn in parallel (each step has its own
    seeded generator, so the result does not depend on ``threads``)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        return list(ex.map(lambda k: decode_step_inputs(w, k), range(k0, k1)))


def conv_params(dim: int, k: int, seed: int, with_bias: bool = True):
    """Depthwise causal conv taps (dim, k) and bias (dim,) in fp32, drawn
    uniform in +-1/sqrt(k) (the fan-in bound of a default grouped Conv1d)."""
    rng = np.random.default_rng([seed, 7919])
    bound = 1.0 / np.sqrt(k)
    w = rng.uniform(-bound, bound, size=(dim, k)).astype(np.float32)
    b = rng.uniform(-bound, bound, size=dim).astype(np.float32) if with_bias else None
    return w, b
