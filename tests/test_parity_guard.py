"""GPU checks that the kernels write exactly their outputs and nothing else.

* Guard bands: every output lies inside a larger buffer filled with a sentinel
  bit pattern before and after it; ragged sequence lengths (the last chunk of a
  part shorter than the prefetch chunk), ragged channel counts (lanes past dim)
  and the last batch row (whose overflow would land past the array) must leave
  every sentinel word unchanged, in the forward (both directions, with and
  without the variants) and the backward (its per-element gradients).
* Optional backward outputs: dD, ddelta_bias, dh0 and dconv_bias may be NULL
  at the C ABI ("skip"); the remaining gradients must then be bit-equal to
  those of the call that returns everything.

Both go through the C ABI (the forward via the Python binding with
preallocated outputs, the backward by ctypes with chosen pointers), and the
outputs are also compared with the fp64 oracle.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import selscan_inputs as si
import selective_state_space_selscan_amd as ss
from parity_util import TOL, rel_err, to_np

pytestmark = pytest.mark.gpu

GUARD = 4096          # elements of sentinel before and after each output
SENT16 = 0x7FA5       # a NaN pattern no finite result has (bf16)
SENT32 = 0x7FC0DEAD   # likewise for fp32


def say(*a):
    print(*a, flush=True)


class Guarded:
    """An output tensor of ``shape`` inside a sentinel-filled buffer."""

    def __init__(self, shape, dtype, device):
        n = int(np.prod(shape))
        self.buf = torch.empty(GUARD + n + GUARD, dtype=dtype, device=device)
        self._bits().fill_(self._sentinel())
        self.n = n
        self.t = self.buf[GUARD:GUARD + n].view(*shape)
        assert self.t.data_ptr() % 16 == 0

    def _bits(self):
        return self.buf.view(torch.int16 if self.buf.dtype == torch.bfloat16 else torch.int32)

    def _sentinel(self):
        return SENT16 if self.buf.dtype == torch.bfloat16 else SENT32

    def intact(self) -> bool:
        bits, s = self._bits(), self._sentinel()
        return bool((bits[:GUARD] == s).all() and (bits[GUARD + self.n:] == s).all())


def torch_dtype(dtype):
    return torch.bfloat16 if dtype == si.BF16 else torch.float32


VARIANTS = [("plain", 0, 0), ("rev", ss.SELSCAN_FLAG_REVERSE, 0),
            ("zoh_rev_conv4", ss.SELSCAN_FLAG_ZOH_EXACT | ss.SELSCAN_FLAG_REVERSE, 4),
            ("conv3", 0, 3)]


@pytest.mark.parametrize("shape", [(3, 1, 100), (2, 7, 65), (2, 2049, 130), (1, 4099, 64),
                                   (4, 13, 1)])
@pytest.mark.parametrize("variant", VARIANTS, ids=[v[0] for v in VARIANTS])
@pytest.mark.parametrize("dtype", [si.BF16, si.F32])
def test_fwd_writes_only_its_outputs(device, shape, variant, dtype):
    batch, L, dim = shape
    name, flags, k = variant
    say("case fwd guard", shape, name, dtype)
    inp = si.make_fwd_inputs(batch, L, dim, 16, dtype, True, seed=batch * 7 + L + dim, h0=True)
    t = si.fwd_tensors(inp, device)
    yg = Guarded((batch, L, dim), torch_dtype(dtype), device)
    hg = Guarded((batch, dim, 16), torch.float32, device)
    cw = cb = None
    if k:
        cw, cb = si.conv_params(dim, k, 5)
    if flags or k:
        ss.selscan_fwd_ex(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                          t["delta_bias"], True, t["h0"], return_last_state=True, flags=flags,
                          conv_weight=None if cw is None else torch.from_numpy(cw).to(device),
                          conv_bias=None if cb is None else torch.from_numpy(cb).to(device),
                          y=yg.t, h_last=hg.t)
    else:
        ss.selscan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                       t["delta_bias"], True, t["h0"], return_last_state=True, y=yg.t,
                       h_last=hg.t)
    torch.cuda.synchronize()
    assert yg.intact(), "y: a store landed outside the output"
    assert hg.intact(), "h_last: a store landed outside the output"
    ey, eh = oracle.fwd_inputs(inp, flags=flags, conv_w=cw, conv_b=cb)
    assert rel_err(to_np(yg.t), ey) <= TOL[dtype]
    assert rel_err(to_np(hg.t), eh) <= TOL[dtype]


# ---------------------------------------------------------------------------
# the backward through ctypes
# ---------------------------------------------------------------------------
def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def run_bwd_abi(t, dy, outs, flags=0, conv=None, dtype=si.BF16, workspace=None):
    """selscan_bwd_ex with the given output tensors (None = NULL)."""
    batch, L, dim = t["u"].shape
    N = t["A"].shape[1]
    code = ss.SELSCAN_BF16 if dtype == si.BF16 else ss.SELSCAN_F32
    wsb = ss.selscan_bwd_workspace_bytes(batch, L, dim, N, code)
    ws = workspace if workspace is not None else torch.empty(wsb, dtype=torch.uint8,
                                                             device=t["u"].device)
    cw, cb = (None, None) if conv is None else conv
    k = 0 if cw is None else cw.shape[1]
    rc = ss.lib().selscan_bwd_ex(
        _p(t["u"]), _p(t["delta"]), _p(t["A"]), _p(t["Bm"]), _p(t["Cm"]), _p(t["D_skip"]),
        _p(t["z"]), _p(t["delta_bias"]), 1, _p(t["h0"]), _p(dy), None,
        _p(outs["du"]), _p(outs["ddelta"]), _p(outs["dA"]), _p(outs["dB"]), _p(outs["dC"]),
        _p(outs.get("dD")), _p(outs["dz"]), _p(outs.get("ddelta_bias")), _p(outs.get("dh0")),
        flags, _p(cw), _p(cb), k, _p(outs.get("dconv_weight")), _p(outs.get("dconv_bias")),
        batch, L, dim, N, code, _p(ws), wsb, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, ss.status_string(rc)


def bwd_setup(device, shape, dtype, k, seed):
    batch, L, dim = shape
    inp = si.make_fwd_inputs(batch, L, dim, 16, dtype, True, seed=seed, h0=True)
    t = si.fwd_tensors(inp, device)
    rng = np.random.default_rng(seed + 1)
    dyv = rng.standard_normal((batch, L, dim)).astype(np.float32)
    if dtype == si.BF16:
        dyv = si.bf16_round_np(dyv)[1]
    dy = torch.from_numpy(dyv).to(device).to(torch_dtype(dtype))
    conv = None
    if k:
        cw, cb = si.conv_params(dim, k, seed + 2)
        conv = (torch.from_numpy(cw).to(device), torch.from_numpy(cb).to(device))
    return inp, t, dyv, dy, conv


def full_outputs(shape, dtype, device, k):
    batch, L, dim = shape
    f32, dt = torch.float32, torch_dtype(dtype)
    o = dict(du=torch.empty(shape, dtype=dt, device=device),
             ddelta=torch.empty(shape, dtype=dt, device=device),
             dz=torch.empty(shape, dtype=dt, device=device),
             dA=torch.empty((dim, 16), dtype=f32, device=device),
             dB=torch.empty((batch, L, 16), dtype=f32, device=device),
             dC=torch.empty((batch, L, 16), dtype=f32, device=device),
             dD=torch.empty(dim, dtype=f32, device=device),
             ddelta_bias=torch.empty(dim, dtype=f32, device=device),
             dh0=torch.empty((batch, dim, 16), dtype=f32, device=device))
    if k:
        o["dconv_weight"] = torch.empty((dim, k), dtype=f32, device=device)
        o["dconv_bias"] = torch.empty(dim, dtype=f32, device=device)
    return o


@pytest.mark.parametrize("shape", [(3, 1, 100), (2, 2049, 130), (1, 1031, 64)])
@pytest.mark.parametrize("variant", VARIANTS, ids=[v[0] for v in VARIANTS])
def test_bwd_writes_only_its_outputs(device, shape, variant):
    name, flags, k = variant
    say("case bwd guard", shape, name)
    dtype = si.BF16
    inp, t, dyv, dy, conv = bwd_setup(device, shape, dtype, k, seed=sum(shape))
    outs = full_outputs(shape, dtype, device, k)
    guards = {key: Guarded(outs[key].shape, outs[key].dtype, device) for key in outs}
    for key in outs:
        outs[key] = guards[key].t
    run_bwd_abi(t, dy, outs, flags, conv, dtype)
    torch.cuda.synchronize()
    for key, g in guards.items():
        assert g.intact(), "%s: a store landed outside the output" % key
    cw = None if conv is None else conv[0].cpu().numpy()
    cb = None if conv is None else conv[1].cpu().numpy()
    eg = oracle.bwd(inp.u.value, inp.delta.value, inp.A, inp.Bm.value, inp.Cm.value, dyv,
                    inp.D_skip, inp.z.value, inp.delta_bias, True, inp.h0, flags=flags,
                    conv_w=cw, conv_b=cb)
    for key, ekey in (("du", "du"), ("ddelta", "ddelta"), ("dz", "dz"), ("dA", "dA"),
                      ("dB", "dB"), ("dC", "dC"), ("dD", "dD"), ("ddelta_bias", "dbias"),
                      ("dh0", "dh0")):
        e = rel_err(to_np(outs[key]), eg[ekey])
        assert e <= TOL[dtype], (key, e)


@pytest.mark.parametrize("variant", [("plain", 0, 0), ("conv4", 0, 4),
                                     ("zoh_rev_conv2", 3, 2)], ids=lambda v: v[0])
@pytest.mark.parametrize("shape", [(2, 300, 96), (1, 2049, 64)])
def test_bwd_optional_outputs_may_be_null(device, variant, shape):
    """NULL dD, ddelta_bias, dh0 (and dconv_bias) are skipped; every other
    gradient is bit-equal to the full call's."""
    name, flags, k = variant
    say("case bwd null outputs", shape, name)
    dtype = si.BF16
    _, t, _, dy, conv = bwd_setup(device, shape, dtype, k, seed=11)
    full = full_outputs(shape, dtype, device, k)
    run_bwd_abi(t, dy, full, flags, conv, dtype)
    part = full_outputs(shape, dtype, device, k)
    for key in ("dD", "ddelta_bias", "dh0", "dconv_bias"):
        part.pop(key, None)
    run_bwd_abi(t, dy, part, flags, conv, dtype)
    torch.cuda.synchronize()
    for key in part:
        assert torch.equal(part[key], full[key]), key
