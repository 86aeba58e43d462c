"""GPU check of selscan_fwd_noalloc, the forward for callers that cannot
allocate: its workspace is the library's fixed device scratch.

It is called through the C ABI (ctypes) and compared with selscan_fwd (the
same kernels and plan, so bit for bit) and with the fp64 oracle (to the
parity tolerances), on two calls in a row, the second with a smaller input
(the scratch keeps the first call's contents, which must not leak into the
second), then once more at the first size.  (The host-side refusal of
shapes beyond the scratch is in tests/test_abi.py.)
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

SCRATCH_BYTES = 128 << 20


def say(*a):
    print(*a, flush=True)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def call_noalloc(t, y, h_last, dtype):
    batch, L, dim = t["u"].shape
    N = t["A"].shape[1]
    code = ss.SELSCAN_BF16 if dtype == si.BF16 else ss.SELSCAN_F32
    return ss.lib().selscan_fwd_noalloc(
        _p(t["u"]), _p(t["delta"]), _p(t["A"]), _p(t["Bm"]), _p(t["Cm"]), _p(t["D_skip"]),
        _p(t["z"]), _p(t["delta_bias"]), 1, _p(t["h0"]), _p(y), _p(h_last), batch, L, dim, N,
        code, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def check_once(device, shape, dtype, seed):
    batch, L, dim = shape
    say("case noalloc", shape, dtype)
    inp = si.make_fwd_inputs(batch, L, dim, 16, dtype, True, seed=seed, h0=True)
    t = si.fwd_tensors(inp, device)
    tdt = torch.bfloat16 if dtype == si.BF16 else torch.float32
    y = torch.full((batch, L, dim), float("nan"), dtype=tdt, device=device)
    hl = torch.full((batch, dim, 16), float("nan"), dtype=torch.float32, device=device)
    assert call_noalloc(t, y, hl, dtype) == 0
    ry, rh = ss.selscan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                            t["delta_bias"], True, t["h0"], return_last_state=True)
    torch.cuda.synchronize()
    assert torch.equal(y, ry) and torch.equal(hl, rh), "differs from selscan_fwd"
    ey, eh = oracle.fwd_inputs(inp)
    e1, e2 = rel_err(to_np(y), ey), rel_err(to_np(hl), eh)
    say("  rel_err y=%.3g h_last=%.3g" % (e1, e2))
    assert e1 <= TOL[dtype] and e2 <= TOL[dtype]


@pytest.mark.parametrize("dtype", [si.BF16, si.F32])
def test_noalloc_matches_selscan_fwd_twice_then_smaller(device, dtype):
    big, small = (8, 2048, 1536), (2, 333, 100)
    need = ss.selscan_fwd_workspace_bytes(*big, 16, 1 if dtype == si.BF16 else 0)
    assert 0 < need <= SCRATCH_BYTES
    check_once(device, big, dtype, seed=71)
    check_once(device, small, dtype, seed=72)
    check_once(device, big, dtype, seed=73)
