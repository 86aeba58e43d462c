"""GPU parity of the single-pass forward with decoupled look-back
(SELSCAN_FORCE_PLAN=lookback) against the fp64 oracle.

The plan changes only how a sequence part gets its entry state (a look-back
over the flags and states the earlier parts publish, instead of a fold of a
separate summary pass), so every case of the default plan's parity applies:
the workloads (sampled channels for the two largest), many parts with ragged
tails, every N, general A, h0, softplus off, and repeated calls (the flags
and the ticket counter are cleared per call).  Unlike the two-pass plan, the
look-back plan is not bitwise repeatable (see the last test).
"""
import numpy as np
import pytest
import torch

import oracle
import selscan_inputs as si
import selective_state_space_selscan_amd as ss
from parity_util import TOL, rel_err, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def lookback_plan(monkeypatch):
    monkeypatch.setenv("SELSCAN_FORCE_PLAN", "lookback")


def say(*a):
    print(*a, flush=True)


def check(inp, device, channels=None, what="", softplus=True):
    say("case", what, inp.batch, inp.L, inp.dim, inp.N, inp.dtype)
    t = si.fwd_tensors(inp, device)
    y, hL = ss.selscan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                           t["delta_bias"], softplus, t["h0"], return_last_state=True)
    torch.cuda.synchronize()
    sub = inp if channels is None else si.channel_slice(inp, channels)
    ey, ehL = oracle.fwd(sub.u.value, sub.delta.value, sub.A, sub.Bm.value, sub.Cm.value,
                         sub.D_skip, None if sub.z is None else sub.z.value, sub.delta_bias,
                         softplus, sub.h0)
    gy, gh = to_np(y), to_np(hL)
    if channels is not None:
        gy, gh = gy[..., channels], gh[:, channels]
    tol = TOL[inp.dtype]
    ry, rh = rel_err(gy, ey), rel_err(gh, ehL)
    say("  rel_err y=%.3g h_last=%.3g (tol %.1g)" % (ry, rh, tol))
    assert ry <= tol and rh <= tol, (ry, rh)
    return y, hL


def sample_channels(dim, k, seed=0):
    rng = np.random.default_rng(seed)
    c = rng.choice(dim, size=min(k, dim), replace=False)
    c[:2] = [0, dim - 1]
    return np.sort(np.unique(c))


@pytest.mark.parametrize("name,k", [("tiny_f32", None), ("mamba130m_layer", None),
                                    ("long_seq", 32), ("large_layer", 64)])
def test_lookback_workloads(device, name, k):
    w = si.WORKLOADS[name]
    inp = si.workload_fwd_inputs(w, D_value=0.0, gate=False)
    check(inp, device, None if k is None else sample_channels(w.dim, k), name)


@pytest.mark.parametrize("dtype", [si.F32, si.BF16])
@pytest.mark.parametrize("N", [4, 8, 16, 32, 64])
def test_lookback_every_state_size(device, N, dtype):
    inp = si.make_fwd_inputs(2, 700, 130, N, dtype, True, seed=1400 + N, h0=True, D_value=None)
    check(inp, device, what="N%d" % N)


@pytest.mark.parametrize("shape", [(1, 1, 64), (3, 5, 100), (2, 777, 65), (1, 4097, 192),
                                   (5, 129, 33)])
def test_lookback_ragged(device, shape):
    batch, L, dim = shape
    inp = si.make_fwd_inputs(batch, L, dim, 16, si.BF16, True, seed=1450 + sum(shape), h0=True)
    check(inp, device, what="ragged")


def test_lookback_unstructured_A_and_no_softplus(device):
    inp = si.make_fwd_inputs(2, 3000, 96, 16, si.F32, True, seed=1470, h0=True)
    rng = np.random.default_rng(1471)
    inp.A = (-np.exp(rng.uniform(-4.0, 2.5, size=(96, 16)))).astype(np.float32)
    check(inp, device, what="unstructured")
    inp.delta.value[:] = np.abs(inp.delta.value) * 0.05
    inp.delta_bias = np.full(96, 1e-3, np.float32)
    check(inp, device, what="no_softplus", softplus=False)


def test_lookback_repeated_calls_agree(device):
    """The flags and the ticket counter are cleared on every call, so repeated
    calls all give correct results.  They need not be bit-identical: a part
    uses its predecessor's inclusive state when it is already published and
    otherwise composes the aggregates before it, which rounds differently."""
    inp = si.make_fwd_inputs(4, 5000, 256, 16, si.BF16, True, seed=1480, h0=True)
    t = si.fwd_tensors(inp, device)
    outs = [ss.selscan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                           t["delta_bias"], True, t["h0"], return_last_state=True)
            for _ in range(3)]
    torch.cuda.synchronize()
    ey, ehL = oracle.fwd(inp.u.value, inp.delta.value, inp.A, inp.Bm.value, inp.Cm.value,
                         inp.D_skip, inp.z.value, inp.delta_bias, True, inp.h0)
    for y, h in outs:
        assert rel_err(to_np(y), ey) <= TOL["bf16"] and rel_err(to_np(h), ehL) <= TOL["bf16"]


def test_lookback_gave_up_wait_is_reported(device, monkeypatch):
    """With a poll limit of 0 every wait of a part after the first gives up at
    once (no wave ever waits, so every kernel still runs to its end): the
    status call reports SELSCAN_ERR_TIMEOUT and those parts come out NaN.
    With the default limit the same call is correct and reports OK."""
    inp = si.make_fwd_inputs(2, 3000, 128, 16, si.BF16, True, seed=1490, h0=True)
    t = si.fwd_tensors(inp, device)
    code = ss.SELSCAN_BF16
    ws = torch.empty(ss.selscan_fwd_workspace_bytes(2, 3000, 128, 16, code), dtype=torch.uint8,
                     device=device)
    monkeypatch.setenv("SELSCAN_LOOKBACK_SPIN_LIMIT", "0")
    say("case lookback spin limit 0")
    y = ss.selscan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                       t["delta_bias"], True, t["h0"], workspace=ws)
    with pytest.raises(ss.SelscanError) as e:
        ss.selscan_fwd_status(ws)
    assert e.value.status == 8   # SELSCAN_ERR_TIMEOUT
    yn = to_np(y)
    assert np.isnan(yn[:, -1]).all()          # the last part is poisoned
    assert not np.isnan(yn[:, 0]).any()       # the first part never waits
    monkeypatch.delenv("SELSCAN_LOOKBACK_SPIN_LIMIT")
    say("case lookback default spin limit")
    y = ss.selscan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                       t["delta_bias"], True, t["h0"], workspace=ws)
    ss.selscan_fwd_status(ws)   # raises on a timeout
    ey, _ = oracle.fwd_inputs(inp)
    assert rel_err(to_np(y), ey) <= TOL["bf16"]
