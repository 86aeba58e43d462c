"""GPU parity of the ablation plans of the forward against the fp64 oracle.

SELSCAN_FORCE_PLAN=chunked selects the workgroup-chunked kernel: the waves of
a workgroup share 64 channels, each runs one segment of a chunk from zero, the
segment aggregates are exchanged through LDS with one barrier and every wave
re-runs its segment from its true entry state (the chunked scan of the paper
walkthrough (m.lqnn.cn) §3.2, the carry between segments staged in LDS).
SELSCAN_FORCE_PLAN=dpp selects the in-wave scan over time: the lanes of a wave
hold 64 consecutive steps of one channel and the pairs (A_bar, B_bar u) are
scanned across them with DPP row shifts and row broadcasts (the parallel scan
of the Mamba tutorial (pwwt.cn) §3.2 with the associative operator of the
selection-mechanism article (discosf.com) §3.1), the state between tiles
carried in scalar registers; shapes with few channels also split the
sequence into parts joined by the summary and carry passes.  Both ship in
the library and are reachable through selscan_fwd, so they face the default
plan's parity cases: the tiny and layer workloads, ragged shapes (tails,
lanes past dim, partial tiles, many parts), every N in fp32 and bf16, h0,
general A and softplus off.
"""
import numpy as np
import pytest
import torch

import oracle
import selscan_inputs as si
import selective_state_space_selscan_amd as ss
from parity_util import TOL, rel_err, to_np

pytestmark = pytest.mark.gpu

PLANS = ["chunked", "dpp"]


def say(*a):
    print(*a, flush=True)


def check(inp, device, plan, monkeypatch, what="", softplus=True):
    monkeypatch.setenv("SELSCAN_FORCE_PLAN", plan)
    say("case", plan, what, inp.batch, inp.L, inp.dim, inp.N, inp.dtype)
    t = si.fwd_tensors(inp, device)
    y, hL = ss.selscan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                           t["delta_bias"], softplus, t["h0"], return_last_state=True)
    torch.cuda.synchronize()
    ey, ehL = oracle.fwd(inp.u.value, inp.delta.value, inp.A, inp.Bm.value, inp.Cm.value,
                         inp.D_skip, None if inp.z is None else inp.z.value, inp.delta_bias,
                         softplus, inp.h0)
    tol = TOL[inp.dtype]
    ry, rh = rel_err(to_np(y), ey), rel_err(to_np(hL), ehL)
    say("  rel_err y=%.3g h_last=%.3g (tol %.1g)" % (ry, rh, tol))
    assert ry <= tol and rh <= tol, (ry, rh)


@pytest.mark.parametrize("plan", PLANS)
@pytest.mark.parametrize("name", ["tiny_f32", "mamba130m_layer"])
@pytest.mark.parametrize("scan_only", [False, True])
def test_plan_workloads(device, monkeypatch, plan, name, scan_only):
    w = si.WORKLOADS[name]
    kw = dict(D_value=0.0, gate=False) if scan_only else {}
    check(si.workload_fwd_inputs(w, **kw), device, plan, monkeypatch, name)


@pytest.mark.parametrize("plan", PLANS)
@pytest.mark.parametrize("dtype", [si.F32, si.BF16])
@pytest.mark.parametrize("N", [4, 8, 16, 32, 64])
def test_plan_every_state_size(device, monkeypatch, plan, N, dtype):
    inp = si.make_fwd_inputs(2, 700, 130, N, dtype, True, seed=1600 + N, h0=True, D_value=None)
    check(inp, device, plan, monkeypatch, "N%d" % N)


@pytest.mark.parametrize("plan", PLANS)
@pytest.mark.parametrize("shape", [(1, 1, 64), (3, 5, 100), (2, 777, 65), (1, 4097, 192),
                                   (5, 129, 33), (1, 20000, 64)])
def test_plan_ragged(device, monkeypatch, plan, shape):
    batch, L, dim = shape
    inp = si.make_fwd_inputs(batch, L, dim, 16, si.BF16, True, seed=1650 + sum(shape), h0=True)
    check(inp, device, plan, monkeypatch, "ragged%s" % (shape,))


@pytest.mark.parametrize("plan", PLANS)
def test_plan_unstructured_A_and_no_softplus(device, monkeypatch, plan):
    inp = si.make_fwd_inputs(2, 3000, 96, 16, si.F32, True, seed=1670, h0=True)
    rng = np.random.default_rng(1671)
    inp.A = (-np.exp(rng.uniform(-4.0, 2.5, size=(96, 16)))).astype(np.float32)
    check(inp, device, plan, monkeypatch, "unstructured")
    inp.delta.value[:] = np.abs(inp.delta.value) * 0.05
    inp.delta_bias = np.full(96, 1e-3, np.float32)
    check(inp, device, plan, monkeypatch, "no_softplus", softplus=False)
