"""GPU parity of the backward (selscan_bwd) against the fp64 oracle backward.

Every gradient is compared element by element with ``oracle.bwd`` on the same
seeded inputs and upstream gradients.  Per-element gradients (du, ddelta, dz)
use the forward's tolerances; gradients that are sums over many terms (dA,
dB, dC, dD, ddelta_bias: over channels, or over batch and time) are compared
with the same metric, their error floored at the RMS of the reference.
"""
import numpy as np
import pytest
import torch

import oracle
import selscan_inputs as si
import selective_state_space_selscan_amd as ss
from parity_util import TOL, rel_err, to_np

pytestmark = pytest.mark.gpu

NAMES = ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0")
ORACLE_NAME = {"ddelta_bias": "dbias"}


def say(*a):
    print(*a, flush=True)


def upstream(inp, seed, with_dh_last=True):
    rng = np.random.default_rng([seed, 4242])
    dy = rng.standard_normal((inp.batch, inp.L, inp.dim)).astype(np.float32)
    if inp.dtype == si.BF16:
        dy = si.bf16_round_np(dy)[1]
    dhl = rng.standard_normal((inp.batch, inp.dim, inp.N)).astype(np.float32) \
        if with_dh_last else None
    return dy, dhl


def run_bwd(inp, dy, dhl, device, softplus=True):
    t = si.fwd_tensors(inp, device)
    tdy = torch.from_numpy(dy).to(device).to(t["u"].dtype)
    tdhl = None if dhl is None else torch.from_numpy(dhl).to(device)
    g = ss.selscan_bwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], tdy, t["D_skip"], t["z"],
                       t["delta_bias"], softplus, t["h0"], tdhl)
    torch.cuda.synchronize()
    return g


def check_bwd(inp, device, seed, what="", softplus=True, with_dh_last=True, tol=None):
    tol = TOL[inp.dtype] if tol is None else tol
    say("case", what, inp.batch, inp.L, inp.dim, inp.N, inp.dtype)
    dy, dhl = upstream(inp, seed, with_dh_last)
    g = run_bwd(inp, dy, dhl, device, softplus)
    ref = oracle.bwd(inp.u.value, inp.delta.value, inp.A, inp.Bm.value, inp.Cm.value, dy,
                     inp.D_skip, None if inp.z is None else inp.z.value, inp.delta_bias,
                     softplus, inp.h0, dhl)
    errs = {}
    for k in NAMES:
        r = ref[ORACLE_NAME.get(k, k)]
        if g[k] is None or r is None:
            continue
        errs[k] = rel_err(to_np(g[k]), r)
    say("  rel_err " + " ".join("%s=%.2g" % kv for kv in errs.items()) + " (tol %.1g)" % tol)
    bad = {k: e for k, e in errs.items() if not e <= tol}
    assert not bad, bad
    return g


@pytest.mark.parametrize("dtype", [si.F32, si.BF16])
def test_bwd_medium(device, dtype):
    """Several channel groups, lanes past dim, a ragged tail, many parts."""
    inp = si.make_fwd_inputs(2, 777, 130, 16, dtype, True, seed=1200, h0=True)
    check_bwd(inp, device, 1201, "medium")


@pytest.mark.parametrize("dtype", [si.F32, si.BF16])
def test_bwd_minimal_arguments(device, dtype):
    """No gate, D, bias, h0 or dh_last."""
    inp = si.make_fwd_inputs(2, 500, 64, 16, dtype, False, seed=1210, h0=False,
                             with_bias=False, D_value=None)
    inp.D_skip = None
    check_bwd(inp, device, 1211, "minimal", with_dh_last=False)


@pytest.mark.parametrize("N", [4, 8, 32, 64])
@pytest.mark.parametrize("dtype", [si.F32, si.BF16])
def test_bwd_every_state_size(device, N, dtype):
    inp = si.make_fwd_inputs(2, 300, 96, N, dtype, True, seed=1220 + N, h0=True)
    check_bwd(inp, device, 1221 + N, "N%d" % N)


@pytest.mark.parametrize("N,L", [(16, 900), (4, 300), (64, 250)])
def test_bwd_unstructured_A(device, N, L):
    inp = si.make_fwd_inputs(2, L, 160, N, si.F32, True, seed=1240 + N, h0=True)
    rng = np.random.default_rng(1241 + N)
    inp.A = (-np.exp(rng.uniform(-4.0, 2.5, size=(160, N)))).astype(np.float32)
    check_bwd(inp, device, 1242 + N, "unstructured")


@pytest.mark.parametrize("dtype", [si.F32, si.BF16])
@pytest.mark.parametrize("N", [4, 16, 64])
def test_bwd_mixed_structured_and_general_A(device, N, dtype):
    """Channel groups with structured A and with general A in one call (the
    main pass runs the first in one launch and the second in another)."""
    inp = si.make_fwd_inputs(2, 700, 320, N, dtype, True, seed=1250 + N, h0=True)
    inp.A = si.mixed_A(320, N, 1251 + N)
    check_bwd(inp, device, 1252 + N, "mixed A N%d" % N)


@pytest.mark.parametrize("shape", [(1, 1, 64), (1, 2, 1), (3, 3, 100), (2, 5, 65),
                                   (1, 17, 130), (2, 2049, 64)])
def test_bwd_ragged(device, shape):
    batch, L, dim = shape
    inp = si.make_fwd_inputs(batch, L, dim, 16, si.BF16, True, seed=1260 + sum(shape), h0=True)
    check_bwd(inp, device, 1261 + sum(shape), "ragged")


def test_bwd_without_softplus(device):
    inp = si.make_fwd_inputs(2, 600, 96, 16, si.F32, True, seed=1280, h0=True)
    inp.delta.value[:] = np.abs(inp.delta.value) * 0.05
    inp.delta_bias = np.full(96, 1e-3, np.float32)
    check_bwd(inp, device, 1281, "no_softplus", softplus=False)


def test_bwd_bitwise_repeatable(device):
    inp = si.make_fwd_inputs(2, 1500, 200, 16, si.BF16, True, seed=1290, h0=True)
    dy, dhl = upstream(inp, 1291)
    g1 = run_bwd(inp, dy, dhl, device)
    g2 = run_bwd(inp, dy, dhl, device)
    for k in NAMES:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), k


def test_bwd_layer_workload(device):
    """The 130M-layer shape (batch 8, L 2048, D 1536, N 16, bf16, gate, D,
    bias), every gradient against the oracle in full."""
    w = si.WORKLOADS["mamba130m_layer"]
    inp = si.workload_fwd_inputs(w)
    check_bwd(inp, device, 1300, "mamba130m_layer", with_dh_last=False)


def test_bwd_long_sequence_many_parts(device):
    """One channel group over a long sequence: 512 parts, so the entry states
    come from the two-level carry (blocks of 64 part summaries), in both
    directions (h0 from the left, dh_last from the right)."""
    inp = si.make_fwd_inputs(1, 8192, 64, 16, si.F32, True, seed=1310, h0=True)
    check_bwd(inp, device, 1311, "long/many parts")
