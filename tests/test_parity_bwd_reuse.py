"""The backward reading the forward's part state (SELSCAN_FLAG_REUSE_FWD_STATE),
and also its checkpoints (SELSCAN_FLAG_KEEP_CHECKPOINTS).

After a forward (selscan_fwd, or selscan_fwd_ex with REVERSE alone) in a
workspace, selscan_bwd_ex with the flag in that workspace skips the forward's
summary and carry passes.  Both sides run the same plan and the same
arithmetic, so every gradient is bit for bit that of the backward that
recomputes them in a workspace of its own; the shapes cover many parts (entry
states reused), 2-4 parts (the forward folds in its main pass and leaves no
entry states: the backward runs the carry on the reused summaries), one part
(nothing to reuse) and the two-level carry.
"""
import numpy as np
import pytest
import torch

import oracle
import selscan_inputs as si
import selective_state_space_selscan_amd as ss
from parity_util import TOL, rel_err, to_np

pytestmark = pytest.mark.gpu

REV, REUSE = ss.SELSCAN_FLAG_REVERSE, ss.SELSCAN_FLAG_REUSE_FWD_STATE
KEEP = ss.SELSCAN_FLAG_KEEP_CHECKPOINTS
ORACLE_NAME = {"ddelta_bias": "dbias"}
NAMES = ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0")


def say(*a):
    print(*a, flush=True)


CASES = [  # (batch, L, dim), dtype, forced part count
    ((2, 1234, 192), si.BF16, None),
    ((3, 517, 130), si.F32, None),
    ((2, 777, 130), si.BF16, 3),
    ((2, 12, 100), si.F32, None),        # one part
    ((1, 8192, 64), si.BF16, None),      # hundreds of parts: two-level carry
]


@pytest.mark.parametrize("flags", [0, REV], ids=["plain", "reverse"])
@pytest.mark.parametrize("shape,dtype,parts", CASES,
                         ids=["%dx%dx%d-%s-%s" % (c[0] + (c[1], c[2])) for c in CASES])
def test_bwd_reusing_forward_state_is_bitwise_equal(device, monkeypatch, flags, shape, dtype,
                                                    parts):
    if parts:
        monkeypatch.setenv("SELSCAN_STREAM_PARTS", str(parts))
    batch, L, dim = shape
    say("case reuse", flags, shape, dtype, parts)
    inp = si.make_fwd_inputs(batch, L, dim, 16, dtype, True, seed=1800 + L, h0=True)
    t = si.fwd_tensors(inp, device)
    rng = np.random.default_rng([1801, L])
    dy = torch.from_numpy(rng.standard_normal((batch, L, dim)).astype(np.float32)).to(device)
    dy = dy.to(t["u"].dtype)
    dhl = torch.from_numpy(rng.standard_normal((batch, dim, 16)).astype(np.float32)).to(device)
    code = ss.SELSCAN_BF16 if dtype == si.BF16 else ss.SELSCAN_F32
    nb = ss.selscan_bwd_workspace_bytes(batch, L, dim, 16, code)
    ws = torch.empty(nb, dtype=torch.uint8, device=device)
    args = (t["u"], t["delta"], t["A"], t["Bm"], t["Cm"])
    if flags:
        ss.selscan_fwd_ex(*args, t["D_skip"], t["z"], t["delta_bias"], True, t["h0"], flags=flags,
                          workspace=ws)
    else:
        ss.selscan_fwd(*args, t["D_skip"], t["z"], t["delta_bias"], True, t["h0"], workspace=ws)
    g_reuse = ss.selscan_bwd_ex(*args, dy, t["D_skip"], t["z"], t["delta_bias"], True, t["h0"],
                                dhl, flags=flags | REUSE, workspace=ws)
    g_own = ss.selscan_bwd_ex(*args, dy, t["D_skip"], t["z"], t["delta_bias"], True, t["h0"],
                              dhl, flags=flags)
    torch.cuda.synchronize()
    for k in NAMES:
        assert torch.equal(g_reuse[k], g_own[k]), k


def test_bwd_reuse_on_the_layer_workload(device):
    """batch 8, L 2048, D 1536, N 16, bf16, gate: the bench's backward shape."""
    w = si.WORKLOADS["mamba130m_layer"]
    inp = si.workload_fwd_inputs(w)
    t = si.fwd_tensors(inp, device)
    dy = torch.randn((w.batch, w.L, w.dim), device=device,
                     generator=torch.Generator(device=device).manual_seed(1802)).to(t["u"].dtype)
    ws = torch.empty(ss.selscan_bwd_workspace_bytes(w.batch, w.L, w.dim, w.N, ss.SELSCAN_BF16),
                     dtype=torch.uint8, device=device)
    args = (t["u"], t["delta"], t["A"], t["Bm"], t["Cm"])
    ss.selscan_fwd(*args, t["D_skip"], t["z"], t["delta_bias"], True, None, workspace=ws)
    g_reuse = ss.selscan_bwd_ex(*args, dy, t["D_skip"], t["z"], t["delta_bias"], True, None,
                                None, flags=REUSE, workspace=ws)
    g_own = ss.selscan_bwd(*args, dy, t["D_skip"], t["z"], t["delta_bias"], True, None, None)
    torch.cuda.synchronize()
    for k in NAMES:
        assert torch.equal(g_reuse[k], g_own[k]), k


def test_reuse_needs_the_forward_workspace(device):
    inp = si.make_fwd_inputs(1, 64, 64, 16, si.F32, True, seed=1803)
    t = si.fwd_tensors(inp, device)
    dy = torch.zeros_like(t["u"])
    with pytest.raises(ValueError):
        ss.selscan_bwd_ex(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], dy, flags=REUSE)


@pytest.mark.parametrize("flags", [0, REV], ids=["plain", "reverse"])
@pytest.mark.parametrize("N", [4, 16, 64])
@pytest.mark.parametrize("shape,dtype,parts", CASES,
                         ids=["%dx%dx%d-%s-%s" % (c[0] + (c[1], c[2])) for c in CASES])
def test_bwd_with_kept_checkpoints(device, monkeypatch, flags, N, shape, dtype, parts):
    """The forward keeps the checkpoints (y and h_last bit for bit those of
    the plain forward) and the backward reads them with the part state: every
    gradient against the oracle."""
    if parts:
        monkeypatch.setenv("SELSCAN_STREAM_PARTS", str(parts))
    batch, L, dim = shape
    if batch * L * dim * N > 40_000_000:
        L = 40_000_000 // (batch * dim * N)
    say("case keep", flags, N, (batch, L, dim), dtype, parts)
    inp = si.make_fwd_inputs(batch, L, dim, N, dtype, True, seed=1810 + L + N, h0=True)
    t = si.fwd_tensors(inp, device)
    rng = np.random.default_rng([1811, L, N])
    dy = torch.from_numpy(rng.standard_normal((batch, L, dim)).astype(np.float32)).to(device)
    dy = dy.to(t["u"].dtype)
    dhl = torch.from_numpy(rng.standard_normal((batch, dim, N)).astype(np.float32)).to(device)
    code = ss.SELSCAN_BF16 if dtype == si.BF16 else ss.SELSCAN_F32
    ws = torch.empty(ss.selscan_bwd_workspace_bytes(batch, L, dim, N, code), dtype=torch.uint8,
                     device=device)
    args = (t["u"], t["delta"], t["A"], t["Bm"], t["Cm"])
    y_keep, h_keep = ss.selscan_fwd_ex(*args, t["D_skip"], t["z"], t["delta_bias"], True, t["h0"],
                                       return_last_state=True, flags=flags | KEEP, workspace=ws)
    g = ss.selscan_bwd_ex(*args, dy, t["D_skip"], t["z"], t["delta_bias"], True, t["h0"], dhl,
                          flags=flags | REUSE | KEEP, workspace=ws)
    y, h = ss.selscan_fwd_ex(*args, t["D_skip"], t["z"], t["delta_bias"], True, t["h0"],
                             return_last_state=True, flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(y_keep, y) and torch.equal(h_keep, h)
    ref = oracle.bwd(inp.u.value, inp.delta.value, inp.A, inp.Bm.value, inp.Cm.value,
                     to_np(dy), inp.D_skip, inp.z.value, inp.delta_bias, True, inp.h0, to_np(dhl),
                     flags=flags)
    tol = TOL[dtype]
    errs = {k: rel_err(to_np(g[k]), ref[ORACLE_NAME.get(k, k)]) for k in NAMES}
    say("  rel_err " + " ".join("%s=%.2g" % kv for kv in errs.items()) + " (tol %.1g)" % tol)
    assert all(e <= tol for e in errs.values()), errs


def test_kept_checkpoints_on_the_layer_workload(device):
    """The bench's training-step pair with the checkpoints kept: the
    gradients against those of the backward that recomputes everything
    (both within rounding of the exact gradients)."""
    w = si.WORKLOADS["mamba130m_layer"]
    inp = si.workload_fwd_inputs(w)
    t = si.fwd_tensors(inp, device)
    dy = torch.randn((w.batch, w.L, w.dim), device=device,
                     generator=torch.Generator(device=device).manual_seed(1812)).to(t["u"].dtype)
    ws = torch.empty(ss.selscan_bwd_workspace_bytes(w.batch, w.L, w.dim, w.N, ss.SELSCAN_BF16),
                     dtype=torch.uint8, device=device)
    args = (t["u"], t["delta"], t["A"], t["Bm"], t["Cm"])
    ss.selscan_fwd_ex(*args, t["D_skip"], t["z"], t["delta_bias"], True, None, flags=KEEP,
                      workspace=ws)
    g_keep = ss.selscan_bwd_ex(*args, dy, t["D_skip"], t["z"], t["delta_bias"], True, None,
                               None, flags=REUSE | KEEP, workspace=ws)
    g_own = ss.selscan_bwd(*args, dy, t["D_skip"], t["z"], t["delta_bias"], True, None, None)
    torch.cuda.synchronize()
    for k in NAMES:
        if g_own[k] is None:
            continue
        e = rel_err(to_np(g_keep[k]), to_np(g_own[k]))
        say("  %s rel_err %.2g bitwise %s" % (k, e, torch.equal(g_keep[k], g_own[k])))
        assert e <= TOL["bf16"], (k, e)


def test_keep_needs_a_backward_workspace(device):
    inp = si.make_fwd_inputs(1, 64, 64, 16, si.F32, True, seed=1813)
    t = si.fwd_tensors(inp, device)
    with pytest.raises(ValueError):
        ss.selscan_fwd_ex(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], flags=KEEP)
