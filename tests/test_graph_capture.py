"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Every entry point launches kernels only (no allocation, no memset, no
synchronisation), so a graph can hold a forward, its backward and decode
steps, which is how a caller removes the per-call launch overhead.  Each
test captures once, then replays several times with new inputs copied into
the captured buffers and with eager work of the program between the
replays, and checks every replay bit for bit against eager calls on the same
inputs (every kernel here is deterministic), and once against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import selscan_inputs as si
import selective_state_space_selscan_amd as ss
from parity_util import TOL, rel_err, to_np

pytestmark = pytest.mark.gpu

SHAPE = (2, 1000, 130, 16)   # several parts, a ragged tail, lanes past dim


def say(*a):
    print(*a, flush=True)


def fresh_inputs(seed, dtype=si.BF16):
    batch, L, dim, N = SHAPE
    return si.make_fwd_inputs(batch, L, dim, N, dtype, True, seed=seed, h0=True)


def load_into(t, inp, device):
    """Copy a new input set into the captured input tensors."""
    new = si.fwd_tensors(inp, device)
    for k, v in t.items():
        if v is not None:
            v.copy_(new[k])


def capture(fn):
    """Warm up on a side stream (torch's rule for capture), then capture."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    return g, out


@pytest.mark.parametrize("plan", [None, "lookback"])
def test_forward_in_a_graph(device, monkeypatch, plan):
    if plan:
        monkeypatch.setenv("SELSCAN_FORCE_PLAN", plan)
    say("case graph forward", plan)
    batch, L, dim, N = SHAPE
    t = si.fwd_tensors(fresh_inputs(2000), device)
    y = torch.empty_like(t["u"])
    h_last = torch.empty((batch, dim, N), dtype=torch.float32, device=device)
    ws = torch.empty(max(1, ss.selscan_fwd_workspace_bytes(batch, L, dim, N, ss.SELSCAN_BF16)),
                     dtype=torch.uint8, device=device)

    def fwd():
        return ss.selscan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                              t["delta_bias"], True, t["h0"], y=y, h_last=h_last, workspace=ws)

    g, _ = capture(fwd)
    for k in range(3):
        inp = fresh_inputs(2001 + k)
        load_into(t, inp, device)
        g.replay()
        torch.cuda.synchronize()
        gy, gh = y.clone(), h_last.clone()
        # eager work between replays, on the same buffers
        ey = ss.selscan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                            t["delta_bias"], True, t["h0"], return_last_state=True)
        torch.cuda.synchronize()
        if plan is None:
            assert torch.equal(gy, ey[0]) and torch.equal(gh, ey[1]), "replay %d" % k
        if plan is None and k > 0:
            continue
        # the look-back plan's results may differ in rounding from call to
        # call (a part uses an inclusive state or composes aggregates), so
        # that two calls' bf16 outputs can differ by one unit in the last
        # place: every replay is checked against the oracle instead
        oy, oh = oracle.fwd_inputs(inp)
        ry, rh = rel_err(to_np(gy), oy), rel_err(to_np(gh), oh)
        assert ry <= TOL["bf16"] and rh <= TOL["bf16"], ("replay %d" % k, ry, rh)


def test_backward_in_a_graph(device):
    say("case graph backward")
    batch, L, dim, N = SHAPE
    t = si.fwd_tensors(fresh_inputs(2010), device)
    rng = np.random.default_rng(2011)
    dy = torch.from_numpy(rng.standard_normal((batch, L, dim)).astype(np.float32)).to(device)
    dy = dy.to(t["u"].dtype)
    dhl = torch.from_numpy(rng.standard_normal((batch, dim, N)).astype(np.float32)).to(device)
    ws = torch.empty(ss.selscan_bwd_workspace_bytes(batch, L, dim, N, ss.SELSCAN_BF16),
                     dtype=torch.uint8, device=device)

    def bwd():
        return ss.selscan_bwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], dy, t["D_skip"],
                              t["z"], t["delta_bias"], True, t["h0"], dhl, workspace=ws)

    g, grads = capture(bwd)
    for k in range(3):
        load_into(t, fresh_inputs(2012 + k), device)
        dy.copy_(torch.from_numpy(rng.standard_normal((batch, L, dim)).astype(np.float32))
                 .to(device).to(dy.dtype))
        g.replay()
        torch.cuda.synchronize()
        got = {n: (None if v is None else v.clone()) for n, v in grads.items()}
        eager = bwd()
        torch.cuda.synchronize()
        for n, v in got.items():
            if v is not None:
                assert torch.equal(v, eager[n]), "replay %d, %s" % (k, n)


def test_conv_variant_backward_in_a_graph(device):
    """The conv prologue's backward: its checkpoint pass, the main pass on
    the stored conv output and the epilogue, with exact ZOH and reverse."""
    say("case graph variant backward")
    batch, L, dim, N = SHAPE
    inp = fresh_inputs(2020)
    t = si.fwd_tensors(inp, device)
    cw, cb = (torch.from_numpy(x).to(device) for x in si.conv_params(dim, 4, 2021))
    rng = np.random.default_rng(2022)
    dy = torch.from_numpy(rng.standard_normal((batch, L, dim)).astype(np.float32)).to(device)
    dy = dy.to(t["u"].dtype)
    flags = ss.SELSCAN_FLAG_ZOH_EXACT | ss.SELSCAN_FLAG_REVERSE
    ws = torch.empty(ss.selscan_bwd_workspace_bytes(batch, L, dim, N, ss.SELSCAN_BF16),
                     dtype=torch.uint8, device=device)

    def bwd(f):
        return ss.selscan_bwd_ex(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], dy, t["D_skip"],
                                 t["z"], t["delta_bias"], True, t["h0"], None, flags=f,
                                 conv_weight=cw, conv_bias=cb, workspace=ws)

    for f in (0, flags):
        g, grads = capture(lambda: bwd(f))
        for k in range(2):
            load_into(t, fresh_inputs(2023 + k), device)
            g.replay()
            torch.cuda.synchronize()
            got = {n: (None if v is None else v.clone()) for n, v in grads.items()}
            eager = bwd(f)
            torch.cuda.synchronize()
            for n, v in got.items():
                if v is not None:
                    assert torch.equal(v, eager[n]), "flags %d replay %d, %s" % (f, k, n)


def test_decode_steps_in_a_graph(device):
    """Eight decode steps in one graph, on a state the graph updates in place."""
    say("case graph decode")
    batch, dim, N = 16, 300, 16
    rng = np.random.default_rng(2030)
    A = torch.from_numpy(si.s4d_real_A(dim, N)).to(device)
    D = torch.from_numpy(rng.standard_normal(dim).astype(np.float32)).to(device)
    bias = torch.from_numpy(si.dt_bias(rng, dim)).to(device)
    steps = 8
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(device).to(torch.bfloat16)
    ins = [dict(u=bf(rng.standard_normal((batch, dim))), delta=bf(0.5 * rng.standard_normal((batch, dim))),
                Bm=bf(rng.standard_normal((batch, N))), Cm=bf(rng.standard_normal((batch, N))),
                z=bf(rng.standard_normal((batch, dim)))) for _ in range(steps)]
    state = torch.zeros((batch, dim, N), dtype=torch.float32, device=device)
    ys = [torch.empty((batch, dim), dtype=torch.bfloat16, device=device) for _ in range(steps)]

    def run(st, outs):
        for s in range(steps):
            x = ins[s]
            ss.selscan_state_update(st, x["u"], x["delta"], A, x["Bm"], x["Cm"], D, x["z"], bias,
                                    True, y=outs[s])
        return outs

    g, _ = capture(lambda: run(state, ys))
    ref_state = torch.zeros_like(state)
    ref_ys = [torch.empty_like(y) for y in ys]
    for k in range(3):
        # start the eager copy from the graph's current state, then advance both
        ref_state.copy_(state)
        g.replay()
        run(ref_state, ref_ys)
        torch.cuda.synchronize()
        assert torch.equal(state, ref_state), "replay %d" % k
        for a, b in zip(ys, ref_ys):
            assert torch.equal(a, b), "replay %d" % k
