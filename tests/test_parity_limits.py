"""GPU parity at the size limits of the C ABI.

* dim = 2^24, the largest channel count (every per-chunk buffer range and
  offset of the kernels stays within 32 bits up to there): forward (with h0
  and h_last), backward and the decode step, checked against the oracle on a
  sample of channels that includes the last ones.  Channels are independent,
  so the oracle on the sampled channels gives exactly their outputs.  The
  backward's dB and dC are sums over every channel; they are checked with
  identities that hold at any size: with D = 0, y is linear in C, so
  sum dC * C = sum dy * y, and with a zero initial state also linear in B,
  so sum dB * B = sum dy * y.
* a long sequence on a single channel group (L = 2^19, batch 1, dim 64):
  the most sequence parts the plan makes, checked in full.
"""
import numpy as np
import pytest
import torch

import oracle
import selscan_inputs as si
import selective_state_space_selscan_amd as ss
from parity_util import TOL, rel_err, to_np

pytestmark = pytest.mark.gpu

MAX_DIM = 1 << 24


def say(*a):
    print(*a, flush=True)


def sampled(dim, k, seed):
    rng = np.random.default_rng(seed)
    c = np.unique(np.concatenate([rng.choice(dim, size=k, replace=False),
                                  [0, 63, 64, dim - 65, dim - 64, dim - 2, dim - 1]]))
    return np.sort(c)


def test_max_dim_forward(device):
    inp = si.make_fwd_inputs(1, 5, MAX_DIM, 4, si.BF16, True, seed=1600, h0=True)
    say("case max_dim forward", inp.batch, inp.L, inp.dim, inp.N)
    t = si.fwd_tensors(inp, device)
    y, hL = ss.selscan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                           t["delta_bias"], True, t["h0"], return_last_state=True)
    torch.cuda.synchronize()
    ch = sampled(MAX_DIM, 200, 1601)
    ey, eh = oracle.fwd_inputs(si.channel_slice(inp, ch))
    ry, rh = rel_err(to_np(y[..., ch]), ey), rel_err(to_np(hL[:, ch]), eh)
    say("  rel_err y=%.3g h_last=%.3g" % (ry, rh))
    assert ry <= TOL[si.BF16] and rh <= TOL[si.BF16]


def test_max_dim_backward(device):
    inp = si.make_fwd_inputs(1, 6, MAX_DIM, 4, si.F32, True, seed=1610, h0=True)
    say("case max_dim backward", inp.batch, inp.L, inp.dim, inp.N)
    rng = np.random.default_rng(1611)
    dy = rng.standard_normal((1, 6, MAX_DIM), dtype=np.float32)
    t = si.fwd_tensors(inp, device)
    g = ss.selscan_bwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"],
                       torch.from_numpy(dy).to(device), t["D_skip"], t["z"], t["delta_bias"],
                       True, t["h0"])
    torch.cuda.synchronize()
    ch = sampled(MAX_DIM, 200, 1612)
    sub = si.channel_slice(inp, ch)
    ref = oracle.bwd(sub.u.value, sub.delta.value, sub.A, sub.Bm.value, sub.Cm.value,
                     np.ascontiguousarray(dy[..., ch]), sub.D_skip, sub.z.value, sub.delta_bias,
                     True, sub.h0)
    errs = {
        "du": rel_err(to_np(g["du"][..., ch]), ref["du"]),
        "ddelta": rel_err(to_np(g["ddelta"][..., ch]), ref["ddelta"]),
        "dz": rel_err(to_np(g["dz"][..., ch]), ref["dz"]),
        "dA": rel_err(to_np(g["dA"][ch]), ref["dA"]),
        "dD": rel_err(to_np(g["dD"][ch]), ref["dD"]),
        "ddelta_bias": rel_err(to_np(g["ddelta_bias"][ch]), ref["dbias"]),
        "dh0": rel_err(to_np(g["dh0"][:, ch]), ref["dh0"]),
    }
    say("  rel_err " + " ".join("%s=%.2g" % kv for kv in errs.items()))
    bad = {k: e for k, e in errs.items() if not e <= TOL[si.F32]}
    assert not bad, bad
    # dC[b,t,n] = sum_d dy[b,t,d] SiLU(z) h_t[b,d,n]: with zero D, y = (C.h) SiLU(z)
    # is linear in C, so sum_{t,n} dC[t,n] C[t,n] equals sum dy * y.
    inp0 = si.make_fwd_inputs(1, 6, MAX_DIM, 4, si.F32, True, seed=1610, h0=True, D_value=0.0)
    t0 = si.fwd_tensors(inp0, device)
    y0 = ss.selscan_fwd(t0["u"], t0["delta"], t0["A"], t0["Bm"], t0["Cm"], t0["D_skip"],
                        t0["z"], t0["delta_bias"], True, t0["h0"])
    g0 = ss.selscan_bwd(t0["u"], t0["delta"], t0["A"], t0["Bm"], t0["Cm"],
                        torch.from_numpy(dy).to(device), t0["D_skip"], t0["z"],
                        t0["delta_bias"], True, t0["h0"])
    torch.cuda.synchronize()
    rhs = float((torch.from_numpy(dy).to(device).double() * y0.double()).sum())
    lhs = float((g0["dC"].double() * t0["Cm"].double()).sum())
    say("  sum dC*C=%.6g sum dy*y=%.6g" % (lhs, rhs))
    assert abs(lhs - rhs) <= 1e-4 * max(1.0, abs(rhs))
    # likewise h, hence y, is linear in B when the initial state is zero (h0
    # absent here): sum dB * B = sum dy * y
    y1 = ss.selscan_fwd(t0["u"], t0["delta"], t0["A"], t0["Bm"], t0["Cm"], t0["D_skip"],
                        t0["z"], t0["delta_bias"], True, None)
    g1 = ss.selscan_bwd(t0["u"], t0["delta"], t0["A"], t0["Bm"], t0["Cm"],
                        torch.from_numpy(dy).to(device), t0["D_skip"], t0["z"],
                        t0["delta_bias"], True, None)
    torch.cuda.synchronize()
    rhs1 = float((torch.from_numpy(dy).to(device).double() * y1.double()).sum())
    lhs1 = float((g1["dB"].double() * t0["Bm"].double()).sum())
    say("  sum dB*B=%.6g sum dy*y=%.6g" % (lhs1, rhs1))
    assert abs(lhs1 - rhs1) <= 1e-4 * max(1.0, abs(rhs1))


def test_max_dim_state_update(device):
    rng = np.random.default_rng(1620)
    N = 4
    A = -np.tile(np.arange(1, N + 1, dtype=np.float32), (MAX_DIM, 1))
    state0 = rng.standard_normal((1, MAX_DIM, N)).astype(np.float32)
    u = si.bf16_round_np(rng.standard_normal((1, MAX_DIM)).astype(np.float32))[1]
    delta = si.bf16_round_np((0.5 * rng.standard_normal((1, MAX_DIM))).astype(np.float32))[1]
    Bm = si.bf16_round_np(rng.standard_normal((1, N)).astype(np.float32))[1]
    Cm = si.bf16_round_np(rng.standard_normal((1, N)).astype(np.float32))[1]
    bias = np.full(MAX_DIM, -3.0, np.float32)
    say("case max_dim state_update", MAX_DIM, N)
    dev = lambda a: torch.from_numpy(a).to(device)
    state = dev(state0)
    y = ss.selscan_state_update(state, dev(u).bfloat16(), dev(delta).bfloat16(), dev(A),
                                dev(Bm).bfloat16(), dev(Cm).bfloat16(), None, None, dev(bias),
                                True)
    torch.cuda.synchronize()
    ch = sampled(MAX_DIM, 200, 1621)
    ost = state0[:, ch].astype(np.float64)
    ey = oracle.state_update(ost, u[:, ch], delta[:, ch], A[ch], Bm, Cm, None, None, bias[ch],
                             True)
    ry, rs = rel_err(to_np(y)[:, ch], ey), rel_err(to_np(state)[:, ch], ost)
    say("  rel_err y=%.3g state=%.3g" % (ry, rs))
    assert ry <= TOL[si.BF16] and rs <= TOL[si.F32]


def test_long_sequence_single_group(device):
    L = 1 << 19
    inp = si.make_fwd_inputs(1, L, 64, 16, si.BF16, True, seed=1630, h0=True)
    say("case long single group", inp.batch, inp.L, inp.dim, inp.N)
    t = si.fwd_tensors(inp, device)
    y, hL = ss.selscan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                           t["delta_bias"], True, t["h0"], return_last_state=True)
    torch.cuda.synchronize()
    ey, eh = oracle.fwd_inputs(inp)
    ry, rh = rel_err(to_np(y), ey), rel_err(to_np(hL), eh)
    say("  rel_err y=%.3g h_last=%.3g" % (ry, rh))
    assert ry <= TOL[si.BF16] and rh <= TOL[si.BF16]
